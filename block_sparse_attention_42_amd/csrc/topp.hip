// Top-p selection over competition domains on gfx950.
//
// Page: "Competition Domains Matter ... (EG-Sparse)": per-head attention
// entropy (its Eq. 3); the domain hierarchy of its Section 3.3 (per-row
// local, per-head global, grouped cross-head split at the entropy median,
// all-head global) and its deployed routing (low-entropy heads share one
// pool, the others stay per-row local); top-p of a domain's score mass; the
// value-aware score of the cross-head pool (P' times the norm of the key
// cluster's value centroid); the one-key-per-row safeguard.
//
// Mass is counted in fixed point, m(s) = floor(s * 2^32) + 1, so a pool's
// mass is an exact integer whatever the summation order, and its threshold
// -- the largest score T with mass(score >= T) >= ceil(p * mass(pool)) --
// is found by a radix select over the scores' order keys with integer bin
// masses (four 8-bit passes, integer atomics).  A per-row local domain finds
// its T by the same radix select inside one wave, with the bins in that
// wave's LDS.  Every block with score >= T is kept.
//
// Kernels, in launch order (grid-wide dependencies between them):
//   tp_row_entropy    one wave per row: sum_j -P log(P + eps) (float64, the
//                     log by its own series); the workgroups past the rows
//                     take the norms of the pooled value rows (value-aware
//                     scores)
//   tp_head_entropy   one workgroup per head: the mean over its rows
//   tp_pools          one workgroup per batch element: median split, pool of
//                     every head, pool state cleared
//   tp_hist (x4)      radix passes of the pooled thresholds: integer bin
//                     masses of a few rows per workgroup, each pass
//                     into its own bins; a pass starts by deriving the digits
//                     of the passes before it from their bins (every wave, the
//                     same suffix scans), and the first pass's bins add up to
//                     the pool's mass, which sets the target
//   tp_select         one wave per row: threshold (the pool's, derived from
//                     its four bin sets, or the row's own radix select),
//                     safeguard, frame-0 rows, text columns, compaction
#include <algorithm>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kTpThreads = 256;
constexpr int kTpPerLane = 32;     // rows of up to 2048 key blocks: 32 slots a lane
constexpr int kMinHistRows = 8;    // rows of one head per histogram workgroup, at least
constexpr int kBatch = 8;          // loads a thread issues before it uses them
constexpr int kNormRows = 16;      // pooled value rows per norm workgroup
constexpr int kMaxHeads = 4096;    // heads of a batch element (head entropies in LDS)

struct PoolState {
  unsigned long long bins[4][256];   // integer bin masses of each radix pass
};

__device__ __forceinline__ uint32_t okey(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long fixed_mass(float s) {
  return (unsigned long long)floor((double)s * 4294967296.0) + 1ull;
}

struct Ws {
  double* row_ent;        // [BH * nqb]
  double* head_ent;       // [BH]
  int32_t* pool;          // [BH]
  float* vnorm;           // [BH * vstride]
  PoolState* ps;          // [npools]
};

__device__ __forceinline__ Ws ws_of(const TopPArgs& a) {
  char* p = reinterpret_cast<char*>(a.ws);
  Ws w;
  w.row_ent = reinterpret_cast<double*>(p);
  p += sizeof(double) * (size_t)a.BH * a.nqb;
  w.head_ent = reinterpret_cast<double*>(p);
  p += sizeof(double) * (size_t)a.BH;
  w.pool = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * (size_t)((a.BH + 3) / 4 * 4);
  w.vnorm = reinterpret_cast<float*>(p);
  p += sizeof(float) * (size_t)a.BH * ((a.nkb + 3) / 4 * 4);
  w.ps = reinterpret_cast<PoolState*>(p);
  return w;
}

// Correctly rounded square root of x >= 0.  The compiler's root may be the
// hardware's approximate one; it is moved to the float whose rounding
// interval holds sqrt(x), decided exactly in double: a midpoint of two
// adjacent floats has at most 25 significant bits, so its square is exact.
__device__ __forceinline__ float sqrt_rn(float x) {
  float s = __builtin_sqrtf(x);
  const double xd = (double)x;
  for (int it = 0; it < 3; ++it) {
    const uint32_t u = __float_as_uint(s);
    const double d = (double)s;
    const double hi = 0.5 * (d + (double)__uint_as_float(u + 1u));
    if (xd >= hi * hi) {
      s = __uint_as_float(u + 1u);
    } else if (u > 0u) {
      const double lo = 0.5 * (d + (double)__uint_as_float(u - 1u));
      if (xd < lo * lo) s = __uint_as_float(u - 1u);
    }
  }
  return s;
}

// Norms of kNormRows pooled value rows: the rows are staged in LDS by the
// whole workgroup (coalesced), then one thread per row sums its squares in
// ascending channel order.
__device__ void value_norms(const TopPArgs& a, const Ws& w, int g) {
  __shared__ float rows[kNormRows * (128 + 1)];
  const int D = a.D, ld = D + 1;
  const int64_t e0 = (int64_t)g * kNormRows;                 // first row: bh * nkb + j
  const int64_t nrows = (int64_t)a.BH * a.nkb;
  const int nr = (int)min((int64_t)kNormRows, nrows - e0);
  const float4* src = reinterpret_cast<const float4*>(a.vp + e0 * D);
  for (int c = threadIdx.x; c < nr * D / 4; c += kTpThreads) {
    const float4 x = src[c];
    const int r = (4 * c) / D, d = (4 * c) % D;
    float* dst = rows + r * ld + d;
    dst[0] = x.x;
    dst[1] = x.y;
    dst[2] = x.z;
    dst[3] = x.w;
  }
  __syncthreads();
  if ((int)threadIdx.x < nr) {
    const float* v = rows + threadIdx.x * ld;
    float acc = 0.0f;
    for (int d = 0; d < D; ++d) acc = __fadd_rn(acc, __fmul_rn(v[d], v[d]));
    const int64_t e = e0 + threadIdx.x;
    const int bh = (int)(e / a.nkb), j = (int)(e % a.nkb);
    w.vnorm[(int64_t)bh * a.vstride + j] = sqrt_rn(acc);
  }
}

// Natural log of a positive normal double.  x = 2^e m with m in
// [sqrt(1/2), sqrt(2)); log m = 2 atanh(f) with f = (m - 1) / (m + 1), summed
// as its odd power series 2 (f + f^3/3 + f^5/5 + ...) -- |f| <= 0.172, so
// eleven terms reach double precision -- and e ln 2 is added in two parts
// (ln 2 to 32 significant bits, exact when multiplied by e, and the rest).
// Within a few ulps of the correctly rounded log.
__device__ __forceinline__ double log_pos(double x) {
  int e;
  double m = frexp(x, &e);                                   // m in [1/2, 1)
  if (m < 0.70710678118654752440) {
    m *= 2.0;
    e -= 1;
  }
  const double f = (m - 1.0) / (m + 1.0);
  const double f2 = f * f;
  double p = 2.0 / 21.0;
#pragma unroll
  for (int k = 9; k >= 0; --k) p = fma(p, f2, 2.0 / (double)(2 * k + 1));
  constexpr double kLn2Hi = 0x1.62e42ff000000p-1, kLn2Lo = -0x1.718432a1b0e26p-35;
  const double ed = (double)e;
  return fma(ed, kLn2Hi, fma(ed, kLn2Lo, f * p));
}

// one wave per row; workgroups from ent_groups on compute value norms
__global__ __launch_bounds__(kTpThreads) void tp_row_entropy(TopPArgs a, int ent_groups) {
  const Ws w = ws_of(a);
  if ((int)blockIdx.x >= ent_groups) {                       // uniform per workgroup
    value_norms(a, w, (int)blockIdx.x - ent_groups);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kTpThreads / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.BH * a.nqb) return;                  // uniform per wave
  const float* s = a.scores + row * a.nkb;
  const double eps = (double)a.eps;
  double acc = 0.0;
  for (int j = lane; j < a.nkb; j += 64) {
    const double p = (double)s[j];
    acc -= p * log_pos(p + eps);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) w.row_ent[row] = acc;
}

// one workgroup per head: the mean of its row entropies
__global__ __launch_bounds__(kTpThreads) void tp_head_entropy(TopPArgs a) {
  __shared__ double red[kTpThreads];
  const Ws w = ws_of(a);
  const int bh = blockIdx.x;
  const double* r = w.row_ent + (int64_t)bh * a.nqb;
  double acc = 0.0;
  for (int i = threadIdx.x; i < a.nqb; i += kTpThreads) acc += r[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = kTpThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double e = red[0] / (double)a.nqb;
    w.head_ent[bh] = e;
    if (a.entropy_out) a.entropy_out[bh] = e;
  }
}

// one workgroup per batch element
__global__ __launch_bounds__(kTpThreads) void tp_pools(TopPArgs a) {
  __shared__ double hent[kMaxHeads];
  const Ws w = ws_of(a);
  const int b = blockIdx.x;
  const int H = a.H;
  for (int h = threadIdx.x; h < H; h += kTpThreads) hent[h] = w.head_ent[b * H + h];
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += kTpThreads) {
    int rank = 0;
    for (int o = 0; o < H; ++o) rank += (hent[o] < hent[h] || (hent[o] == hent[h] && o < h)) ? 1 : 0;
    const bool low = rank < H / 2;
    int pid;
    switch (a.domain) {
      case 1: pid = b * H + h; break;                          // per-head global
      case 2: pid = 2 * b + (low ? 0 : 1); break;              // grouped cross-head
      case 3: pid = b; break;                                  // all-head global
      case 4: pid = low ? b : -1; break;                       // EG-Sparse routing
      default: pid = -1; break;                                // per-row local
    }
    w.pool[b * H + h] = pid;
  }
  // clear the state of this batch element's pools
  int lo, hi;
  switch (a.domain) {
    case 1: lo = b * H; hi = b * H + H; break;
    case 2: lo = 2 * b; hi = 2 * b + 2; break;
    case 3: case 4: lo = b; hi = b + 1; break;
    default: lo = hi = 0; break;
  }
  for (int q = lo; q < hi; ++q) {
    unsigned long long* bins = &w.ps[q].bins[0][0];
    for (int d = threadIdx.x; d < 4 * 256; d += kTpThreads) bins[d] = 0ull;
  }
}

// Digit of one radix pass, by one wave: v[b] is the mass of digit 4 lane + b
// inside the current prefix group.  Suffix sums (mass of digits >= d); the
// digit is the largest d whose suffix reaches rem, and the mass of the larger
// digits leaves rem.  In the first pass the bins hold the whole domain, so
// their sum is its mass and rem starts at ceil(p * mass).
__device__ __forceinline__ int wave_digit(unsigned long long (&v)[4], unsigned long long& rem, bool first,
                                          double top_p, int lane) {
  v[2] += v[3];
  v[1] += v[2];
  v[0] += v[1];
  unsigned long long above = 0ull;                           // digits of the lanes above
  unsigned long long x = v[0];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_down(x, o, 64);
    if (lane + o < 64) {
      above += y;
      x += y;
    }
  }
  if (first) rem = (unsigned long long)ceil(top_p * (double)__shfl(x, 0, 64));
  // x: suffix from digit 4l on; above: from digit 4l + 4 on
  int dig = -1;
  unsigned long long past = 0ull;
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    const unsigned long long sb = v[b] + above;                        // digits >= 4l + b
    const unsigned long long sn = (b == 3 ? 0ull : v[b + 1]) + above;  // digits >= 4l + b + 1
    if (dig < 0 && sb >= rem && sn < rem) {
      dig = 4 * lane + b;
      past = sn;
    }
  }
  const uint64_t who = __ballot(dig >= 0);
  if (who == 0ull) return 0;                                 // only an empty domain (never a pool in use)
  const int src = (int)__builtin_ctzll(who);
  dig = __shfl(dig, src, 64);
  rem -= __shfl(past, src, 64);
  return dig;
}

// The order-key digits of a pool's threshold chosen by its first `passes`
// radix passes (every wave that needs them derives them from the bins).
__device__ __forceinline__ uint32_t pool_prefix(const TopPArgs& a, const PoolState* ps, int passes, int lane) {
  unsigned long long v[4][4];                                // every pass's bins, loaded together
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int b = 0; b < 4; ++b) v[d][b] = d < passes ? ps->bins[d][4 * lane + b] : 0ull;
  uint32_t prefix = 0u;
  unsigned long long rem = 0ull;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    if (d < passes) prefix |= (uint32_t)wave_digit(v[d], rem, d == 0, a.top_p, lane) << (24 - 8 * d);
  return prefix;
}

__global__ __launch_bounds__(kTpThreads) void tp_hist(TopPArgs a, int pass, int rows) {
  const int shift = 24 - 8 * pass;
  __shared__ unsigned long long bins[256];
  const Ws w = ws_of(a);
  const int groups = (a.nqb + rows - 1) / rows;
  const int bh = blockIdx.x / groups;
  const int i0 = (blockIdx.x % groups) * rows;
  const int pid = w.pool[bh];
  if (pid < 0) return;                                       // uniform: the head is in no pool
  PoolState* ps = w.ps + pid;
  const int t = threadIdx.x;
  const int i1 = min(i0 + rows, a.nqb);
  const int n = (i1 - i0) * a.nkb;                           // the rows' scores, contiguous
  const float* base = a.scores + ((int64_t)bh * a.nqb + i0) * a.nkb;
  const float* vn = w.vnorm + (int64_t)bh * a.vstride;
  // loads of a batch (elements past the rows read the last one and are
  // skipped): scores and, for value-aware scores, the key blocks' norms
  auto load = [&](int e0, float (&sv)[kBatch], float (&vv)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) sv[u] = base[min(e0 + kTpThreads * u + t, n - 1)];
    if (a.value_aware) {
      int j = (e0 + t) % a.nkb;                              // key block of element u
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        vv[u] = vn[j];
        j += kTpThreads;
        while (j >= a.nkb) j -= a.nkb;
      }
    }
  };
  float sv[kBatch], vv[kBatch];
  load(0, sv, vv);                                           // in flight while the digits are derived
  bins[t] = 0ull;
  const uint32_t prefix = pool_prefix(a, ps, pass, t & 63);
  __syncthreads();
  // most scores share their leading digits: a thread adds up a run of equal
  // digits itself and makes one LDS atomic per run (integer sums: exact in
  // any order)
  uint32_t cur = 256u;
  unsigned long long acc = 0ull;
  for (int e0 = 0; e0 < n; e0 += kTpThreads * kBatch) {
    float cs[kBatch], cv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      cs[u] = sv[u];
      cv[u] = vv[u];
    }
    if (e0 + kTpThreads * kBatch < n) load(e0 + kTpThreads * kBatch, sv, vv);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = e0 + kTpThreads * u + t;
      const float x = a.value_aware ? __fmul_rn(cs[u], cv[u]) : cs[u];
      const uint32_t k = okey(x);
      const bool match = e < n && (shift == 24 || ((k ^ prefix) >> (shift + 8)) == 0u);
      if (match) {
        const uint32_t b = (k >> shift) & 255u;
        if (b != cur) {
          if (acc) atomicAdd(&bins[cur], acc);
          cur = b;
          acc = 0ull;
        }
        acc += fixed_mass(x);
      }
    }
  }
  if (acc) atomicAdd(&bins[cur], acc);
  __syncthreads();
  const unsigned long long v = bins[t];
  if (v) atomicAdd(&ps->bins[pass][t], v);
}

// One row of tp_select with PER live slots per lane (64 * PER >= nkb).
// LDS operations of one wave complete in order; this waits for them and keeps
// the compiler from moving LDS accesses across it
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// floor(s * 2^32) + 1 for the score s >= 0 of an order key, in integers
// (the same value as fixed_mass: s = m * 2^(E - 150) with a 24-bit m)
__device__ __forceinline__ unsigned long long mass_of_key(uint32_t k) {
  const uint32_t u = k & 0x7fffffffu;                        // s >= 0: the key is u | 2^31
  const int E = (int)(u >> 23);
  if (E == 0) return 1ull;                                   // zero or subnormal
  const unsigned long long m = (unsigned long long)((u & 0x7fffffu) | 0x800000u);
  const int sh = E - 118;                                    // s * 2^32 = m * 2^sh
  if (sh >= 0) return sh <= 40 ? (m << sh) + 1ull : fixed_mass(__uint_as_float(u));
  return (sh > -24 ? (m >> (-sh)) : 0ull) + 1ull;
}

// the score of an order key
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The row's order keys stay in registers (PER < 16) or in this wave's LDS
// (krow, slot mm of lane l at mm * 64 + l): only the lane that wrote a slot
// reads it, so the LDS copy needs no synchronization.
template <int PER>
__device__ void select_row(const TopPArgs& a, const Ws& w, int bh, int64_t row, int i, int lane,
                           unsigned long long* bins, uint32_t* krow) {
  constexpr bool kLds = PER >= 16;
  const int n = a.nkb;
  const int pid = w.pool[bh];
  const bool pooled = pid >= 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint8_t* mrow = a.mask ? a.mask + row * n : nullptr;
  int32_t* irow = a.idx + row * n;
  const bool dense = a.frame0_first >= 0 && i >= a.frame0_first && i <= a.frame0_last;

  // order key of every slot; 0 (below every score's key) past the row.  The
  // loads are issued together (slots past the row read the row's last block)
  uint32_t kreg[kLds ? 1 : PER];
  uint32_t inrow = 0u;                                       // slots inside the row
  {
    const float* srow_g = a.scores + row * n;
    float sv[PER];
#pragma unroll
    for (int mm = 0; mm < PER; ++mm) sv[mm] = srow_g[min(lane + 64 * mm, n - 1)];
    if (pooled && a.value_aware) {
      const float* vn = w.vnorm + (int64_t)bh * a.vstride;
#pragma unroll
      for (int mm = 0; mm < PER; ++mm) sv[mm] = __fmul_rn(sv[mm], vn[min(lane + 64 * mm, n - 1)]);
    }
#pragma unroll
    for (int mm = 0; mm < PER; ++mm) {
      const bool in = lane + 64 * mm < n;
      const uint32_t k = in ? okey(sv[mm]) : 0u;
      inrow |= in ? 1u << mm : 0u;
      if constexpr (kLds) krow[mm * 64 + lane] = k;
      else kreg[mm] = k;
    }
  }
  auto key = [&](int mm) -> uint32_t {
    if constexpr (kLds) return krow[mm * 64 + lane];
    else return kreg[mm];
  };
  uint32_t T;
  if (pooled) {
    T = pool_prefix(a, w.ps + pid, 4, lane);
  } else {
    // the row's own threshold: a radix select over its order keys, four
    // 8-bit digits, with integer bin masses in this wave's LDS bins (the
    // same search as the pooled domains').  Pass p visits only the slots
    // that matched the digits of pass p - 1.
    unsigned long long rem = 0ull;
    T = 0u;
    uint32_t cand = inrow;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int b = 0; b < 4; ++b) bins[4 * lane + b] = 0ull;
      wave_lds_sync();
      // a lane adds up a run of equal digits itself and makes one atomic per run
      uint32_t cur = 256u, next = 0u;
      unsigned long long acc = 0ull;
      auto visit = [&](int mm, uint32_t k) {
        if (pass == 0 || ((k ^ T) >> (shift + 8)) == 0u) {
          next |= 1u << mm;
          const uint32_t b = (k >> shift) & 255u;
          if (b != cur) {
            if (acc) atomicAdd(&bins[cur], acc);
            cur = b;
            acc = 0ull;
          }
          acc += mass_of_key(k);
        }
      };
      if constexpr (kLds) {
        for (uint32_t m = cand; m != 0u; m &= m - 1u) {
          const int mm = __builtin_ctz(m);
          visit(mm, krow[mm * 64 + lane]);
        }
      } else {
#pragma unroll
        for (int mm = 0; mm < PER; ++mm)
          if ((cand >> mm) & 1u) visit(mm, kreg[mm]);
      }
      if (acc) atomicAdd(&bins[cur], acc);
      wave_lds_sync();
      // lane l holds digits 4l .. 4l + 3
      unsigned long long v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) v[b] = bins[4 * lane + b];
      T |= (uint32_t)wave_digit(v, rem, pass == 0, a.top_p, lane) << shift;
      cand = next;
      wave_lds_sync();                                       // the bins are cleared next
    }
  }
  // kept: score >= T; a pooled row left empty keeps its first largest block
  bool any = false;
#pragma unroll
  for (int mm = 0; mm < PER; ++mm) any = any || (((inrow >> mm) & 1u) && key(mm) >= T);
  const bool row_empty = !__any(any);
  int safe = -1;
  if (pooled && row_empty) {
    float best = -1.0f;
    int bj = n;
#pragma unroll
    for (int mm = 0; mm < PER; ++mm) {
      const int j = lane + 64 * mm;
      const float sv = key_score(key(mm));
      if (j < n && (sv > best || (sv == best && j < bj))) {
        best = sv;
        bj = j;
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float ob = __shfl_xor(best, s, 64);
      const int oj = __shfl_xor(bj, s, 64);
      if (ob > best || (ob == best && oj < bj)) {
        best = ob;
        bj = oj;
      }
    }
    safe = bj;
  }
  int run = 0;
#pragma unroll
  for (int mm = 0; mm < PER; ++mm) {
    const int j = lane + 64 * mm;
    if (64 * mm >= n) break;
    const bool in = j < n;
    bool sel = in && (dense || key(mm) >= T || j == safe || j <= a.text_last);
    const uint64_t bsel = __ballot(sel);
    const int pos = run + __popcll(bsel & below);
    if (in && mrow) mrow[j] = sel ? 1 : 0;
    if (sel) irow[pos] = j;
    run += __popcll(bsel);
  }
  if (lane == 0) a.cnt[row] = run;
}
template <int PER>
__global__ __launch_bounds__(kTpThreads) void tp_select(TopPArgs a) {
  __shared__ unsigned long long sel_bins[256 * (kTpThreads / 64)];
  __shared__ uint32_t sel_rows[PER >= 16 ? 64 * PER * (kTpThreads / 64) : 1];
  const Ws w = ws_of(a);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kTpThreads / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.BH * a.nqb) return;                  // uniform per wave
  const int bh = (int)(row / a.nqb);
  const int i = (int)(row % a.nqb);
  select_row<PER>(a, w, bh, row, i, lane, sel_bins + 256 * (threadIdx.x >> 6),
                  sel_rows + (PER >= 16 ? 64 * PER * (threadIdx.x >> 6) : 0));
}

}  // namespace

int64_t topp_workspace_bytes(int64_t BH, int64_t B, int64_t nqb, int64_t nkb) {
  const int64_t npools = BH > 2 * B ? BH : 2 * B;
  return (int64_t)sizeof(double) * BH * nqb + (int64_t)sizeof(double) * BH +
         (int64_t)sizeof(int32_t) * ((BH + 3) / 4 * 4) + (int64_t)sizeof(float) * BH * ((nkb + 3) / 4 * 4) +
         (int64_t)sizeof(PoolState) * npools;
}

hipError_t launch_topp(const TopPArgs& a, hipStream_t stream) {
  const unsigned wave_groups = (unsigned)(((int64_t)a.BH * a.nqb + 3) / 4);
  const unsigned norm_groups =
      a.value_aware && a.domain != 0 ? (unsigned)(((int64_t)a.BH * a.nkb + kNormRows - 1) / kNormRows) : 0u;
  hipLaunchKernelGGL(tp_row_entropy, dim3(wave_groups + norm_groups), dim3(kTpThreads), 0, stream, a,
                     (int)wave_groups);
  hipLaunchKernelGGL(tp_head_entropy, dim3((unsigned)a.BH), dim3(kTpThreads), 0, stream, a);
  hipLaunchKernelGGL(tp_pools, dim3((unsigned)a.B), dim3(kTpThreads), 0, stream, a);
  if (a.domain != 0) {
    // every workgroup of a pool adds its bins to the pool's with global
    // atomics, so a pool gets between 512 and 2048 workgroups: about one per
    // 16 K scores (enough loads in flight for large pools, few atomics on the
    // same bins for small ones)
    const int64_t heads = a.domain == 1 ? 1 : a.domain == 3 ? a.H : (a.H + 1) / 2;
    const int64_t groups = std::min<int64_t>(2048, std::max<int64_t>(512, heads * a.nqb * a.nkb / 16384));
    const int rows = (int)std::min<int64_t>(a.nqb, std::max<int64_t>(kMinHistRows, (heads * a.nqb + groups - 1) / groups));
    const unsigned hist_groups = (unsigned)((int64_t)a.BH * ((a.nqb + rows - 1) / rows));
    for (int pass = 0; pass < 4; ++pass)
      hipLaunchKernelGGL(tp_hist, dim3(hist_groups), dim3(kTpThreads), 0, stream, a, pass, rows);
  }
  const int per = (a.nkb + 63) / 64;
  if (per <= 1) hipLaunchKernelGGL(tp_select<1>, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
  else if (per <= 2) hipLaunchKernelGGL(tp_select<2>, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
  else if (per <= 4) hipLaunchKernelGGL(tp_select<4>, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
  else if (per <= 8) hipLaunchKernelGGL(tp_select<8>, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
  else if (per <= 16) hipLaunchKernelGGL(tp_select<16>, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
  else hipLaunchKernelGGL(tp_select<kTpPerLane>, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
