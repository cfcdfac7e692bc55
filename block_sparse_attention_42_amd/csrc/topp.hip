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
//   tp_row_entropy    one wave per row: sum_j -P log(P + eps) (float64)
//   tp_head_entropy   one workgroup per head: the mean over its rows
//   tp_pools          one workgroup per batch element: median split, pool of
//                     every head, pool state cleared
//   tp_value_norm     norm of every pooled value row (value-aware scores)
//   tp_row_total      one wave per pooled row: its mass
//   tp_pool_target    one workgroup per pool: total, target = ceil(p * total)
//   tp_hist, tp_digit (x4)  radix passes of the pooled thresholds: integer
//                     bin masses of 16 rows per workgroup, then per pool a
//                     suffix scan picks the digit
//   tp_select         one wave per row: threshold (the pool's, or its own
//                     radix select), safeguard, frame-0 rows, text columns,
//                     compaction
#include <type_traits>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kTpThreads = 256;
constexpr int kTpPerLane = 32;     // rows of up to 2048 key blocks in registers

struct PoolState {
  unsigned long long total, target, rem;
  uint32_t prefix, used;
  unsigned long long bins[256];
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
  unsigned long long* row_tot;   // [BH * nqb]
  double* head_ent;       // [BH]
  int32_t* pool;          // [BH]
  float* vnorm;           // [BH * nkb]
  PoolState* ps;          // [npools]
};

constexpr int kRowsPerHist = 16;   // rows of one head per histogram workgroup

__device__ __forceinline__ Ws ws_of(const TopPArgs& a) {
  char* p = reinterpret_cast<char*>(a.ws);
  Ws w;
  w.row_ent = reinterpret_cast<double*>(p);
  p += sizeof(double) * (size_t)a.BH * a.nqb;
  w.row_tot = reinterpret_cast<unsigned long long*>(p);
  p += sizeof(unsigned long long) * (size_t)a.BH * a.nqb;
  w.head_ent = reinterpret_cast<double*>(p);
  p += sizeof(double) * (size_t)a.BH;
  w.pool = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * (size_t)((a.BH + 1) / 2 * 2);
  w.vnorm = reinterpret_cast<float*>(p);
  p += sizeof(float) * (size_t)a.BH * ((a.nkb + 3) / 4 * 4);
  w.ps = reinterpret_cast<PoolState*>(p);
  return w;
}

// the ranking score of block j of a row of head bh
__device__ __forceinline__ float score_of(const TopPArgs& a, const Ws& w, int bh, int64_t row, int j, bool pooled) {
  const float s = a.scores[row * a.nkb + j];
  return (a.value_aware && pooled) ? __fmul_rn(s, w.vnorm[(int64_t)bh * a.vstride + j]) : s;
}

// one wave per row
__global__ __launch_bounds__(kTpThreads) void tp_row_entropy(TopPArgs a) {
  const Ws w = ws_of(a);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kTpThreads / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.BH * a.nqb) return;                  // uniform per wave
  const float* s = a.scores + row * a.nkb;
  const double eps = (double)a.eps;
  double acc = 0.0;
  for (int j = lane; j < a.nkb; j += 64) {
    const double p = (double)s[j];
    acc -= p * log(p + eps);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) w.row_ent[row] = acc;
}

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

__global__ __launch_bounds__(kTpThreads) void tp_pools(TopPArgs a) {
  const Ws w = ws_of(a);
  const int b = blockIdx.x;
  const int H = a.H;
  const double* hent = w.head_ent + (int64_t)b * H;
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
    PoolState* ps = w.ps + q;
    for (int d = threadIdx.x; d < 256; d += kTpThreads) ps->bins[d] = 0ull;
    if (threadIdx.x == 0) {
      ps->total = 0ull;
      ps->target = 0ull;
      ps->rem = 0ull;
      ps->prefix = 0u;
      ps->used = 0u;
    }
  }
}

__global__ __launch_bounds__(kTpThreads) void tp_value_norm(TopPArgs a) {
  const Ws w = ws_of(a);
  const int64_t e = (int64_t)blockIdx.x * kTpThreads + threadIdx.x;   // bh * nkb + j
  if (e >= (int64_t)a.BH * a.nkb) return;
  const int bh = (int)(e / a.nkb), j = (int)(e % a.nkb);
  const float* v = a.vp + e * a.D;
  // the loads are independent (16 bytes each, all issued up front); the sum
  // is the ascending-channel chain
  float acc = 0.0f;
  auto chain = [&](auto dn) {
    constexpr int DN = decltype(dn)::value;
    float4 x[DN / 4];
#pragma unroll
    for (int c = 0; c < DN / 4; ++c) x[c] = *reinterpret_cast<const float4*>(v + 4 * c);
#pragma unroll
    for (int c = 0; c < DN / 4; ++c) {
      acc = __fadd_rn(acc, __fmul_rn(x[c].x, x[c].x));
      acc = __fadd_rn(acc, __fmul_rn(x[c].y, x[c].y));
      acc = __fadd_rn(acc, __fmul_rn(x[c].z, x[c].z));
      acc = __fadd_rn(acc, __fmul_rn(x[c].w, x[c].w));
    }
  };
  if (a.D == 128) chain(std::integral_constant<int, 128>{});
  else chain(std::integral_constant<int, 64>{});
  w.vnorm[(int64_t)bh * a.vstride + j] = __fsqrt_rn(acc);
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

__global__ __launch_bounds__(kTpThreads) void tp_row_total(TopPArgs a) {
  const Ws w = ws_of(a);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kTpThreads / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.BH * a.nqb) return;                  // uniform per wave
  const int bh = (int)(row / a.nqb);
  if (w.pool[bh] < 0) return;
  unsigned long long acc = 0ull;
  for (int j = lane; j < a.nkb; j += 64) acc += fixed_mass(score_of(a, w, bh, row, j, true));
  acc = wave_sum_u64(acc);
  if (lane == 0) w.row_tot[row] = acc;
}

__global__ __launch_bounds__(kTpThreads) void tp_pool_target(TopPArgs a) {
  __shared__ unsigned long long red[kTpThreads];
  const Ws w = ws_of(a);
  const int q = blockIdx.x;
  unsigned long long acc = 0ull;
  int mine = 0;
  for (int bh = 0; bh < a.BH; ++bh) {
    if (w.pool[bh] != q) continue;                           // uniform
    const unsigned long long* rt = w.row_tot + (int64_t)bh * a.nqb;
    for (int i = threadIdx.x; i < a.nqb; i += kTpThreads) acc += rt[i];
    ++mine;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = kTpThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    PoolState* ps = w.ps + q;
    ps->used = mine > 0 ? 1u : 0u;
    ps->total = red[0];
    ps->target = (unsigned long long)ceil(a.top_p * (double)red[0]);
    ps->rem = ps->target;
    ps->prefix = 0u;
  }
}

__global__ __launch_bounds__(kTpThreads) void tp_hist(TopPArgs a, int shift) {
  __shared__ unsigned long long bins[256];
  const Ws w = ws_of(a);
  const int groups = (a.nqb + kRowsPerHist - 1) / kRowsPerHist;
  const int bh = blockIdx.x / groups;
  const int i0 = (blockIdx.x % groups) * kRowsPerHist;
  const int pid = w.pool[bh];
  if (pid < 0) return;
  bins[threadIdx.x] = 0ull;
  __syncthreads();
  const uint32_t prefix = w.ps[pid].prefix;
  const int i1 = min(i0 + kRowsPerHist, a.nqb);
  // most scores share their leading digits: a thread adds up a run of equal
  // digits itself and makes one LDS atomic per run (integer sums: exact in
  // any order)
  uint32_t cur = 256u;
  unsigned long long acc = 0ull;
  for (int i = i0; i < i1; ++i) {
    const int64_t row = (int64_t)bh * a.nqb + i;
    for (int j = threadIdx.x; j < a.nkb; j += kTpThreads) {
      const float s = score_of(a, w, bh, row, j, true);
      const uint32_t k = okey(s);
      const bool match = shift == 24 || ((k ^ prefix) >> (shift + 8)) == 0u;
      if (match) {
        const uint32_t b = (k >> shift) & 255u;
        if (b != cur) {
          if (acc) atomicAdd(&bins[cur], acc);
          cur = b;
          acc = 0ull;
        }
        acc += fixed_mass(s);
      }
    }
  }
  if (acc) atomicAdd(&bins[cur], acc);
  __syncthreads();
  const unsigned long long v = bins[threadIdx.x];
  if (v) atomicAdd(&w.ps[pid].bins[threadIdx.x], v);
}

// per pool: suffix sums of the bins (mass of digits >= d inside the current
// prefix group); the digit is the largest d whose suffix reaches the
// remaining target, and the mass of the larger digits leaves the target
__global__ __launch_bounds__(kTpThreads) void tp_digit(TopPArgs a, int shift) {
  __shared__ unsigned long long suf[257];
  const Ws w = ws_of(a);
  PoolState* ps = w.ps + blockIdx.x;
  if (!ps->used) return;                                     // uniform
  const int d = threadIdx.x;
  suf[d] = ps->bins[d];
  if (d == 0) suf[256] = 0ull;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {                        // suffix scan, integer: any order is exact
    const unsigned long long v = d + o < 256 ? suf[d + o] : 0ull;
    __syncthreads();
    suf[d] += v;
    __syncthreads();
  }
  const unsigned long long rem = ps->rem;
  __syncthreads();
  if (suf[d] >= rem && suf[d + 1] < rem) {
    ps->rem = rem - suf[d + 1];
    ps->prefix |= (uint32_t)d << shift;
  }
  ps->bins[d] = 0ull;
}

// One row of tp_select with PER live slots per lane (64 * PER >= nkb).
// LDS operations of one wave complete in order; this waits for them and keeps
// the compiler from moving LDS accesses across it
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The row's scores stay in registers (PER < 16) or in this wave's LDS
// (srow, slot mm of lane l at mm * 64 + l): only the lane that wrote a slot
// reads it, so the LDS copy needs no synchronization.
template <int PER>
__device__ void select_row(const TopPArgs& a, const Ws& w, int bh, int64_t row, int i, int lane,
                           unsigned long long* bins, float* srow) {
  constexpr bool kLds = PER >= 16;
  const int n = a.nkb;
  const int pid = w.pool[bh];
  const bool pooled = pid >= 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint8_t* mrow = a.mask ? a.mask + row * n : nullptr;
  int32_t* irow = a.idx + row * n;
  const bool dense = a.frame0_first >= 0 && i >= a.frame0_first && i <= a.frame0_last;

  float sreg[kLds ? 1 : PER];
#pragma unroll
  for (int mm = 0; mm < PER; ++mm) {
    const int j = lane + 64 * mm;
    const float v = j < n ? score_of(a, w, bh, row, j, pooled) : 0.0f;
    if constexpr (kLds) srow[mm * 64 + lane] = v;
    else sreg[mm] = v;
  }
  auto sc = [&](int mm) -> float {
    if constexpr (kLds) return srow[mm * 64 + lane];
    else return sreg[mm];
  };
  // order key of slot mm; 0 (below every score's key) past the row
  auto key = [&](int mm) { return lane + 64 * mm < n ? okey(sc(mm)) : 0u; };
  uint32_t T;
  if (pooled) {
    T = w.ps[pid].prefix;
  } else {
    // the row's own threshold: a radix select over its order keys, four
    // 8-bit digits, with integer bin masses in this wave's LDS bins (the
    // same search as the pooled domains')
    unsigned long long tot = 0ull;
#pragma unroll
    for (int mm = 0; mm < PER; ++mm)
      if (lane + 64 * mm < n) tot += fixed_mass(sc(mm));
    tot = wave_sum_u64(tot);
    unsigned long long rem = (unsigned long long)ceil(a.top_p * (double)tot);
    T = 0u;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int b = 0; b < 4; ++b) bins[4 * lane + b] = 0ull;
      wave_lds_sync();
      // a lane adds up a run of equal digits itself and makes one atomic per run
      uint32_t cur = 256u;
      unsigned long long acc = 0ull;
#pragma unroll
      for (int mm = 0; mm < PER; ++mm) {
        const bool match = lane + 64 * mm < n && (shift == 24 || ((key(mm) ^ T) >> (shift + 8)) == 0u);
        if (match) {
          const uint32_t b = (key(mm) >> shift) & 255u;
          if (b != cur) {
            if (acc) atomicAdd(&bins[cur], acc);
            cur = b;
            acc = 0ull;
          }
          acc += fixed_mass(sc(mm));
        }
      }
      if (acc) atomicAdd(&bins[cur], acc);
      wave_lds_sync();
      // suffix sums: lane l holds digits 4l .. 4l + 3
      unsigned long long v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) v[b] = bins[4 * lane + b];
      v[2] += v[3];
      v[1] += v[2];
      v[0] += v[1];
      unsigned long long above = 0ull;                       // digits of the lanes above
      unsigned long long x = v[0];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_down(x, o, 64);
        if (lane + o < 64) {
          above += y;
          x += y;
        }
      }
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
      const int src = (int)__builtin_ctzll(who);
      dig = __shfl(dig, src, 64);
      past = __shfl(past, src, 64);
      rem -= past;
      T |= (uint32_t)dig << shift;
      wave_lds_sync();                                       // the bins are cleared next
    }
  }
  // kept: score >= T; a pooled row left empty keeps its first largest block
  bool any = false;
#pragma unroll
  for (int mm = 0; mm < PER; ++mm) any = any || (lane + 64 * mm < n && key(mm) >= T);
  const bool row_empty = !__any(any);
  int safe = -1;
  if (pooled && row_empty) {
    float best = -1.0f;
    int bj = n;
#pragma unroll
    for (int mm = 0; mm < PER; ++mm) {
      const int j = lane + 64 * mm;
      if (j < n && (sc(mm) > best || (sc(mm) == best && j < bj))) {
        best = sc(mm);
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

// PER: slots per lane, 64 * PER >= nkb (a kernel per PER, so each gets its
// own register allocation)
template <int PER>
__global__ __launch_bounds__(kTpThreads) void tp_select(TopPArgs a) {
  __shared__ unsigned long long sel_bins[256 * (kTpThreads / 64)];
  __shared__ float sel_rows[PER >= 16 ? 64 * PER * (kTpThreads / 64) : 1];
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
  return (int64_t)sizeof(double) * BH * nqb + (int64_t)sizeof(unsigned long long) * BH * nqb +
         (int64_t)sizeof(double) * BH +
         (int64_t)sizeof(int32_t) * ((BH + 1) / 2 * 2) + (int64_t)sizeof(float) * BH * ((nkb + 3) / 4 * 4) +
         (int64_t)sizeof(PoolState) * npools;
}

hipError_t launch_topp(const TopPArgs& a, hipStream_t stream) {
  const unsigned wave_groups = (unsigned)(((int64_t)a.BH * a.nqb + 3) / 4);
  hipLaunchKernelGGL(tp_row_entropy, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
  hipLaunchKernelGGL(tp_head_entropy, dim3((unsigned)a.BH), dim3(kTpThreads), 0, stream, a);
  hipLaunchKernelGGL(tp_pools, dim3((unsigned)a.B), dim3(kTpThreads), 0, stream, a);
  if (a.value_aware) {
    const int64_t n = (int64_t)a.BH * a.nkb;
    hipLaunchKernelGGL(tp_value_norm, dim3((unsigned)((n + kTpThreads - 1) / kTpThreads)), dim3(kTpThreads), 0,
                       stream, a);
  }
  if (a.domain != 0) {
    hipLaunchKernelGGL(tp_row_total, dim3(wave_groups), dim3(kTpThreads), 0, stream, a);
    hipLaunchKernelGGL(tp_pool_target, dim3((unsigned)a.npools), dim3(kTpThreads), 0, stream, a);
    const unsigned hist_groups = (unsigned)((int64_t)a.BH * ((a.nqb + kRowsPerHist - 1) / kRowsPerHist));
    for (int shift = 24; shift >= 0; shift -= 8) {
      hipLaunchKernelGGL(tp_hist, dim3(hist_groups), dim3(kTpThreads), 0, stream, a, shift);
      hipLaunchKernelGGL(tp_digit, dim3((unsigned)a.npools), dim3(kTpThreads), 0, stream, a, shift);
    }
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
