// Block logits, per-row selection, overrides and compaction on gfx950.
//
// Pages: "Attention matrix view: make only frame-0 query rows dense"
// (sec. 4 override formula, sec. 6 top-k first then frame-0 rows
// overwritten, sec. 7 text blocks always kept); "Competition Domains Matter
// ... (EG-Sparse)" (Eq. 2 cluster-size-weighted centroid softmax, the
// one-key-per-row safeguard); "AB-Attention" (TL;DR: blocks sampled in
// proportion to importance, reweighted by inverse inclusion probability).
//
// One workgroup (8 waves) takes R consecutive query blocks of one head (R
// is 8 or 4, chosen per launch so that the grid holds at least three
// workgroups per CU; at most 128 registers a lane and at most half a CU's
// LDS let two workgroups share a CU, so that one's selection overlaps the
// other's logits):
//   A. all 512 threads compute the R x nkb float32 logits into LDS, each
//      logit as a sequential non-fused multiply-add chain over D in
//      ascending order (the library's contract, so the integer decisions
//      that follow are bit-reproducible); a thread owns all R rows x JT key
//      blocks, so each q or k chunk it reads feeds several chains;
//   B. each wave then owns one row at a time: for top-k, the k-th largest
//      logit by a bitwise search over keys held in registers (rows of more
//      than 2048 blocks: a radix select with four 8-bit passes over a
//      per-wave LDS histogram), then a ballot-ordered compaction; for
//      sampling, exp / water-filling / Philox draws (one evaluation per four
//      blocks) / log-weights.  Frame-0 rows skip straight to "all blocks";
//      text columns are OR-ed in.
#include <atomic>

#include "bsa_internal.h"
#include "spec_math.h"

namespace bsa {
namespace {

constexpr int kMaskThreads = 512;
constexpr int kMaskWaves = kMaskThreads / 64;
constexpr int kMaxPerLane = 32;          // sampling: nkb <= 64 * 32
constexpr int kRegKeys = 64 * kMaxPerLane;   // top-k rows up to this length keep their keys in registers
constexpr size_t kMaskLdsCap = 160 * 1024;

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t order_key(float z) {
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

// ---- Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011) -------------------
// 128-bit product of two 64-bit words from four 32 x 32 -> 64 multiply-adds:
// with a = a1 2^32 + a0 and b likewise, t = a1 b0 + hi(a0 b0) and
// u = a0 b1 + lo(t) cannot overflow, and a b = (a1 b1 + hi(t) + hi(u)) 2^64
// + lo(u) 2^32 + lo(a0 b0).
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32), b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t t = (uint64_t)a1 * b0 + (p00 >> 32);
  const uint64_t u = (uint64_t)a0 * b1 + (uint32_t)t;
  lo = (u << 32) | (uint32_t)p00;
  hi = (uint64_t)a1 * b1 + (t >> 32) + (u >> 32);
}

// The four 64-bit output words of counter (c0, c1, 0, 0) under key (k0, 0).
__device__ __forceinline__ void philox4(uint64_t c0, uint64_t c1, uint64_t k0, uint64_t (&x)[4]) {
  const uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  const uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = c0, x1 = c1, x2 = 0, x3 = 0;
  uint64_t key0 = k0, key1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { key0 += kW0; key1 += kW1; }
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(kM0, x0, hi0, lo0);
    mulhilo64(kM1, x2, hi1, lo1);
    const uint64_t n0 = hi1 ^ x1 ^ key0, n2 = hi0 ^ x3 ^ key1;
    x0 = n0; x1 = lo1; x2 = n2; x3 = lo0;
  }
  x[0] = x0; x[1] = x1; x[2] = x2; x[3] = x3;
}

// ---- radix select of the k-th largest order key of a row ------------------
// Returns T (the k-th largest key) and `need`, the number of keys equal to T
// that belong to the top k (those with the lowest indices).
__device__ void radix_select(const float* zr, int n, int k, int* hist, uint32_t& T, int& need) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) hist[b] = 0;
    wave_lds_sync();
    for (int j = lane; j < n; j += 64) {
      const uint32_t key = order_key(zr[j]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    wave_lds_sync();
    // lane L holds bins 255-4L .. 252-4L (descending digit order)
    int c[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) { c[q] = hist[255 - 4 * lane - q]; s += c[q]; }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int excl = incl - s;
    int digit = 0, above = 0, run = excl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (run < need && run + c[q] >= need) { digit = 255 - 4 * lane - q; above = run; }
      run += c[q];
    }
    const uint64_t hit = __ballot(excl < need && incl >= need);
    const int src = __ffsll((unsigned long long)hit) - 1;
    digit = __shfl(digit, src, 64);
    above = __shfl(above, src, 64);
    need -= above;
    prefix |= (uint32_t)digit << shift;
    pmask |= 255u << shift;
    wave_lds_sync();
  }
  T = prefix;
}

// ---- top-k of a row whose order keys fit in registers ----------------------
// Slot mm of a lane holds block lane + 64 mm; empty slots hold 0, below the
// key of every finite logit.  The k-th largest key T is found bit by bit from
// the top: the largest T with at least k keys >= T, each count a sum of
// ballot popcounts.  The search stops early once exactly k keys are >= T
// (those are then the top k whatever the lower bits).  need = keys equal to
// T that belong to the top k, which are the lowest-index ones.  Then the
// ascending compaction, with the text columns OR-ed in.
template <int PER>
__device__ __forceinline__ void topk_row(const float* zr, int n, int k, int text_last, int lane, uint64_t below,
                                         uint8_t* mrow, int32_t* irow, float* wrow, int32_t* cnt_out) {
  uint32_t kk[PER];
#pragma unroll
  for (int mm = 0; mm < PER; ++mm) {
    const int j = lane + 64 * mm;
    kk[mm] = j < n ? order_key(zr[j]) : 0u;
  }
  uint32_t T = 0;
  if (k < n) {
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = T | (1u << b);
      int c = 0;
#pragma unroll
      for (int mm = 0; mm < PER; ++mm) c += __popcll(__ballot(kk[mm] >= cand));
      if (c >= k) {
        T = cand;
        if (c == k) break;
      }
    }
  }
  int gt = 0;
#pragma unroll
  for (int mm = 0; mm < PER; ++mm) gt += __popcll(__ballot(kk[mm] > T));
  const int need = k - gt;
  int run_eq = 0, run_sel = 0;
#pragma unroll
  for (int mm = 0; mm < PER; ++mm) {
    const int j = lane + 64 * mm;
    const bool in = j < n;
    const uint32_t key = kk[mm];
    const bool eq = in && key == T;
    const uint64_t beq = __ballot(eq);
    const int eq_rank = run_eq + __popcll(beq & below);
    bool sel = in && (key > T || (eq && eq_rank < need));
    if (in && j <= text_last) sel = true;
    const uint64_t bsel = __ballot(sel);
    const int pos = run_sel + __popcll(bsel & below);
    if (in && mrow) mrow[j] = sel ? 1 : 0;
    if (sel) {
      irow[pos] = j;
      if (wrow) wrow[pos] = 0.0f;
    }
    run_eq += __popcll(beq);
    run_sel += __popcll(bsel);
  }
  if (lane == 0) *cnt_out = run_sel;
}

// Logits of R query rows (q rows in LDS) against every key block: thread tid
// owns key blocks base + tid + jj * kMaskThreads for each pass `base`.  Each
// logit is the sequential non-fused chain over d ascending.  A thread's key
// row is read in 16-byte chunks kept PF chunks ahead of their use (one
// 128-byte line per key in flight when JT = 1).
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int R, int JT, int D>
__device__ __forceinline__ void logits_rows(const MaskArgs& a, const float* kbase, const float* q, float* zs,
                                            int n, int nrows, int tid) {
  constexpr int NC = D / 4;
  constexpr int PF = 8 / JT;
  for (int base = 0; base < n; base += kMaskThreads * JT) {
    float acc[R][JT];
    const f32x4_t* kr[JT];
#pragma unroll
    for (int jj = 0; jj < JT; ++jj) {
      const int j = min(base + tid + jj * kMaskThreads, n - 1);
      kr[jj] = reinterpret_cast<const f32x4_t*>(kbase + (int64_t)j * D);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][jj] = 0.0f;
    }
    f32x4_t ring[PF][JT];
#pragma unroll
    for (int c = 0; c < PF; ++c)
#pragma unroll
      for (int jj = 0; jj < JT; ++jj) ring[c][jj] = kr[jj][c];
#pragma nounroll
    for (int c0 = 0; c0 < NC; c0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int c = c0 + u;
        f32x4_t kv[JT];
#pragma unroll
        for (int jj = 0; jj < JT; ++jj) {
          kv[jj] = ring[u][jj];
          ring[u][jj] = kr[jj][min(c + PF, NC - 1)];   // past the row's end: a harmless reread
        }
        f32x4_t qc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) qc[r] = *reinterpret_cast<const f32x4_t*>(q + r * D + 4 * c);
        // the R x JT chains advance together, one component at a time
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int jj = 0; jj < JT; ++jj) acc[r][jj] = __fadd_rn(acc[r][jj], __fmul_rn(qc[r][e], kv[jj][e]));
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < JT; ++jj) {
      const int j = base + tid + jj * kMaskThreads;
      if (j < n) {
        const float lc = (j == n - 1) ? a.ln_last : a.ln_full;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r < nrows) {
            float z = __fmul_rn(acc[r][jj], a.scale);
            if (a.log_cluster) z = __fadd_rn(z, lc);
            if (z == 0.0f) z = 0.0f;                // -0 -> +0
            zs[r * n + j] = z;
          }
        }
      }
    }
  }
}

// LDS of one workgroup: the R x nkb logits, the R query rows and (top-k rows
// longer than kRegKeys only) one 256-bin histogram per wave.
__host__ __device__ constexpr size_t mask_lds_bytes(int R, int n, int D, bool radix) {
  return ((size_t)R * n + (size_t)R * D) * 4 + (radix ? (size_t)kMaskWaves * 256 * 4 : 0);
}

// R: query blocks per workgroup; JT: key blocks per thread in the logits
// phase (1 or 2); SAMPLE: the selection mode (a kernel per mode keeps the
// top-k kernel's registers free of the sampling state).
template <int R, int JT, bool SAMPLE>
__global__ __launch_bounds__(kMaskThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void mask_kernel(MaskArgs a) {
  constexpr int kMaxRows = R;
  extern __shared__ __attribute__((aligned(16))) float lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ngroups = (a.nqb + R - 1) / R;
  const int bh = blockIdx.x / ngroups;
  const int i0 = (blockIdx.x % ngroups) * R;
  const int nrows = min(R, a.nqb - i0);
  const int n = a.nkb;
  const int D = a.D;
  float* zs = lds;                                           // [R][n]
  float* qs = lds + (size_t)R * n;                           // [R][D]
  int* hist_all = reinterpret_cast<int*>(qs + (size_t)R * (a.imp ? 0 : D));   // [waves][256]

  // ---- A. logits (or the given importance rows) ---------------------------
  // Each thread owns all R rows x JT key blocks: every wave reads the same q
  // row chunk (an LDS broadcast) and its lanes' own k rows, so one 16-byte q
  // read feeds 4 JT products and one k read (the costly, scattered one) 4 R.
  // Rows past nrows see zero q rows and are not stored.
  if (a.imp) {
    // selection from a given importance matrix: its rows are the scores
    const float* src = a.imp + ((int64_t)bh * a.nqb + i0) * n;
    for (int e = tid; e < nrows * n; e += kMaskThreads) zs[e] = src[e];
  } else {
    const float* qsrc = a.qp + ((int64_t)bh * a.nqb + i0) * D;
    for (int e = tid; e < kMaxRows * D; e += kMaskThreads) qs[e] = e < nrows * D ? qsrc[e] : 0.0f;
    __syncthreads();
    const float* kbase = a.kp + (int64_t)bh * n * D;
    if (D == 128) logits_rows<R, JT, 128>(a, kbase, qs, zs, n, nrows, tid);
    else logits_rows<R, JT, 64>(a, kbase, qs, zs, n, nrows, tid);
  }
  __syncthreads();

  // ---- B. per-row selection ------------------------------------------------
  int* hist = hist_all + wave * 256;
  const uint64_t below = lanes_below();
  for (int r = wave; r < nrows; r += kMaskWaves) {
    const int i = i0 + r;
    const int64_t rowid = (int64_t)bh * a.nqb + i;
    uint8_t* mrow = a.mask ? a.mask + rowid * n : nullptr;
    int32_t* irow = a.idx + rowid * n;
    float* wrow = a.logw ? a.logw + rowid * n : nullptr;
    const bool dense = a.frame0_first >= 0 && i >= a.frame0_first && i <= a.frame0_last;
    if (dense) {
      for (int j = lane; j < n; j += 64) {
        if (mrow) mrow[j] = 1;
        irow[j] = j;
        if (wrow) wrow[j] = 0.0f;
      }
      if (lane == 0) a.cnt[rowid] = n;
      continue;
    }
    const float* zr = zs + r * n;

    if (!SAMPLE && n <= kRegKeys) {
      int P = 64;
      while (P < n) P <<= 1;
      int32_t* co = a.cnt + rowid;
      switch (P / 64) {
        case 1: topk_row<1>(zr, n, a.topk, a.text_last, lane, below, mrow, irow, wrow, co); break;
        case 2: topk_row<2>(zr, n, a.topk, a.text_last, lane, below, mrow, irow, wrow, co); break;
        case 4: topk_row<4>(zr, n, a.topk, a.text_last, lane, below, mrow, irow, wrow, co); break;
        case 8: topk_row<8>(zr, n, a.topk, a.text_last, lane, below, mrow, irow, wrow, co); break;
        case 16: topk_row<16>(zr, n, a.topk, a.text_last, lane, below, mrow, irow, wrow, co); break;
        default: topk_row<32>(zr, n, a.topk, a.text_last, lane, below, mrow, irow, wrow, co); break;
      }
      continue;
    }
    if (!SAMPLE) {
      // rows longer than the register budget: radix select over LDS
      uint32_t T;
      int need;
      radix_select(zr, n, a.topk, hist, T, need);
      int run_eq = 0, run_sel = 0;
      for (int base = 0; base < n; base += 64) {
        const int j = base + lane;
        const bool in = j < n;
        const uint32_t key = in ? order_key(zr[j]) : 0u;
        const bool eq = in && key == T;
        const uint64_t beq = __ballot(eq);
        const int eq_rank = run_eq + __popcll(beq & below);
        bool sel = in && (key > T || (eq && eq_rank < need));
        if (in && j <= a.text_last) sel = true;
        const uint64_t bsel = __ballot(sel);
        const int pos = run_sel + __popcll(bsel & below);
        if (in && mrow) mrow[j] = sel ? 1 : 0;
        if (sel) {
          irow[pos] = j;
          if (wrow) wrow[pos] = 0.0f;
        }
        run_eq += __popcll(beq);
        run_sel += __popcll(bsel);
      }
      if (lane == 0) a.cnt[rowid] = run_sel;
      continue;
    }

    // ---- sampling ----------------------------------------------------------
    // max and first argmax of z
    float m = -INFINITY;
    int am = n;
    for (int j = lane; j < n; j += 64) {
      const float z = zr[j];
      if (z > m) { m = z; am = j; }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float om = __shfl_xor(m, s, 64);
      const int oa = __shfl_xor(am, s, 64);
      if (om > m || (om == m && oa < am)) { m = om; am = oa; }
    }
    // e_j, element j = lane + 64*mm
    int P = 64;
    while (P < n) P <<= 1;
    const int per = P / 64;
    float e[kMaxPerLane];
#pragma unroll
    for (int mm = 0; mm < kMaxPerLane; ++mm) {
      const int j = lane + 64 * mm;
      // weights in proportion to exp(z - max z), or the given importance
      e[mm] = (mm < per && j < n) ? (a.imp ? zr[j] : exp_le0(__fsub_rn(zr[j], m))) : 0.0f;
    }
    const float E = a.expected;
    uint32_t cap = 0;
    float c = 0.0f;
    const bool all_in = (double)E >= (double)n;
    if (!all_in) {
      int ncap = 0;
      for (int iter = 0; iter <= n + 1; ++iter) {
        float v[kMaxPerLane];
#pragma unroll
        for (int mm = 0; mm < kMaxPerLane; ++mm) v[mm] = ((cap >> mm) & 1u) ? 0.0f : e[mm];
        // halves-folding tree: in-lane levels, then across lanes
#pragma unroll
        for (int h = kMaxPerLane / 2; h >= 1; h >>= 1) {
          if (h < per) {
#pragma unroll
            for (int mm = 0; mm < h; ++mm) v[mm] = __fadd_rn(v[mm], v[mm + h]);
          }
        }
        float sig = v[0];
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) {
          const float o = __shfl_down(sig, s, 64);
          if (lane < s) sig = __fadd_rn(sig, o);
        }
        sig = __shfl(sig, 0, 64);
        const float num = __fsub_rn(E, (float)ncap);
        c = (num > 0.0f && sig > 0.0f) ? __fdiv_rn(num, sig) : 0.0f;
        uint32_t grown = cap;
#pragma unroll
        for (int mm = 0; mm < kMaxPerLane; ++mm)
          if (__fmul_rn(c, e[mm]) >= 1.0f) grown |= 1u << mm;
        if (!__any(grown != cap)) break;
        cap = grown;
        ncap = wave_sum_int(__popc(cap));
      }
    }
    // draws: counter j / 4 gives the top 24 bits of word j % 4 for block j;
    // one Philox evaluation per counter, the draws staged (as 24-bit integers,
    // exact in float) in the row's logit slots, which are no longer needed:
    // e holds what follows from them
    float* ur = zs + r * n;
    for (int cc = lane; cc < (n + 3) / 4; cc += 64) {
      uint64_t x[4];
      philox4((uint64_t)rowid, (uint64_t)cc, a.seed, x);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (4 * cc + w < n) ur[4 * cc + w] = (float)(uint32_t)(x[w] >> 40);
    }
    wave_lds_sync();
    // pi_j = 1 for capped blocks (and all of a row with E >= n), else c e_j;
    // recomputed where needed rather than held, to keep registers free
    auto pi_of = [&](int mm) { return (all_in || ((cap >> mm) & 1u)) ? 1.0f : __fmul_rn(c, e[mm]); };
    // draws
    uint32_t selbits = 0, forced = 0;
#pragma unroll
    for (int mm = 0; mm < kMaxPerLane; ++mm) {
      const int j = lane + 64 * mm;
      if (mm < per && j < n) {
        const float u = ur[j] * 5.9604644775390625e-08f;   // 2^-24
        if (u < pi_of(mm)) selbits |= 1u << mm;
      }
    }
    const bool any_sel = __any(selbits != 0);
    if (!any_sel && (am & 63) == lane) {
      // safeguard block: kept with weight 0
      selbits |= 1u << (am >> 6);
      forced = 1u << (am >> 6);
    }
    int run_sel = 0;
#pragma unroll
    for (int mm = 0; mm < kMaxPerLane; ++mm) {
      if (mm < per) {
        const int j = lane + 64 * mm;
        const bool in = j < n;
        bool sel = in && ((selbits >> mm) & 1u);
        const float pim = ((forced >> mm) & 1u) ? 1.0f : pi_of(mm);
        float w = (sel && pim < 1.0f) ? -logf(pim) : 0.0f;
        if (in && j <= a.text_last) { sel = true; w = 0.0f; }
        const uint64_t bsel = __ballot(sel);
        const int pos = run_sel + __popcll(bsel & below);
        if (in && mrow) mrow[j] = sel ? 1 : 0;
        if (sel) {
          irow[pos] = j;
          wrow[pos] = w;
        }
        run_sel += __popcll(bsel);
      }
    }
    if (lane == 0) a.cnt[rowid] = run_sel;
  }
}

}  // namespace

namespace {

constexpr int kMaxDevices = 64;
std::atomic<uint32_t> g_mask_lds_raised[kMaxDevices];   // per device: bit per (R, JT)

template <int R, int JT, bool SAMPLE>
hipError_t launch_rj(const MaskArgs& a, size_t lds, unsigned grid, hipStream_t stream) {
  if (lds > 64 * 1024) {   // above the default dynamic LDS limit: raise it once per device
    const void* f = reinterpret_cast<const void*>(&mask_kernel<R, JT, SAMPLE>);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint32_t bit = 1u << (4 * (SAMPLE ? 1 : 0) + 2 * (R == 8 ? 1 : 0) + (JT == 1 ? 0 : 1));
    const bool known = dev >= 0 && dev < kMaxDevices;
    if (!known || !(g_mask_lds_raised[dev].load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaskLdsCap);
      if (e != hipSuccess) return e;
      if (known) g_mask_lds_raised[dev].fetch_or(bit, std::memory_order_release);
    }
  }
  hipLaunchKernelGGL((mask_kernel<R, JT, SAMPLE>), dim3(grid), dim3(kMaskThreads), lds, stream, a);
  return hipGetLastError();
}

template <int R, bool SAMPLE>
hipError_t launch_rs(const MaskArgs& a, int jt, size_t lds, unsigned grid, hipStream_t stream) {
  if (jt == 2) return launch_rj<R, 2, SAMPLE>(a, lds, grid, stream);
  return launch_rj<R, 1, SAMPLE>(a, lds, grid, stream);
}

template <int R>
hipError_t launch_r(const MaskArgs& a, int jt, size_t lds, unsigned grid, hipStream_t stream) {
  return a.mode == 1 ? launch_rs<R, true>(a, jt, lds, grid, stream) : launch_rs<R, false>(a, jt, lds, grid, stream);
}

}  // namespace

hipError_t launch_mask(const MaskArgs& a, hipStream_t stream) {
  const bool radix = a.mode == 0 && a.nkb > kRegKeys;
  const int D = a.imp ? 0 : a.D;
  // rows per workgroup: eight (each key-row read feeds R logits) if the grid
  // still holds three workgroups per CU and two fit a CU's LDS; else four
  int R = 4;
  for (int r : {8}) {
    const int64_t groups = (int64_t)a.BH * ((a.nqb + r - 1) / r);
    if (groups >= 3 * 256 && mask_lds_bytes(r, a.nkb, D, radix) <= kMaskLdsCap / 2) { R = r; break; }
  }
  const size_t lds = mask_lds_bytes(R, a.nkb, D, radix);
  if (lds > kMaskLdsCap) return hipErrorInvalidValue;
  const int ngroups = (a.nqb + R - 1) / R;
  const int64_t grid = (int64_t)a.BH * ngroups;
  // key blocks per thread: the fewest passes x JT (per-lane work), ties to
  // the larger JT (fewer q reads per product).  Splitting a workgroup's rows
  // over thread groups (fewer rows, more key blocks per thread) measured
  // slower at every shape tried: it multiplies the scattered k reads.
  int jt = 1, best = 1 << 30;
  for (int t : {1, 2}) {
    const int work = ((a.nkb + kMaskThreads * t - 1) / (kMaskThreads * t)) * t;
    if (work <= best) { best = work; jt = t; }
  }
  if (R == 8) return launch_r<8>(a, jt, lds, (unsigned)grid, stream);
  return launch_r<4>(a, jt, lds, (unsigned)grid, stream);
}

}  // namespace bsa
