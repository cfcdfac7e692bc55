// Intra-block clustering selector on gfx950: block importance from k-means
// representatives of each query block.
//
// Page: "AB-Attention: accurate block-sparse attention for video diffusion"
// (TL;DR item 1 and the flowchart's intra-block cluster box: the queries of a
// query block are clustered only inside the block, without permuting tokens,
// and the representatives give the importance of every key block); the
// cluster-size-weighted softmax of a representative over the key-block
// summaries is Eq. 2 (P') of "Competition Domains Matter ... (EG-Sparse)".
//
// One workgroup (8 waves) per G consecutive query blocks of one head, with
// G * C <= 16 centroid rows:
//   1. for each block in turn: its valid query tokens go to LDS as float32
//      (rows padded by four floats, so a thread per token reads 16-byte
//      chunks without bank conflicts), then Lloyd k-means: centroid c starts at token
//      floor(c n / C); each round assigns every token (one thread per
//      (token, cluster) distance, a sequential non-fused chain over the
//      channels; the lowest cluster among equals) and replaces every
//      non-empty centroid by the mean of its tokens (one thread per
//      (cluster, channel) walks the cluster's member set, a 64-bit ballot of
//      the assignment, in ascending token order); a final assignment gives
//      the cluster sizes;
//   2. logits of every centroid of the group against every key-block summary
//      (the same chain as the block logits of the mask): a thread owns all
//      the group's centroid rows (8 or 16) x JT key blocks, so each summary
//      read from L2 feeds that many chains and each centroid read is an LDS
//      broadcast;
//   3. per non-empty centroid row, one wave: row max, e = exp(z - max) by the
//      fixed-order exponential, the sum by a halving tree over the row padded
//      to a power of two (pairs k, k + h at every level; the levels of 64 and
//      more inside each lane's registers, the rest by lane shuffles);
//   4. the importance of every block: fl32(w p) with p = e / sum and
//      w = m_c / n accumulated over its clusters in ascending order.
// Every operation is a single float32 rounding in a fixed order, so the
// importance (and the selection that ranks it) is reproducible bit for bit.
#include <atomic>

#include "bsa_internal.h"
#include "spec_math.h"

namespace bsa {
namespace {

constexpr int kImpThreads = 512;
constexpr int kImpWaves = kImpThreads / 64;
constexpr int kImpRows = 16;    // centroid rows of a workgroup
constexpr int kImpZMax = 16384; // logits of a workgroup (G * C * nkb)
constexpr int kImpPrefetch = 64 * 128 / kImpThreads;   // token elements per thread (q_block * D <= 8192)
constexpr int kMembWords = 1;   // 64-token words of a cluster's member set (q_block is 32 or 64)
constexpr int kImpMaxC = 16;    // clusters per block (G * C <= 16)

// Sum of e_k = exp(z_k - mx) over a row of nkb logits by the halving tree
// over the row padded to P (a power of two, P >= 2): level h adds k and
// k + h for every k < h.  The first level computes the exponentials and
// writes them back over the logits.  Lane l keeps the level-(P/2) values
// k = l + 64 m (m < M) in registers, so every level h >= 64 stays inside the
// lane; the levels below 64 go through lane shuffles.  Wave-uniform call.
template <int M>
__device__ float row_tree_sum(float* zr, int nkb, int P, float mx, int lane) {
  const int h0 = P / 2;
  float V[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int k = lane + 64 * m;
    float v = 0.0f;
    if (k < h0) {
      const float e0 = k < nkb ? exp_le0(__fsub_rn(zr[k], mx)) : 0.0f;
      const float e1 = k + h0 < nkb ? exp_le0(__fsub_rn(zr[k + h0], mx)) : 0.0f;
      if (k < nkb) zr[k] = e0;
      if (k + h0 < nkb) zr[k + h0] = e1;
      v = __fadd_rn(e0, e1);
    }
    V[m] = v;
  }
#pragma unroll
  for (int hh = M / 2; hh >= 1; hh >>= 1)
#pragma unroll
    for (int m = 0; m < hh; ++m) V[m] = __fadd_rn(V[m], V[m + hh]);
  float v = V[0];
  for (int h = (h0 < 64 ? h0 : 64) / 2; h >= 1; h >>= 1) {
    const float o = __shfl_down(v, h, 64);
    if (lane < h) v = __fadd_rn(v, o);
  }
  return __shfl(v, 0, 64);
}

// Logits of the group's first RR centroid rows (zero rows unused) against
// the key-block summaries: a thread owns all rows x JT key blocks, each logit
// a sequential non-fused chain over the D channels in ascending order.  The
// summaries stream through a ring of registers PF chunks ahead; the
// centroid chunks are LDS broadcasts at compile-time offsets.
template <int JT, int D, int RR>
__device__ __forceinline__ void centroid_logits(const ImpArgs& a, const float* kbase, const float* mu_all, float* zs,
                                                int nkb, int R, int tid) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int NC = D / 4;
  constexpr int PF = RR * JT >= 64 ? 1 : 8 / JT;   // chunks ahead (64 chains: the registers are spent)
  for (int base = 0; base < nkb; base += kImpThreads * JT) {
    float acc[RR][JT];
    const f32x4_t* kr[JT];
#pragma unroll
    for (int jj = 0; jj < JT; ++jj) {
      const int j = min(base + tid + jj * kImpThreads, nkb - 1);
      kr[jj] = reinterpret_cast<const f32x4_t*>(kbase + (int64_t)j * D);
#pragma unroll
      for (int r = 0; r < RR; ++r) acc[r][jj] = 0.0f;
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
#pragma unroll
        for (int r = 0; r < RR; ++r) {
          const f32x4_t m = *reinterpret_cast<const f32x4_t*>(mu_all + r * D + 4 * c);
#pragma unroll
          for (int jj = 0; jj < JT; ++jj) {
            float t = acc[r][jj];
            t = __fadd_rn(t, __fmul_rn(m[0], kv[jj][0]));
            t = __fadd_rn(t, __fmul_rn(m[1], kv[jj][1]));
            t = __fadd_rn(t, __fmul_rn(m[2], kv[jj][2]));
            t = __fadd_rn(t, __fmul_rn(m[3], kv[jj][3]));
            acc[r][jj] = t;
          }
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < JT; ++jj) {
      const int j = base + tid + jj * kImpThreads;
      if (j < nkb) {
        const float lc = (j == nkb - 1) ? a.ln_last : a.ln_full;
#pragma unroll
        for (int r = 0; r < RR; ++r) {
          if (r < R) {
            float z = __fmul_rn(acc[r][jj], a.scale);
            if (a.log_cluster) z = __fadd_rn(z, lc);
            if (z == 0.0f) z = 0.0f;                  // -0 -> +0
            zs[r * nkb + j] = z;
          }
        }
      }
    }
  }
}

template <typename T, int JT>
__global__ __launch_bounds__(kImpThreads) void importance_kernel(ImpArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ __attribute__((aligned(16))) float mu_all[kImpRows * 128];   // centroids of the group, zero rows unused
  __shared__ int msz_all[kImpRows];                   // cluster sizes (0: empty or c >= C_eff)
  __shared__ int n_all[kImpRows];                     // valid tokens of each block
  __shared__ float zsum[kImpRows];                    // row sums of e
  __shared__ uint64_t memb[kImpMaxC][kMembWords];     // tokens of each cluster of the current block
  __shared__ uint64_t memb_prev[kImpMaxC][kMembWords];   // the same after the assignment before
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int D = a.D;
  const int DP = D + 4;                               // token row stride: 16-byte rows, no bank conflicts
  const int nkb = a.nkb;
  const int C = a.C;
  const int ngroups = (a.nqb + a.G - 1) / a.G;
  const int bh = blockIdx.x / ngroups;
  const int i0 = (blockIdx.x % ngroups) * a.G;
  const int nblk = min(a.G, a.nqb - i0);

  // area A: the tokens of one block during k-means, then the logit rows
  float* xs = lds;                                    // [q_block][D + 4]
  float* zs = lds;                                    // [G * C][nkb]
  float* dist = lds + a.area_a + a.q_block;          // [C][q_block] (after q_block spare words)

  for (int e = tid; e < kImpRows * 128; e += kImpThreads) mu_all[e] = 0.0f;
  if (tid < kImpRows) msz_all[tid] = 0;
  __syncthreads();

  // ---- 1. k-means of every block of the group, one block at a time ----
  // The tokens of the next block are loaded into registers while this one
  // is clustered (a thread holds elements tid + k * kImpThreads).
  auto block_tokens = [&](int g) {
    const int64_t lo = (int64_t)(i0 + g) * a.q_block;
    return reinterpret_cast<const T*>(a.q) + ((int64_t)bh * a.seq_alloc + lo) * D;
  };
  auto block_n = [&](int g) { return (int)min((int64_t)a.q_block, a.S - (int64_t)(i0 + g) * a.q_block); };
  // 16-byte chunks of a block's tokens, all of a thread's loads issued
  // together (chunks past the block read its first chunk and are dropped)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int kEpc = 16 / (int)sizeof(T);           // elements per chunk
  constexpr int kChunks = kImpPrefetch / kEpc;        // chunks per thread
  u32x4_t pre[kChunks];
  auto prefetch = [&](int g) {
    const u32x4_t* qb = reinterpret_cast<const u32x4_t*>(block_tokens(g));
    const int nc = block_n(g) * D / kEpc;
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int c = tid + k * kImpThreads;
      pre[k] = qb[c < nc ? c : 0];
    }
  };
  prefetch(0);
  for (int g = 0; g < nblk; ++g) {
    const int n = block_n(g);
    const int ce = min(C, n);
    float* mu = mu_all + g * C * D;
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int e = (tid + k * kImpThreads) * kEpc;   // first element of the chunk
      if (e < n * D) {
        float* dst = xs + (e / D) * DP + e % D;       // kEpc consecutive channels of one token
        if constexpr (sizeof(T) == 2) {
          const u32x4_t w = pre[k];
          *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                                        __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
          *reinterpret_cast<float4*>(dst + 4) = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                                            __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
        } else {
          const u32x4_t w = pre[k];
          *reinterpret_cast<float4*>(dst) =
              make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3]));
        }
      }
    }
    if (g + 1 < nblk) prefetch(g + 1);
    __syncthreads();
    for (int e = tid; e < ce * D; e += kImpThreads) {
      const int c = e / D, d = e % D;
      mu[e] = xs[((c * n) / ce) * DP + d];
    }
    __syncthreads();
    // distance of every (token, cluster) pair by its own thread, then the
    // nearest cluster of every token (lowest index among equals); with one
    // cluster every token is in it and no distance is needed
    // The assignment leaves, per cluster, the bit set of its tokens (bit t:
    // token t, n <= 64), written by ballot from the wave that took the tokens.
    auto assign = [&]() {
      if (ce > 1) {
        for (int e = tid; e < n * ce; e += kImpThreads) {
          const int t = e % n, c = e / n;
          const float* xr = xs + t * DP;
          const float* mr = mu + c * D;
          float acc = 0.0f;
#pragma unroll 4
          for (int d = 0; d < D; d += 4) {
            const float4 x4 = *reinterpret_cast<const float4*>(xr + d);
            const float4 m4 = *reinterpret_cast<const float4*>(mr + d);
            float df = __fsub_rn(x4.x, m4.x);
            acc = __fadd_rn(acc, __fmul_rn(df, df));
            df = __fsub_rn(x4.y, m4.y);
            acc = __fadd_rn(acc, __fmul_rn(df, df));
            df = __fsub_rn(x4.z, m4.z);
            acc = __fadd_rn(acc, __fmul_rn(df, df));
            df = __fsub_rn(x4.w, m4.w);
            acc = __fadd_rn(acc, __fmul_rn(df, df));
          }
          dist[e] = acc;
        }
        __syncthreads();
      }
      if (wave < kMembWords) {                        // tokens 64 wave + lane: nearest cluster (lowest among equals)
        const int t = tid;
        int best = -1;
        if (t < n) {
          best = 0;
          float bd = dist[t];
          for (int c = 1; c < ce; ++c) {
            const float v = dist[c * n + t];
            if (v < bd) {
              bd = v;
              best = c;
            }
          }
          if (ce == 1) best = 0;
        }
        for (int c = 0; c < ce; ++c) {
          const uint64_t bits = __ballot(best == c);
          if (lane == 0) {
            memb_prev[c][wave] = memb[c][wave];
            memb[c][wave] = bits;
          }
        }
      }
      __syncthreads();
    };
    // the members of cluster c in ascending token order (wave-uniform c)
    auto members = [&](int c, auto&& f) {
#pragma unroll
      for (int wd = 0; wd < kMembWords; ++wd) {
        uint64_t m = memb[c][wd];
        m = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(m >> 32)) << 32) |
            (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)m);
        while (m) {
          const int t = 64 * wd + (int)__builtin_ctzll(m);
          m &= m - 1;
          f(t);
        }
      }
    };
    auto size_of = [&](int c) {
      int m = 0;
#pragma unroll
      for (int wd = 0; wd < kMembWords; ++wd) m += __popcll(memb[c][wd]);
      return m;
    };
    // Lloyd's rounds end early once an assignment repeats the one before it:
    // the means of the same members are the same centroids, so every later
    // round would repeat it too (and the final assignment is this one)
    bool converged = false;
    for (int it = 0; it < a.T; ++it) {
      assign();
      if (it > 0) {
        bool same = true;                             // the same LDS words for every thread: uniform
        for (int c = 0; c < ce; ++c)
#pragma unroll
          for (int wd = 0; wd < kMembWords; ++wd) same = same && memb[c][wd] == memb_prev[c][wd];
        if (same) {
          converged = true;
          break;
        }
      }
      for (int e = tid; e < ce * D; e += kImpThreads) {
        const int c = e / D, d = e % D;                // c is the same across a wave (D is 64 or 128)
        // the members' channel d in ascending token order
        float acc = 0.0f;
        members(c, [&](int t) { acc = __fadd_rn(acc, xs[t * DP + d]); });
        const int m = size_of(c);
        if (m > 0) mu[e] = __fdiv_rn(acc, (float)m);
      }
      __syncthreads();
    }
    if (!converged) assign();
    if (tid < ce) msz_all[g * C + tid] = size_of(tid);
    if (tid == 0) n_all[g] = n;
    __syncthreads();                                  // xs and the member sets are reused by the next block
  }

  // ---- 2. logits of every centroid row against every key-block summary ----
  const int R = nblk * C;
  {
    const float* kbase = a.kp + (int64_t)bh * nkb * D;
    // a group of at most 8 centroid rows (G = 2 at long rows) computes only those
    if (a.G * C <= 8) {
      if (D == 128) centroid_logits<JT, 128, 8>(a, kbase, mu_all, zs, nkb, R, tid);
      else centroid_logits<JT, 64, 8>(a, kbase, mu_all, zs, nkb, R, tid);
    } else {
      if (D == 128) centroid_logits<JT, 128, kImpRows>(a, kbase, mu_all, zs, nkb, R, tid);
      else centroid_logits<JT, 64, kImpRows>(a, kbase, mu_all, zs, nkb, R, tid);
    }
  }
  __syncthreads();

  // ---- 3. softmax sums of every non-empty centroid row, one wave per row ----
  int P = 1;
  while (P < nkb) P <<= 1;
  for (int r = wave; r < R; r += kImpWaves) {
    if (msz_all[r] == 0) continue;                    // uniform per wave
    float* zr = zs + r * nkb;
    float mx = -INFINITY;
    for (int j = lane; j < nkb; j += 64) mx = fmaxf(mx, zr[j]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s, 64));   // max is exact in any order
    float Z;
    if (P == 1) {
      if (lane == 0) zr[0] = exp_le0(__fsub_rn(zr[0], mx));
      Z = __shfl(exp_le0(__fsub_rn(mx, mx)), 0, 64);
    } else {
      switch (P <= 128 ? 1 : P / 128) {
        case 1: Z = row_tree_sum<1>(zr, nkb, P, mx, lane); break;
        case 2: Z = row_tree_sum<2>(zr, nkb, P, mx, lane); break;
        case 4: Z = row_tree_sum<4>(zr, nkb, P, mx, lane); break;
        case 8: Z = row_tree_sum<8>(zr, nkb, P, mx, lane); break;
        case 16: Z = row_tree_sum<16>(zr, nkb, P, mx, lane); break;
        case 32: Z = row_tree_sum<32>(zr, nkb, P, mx, lane); break;
        default: Z = row_tree_sum<64>(zr, nkb, P, mx, lane); break;
      }
    }
    if (lane == 0) zsum[r] = Z;
  }
  __syncthreads();

  // ---- 4. importance: token-share-weighted sum over the clusters ----
  for (int e = tid; e < nblk * nkb; e += kImpThreads) {
    const int g = e / nkb, j = e % nkb;
    float imp = 0.0f;
    for (int c = 0; c < C; ++c) {
      const int r = g * C + c;
      const int m = msz_all[r];
      if (m == 0) continue;
      const float w = __fdiv_rn((float)m, (float)n_all[g]);
      imp = __fadd_rn(imp, __fmul_rn(w, __fdiv_rn(zs[r * nkb + j], zsum[r])));
    }
    a.imp[((int64_t)bh * a.nqb + i0 + g) * nkb + j] = imp;
  }
}

// The dynamic LDS cap of each importance kernel is raised once per device to
// the most any launch may ask for (the host refuses geometries needing more),
// so later calls make no runtime call besides the launch: they can be
// captured in a graph.
constexpr int kImpLdsCap = 96 * 1024;
constexpr int kMaxDevices = 64;
std::atomic<uint32_t> g_lds_cap_raised[kMaxDevices];   // per device: bit per (JT, dtype)

template <int JT>
hipError_t launch_jt(const ImpArgs& a, int dtype, size_t lds, unsigned grid, hipStream_t stream) {
  const void* f = dtype == 0 ? reinterpret_cast<const void*>(&importance_kernel<bf16_t, JT>)
                             : reinterpret_cast<const void*>(&importance_kernel<float, JT>);
  if (lds > (size_t)kImpLdsCap) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = 1u << (2 * (JT == 1 ? 0 : (JT == 2 ? 1 : 2)) + (dtype == 0 ? 0 : 1));
  const bool known = dev >= 0 && dev < kMaxDevices;
  if (!known || !(g_lds_cap_raised[dev].load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kImpLdsCap);
    if (e != hipSuccess) return e;
    if (known) g_lds_cap_raised[dev].fetch_or(bit, std::memory_order_release);
  }
  if (dtype == 0)
    hipLaunchKernelGGL((importance_kernel<bf16_t, JT>), dim3(grid), dim3(kImpThreads), lds, stream, a);
  else
    hipLaunchKernelGGL((importance_kernel<float, JT>), dim3(grid), dim3(kImpThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

// Query blocks per workgroup: more blocks share each key-summary read, but
// their k-means runs one block after another.  With one cluster k-means is
// only the mean, so up to 16 blocks; with more clusters at most 4 (measured
// on MI355X: C = 2 runs 10 % faster with 4 than with 8).
int importance_group(int C, int nkb, int nqb) {
  int g = kImpRows / C;
  if (C > 1 && g > 4) g = 4;
  const int zg = kImpZMax / (C * nkb);
  if (zg < g) g = zg;
  if (g > nqb) g = nqb;
  return g < 1 ? 1 : g;
}

size_t importance_lds_bytes(const ImpArgs& a) {
  const size_t tok = (size_t)a.q_block * (a.D + 4);
  const size_t z = (size_t)a.G * a.C * a.nkb;
  const size_t area = tok > z ? tok : z;
  return sizeof(float) * (area + (size_t)a.q_block + (size_t)a.C * a.q_block);
}

hipError_t launch_importance(const ImpArgs& a0, int dtype, hipStream_t stream) {
  ImpArgs a = a0;
  const size_t tok = (size_t)a.q_block * (a.D + 4);
  const size_t z = (size_t)a.G * a.C * a.nkb;
  a.area_a = (int32_t)(tok > z ? tok : z);
  const size_t lds = importance_lds_bytes(a);
  const unsigned grid = (unsigned)((int64_t)a.BH * ((a.nqb + a.G - 1) / a.G));
  // key blocks per thread: the fewest passes x JT, ties to the larger JT
  int best = 1;
  int64_t cost = INT64_MAX;
  for (int t : {1, 2, 4}) {
    const int64_t c = (int64_t)((a.nkb + kImpThreads * t - 1) / (kImpThreads * t)) * t;
    if (c <= cost) {
      cost = c;
      best = t;
    }
  }
  if (best == 4) return launch_jt<4>(a, dtype, lds, grid, stream);
  if (best == 2) return launch_jt<2>(a, dtype, lds, grid, stream);
  return launch_jt<1>(a, dtype, lds, grid, stream);
}

}  // namespace bsa
