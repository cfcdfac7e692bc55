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
// One workgroup (4 waves) per (b, h, query block):
//   1. the block's valid query tokens go to LDS as float32 (rows padded by
//      one float, so a thread per token reads without bank conflicts);
//   2. Lloyd k-means: centroid c starts at token floor(c n / C); each round
//      assigns every token (one thread per (token, cluster) distance, a
//      sequential non-fused chain over the channels; the lowest cluster
//      among equals) and replaces every non-empty centroid by the mean of
//      its tokens (one thread per (cluster, channel), ascending tokens); a
//      final assignment gives the cluster sizes;
//   3. logits of every centroid against every key-block summary (the same
//      chain as the block logits of the mask), the summaries staged through
//      LDS in chunks of 64 with coalesced loads, one thread per (key block,
//      cluster);
//   4. per non-empty cluster: row max, e = exp(z - max) by the fixed-order
//      exponential, the sum by a halving tree over the row padded to a
//      power of two (levels of 64 and more through LDS, the rest by lane
//      shuffles inside one wave, the same pairs), p = e / sum; the importance
//      accumulates fl32(w p) with w = m_c / n, clusters in ascending order.
// Every operation is a single float32 rounding in a fixed order, so the
// importance (and the selection that ranks it) is reproducible bit for bit.
#include "bsa_internal.h"
#include "spec_math.h"

namespace bsa {
namespace {

constexpr int kImpThreads = 256;
constexpr int kMaxClusters = 8;
constexpr int kMaxOwned = 32;   // key blocks per thread: nkb <= 8192
constexpr int kChunk = 64;      // key-block summaries per LDS chunk

template <typename T>
__device__ __forceinline__ float widen(const T* p, int64_t e);
template <>
__device__ __forceinline__ float widen<bf16_t>(const bf16_t* p, int64_t e) {
  return __uint_as_float((uint32_t)p[e].bits << 16);
}
template <>
__device__ __forceinline__ float widen<float>(const float* p, int64_t e) {
  return p[e];
}

// floats of the area that holds the tokens, then the key-block chunks
__host__ __device__ inline int tok_floats(int q_block, int D) {
  const int t = q_block * (D + 1), k = kChunk * (D + 4);
  return t > k ? t : k;
}

template <typename T>
__global__ __launch_bounds__(kImpThreads) void importance_kernel(ImpArgs a) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;                   // bh * nqb + i
  const int bh = (int)(row / a.nqb);
  const int i = (int)(row % a.nqb);
  const int D = a.D;
  const int DP = D + 1;
  const int nkb = a.nkb;
  const int64_t lo = (int64_t)i * a.q_block;
  const int n = (int)min((int64_t)a.q_block, a.S - lo);
  const int ce = min(a.C, n);

  float* xs = lds;                                   // [q_block][D + 1], later [kChunk][D + 4]
  float* mu = xs + tok_floats(a.q_block, D);         // [C][D]
  int* asg = reinterpret_cast<int*>(mu + a.C * D);   // [q_block]
  int* msz = asg + a.q_block;                        // [8]
  float* dist = reinterpret_cast<float*>(msz + kMaxClusters); // [C][q_block]
  float* zb = dist + a.C * a.q_block;                // [C][nkb]
  float* red = zb + a.C * nkb;                       // [max(256, P / 2)]

  // ---- 1. tokens ----
  const T* qb = reinterpret_cast<const T*>(a.q) + ((int64_t)bh * a.seq_alloc + lo) * D;
  for (int e = tid; e < n * D; e += kImpThreads) xs[(e / D) * DP + e % D] = widen(qb, e);
  __syncthreads();
  for (int e = tid; e < ce * D; e += kImpThreads) {
    const int c = e / D, d = e % D;
    mu[e] = xs[((c * n) / ce) * DP + d];
  }
  __syncthreads();

  // ---- 2. k-means ----
  // distance of every (token, cluster) pair by its own thread, then the
  // nearest cluster of every token (lowest index among equals)
  auto assign = [&]() {
    for (int e = tid; e < n * ce; e += kImpThreads) {
      const int t = e % n, c = e / n;
      const float* xr = xs + t * DP;
      const float* mr = mu + c * D;
      float acc = 0.0f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        const float df = __fsub_rn(xr[d], mr[d]);
        acc = __fadd_rn(acc, __fmul_rn(df, df));
      }
      dist[e] = acc;
    }
    __syncthreads();
    for (int t = tid; t < n; t += kImpThreads) {
      int best = 0;
      float bd = dist[t];
      for (int c = 1; c < ce; ++c) {
        const float v = dist[c * n + t];
        if (v < bd) {
          bd = v;
          best = c;
        }
      }
      asg[t] = best;
    }
    __syncthreads();
  };
  for (int it = 0; it < a.T; ++it) {
    assign();
    for (int e = tid; e < ce * D; e += kImpThreads) {
      const int c = e / D, d = e % D;
      // members in ascending token order; a non-member adds +0, which leaves
      // a nonzero sum unchanged and can only turn a -0 sum into +0 (the same
      // distances and logits: both enter through x - mu and mu * k, and a
      // zero logit is stored as +0)
      float acc = 0.0f;
      int m = 0;
#pragma unroll 8
      for (int t = 0; t < n; ++t) {
        const bool in = asg[t] == c;
        acc = __fadd_rn(acc, in ? xs[t * DP + d] : 0.0f);
        m += in ? 1 : 0;
      }
      if (m > 0) mu[e] = __fdiv_rn(acc, (float)m);
    }
    __syncthreads();
  }
  assign();
  if (tid < ce) {
    int m = 0;
    for (int t = 0; t < n; ++t) m += asg[t] == tid ? 1 : 0;
    msz[tid] = m;
  }
  __syncthreads();

  // ---- 3. logits of every centroid against every key-block summary ----
  // The summaries go through LDS (the token area, free by now) in chunks of
  // kChunk rows with coalesced loads; one thread per (row of the chunk,
  // cluster), threads of a wave on consecutive rows of one cluster.
  const float* kb = a.kp + (int64_t)bh * nkb * D;
  const int KS = D + 4;                              // padded row stride (16-byte rows)
  float* ks = xs;
  for (int j0 = 0; j0 < nkb; j0 += kChunk) {
    const int nj = min(kChunk, nkb - j0);
    __syncthreads();                                 // the previous chunk is consumed
    const int D4 = D / 4;
    for (int e = tid; e < nj * D4; e += kImpThreads) {
      const int r = e / D4, c4 = e % D4;
      *reinterpret_cast<float4*>(ks + r * KS + 4 * c4) =
          *reinterpret_cast<const float4*>(kb + (int64_t)(j0 + r) * D + 4 * c4);
    }
    __syncthreads();
    for (int e = tid; e < kChunk * ce; e += kImpThreads) {
      const int jl = e % kChunk, c = e / kChunk;
      if (jl >= nj) continue;
      const float* kr = ks + jl * KS;
      const float* mr = mu + c * D;
      float acc = 0.0f;
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(kr + d);
        const float4 m = *reinterpret_cast<const float4*>(mr + d);
        acc = __fadd_rn(acc, __fmul_rn(m.x, kv.x));
        acc = __fadd_rn(acc, __fmul_rn(m.y, kv.y));
        acc = __fadd_rn(acc, __fmul_rn(m.z, kv.z));
        acc = __fadd_rn(acc, __fmul_rn(m.w, kv.w));
      }
      const int j = j0 + jl;
      const float lc = (j == nkb - 1) ? a.ln_last : a.ln_full;
      float z = __fmul_rn(acc, a.scale);
      if (a.log_cluster) z = __fadd_rn(z, lc);
      if (z == 0.0f) z = 0.0f;                      // -0 -> +0
      zb[c * nkb + j] = z;
    }
  }
  __syncthreads();

  // ---- 4. softmax of every non-empty cluster, token-share-weighted sum ----
  int P = 1;
  while (P < nkb) P <<= 1;
  float imp[kMaxOwned];
#pragma unroll
  for (int r = 0; r < kMaxOwned; ++r) imp[r] = 0.0f;
  for (int c = 0; c < ce; ++c) {
    if (msz[c] == 0) continue;                       // uniform: msz is in LDS
    float* zc = zb + c * nkb;
    float m = -INFINITY;
    for (int j = tid; j < nkb; j += kImpThreads) m = fmaxf(m, zc[j]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));   // max is exact in any order
    __syncthreads();
    for (int j = tid; j < nkb; j += kImpThreads) zc[j] = exp_le0(__fsub_rn(zc[j], M));
    __syncthreads();
    float Z;
    if (P == 1) {
      Z = zc[0];
    } else {
      const int h0 = P / 2;
      for (int k = tid; k < h0; k += kImpThreads) {
        const float v0 = k < nkb ? zc[k] : 0.0f;
        const float v1 = k + h0 < nkb ? zc[k + h0] : 0.0f;
        red[k] = __fadd_rn(v0, v1);
      }
      __syncthreads();
      // halving levels across waves through LDS while more than 64 values
      // remain, the rest inside wave 0 with the same pairs (lane k adds lane
      // k + h)
      int cnt = h0;
      for (; cnt > 64; cnt >>= 1) {
        const int h = cnt >> 1;
        for (int k = tid; k < h; k += kImpThreads) red[k] = __fadd_rn(red[k], red[k + h]);
        __syncthreads();
      }
      if (tid < 64) {
        float v = tid < cnt ? red[tid] : 0.0f;
        for (; cnt > 1; cnt >>= 1) {
          const int h = cnt >> 1;
          const float o = __shfl_down(v, h, 64);
          if (tid < h) v = __fadd_rn(v, o);
        }
        if (tid == 0) red[0] = v;
      }
      __syncthreads();
      Z = red[0];
    }
    const float w = __fdiv_rn((float)msz[c], (float)n);
#pragma unroll
    for (int r = 0; r < kMaxOwned; ++r) {
      const int j = tid + r * kImpThreads;
      if (j < nkb) imp[r] = __fadd_rn(imp[r], __fmul_rn(w, __fdiv_rn(zc[j], Z)));
    }
    __syncthreads();                                 // red is reused by the next cluster
  }
  float* out = a.imp + row * nkb;
#pragma unroll
  for (int r = 0; r < kMaxOwned; ++r) {
    const int j = tid + r * kImpThreads;
    if (j < nkb) out[j] = imp[r];
  }
}

}  // namespace

size_t importance_lds_bytes(const ImpArgs& a) {
  int P = 1;
  while (P < a.nkb) P <<= 1;
  const size_t red = (size_t)(P / 2 > kImpThreads ? P / 2 : kImpThreads);
  return sizeof(float) * ((size_t)tok_floats(a.q_block, a.D) + (size_t)a.C * a.D + (size_t)a.q_block +
                          kMaxClusters + (size_t)a.C * a.q_block + (size_t)a.C * a.nkb + red);
}

hipError_t launch_importance(const ImpArgs& a, int dtype, hipStream_t stream) {
  const size_t lds = importance_lds_bytes(a);
  const int64_t grid = (int64_t)a.BH * a.nqb;
  if (dtype == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&importance_kernel<bf16_t>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(importance_kernel<bf16_t>, dim3((unsigned)grid), dim3(kImpThreads), lds, stream, a);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&importance_kernel<float>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(importance_kernel<float>, dim3((unsigned)grid), dim3(kImpThreads), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bsa
