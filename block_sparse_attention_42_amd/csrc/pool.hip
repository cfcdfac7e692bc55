// Block mean pooling on gfx950 (AB-Attention page, TL;DR: block scores come
// from coarse per-block summaries; EG-Sparse page: centroids of clusters of
// n tokens).  HBM-bound: every input byte is read once, with 16-byte loads
// coalesced along D.
//
// Each thread owns 8 consecutive channels of one block and adds the block's
// valid rows in ascending order in float32, then divides once by the row
// count; this order is part of the library's contract so the result is
// bit-reproducible and independent of the launch shape.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kUnroll = 8;

__device__ inline void widen8(const uint4& raw, float (&v)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[2 * c] = __uint_as_float(w[c] << 16);
    v[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
  }
}

template <typename T>
struct Row8;

template <>
struct Row8<bf16_t> {
  uint4 raw;
  __device__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ void get(float (&v)[8]) const { widen8(raw, v); }
};

template <>
struct Row8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ void get(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <typename T>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolArgs a) {
  const int lanes_per_block = a.D / 8;                  // threads per pooled row
  const int64_t gid = (int64_t)blockIdx.x * kPoolThreads + threadIdx.x;
  const int64_t total = (int64_t)a.BH * a.nb * lanes_per_block;
  if (gid >= total) return;
  const int c8 = (int)(gid % lanes_per_block);
  const int64_t rowid = gid / lanes_per_block;           // bh * nb + i
  const int i = (int)(rowid % a.nb);
  const int64_t bh = rowid / a.nb;
  const int64_t t0 = (int64_t)i * a.block;
  const int n = (int)min<int64_t>(a.block, a.S - t0);
  const T* src = reinterpret_cast<const T*>(a.x) + (bh * a.seq_alloc + t0) * a.D + c8 * 8;

  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;

  for (int t = 0; t < n; t += kUnroll) {
    Row8<T> r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (t + u < n) r[u].load(src + (int64_t)(t + u) * a.D);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t + u < n) {
        float v[8];
        r[u].get(v);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __fadd_rn(acc[c], v[c]);
      }
    }
  }
  const float fn = (float)n;
  float4 o0, o1;
  o0.x = __fdiv_rn(acc[0], fn); o0.y = __fdiv_rn(acc[1], fn);
  o0.z = __fdiv_rn(acc[2], fn); o0.w = __fdiv_rn(acc[3], fn);
  o1.x = __fdiv_rn(acc[4], fn); o1.y = __fdiv_rn(acc[5], fn);
  o1.z = __fdiv_rn(acc[6], fn); o1.w = __fdiv_rn(acc[7], fn);
  float4* dst = reinterpret_cast<float4*>(a.out + rowid * a.D + c8 * 8);
  dst[0] = o0;
  dst[1] = o1;
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, int dtype, hipStream_t stream) {
  const int64_t total = (int64_t)a.BH * a.nb * (a.D / 8);
  const int64_t grid = (total + kPoolThreads - 1) / kPoolThreads;
  if (dtype == 0)
    hipLaunchKernelGGL(pool_kernel<bf16_t>, dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(pool_kernel<float>, dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
