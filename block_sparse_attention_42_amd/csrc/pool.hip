// Block mean pooling on gfx950 (AB-Attention page, TL;DR: block scores come
// from coarse per-block summaries; EG-Sparse page: centroids of clusters of
// n tokens).  HBM-bound: every input byte is read once, with loads
// coalesced along D.
//
// Each thread owns 4 consecutive channels of one block and adds the block's
// valid rows in ascending order in float32, then divides once by the row
// count; this order is part of the library's contract so the result is
// bit-reproducible and independent of the launch shape.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kUnroll = 8;
constexpr int kChannels = 4;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Four consecutive channels of one row: an 8-byte load for bf16, 16 bytes
// for float32.  Four channels per thread (rather than eight) doubles the
// waves in flight, which measured about 20 % faster at head_dim 128.  The
// loads are non-temporal: each input byte is read once here, and streaming
// it past the caches measured 4-10 % faster on MI355X (1.46 GB of Q and K:
// 0.273 -> 0.245 ms).
template <typename T>
struct Row4;

template <>
struct Row4<bf16_t> {
  u32x2_t raw;
  __device__ void load(const bf16_t* p) { raw = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)); }
  __device__ void get(float (&v)[4]) const {
    v[0] = __uint_as_float(raw.x << 16);
    v[1] = __uint_as_float(raw.x & 0xffff0000u);
    v[2] = __uint_as_float(raw.y << 16);
    v[3] = __uint_as_float(raw.y & 0xffff0000u);
  }
};

template <>
struct Row4<float> {
  f32x4_t raw;
  __device__ void load(const float* p) { raw = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p)); }
  __device__ void get(float (&v)[4]) const {
    v[0] = raw.x; v[1] = raw.y; v[2] = raw.z; v[3] = raw.w;
  }
};

// Rows of one pooled block a lane keeps in flight: all of a block's loads
// are issued before its first add (32 rows of 8 bytes, 16 of 16 bytes).
template <typename T>
constexpr int kChunk = sizeof(T) == 2 ? 32 : 16;

// One lane: channels c4*4 .. c4*4+3 of pooled row `rowid` (= bh * nb + i).
// A full block's rows are loaded in chunks of kChunk and added in ascending
// order; the last (short) block of a head takes the guarded loop.
template <typename T, int kBlock>
__device__ __forceinline__ void pool_lane(const PoolArgs& a, int64_t rowid, int c4) {
  const int i = (int)(rowid % a.nb);
  const int64_t bh = rowid / a.nb;
  const int64_t t0 = (int64_t)i * kBlock;
  const int n = (int)min<int64_t>(kBlock, a.S - t0);
  const T* src = reinterpret_cast<const T*>(a.x) + (bh * a.seq_alloc + t0) * a.D + c4 * kChannels;

  float acc[kChannels];
#pragma unroll
  for (int c = 0; c < kChannels; ++c) acc[c] = 0.0f;
  auto add = [&](const Row4<T>& r) {
    float v[kChannels];
    r.get(v);
#pragma unroll
    for (int c = 0; c < kChannels; ++c) acc[c] = __fadd_rn(acc[c], v[c]);
  };
  constexpr int kC = kChunk<T> < kBlock ? kChunk<T> : kBlock;
  if (n == kBlock) {
#pragma unroll
    for (int t = 0; t < kBlock; t += kC) {
      Row4<T> r[kC];
#pragma unroll
      for (int u = 0; u < kC; ++u) r[u].load(src + (int64_t)(t + u) * a.D);
#pragma unroll
      for (int u = 0; u < kC; ++u) add(r[u]);
    }
  } else {
    for (int t = 0; t < n; t += kUnroll) {
      Row4<T> r[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (t + u < n) r[u].load(src + (int64_t)(t + u) * a.D);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (t + u < n) add(r[u]);
    }
  }
  const float fn = (float)n;
  float4 o;
  o.x = __fdiv_rn(acc[0], fn); o.y = __fdiv_rn(acc[1], fn);
  o.z = __fdiv_rn(acc[2], fn); o.w = __fdiv_rn(acc[3], fn);
  *reinterpret_cast<float4*>(a.out + rowid * a.D + c4 * kChannels) = o;
}

// One launch pools up to two tensors (Q with q_block and K with k_block):
// workgroups [0, first[1]) take job 0, the rest job 1.
struct PoolJobs {
  PoolArgs job[2];
  int64_t first[2];   // first workgroup of each job
};

template <typename T>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolJobs jobs) {
  const int j = (int64_t)blockIdx.x >= jobs.first[1] ? 1 : 0;
  const PoolArgs& a = jobs.job[j];
  const int lanes_per_block = a.D / kChannels;         // threads per pooled row
  const int64_t gid = ((int64_t)blockIdx.x - jobs.first[j]) * kPoolThreads + threadIdx.x;
  const int64_t total = (int64_t)a.BH * a.nb * lanes_per_block;
  if (gid >= total) return;
  const int c4 = (int)(gid % lanes_per_block);
  const int64_t rowid = gid / lanes_per_block;
  switch (a.block) {
    case 16: pool_lane<T, 16>(a, rowid, c4); break;
    case 32: pool_lane<T, 32>(a, rowid, c4); break;
    default: pool_lane<T, 64>(a, rowid, c4); break;
  }
}

}  // namespace

hipError_t launch_pool_jobs(const PoolArgs* jobs, int njobs, int dtype, hipStream_t stream) {
  PoolJobs pj;
  int64_t grid = 0;
  for (int j = 0; j < 2; ++j) {
    pj.job[j] = jobs[j < njobs ? j : 0];
    pj.first[j] = grid;
    if (j < njobs) {
      const int64_t total = (int64_t)jobs[j].BH * jobs[j].nb * (jobs[j].D / kChannels);
      grid += (total + kPoolThreads - 1) / kPoolThreads;
    } else {
      pj.first[j] = grid;   // no workgroup reaches a missing job
    }
  }
  if (njobs == 1) pj.first[1] = INT64_MAX;
  if (dtype == 0)
    hipLaunchKernelGGL(pool_kernel<bf16_t>, dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, pj);
  else
    hipLaunchKernelGGL(pool_kernel<float>, dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, pj);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs& a, int dtype, hipStream_t stream) {
  return launch_pool_jobs(&a, 1, dtype, stream);
}

}  // namespace bsa
