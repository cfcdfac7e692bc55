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

// bf16: one wave per span of kSpan consecutive rows of one head (contiguous in
// memory, at most 16 KB; spans start on block boundaries since every block
// size divides kSpan).  The wave reads its span with 16-byte coalesced
// non-temporal loads (each instruction 1 KB of consecutive bytes), stages it
// in LDS, and then lane l adds channels l*CPL .. l*CPL+CPL-1 (CPL = D/64) of
// each block of the span over its rows in ascending order.  Against the
// per-lane kernel (each load instruction two 256-byte rows 16 KB apart) this
// measured 22 % faster for the 201 MB of Q and K at the Wan-like shape on
// MI355X (0.049 -> 0.0385 ms) and 1.5 % at the HunyuanVideo-like one.
constexpr int kSpan = 64;
constexpr int kSpanBytes = kSpan * 128 * 2;

// The block means of one staged span: rows of a full block unrolled (their
// LDS reads issued ahead of the adds), the short last block of a head by a
// loop; the adds in ascending row order either way.
template <int kBlock>
__device__ __forceinline__ void span_sums(const PoolArgs& a, const uint32_t* st, int nrow, int64_t row0, int lane) {
#pragma unroll
  for (int r0 = 0; r0 < kSpan; r0 += kBlock) {
    if (r0 >= nrow) break;
    const int n = min(kBlock, nrow - r0);
    const float fn = (float)n;
    float* out = a.out + (row0 + r0 / kBlock) * a.D;
    if (a.D == 128) {
      float acc0 = 0.0f, acc1 = 0.0f;
      const uint32_t* sw = st + r0 * 64 + lane;
      auto add = [&](uint32_t x) {
        acc0 = __fadd_rn(acc0, __uint_as_float(x << 16));
        acc1 = __fadd_rn(acc1, __uint_as_float(x & 0xffff0000u));
      };
      if (n == kBlock) {
#pragma unroll
        for (int t = 0; t < kBlock; ++t) add(sw[t * 64]);
      } else {
        for (int t = 0; t < n; ++t) add(sw[t * 64]);
      }
      float2 o;
      o.x = __fdiv_rn(acc0, fn);
      o.y = __fdiv_rn(acc1, fn);
      *reinterpret_cast<float2*>(out + 2 * lane) = o;
    } else {   // D = 64: one channel a lane
      const uint16_t* sh = reinterpret_cast<const uint16_t*>(st) + r0 * 64 + lane;
      float acc = 0.0f;
      if (n == kBlock) {
#pragma unroll
        for (int t = 0; t < kBlock; ++t) acc = __fadd_rn(acc, __uint_as_float((uint32_t)sh[t * 64] << 16));
      } else {
        for (int t = 0; t < n; ++t) acc = __fadd_rn(acc, __uint_as_float((uint32_t)sh[t * 64] << 16));
      }
      out[lane] = __fdiv_rn(acc, fn);
    }
  }
}

// One wave per workgroup: a CU then holds up to ten span waves (16 KB of LDS
// each) instead of two four-wave workgroups (measured 5 % faster at the
// Wan-like shapes, 1 % at the HunyuanVideo-like one).
constexpr int kSpanWaves = 1;

__global__ __launch_bounds__(kSpanWaves * 64) void pool_span_kernel(PoolJobs jobs) {
  __shared__ __attribute__((aligned(16))) uint32_t stage[kSpanWaves][kSpanBytes / 4];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int j = (int64_t)blockIdx.x >= jobs.first[1] ? 1 : 0;
  const PoolArgs& a = jobs.job[j];
  const int64_t nspan = (a.S + kSpan - 1) / kSpan;        // spans per head
  const int64_t sp = ((int64_t)blockIdx.x - jobs.first[j]) * kSpanWaves + wave;
  if (sp >= (int64_t)a.BH * nspan) return;
  const int64_t bh = sp / nspan;
  const int64_t t0 = (sp % nspan) * kSpan;
  const int nrow = (int)min<int64_t>(kSpan, a.S - t0);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t* src =
      reinterpret_cast<const u32x4_t*>(reinterpret_cast<const bf16_t*>(a.x) + (bh * a.seq_alloc + t0) * a.D);
  const int chunks = nrow * a.D / 8;                       // 16-byte chunks of the span's valid rows
  constexpr int kPer = kSpanBytes / 16 / 64;               // chunks per lane (D = 128)
  u32x4_t r[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k;
    if (c < chunks) r[k] = __builtin_nontemporal_load(src + c);
  }
  u32x4_t* st = reinterpret_cast<u32x4_t*>(stage[wave]);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k;
    if (c < chunks) st[c] = r[k];
  }
  // the lanes read what other lanes of the wave wrote
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int64_t row0 = bh * a.nb + t0 / a.block;           // first pooled row of the span
  switch (a.block) {
    case 16: span_sums<16>(a, stage[wave], nrow, row0, lane); break;
    case 32: span_sums<32>(a, stage[wave], nrow, row0, lane); break;
    default: span_sums<64>(a, stage[wave], nrow, row0, lane); break;
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
  if (dtype == 0) {
    // bf16: the span kernel, kSpanWaves spans per workgroup
    int64_t g = 0;
    for (int j = 0; j < 2; ++j) {
      pj.first[j] = g;
      if (j < njobs) g += ((int64_t)jobs[j].BH * ((jobs[j].S + kSpan - 1) / kSpan) + kSpanWaves - 1) / kSpanWaves;
    }
    if (njobs == 1) pj.first[1] = INT64_MAX;
    hipLaunchKernelGGL(pool_span_kernel, dim3((unsigned)g), dim3(kSpanWaves * 64), 0, stream, pj);
  } else {
    hipLaunchKernelGGL(pool_kernel<float>, dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, pj);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs& a, int dtype, hipStream_t stream) {
  return launch_pool_jobs(&a, 1, dtype, stream);
}

}  // namespace bsa
