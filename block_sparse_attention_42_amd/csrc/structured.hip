// Structured block lists on gfx950: per-head frame contexts over the same
// sparse forward.
//
// Pages: "Efficient Autoregressive Video Diffusion with Dummy Head" (frame
// attention scores of its Step 0; the per-class contexts of its Steps 2 and
// 3: sink heads see the sink frame and the current frame, neighbor heads the
// last L frames, dummy heads the current frame or frames i-1 and i); the
// block-causal frame mask of "Purpose of the block-causal mask ..." (a frame
// attends to itself and earlier frames); "Attention matrix view: make only
// frame-0 query rows dense" (token packing [text] + [frame 0] + ..., sec. 1;
// dense frame-0 rows, sec. 4; text blocks, sec. 7).
//
// A block covers the interval of frames of its valid tokens (text is frame
// -1).  A query block's context is the union over its frames of its head
// class's frames; text is in every context and a query block holding text
// sees everything.  A key block is listed iff its frame interval meets the
// context.  All of it is integer logic on the geometry.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kStThreads = 256;
constexpr int kFsThreads = 1024;          // frame scores: one workgroup of 16 waves per head

__device__ __forceinline__ int frame_of(const StructArgs& a, int64_t t) {
  return t < a.text_len ? -1 : (int)((t - a.text_len) / a.tpf);
}

// Token frames are monotone in t, so a frame's tokens form one run of
// blocks.  first_block(f): the first block whose first token is in frame f
// or later; block_of_first(f) / block_of_last(f): the blocks holding the
// first / last token of frame f.
__device__ __forceinline__ int64_t frame_start(const StructArgs& a, int f) {
  const int64_t t = a.text_len + (int64_t)f * a.tpf;
  return t < a.S ? t : a.S;
}
__device__ __forceinline__ int first_block(const StructArgs& a, int f) {
  return (int)((frame_start(a, f) + a.k_block - 1) / a.k_block);
}
__device__ __forceinline__ int block_of_first(const StructArgs& a, int f) {
  return (int)(frame_start(a, f) / a.k_block);
}
__device__ __forceinline__ int block_of_last(const StructArgs& a, int f) {
  return (int)((frame_start(a, f + 1) - 1) / a.k_block);
}

// One workgroup per (b, h), one thread per query block (strided).  A scored
// row (first token in frame f >= 1) sums P' over three runs of key blocks
// (first token in frame 0; in frames max(1, f-L+1) .. f-1; in frame f),
// normalizes the three to sum 1 and adds them to the thread's total; the
// totals are then added by a fixed tree.  The runs' bounds come from a table
// of first_block(f) in LDS.
__global__ __launch_bounds__(kFsThreads) void frame_score_kernel(StructArgs a) {
  __shared__ double red[4][kFsThreads];
  __shared__ int fb[kMaxStructFrames + 2];
  const int bh = blockIdx.x;
  const int nf = a.frames;                                     // first_block(0 .. nf + 1)
  for (int f = threadIdx.x; f <= nf + 1; f += kFsThreads) fb[f] = first_block(a, f);
  __syncthreads();
  double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, rows = 0.0;
  for (int i = threadIdx.x; i < a.nqb; i += kFsThreads) {
    const int f = frame_of(a, (int64_t)i * a.q_block);
    if (f < 1) continue;
    const float* p = a.scores + ((int64_t)bh * a.nqb + i) * a.nkb;
    const int nb = f - a.window + 1 > 1 ? f - a.window + 1 : 1;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    // ascending j in each run (unrolled so several loads are in flight)
#pragma unroll 8
    for (int j = fb[0]; j < fb[1]; ++j) s0 += (double)p[j];
#pragma unroll 8
    for (int j = fb[nb]; j < fb[f]; ++j) s1 += (double)p[j];
#pragma unroll 8
    for (int j = fb[f]; j < fb[f + 1]; ++j) s2 += (double)p[j];
    const double s = s0 + s1 + s2;
    rows += 1.0;
    if (s > 0.0) {
      acc0 += s0 / s;
      acc1 += s1 / s;
      acc2 += s2 / s;
    }
  }
  red[0][threadIdx.x] = acc0;
  red[1][threadIdx.x] = acc1;
  red[2][threadIdx.x] = acc2;
  red[3][threadIdx.x] = rows;
  __syncthreads();
  for (int h = kFsThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h)
      for (int k = 0; k < 4; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x < 3) a.alpha[bh * 3 + threadIdx.x] = red[threadIdx.x][0] / (red[3][0] > 0.0 ? red[3][0] : 1.0);
}

// One wave per (b, h, query block).  The context is a run of frames
// [lo, hi] (plus the sink frame for sink heads, plus the text), so the
// listed key blocks are the union of at most four runs of block indices,
// found once per row; each lane then only compares its block index.
__global__ __launch_bounds__(kStThreads) void struct_lists_kernel(StructArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kStThreads / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)a.BH * a.nqb) return;                   // uniform per wave
  const int bh = (int)(row / a.nqb);
  const int i = (int)(row % a.nqb);
  const int n = a.nkb;
  const int cls = a.classes[bh];
  const int64_t qlo = (int64_t)i * a.q_block;
  const int64_t qhi = (qlo + a.q_block < a.S ? qlo + a.q_block : a.S) - 1;
  const int q0 = frame_of(a, qlo), q1 = frame_of(a, qhi);
  const bool dense = a.frame0_first >= 0 && i >= a.frame0_first && i <= a.frame0_last;
  const bool all = q0 < 0 || (cls == 0 && !a.block_causal) || dense;
  int lo;
  switch (cls) {
    case 0: lo = 0; break;                                      // full, block-causal
    case 1: lo = q0; break;                                     // sink
    case 2: lo = q0 - a.window + 1 > 0 ? q0 - a.window + 1 : 0; break;   // neighbor
    default: lo = a.dummy_prev && q0 >= 1 ? q0 - 1 : q0; break; // dummy
  }
  // runs of listed key blocks (empty runs have first > last)
  const int r0 = all ? n : block_of_first(a, lo), r1 = all ? n : block_of_last(a, q1);
  const int s0 = cls == 1 ? block_of_first(a, 0) : n, s1 = cls == 1 ? block_of_last(a, 0) : -1;
  const int tl = a.text_len > 0 ? (int)((a.text_len - 1) / a.k_block) : -1;
  const int txt = tl > a.text_last ? tl : a.text_last;
  uint8_t* mrow = a.mask ? a.mask + row * n : nullptr;
  int32_t* irow = a.idx + row * n;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int run = 0;
  for (int base = 0; base < n; base += 64) {
    const int j = base + lane;
    const bool in = j < n;
    const bool sel = in && (all || j <= txt || (j >= r0 && j <= r1) || (j >= s0 && j <= s1));
    const uint64_t bsel = __ballot(sel);
    const int pos = run + __popcll(bsel & below);
    if (in && mrow) mrow[j] = sel ? 1 : 0;
    if (sel) irow[pos] = j;
    run += __popcll(bsel);
  }
  if (lane == 0) a.cnt[row] = run;
}

}  // namespace

hipError_t launch_frame_scores(const StructArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(frame_score_kernel, dim3((unsigned)a.BH), dim3(kFsThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_struct_lists(const StructArgs& a, hipStream_t stream) {
  const unsigned groups = (unsigned)(((int64_t)a.BH * a.nqb + 3) / 4);
  hipLaunchKernelGGL(struct_lists_kernel, dim3(groups), dim3(kStThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
