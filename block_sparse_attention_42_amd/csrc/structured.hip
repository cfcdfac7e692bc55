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
// context.  All of it is integer logic on the geometry, one wave per row.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kStThreads = 256;

__device__ __forceinline__ int frame_of(const StructArgs& a, int64_t t) {
  return t < a.text_len ? -1 : (int)((t - a.text_len) / a.tpf);
}

__global__ __launch_bounds__(kStThreads) void frame_score_kernel(StructArgs a) {
  __shared__ double red[3][kStThreads];
  const int bh = blockIdx.x;
  double acc[3] = {0.0, 0.0, 0.0};
  for (int i = threadIdx.x; i < a.nqb; i += kStThreads) {
    const int f = frame_of(a, (int64_t)i * a.q_block);
    if (f < 1) continue;
    const float* p = a.scores + ((int64_t)bh * a.nqb + i) * a.nkb;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    const int nb_lo = f - a.window + 1 > 1 ? f - a.window + 1 : 1;
    for (int j = 0; j < a.nkb; ++j) {
      const int kf = frame_of(a, (int64_t)j * a.k_block);
      const double v = (double)p[j];
      if (kf == 0) s0 += v;
      else if (kf >= nb_lo && kf <= f - 1) s1 += v;
      else if (kf == f) s2 += v;
    }
    const double s = s0 + s1 + s2;
    if (s > 0.0) {
      acc[0] += s0 / s;
      acc[1] += s1 / s;
      acc[2] += s2 / s;
    }
  }
  for (int k = 0; k < 3; ++k) red[k][threadIdx.x] = acc[k];
  __syncthreads();
  for (int h = kStThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h)
      for (int k = 0; k < 3; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x < 3) {
    int rows = 0;
    for (int i = 0; i < a.nqb; ++i) rows += frame_of(a, (int64_t)i * a.q_block) >= 1 ? 1 : 0;
    a.alpha[bh * 3 + threadIdx.x] = red[threadIdx.x][0] / (double)(rows > 0 ? rows : 1);
  }
}

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
  // the context: everything, or the sink frame (optional) plus one interval
  bool all = q0 < 0 || (cls == 0 && !a.block_causal);
  bool sink = false;
  int lo = 0, hi = q1;
  switch (cls) {
    case 0: lo = 0; break;                                      // full, block-causal
    case 1: sink = true; lo = q0; break;                        // sink
    case 2: lo = q0 - a.window + 1 > 0 ? q0 - a.window + 1 : 0; break;   // neighbor
    default: lo = a.dummy_prev && q0 >= 1 ? q0 - 1 : q0; break; // dummy
  }
  const bool dense = a.frame0_first >= 0 && i >= a.frame0_first && i <= a.frame0_last;
  all = all || dense;
  uint8_t* mrow = a.mask ? a.mask + row * n : nullptr;
  int32_t* irow = a.idx + row * n;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int run = 0;
  for (int base = 0; base < n; base += 64) {
    const int j = base + lane;
    const bool in = j < n;
    bool sel = false;
    if (in) {
      const int64_t klo = (int64_t)j * a.k_block;
      const int64_t khi = (klo + a.k_block < a.S ? klo + a.k_block : a.S) - 1;
      const int k0 = frame_of(a, klo), k1 = frame_of(a, khi);
      sel = all || k0 < 0 || (k0 <= hi && k1 >= lo) || (sink && k0 <= 0 && k1 >= 0) || j <= a.text_last;
    }
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
  hipLaunchKernelGGL(frame_score_kernel, dim3((unsigned)a.BH), dim3(kStThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_struct_lists(const StructArgs& a, hipStream_t stream) {
  const unsigned groups = (unsigned)(((int64_t)a.BH * a.nqb + 3) / 4);
  hipLaunchKernelGGL(struct_lists_kernel, dim3(groups), dim3(kStThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
