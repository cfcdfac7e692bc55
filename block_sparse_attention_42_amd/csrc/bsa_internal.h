// Internal declarations shared by the host entry points (abi.cpp) and the
// gfx950 kernels (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// bfloat16 storage element (bit pattern only; arithmetic is done in float32).
struct bf16_t {
  uint16_t bits;
};

// Launch arguments of the pooling kernel.
struct PoolArgs {
  const void* x;      // [BH, seq_alloc, D]
  float* out;         // [BH, nb, D]
  int64_t seq_alloc;
  int64_t S;
  int32_t BH, D, block, nb;
};

// Launch arguments of the mask kernel.
struct MaskArgs {
  const float* qp;    // [BH, nqb, D]
  const float* kp;    // [BH, nkb, D]
  uint8_t* mask;      // [BH, nqb, nkb] or null
  int32_t* cnt;       // [BH, nqb]
  int32_t* idx;       // [BH, nqb, nkb]
  float* logw;        // [BH, nqb, nkb] or null
  int32_t H, BH, nqb, nkb, D;
  int32_t mode;       // 0 top-k, 1 sample
  int32_t topk;
  float expected;
  float scale;        // fp32(1/sqrt(D))
  int32_t log_cluster;
  float ln_full;      // fp32(ln k_block)
  float ln_last;      // fp32(ln n_last)
  int32_t frame0_first, frame0_last;   // -1 if off
  int32_t text_last;                   // -1 if off
  uint64_t seed;
  const float* imp;   // [BH, nqb, nkb] block importance to select from (qp, kp unused), or null
};

// Launch arguments of the top-p / competition-domain selection kernels.
struct TopPArgs {
  const float* scores;   // [BH, nqb, nkb] P' (>= 0)
  const float* vp;       // [BH, nkb, D] pooled values (value-aware scores) or null
  void* ws;              // workspace (topp_workspace_bytes)
  double* entropy_out;   // [BH] or null
  uint8_t* mask;         // [BH, nqb, nkb] or null
  int32_t* cnt;          // [BH, nqb]
  int32_t* idx;          // [BH, nqb, nkb]
  int32_t B, H, BH, nqb, nkb, D;
  int32_t vstride;       // row stride of the value norms in the workspace
  int32_t npools;
  int32_t domain;        // 0 row, 1 head, 2 split, 3 all, 4 EG-Sparse routing
  int32_t value_aware;
  double top_p;
  float eps;
  int32_t frame0_first, frame0_last;   // -1 if off
  int32_t text_last;                   // -1 if off
};

// Launch arguments of the structured-list kernels (per-head frame contexts).
constexpr int kMaxStructFrames = 4096;   // frame-score table in LDS

struct StructArgs {
  const float* scores;   // [BH, nqb, nkb] P' (frame scores) or null
  double* alpha;         // [BH, 3] frame scores out
  const int32_t* classes;   // [BH] head classes: 0 full, 1 sink, 2 neighbor, 3 dummy
  uint8_t* mask;         // [BH, nqb, nkb] or null
  int32_t* cnt;          // [BH, nqb]
  int32_t* idx;          // [BH, nqb, nkb]
  int64_t S;
  int64_t text_len;
  int64_t tpf;           // tokens per frame (>= 1)
  int32_t frames;        // latent frames (<= kMaxStructFrames for frame scores)
  int32_t BH, nqb, nkb, q_block, k_block;
  int32_t window;        // L: frames a neighbor head sees, the current one included
  int32_t dummy_prev, block_causal;
  int32_t frame0_first, frame0_last;   // -1 if off
  int32_t text_last;                   // -1 if off
};

// Launch arguments of the block-importance kernel (intra-block clusters).
struct ImpArgs {
  const void* q;      // [BH, seq_alloc, D]
  const float* kp;    // [BH, nkb, D]
  float* imp;         // [BH, nqb, nkb]
  int64_t seq_alloc;
  int64_t S;
  int32_t BH, nqb, nkb, D, q_block;
  int32_t C, T;       // clusters per query block (1..8), Lloyd rounds
  float scale;        // fp32(1/sqrt(D))
  int32_t log_cluster;
  float ln_full;      // fp32(ln k_block)
  float ln_last;      // fp32(ln n_last)
  int32_t G;          // query blocks per workgroup (importance_group)
  int32_t area_a;     // floats of the shared token / logit area (set by the launcher)
};

// Launch arguments of the sparse forward kernel.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cnt;
  const int32_t* idx;
  const float* logw;  // or null
  void* out;
  float* lse;         // or null
  int64_t seq_alloc;
  int64_t S;
  int32_t BH, nqb, nkb, q_block, k_block;
  float scale_log2;   // softmax scale * log2(e)
  // launch schedule (performance only; every (head, query block) runs once)
  int32_t dense_first, dense_last;   // frame-0 query blocks, run first (-1, -1: none)
  int32_t period;                    // query blocks per frame, rounded (>= 1)
  int32_t per_xcd;                   // remaining work items per XCD
  int32_t n_dense;                   // dense work items: BH * dense rows * split
  int32_t order;                     // 0: frame-position runs, 1: frame runs of every head
  // key split of the frame-0 rows (split > 1): work item t < n_dense covers
  // part t % split of its row's list and leaves its partial softmax state in
  // ws; a second kernel merges the parts into out and lse
  int32_t split;                     // 1: off
  float* ws;                         // partial states (split > 1), see split_ws_floats
};

// Workspace of the key split, in floats: per dense work item, the
// unnormalized O rows (q_block x D), then the reference maxima (q_block, log2
// domain) and the row sums (q_block) of all items.
inline int64_t split_ws_floats(int64_t items, int32_t q_block, int32_t D) {
  return items * q_block * (int64_t)D + 2 * items * q_block;
}

// Work items of the forward launch: the frame-0 (longest) rows of every head
// first, dealt round-robin over the XCDs, then the other rows.  Order 0: in
// contiguous per-XCD runs of consecutive work items (head-major; inside a
// head, query blocks at the same in-frame position of successive frames are
// adjacent), so that rows running together on one XCD share key blocks in
// its L2.  Order 1: XCD x takes the x-th eighth of every head's other rows
// (a run of frames), head-major, in index order.
constexpr int kXcds = 8;
inline int64_t forward_grid(const FwdArgs& a) { return (int64_t)a.n_dense + (int64_t)kXcds * a.per_xcd; }

// Device scratch owned by the library (scratch.hip): the partial states of
// bsa_forward_split_static, at most this many bytes on each GPU.
constexpr int64_t kStaticScratchBytes = 32LL << 20;
// Device address of the current GPU's copy (looked up once per device).
hipError_t static_scratch(float** ptr);

hipError_t launch_pool(const PoolArgs& a, int dtype, hipStream_t stream);
// Pools one or two tensors (jobs[0], jobs[1]) in a single launch.
hipError_t launch_pool_jobs(const PoolArgs* jobs, int njobs, int dtype, hipStream_t stream);
hipError_t launch_mask(const MaskArgs& a, hipStream_t stream);
int importance_group(int C, int nkb, int nqb);
size_t importance_lds_bytes(const ImpArgs& a);
int64_t topp_workspace_bytes(int64_t BH, int64_t B, int64_t nqb, int64_t nkb);
hipError_t launch_topp(const TopPArgs& a, hipStream_t stream);
hipError_t launch_frame_scores(const StructArgs& a, hipStream_t stream);
hipError_t launch_struct_lists(const StructArgs& a, hipStream_t stream);
hipError_t launch_importance(const ImpArgs& a, int dtype, hipStream_t stream);
hipError_t launch_forward(const FwdArgs& a, int dtype, int head_dim, hipStream_t stream);
// The 64-key-step forward kernel and the shapes it covers (launch_forward
// picks it for them).
bool forward_wide_supported(int dtype, int head_dim, int q_block, int k_block);
hipError_t launch_forward_wide(const FwdArgs& a, hipStream_t stream);
// The float32 forward (float32 matrix products and softmax).
hipError_t launch_forward_f32(const FwdArgs& a, int head_dim, hipStream_t stream);

}  // namespace bsa
