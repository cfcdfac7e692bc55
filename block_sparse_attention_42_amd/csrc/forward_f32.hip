// Block-sparse attention forward for float32 Q/K/V on gfx950: float32
// products on the matrix cores (v_mfma_f32_32x32x2_f32), float32 softmax.
//
// Pages: "AB-Attention: accurate block-sparse attention for video diffusion"
// (TL;DR: exact attention on the selected key/value blocks; key blocks
// smaller than a tile gathered into one tile; inverse-inclusion-probability
// reweighting as an additive log-weight) and "Attention matrix view: make
// only frame-0 query rows dense" (sec. 2).
//
// The same work decomposition as the bf16 kernels, without their pipeline:
// one wave per (b, h, query block) of 32 or 64 rows, the block's key list
// walked in 32-key sub-tiles (16-key blocks two per sub-tile), S^T = K Q^T
// and O^T += V^T P^T as 32 x 32 tiles, each lane owning one query column.
// The operands come straight from memory (float32 rows are read once per
// sub-tile and stay in L2), rows past the valid keys read as zeros.  Online
// softmax in the log2 domain with the reference max moved at every sub-tile.
//
// Operand layouts of the 32 x 32 x 2 float32 product (per lane l, column
// c = l % 32, half h = l / 32): A supplies element (row c, k = h), B element
// (k = h, column c); accumulator register r holds row 8(r/4) + 4h + r%4 of
// column c.  For S^T the k pair is two channels 2s, 2s + 1; for O^T it is the
// two keys whose P values the lanes of each half hold in register t, so
// P^T feeds the product straight from the accumulator layout of S^T.
#include "fwd_common.h"

namespace bsa {
namespace {

using namespace fwdc;

template <int D, int QT, int BK>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64))) void fwd_f32_kernel(FwdArgs a) {
  constexpr int SUB = 32;                           // keys per sub-tile
  constexpr int NBLK = BK >= SUB ? 1 : SUB / BK;    // list entries per sub-tile
  constexpr int PART = SUB / NBLK;                  // keys of one entry in a sub-tile
  constexpr int DS = D / 2;                         // k steps of S^T
  constexpr int DT = D / 32;                        // d tiles of O^T
  const int lane = threadIdx.x;
  const int qc = lane & 31;
  const int hf = lane >> 5;

  int bh, qb;
  if (!schedule(a, blockIdx.x, bh, qb)) return;
  const int64_t rowid = (int64_t)bh * a.nqb + qb;
  const int cnt_row = __builtin_amdgcn_readfirstlane(min(max(a.cnt[rowid], 0), a.nkb));
  // a split frame-0 row: this item walks entries lo .. lo + cnt - 1 of the list
  const bool part_item = a.split > 1 && (int)blockIdx.x < a.n_dense;
  const int part = part_item ? (int)blockIdx.x % a.split : 0;
  const int lo = part_item ? (int)((int64_t)part * cnt_row / a.split) : 0;
  const int cnt = part_item ? (int)((int64_t)(part + 1) * cnt_row / a.split) - lo : cnt_row;
  // rows past the head's last query block (seq_alloc > nqb * q_block)
  if (qb == a.nqb - 1 && part == 0) zero_tail_rows<float, D>(a, bh, lane);
  const int nsub = (cnt * BK + SUB - 1) / SUB;

  const float* Qb = reinterpret_cast<const float*>(a.q) + (int64_t)bh * a.seq_alloc * D;
  const float* Kb = reinterpret_cast<const float*>(a.k) + (int64_t)bh * a.seq_alloc * D;
  const float* Vb = reinterpret_cast<const float*>(a.v) + (int64_t)bh * a.seq_alloc * D;
  const int32_t* lst = a.idx + rowid * a.nkb + lo;
  const float* lw = a.logw ? a.logw + rowid * a.nkb + lo : nullptr;
  const int64_t q0 = (int64_t)qb * a.q_block;

  // Q^T B operands: element (k = hf, column qc) of step s is Q[q][2s + hf]
  float qf[QT][DS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t q = q0 + 32 * qt + qc;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[qt][s] = q < a.S ? Qb[q * D + 2 * s + hf] : 0.0f;
  }

  float m_run[QT], l_run[QT];
  f32x16 o[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x16{};
  }

  // list entry and log-weight of part b of sub-tile u (entry -1 past the list)
  auto entry = [&](int u, int b, int& j, float& w) {
    const int pos = (u * SUB + b * PART) / BK;
    j = pos < cnt ? lst[pos] : -1;
    w = (pos < cnt && lw) ? lw[pos] : 0.0f;
  };
  int nj[NBLK];
  float nw[NBLK];
#pragma unroll
  for (int b = 0; b < NBLK; ++b) entry(0, b, nj[b], nw[b]);
  for (int u = 0; u < nsub; ++u) {
    // the list entries of the sub-tile (fetched one sub-tile ahead): first
    // key, valid keys, log2 weight
    int key0[NBLK], valid[NBLK];
    float bias[NBLK];
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int g = u * SUB + b * PART;
      const int j = nj[b];
      key0[b] = 0;
      valid[b] = 0;
      bias[b] = 0.0f;
      if ((uint32_t)j < (uint32_t)a.nkb) {
        key0[b] = j * BK + g % BK;
        const int64_t rest = a.S - key0[b];
        valid[b] = rest < PART ? (rest > 0 ? (int)rest : 0) : PART;
        bias[b] = nw[b] * 1.4426950408889634f;
      }
    }
#pragma unroll
    for (int b = 0; b < NBLK; ++b) entry(u + 1, b, nj[b], nw[b]);
    // the sub-tile's K and V operands, all loads issued before the first
    // product so that their latencies overlap: key row qc of the tile in the
    // S^T A operand; for the P V products, the keys of register t
    const int kp = qc / PART, ko = qc % PART;
    const bool kvalid = ko < valid[kp];
    const float* krow = Kb + (int64_t)(key0[kp] + ko) * D;
    float kv[DS];
#pragma unroll
    for (int st = 0; st < DS; ++st) kv[st] = kvalid ? krow[2 * st + hf] : 0.0f;
    // (V ahead of the products where the registers allow: not for 64 rows
    // at head_dim 128, whose Q and O already take 256 of them)
    constexpr bool kVAhead = D * QT <= 128;
    auto v_of = [&](int t, int dt) {
      const int i = 8 * (t >> 2) + 4 * hf + (t & 3);
      const int ip = i / PART, io = i % PART;
      return io < valid[ip] ? Vb[(int64_t)(key0[ip] + io) * D + 32 * dt + qc] : 0.0f;
    };
    float vv[kVAhead ? 16 : 1][DT];
    if constexpr (kVAhead) {
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vv[t][dt] = v_of(t, dt);
    }
    // S^T in two interleaved chains (even and odd channel pairs) added at the
    // end: each accumulator takes half the D/2 roundings, which at logits of
    // magnitude ~100 keeps the rounding of p near float32's own
    f32x16 s[QT], s2[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      s[qt] = f32x16{};
      s2[qt] = f32x16{};
    }
#pragma unroll
    for (int st = 0; st < DS; st += 2) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        s[qt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[st], qf[qt][st], s[qt], 0, 0, 0);
        s2[qt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[st + 1], qf[qt][st + 1], s2[qt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) s[qt] += s2[qt];
    // log2-domain logits of this lane's 16 keys; keys past the valid ones -inf
    float p[QT][16];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * hf + (r & 3);
        const int ip = i / PART;
        const float t = (i % PART) < valid[ip] ? s[qt][r] * a.scale_log2 + bias[ip] : -INFINITY;
        p[qt][r] = t;
        mx = fmaxf(mx, t);
      }
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run[qt], mx);
      const float mu = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = exp2f(m_run[qt] - mu);
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[qt][r] = exp2f(p[qt][r] - mu);
        ls += p[qt][r];
      }
      l_run[qt] = l_run[qt] * alpha + ls;
      m_run[qt] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[qt][dt] *= alpha;
    }
    // O^T += V^T P^T: step t pairs key 8(t/4) + t%4 (lanes 0-31) with key
    // 8(t/4) + 4 + t%4 (lanes 32-63), the keys of register t
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float v = kVAhead ? vv[kVAhead ? t : 0][dt] : v_of(t, dt);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(v, p[qt][t], o[qt][dt], 0, 0, 0);
      }
  }

  // ---- epilogue: normalize (or leave the partial state of a split row) ----
  constexpr int QB = 32 * QT;
  float* Ob = reinterpret_cast<float*>(a.out) + (int64_t)bh * a.seq_alloc * D;
  float* wsO = part_item ? a.ws + (int64_t)blockIdx.x * QB * D : nullptr;
  float* wsM = part_item ? a.ws + (int64_t)a.n_dense * QB * D + (int64_t)blockIdx.x * QB : nullptr;
  float* wsL = part_item ? wsM + (int64_t)a.n_dense * QB : nullptr;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l = add_xor32(l_run[qt]);
    const int64_t row = q0 + 32 * qt + qc;
    if (row >= a.seq_alloc) continue;
    const bool live = row < a.S && l > 0.0f;
    const float inv = part_item ? 1.0f : (live ? 1.0f / l : 0.0f);
    if (hf == 0) {
      if (part_item) {
        wsM[32 * qt + qc] = m_run[qt];
        wsL[32 * qt + qc] = l;
      } else if (a.lse) {
        a.lse[(int64_t)bh * a.seq_alloc + row] = live ? (m_run[qt] + __log2f(l)) * kLn2 : -INFINITY;
      }
    }
    float* dst = part_item ? wsO + (row - q0) * D : Ob + row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r >> 2) + 4 * hf + (r & 3);
        dst[d] = row < a.S ? o[qt][dt][r] * inv : 0.0f;
      }
  }
}

template <int D, int QT>
hipError_t launch_bk(const FwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)forward_grid(a)), block(64);
  switch (a.k_block) {
    case 16: hipLaunchKernelGGL((fwd_f32_kernel<D, QT, 16>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((fwd_f32_kernel<D, QT, 32>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((fwd_f32_kernel<D, QT, 64>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_q(const FwdArgs& a, hipStream_t stream) {
  return a.q_block == 32 ? launch_bk<D, 1>(a, stream) : launch_bk<D, 2>(a, stream);
}

}  // namespace

hipError_t launch_forward_f32(const FwdArgs& a, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_q<64>(a, stream) : launch_q<128>(a, stream);
}

}  // namespace bsa
