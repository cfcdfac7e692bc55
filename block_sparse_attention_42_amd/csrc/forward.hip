// Block-sparse attention forward on gfx950 (MI355X).
//
// Pages: "AB-Attention: accurate block-sparse attention for video diffusion"
// (TL;DR: exact attention only on the selected key/value blocks; key blocks
// smaller than a tile gathered into full tiles; inverse-inclusion-probability
// reweighting) and "Attention matrix view: make only frame-0 query rows
// dense" (sec. 2: a dense row attends to every key/value token).
//
// Work decomposition:
//   * one workgroup = one wave = one (b, h, query block) of 32 or 64 rows.
//     The wave may use up to 512 registers (one wave per SIMD): the Q
//     fragments and the O^T accumulators of the whole query block live in
//     AGPRs, the two score tiles and the softmax state in VGPRs, so every
//     K/V byte read from LDS feeds all rows of the block;
//   * the block's selected key blocks are walked in 32-key sub-tiles
//     (16-key blocks are gathered two per sub-tile);
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (issued as
//     inline asm with fixed register classes, so the compiler never shuffles
//     accumulators between register files): each lane owns one query column
//     of a 32-row tile, so the running max, sum and rescale stay in the lane
//     (one permlane32 swap joins the two key halves);
//   * K and V sub-tiles go from HBM/L2 to LDS by buffer-load DMA into two
//     slots each (K two sub-tiles ahead, V one ahead). A group of loads
//     shares one scalar row offset and differs only in the literal
//     immediate; the waits before LDS reads are explicit in-order vmcnt
//     counts. K is read back with ds_read_b128, V^T with the transposing
//     ds_read_b64_tr_b16, both from XOR-swizzled layouts;
//   * the list entries (key block, log-weight) are fetched by vector loads
//     five sub-tiles ahead and broadcast with readlane, so no scalar-cache
//     wait ever blocks the tile loads;
//   * software pipeline per sub-tile u: phase 1 issues the S(u+1) MFMAs with
//     the exponentials of S(u) and the V(u+1) loads between them; phase 2
//     issues the P V MFMAs of u with the rest of the exponentials, the row
//     max of S(u+1) and the K(u+3) loads between them;
//   * softmax in the log2 domain with lazy rescaling (the reference max moves
//     only when a row max grows by more than 8), scale and per-block
//     log-weight folded into one multiply-add, row sums by v_dot2 over the
//     same bf16 P the P V product uses.
#include "fwd_common.h"

namespace bsa {
namespace {

using namespace fwdc;

template <typename T, int D, int QT, int BK>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(1, 1)))
void fwd_kernel(FwdArgs a) {
  // bf16 tiles go HBM -> LDS directly (the kernel is instantiated for bf16
  // only: float32 inputs take the float32 kernel)
  constexpr bool kDma = sizeof(T) == 2;
  constexpr uint32_t ES = sizeof(T);
  constexpr uint32_t RB = D * ES;      // bytes per K/V row in memory
  constexpr int KC = D / 16;           // k chunks of the Q.K contraction (32x32x16)
  constexpr int DT = D / 32;           // d tiles of O^T
  constexpr int KCH = D / 8;           // 16-byte (8 x bf16) chunks per row
  constexpr int SUB = 32;              // keys per sub-tile
  constexpr int TILE_E = SUB * D;      // bf16 elements of one K or V sub-tile in LDS
  constexpr int NLD = SUB * KCH / 64;  // chunks per lane per sub-tile
  constexpr int RPL = 64 / KCH;        // sub-tile rows per load round
  constexpr int NBLK = BK >= SUB ? 1 : SUB / BK;   // key blocks per sub-tile
  constexpr int PART = SUB / NBLK;
  constexpr float kTau = 8.0f;         // lazy rescale: tolerated growth of the running max (log2)
  static_assert(NBLK <= 2 && PART % RPL == 0 && NLD >= 1, "tile shape");
  // One LDS array per ring slot: the compiler then knows which tile loads a
  // read can depend on, and never waits for the loads still in flight into
  // the other slots.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[TILE_E], k_lds1[TILE_E];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[TILE_E], v_lds1[TILE_E];
  // destination of the tile loads of a step whose tile is loaded separately
  // (partial tiles): the instructions still run, their data is discarded
  // (4 KB: a group of loads writes up to 4 consecutive KB)
  __shared__ __attribute__((aligned(16))) uint16_t sink_lds[4 * 64 * 8];

  const int lane = threadIdx.x;
  const int qc = lane & 31;            // query column of S^T / O^T, key row of the K operand
  const int hf = lane >> 5;            // 0/1: k half of the operands, row half of the accumulators

  int bh, qb;
  if (!schedule(a, blockIdx.x, bh, qb)) return;
  const int64_t rowid = (int64_t)bh * a.nqb + qb;
  // (read-first-lane: row values are wave-uniform and should live in scalar registers)
  const int cnt_row = __builtin_amdgcn_readfirstlane(min(max(a.cnt[rowid], 0), a.nkb));   // never past nkb slots
  // a split frame-0 row: this item walks entries lo .. lo + cnt - 1 of the list
  const bool part_item = a.split > 1 && (int)blockIdx.x < a.n_dense;
  const int part = part_item ? (int)blockIdx.x % a.split : 0;
  const int lo = part_item ? (int)((int64_t)part * cnt_row / a.split) : 0;
  const int cnt = part_item ? (int)((int64_t)(part + 1) * cnt_row / a.split) - lo : cnt_row;
  // rows past the head's last query block (seq_alloc > nqb * q_block)
  if (qb == a.nqb - 1 && part == 0) zero_tail_rows<T, D>(a, bh, lane);
  const int nsub = (cnt * BK + SUB - 1) / SUB;          // 32-key sub-tiles of the row

  const T* Qb = reinterpret_cast<const T*>(a.q) + (int64_t)bh * a.seq_alloc * D;
  const T* Kb = reinterpret_cast<const T*>(a.k) + (int64_t)bh * a.seq_alloc * D;
  const T* Vb = reinterpret_cast<const T*>(a.v) + (int64_t)bh * a.seq_alloc * D;
  const int64_t q0 = (int64_t)qb * a.q_block;
  const int S32 = (int)a.S;

  const bool has_w = a.logw != nullptr;

  const uint32_t nbytes = (uint32_t)a.seq_alloc * RB;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)Qb, 0, (int)nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)Kb, 0, (int)nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, 0, (int)nbytes, 0x00020000);

  // ---- Q^T fragments (B operand of S^T = K Q^T): Q[q][16c + 8hf .. +7] ----
  // rows past S read zeros
  bf16x8 qf[QT][KC];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t row = q0 + 32 * qt + qc;
    const uint32_t off = row < a.S ? (uint32_t)row * RB + (uint32_t)(8 * hf) * ES : kOob;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[qt][c] = as_frag(Row8<T>::buf(rq, off + (uint32_t)(16 * c) * ES, 0));
  }
  // Q is only ever an MFMA operand: keep it in the accumulation registers,
  // leaving the vector registers to the score tiles and the softmax.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int c = 0; c < KC; ++c) asm volatile("" : "+a"(qf[qt][c]));

  // ---- sub-tile geometry: first key, valid keys and log2 weight of each part ----
  // The list entries (and log-weights) of a sub-tile are fetched by vector
  // loads, lane b taking part b, several steps before they are needed: the
  // loads are ordered with the tile loads, so no wait on them ever blocks the
  // LDS reads (as a scalar-cache load's wait would).
  const uint32_t lbytes = (uint32_t)(a.nkb - lo) * 4u;
  const int64_t lbase = rowid * a.nkb + lo;
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)(a.idx + lbase), 0, (int)lbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(has_w ? (void*)(a.logw + lbase) : (void*)(a.idx + lbase), 0,
                                        (int)lbytes, 0x00020000);
  struct Raw {
    int j;      // lane b: list entry of part b
    int w;      // lane b: its log-weight bits
  };
  struct Info {
    int key0[NBLK];      // first key of each part (0 if none)
    int valid[NBLK];     // valid keys of each part (0 if none)
    float bias[NBLK];    // log2-domain weight of each part
  };
  auto fetch = [&](int u) {
    const int b = lane < NBLK ? lane : 0;
    const uint32_t pos = (uint32_t)(u * SUB + b * PART) / (uint32_t)BK;
    const uint32_t off = min(pos, (uint32_t)max(cnt - 1, 0)) * 4u;   // every row has nkb >= 1 slots
    Raw r;
    if constexpr (NBLK == 1) {   // one entry for all lanes: a scalar offset
      r.j = (int)__builtin_amdgcn_raw_buffer_load_b32(rl, 0, (int)off, 0);
      r.w = (int)__builtin_amdgcn_raw_buffer_load_b32(rw, 0, (int)off, 0);
    } else {
      r.j = (int)__builtin_amdgcn_raw_buffer_load_b32(rl, (int)off, 0, 0);
      r.w = (int)__builtin_amdgcn_raw_buffer_load_b32(rw, (int)off, 0, 0);
    }
    return r;
  };
  auto info = [&](int u, const Raw& r) {
    Info si;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int g = u * SUB + b * PART;
      const int pos = g / BK;
      const int jr = __builtin_amdgcn_readlane(r.j, b);
      const bool ok = pos < cnt && (uint32_t)jr < (uint32_t)a.nkb;
      const int key0 = jr * BK + g % BK;
      si.key0[b] = ok ? key0 : 0;
      // keys of the part before the end of the sequence, in [0, PART]
      const int rest = S32 - key0;
      si.valid[b] = ok ? (rest < PART ? (rest > 0 ? rest : 0) : PART) : 0;
      const float w = has_w ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(r.w, b)) : 0.0f;
      si.bias[b] = ok ? w * 1.4426950408889634f : 0.0f;
    }
    return si;
  };
  // A 64-key block spans two sub-tiles: the list entry of an odd sub-tile is
  // that of the even one before it, so even steps fetch nothing and the
  // second sub-tile's geometry follows from the first's.
  constexpr bool kPair = BK == 2 * SUB;
  auto info_second = [&](const Info& first) {
    Info si;
    const bool ok = first.valid[0] > 0;   // a listed block has keys in its first half
    const int key0 = first.key0[0] + SUB;
    const int rest = S32 - key0;
    si.key0[0] = ok ? key0 : 0;
    si.valid[0] = ok ? (rest < SUB ? (rest > 0 ? rest : 0) : SUB) : 0;
    si.bias[0] = first.bias[0];
    return si;
  };
  auto is_full = [&](const Info& si) {
    bool full = true;
#pragma unroll
    for (int p = 0; p < NBLK; ++p) full = full && si.valid[p] == PART;
    return full;
  };

  // ---- K / V sub-tile -> LDS ring slot ----
  // Load n of this lane fills LDS chunk n*64 + lane of the slot: tile row
  // r = n*RPL + lane/KCH, holding logical chunk (lane % KCH) ^ swizzle(r);
  // all rows of one load round belong to one part.  Rows past the valid keys
  // (or of a missing part) read zeros.
  //   K rows are read back as 16-byte A-operand pieces, 16 consecutive rows
  //   at one logical chunk per access: swizzle r & 15 (D = 128) or
  //   (r >> 1) & 7 (D = 64) spreads them over the banks.
  //   V rows are read with the transposing 8-byte load, 4 consecutive rows x 4
  //   chunks per 16 lanes: swizzle 4(r & 3) (D = 128) or 4((r >> 1) & 1).
  // Both swizzles only touch chunk bits, so every LDS read address is a lane
  // base XOR a per-fragment constant.
  const int vrow = lane / KCH;
  auto swz_k = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto chunk_off = [&](int n, bool is_k) {
    const int r = n * RPL + vrow;
    return (uint32_t)(vrow * D + ((lane % KCH) ^ (is_k ? swz_k(r) : swz_v<D>(r))) * 8) * ES;
  };
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  auto lds_frag = [](const lds_u8* p) {
    const u32x4 v = *reinterpret_cast<const lds_u32x4*>(p);
    return as_frag(make_uint4(v[0], v[1], v[2], v[3]));
  };
  auto kslot = [&](int s) { return s == 0 ? (lds_u16*)k_lds0 : (lds_u16*)k_lds1; };
  auto vslot = [&](int s) { return s == 0 ? (lds_u16*)v_lds0 : (lds_u16*)v_lds1; };
  // load n of a full tile, or (redirect) the same load into the sink.  The
  // instruction's immediate offset moves both the global and the LDS address,
  // so the loads of one group of G rounds share one scalar offset and one LDS
  // base (M0) and differ only in the immediate (n % G) KB; a group never
  // straddles two key blocks.
  constexpr int G = (PART / RPL) < 4 ? (PART / RPL) : 4;
  auto load_fast = [&](__amdgpu_buffer_rsrc_t rsrc, const Info& si, lds_u16* dst, bool is_k, int n, bool redirect) {
    const int g0 = (n / G) * G;                 // first round of the group
    const int part = (g0 * RPL) / PART;
    const int r0 = g0 * RPL - part * PART;
    const uint32_t so = ((uint32_t)si.key0[part] + (uint32_t)r0) * RB;
    lds_u16* d = redirect ? (lds_u16*)sink_lds : dst + g0 * 64 * 8;
    auto* ld = (__attribute__((address_space(3))) void*)d;
    const int vo = (int)chunk_off(n, is_k);
    switch (n % G) {   // the immediate must be a literal; n is known after unrolling
      case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, ld, 16, vo, (int)so, 0, 0); break;
      case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, ld, 16, vo, (int)so, 1024, 0); break;
      case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, ld, 16, vo, (int)so, 2048, 0); break;
      default: __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, ld, 16, vo, (int)so, 3072, 0); break;
    }
  };
  auto load_one = [&](__amdgpu_buffer_rsrc_t rsrc, const Info& si, lds_u16* dst, bool is_k, int n, bool full) {
    const int part = (n * RPL) / PART;
    const int r0 = n * RPL - part * PART;   // first row of the round inside its part
    const uint32_t so = ((uint32_t)si.key0[part] + (uint32_t)r0) * RB;
    const uint32_t co = chunk_off(n, is_k);
    if constexpr (kDma) {
      const uint32_t vo = full ? co : (vrow < si.valid[part] - r0 ? co + so : kOob);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(dst + n * 64 * 8), 16, (int)vo, (int)(full ? so : 0u), 0, 0);
    } else {
      const uint32_t vo = vrow < si.valid[part] - r0 ? co + so : kOob;
      const uint4 x = Row8<T>::buf(rsrc, vo, 0);
      *reinterpret_cast<lds_u32x4*>(dst + (n * 64 + lane) * 8) = u32x4{x.x, x.y, x.z, x.w};
    }
  };
  auto load_tile = [&](__amdgpu_buffer_rsrc_t rsrc, const Info& si, lds_u16* dst, bool is_k, auto known_full) {
    const bool full = decltype(known_full)::value || is_full(si);
#pragma unroll
    for (int n = 0; n < NLD; ++n) load_one(rsrc, si, dst, is_k, n, full);
  };

  // ---- S^T(u) = K(u) Q^T ----
  // K A-operand read of chunk c: tile row qc, logical chunk 2c + hf:
  // byte address ka ^ (c * 32).
  const uint32_t ka = (uint32_t)(qc * KCH * 16) | (uint32_t)((hf ^ swz_k(qc)) * 16);
  auto qk = [&](int ks, f32x16 (&s)[QT]) {
    const lds_u8* kt = reinterpret_cast<const lds_u8*>(kslot(ks));
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) s[qt] = f32x16{};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const bf16x8 kf = lds_frag(kt + (ka ^ (uint32_t)(c * 32)));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qt][c], s[qt], 0, 0, 0);
    }
  };

  // accumulator register r of this lane is tile row 8*(r/4) + 4*hf + r%4
  auto mask = [&](f32x16 (&s)[QT], const Info& si) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * hf + (r & 3);
      const int p = row / PART;
      // (select, not an indexed read: the geometry must stay in scalar registers)
      const int v = p == 0 ? si.valid[0] : si.valid[NBLK - 1];
      const bool bad = row - p * PART >= v;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        if (bad) s[qt][r] = -INFINITY;
    }
  };

  // row max of S(u) in the log2 domain: the lane's 16 keys, then lane ^ 32
  auto rowmax = [&](const f32x16 (&s)[QT], const Info& si, float (&mx)[QT]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const f32x16& x = s[qt];
      const float m0 = fmaxf(fmaxf(fmaxf(fmaxf(x[0], x[1]), x[2]), fmaxf(x[3], x[4])), fmaxf(fmaxf(x[5], x[6]), x[7]));
      const float m1 = fmaxf(fmaxf(fmaxf(fmaxf(x[8], x[9]), x[10]), fmaxf(x[11], x[12])),
                             fmaxf(fmaxf(x[13], x[14]), x[15]));
      float m;
      if constexpr (NBLK == 2) m = fmaxf(m0 * a.scale_log2 + si.bias[0], m1 * a.scale_log2 + si.bias[1]);
      else m = fmaxf(m0, m1) * a.scale_log2 + si.bias[0];
      mx[qt] = max_xor32(m);
    }
  };

  float m_run[QT], l_run[QT];
  float thr[QT];   // m_run + kTau: a row max above it moves the reference
  f32x16 o[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    thr[qt] = -INFINITY;
    l_run[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x16{};
  }

  // lazy rescale: the reference max moves only when a row max grows by more
  // than kTau (so every p <= 2^kTau); O and l are rescaled only then
  auto rescale = [&](const float (&mx)[QT]) {
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) grow = grow || mx[qt] > thr[qt];
    if (__any(grow)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float m_new = mx[qt] > thr[qt] ? mx[qt] : m_run[qt];
        const float alpha = fast_exp2(m_run[qt] - (m_new == -INFINITY ? 0.0f : m_new));
        m_run[qt] = m_new;
        thr[qt] = m_new + kTau;
        l_run[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          o[qt][dt] *= alpha;
          // one tile at a time: each is back in its accumulators before the next
          if constexpr (kDma) asm volatile("" : "+a"(o[qt][dt]));
        }
      }
    }
  };

  // P(u) = exp2(S(u) * scale + bias - m) as bf16 P^T B operands; the row sum
  // adds exactly these bf16 values (v_dot2 with ones).  P^T B operand of key
  // chunk c holds keys 16c + 8(e/4) + 4hf + e%4 = accumulator registers 8c + e.
  auto softmax = [&](const f32x16 (&s)[QT], const Info& si, bf16x8 (&pb)[QT][2]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mu = m_run[qt] == -INFINITY ? 0.0f : m_run[qt];
      const float off0 = si.bias[0] - mu;
      const float off1 = si.bias[NBLK - 1] - mu;
      float ps = 0.0f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const int r = 8 * c + 2 * k2;
          const float p0 = fast_exp2(s[qt][r] * a.scale_log2 + (r < 8 ? off0 : off1));
          const float p1 = fast_exp2(s[qt][r + 1] * a.scale_log2 + (r < 8 ? off0 : off1));
          w[k2] = pack_bf16x2(p0, p1);
          ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[k2]), kOnes2, ps, false);
        }
        pb[qt][c] = as_frag(make_uint4(w[0], w[1], w[2], w[3]));
      }
      l_run[qt] += ps;
    }
  };

  // V^T A-operand transposing reads: 16-lane group g = lane/16 covers d columns
  // 16*(g & 1) + [0, 16) of d tile dt; lane i of the group addresses tile row
  // 16c + 8hh + 4hf + i/4 and columns 32dt + 16(g & 1) + 4(i & 3):
  // byte address va ^ (dt * 64) + (16c + 8hh) rows.
  const uint32_t va = [&] {
    const int i = lane & 15, g = lane >> 4;
    const int r = 4 * hf + (i >> 2);
    const int lc = 2 * (g & 1) + ((i & 3) >> 1);
    return (uint32_t)(r * D * 2) | (uint32_t)((lc ^ swz_v<D>(r)) * 16) | (uint32_t)((i & 1) * 8);
  }();
  auto pv = [&](int vs, const bf16x8 (&pb)[QT][2]) {
    const lds_u8* vt = reinterpret_cast<const lds_u8*>(vslot(vs));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const lds_u8* vp = vt + (va ^ (uint32_t)(dt * 64)) + (16 * c) * D * 2;
        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vp));
        const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vp + 8 * D * 2));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[qt][c], o[qt][dt], 0, 0, 0);
      }
    }
  };

  // Hazard fences for vector code that reads MFMA results: the nops, then
  // empty ordering points on the values, so the reads cannot move above them.
  auto fence_s = [&](f32x16 (&t)[QT]) {
    asm volatile("s_nop 11" ::: "memory");
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) asm volatile("" : "+v"(t[qt]));
  };
  auto fence_o = [&]() {
    asm volatile("s_nop 11" ::: "memory");
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) asm volatile("" : "+a"(o[qt][dt]));
  };

  // Vector-memory instructions retire in issue order, and every step issues
  // them in the same order: its list loads (two, none in the even steps of
  // 64-key blocks), the NLD V(u+1) loads (one
  // after each of the first NLD MFMAs of phase 1), the NLD K(u+3) loads (one
  // after each of the first NLD MFMAs of phase 2); a partial tile adds its own
  // NLD loads before them.  A wait for a tile counts the loads issued after
  // the tile's last one up to the wait: vmcnt(that count) lets the tile land,
  // and is merely conservative after a partial tile (more loads were issued).
  // In the prologue a tile is followed by two others (2 NLD loads).
  auto tile_wait = [&](auto n) {
    if constexpr (kDma) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(decltype(n)::value) : "memory");
  };
  static_assert(NLD <= KC && NLD <= 2 * DT * QT, "tile loads must fit in the MFMAs of a phase");

  // ---- pipeline ----
  // Step u (p = u & 1): sc[p] holds S(u) (masked, its max folded into
  // m_run); the K(u+1) fragments are in registers, K(u+2) is in K slot u % 2
  // and V(u) in V slot u % 2.
  //   phase 1: S(u+1) MFMAs into sc[p^1], with the exponentials of the first
  //            half of S(u) (P(u) and its row sums) and the V(u+1) loads into
  //            V slot (u+1) % 2 (last read by step u-1) between them; the
  //            V(u) fragments are read from LDS from the last MFMAs on;
  //   phase 2: P(u) V(u) MFMAs, with the second half of the exponentials, the
  //            row max of S(u+1) and the K(u+3) loads into K slot (u+1) % 2
  //            between them; the K(u+2) fragments are read during the last
  //            MFMAs;
  //   then the rescale for S(u+1) if a row max grew past the tolerance.
  // Sub-tiles past the list load zeros and never reach O.  The waits for the
  // tile loads are explicit vmcnt counts (see tile_wait).
  if (nsub > 0) {
    f32x16 sc[2][QT];
    Info i_u = info(0, fetch(0));   // sub-tile u
    Info i_u1 = info(1, fetch(1));  // u + 1
    Info i_u2 = info(2, fetch(2));  // u + 2
    Raw r3 = fetch(3);              // u + 3
    Raw r4 = fetch(4);              // u + 4
    load_tile(rk, i_u, kslot(0), true, std::false_type{});
    load_tile(rk, i_u1, kslot(1), true, std::false_type{});
    load_tile(rv, i_u, vslot(0), false, std::false_type{});
    if constexpr (kDma) {
      // S(0) (the Q fragments were just written into AGPRs by vector moves);
      // K(0) was followed by the K(1) and V(0) loads
      asm volatile("s_waitcnt vmcnt(%0)\n s_nop 1" ::"n"(2 * NLD) : "memory");
      const lds_u8* kt = reinterpret_cast<const lds_u8*>(kslot(0));
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const bf16x8 kf = lds_frag(kt + (ka ^ (uint32_t)(c * 32)));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if (c == 0) mma_s_first(sc[0][qt], kf, qf[qt][c]);
          else mma_s(sc[0][qt], kf, qf[qt][c]);
        }
      }
      load_tile(rk, i_u2, kslot(0), true, std::false_type{});
      fence_s(sc[0]);
    } else {
      qk(0, sc[0]);
      load_tile(rk, i_u2, kslot(0), true, std::false_type{});
    }
    if (!is_full(i_u)) mask(sc[0], i_u);
    {
      float mx[QT];
      rowmax(sc[0], i_u, mx);
      rescale(mx);
    }

    bf16x8 kf[KC];          // K(u+1) fragments at the start of step u
    float row_mx[QT];       // row max of S(u+1), in the log2 domain
    if constexpr (kDma) {
      // K(1) was followed by the V(0) and K(2) loads
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLD) : "memory");
      const lds_u8* kt = reinterpret_cast<const lds_u8*>(kslot(1));
#pragma unroll
      for (int c = 0; c < KC; ++c) kf[c] = lds_frag(kt + (ka ^ (uint32_t)(c * 32)));
    }
    // one step of the matrix-core pipeline (bf16 tiles in LDS by DMA)
    //   phase 1: the S(u+1) MFMAs (K(u+1) fragments read at the end of the
    //            previous step), with the exponentials of the first half of the
    //            keys of S(u) and the V(u+1) loads between them;
    //   phase 2: the P(u) V(u) MFMAs, first half of the keys first: the
    //            exponentials of the second half run between the first half's
    //            MFMAs, the row max of S(u+1) between the second half's; the
    //            K(u+3) loads go in between, V fragments are read two ahead,
    //            and the K(u+2) fragments for the next step are read last.
    auto step_mma = [&](auto par, const Info& i_u3) {
      constexpr int p = decltype(par)::value;   // u & 1
      f32x16 (&scur)[QT] = sc[p];
      f32x16 (&snext)[QT] = sc[p ^ 1];
      const bool part_v = !is_full(i_u1);    // V(u+1) / S(u+1) has invalid keys
      const bool part_k = !is_full(i_u3);    // K(u+3) has invalid keys
      // softmax offsets of S(u): bias of each part minus the reference max
      float off[QT][NBLK];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int b = 0; b < NBLK; ++b) off[qt][b] = i_u.bias[b] - m_run[qt];
      // a partial V(u+1) is loaded here with zeroed rows; the interleaved
      // loads below then go to the sink
      if (part_v) load_tile(rv, i_u1, vslot(p ^ 1), false, std::false_type{});

      // exponential pair k (keys 2k, 2k+1 of the lane's half) of q-tile qt
      uint32_t pw[QT][8];
      // exponential pair k (keys 2k, 2k+1 of the lane's half) of every q-tile:
      // the q-tiles' chains are independent, so their latencies overlap
      auto pair = [&](int k) {
        const int b = (2 * k < 8) ? 0 : NBLK - 1;
        float p0[QT], p1[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) pin_after(off[qt][b]);   // after the MFMA before it
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          p0[qt] = scur[qt][2 * k] * a.scale_log2 + off[qt][b];
          p1[qt] = scur[qt][2 * k + 1] * a.scale_log2 + off[qt][b];
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          p0[qt] = fast_exp2(p0[qt]);
          p1[qt] = fast_exp2(p1[qt]);
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) pw[qt][k] = pack_bf16x2(p0[qt], p1[qt]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[qt][k]), kOnes2, l_run[qt], false);
          pin_before(pw[qt][k]);               // before the MFMA after it
          pin_before(l_run[qt]);
        }
      };

      const lds_u8* vt = reinterpret_cast<const lds_u8*>(vslot(p));
      constexpr int NVF = DT * 2;          // V fragments, c-major: f = c * DT + dt
      auto read_vf = [&](int f) {
        const int c = f / DT, dt = f % DT;
        const lds_u8* vp = vt + (va ^ (uint32_t)(dt * 64)) + (16 * c) * D * 2;
        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vp));
        const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vp + 8 * D * 2));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vfr[NVF];
      // ---- phase 1: pairs k = 0..3 of each q-tile (P chunk c = 0) ----
      constexpr int NM = KC * QT;          // MFMAs of S(u+1)
      constexpr int NP1 = 4;               // pair groups in phase 1 (k = 0..3)
      // the first two V(u) fragments are read during the last MFMAs of phase
      // 1, the others two ahead of their MFMAs; V(u) was followed by K(u+2),
      // the list loads and the V(u+1) loads issued so far
      constexpr int IV = NM > 4 ? NM - 4 : 0;
      constexpr int NF = (kPair && p == 0) ? 0 : 2;   // list loads of this step
      constexpr int NWV = NLD + NF + (IV < NLD ? IV : NLD);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int c = i / QT, qt2 = i % QT;
        if (i == IV) {
          tile_wait(std::integral_constant<int, NWV>{});   // V(u) landed
          vfr[0] = read_vf(0);
          if (NVF > 1) vfr[1] = read_vf(1);
        }
        // pairs placed after MFMA i: e with e * NM / NP1 == i
        if (c == 0) mma_s_first(snext[qt2], kf[c], qf[qt2][c]);
        else mma_s(snext[qt2], kf[c], qf[qt2][c]);
        if (i < NLD) load_fast(rv, i_u1, vslot(p ^ 1), false, i, part_v);
#pragma unroll
        for (int e = 0; e < NP1; ++e) {
          if (e * NM / NP1 == i) pair(e);
        }
      }
      if (part_v) {
        fence_s(snext);
        mask(snext, i_u1);
      }
      // a partial K(u+3) goes into K slot (u+1) % 2 now that phase 1 has read it
      if (part_k) load_tile(rk, i_u3, kslot(p ^ 1), true, std::false_type{});

      // ---- phase 2 ----
      bf16x8 pb[QT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        pb[qt][0] = as_frag(make_uint4(pw[qt][0], pw[qt][1], pw[qt][2], pw[qt][3]));
      // 2 wait states between the last P writes and the first MFMA reading them
      asm volatile("s_nop 1" ::: "memory");
      constexpr int NH = DT * QT;          // MFMAs per half
      constexpr int NP2 = 4;               // pair groups k = 4..7 in the first half
      float mx[QT];
      // row max of S(u+1), in steps spread over the second half
      float rm[QT][6];
      auto rowmax_part = [&](int qt, int st) {
        const f32x16& x = snext[qt];
        float* r = rm[qt];
        switch (st) {
          case 0: r[0] = max3(x[0], x[1], x[2]); r[1] = max3(x[3], x[4], x[5]); pin_before(r[1]); break;
          case 1: r[2] = max3(x[8], x[9], x[10]); r[3] = max3(x[11], x[12], x[13]); pin_before(r[3]); break;
          case 2: r[0] = max3(r[0], r[1], x[6]); r[2] = max3(r[2], r[3], x[14]); pin_before(r[2]); break;
          case 3: {
            r[0] = max3(r[0], x[7], x[7]);
            r[2] = max3(r[2], x[15], x[15]);
            float m;
            if constexpr (NBLK == 2) {
              const float m0 = r[0] * a.scale_log2 + i_u1.bias[0];
              const float m1 = r[2] * a.scale_log2 + i_u1.bias[1];
              m = max3(m0, m1, m1);
            } else {
              m = max3(r[0], r[2], r[2]) * a.scale_log2 + i_u1.bias[0];
            }
            r[4] = m;
            pin_before(r[4]);
            break;
          }
          default: {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(r[4]), __float_as_uint(r[4]), false, false);
            mx[qt] = max3(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1]));
            pin_before(mx[qt]);
            break;
          }
        }
      };
      constexpr int NRS = 5;               // row max steps per q-tile
      constexpr int JK = 2 * NH > 4 ? 2 * NH - 4 : 0;
      constexpr int NWK = NF + NLD + (JK + 1 < NLD ? JK + 1 : NLD);
#pragma unroll
      for (int j = 0; j < 2 * NH; ++j) {
        const int f = j / QT, qt = j % QT;
        const int c = f / DT, dt = f % DT;
        if (qt == 0 && f + 2 < NVF) vfr[f + 2] = read_vf(f + 2);
        if (j == NH) {
          // P chunk c = 1 complete before its first MFMA (2 wait states)
#pragma unroll
          for (int q2 = 0; q2 < QT; ++q2)
            pb[q2][1] = as_frag(make_uint4(pw[q2][4], pw[q2][5], pw[q2][6], pw[q2][7]));
          asm volatile("s_nop 1" ::: "memory");
          // the row max reads S(u+1) from here on (8+ MFMAs after its last one)
#pragma unroll
          for (int t = 0; t < QT; ++t) asm volatile("" : "+v"(snext[t]));
        }
        mma_o(o[qt][dt], vfr[f], pb[qt][c]);
        if (j < NLD) load_fast(rk, i_u3, kslot(p ^ 1), true, j, part_k);
        if (j < NH) {
          // pairs k = 4..7 spread over the first half
#pragma unroll
          for (int e = 0; e < NP2; ++e) {
            if (e * NH / NP2 == j) pair(4 + e);
          }
        } else {
          // row max steps spread over the second half
          const int jj = j - NH;
#pragma unroll
          for (int e = 0; e < NRS; ++e) {
            if (e * NH / NRS == jj) {
#pragma unroll
              for (int q2 = 0; q2 < QT; ++q2) rowmax_part(q2, e);
            }
          }
        }
        // K(u+2) fragments for the next step, read during the last MFMAs; K(u+2)
        // was followed by the list loads, V(u+1) and the K(u+3) loads so far
        if (j == JK) {
          const lds_u8* kt = reinterpret_cast<const lds_u8*>(kslot(p));
          tile_wait(std::integral_constant<int, NWK>{});   // K(u+2) landed
#pragma unroll
          for (int c2 = 0; c2 < KC; ++c2) kf[c2] = lds_frag(kt + (ka ^ (uint32_t)(c2 * 32)));
        }
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) row_mx[qt] = mx[qt];
    };

    auto step = [&](auto par, auto full, int u, const Info& i_u3) {
      constexpr int p = decltype(par)::value;   // u & 1
      constexpr bool kFull = decltype(full)::value;
      // list entry of sub-tile u + 5, used two steps from now (the same as
      // that of u + 4 when a block spans two sub-tiles and u is even)
      Raw r5;
      if constexpr (kPair && p == 0) r5 = r4;
      else r5 = fetch(u + 5);
      if constexpr (kDma) {
        step_mma(par, i_u3);
      } else {
        load_tile(rv, i_u1, vslot(p ^ 1), false, full);
        bf16x8 pb[QT][2];
        qk(p ^ 1, sc[p ^ 1]);
        softmax(sc[p], i_u, pb);
        if constexpr (!kFull) {
          if (!is_full(i_u1)) mask(sc[p ^ 1], i_u1);
        }
        pv(p, pb);
        load_tile(rk, i_u3, kslot(p ^ 1), true, full);
      }
      float mx[QT];
      if constexpr (kDma) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mx[qt] = row_mx[qt];
      } else {
        rowmax(sc[p ^ 1], i_u1, mx);
      }
      if (u + 1 < nsub) {
        if constexpr (kDma) {
          // vector reads of O (rescale) 12+ wait states after the last P V MFMA
          bool grow = false;
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) grow = grow || mx[qt] > thr[qt];
          if (__any(grow)) {
            fence_o();
            rescale(mx);
          }
        } else {
          rescale(mx);
        }
      }
      i_u = i_u1;
      i_u1 = i_u2;
      i_u2 = i_u3;
      r3 = r4;
      r4 = r5;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto step_any = [&](auto par, int u) {
      Info i_u3;
      if constexpr (kPair && decltype(par)::value == 0) i_u3 = info_second(i_u2);   // u + 3 odd
      else i_u3 = info(u + 3, r3);
      if constexpr (kDma) {
        step(par, std::true_type{}, u, i_u3);   // partial tiles are handled inside
      } else {
        if (is_full(i_u1) && is_full(i_u3)) step(par, std::true_type{}, u, i_u3);
        else step(par, std::false_type{}, u, i_u3);
      }
    };
    for (int u = 0; u < nsub; u += 2) {
      step_any(I0{}, u);
      if (u + 1 < nsub) step_any(I1{}, u + 1);
    }
  }
  // vector reads of O (epilogue) 12+ wait states after the last P V MFMA
  if constexpr (kDma) fence_o();
  // the last sub-tiles' (zero) loads must land before the LDS is reused
  if constexpr (kDma) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: normalize, LSE, rows out through LDS for coalesced stores ----
  // 16 rows of float32 per pass in K slot 0, 16-byte chunks XOR-swizzled by
  // the row so the column writes of 16 rows fall on distinct banks.
  // A part of a split row leaves O unnormalized, with its reference max and
  // row sum, in its workspace slot instead.
  float* ostage = reinterpret_cast<float*>(k_lds0);
  T* Ob = reinterpret_cast<T*>(a.out) + (int64_t)bh * a.seq_alloc * D;
  constexpr int QB = 32 * QT;
  float* wsO = part_item ? a.ws + (int64_t)blockIdx.x * QB * D : nullptr;
  float* wsM = part_item ? a.ws + (int64_t)a.n_dense * QB * D + (int64_t)blockIdx.x * QB : nullptr;
  float* wsL = part_item ? wsM + (int64_t)a.n_dense * QB : nullptr;
  constexpr int C8 = D / 8;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l = add_xor32(l_run[qt]);
    const float inv = part_item ? 1.0f : (l > 0.0f ? 1.0f / l : 0.0f);
    const int64_t qrow0 = q0 + 32 * qt;
    if (part_item) {
      if (hf == 0) {
        wsM[32 * qt + qc] = m_run[qt];
        wsL[32 * qt + qc] = l;
      }
    } else if (hf == 0 && a.lse) {
      const int64_t row = qrow0 + qc;
      const float mu = m_run[qt] == -INFINITY ? 0.0f : m_run[qt];
      if (row < a.seq_alloc)
        a.lse[(int64_t)bh * a.seq_alloc + row] = (row < a.S && l > 0.0f) ? (mu + __log2f(l)) * kLn2 : -INFINITY;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // O^T register r of d tile dt is d = 32dt + 8(r/4) + 4hf + r%4 of query qc
      if ((qc >> 4) == half) {
        const int q = qc & 15;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          f32x16 t = o[qt][dt];
          if constexpr (kDma) asm volatile("" : "+v"(t));   // one tile in vector registers at a time
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int ch = 8 * dt + 2 * r4 + hf;
            *reinterpret_cast<f32x4*>(ostage + q * D + ((ch ^ q) * 4)) =
                f32x4{t[4 * r4], t[4 * r4 + 1], t[4 * r4 + 2], t[4 * r4 + 3]} * inv;
          }
        }
      }
      for (int e = lane; e < 16 * C8; e += 64) {
        const int q = e / C8, c8 = e % C8;
        const int64_t row = qrow0 + 16 * half + q;
        if (row >= a.seq_alloc) continue;
        float v[8];
        if (row < a.S) {
          const float4 x = *reinterpret_cast<const float4*>(ostage + q * D + (((2 * c8) ^ q) * 4));
          const float4 y = *reinterpret_cast<const float4*>(ostage + q * D + (((2 * c8 + 1) ^ q) * 4));
          v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
          v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) v[c] = 0.0f;
        }
        if (part_item) store8<float>(wsO + (row - q0) * D + c8 * 8, v);
        else store8<T>(Ob + row * D + c8 * 8, v);
      }
    }
  }
}

// Merge of the parts of split frame-0 rows.  Part p of a row holds, per
// query row, unnormalized O_p, the reference max m_p (log2 domain) and the
// row sum l_p of its own key blocks; with M = max_p m_p and w_p = 2^(m_p - M)
// the row's attention over the union of the parts is sum_p w_p O_p divided
// by sum_p w_p l_p, and its LSE is (M + log2 sum_p w_p l_p) ln 2: the same
// exact softmax the one-wave row computes (AB-Attention page, TL;DR).  A part
// with no keys (m_p = -inf) adds nothing; a row with none is 0, LSE -inf.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(FwdArgs a) {
  constexpr int C8 = D / 8;
  const int QB = a.q_block, P = a.split;
  const int per_row = (QB * C8 + 255) / 256;       // workgroups per split row
  const int r = blockIdx.x / per_row;              // split row: items r * split .. + split - 1
  const int bh = r % a.BH, qb = a.dense_first + r / a.BH;
  const int64_t q0 = (int64_t)qb * QB;
  const float* wsO = a.ws;
  const float* wsM = a.ws + (int64_t)a.n_dense * QB * D;
  const float* wsL = wsM + (int64_t)a.n_dense * QB;
  T* Ob = reinterpret_cast<T*>(a.out) + (int64_t)bh * a.seq_alloc * D;
  {
    const int e = (blockIdx.x % per_row) * 256 + threadIdx.x;   // (query row, 8-channel chunk) of the row
    if (e >= QB * C8) return;
    const int q = e / C8, c8 = e % C8;
    const int64_t row = q0 + q;
    if (row >= a.seq_alloc) return;
    float M = -INFINITY;
    for (int p = 0; p < P; ++p) M = fmaxf(M, wsM[((int64_t)r * P + p) * QB + q]);
    float L = 0.0f;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
    for (int p = 0; p < P; ++p) {
      const int64_t it = (int64_t)r * P + p;
      const float mp = wsM[it * QB + q];
      if (mp == -INFINITY) continue;
      const float w = exp2f(mp - M);
      L += w * wsL[it * QB + q];
      const float4* src = reinterpret_cast<const float4*>(wsO + (it * QB + q) * D + c8 * 8);
      const float4 x = src[0], y = src[1];
      acc[0] += w * x.x; acc[1] += w * x.y; acc[2] += w * x.z; acc[3] += w * x.w;
      acc[4] += w * y.x; acc[5] += w * y.y; acc[6] += w * y.z; acc[7] += w * y.w;
    }
    const bool live = row < a.S && L > 0.0f;
    const float inv = live ? 1.0f / L : 0.0f;
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = live ? acc[c] * inv : 0.0f;
    store8<T>(Ob + row * D + c8 * 8, v);
    if (c8 == 0 && a.lse) a.lse[(int64_t)bh * a.seq_alloc + row] = live ? (M + __log2f(L)) * kLn2 : -INFINITY;
  }
}

template <typename T>
hipError_t launch_merge(const FwdArgs& a, int head_dim, hipStream_t stream) {
  const int per_row = (a.q_block * (head_dim / 8) + 255) / 256;
  const dim3 grid((unsigned)((int64_t)(a.n_dense / a.split) * per_row)), block(256);
  if (head_dim == 64) hipLaunchKernelGGL((merge_kernel<T, 64>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((merge_kernel<T, 128>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int QT>
hipError_t launch_bk(const FwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)forward_grid(a));
  const dim3 block(64);
  switch (a.k_block) {
    case 16: hipLaunchKernelGGL((fwd_kernel<T, D, QT, 16>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((fwd_kernel<T, D, QT, 32>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((fwd_kernel<T, D, QT, 64>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_q(const FwdArgs& a, hipStream_t stream) {
  return a.q_block == 32 ? launch_bk<T, D, 1>(a, stream) : launch_bk<T, D, 2>(a, stream);
}

template <typename T>
hipError_t launch_d(const FwdArgs& a, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_q<T, 64>(a, stream) : launch_q<T, 128>(a, stream);
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, int dtype, int head_dim, hipStream_t stream) {
  const hipError_t e = dtype != 0 ? launch_forward_f32(a, head_dim, stream)
                       : forward_wide_supported(dtype, head_dim, a.q_block, a.k_block)
                           ? launch_forward_wide(a, stream)
                           : launch_d<bf16_t>(a, head_dim, stream);
  if (e != hipSuccess || a.split <= 1 || a.n_dense == 0) return e;
  return dtype == 0 ? launch_merge<bf16_t>(a, head_dim, stream) : launch_merge<float>(a, head_dim, stream);
}

}  // namespace bsa
