// Block-sparse attention forward on gfx950 (MI355X).
//
// Pages: "AB-Attention: accurate block-sparse attention for video diffusion"
// (TL;DR: exact attention only on the selected key/value blocks; key blocks
// smaller than a tile gathered into full tiles; inverse-inclusion-probability
// reweighting) and "Attention matrix view: make only frame-0 query rows
// dense" (sec. 2: a dense row attends to every key/value token).
//
// Work decomposition (CDNA4-first):
//   * one workgroup = one (b, h, query block) of QROWS rows, 4 waves;
//   * the row's selected key blocks are cut into 64-key tiles (64/BK blocks
//     per tile, so 16-key blocks are gathered four per tile), and the tiles
//     are dealt round-robin to the 4 waves; every wave keeps all QROWS rows,
//     so no K/V tile is shared between waves and the only cross-wave step is
//     one log-sum-exp merge at the end;
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 (float32
//     accumulate).  Computing the transposes keeps each query row in a fixed
//     lane (lane & 15) for S, P and O alike, so the online-softmax state
//     (running max, partial sum, rescale) never moves between lanes;
//   * K rows are loaded straight from HBM/L2 into the A-operand registers
//     (16 bytes per lane), in a permuted order chosen so that the P^T
//     B-operand of each lane covers 8 consecutive keys; V goes through a
//     per-wave LDS tile that is read back transposed;
//   * softmax in the log2 domain (exp2 on the hardware transcendental),
//     scale and per-block log-weight folded into one multiply-add.
#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kFwdThreads = 128;   // two waves: each owns half of the query block's rows
constexpr int kWaves = 2;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kListCap = 2048;     // list entries of a row cached in LDS (the rest read from global)

template <typename T>
struct Ld8;

template <>
struct Ld8<bf16_t> {
  static __device__ __forceinline__ uint4 raw(const bf16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <>
struct Ld8<float> {
  static __device__ __forceinline__ uint4 raw(const float* p) {
    const float4 x = reinterpret_cast<const float4*>(p)[0];
    const float4 y = reinterpret_cast<const float4*>(p)[1];
    uint4 r;
    r.x = pack_bf16x2(x.x, x.y);
    r.y = pack_bf16x2(x.z, x.w);
    r.z = pack_bf16x2(y.x, y.y);
    r.w = pack_bf16x2(y.z, y.w);
    return r;
  }
};

__device__ __forceinline__ bf16x8 as_frag(uint4 r) { return __builtin_bit_cast(bf16x8, r); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOob = 0x80000000u;   // byte offset past any buffer: the load returns zeros

// Range-checked loads of 8 consecutive elements (as 8 bf16) through a buffer
// resource; an offset >= the resource size reads zeros, so invalid key rows
// need no branch.
template <typename T>
struct BufLd8;

template <>
struct BufLd8<bf16_t> {
  static __device__ __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, uint32_t elem_off) {
    const uint32_t byte = elem_off == kOob ? kOob : elem_off * 2u;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
};

template <>
struct BufLd8<float> {
  static __device__ __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, uint32_t elem_off) {
    const uint32_t byte = elem_off == kOob ? kOob : elem_off * 4u;
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte, 0, 0);
    const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(byte == kOob ? kOob : byte + 16u), 0, 0);
    uint4 o;
    o.x = pack_bf16x2(__uint_as_float(x[0]), __uint_as_float(x[1]));
    o.y = pack_bf16x2(__uint_as_float(x[2]), __uint_as_float(x[3]));
    o.z = pack_bf16x2(__uint_as_float(y[0]), __uint_as_float(y[1]));
    o.w = pack_bf16x2(__uint_as_float(y[2]), __uint_as_float(y[3]));
    return o;
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ void store8(T* dst, const float (&v)[8]);

template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* dst, const float (&v)[8]) {
  uint4 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  r.z = pack_bf16x2(v[4], v[5]);
  r.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(dst) = r;
}

template <>
__device__ __forceinline__ void store8<float>(float* dst, const float (&v)[8]) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS chunk swizzles (16-byte chunks of a row of D bf16).  K rows are read
// as 16-byte A-operand pieces by 16 lanes at once; V rows are read with the
// transposing 8-byte load by groups of 4 lanes per row.  The XOR patterns
// below put those simultaneous accesses on distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128) return 4 * (r >> 3) + (r & 3);                 // 0..15
  else return ((r >> 1) & 1) | (((r >> 3) & 3) << 1);                    // 0..7
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {                            // even: keeps chunk pairs
  if constexpr (D == 128) return 2 * ((r & 3) | (((r >> 3) & 1) << 2));  // 0..14
  else return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));              // 0..6
}

// Row of the 32-key sub-tile supplied by A-operand row m of S^T M-tile mt.
// With this order the accumulator rows a lane holds for M-tiles 0 and 1 are
// the 8 consecutive keys 8*(lane/16) + 0..7 -- exactly the K-range the lane
// supplies as B operand of O^T += V^T P^T.
__device__ __forceinline__ int a_row(int mt, int m) { return 8 * (m >> 2) + 4 * mt + (m & 3); }

template <typename T, int D, int QROWS, int BK>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_kernel(FwdArgs a) {
  constexpr int RW = QROWS / kWaves;   // query rows per wave
  constexpr int NT = RW / 16;          // query column tiles of S^T / O^T
  constexpr int DC = D / 32;           // K-chunks of the Q.K contraction
  constexpr int DT = D / 16;           // d row tiles of O^T
  constexpr int KCH = D / 8;           // 16-byte chunks per row
  constexpr int SUB = 32;              // keys per sub-tile
  constexpr int TILE_E = SUB * D;      // bf16 elements of one K (or V) sub-tile
  constexpr int NLD = SUB * KCH / kFwdThreads;   // 16-byte loads per thread per operand
  constexpr int RPL = kFwdThreads / KCH;         // tile rows covered by one load round
  constexpr int NBLK = BK >= SUB ? 1 : SUB / BK; // key blocks per sub-tile
  constexpr int OS = D + 4;            // LDS row stride of the output staging (floats)
  constexpr float kTau = 8.0f;         // lazy rescale: tolerated growth of the running max (log2)
  static_assert(NT >= 1 && NLD >= 1 && NBLK <= 2, "tile shape");
  constexpr int kTileHalves = 2 * 2 * TILE_E;                     // bf16 units
  constexpr int kStageHalves = QROWS * OS * 2;                     // output staging, bf16 units
  // two stages of (K, V) sub-tiles; reused for the output rows at the end
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kTileHalves > kStageHalves ? kTileHalves : kStageHalves];
  __shared__ uint16_t lst[kListCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;           // query column (S^T, O^T) / A-operand row
  const int grp = lane >> 4;           // 0..3: K sub-range of the operands

  // heaviest-first order: all heads of query block 0, then of block 1, ...
  const int bh = blockIdx.x % a.BH;
  const int qb = blockIdx.x / a.BH;
  const int64_t rowid = (int64_t)bh * a.nqb + qb;
  const int cnt = min(max(a.cnt[rowid], 0), a.nkb);   // a row never reads past its nkb slots
  const int32_t* list = a.idx + rowid * a.nkb;
  const float* lw = a.logw ? a.logw + rowid * a.nkb : nullptr;
  const int nsub = (cnt * BK + SUB - 1) / SUB;          // 32-key sub-tiles of the row

  const T* Qb = reinterpret_cast<const T*>(a.q) + (int64_t)bh * a.seq_alloc * D;
  const T* Kb = reinterpret_cast<const T*>(a.k) + (int64_t)bh * a.seq_alloc * D;
  const T* Vb = reinterpret_cast<const T*>(a.v) + (int64_t)bh * a.seq_alloc * D;
  const int64_t q0 = (int64_t)qb * a.q_block + wave * RW;     // this wave's first row
  const int S32 = (int)a.S;

  // ---- the row's block list in LDS (entries past kListCap read from global) ----
  for (int e = tid; e < min(cnt, kListCap); e += kFwdThreads) {
    const int j = list[e];
    lst[e] = (j >= 0 && j < a.nkb) ? (uint16_t)j : (uint16_t)0xffff;
  }
  __syncthreads();
  auto block_at = [&](int pos) -> int {          // -1: past the list or a bad index
    int j = -1;
    if (pos < cnt) {
      if (pos < kListCap) {
        j = lst[pos];
        j = j == 0xffff ? -1 : j;
      } else {
        j = list[pos];
        j = (j >= 0 && j < a.nkb) ? j : -1;
      }
    }
    return __builtin_amdgcn_readfirstlane(j);     // wave-uniform
  };

  const uint32_t nbytes = (uint32_t)a.seq_alloc * (uint32_t)D * (uint32_t)sizeof(T);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)Kb, 0, (int)nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, 0, (int)nbytes, 0x00020000);

  // ---- Q^T fragments (B operand of S^T = K Q^T), kept for the whole row ----
  bf16x8 qf[NT][DC];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t row = q0 + nt * 16 + col;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (row < a.S) r = Ld8<T>::raw(Qb + row * D + dc * 32 + grp * 8);
      qf[nt][dc] = as_frag(r);
    }
  }

  // ---- per-thread constant offsets ----
  // Staging load n of this thread fills LDS chunk n*128 + tid: tile row
  // srow(n) = n*RPL + tid/KCH, holding logical chunk (tid % KCH) ^ swizzle(row).
  // Its global element offset is key0(part) * D + (row - part*PART) * D + chunk*8;
  // the part of load n is the same for every thread, so only the last two terms
  // (kc/vc) are per-thread constants.
  constexpr int PART = SUB / NBLK;
  int rin[NLD];
  uint32_t kc[NLD], vc[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int r = n * RPL + tid / KCH;
    rin[n] = r - ((n * RPL) / PART) * PART;
    kc[n] = (uint32_t)(rin[n] * D + ((tid % KCH) ^ swz_k<D>(r)) * 8);
    vc[n] = (uint32_t)(rin[n] * D + ((tid % KCH) ^ swz_v<D>(r)) * 8);
  }
  // K A-operand reads.  For row r = a_row(mt, col) the swizzled chunk is
  // (4*dc + grp) ^ swz_k(r) = (4*dc) ^ (grp ^ swz_k(r)), and the row term has
  // zero bits where the chunk index lives, so byte address = ka ^ (dc * 64),
  // plus 4 rows (8*D bytes) for mt = 1 (row + 4 leaves swz_k unchanged).
  const uint32_t ka = [&] {
    const int r = a_row(0, col);
    return (uint32_t)(r * KCH * 16) | (uint32_t)(((uint32_t)grp ^ (uint32_t)swz_k<D>(r)) * 16);
  }();
  // V^T transposing reads for (dt, hh): row r = 8*grp + 4*hh + col/4, logical
  // chunk 2*dt + (col&3)/2, pair swizzle s: byte address = va ^ (dt * 32), plus
  // 4 rows (8*D bytes) for hh = 1 (row + 4 leaves swz_v unchanged).
  const uint32_t va = [&] {
    const int r = 8 * grp + (col >> 2);
    return (uint32_t)(r * D * 2) | (uint32_t)(swz_v<D>(r) * 16) | (uint32_t)(((col & 3) >> 1) * 16) |
           (uint32_t)((col & 1) * 8);
  }();

  float m_run[NT];
  f32x4 o[DT][NT], lacc[NT];           // O^T and the row sums (ones-row MFMA)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    lacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = as_frag(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));

  // ---- sub-tile geometry: key blocks, first key, valid keys, log2 weight ----
  struct SubInfo {
    int key0[NBLK];      // first key of each block part, or -1
    int valid[NBLK];     // valid keys of each part (0..min(BK,32))
    float bias[NBLK];
  };
  auto info = [&](int u) {
    SubInfo si;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int g = u * SUB + b * (SUB / NBLK);
      const int pos = g / BK;
      const int j = block_at(pos);
      const int key0 = j * BK + g % BK;
      si.key0[b] = j >= 0 ? key0 : -1;
      si.valid[b] = j >= 0 ? min(max(S32 - key0, 0), SUB / NBLK) : 0;
      si.bias[b] = (lw && j >= 0) ? lw[pos] * 1.4426950408889634f : 0.0f;
    }
    return si;
  };

  // ---- staging: both waves load half of a sub-tile, 16 bytes per load ----
  uint4 kst[NLD], vst[NLD];
  auto stage = [&](int u) {
    const SubInfo si = info(u);
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int b = (n * RPL) / PART;                // the part is the same for all threads of load n
      const bool ok = rin[n] < si.valid[b];
      const uint32_t base = (uint32_t)si.key0[b] * (uint32_t)D;
      kst[n] = BufLd8<T>::load(rk, ok ? base + kc[n] : kOob);
      vst[n] = BufLd8<T>::load(rv, ok ? base + vc[n] : kOob);
    }
  };
  auto commit = [&](int stage_buf) {
    uint16_t* tk = tiles + stage_buf * 2 * TILE_E;
    uint16_t* tv = tk + TILE_E;
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      *reinterpret_cast<uint4*>(tk + (n * kFwdThreads + tid) * 8) = kst[n];
      *reinterpret_cast<uint4*>(tv + (n * kFwdThreads + tid) * 8) = vst[n];
    }
  };

  // ---- one sub-tile of attention from LDS buffer `buf` ----
  auto compute = [&](int u, const int buf) {
    const unsigned char* tk = reinterpret_cast<const unsigned char*>(tiles) + buf * 2 * TILE_E * 2;
    const unsigned char* tv = tk + TILE_E * 2;
    const SubInfo si = info(u);
    // this lane's 8 accumulator rows are tile rows 8*grp .. 8*grp+7 (one part)
    const int part = NBLK == 1 ? 0 : (grp >> 1);
    const int lim = min(max(si.valid[NBLK == 1 ? 0 : part] - (NBLK == 1 ? 8 * grp : 8 * (grp & 1)), 0), 8);
    float bias = si.bias[0];
    if constexpr (NBLK == 2) bias = part ? si.bias[1] : si.bias[0];
    bool full = true;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) full = full && si.valid[b] == SUB / NBLK;

    // S^T = K Q^T
    f32x4 sacc[2][NT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      bf16x8 kf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kf[dc] = as_frag(*reinterpret_cast<const uint4*>(tk + mt * (8 * D) + (ka ^ (uint32_t)(dc * 64))));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[dc], qf[nt][dc], c, 0, 0, 0);
        sacc[mt][nt] = c;
      }
    }
    if (!full) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            if (4 * mt + r >= lim) sacc[mt][nt][r] = -INFINITY;
    }
    // row max of the raw scores (scale > 0; the lane's 8 keys share one weight)
    bool grow = false;
    float mrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][nt][0], sacc[0][nt][1]), fmaxf(sacc[0][nt][2], sacc[0][nt][3])),
                       fmaxf(fmaxf(sacc[1][nt][0], sacc[1][nt][1]), fmaxf(sacc[1][nt][2], sacc[1][nt][3])));
      mx = mx * a.scale_log2 + bias;
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      mrow[nt] = mx;
      grow |= mx > m_run[nt] + kTau;
    }
    // lazy rescale: the reference max only moves when a row's max grows by more
    // than kTau (so p <= 2^kTau); O and l are rescaled only then
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float m_new = mrow[nt] > m_run[nt] + kTau ? mrow[nt] : m_run[nt];
        const float alpha = fast_exp2(m_run[nt] - (m_new == -INFINITY ? 0.0f : m_new));
        m_run[nt] = m_new;
        lacc[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][nt] *= alpha;
      }
    }
    // p = exp2(s * scale + bias - m); P^T as B operand (keys 8*grp + e)
    bf16x8 pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float off = bias - (m_run[nt] == -INFINITY ? 0.0f : m_run[nt]);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(sacc[e >> 2][nt][e & 3] * a.scale_log2 + off);
      uint4 w;
      w.x = pack_bf16x2(p[0], p[1]);
      w.y = pack_bf16x2(p[2], p[3]);
      w.z = pack_bf16x2(p[4], p[5]);
      w.w = pack_bf16x2(p[6], p[7]);
      pb[nt] = as_frag(w);
      lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[nt], lacc[nt], 0, 0, 0);
    }
    // O^T += V^T P^T with V^T fragments from transposing LDS reads
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const unsigned char* vp = tv + (va ^ (uint32_t)(dt * 32));
      const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vp));
      const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vp + 8 * D));
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[nt], o[dt][nt], 0, 0, 0);
    }
  };

  // ---- pipeline: sub-tile u computed from buffer u&1 while u+2 loads ----
  if (nsub > 0) {
    stage(0);
    commit(0);
    if (nsub > 1) stage(1);
  }
  __syncthreads();
  for (int u = 0; u < nsub; ++u) {
    const int buf = u & 1;
    // sub-tile u+1 (staged during the previous step) -> the other buffer;
    // then start loading sub-tile u+2 while this one is computed
    if (u + 1 < nsub) {
      commit(buf ^ 1);
      if (u + 2 < nsub) stage(u + 2);
    }
    compute(u, buf);
    __syncthreads();   // buffer `buf` is rewritten two steps later; buf^1 is complete for step u+1
  }

  // ---- epilogue: normalize, LSE, rows out through LDS for coalesced stores ----
  float* ostage = reinterpret_cast<float*>(tiles) + wave * RW * OS;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = lacc[nt][0];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(ostage + (nt * 16 + col) * OS + dt * 16 + 4 * grp) = o[dt][nt] * inv;
    if (grp == 0 && a.lse) {
      const int64_t row = q0 + nt * 16 + col;
      const float mu = m_run[nt] == -INFINITY ? 0.0f : m_run[nt];
      if (row < a.seq_alloc)
        a.lse[(int64_t)bh * a.seq_alloc + row] = (row < a.S && l > 0.0f) ? (mu + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  T* Ob = reinterpret_cast<T*>(a.out) + (int64_t)bh * a.seq_alloc * D;
  constexpr int C8 = D / 8;
  for (int e = lane; e < RW * C8; e += 64) {
    const int q = e / C8, c8 = e % C8;
    const int64_t row = q0 + q;
    if (row >= a.seq_alloc) continue;
    float v[8];
    if (row < a.S) {
      const float4 x = *reinterpret_cast<const float4*>(ostage + q * OS + c8 * 8);
      const float4 y = *reinterpret_cast<const float4*>(ostage + q * OS + c8 * 8 + 4);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = 0.0f;
    }
    store8<T>(Ob + row * D + c8 * 8, v);
  }
}

template <typename T, int D, int QROWS>
hipError_t launch_bk(const FwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.BH * a.nqb));
  switch (a.k_block) {
    case 16: hipLaunchKernelGGL((fwd_kernel<T, D, QROWS, 16>), grid, dim3(kFwdThreads), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((fwd_kernel<T, D, QROWS, 32>), grid, dim3(kFwdThreads), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((fwd_kernel<T, D, QROWS, 64>), grid, dim3(kFwdThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_q(const FwdArgs& a, hipStream_t stream) {
  return a.q_block == 32 ? launch_bk<T, D, 32>(a, stream) : launch_bk<T, D, 64>(a, stream);
}

template <typename T>
hipError_t launch_d(const FwdArgs& a, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_q<T, 64>(a, stream) : launch_q<T, 128>(a, stream);
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, int dtype, int head_dim, hipStream_t stream) {
  return dtype == 0 ? launch_d<bf16_t>(a, head_dim, stream) : launch_d<float>(a, head_dim, stream);
}

}  // namespace bsa
