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

constexpr float kLn2 = 0.69314718055994530942f;

template <typename T>
struct Ld8;

template <>
struct Ld8<bf16_t> {
  static __device__ __forceinline__ uint4 raw(const bf16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
};

// Two floats as two bf16 (round to nearest even) in one dword: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};


// x combined with the same register of lane ^ 32 (one v_permlane32_swap).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS chunk swizzles of the 32-row K and V sub-tiles (16-byte chunks of a row
// of D bf16).  K rows are read as 16-byte A-operand pieces, 16 consecutive
// rows at the same logical chunk per access; V rows are read with the
// transposing 8-byte load, 4 consecutive rows x 4 chunks per 16 lanes.  The
// XOR patterns put each access group on distinct banks; they only touch chunk
// bits, so every address is (lane base) ^ (per-fragment constant).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128) return 4 * (r & 3);
  else return 4 * ((r >> 1) & 1);
}

// blockIdx -> (head, query block); false for the few padding workgroups.
__device__ __forceinline__ bool schedule(const FwdArgs& a, int t, int& bh, int& qb) {
  if (t < a.n_dense) {
    bh = t % a.BH;
    qb = a.dense_first + t / a.BH;
    return true;
  }
  const int nd = a.dense_first >= 0 ? a.dense_last - a.dense_first + 1 : 0;
  const int ns = a.nqb - nd;                       // other rows per head
  const int x = t % kXcds, k = t / kXcds;
  const int k0 = (a.n_dense + kXcds - 1 - x) / kXcds;
  const int ls = x * a.per_xcd + (k - k0);         // rank among the other rows
  if (ls >= a.BH * ns) return false;
  bh = ls / ns;
  const int r = ls % ns;
  // r-th row of the head when rows are ordered by (index mod period, index)
  const int P = a.period;
  const int c = (ns + P - 1) / P;
  const int m = ns % P == 0 ? P : ns % P;          // residues with c rows; the rest have c - 1
  int res, kk;
  if (r < m * c) {
    res = r / c;
    kk = r % c;
  } else {
    const int r2 = r - m * c;
    res = m + r2 / (c - 1);
    kk = r2 % (c - 1);
  }
  const int s = res + kk * P;
  qb = (a.dense_first < 0 || s < a.dense_first) ? s : s + nd;
  return true;
}

template <typename T, int D, int QROWS, int BK>
__global__ __launch_bounds__(QROWS * 2, QROWS == 64 ? 2 : 1) void fwd_kernel(FwdArgs a) {
  constexpr bool kDma = sizeof(T) == 2;  // bf16 tiles go HBM -> LDS directly; f32 is converted in registers
  constexpr int NW = QROWS / 32;       // waves: each owns 32 query rows
  constexpr int NTH = NW * 64;         // threads
  constexpr int KC = D / 16;           // K-chunks of the Q.K contraction (32x32x16)
  constexpr int DT = D / 32;           // d tiles of O^T
  constexpr int KCH = D / 8;           // 16-byte chunks per row
  constexpr int SUB = 32;              // keys per sub-tile
  constexpr int TILE_E = SUB * D;      // bf16 elements of one K (or V) sub-tile
  constexpr int NLD = SUB * KCH / NTH; // 16-byte loads per thread per operand
  constexpr int RPL = NTH / KCH;       // tile rows covered by one load round
  constexpr int NBLK = BK >= SUB ? 1 : SUB / BK;   // key blocks per sub-tile
  constexpr int PART = SUB / NBLK;
  constexpr int OS = D + 4;            // LDS row stride of the output staging (floats)
  constexpr float kTau = 8.0f;         // lazy rescale: tolerated growth of the running max (log2)
  static_assert(NW >= 1 && NLD >= 1 && NBLK <= 2, "tile shape");
  constexpr int kTileHalves = 4 * TILE_E;          // K0, V0, K1, V1 (bf16 units)
  constexpr int kStageHalves = QROWS * OS * 2;     // output staging (bf16 units)
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kTileHalves > kStageHalves ? kTileHalves : kStageHalves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int qc = lane & 31;            // query column of S^T / O^T, A-operand row
  const int hf = lane >> 5;            // 0/1: K half of the operands, row half of the accumulators

  int bh, qb;
  if (!schedule(a, blockIdx.x, bh, qb)) return;
  const int64_t rowid = (int64_t)bh * a.nqb + qb;
  const int cnt = min(max(a.cnt[rowid], 0), a.nkb);   // a row never reads past its nkb slots
  const int32_t* list = a.idx + rowid * a.nkb;
  const float* lw = a.logw ? a.logw + rowid * a.nkb : nullptr;
  const int nsub = (cnt * BK + SUB - 1) / SUB;          // 32-key sub-tiles of the row

  const T* Qb = reinterpret_cast<const T*>(a.q) + (int64_t)bh * a.seq_alloc * D;
  const T* Kb = reinterpret_cast<const T*>(a.k) + (int64_t)bh * a.seq_alloc * D;
  const T* Vb = reinterpret_cast<const T*>(a.v) + (int64_t)bh * a.seq_alloc * D;
  const int64_t q0 = (int64_t)qb * a.q_block + wave * 32;     // this wave's first row
  const int S32 = (int)a.S;

  // block index of list slot pos (-1 past the list or for a bad index) and its
  // log2-domain weight.  The lists are read-only for the whole launch, so they
  // are read through the constant address space: uniform indices become scalar
  // loads that never wait on the tile loads in flight.
  typedef const __attribute__((address_space(4))) int32_t* cint_p;
  typedef const __attribute__((address_space(4))) float* cflt_p;
  const cint_p lst = (cint_p)list;
  const cflt_p lwr = (cflt_p)lw;
  auto block_at = [&](int pos) -> int {
    if (pos >= cnt) return -1;
    const int j = lst[pos];
    return (j >= 0 && j < a.nkb) ? j : -1;
  };

  const uint32_t nbytes = (uint32_t)a.seq_alloc * (uint32_t)D * (uint32_t)sizeof(T);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)Kb, 0, (int)nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, 0, (int)nbytes, 0x00020000);

  // ---- Q^T fragments (B operand of S^T = K Q^T): Q[q][16c + 8hf .. +7] ----
  bf16x8 qf[KC];
  {
    const int64_t row = q0 + qc;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (row < a.S) r = Ld8<T>::raw(Qb + row * D + c * 16 + hf * 8);
      qf[c] = as_frag(r);
    }
  }

  // ---- per-thread constant offsets ----
  // Tile load n of this thread fills LDS chunk n*NTH + tid: tile row
  // r = n*RPL + tid/KCH, holding logical chunk (tid % KCH) ^ swizzle(r).  Its
  // global element offset is key0(part) * D + (r - part*PART) * D + chunk*8,
  // and the part of load n is the same for every thread.
  int rin[NLD];
  uint32_t kc[NLD], vc[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int r = n * RPL + tid / KCH;
    rin[n] = r - ((n * RPL) / PART) * PART;
    kc[n] = (uint32_t)(rin[n] * D + ((tid % KCH) ^ swz_k<D>(r)) * 8);
    vc[n] = (uint32_t)(rin[n] * D + ((tid % KCH) ^ swz_v<D>(r)) * 8);
  }
  // K A-operand read of chunk c: tile row qc, logical chunk 2c + hf:
  // byte address ka ^ (c * 32).
  const uint32_t ka = (uint32_t)(qc * KCH * 16) | (uint32_t)((hf ^ swz_k<D>(qc)) * 16);
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

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

  // ---- sub-tile geometry: first key, valid keys and log2 weight of each part ----
  // The raw list entries of a sub-tile are fetched (scalar loads) one step
  // before they are turned into its geometry, so the loads never stall a step.
  struct Raw {
    int j[NBLK];
    float w[NBLK];
  };
  struct SubInfo {
    int key0[NBLK];      // first key of each part (0 if none)
    int valid[NBLK];     // valid keys of each part
    float bias[NBLK];
  };
  auto fetch = [&](int u) {
    Raw r;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int pos = (u * SUB + b * PART) / BK;
      r.j[b] = block_at(pos);
      r.w[b] = (pos < cnt && lwr) ? lwr[pos] : 0.0f;
    }
    return r;
  };
  auto make_info = [&](int u, const Raw& r) {
    SubInfo si;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int g = u * SUB + b * PART;
      const int j = r.j[b];
      const int key0 = j * BK + g % BK;
      si.key0[b] = j >= 0 ? key0 : 0;
      si.valid[b] = j >= 0 ? min(max(S32 - key0, 0), PART) : 0;
      si.bias[b] = j >= 0 ? r.w[b] * 1.4426950408889634f : 0.0f;
    }
    return si;
  };

  auto kbuf = [&](int b) { return tiles + b * 2 * TILE_E; };
  auto vbuf = [&](int b) { return tiles + b * 2 * TILE_E + TILE_E; };

  // ---- a sub-tile's K and V rows -> LDS buffer b ----
  uint4 kst[kDma ? 1 : NLD], vst[kDma ? 1 : NLD];   // f32 only: staged in registers
  auto load_tiles = [&](const SubInfo& si, int b) {
    bool full = true;
#pragma unroll
    for (int p = 0; p < NBLK; ++p) full = full && si.valid[p] == PART;
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int part = (n * RPL) / PART;
      const bool ok = rin[n] < si.valid[part];
      const uint32_t base = (uint32_t)si.key0[part] * (uint32_t)D;
      if constexpr (kDma) {
        // this wave's 64 lanes fill 1 KB of LDS at chunk n*NTH + 64*wave.  A full
        // sub-tile adds the uniform block base as soffset to constant voffsets;
        // otherwise invalid rows get an out-of-range voffset (the load writes zeros).
        uint32_t kv, vv, so;
        if (full) {
          kv = kc[n] * 2u;
          vv = vc[n] * 2u;
          so = base * 2u;
        } else {
          kv = ok ? (base + kc[n]) * 2u : kOob;
          vv = ok ? (base + vc[n]) * 2u : kOob;
          so = 0;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(kbuf(b) + (n * NTH + 64 * wave) * 8), 16, (int)kv, (int)so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(vbuf(b) + (n * NTH + 64 * wave) * 8), 16, (int)vv, (int)so, 0, 0);
      } else {
        kst[n] = BufLd8<T>::load(rk, ok ? base + kc[n] : kOob);
        vst[n] = BufLd8<T>::load(rv, ok ? base + vc[n] : kOob);
      }
    }
    if constexpr (!kDma) {
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        *reinterpret_cast<uint4*>(kbuf(b) + (n * NTH + tid) * 8) = kst[n];
        *reinterpret_cast<uint4*>(vbuf(b) + (n * NTH + tid) * 8) = vst[n];
      }
    }
  };

  // ---- one sub-tile: S^T = K Q^T, online softmax, O^T += V^T P^T ----
  // accumulator register r of this lane is tile row 8*(r/4) + 4*hf + r%4
  auto compute = [&](const SubInfo& si, int b) {
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(kbuf(b));
    const unsigned char* vt = reinterpret_cast<const unsigned char*>(vbuf(b));
    f32x16 sc = f32x16{};
    {
      bf16x8 kf[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) kf[c] = as_frag(*reinterpret_cast<const uint4*>(kt + (ka ^ (uint32_t)(c * 32))));
#pragma unroll
      for (int c = 0; c < KC; ++c) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[c], sc, 0, 0, 0);
    }
    bool full = true;
#pragma unroll
    for (int p = 0; p < NBLK; ++p) full = full && si.valid[p] == PART;
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * hf + (r & 3);
        const int p = row / PART;
        if (row - p * PART >= si.valid[p]) sc[r] = -INFINITY;
      }
    }
    // row max: the lane's 16 keys (v_max3 chains), then lane ^ 32 (scale > 0,
    // one weight per part)
    const float mx0 = fmaxf(fmaxf(fmaxf(fmaxf(sc[0], sc[1]), sc[2]), fmaxf(sc[3], sc[4])),
                            fmaxf(fmaxf(sc[5], sc[6]), sc[7]));
    const float mx1 = fmaxf(fmaxf(fmaxf(fmaxf(sc[8], sc[9]), sc[10]), fmaxf(sc[11], sc[12])),
                            fmaxf(fmaxf(sc[13], sc[14]), sc[15]));
    float mx;
    if constexpr (NBLK == 2) mx = fmaxf(mx0 * a.scale_log2 + si.bias[0], mx1 * a.scale_log2 + si.bias[1]);
    else mx = fmaxf(mx0, mx1) * a.scale_log2 + si.bias[0];
    mx = max_xor32(mx);
    // lazy rescale: the reference max moves only when the row max grows by more
    // than kTau (so p <= 2^kTau); O and l are rescaled only then
    if (__any(mx > m_run + kTau)) {
      const float m_new = mx > m_run + kTau ? mx : m_run;
      const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.0f : m_new));
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    const float mu = m_run == -INFINITY ? 0.0f : m_run;
    const float off0 = si.bias[0] - mu;
    const float off1 = si.bias[NBLK - 1] - mu;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(sc[r] * a.scale_log2 + (r < 8 ? off0 : off1));
    // P^T B operand of key chunk c: keys 16c + 8(e/4) + 4hf + e%4 = registers 8c + e;
    // the row sum adds exactly these bf16 values (v_dot2 with ones)
    bf16x8 pb[2];
    float ps = 0.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        w[k2] = pack_bf16x2(p[8 * c + 2 * k2], p[8 * c + 2 * k2 + 1]);
        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[k2]), kOnes2, ps, false);
      }
      pb[c] = as_frag(make_uint4(w[0], w[1], w[2], w[3]));
    }
    l_run += ps;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x8 vf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const unsigned char* vp = vt + (va ^ (uint32_t)(dt * 64)) + (16 * c) * D * 2;
        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vp));
        const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vp + 8 * D * 2));
        vf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c], pb[c], o[dt], 0, 0, 0);
    }
  };

  // ---- pipeline: one barrier per sub-tile ----
  // step u: wait for this wave's loads of sub-tile u, barrier (everyone's data
  // of u is in buffer u&1 and buffer (u+1)&1 is no longer read), start loading
  // sub-tile u+1 into buffer (u+1)&1, compute sub-tile u.
  SubInfo si_cur;
  Raw raw_next;
  if (nsub > 0) {
    si_cur = make_info(0, fetch(0));
    load_tiles(si_cur, 0);
    if (nsub > 1) raw_next = fetch(1);
  }
  for (int u = 0; u < nsub; ++u) {
    const int b = u & 1;
    if constexpr (kDma) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    SubInfo si_next;
    if (u + 1 < nsub) {
      si_next = make_info(u + 1, raw_next);
      load_tiles(si_next, b ^ 1);
      if (u + 2 < nsub) raw_next = fetch(u + 2);
    }
    compute(si_cur, b);
    si_cur = si_next;
  }
  __syncthreads();

  // ---- epilogue: normalize, LSE, rows out through LDS for coalesced stores ----
  const float l = add_xor32(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* ostage = reinterpret_cast<float*>(tiles) + wave * 32 * OS;
  // O^T register r of d tile dt is d = 32dt + 8(r/4) + 4hf + r%4 of query qc
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<f32x4*>(ostage + qc * OS + 32 * dt + 8 * r4 + 4 * hf) =
          f32x4{o[dt][4 * r4], o[dt][4 * r4 + 1], o[dt][4 * r4 + 2], o[dt][4 * r4 + 3]} * inv;
  if (hf == 0 && a.lse) {
    const int64_t row = q0 + qc;
    const float mu = m_run == -INFINITY ? 0.0f : m_run;
    if (row < a.seq_alloc)
      a.lse[(int64_t)bh * a.seq_alloc + row] = (row < a.S && l > 0.0f) ? (mu + __log2f(l)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  T* Ob = reinterpret_cast<T*>(a.out) + (int64_t)bh * a.seq_alloc * D;
  constexpr int C8 = D / 8;
  for (int e = lane; e < 32 * C8; e += 64) {
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
  const dim3 grid((unsigned)forward_grid(a));
  const dim3 block(QROWS * 2);
  switch (a.k_block) {
    case 16: hipLaunchKernelGGL((fwd_kernel<T, D, QROWS, 16>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((fwd_kernel<T, D, QROWS, 32>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((fwd_kernel<T, D, QROWS, 64>), grid, block, 0, stream, a); break;
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
