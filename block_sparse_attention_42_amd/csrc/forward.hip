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

constexpr int kFwdThreads = 256;
constexpr int kWaves = 4;
constexpr float kLn2 = 0.69314718055994530942f;

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

// Key slot (0..63 of a tile) held by row m of S^T M-tile mt.  Chosen so the
// accumulator rows a lane holds for M-tiles 2c and 2c+1 are the 8
// consecutive keys 32c + 8*(lane/16) + 0..7, which is exactly the K-range
// the lane must supply as B operand of O^T += V^T P^T.
__device__ __forceinline__ int a_slot(int mt, int m) {
  return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

template <typename T, int D, int QROWS, int BK>
__global__ __launch_bounds__(kFwdThreads) void fwd_kernel(FwdArgs a) {
  constexpr int NT = QROWS / 16;       // query column tiles of S^T / O^T
  constexpr int DC = D / 32;           // K-chunks of the Q.K contraction
  constexpr int DT = D / 16;           // d row tiles of O^T
  constexpr int NSUB = 64 / BK;        // key blocks per 64-key tile
  constexpr int VS = D + 2;            // LDS row stride of the V tile (bf16 units)
  constexpr int VBUF = 64 * VS;        // per-wave V tile (bf16 units)
  constexpr int OS = D + 4;            // LDS row stride of the merge buffers (floats)
  constexpr int kVBytes = kWaves * VBUF * 2;
  constexpr int kMergeBytes = 2 * QROWS * OS * 4;
  constexpr int kMainBytes = kVBytes > kMergeBytes ? kVBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kMainBytes + 2 * kWaves * QROWS * 4];
  uint16_t* vbuf_all = reinterpret_cast<uint16_t*>(smem);
  float* merge = reinterpret_cast<float*>(smem);
  float* st_m = reinterpret_cast<float*>(smem + kMainBytes);
  float* st_l = st_m + kWaves * QROWS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;           // query column (S^T, O^T) / A-operand row
  const int grp = lane >> 4;           // 0..3: K sub-range of the operands

  const int bh = blockIdx.x % a.BH;
  const int qb = blockIdx.x / a.BH;    // query block: all heads of block 0 first
  const int64_t rowid = (int64_t)bh * a.nqb + qb;
  const int cnt = min(max(a.cnt[rowid], 0), a.nkb);   // a row never reads past its nkb slots
  const int32_t* list = a.idx + rowid * a.nkb;
  const float* lw = a.logw ? a.logw + rowid * a.nkb : nullptr;
  const int ntiles = (cnt + NSUB - 1) / NSUB;

  const T* Qb = reinterpret_cast<const T*>(a.q) + (int64_t)bh * a.seq_alloc * D;
  const T* Kb = reinterpret_cast<const T*>(a.k) + (int64_t)bh * a.seq_alloc * D;
  const T* Vb = reinterpret_cast<const T*>(a.v) + (int64_t)bh * a.seq_alloc * D;
  const int64_t q0 = (int64_t)qb * a.q_block;
  const int64_t S = a.S;

  // ---- Q^T fragments (B operand of S^T = K Q^T), kept for the whole row ----
  bf16x8 qf[NT][DC];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t row = q0 + nt * 16 + col;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (row < S) r = Ld8<T>::raw(Qb + row * D + dc * 32 + grp * 8);
      qf[nt][dc] = as_frag(r);
    }
  }

  float m_run[NT], l_run[NT];
  f32x4 o[DT][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint16_t* vbuf = vbuf_all + wave * VBUF;

  for (int t = wave; t < ntiles; t += kWaves) {
    // ---- the tile's key blocks (wave-uniform) ----
    int jsub[NSUB], lim[NSUB];
    float bias[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int pos = t * NSUB + s;
      int j = pos < cnt ? list[pos] : -1;
      if (j >= a.nkb) j = -1;
      jsub[s] = j;
      lim[s] = j >= 0 ? (int)min<int64_t>(BK, S - (int64_t)j * BK) : 0;   // valid keys of the block
      bias[s] = (j >= 0 && lw) ? lw[pos] * 1.4426950408889634f : 0.0f;
    }

    // ---- V rows of the tile: global -> registers (issued early) ----
    constexpr int LPR = D / 8;                 // lanes per V row
    constexpr int RPI = 64 / LPR;              // rows per iteration
    uint4 vst[64 / RPI];
#pragma unroll
    for (int it = 0; it < 64 / RPI; ++it) {
      const int slot = it * RPI + lane / LPR;
      const int s = slot / BK, kin = slot % BK;
      uint4 r = make_uint4(0, 0, 0, 0);
      if (jsub[s] >= 0 && kin < lim[s])
        r = Ld8<T>::raw(Vb + ((int64_t)jsub[s] * BK + kin) * D + (lane % LPR) * 8);
      vst[it] = r;
    }

    // ---- K fragments (A operand), permuted rows ----
    bf16x8 kf[4][DC];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int slot = a_slot(mt, col);
      const int s = slot / BK, kin = slot % BK;
      const bool ok = jsub[s] >= 0 && kin < lim[s];
      const int64_t key = (int64_t)jsub[s] * BK + kin;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        uint4 r = make_uint4(0, 0, 0, 0);
        if (ok) r = Ld8<T>::raw(Kb + key * D + dc * 32 + grp * 8);
        kf[mt][dc] = as_frag(r);
      }
    }

    // ---- S^T = K Q^T ----
    f32x4 sacc[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt][dc], qf[nt][dc], c, 0, 0, 0);
        sacc[mt][nt] = c;
      }

    // ---- scale, log-weight, key mask (log2 domain) ----
    // accumulator element (mt, r) of this lane is key slot 32(mt/2)+8grp+4(mt&1)+r
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 32 * (mt >> 1) + 8 * grp + 4 * (mt & 1) + r;
        const int s = slot / BK, kin = slot % BK;
        const bool ok = jsub[s] >= 0 && kin < lim[s];
        const float b = bias[s];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float x = sacc[mt][nt][r] * a.scale_log2 + b;
          sacc[mt][nt][r] = ok ? x : -INFINITY;
        }
      }
    }

    // ---- online softmax ----
    float alpha[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[mt][nt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      alpha[nt] = fast_exp2(m_run[nt] - m_use);
      m_run[nt] = m_new;
      float ps = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(sacc[mt][nt][r] - m_use);
          sacc[mt][nt][r] = p;
          ps += p;
        }
      l_run[nt] = l_run[nt] * alpha[nt] + ps;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][nt] *= alpha[nt];
    }

    // ---- P^T as B operand: keys 32c + 8grp + e ----
    bf16x8 pb[2][NT];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint4 r;
        r.x = pack_bf16x2(sacc[2 * c][nt][0], sacc[2 * c][nt][1]);
        r.y = pack_bf16x2(sacc[2 * c][nt][2], sacc[2 * c][nt][3]);
        r.z = pack_bf16x2(sacc[2 * c + 1][nt][0], sacc[2 * c + 1][nt][1]);
        r.w = pack_bf16x2(sacc[2 * c + 1][nt][2], sacc[2 * c + 1][nt][3]);
        pb[c][nt] = as_frag(r);
      }

    // ---- V tile into this wave's LDS buffer, row-major [slot][d] ----
#pragma unroll
    for (int it = 0; it < 64 / RPI; ++it) {
      const int slot = it * RPI + lane / LPR;
      uint32_t* dst = reinterpret_cast<uint32_t*>(vbuf + slot * VS + (lane % LPR) * 8);
      dst[0] = vst[it].x;
      dst[1] = vst[it].y;
      dst[2] = vst[it].z;
      dst[3] = vst[it].w;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint16_t* src = vbuf + (32 * c + 8 * grp) * VS + dt * 16 + col;
        uint4 r;
        r.x = (uint32_t)src[0 * VS] | ((uint32_t)src[1 * VS] << 16);
        r.y = (uint32_t)src[2 * VS] | ((uint32_t)src[3 * VS] << 16);
        r.z = (uint32_t)src[4 * VS] | ((uint32_t)src[5 * VS] << 16);
        r.w = (uint32_t)src[6 * VS] | ((uint32_t)src[7 * VS] << 16);
        const bf16x8 vf = as_frag(r);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[c][nt], o[dt][nt], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  // ---- merge the 4 waves: log-sum-exp of (m, l), then sum of O ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    l_run[nt] = l;
    if (grp == 0) {
      st_m[wave * QROWS + nt * 16 + col] = m_run[nt];
      st_l[wave * QROWS + nt * 16 + col] = l;
    }
  }
  __syncthreads();
  float L[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int q = nt * 16 + col;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st_m[w * QROWS + q]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += st_l[w * QROWS + q] * fast_exp2(st_m[w * QROWS + q] - Mu);
    L[nt] = sum;
    const float self = fast_exp2(m_run[nt] - Mu);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][nt] *= self;
    if (wave == 0 && grp == 0 && a.lse) {
      const int64_t row = q0 + q;
      if (row < a.seq_alloc)
        a.lse[(int64_t)bh * a.seq_alloc + row] = (row < S && sum > 0.0f) ? (Mu + __log2f(sum)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();   // V tiles no longer read: the region becomes the merge buffers

  // this lane's O^T element (dt, nt, r) is O[q = 16nt + col][d = 16dt + 4grp + r]
  auto put = [&](float* buf) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(buf + (nt * 16 + col) * OS + dt * 16 + 4 * grp) = o[dt][nt];
  };
  auto add = [&](const float* buf) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt][nt] += *reinterpret_cast<const f32x4*>(buf + (nt * 16 + col) * OS + dt * 16 + 4 * grp);
  };
  float* buf0 = merge;
  float* buf1 = merge + QROWS * OS;
  if (wave >= 2) put(wave == 2 ? buf0 : buf1);
  __syncthreads();
  if (wave < 2) add(wave == 0 ? buf0 : buf1);
  __syncthreads();
  if (wave == 1) put(buf0);
  __syncthreads();
  if (wave == 0) {
    add(buf0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float inv = L[nt] > 0.0f ? 1.0f / L[nt] : 0.0f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][nt] *= inv;
    }
    put(buf1);
  }
  __syncthreads();

  // ---- coalesced output rows ----
  T* Ob = reinterpret_cast<T*>(a.out) + (int64_t)bh * a.seq_alloc * D;
  constexpr int C8 = D / 8;
  for (int e = tid; e < QROWS * C8; e += kFwdThreads) {
    const int q = e / C8, c8 = e % C8;
    const int64_t row = q0 + q;
    if (row >= a.seq_alloc) continue;
    float v[8];
    if (row < S) {
      const float4 x = *reinterpret_cast<const float4*>(buf1 + q * OS + c8 * 8);
      const float4 y = *reinterpret_cast<const float4*>(buf1 + q * OS + c8 * 8 + 4);
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
