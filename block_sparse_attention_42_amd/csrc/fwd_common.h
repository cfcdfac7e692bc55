// Device helpers shared by the sparse forward kernels (forward.hip,
// forward_wide.hip): vector types, bf16 packing, the matrix instructions
// with fixed register files, lane exchanges and the launch schedule.
#pragma once

#include <type_traits>

#include "bsa_internal.h"

namespace bsa {
namespace fwdc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr uint32_t kOob = 0x80000000u;   // byte offset past any buffer: the load returns zeros

// Two floats as two bf16 (round to nearest even) in one dword: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_frag(uint4 r) { return __builtin_bit_cast(bf16x8, r); }

__device__ __forceinline__ uint4 pack8(u32x4 x, u32x4 y) {
  uint4 o;
  o.x = pack_bf16x2(__uint_as_float(x[0]), __uint_as_float(x[1]));
  o.y = pack_bf16x2(__uint_as_float(x[2]), __uint_as_float(x[3]));
  o.z = pack_bf16x2(__uint_as_float(y[0]), __uint_as_float(y[1]));
  o.w = pack_bf16x2(__uint_as_float(y[2]), __uint_as_float(y[3]));
  return o;
}

// 8 consecutive elements of a row as 8 bf16 (float rows are rounded).
template <typename T>
struct Row8;

template <>
struct Row8<bf16_t> {
  static __device__ __forceinline__ uint4 ld(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ uint4 buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
};

template <>
struct Row8<float> {
  static __device__ __forceinline__ uint4 ld(const float* p) {
    const float4 x = reinterpret_cast<const float4*>(p)[0];
    const float4 y = reinterpret_cast<const float4*>(p)[1];
    return pack8(u32x4{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)},
                 u32x4{__float_as_uint(y.x), __float_as_uint(y.y), __float_as_uint(y.z), __float_as_uint(y.w)});
  }
  static __device__ __forceinline__ uint4 buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 16u), (int)soff, 0);
    return pack8(x, y);
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

// x combined with the same register of lane ^ 32 (one v_permlane32_swap).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- matrix instructions with fixed register files ----
// The score tiles S^T are produced by MFMAs and consumed by vector code, so
// they live in VGPRs; the O^T accumulators, the Q fragments and the K and V
// fragments read from LDS are only ever MFMA operands and live in AGPRs.  The compiler cannot be told that per
// instruction, so these MFMAs are written as inline assembly with register
// class constraints.  Because the compiler does not see them as MFMAs, the
// code around them keeps the hardware's wait-state rules itself: a vector
// write of an MFMA source needs 2 wait states before the MFMA, and a vector
// read of an MFMA result needs 12 after it (8-pass 32x32x16).
__device__ __forceinline__ void mma_s_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "a"(a), "a"(b) : "memory");
}
__device__ __forceinline__ void mma_s(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "a"(a), "a"(b) : "memory");
}
__device__ __forceinline__ void mma_o(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "a"(a), "v"(b) : "memory");
}
// max of three floats (no NaN canonicalization: the inputs are finite or -inf)
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// The "memory" clobber keeps every memory instruction (tile loads, LDS reads)
// where the source puts it relative to these MFMAs.
// Empty ordering points: work reading x is placed after (pin_after), work
// producing x before (pin_before), relative to the neighbouring asm.
template <typename X>
__device__ __forceinline__ void pin_after(X& x) { asm volatile("" : "+v"(x)); }
template <typename X>
__device__ __forceinline__ void pin_before(const X& x) { asm volatile("" ::"v"(x)); }

// LDS chunk swizzle of a 32-row V sub-tile (16-byte chunks of a row of D
// bf16).  V is read with the transposing 8-byte load, 4 consecutive rows x 4
// chunks per 16 lanes; the XOR puts each such group on distinct banks and only
// touches chunk bits, so every read address is (lane base) ^ (constant).
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128) return 4 * (r & 3);
  else return 4 * ((r >> 1) & 1);
}

// blockIdx -> (head, query block); false for the few padding workgroups.
__device__ __forceinline__ bool schedule(const FwdArgs& a, int t, int& bh, int& qb) {
  if (t < a.n_dense) {
    const int r = t / a.split;                     // the split parts of a row are adjacent items
    bh = r % a.BH;
    qb = a.dense_first + r / a.BH;
    return true;
  }
  const int nd = a.dense_first >= 0 ? a.dense_last - a.dense_first + 1 : 0;
  const int ns = a.nqb - nd;                       // other rows per head
  const int x = t % kXcds, k = t / kXcds;
  const int k0 = (a.n_dense + kXcds - 1 - x) / kXcds;
  if (a.order == 1) {                              // the x-th run of frames of every head
    const int lo = (int)((int64_t)x * ns / kXcds), len = (int)((int64_t)(x + 1) * ns / kXcds) - lo;
    const int pos = k - k0;
    if (pos >= a.BH * len) return false;           // also every item when len == 0
    bh = pos / len;
    const int s = lo + pos % len;
    qb = (a.dense_first < 0 || s < a.dense_first) ? s : s + nd;
    return true;
  }
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

// Rows [nqb * q_block, seq_alloc) of a head belong to no query block (a
// caller may allocate more rows than the blocks cover): the work item of the
// head's last query block writes them as 0 and their LSE as -inf.
template <typename T, int D>
__device__ __forceinline__ void zero_tail_rows(const FwdArgs& a, int bh, int lane) {
  const int64_t t0 = (int64_t)a.nqb * a.q_block;
  if (t0 >= a.seq_alloc) return;
  T* Ob = reinterpret_cast<T*>(a.out) + (int64_t)bh * a.seq_alloc * D;
  uint4* dst = reinterpret_cast<uint4*>(Ob + t0 * D);   // 16-byte aligned: D * sizeof(T) is a multiple of 16
  const int64_t n = (a.seq_alloc - t0) * D * (int64_t)sizeof(T) / 16;
  for (int64_t e = lane; e < n; e += 64) dst[e] = make_uint4(0u, 0u, 0u, 0u);
  if (a.lse)
    for (int64_t r = t0 + lane; r < a.seq_alloc; r += 64) a.lse[(int64_t)bh * a.seq_alloc + r] = -INFINITY;
}

// f(integral_constant<int, I>) for I = B .. E-1, expanded at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace fwdc
}  // namespace bsa
