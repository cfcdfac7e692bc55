// Float32 functions whose every operation and rounding is fixed, shared by
// the kernels whose results decide integers (which blocks are selected), so
// that they reproduce a written-out reference bit for bit.
#pragma once

#include <hip/hip_runtime.h>

namespace bsa {

// ---- e^t for t <= 0, float32, fixed operation sequence ----------------------
// Cody & Waite argument reduction (W. J. Cody, W. Waite, "Software Manual for
// the Elementary Functions", 1980): n = round(t*log2 e), x = t - n*ln2 with
// ln2 split into a 15-bit high part (n*ln2_hi exact) and a low part; e^x by
// the degree-7 Taylor polynomial (Horner, no fused multiply-add); result
// r * 2^n.  Arguments with t*log2 e < -125 give 0.
__device__ inline __attribute__((always_inline)) float exp_le0(float t) {
  const float kLog2e = (float)1.4426950408889634;
  const float kLn2Hi = (float)0.693145751953125;
  const float kLn2Lo = (float)(0.6931471805599453 - 0.693145751953125);
  const float c0 = (float)(1.0 / 1.0), c1 = (float)(1.0 / 1.0), c2 = (float)(1.0 / 2.0);
  const float c3 = (float)(1.0 / 6.0), c4 = (float)(1.0 / 24.0), c5 = (float)(1.0 / 120.0);
  const float c6 = (float)(1.0 / 720.0), c7 = (float)(1.0 / 5040.0);
  float y = __fmul_rn(t, kLog2e);
  const bool flush = y < -125.0f;
  if (flush) { t = 0.0f; y = 0.0f; }
  const float n = floorf(__fadd_rn(y, 0.5f));
  float x = __fsub_rn(t, __fmul_rn(n, kLn2Hi));
  x = __fsub_rn(x, __fmul_rn(n, kLn2Lo));
  float r = c7;
  r = __fadd_rn(__fmul_rn(r, x), c6);
  r = __fadd_rn(__fmul_rn(r, x), c5);
  r = __fadd_rn(__fmul_rn(r, x), c4);
  r = __fadd_rn(__fmul_rn(r, x), c3);
  r = __fadd_rn(__fmul_rn(r, x), c2);
  r = __fadd_rn(__fmul_rn(r, x), c1);
  r = __fadd_rn(__fmul_rn(r, x), c0);
  const float out = ldexpf(r, (int)n);
  return flush ? 0.0f : out;
}

}  // namespace bsa
