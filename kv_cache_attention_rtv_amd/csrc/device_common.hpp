// Device helpers shared by the library's kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtv {

constexpr int kWave = 64;
constexpr int kTileKeys = 64;          // slots per V-transposed tile / attention key tile

// position of key `k` (0..63) inside a transposed V tile row (the byte order
// of the attention's matrix-core operand)
__device__ __forceinline__ int vt_pos_of_key(int k) {
  const int h = (k >> 2) & 1;
  const int b = ((k >> 5) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
  return h * 32 + b;
}
constexpr float kFp8Max = 448.0f;

// ---- bf16 ---------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// round-to-nearest-even f32 -> bf16 bits (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---- e4m3 ---------------------------------------------------------------
// Two non-negative floats to two OCP E4M3FN codes (round to nearest even) in
// the low (sel = false) or high (sel = true) half of `old`; byte 0/2 <- a.
// Inputs are clamped to 448 first, which makes the conversion saturating.
template <bool kHigh>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old) {
  a = fminf(a, kFp8Max);
  b = fminf(b, kFp8Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHigh);
}

// Correctly rounded |x| / s for s > 0 (normal), given r = RN(1/s):
// q0 = RN(|x| r) is within one ulp of the quotient, the remainder |x| - q0 s
// is exact with a fused multiply-add, and one corrected step gives RN(|x|/s)
// (Markstein's theorem on division with a correctly rounded reciprocal).
__device__ __forceinline__ float div_rn(float ax, float s, float r) {
  float q0 = ax * r;
  float rem = __builtin_fmaf(-q0, s, ax);
  return __builtin_fmaf(rem, r, q0);
}

// Per-row quantization parameters: scale = RN(amax/448); the division works
// on (|x| * pre, s * pre) with pre = 2^64 when s is tiny so that the
// reciprocal and the remainder stay in the normal range (scaling by a power
// of two does not change the quotient).
struct RowQuant {
  float s;      // stored scale
  float ss;     // s * pre
  float r;      // RN(1 / ss)
  float pre;    // 1 or 2^64
};

__device__ __forceinline__ RowQuant row_quant(float amax) {
  RowQuant q;
  q.s = amax / kFp8Max;                     // correctly rounded f32 division
  q.pre = (q.s < 0x1p-100f) ? 0x1p64f : 1.0f;
  q.ss = q.s * q.pre;
  q.r = 1.0f / q.ss;                        // correctly rounded f32 division
  return q;
}

// e4m3 code (as 0..255 in the low byte) of x under row parameters q.
__device__ __forceinline__ float quant_mag(float x, const RowQuant& q) {
  return div_rn(fabsf(x) * q.pre, q.ss, q.r);
}

// ---- row quantization, fast form ------------------------------------------
// For amax in [448 * 2^-100, FLT_MAX] (scale >= 2^-100, normal) the same codes
// and scale as row_quant / quant4 with fewer operations:
//  * scale: q0 = RN(amax * RN(1/448)), s = RN(q0 + (amax - q0 * 448) RN(1/448))
//    with fused operations; equal to the correctly rounded amax / 448 for
//    every float amax of the range (checked exhaustively on the host);
//  * x / s on the signed value: q0 = RN(x r), e = q0 s - x (exact), RN(q0 -
//    e r) has the magnitude of div_rn(|x|, s, r) and the sign of x, also when
//    it is zero;
//  * the e4m3 conversion without the clamp: |x / s| <= RN(amax / s) <= 448 (1 +
//    2^-23), which the conversion rounds to 448 (the overflow midpoint is 464);
//    a signed zero or a negative value that rounds to zero gives 0x80.
// Rows outside the range (all-zero, tiny or non-finite amax) take row_quant.
constexpr float kFastAmaxMin = 0x1.cp-92f;  // 448 * 2^-100
__device__ __forceinline__ bool fast_amax(float amax) {
  return amax >= kFastAmaxMin && amax <= 0x1.fffffep127f;
}
__device__ __forceinline__ float scale448(float amax) {
  constexpr float r = 1.0f / kFp8Max;
  const float q0 = amax * r;
  return __builtin_fmaf(__builtin_fmaf(-q0, kFp8Max, amax), r, q0);
}
__device__ __forceinline__ float div_signed(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-e, r, q0);
}
__device__ __forceinline__ uint32_t quant4_fast(float x0, float x1, float x2, float x3, float s, float r) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(div_signed(x0, s, r), div_signed(x1, s, r), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(div_signed(x2, s, r), div_signed(x3, s, r), (int)w, true);
}

// sign bits of four floats -> 0x80 in each byte whose float is negative
__device__ __forceinline__ uint32_t sign_bytes4(float a, float b, float c, float d) {
  return ((__float_as_uint(a) >> 31) << 7) | ((__float_as_uint(b) >> 31) << 15) |
         ((__float_as_uint(c) >> 31) << 23) | ((__float_as_uint(d) >> 31) << 31);
}

// Quantize four values of a row to four codes in one dword (byte k <- x_k).
// Branch-free: for an all-zero row (s == 0) the quotient is garbage and the
// select keeps only the signed zeros.
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3,
                                           const RowQuant& q) {
  const uint32_t signs = sign_bytes4(x0, x1, x2, x3);
  uint32_t w = cvt_fp8x2<false>(quant_mag(x0, q), quant_mag(x1, q), 0u);
  w = cvt_fp8x2<true>(quant_mag(x2, q), quant_mag(x3, q), w);
  return q.s == 0.0f ? signs : (w | signs);
}

// Codes of one row held as two parts of N values each (N a multiple of 4),
// into N / 4 dwords per part, and the row's scale.  `fast` (every row of the
// wave in the fast range, so that the branch is uniform) selects the short
// form; otherwise row_quant / quant4.
template <int N>
__device__ __forceinline__ float quant_row(const float (&x0)[N], const float (&x1)[N], uint32_t (&c0)[N / 4],
                                           uint32_t (&c1)[N / 4], float amax, bool fast) {
  if (__builtin_expect(fast, 1)) {
    const float s = scale448(amax);
    const float r = 1.0f / s;                 // correctly rounded f32 division
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      c0[i] = quant4_fast(x0[4 * i], x0[4 * i + 1], x0[4 * i + 2], x0[4 * i + 3], s, r);
      c1[i] = quant4_fast(x1[4 * i], x1[4 * i + 1], x1[4 * i + 2], x1[4 * i + 3], s, r);
    }
    return s;
  }
  const RowQuant q = row_quant(amax);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    c0[i] = quant4(x0[4 * i], x0[4 * i + 1], x0[4 * i + 2], x0[4 * i + 3], q);
    c1[i] = quant4(x1[4 * i], x1[4 * i + 1], x1[4 * i + 2], x1[4 * i + 3], q);
  }
  return q.s;
}

// ---- XCD-aware block order ------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Renumber so that each XCD walks a contiguous range of the logical
// work list: logical = (b % 8) * ceil(n/8) + b / 8.  Returns -1 for the padding
// blocks when n is not a multiple of 8 (the grid is rounded up to 8).
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = (n + 7) >> 3;
  const int logical = (b & 7) * per + (b >> 3);
  return logical < n ? logical : -1;
}

}  // namespace rtv
