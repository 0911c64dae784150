// Device helpers shared by the gfx950 kernels of the fused MLA query
// up-projection: MXFP8 element/scale encoding, bf16 rounding, token
// coordinates, MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int FMT_BSHD = 0;
constexpr int FMT_SBHD = 1;
constexpr int FMT_THD = 2;

// ---------------------------------------------------------------------------
// bf16 <-> fp32. Round to nearest, ties to even; NaN stays a quiet NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u | ((u >> 16) & 0x8000u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------------------
// MXFP8 (OCP Microscaling Formats v1.0, E4M3 elements, E8M0 scales).
// Both helpers work on the float32 bit pattern with integer arithmetic only,
// so results do not depend on the denormal mode of the floating-point unit.
// ---------------------------------------------------------------------------

// |x| bit pattern; integer max over a block gives the bits of amax for finite
// values, and any NaN/Inf in the block yields a value >= 0x7F800000.
__device__ __forceinline__ uint32_t abs_bits(float x) {
  return __float_as_uint(x) & 0x7FFFFFFFu;
}

// Block exponent E = clamp(floor(log2 amax) - 8, -127, 127), from amax bits.
// amax = 0 and float32 subnormal amax both give -127 (floor(log2) <= -127).
// The largest finite float32 gives 119, so the upper clamp never binds.
__device__ __forceinline__ int mx_block_exp(uint32_t amax_bits) {
  int ev = (int)(amax_bits >> 23);
  int e = ev - 127 - 8;
  return e < -127 ? -127 : e;
}

// E4M3 code of x * 2^-E: round to nearest, ties to even, saturating to
// +-448, sign of zero kept. x must be finite.
//   value of x = M * 2^q (M the 24-bit significand with its hidden bit);
//   L = floor(log2 |y|) for y = x * 2^-E;  the E4M3 spacing at y is
//   2^(max(L,-6) - 3);  R = y / spacing rounded to nearest even;
//   normal range: code = ((L+7) << 3) + (R - 8)  (R = 16 carries into the
//   exponent field by itself); subnormal range (L < -6): code = R.
__device__ __forceinline__ uint32_t e4m3_encode(float x, int E) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a == 0) return sign;
  int ev = (int)(a >> 23);
  uint32_t M = a & 0x7FFFFFu;
  int q;
  if (ev == 0) {
    q = -149;
  } else {
    M |= 0x800000u;
    q = ev - 150;
  }
  int msb = 31 - __clz(M);
  int L = msb + q - E;
  int ulp_e = (L < -6 ? -6 : L) - 3;
  int shift = ulp_e - (q - E);
  uint32_t R;
  if (shift <= 0) {
    R = M << (-shift);  // y / spacing < 16 here, so this cannot overflow
  } else if (shift > 25) {
    R = 0;              // M < 2^24 <= half a spacing
  } else {
    uint32_t keep = M >> shift;
    uint32_t rem = M & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    R = keep + ((rem > half || (rem == half && (keep & 1u))) ? 1u : 0u);
  }
  uint32_t code;
  if (L < -6) {
    code = R;
  } else {
    int c = ((L + 7) << 3) + (int)R - 8;
    code = c > 0x7E ? 0x7Eu : (uint32_t)c;
  }
  return sign | code;
}

// ---------------------------------------------------------------------------
// Token row -> (position, b, s). See the token-format comment in mla_qup.h.
// ---------------------------------------------------------------------------
struct TokenMap {
  int fmt;
  int B, S;
  const int32_t* cu;
  int nseq;
};

__device__ __forceinline__ void token_coords(const TokenMap& tm, int64_t t, int& pos, int& b,
                                             int& s) {
  if (tm.fmt == FMT_BSHD) {
    b = (int)(t / tm.S);
    s = (int)(t - (int64_t)b * tm.S);
    pos = s;
  } else if (tm.fmt == FMT_SBHD) {
    s = (int)(t / tm.B);
    b = (int)(t - (int64_t)s * tm.B);
    pos = s;
  } else {
    // largest j with cu[j] <= t (binary search over nseq+1 entries)
    int lo = 0, hi = tm.nseq;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if ((int64_t)tm.cu[mid] <= t) lo = mid; else hi = mid;
    }
    pos = (int)(t - tm.cu[lo]);
    b = 0;
    s = (int)t;
  }
}

}  // namespace mla
