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
// bf16 <-> fp32. fp32 -> bf16 is gfx950's v_cvt_pk_bf16_f32 (two values per
// instruction): round to nearest, ties to even, denormals kept, NaN stays NaN;
// it agrees bit for bit with integer round-to-nearest-even on every tie of
// every upper half-word and on a strided sweep of all fp32 patterns.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return pack_bf16x2(f, 0.0f) & 0xFFFFu;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// ---------------------------------------------------------------------------
// Exchange between the two halves of a wave (gfx950 v_permlane32_swap): the
// upper 32 lanes of `a` trade places with the lower 32 lanes of `b`. Lane l
// < 32 gets {a[l], a[l + 32]}; lane l >= 32 gets {b[l - 32], b[l]}.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2_t swap_halves(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return u32x2_t{r[0], r[1]};
}

// ---------------------------------------------------------------------------
// MXFP8 (OCP Microscaling Formats v1.0, E4M3 elements, E8M0 scales).
// The block exponent comes from the float32 bit pattern of amax by integer
// arithmetic, so it does not depend on the denormal mode of the FP unit.
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

// Four E4M3 codes (little-endian bytes of the result) of x0..x3 * 2^-E with
// gfx950's scaled convert. v_cvt_scalef32_pk_fp8_f32 computes
// fp8(x / scale) with round-to-nearest-even but does not saturate (values
// past the last rounding boundary, 464, become NaN), so inputs are first
// clamped to +-448 * 2^E: the OCP MX rule, saturating at the largest normal.
// Requires finite inputs and -127 <= E <= 119.
typedef short v2i16_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t e4m3_pack4(float x0, float x1, float x2, float x3, int E) {
  const float scale = __uint_as_float(E > -127 ? (uint32_t)(E + 127) << 23 : 0x00400000u);
  const float lim = __uint_as_float(((uint32_t)(E + 135) << 23) | 0x00600000u);  // 1.75 * 2^(E+8)
  // one v_med3_f32 each (finite inputs: no NaN rule involved; -0 stays -0)
  x0 = __builtin_amdgcn_fmed3f(x0, -lim, lim);
  x1 = __builtin_amdgcn_fmed3f(x1, -lim, lim);
  x2 = __builtin_amdgcn_fmed3f(x2, -lim, lim);
  x3 = __builtin_amdgcn_fmed3f(x3, -lim, lim);
  v2i16_t o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, x0, x1, scale, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, x2, x3, scale, true);
  return __builtin_bit_cast(uint32_t, o);
}

// ---------------------------------------------------------------------------
// Direct global->LDS staging (gfx950 global_load_lds_dwordx4). Each kernel
// that uses it issues no other vector-memory load inside its pipelined loop,
// so a per-wave s_waitcnt vmcnt count names exactly which stages have landed.
// ---------------------------------------------------------------------------

// 16 bytes per lane: lane i of the wave writes LDS bytes [lds_addr + 16 i,
// +16) from global sbase + voff (sbase wave-uniform).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the compiler's implied full memory wait.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// 8-byte LDS read at an LDS byte address (ds_read_b64; 8-byte aligned).
__device__ __forceinline__ float2 lds_read_f2(uint32_t addr) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = *reinterpret_cast<__attribute__((address_space(3))) const f32x2_t*>((uintptr_t)addr);
  return make_float2(v[0], v[1]);
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

// BSHD and SBHD (fmt one of the two): t = b S + s or t = s B + b.
__device__ __forceinline__ void token_coords_dense(const TokenMap& tm, int t32, int& pos, int& b, int& s) {
  if (tm.fmt == FMT_BSHD) {
    b = t32 / tm.S;
    s = t32 - b * tm.S;
  } else {
    s = t32 / tm.B;
    b = t32 - s * tm.B;
  }
  pos = s;
}

__device__ __forceinline__ void token_coords(const TokenMap& tm, int64_t t, int& pos, int& b,
                                             int& s) {
  const int t32 = (int)t;  // T < 2^31 (validated by the C ABI)
  if (tm.fmt == FMT_BSHD || tm.fmt == FMT_SBHD) {
    token_coords_dense(tm, t32, pos, b, s);
  } else {
    // largest j with cu[j] <= t (binary search over nseq+1 entries)
    int lo = 0, hi = tm.nseq;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (tm.cu[mid] <= t32) lo = mid; else hi = mid;
    }
    pos = t32 - tm.cu[lo];
    b = 0;
    s = t32;
  }
}

// token_coords for a lane whose token t lies in a run [base, last] that is
// the same for the whole wave. For THD the sequence search then runs once per
// wave on scalar loads, which count against lgkmcnt and so never wait for the
// vector-memory loads (DMA) in flight, and each lane takes the last sequence
// start at or before its token among the starts inside the run.
__device__ __forceinline__ void token_coords_run(const TokenMap& tm, int64_t t, int base, int last, int& pos,
                                                 int& b, int& s) {
  if (tm.fmt == FMT_BSHD || tm.fmt == FMT_SBHD) {
    token_coords_dense(tm, (int)t, pos, b, s);
    return;
  }
  typedef __attribute__((address_space(4))) const int32_t cint32;
  const cint32* cu = (const cint32*)tm.cu;
  base = __builtin_amdgcn_readfirstlane(base);
  last = __builtin_amdgcn_readfirstlane(last);
  const int t32 = (int)t;
  int lo = 0, hi = tm.nseq;  // largest j < nseq with cu[j] <= base
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= base) lo = mid; else hi = mid;
  }
  int start = cu[lo];
  for (int j = lo + 1; j < tm.nseq; ++j) {  // sequence starts inside the run
    const int c = cu[j];
    if (c > last) break;
    if (c <= t32) start = c;
  }
  pos = t32 - start;
  b = 0;
  s = t32;
}

}  // namespace mla
