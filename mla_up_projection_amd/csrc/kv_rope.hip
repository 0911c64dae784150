// KV side of the MLA attention inputs for gfx950: the fresh key and value
// outputs of the KV rotary (page "Fix fused MLA YaRN RoPE query kernel
// corrupting upstream tensor in-place", Solution: the KV path writes new
// key and value buffers) and their MXFP8 quantization with the query's BHSD
// scale layout (page "Add support for fused Q Up-Proj GEMM/RoPE/Quant.",
// flowchart: key and value each pass an MXFP8 quantization before the BHSD
// scale transpose). Per token t and head h:
//   key[t, h]   = [k_nope[t, h] | rotate(k_pe[t], pos_t)]   (k_pe shared by all heads)
//   value[t, h] = v[t, h]
// with kv[t, h] = [k_nope | v]. HBM-bound: each kv element is read once and
// each output element written once (2 bytes, or 1 + 1/32 for MXFP8).
//
// One thread owns 8 consecutive output elements of one (t, h) row of
// [key | value] (one 16-byte load of kv or k_pe); for MXFP8 the four threads
// of a 32-element block are lanes 4j .. 4j + 3 and share the block amax
// through two xor-shuffles, as in the row quantizer.
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

__global__ __launch_bounds__(256) void kv_rope_kernel(KvParams p) {
  const int Dk = p.d_nope + p.d_rope;
  const int row_in = p.d_nope + p.d_v;
  const int gpr = (Dk + p.d_v) / 8;  // 8-element groups per (t, h) row
  const int64_t groups = p.T * p.H * gpr;
  const TokenMap tm{p.fmt, p.B, p.S, p.cu, p.nseq};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    const int64_t row = g / gpr;
    const int e = (int)(g - row * gpr) * 8;
    const int64_t t = row / p.H;
    const int h = (int)(row - t * p.H);
    int pos, b, s;
    token_coords(tm, t, pos, b, s);
    float v[8];
    const bool is_key = e < Dk;
    const int d = is_key ? e : e - Dk;
    if (is_key && d >= p.d_nope) {
      // rope slice: pairs j/2 .. j/2 + 3 of the token's shared k_pe
      const int j = d - p.d_nope;
      const uint4 u = *reinterpret_cast<const uint4*>(p.pe + t * p.d_rope + j);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
      const bool pos_ok = pos >= 0 && pos < p.rope_rows;
      const int64_t trow = (int64_t)(pos_ok ? pos : 0) * p.rope_pairs + j / 2;
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = bf16_bits_to_f32(wv[i] & 0xFFFFu), bb = bf16_bits_to_f32(wv[i] >> 16);
        const float c = pos_ok ? p.cos[trow + i] : nan, sn = pos_ok ? p.sin[trow + i] : nan;
        v[2 * i] = a * c - bb * sn;
        v[2 * i + 1] = a * sn + bb * c;
      }
    } else {
      const int src = is_key ? d : p.d_nope + d;
      const uint4 u = *reinterpret_cast<const uint4*>(p.kv + row * row_in + src);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(wv[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(wv[i] >> 16);
      }
    }
    const int D = is_key ? Dk : p.d_v;
    const int64_t orow = ((int64_t)b * p.H + h) * p.S + s;  // BHSD (b, h, s)
    if (!p.out_mx) {
      uint16_t* dst = static_cast<uint16_t*>(is_key ? p.key : p.value) + orow * D + d;
      *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, abs_bits(v[i]));
      m = max(m, (uint32_t)__shfl_xor((int)m, 1));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2));
      uint32_t c0, c1, sc;
      if (m >= 0x7F800000u) {
        c0 = c1 = 0x7F7F7F7Fu;
        sc = 0xFF;
      } else {
        const int E = mx_block_exp(m);
        c0 = e4m3_pack4(v[0], v[1], v[2], v[3], E);
        c1 = e4m3_pack4(v[4], v[5], v[6], v[7], E);
        sc = (uint32_t)(E + 127);
      }
      uint8_t* dst = static_cast<uint8_t*>(is_key ? p.key : p.value) + orow * D + d;
      *reinterpret_cast<uint2*>(dst) = make_uint2(c0, c1);
      if ((d & 31) == 0) (is_key ? p.key_scales : p.value_scales)[orow * (D / 32) + d / 32] = (uint8_t)sc;
    }
  }
}

}  // namespace

hipError_t launch_kv_rope(const KvParams& p, hipStream_t stream) {
  const int64_t groups = p.T * p.H * ((p.d_nope + p.d_rope + p.d_v) / 8);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
