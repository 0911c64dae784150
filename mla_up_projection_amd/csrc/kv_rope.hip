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
// One thread owns one 32-element block (or 8 elements for bf16 widths that
// are not multiples of 32) of one (t, h) row of [key | value].
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int KV_TOK = 4;         // tokens per workgroup chunk
constexpr int KV_HG = 64;         // heads per workgroup chunk
constexpr int KV_MAX_ROPE = 256;  // widest rope slice (the ABI limits d_rope to this)
constexpr int KV_ROT_PITCH = KV_MAX_ROPE + 4;  // LDS row pitch: tokens' rows in different banks

// A workgroup chunk is KV_TOK consecutive tokens x up to KV_HG heads. The
// workgroup first rotates the tokens' shared k_pe slices once into LDS (with
// the tokens' BHSD coordinates), then each thread takes EPT consecutive output
// elements of one (t, h) row of [key | value]: 32 (one whole MXFP8 block, amax
// in the thread) when both widths are multiples of 32, else 8 (bf16 output).
// Units are numbered head-major, so consecutive lanes write one head's rows
// for consecutive tokens, which are adjacent in BHSD (measured: 111 -> 99 us
// at DeepSeek-V3 shape against token-major units over 8 tokens and all
// heads). The kv loads (16 bytes each) of a unit are issued before any
// arithmetic; rope elements come from LDS.
template <int EPT>
__global__ __launch_bounds__(256) void kv_rope_kernel(KvParams p) {
  constexpr int NG = EPT / 8;
  __shared__ float rot[KV_TOK * KV_ROT_PITCH];
  __shared__ int64_t orow0[KV_TOK];  // BHSD row of head 0: (b H) S + s
  const int Dk = p.d_nope + p.d_rope;
  const int row_in = p.d_nope + p.d_v;
  const int upr = (Dk + p.d_v) / EPT;  // units per (t, h) row
  const int hgroups = (p.H + KV_HG - 1) / KV_HG;
  const int64_t HS = (int64_t)p.H * p.S;
  const TokenMap tm{p.fmt, p.B, p.S, p.cu, p.nseq};
  const int64_t chunks = (p.T + KV_TOK - 1) / KV_TOK * hgroups;
  for (int64_t cki = blockIdx.x; cki < chunks; cki += gridDim.x) {
    const int ck = (int)(cki / hgroups);
    const int h0 = (int)(cki - (int64_t)ck * hgroups) * KV_HG;  // the chunk's heads h0 .. h0 + nh - 1
    const int nh = min(KV_HG, p.H - h0);
    const int t0 = ck * KV_TOK;
    const int nt = min(KV_TOK, (int)p.T - t0);
    __syncthreads();  // the previous chunk's readers of rot / orow0 are done
    for (int i = threadIdx.x; i < nt * (p.d_rope / 2 + 1); i += blockDim.x) {
      const int tl = i / (p.d_rope / 2 + 1);
      const int k = i - tl * (p.d_rope / 2 + 1);  // pair k, or the coordinates at k == d_rope/2
      int pos, b, s;
      token_coords(tm, t0 + tl, pos, b, s);
      if (k == p.d_rope / 2) {
        orow0[tl] = (int64_t)b * HS + s;
      } else {
        const uint32_t ab = *reinterpret_cast<const uint32_t*>(p.pe + (int64_t)(t0 + tl) * p.d_rope + 2 * k);
        const float a = bf16_bits_to_f32(ab & 0xFFFFu), bb = bf16_bits_to_f32(ab >> 16);
        const bool ok = pos >= 0 && pos < p.rope_rows;
        const float nan = __builtin_nanf("");
        const int64_t ti = (int64_t)(ok ? pos : 0) * p.rope_pairs + k;
        const float c = ok ? p.cos[ti] : nan, sn = ok ? p.sin[ti] : nan;
        rot[tl * KV_ROT_PITCH + 2 * k] = a * c - bb * sn;
        rot[tl * KV_ROT_PITCH + 2 * k + 1] = a * sn + bb * c;
      }
    }
    __syncthreads();
    const int n = nh * nt * upr;
    // two units per thread per pass: both units' kv loads are in flight together
    for (int i0 = threadIdx.x; i0 < n; i0 += 2 * blockDim.x) {
      int tl[2], h[2], d0[2];
      bool key[2], live[2];
      uint4 raw[2][NG];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int i = i0 + w * blockDim.x;
        live[w] = i < n;
        const int ii = live[w] ? i : i0;
        const int hl = ii / (nt * upr);  // head-major: head, then token, then unit
        const int rem = ii - hl * (nt * upr);
        tl[w] = rem / upr;
        h[w] = h0 + hl;
        const int e0 = (rem - tl[w] * upr) * EPT;
        key[w] = e0 < Dk;
        d0[w] = key[w] ? e0 : e0 - Dk;
        const int64_t row = (int64_t)(t0 + tl[w]) * p.H + h[w];  // kv row (t, h)
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const int d = d0[w] + 8 * q;
          if (!(key[w] && d >= p.d_nope))
            raw[w][q] = *reinterpret_cast<const uint4*>(p.kv + row * row_in + (key[w] ? d : p.d_nope + d));
        }
      }
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if (!live[w]) continue;
        float v[EPT];
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const int d = d0[w] + 8 * q;
          if (key[w] && d >= p.d_nope) {
            const float* r = rot + tl[w] * KV_ROT_PITCH + (d - p.d_nope);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[8 * q + k] = r[k];
          } else {
            const uint32_t wv[4] = {raw[w][q].x, raw[w][q].y, raw[w][q].z, raw[w][q].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              v[8 * q + 2 * k] = bf16_bits_to_f32(wv[k] & 0xFFFFu);
              v[8 * q + 2 * k + 1] = bf16_bits_to_f32(wv[k] >> 16);
            }
          }
        }
        const bool is_key = key[w];
        const int D = is_key ? Dk : p.d_v;
        const int64_t orow = orow0[tl[w]] + (int64_t)h[w] * p.S;  // BHSD (b, h, s)
        if (!p.out_mx) {
          uint16_t* dst = static_cast<uint16_t*>(is_key ? p.key : p.value) + orow * D + d0[w];
#pragma unroll
          for (int q = 0; q < NG; ++q)
            reinterpret_cast<uint4*>(dst)[q] =
                make_uint4(pack_bf16x2(v[8 * q], v[8 * q + 1]), pack_bf16x2(v[8 * q + 2], v[8 * q + 3]),
                           pack_bf16x2(v[8 * q + 4], v[8 * q + 5]), pack_bf16x2(v[8 * q + 6], v[8 * q + 7]));
        } else if (EPT == 32) {
          uint32_t m = 0;
#pragma unroll
          for (int k = 0; k < EPT; ++k) m = max(m, abs_bits(v[k]));
          uint32_t c[8], sc;
          if (m >= 0x7F800000u) {
#pragma unroll
            for (int k = 0; k < 8; ++k) c[k] = 0x7F7F7F7Fu;
            sc = 0xFF;
          } else {
            const int E = mx_block_exp(m);
#pragma unroll
            for (int k = 0; k < 8; ++k) c[k] = e4m3_pack4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3], E);
            sc = (uint32_t)(E + 127);
          }
          uint8_t* dst = static_cast<uint8_t*>(is_key ? p.key : p.value) + orow * D + d0[w];
          reinterpret_cast<uint4*>(dst)[0] = make_uint4(c[0], c[1], c[2], c[3]);
          reinterpret_cast<uint4*>(dst)[1] = make_uint4(c[4], c[5], c[6], c[7]);
          (is_key ? p.key_scales : p.value_scales)[orow * (D / 32) + d0[w] / 32] = (uint8_t)sc;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_rope(const KvParams& p, hipStream_t stream) {
  const int W = p.d_nope + p.d_rope + p.d_v;
  const bool whole = (p.d_nope + p.d_rope) % 32 == 0 && p.d_v % 32 == 0;  // always so for MXFP8
  (void)W;
  int64_t blocks = (p.T + KV_TOK - 1) / KV_TOK * ((p.H + KV_HG - 1) / KV_HG);
  if (blocks > 65535) blocks = 65535;
  if (blocks == 0) return hipSuccess;
  if (whole)
    hipLaunchKernelGGL(kv_rope_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_rope_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
