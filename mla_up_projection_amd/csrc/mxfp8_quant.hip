// Separable MXFP8 quantization of a row-major matrix along its rows, one
// E8M0 scale per 32 consecutive elements (OCP Microscaling Formats v1.0),
// and along its columns with a transposed store (further below).
// Forward page (file table, review thread): the standalone MXFP8 quantize
// used for operands of the MXFP8 projection. HBM-bound: each element is read
// once (2 or 4 bytes) and written once (1 byte + 1/32 byte of scale).
//
// Four consecutive lanes own one 32-element block, eight elements each
// (one 16-byte bf16 load or two fp32 loads per lane, one 8-byte store); the
// block amax is an integer max over |x| bit patterns reduced across the four
// lanes with two xor-shuffles.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

// Work split of the row quantization: a workgroup takes MQ_U * 256
// consecutive groups of 8 elements; thread i handles groups i, i + 256, ...
// (each of those is one coalesced 1-4 KB wave load), and issues all its loads
// before any arithmetic, so MQ_U 16-byte loads per lane are in flight.
// Codes are [rows, cols] and scales [rows, cols/32] row-major with no row
// padding, so group g's codes start at byte 8 g and its scale is byte g / 4;
// only a row-strided x (ld != cols) needs g's row, found with 32-bit
// division when the group count allows it.
constexpr int MQ_U = 4;

template <bool FP32, bool DENSE, bool IDX32>
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const void* __restrict__ x, int64_t groups,
                                                          int64_t gpr, int64_t ld,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  constexpr int EB = FP32 ? 4 : 2;  // bytes per input element
  const int64_t g0 = (int64_t)blockIdx.x * (256 * MQ_U) + threadIdx.x;
  u32x4_t raw[MQ_U][FP32 ? 2 : 1];
#pragma unroll
  for (int u = 0; u < MQ_U; ++u) {
    int64_t g = g0 + 256 * u;
    if (g >= groups) g = groups - 1;  // recomputes a valid group; stored only if live
    int64_t e;  // element offset of the group in x
    if (DENSE) {
      e = g * 8;
    } else if (IDX32) {
      const uint32_t row = (uint32_t)g / (uint32_t)gpr;
      e = (int64_t)row * ld + (int64_t)((uint32_t)g - row * (uint32_t)gpr) * 8;
    } else {
      const int64_t row = g / gpr;
      e = row * ld + (g - row * gpr) * 8;
    }
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(x) + e * EB);
    raw[u][0] = __builtin_nontemporal_load(src);  // x is read exactly once
    if (FP32) raw[u][FP32 ? 1 : 0] = __builtin_nontemporal_load(src + 1);
  }
#pragma unroll
  for (int u = 0; u < MQ_U; ++u) {
    const int64_t g = g0 + 256 * u;
    float v[8];
    if (FP32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = __uint_as_float(raw[u][0][i]);
        v[4 + i] = __uint_as_float(raw[u][FP32 ? 1 : 0][i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(raw[u][0][i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(raw[u][0][i] >> 16);
      }
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, abs_bits(v[i]));
    // the four lanes of a 32-element block are consecutive (groups are
    // 32-aligned in a row and rows hold whole blocks)
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2));
    uint32_t c0 = 0, c1 = 0, sc;
    if (m >= 0x7F800000u) {
      c0 = c1 = 0x7F7F7F7Fu;
      sc = 0xFF;
    } else {
      const int E = mx_block_exp(m);
      c0 = e4m3_pack4(v[0], v[1], v[2], v[3], E);
      c1 = e4m3_pack4(v[4], v[5], v[6], v[7], E);
      sc = (uint32_t)(E + 127);
    }
    if (g < groups) {
      *reinterpret_cast<uint2*>(codes + g * 8) = make_uint2(c0, c1);
      if ((g & 3) == 0) scales[g >> 2] = (uint8_t)sc;
    }
  }
}

// Quantization along the columns, stored transposed (the blocked axis
// contiguous), for operands whose product reduces over the matrix's rows.
// One workgroup takes 128 rows x 64 columns: 16-byte row loads into LDS
// (16-byte chunk c of row r at chunk c ^ 2 (r / 32), so the column reads
// below touch 8 distinct chunks), then lane l of wave w owns column
// 16 w + l / 4 and the 32-row block l % 4, whole in one thread: amax, scale
// and 32 codes, stored as 32 contiguous bytes (four lanes write a column's
// 128 bytes). Rows at or past `rows` read as zeros.
constexpr int QT_ROWS = 128, QT_COLS = 64;

__global__ __launch_bounds__(256) void mxfp8_quant_t_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ld, int64_t rows_pad,
                                                            uint8_t* __restrict__ codes_t,
                                                            uint8_t* __restrict__ scales_t) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[QT_ROWS * 128];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * QT_COLS;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = 16 * wave + (lane >> 2), b = lane & 3;
  const int64_t c = c0 + cl;
  const int64_t row_tiles = (rows_pad + QT_ROWS - 1) / QT_ROWS;
  // row tiles grid-strided (the launch caps the grid's x extent)
  for (int64_t rt = blockIdx.x; rt < row_tiles; rt += gridDim.x) {
    const int64_t r0 = rt * QT_ROWS;
    __syncthreads();  // the previous tile's readers are done
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 32 * j + (tid >> 3), chunk = tid & 7;
      const int64_t r = r0 + row, cc = c0 + 8 * chunk;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < rows && cc < cols) v = *reinterpret_cast<const uint4*>(x + r * ld + cc);
      *reinterpret_cast<uint4*>(tile + row * 128 + ((chunk ^ (2 * j)) << 4)) = v;
    }
    __syncthreads();
    const int64_t rb = r0 + 32 * b;
    if (c >= cols || rb >= rows_pad) continue;
    const uint8_t* col = tile + ((((cl >> 3) ^ (2 * b)) << 4) + 2 * (cl & 7)) + 32 * b * 128;
    float v[32];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(col + i * 128));
      m = max(m, abs_bits(v[i]));
    }
    uint32_t P[8];
    uint32_t sc;
    if (m >= 0x7F800000u) {
#pragma unroll
      for (int k = 0; k < 8; ++k) P[k] = 0x7F7F7F7Fu;
      sc = 0xFF;
    } else {
      const int E = mx_block_exp(m);
#pragma unroll
      for (int k = 0; k < 8; ++k) P[k] = e4m3_pack4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3], E);
      sc = (uint32_t)(E + 127);
    }
    uint8_t* dst = codes_t + c * rows_pad + rb;
    reinterpret_cast<u32x4_t*>(dst)[0] = u32x4_t{P[0], P[1], P[2], P[3]};
    reinterpret_cast<u32x4_t*>(dst)[1] = u32x4_t{P[4], P[5], P[6], P[7]};
    scales_t[c * (rows_pad / 32) + rb / 32] = (uint8_t)sc;
  }
}

}  // namespace

hipError_t launch_mxfp8_quantize_t(const void* x, int64_t rows, int64_t cols, int64_t ld, int64_t rows_pad,
                                   uint8_t* codes_t, uint8_t* scales_t, hipStream_t stream) {
  const int64_t row_tiles = (rows_pad + QT_ROWS - 1) / QT_ROWS;
  const dim3 grid((unsigned)std::min<int64_t>(row_tiles, 1 << 16), (unsigned)((cols + QT_COLS - 1) / QT_COLS));
  hipLaunchKernelGGL(mxfp8_quant_t_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x), rows,
                     cols, ld, rows_pad, codes_t, scales_t);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quantize(const void* x, int x_fp32, int64_t rows, int64_t cols, int64_t ld,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t gpr = cols / 8;
  const int64_t groups = rows * gpr;
  const dim3 grid((unsigned)((groups + 256 * MQ_U - 1) / (256 * MQ_U)));
  const bool dense = ld == cols, idx32 = groups < ((int64_t)1 << 32);
#define MQ_LAUNCH(F, D, I) \
  hipLaunchKernelGGL((mxfp8_quant_kernel<F, D, I>), grid, dim3(256), 0, stream, x, groups, gpr, ld, codes, scales)
  if (x_fp32) {
    if (dense) MQ_LAUNCH(true, true, true);
    else if (idx32) MQ_LAUNCH(true, false, true);
    else MQ_LAUNCH(true, false, false);
  } else {
    if (dense) MQ_LAUNCH(false, true, true);
    else if (idx32) MQ_LAUNCH(false, false, true);
    else MQ_LAUNCH(false, false, false);
  }
#undef MQ_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
