// Internal launch interface between the C ABI (api.hip) and the kernels.
// Every launcher assumes its arguments were validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_qup.h"

namespace mla {

// Work decomposition shared by the kernels and the host planner (plan.hip).
constexpr int FWD_TILE_T = 128;           // forward tile: tokens
constexpr int FWD_TILE_N = 192;           // forward tile: rows of N
constexpr int IR_THREADS = 128;           // inverse-RoPE workgroup
constexpr int IR_COLS = IR_THREADS * 8;   // its columns
constexpr int IR_ROWS = 64;               // its token rows, at most
// Token rows per band of the MXFP8 backward's fused pass over dq (db
// partials: one row per band).
constexpr int MX_BAND_ROWS = 128;
constexpr int BG_TI = 192;                // backward GEMM tile: output columns
constexpr int BG_TJ = 128;                // backward GEMM tile: output rows
constexpr int BG_WG_PER_CU = 2;           // backward GEMM workgroups per CU

struct FwdParams {
  const void* x;           // bf16 [T,K] or e4m3 codes [T,K]
  const uint8_t* xs;       // MXFP8 x scales [T,K/32]
  const void* w;           // bf16 [N,K] or e4m3 codes [N,K]
  const uint8_t* ws;       // MXFP8 w scales [N,K/32]
  const uint16_t* bias;    // bf16 [N] or nullptr
  int64_t T;
  int K, N, H, D, d_nope, d_rope;
  int fmt, B, S;           // BHSD output dims; THD: B = 1, S = T
  const int32_t* cu;
  int nseq;
  const float* cos;
  const float* sin;
  int rope_rows, rope_pairs;
  int out_mx;              // 1: MXFP8 codes + scales, 0: bf16
  int mx_fp8_mfma;         // MXFP8 operands on the scaled FP8 MFMA (else exact bf16 MFMA)
  int rope_lds;            // set by the launcher: stage each tile's table rows in LDS
  // plain product form (launch_mx_gemm): out[t][n] row-major with stride N,
  // fp32 when out_f32 (else bf16); K split into k_splits stage ranges, range
  // s writing at out + s * split_stride bytes
  int out_f32, k_splits;
  int64_t split_stride;
  void* out;
  uint8_t* out_scales;
};

struct BwdParams {
  const uint16_t* dq;
  const uint16_t* x;
  const uint16_t* w;
  int64_t T;
  int K, N, H, D, d_nope, d_rope;
  int fmt, B, S;
  const int32_t* cu;
  int nseq;
  const float* cos;
  const float* sin;
  int rope_rows, rope_pairs;
  uint16_t* dq_pre;
  uint16_t* dx;
  void* dw;
  int dw_fp32;
  int use_bias;
  uint16_t* db;
  void* workspace;
};

// Workspace plan of the backward: byte offsets into the caller's workspace.
struct BwdPlan {
  int ir_rows;             // token rows per inverse-RoPE workgroup (8..64)
  int db_row_chunks;       // token chunks of the db partial sums (one per such row band)
  size_t db_off, db_bytes;
  int dx_splits;           // reduction splits of the dX GEMM (1 = none)
  size_t dx_off, dx_bytes;
  int dw_splits;           // reduction (token) splits of the dW GEMM (1 = none)
  size_t dw_off, dw_bytes;
  size_t total;
};
// MXFP8 backward workspace: the bf16 backward's db partials, then the
// quantized operands (offsets in bytes, 256-aligned) and dX split partials.
struct MxBwdPlan {
  BwdPlan base;
  int64_t Tp;                    // tokens padded to a multiple of 128
  size_t dq_rows, dq_rows_sc;    // dq_pre along n: codes [T, N], scales [T, N/32]
  size_t dq_t, dq_t_sc;          // dq_pre along t, transposed: [N, Tp], [N, Tp/32]
  size_t w_t, w_t_sc;            // W along n, transposed: [K, N], [K, N/32]
  size_t x_t, x_t_sc;            // X along t, transposed: [K, Tp], [K, Tp/32]
  int dx_splits;                 // reduction splits of dX (fp32 partials [splits, T, K])
  size_t dx_part;
  size_t total;
};
// allow_splits = false plans dX and dW without reduction splits (no split
// partials: the smallest workspace).
BwdPlan plan_bwd(int64_t T, int N, int K, bool use_bias, bool want_dx, bool want_dw, bool allow_splits = true);
// Reduction values per stage of the dX product (64, or 32 when N % 64 != 0).
int dx_stage_depth(int N);

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count();

hipError_t launch_rope_cache(float* cos, float* sin, int rows, int d_rope, double base,
                             const mla_yarn* yarn, hipStream_t stream);
// KV side: fresh key = [k_nope | rotated k_pe] and value, BHSD, bf16 or MXFP8.
struct KvParams {
  const uint16_t* kv;      // bf16 [T, H, d_nope + d_v]
  const uint16_t* pe;      // bf16 [T, d_rope]
  int64_t T;
  int H, d_nope, d_rope, d_v;
  int fmt, B, S;
  const int32_t* cu;
  int nseq;
  const float* cos;
  const float* sin;
  int rope_rows, rope_pairs;
  int out_mx;
  void* key;               // [B, H, S, d_nope + d_rope]
  uint8_t* key_scales;     // [B, H, S, (d_nope + d_rope) / 32]
  void* value;             // [B, H, S, d_v]
  uint8_t* value_scales;   // [B, H, S, d_v / 32]
};
hipError_t launch_kv_rope(const KvParams& p, hipStream_t stream);
hipError_t launch_mxfp8_quantize_t(const void* x, int64_t rows, int64_t cols, int64_t ld, int64_t rows_pad,
                                   uint8_t* codes_t, uint8_t* scales_t, hipStream_t stream);
hipError_t launch_mxfp8_quantize(const void* x, int x_fp32, int64_t rows, int64_t cols,
                                 int64_t ld, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);
hipError_t launch_qup_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_qup_fwd_mx(const FwdParams& p, hipStream_t stream);
// MXFP8 x MXFP8 product out[t][n] = sum_k X[t][k] W[n][k] in the plain form
// (FwdParams: x, xs, w, ws, T, K, N, mx_fp8_mfma, out, out_f32, k_splits,
// split_stride; K % 128 == 0).
hipError_t launch_mx_gemm(const FwdParams& p, hipStream_t stream);
int mx_gemm_tiles(int64_t rows, int cols);
hipError_t launch_qup_bwd(const BwdParams& p, const BwdPlan& plan, hipStream_t stream);
MxBwdPlan plan_bwd_mx(int64_t T, int N, int K, bool use_bias);
hipError_t launch_qup_bwd_mx(const BwdParams& p, const MxBwdPlan& pl, int fp8_mfma, hipStream_t stream);

}  // namespace mla
