// Host-side planning of the backward's work split and workspace (no kernels,
// no HIP calls beyond the cached compute-unit count): inverse-RoPE row bands,
// reduction splits of the dX and dW products, and the byte layout of the
// caller's workspace. Kept apart from the kernels so the C ABI's validation
// and planning build as plain host C++ too (sanitizer builds).
#include "internal.h"

namespace mla {
namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace


// Reduction splits of a backward GEMM: the split count s (1..8) whose rounds
// of resident workgroups cover the work in the least time, ceil(tiles s /
// slots) rounds of ceil(stages / s) stages, preferring fewer splits (each
// split adds an fp32 partial of the output to write and reduce) and at least
// 8 stages per split.
static int split_count(int64_t tiles, int64_t stages) {
  const int cus = device_cu_count();
  const int64_t slots = (int64_t)(cus > 0 ? cus : 256) * BG_WG_PER_CU;
  int best = 1;
  int64_t best_cost = ((tiles + slots - 1) / slots) * stages;
  for (int s = 2; s <= 8; ++s) {
    const int64_t sps = (stages + s - 1) / s;
    if (sps < 8) break;
    const int64_t cost = ((tiles * s + slots - 1) / slots) * sps;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  const int64_t sps = (stages + best - 1) / best;
  return (int)((stages + sps - 1) / sps);  // no empty split
}

// Reduction values per stage of the dX GEMM: 64 (whole 128-byte lines of
// dq_pre per row) when N allows it.
int dx_stage_depth(int N) { return N % 64 == 0 ? 64 : 32; }

static int dx_split_count(int64_t T, int N, int K) {
  const int64_t tiles = ((T + BG_TJ - 1) / BG_TJ) * ((K + BG_TI - 1) / BG_TI);
  return split_count(tiles, N / dx_stage_depth(N));
}

// dW reduces over the tokens, 64 per stage; with few heads (N / 128 row
// tiles) its tiles alone cannot fill the chip. Its output is large, so the
// split count weighs the partials too: a round of stages takes about 1.3 us,
// and each split's fp32 partial (N K 4 bytes) is written once and read once
// by the reduction at about 6 TB/s.
static int dw_split_count(int64_t T, int N, int K) {
  const int64_t tiles = (int64_t)((N + BG_TJ - 1) / BG_TJ) * ((K + BG_TI - 1) / BG_TI);
  const int64_t stages = (T + 63) / 64;
  const int cus = device_cu_count();
  const int64_t slots = (int64_t)(cus > 0 ? cus : 256) * BG_WG_PER_CU;
  const double stage_us = 1.3, part_us = (double)N * K * 8 / 6e6;
  int best = 1;
  double best_cost = (double)((tiles + slots - 1) / slots) * stages * stage_us;
  for (int s = 2; s <= 8; ++s) {
    const int64_t sps = (stages + s - 1) / s;
    if (sps < 8) break;
    const double cost = (double)((tiles * s + slots - 1) / slots) * sps * stage_us + s * part_us;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  const int64_t sps = (stages + best - 1) / best;
  return (int)((stages + sps - 1) / sps);  // no empty split
}

BwdPlan plan_bwd(int64_t T, int N, int K, bool use_bias, bool want_dx, bool want_dw, bool allow_splits) {
  BwdPlan pl{};
  // Rows per inverse-RoPE workgroup: the most (up to 64) that still give
  // 1536 workgroups, the count that runs at copy speed at DeepSeek-V3 shape
  // (with few heads, 64-row bands leave most of the chip idle).
  const int64_t col_blocks = (N + IR_COLS - 1) / IR_COLS;
  pl.ir_rows = 8;
  for (int r = IR_ROWS; r > 8; r /= 2)
    if (col_blocks * ((T + r - 1) / r) >= 1536) {
      pl.ir_rows = r;
      break;
    }
  pl.db_row_chunks = (int)((T + pl.ir_rows - 1) / pl.ir_rows);
  pl.db_off = 0;
  pl.db_bytes = use_bias ? align256((size_t)pl.db_row_chunks * N * 4) : 0;
  pl.dx_splits = want_dx && T > 0 && allow_splits ? dx_split_count(T, N, K) : 1;
  pl.dx_off = pl.db_bytes;
  pl.dx_bytes = pl.dx_splits > 1 ? align256((size_t)pl.dx_splits * T * K * 4) : 0;
  pl.dw_splits = want_dw && T > 0 && allow_splits ? dw_split_count(T, N, K) : 1;
  pl.dw_off = pl.dx_off + pl.dx_bytes;
  pl.dw_bytes = pl.dw_splits > 1 ? align256((size_t)pl.dw_splits * N * K * 4) : 0;
  pl.total = pl.db_bytes + pl.dx_bytes + pl.dw_bytes;
  return pl;
}

static int mx_split_count(int64_t tiles, int64_t stages) {
  const int cus = device_cu_count();
  const int64_t slots = (int64_t)(cus > 0 ? cus : 256) * 2;
  int best = 1;
  int64_t best_cost = ((tiles + slots - 1) / slots) * stages;
  for (int s = 2; s <= 8; ++s) {
    const int64_t sps = (stages + s - 1) / s;
    if (sps < 4) break;
    const int64_t cost = ((tiles * s + slots - 1) / slots) * sps;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  // the kernel gives each split ceil(stages / splits) stages: no split may
  // start past the end
  int s = best;
  while (s > 1 && (int64_t)(s - 1) * ((stages + s - 1) / s) >= stages) --s;
  return s;
}

MxBwdPlan plan_bwd_mx(int64_t T, int N, int K, bool use_bias) {
  MxBwdPlan pl{};
  pl.base = plan_bwd(T, N, K, use_bias, false, false);
  // the fused pass over dq takes bands of MX_BAND_ROWS rows: one db partial
  // row per band
  pl.base.ir_rows = MX_BAND_ROWS;
  pl.base.db_row_chunks = (int)((T + MX_BAND_ROWS - 1) / MX_BAND_ROWS);
  pl.base.db_bytes = use_bias ? align256((size_t)pl.base.db_row_chunks * N * 4) : 0;
  pl.base.total = pl.base.db_bytes;
  pl.Tp = (T + 127) / 128 * 128;
  size_t off = pl.base.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  pl.dq_rows = take((size_t)T * N);
  pl.dq_rows_sc = take((size_t)T * N / 32);
  pl.dq_t = take((size_t)N * pl.Tp);
  pl.dq_t_sc = take((size_t)N * pl.Tp / 32);
  pl.w_t = take((size_t)K * N);
  pl.w_t_sc = take((size_t)K * N / 32);
  pl.x_t = take((size_t)K * pl.Tp);
  pl.x_t_sc = take((size_t)K * pl.Tp / 32);
  pl.dx_splits = T > 0 ? mx_split_count(mx_gemm_tiles(T, K), N / 128) : 1;
  pl.dx_part = pl.dx_splits > 1 ? take((size_t)pl.dx_splits * T * K * 4) : 0;
  pl.total = T > 0 ? off : 0;
  return pl;
}

// Output tiles of the MXFP8 product form (the forward kernel's tiles).
int mx_gemm_tiles(int64_t rows, int cols) {
  return (int)(((rows + FWD_TILE_T - 1) / FWD_TILE_T) * ((cols + FWD_TILE_N - 1) / FWD_TILE_N));
}

}  // namespace mla
