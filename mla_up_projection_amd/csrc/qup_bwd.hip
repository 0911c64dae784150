// Backward of the fused MLA query up-projection for gfx950.
// Page "Add a backwards linear function to be used with the fused mla q
// up-proj" (summary, sequence diagram): the query-output gradient goes
// through the RoPE backward, giving the pre-RoPE projection gradient; the
// linear backward then gives the input and weight gradients; review comment
// "BF16 bias gradient remains missing": with use_bias the bias gradient is
// produced. Page "Fix fused MLA YaRN RoPE query kernel corrupting upstream
// tensor in-place" (review thread): dw = dy^T x with x the saved input.
//
//   inv_rope_kernel : dq [T,N] -> dq_pre [T,N] (bf16), adjoint rotation of
//                     each rope pair; per-chunk fp32 column sums for db.
//                     HBM-bound: 2 B read + 2 B written per element.
//   db_reduce_kernel: db[n] = sum over chunks in a fixed order (per-lane
//                     strided sums, then lane order).
//   bgemm_kernel    : dX = dq_pre W and dW = dq_pre^T X on bf16 MFMA; operands
//                     reach LDS by DMA in memory order, and an operand whose
//                     reduction axis is strided in memory is transposed by the
//                     LDS transpose read (ds_read_b64_tr_b16).
//   split_reduce_kernel: ordered sum of the reduction splits of dX (long N)
//                     or dW (few heads, long T) -> bf16 or fp32.
//   inv_rope_mx_kernel: the MXFP8 backward's one pass over dq: dq_pre, its
//                     codes along n and along the tokens (transposed), and
//                     the db partials.
//   launch_qup_bwd_mx: the MXFP8 backward (operands quantized along each
//                     product's reduction axis, products on the forward
//                     kernel's MXFP8 main loop).
// No floating-point atomics anywhere: results are run-to-run deterministic.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

// ---------------------------------------------------------------------------
// Inverse RoPE + db partials
// ---------------------------------------------------------------------------
// IR_THREADS, IR_COLS (columns per workgroup) and IR_ROWS (token rows per
// workgroup, at most) are shared with the host planner (internal.h).

// Inverse rotation of one (even, odd) pair by the angle whose cosine and sine
// are c and s, with its fused multiply-adds written out so that every kernel
// applying it rounds alike.
__device__ __forceinline__ void inv_rotate(float& a, float& b, float c, float s) {
  const float na = fmaf(a, c, b * s);
  const float nb = fmaf(b, c, -(a * s));
  a = na;
  b = nb;
}

// Bands of `band` token rows (at most IR_ROWS) are strided over the grid's y
// extent, which the launch caps; each band's column sums go to its own db
// partial row.
__global__ __launch_bounds__(IR_THREADS) void inv_rope_kernel(BwdParams p, int band, int64_t bands,
                                                              float* __restrict__ db_part) {
  __shared__ int s_pos[IR_ROWS];
  const TokenMap tm{p.fmt, p.B, p.S, p.cu, p.nseq};
  const int n0 = blockIdx.x * IR_COLS + threadIdx.x * 8;
  const bool col_ok = n0 < p.N;
  const uint16_t* __restrict__ dq = p.dq;
  uint16_t* __restrict__ dq_pre = p.dq_pre;
  const float* __restrict__ cos_t = p.cos;
  const float* __restrict__ sin_t = p.sin;
  const int d0 = (col_ok ? n0 : 0) % p.D;  // 8 consecutive columns stay inside one head
  bool rot[4];
  int pi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = d0 + 2 * k;
    rot[k] = p.d_rope > 0 && d >= p.d_nope;
    pi[k] = rot[k] ? (d - p.d_nope) >> 1 : 0;
  }
  const bool any_rot = rot[0] || rot[1] || rot[2] || rot[3];
  // all four pairs rotated and their table entries 16-byte aligned: one
  // float4 of cos and one of sin per row
  const bool vec4 = rot[0] && rot[3] && (pi[0] & 3) == 0 && (p.rope_pairs & 3) == 0;
  for (int64_t bi = blockIdx.y; bi < bands; bi += gridDim.y) {
    const int64_t r0 = bi * band;
    const int rows = (int)min((int64_t)band, p.T - r0);
    __syncthreads();  // the previous band's readers of s_pos are done
    for (int i = threadIdx.x; i < rows; i += IR_THREADS) {
      int pos, b, s;
      token_coords(tm, r0 + i, pos, b, s);
      s_pos[i] = pos;
    }
    __syncthreads();
    if (!col_ok) continue;
    float sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // Rows in batches of RB: all loads of a batch are issued before any
    // store, so RB 16-byte loads per lane are in flight at once. dq is read
    // exactly once (non-temporal load); dq_pre is read again by the GEMMs.
    constexpr int RB = 8;
    for (int i0 = 0; i0 < rows; i0 += RB) {
      u32x4_t g[RB];
      float cs[RB][4], sn[RB][4];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int i = i0 + j < rows ? i0 + j : rows - 1;
        g[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(dq + (r0 + i) * p.N + n0));
        if (any_rot) {
          const int pos = s_pos[i];
          const bool pos_ok = pos >= 0 && pos < p.rope_rows;
          const int64_t trow = (int64_t)(pos_ok ? pos : 0) * p.rope_pairs;
          if (vec4) {
            const float4 c4 = *reinterpret_cast<const float4*>(cos_t + trow + pi[0]);
            const float4 s4 = *reinterpret_cast<const float4*>(sin_t + trow + pi[0]);
            cs[j][0] = c4.x; cs[j][1] = c4.y; cs[j][2] = c4.z; cs[j][3] = c4.w;
            sn[j][0] = s4.x; sn[j][1] = s4.y; sn[j][2] = s4.z; sn[j][3] = s4.w;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              cs[j][k] = rot[k] ? cos_t[trow + pi[k]] : 1.0f;
              sn[j][k] = rot[k] ? sin_t[trow + pi[k]] : 0.0f;
            }
          }
          if (!pos_ok) {
#pragma unroll
            for (int k = 0; k < 4; ++k) cs[j][k] = sn[j][k] = __builtin_nanf("");
          }
        }
      }
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (i0 + j >= rows) break;
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float a = bf16_bits_to_f32(g[j][k] & 0xFFFFu);
          float b = bf16_bits_to_f32(g[j][k] >> 16);
          if (any_rot && rot[k]) inv_rotate(a, b, cs[j][k], sn[j][k]);
          sum[2 * k] += a;
          sum[2 * k + 1] += b;
          o[k] = pack_bf16x2(a, b);
        }
        *reinterpret_cast<u32x4_t*>(dq_pre + (r0 + i0 + j) * p.N + n0) = u32x4_t{o[0], o[1], o[2], o[3]};
      }
    }
    if (db_part) {
      float* dst = db_part + bi * p.N + n0;
      reinterpret_cast<float4*>(dst)[0] = make_float4(sum[0], sum[1], sum[2], sum[3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(sum[4], sum[5], sum[6], sum[7]);
    }
  }
}

// MXFP8 backward's pass over dq, fused: inverse RoPE into dq_pre (bf16),
// dq_pre quantized along n (the dX operand, [T, N] codes + [T, N/32]
// scales), dq_pre quantized along the tokens and stored transposed (the dW
// operand, [N, Tp] codes + [N, Tp/32] scales, rows past T as zeros), and the
// db partial sums of each 128-row band. One read of dq instead of a second
// pass that reads dq_pre back for the quantization along the tokens.
// Workgroup tile: 128 token rows (four 32-row blocks) x 128 columns, kept in
// LDS as bf16 between the two phases (row pitch 256 B). N is a multiple of
// 128, so every tile is whole along n.
//   Phase 1: thread t takes 8-column chunk t % 16 of rows t / 16 + 16 i
//     (i < 8); the eight 16-byte dq loads and their cos/sin entries are all
//     issued before any arithmetic. Rotates, stores dq_pre, quantizes along n
//     (the four lanes of a 32-column block share its amax through two quad
//     DPP moves); rows past T are zeros in LDS and stored nowhere.
//   Phase 2: wave w takes row block w; lane l the columns 2 l and 2 l + 1:
//     32 four-byte LDS reads down the column pair (one wave reads a 256-byte
//     row per step), one amax per column, 32 codes per column stored as 32
//     contiguous bytes; the four waves write each column's 128 bytes.
// db: each thread sums its 8 rows of its 8 columns in row order; the 16 row
// groups are added in a fixed tree (the four of a wave by xor-shuffles, then
// the four waves in order), so the partial sums are deterministic.
// Bands whose 128 rows are all tokens take a path with no per-row checks.
constexpr int MXB_ROWS = 128;
constexpr int MXB_COLS = 128;
static_assert(MXB_ROWS == MX_BAND_ROWS, "the planner sizes the db partials by this band");

// Largest value of m over the four lanes of an aligned quad (DPP quad
// permutations: lanes xor 1, then xor 2).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, true));
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, true));
  return m;
}

// Float32 bit pattern of the largest |x| over the 2 k bf16 values packed in
// w[0 .. k-1] (low halves and high halves maxed apart, as integers).
template <int K>
__device__ __forceinline__ uint32_t packed_bf16_amax(const uint32_t* w) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    lo = max(lo, w[i] & 0x7FFFu);
    hi = max(hi, w[i] & 0x7FFF0000u);
  }
  return max(lo << 16, hi);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool FULL>
__device__ __forceinline__ void mx_pass_band(const BwdParams& p, int64_t Tp, int64_t band, int rows, int nt0,
                                             float* __restrict__ db_part, uint8_t* __restrict__ rc,
                                             uint8_t* __restrict__ rs, uint8_t* __restrict__ tc,
                                             uint8_t* __restrict__ ts, uint32_t* tile, float (*red)[MXB_COLS],
                                             const int* s_pos) {
  const int tid = threadIdx.x;
  const int64_t r0 = band * MXB_ROWS;

  // ---- phase 1 ----
  const int chunk = tid & 15, rg = tid >> 4;
  const int n0 = nt0 + 8 * chunk;
  const int d0 = n0 % p.D;  // 8 consecutive columns stay inside one head
  bool rot[4];
  int pi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = d0 + 2 * k;
    rot[k] = p.d_rope > 0 && d >= p.d_nope;
    pi[k] = rot[k] ? (d - p.d_nope) >> 1 : 0;
  }
  const bool any_rot = rot[0] || rot[1] || rot[2] || rot[3];
  const bool vec4 = rot[0] && rot[3] && (pi[0] & 3) == 0 && (p.rope_pairs & 3) == 0;
  const int64_t step = (int64_t)16 * p.N;  // elements between a thread's rows
  const uint16_t* src = p.dq + (r0 + rg) * p.N + n0;
  u32x4_t g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (FULL || rg + 16 * i < rows)
      g[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i * step));
    else
      g[i] = u32x4_t{0, 0, 0, 0};
  }
  float cs[8][4], sn[8][4];
  if (any_rot) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pos = s_pos[rg + 16 * i];  // -1: beyond the table; pad rows hold 0
      if (pos >= 0) {
        const float* ct = p.cos + (int64_t)pos * p.rope_pairs;
        const float* st = p.sin + (int64_t)pos * p.rope_pairs;
        if (vec4) {
          const float4 c4 = *reinterpret_cast<const float4*>(ct + pi[0]);
          const float4 s4 = *reinterpret_cast<const float4*>(st + pi[0]);
          cs[i][0] = c4.x; cs[i][1] = c4.y; cs[i][2] = c4.z; cs[i][3] = c4.w;
          sn[i][0] = s4.x; sn[i][1] = s4.y; sn[i][2] = s4.z; sn[i][3] = s4.w;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            cs[i][k] = rot[k] ? ct[pi[k]] : 1.0f;
            sn[i][k] = rot[k] ? st[pi[k]] : 0.0f;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) cs[i][k] = sn[i][k] = __builtin_nanf("");
      }
    }
  }
  float sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint16_t* dst_pre = p.dq_pre + (r0 + rg) * p.N + n0;
  uint8_t* dst_rc = rc ? rc + (r0 + rg) * p.N + n0 : nullptr;
  uint8_t* dst_rs = rs ? rs + (r0 + rg) * (p.N / 32) + n0 / 32 : nullptr;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool live = FULL || rg + 16 * i < rows;
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float a = bf16_lo(g[i][k]);
      float b = bf16_hi(g[i][k]);
      if (any_rot && rot[k]) inv_rotate(a, b, cs[i][k], sn[i][k]);
      if (db_part) {
        sum[2 * k] += live ? a : 0.0f;
        sum[2 * k + 1] += live ? b : 0.0f;
      }
      o[k] = live ? pack_bf16x2(a, b) : 0u;
    }
    *reinterpret_cast<u32x4_t*>(tile + (rg + 16 * i) * (MXB_COLS / 2) + 4 * chunk) = u32x4_t{o[0], o[1], o[2], o[3]};
    if (live) *reinterpret_cast<u32x4_t*>(dst_pre + i * step) = u32x4_t{o[0], o[1], o[2], o[3]};
    if (rc) {
      // along n from the bf16 copy; the four lanes of the block share its row
      const uint32_t m = quad_max_u32(packed_bf16_amax<4>(o));
      uint32_t c0, c1, sc;
      if (m >= 0x7F800000u) {
        c0 = c1 = 0x7F7F7F7Fu;
        sc = 0xFF;
      } else {
        const int E = mx_block_exp(m);
        c0 = e4m3_pack4(bf16_lo(o[0]), bf16_hi(o[0]), bf16_lo(o[1]), bf16_hi(o[1]), E);
        c1 = e4m3_pack4(bf16_lo(o[2]), bf16_hi(o[2]), bf16_lo(o[3]), bf16_hi(o[3]), E);
        sc = (uint32_t)(E + 127);
      }
      if (live) {
        *reinterpret_cast<uint2*>(dst_rc + i * step) = make_uint2(c0, c1);
        if ((chunk & 3) == 0) dst_rs[i * (step / 32)] = (uint8_t)sc;
      }
    }
  }
  if (db_part) {
    // the four row groups of a wave (lanes 16 apart) first: every lane ends
    // with (s0 + s1) + (s2 + s3), whatever its place in the four
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sum[k] += __shfl_xor(sum[k], 16);
      sum[k] += __shfl_xor(sum[k], 32);
    }
    if ((tid & 63) < 16) {
#pragma unroll
      for (int k = 0; k < 8; ++k) red[tid >> 6][8 * chunk + k] = sum[k];
    }
  }
  __syncthreads();

  // ---- phase 2 ----
  if (db_part && (FULL || rows > 0) && tid < MXB_COLS)
    db_part[band * p.N + nt0 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
  if (tc) {
    const int lane = tid & 63, blk = tid >> 6;
    // the column pair as 32 packed bf16 words
    uint32_t wv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) wv[i] = tile[(32 * blk + i) * (MXB_COLS / 2) + lane];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      lo = max(lo, wv[i] & 0x7FFFu);
      hi = max(hi, wv[i] & 0x7FFF0000u);
    }
    const int64_t tb = r0 + 32 * blk;  // first token of the block (< Tp)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t m = h ? hi : lo << 16;
      uint32_t P[8], sc;
      if (m >= 0x7F800000u) {
#pragma unroll
        for (int k = 0; k < 8; ++k) P[k] = 0x7F7F7F7Fu;
        sc = 0xFF;
      } else {
        const int E = mx_block_exp(m);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t* q = wv + 4 * k;
          P[k] = h ? e4m3_pack4(bf16_hi(q[0]), bf16_hi(q[1]), bf16_hi(q[2]), bf16_hi(q[3]), E)
                   : e4m3_pack4(bf16_lo(q[0]), bf16_lo(q[1]), bf16_lo(q[2]), bf16_lo(q[3]), E);
        }
        sc = (uint32_t)(E + 127);
      }
      const int64_t col = nt0 + 2 * lane + h;
      uint8_t* dst = tc + col * Tp + tb;
      reinterpret_cast<u32x4_t*>(dst)[0] = u32x4_t{P[0], P[1], P[2], P[3]};
      reinterpret_cast<u32x4_t*>(dst)[1] = u32x4_t{P[4], P[5], P[6], P[7]};
      ts[col * (Tp / 32) + tb / 32] = (uint8_t)sc;
    }
  }
}

__global__ __launch_bounds__(256) void inv_rope_mx_kernel(BwdParams p, int64_t Tp, float* __restrict__ db_part,
                                                          uint8_t* __restrict__ rc, uint8_t* __restrict__ rs,
                                                          uint8_t* __restrict__ tc, uint8_t* __restrict__ ts,
                                                          int col_tiles) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[MXB_ROWS * MXB_COLS / 2];  // bf16 pairs
  __shared__ float red[4][MXB_COLS];  // db: one row of column sums per wave
  __shared__ int s_pos[MXB_ROWS];
  // one-dimensional grid, column tile fastest: the workgroups of a band are
  // dispatched together and read its rows whole
  const int64_t band = blockIdx.x / (uint32_t)col_tiles;
  const int64_t r0 = band * MXB_ROWS;
  const int rows = (int)max((int64_t)0, min((int64_t)MXB_ROWS, p.T - r0));  // 0 for a band of padding only
  const int nt0 = (int)(blockIdx.x - band * col_tiles) * MXB_COLS;
  const TokenMap tm{p.fmt, p.B, p.S, p.cu, p.nseq};
  if (threadIdx.x < MXB_ROWS) {
    const int i = threadIdx.x;
    int pos = 0;  // pad rows: any row of the table (their values are dropped)
    if (i < rows) {
      int b, s;
      token_coords(tm, r0 + i, pos, b, s);
      if (pos < 0 || pos >= p.rope_rows) pos = -1;
    }
    s_pos[i] = pos;
  }
  __syncthreads();
  if (rows == MXB_ROWS)
    mx_pass_band<true>(p, Tp, band, rows, nt0, db_part, rc, rs, tc, ts, tile, red, s_pos);
  else
    mx_pass_band<false>(p, Tp, band, rows, nt0, db_part, rc, rs, tc, ts, tile, red, s_pos);
}

// db[n] = sum of the per-chunk partials in a fixed order: G lanes per column
// each add every G-th chunk, then the G partial sums are added in lane order.
// G = 8, or 32 when there are many chunks (short token bands) so that each
// lane's serial chain stays short.
constexpr int DBR_COLS = 32;
template <int G>
__global__ __launch_bounds__(DBR_COLS * G) void db_reduce_kernel(const float* __restrict__ part, int chunks,
                                                                int N, uint16_t* __restrict__ db) {
  __shared__ float red[G][DBR_COLS];
  const int c = threadIdx.x % DBR_COLS;
  const int g = threadIdx.x / DBR_COLS;
  const int n = blockIdx.x * DBR_COLS + c;
  float s = 0.0f;
  if (n < N)
    for (int k = g; k < chunks; k += G) s += part[(int64_t)k * N + n];
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && n < N) {
    float t = red[0][c];
#pragma unroll
    for (int q = 1; q < G; ++q) t += red[q][c];
    db[n] = (uint16_t)f32_to_bf16_bits(t);
  }
}

hipError_t launch_db_reduce(const float* part, int chunks, int N, uint16_t* db, hipStream_t stream) {
  const dim3 grid((N + DBR_COLS - 1) / DBR_COLS);
  if (chunks >= 128)
    hipLaunchKernelGGL(db_reduce_kernel<32>, grid, dim3(DBR_COLS * 32), 0, stream, part, chunks, N, db);
  else
    hipLaunchKernelGGL(db_reduce_kernel<8>, grid, dim3(DBR_COLS * 8), 0, stream, part, chunks, N, db);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward GEMMs on bf16 MFMA: out[j][i] = sum over r of P(i, r) Q(j, r).
//   dX[t][k] : i = k, j = t, r = n; P(k, n) = W[n][k]       (n-rows in memory)
//                                    Q(t, n) = dq_pre[t][n] (n contiguous)
//   dW[n][k] : i = k, j = n, r = t; P(k, t) = X[t][k]       (t-rows in memory)
//                                    Q(n, t) = dq_pre[t][n] (t-rows in memory)
// P is always stored with its reduction index r as the row ("MN-major"); Q is
// MN-major for dW and r-contiguous ("K-major") for dX.
//
// Persistent, two independent 256-thread workgroups per CU, tile 192 (i) x
// 128 (j); waves 2 x 2, each 96 (i) x 64 (j) = 3 x 2 blocks of the 32x32x16
// MFMA (P is the MFMA's row operand, so a lane holds 4 consecutive i of one j:
// 16-byte stores). The reduction streams through an LDS ring (2 slots of
// 64-value stages, or 4 slots of 32-value stages) filled by direct
// global->LDS DMA in memory order; nothing is transposed on the way in.
//   * MN-major stage = KS rows (r) x tile width, row pitch RP = 2 x width.
//     Fragments come from ds_read_b64_tr_b16: within each 16-lane group, lane
//     i receives element i%4 of the 8-byte row slices addressed by lanes
//     4e + i/4 (e = 0..3). Lane 16g+s addresses row 8(g/2) + 4h + s/4 (h = 0,
//     1 for the fragment's two reads), columns 16(g%2) + 4(s%4) .. +3 of its
//     32-column block, which yields the MFMA operand layout (lane l: column
//     l%32, reduction values 8(l/32) .. +7).
//     A 32-lane half of such a read touches 4 consecutive rows x 64 bytes;
//     64-byte segments are XOR-swizzled per row so those 4 land in distinct
//     bank quarters: segment s ^ (r & 3) when RP is a multiple of 256 bytes,
//     s ^ ((r >> 1) & 1) when RP = 128 mod 256.
//   * K-major stage = tile rows x 2 KS bytes, 16-byte chunk c of row r stored
//     at c ^ ((r >> 2) & 3) (64-byte rows) or c ^ ((r >> 1) & 7) (128-byte
//     rows), read with ds_read_b128 as in the forward.
//   * A reduction tail (r past the end inside the last stage) is read from a
//     clamped row and zeroed in both MN-major fragments before the MFMA. A
//     K-major Q requires a reduction length that is a multiple of 32.
// ---------------------------------------------------------------------------
// BG_TI, BG_TJ and BG_WG_PER_CU are shared with the host planner (internal.h).
constexpr int BG_THREADS = 256;
constexpr int BG_RPP = BG_TI * 2;          // P row pitch (MN-major), bytes
constexpr int BG_RPQ = BG_TJ * 2;          // Q row pitch when MN-major
constexpr int BG_BI = BG_TI / 64;          // 32-blocks of i per wave (2 waves along i)
constexpr int BG_BJ = BG_TJ / 64;          // 32-blocks of j per wave

// Stage layout for KS reduction values per stage. KS = 32: 4 ring slots of
// 20 KB; KS = 64 (a K-major Q then arrives as whole 128-byte lines per row):
// 2 slots of 40 KB. Both take 80 KB of LDS.
template <int KS>
struct Bg {
  static constexpr int STAGES = KS == 64 ? 2 : 4;
  static constexpr int PB = KS * BG_RPP;     // P part of a slot
  static constexpr int QB = KS * BG_RPQ;     // Q part (MN-major KS rows, or K-major TJ rows x 2 KS bytes)
  static constexpr int SB = PB + QB;
  static constexpr int LP = PB / 4096;       // P DMA loads (1 KB) per wave per stage
  static constexpr int LQ = QB / 4096;
  static constexpr int LPS = LP + LQ;
  static constexpr int NJS = KS / 16;        // k16 MFMA steps per stage
  static constexpr int QROWB = 2 * KS;       // K-major Q: bytes of a row per stage
  static constexpr int QCPR = QROWB / 16;    // its 16-byte chunks
  static constexpr int QRPL = 1024 / QROWB;  // its rows per 1 KB wave load
  static_assert(PB % 4096 == 0 && QB % 4096 == 0, "whole DMA rounds per stage");
};

// K-major chunk swizzle (as in the forward): 64-byte rows c ^ ((r >> 2) & 3),
// 128-byte rows c ^ ((r >> 1) & 7).
template <int ROWB>
__device__ __forceinline__ int k_swz(int r) { return ROWB == 64 ? (r >> 2) & 3 : (r >> 1) & 7; }

template <int RP>
__device__ __forceinline__ int mn_swz(int r) {
  if constexpr (RP % 256 == 0) return r & 3;
  else if constexpr (RP % 256 == 128) return (r >> 1) & 1;
  else return 0;  // RP = 64 or 192 mod 256: consecutive rows already differ
}

struct BGemm {
  const uint8_t* p;
  int64_t ldp;        // bytes between P rows (consecutive r)
  const uint8_t* q;
  int64_t ldq;        // bytes between Q rows (r for MN-major, j for K-major)
  int I, J;           // output columns / rows; I % 8 == 0
  int64_t R;          // reduction length
  int splits;         // reduction splits; split z covers stages [z*sps, (z+1)*sps)
  int sps;
  void* out;          // [splits][J][I] (fp32) or [J][I] (bf16), by the kernel's F32
};

struct BgGrid {
  int ti, tj, per, total;
};

__device__ __forceinline__ void bg_coords(const BgGrid& g, int u, int& z, int& ti, int& tj) {
  int v = u;
  if ((g.total & 7) == 0) v = (u & 7) * (g.total >> 3) + (u >> 3);  // one run of v per XCD
  z = v / g.per;
  const int w = v - z * g.per;
  ti = w % g.ti;  // i fastest: the tiles sharing a Q slice run together
  tj = w / g.ti;
}

// Per-lane DMA sources of one tile (independent of the stage).
template <int KS>
struct BgDma {
  int pr[Bg<KS>::LP];       // P: stage row
  uint32_t pc[Bg<KS>::LP];  // P: byte offset inside the row (tile column base included)
  int qr[Bg<KS>::LQ];       // Q MN-major: stage row; K-major: unused
  uint32_t qc[Bg<KS>::LQ];  // Q MN-major: byte offset in row; K-major: row offset + chunk
};

// Chunk e (16 bytes) of an MN-major stage of `COLS` columns: its stage row
// and the byte offset of its source in that row, columns clamped into the
// matrix (clamped chunks only feed discarded outputs).
template <int COLS>
__device__ __forceinline__ void mn_src(int e, int col0, int cols, int& row, uint32_t& off) {
  constexpr int CPR = COLS / 8;
  row = e / CPR;
  const int cp = e - row * CPR;
  int gc = 4 * ((cp >> 2) ^ mn_swz<COLS * 2>(row)) + (cp & 3);
  const int last = (cols - col0) / 8 - 1;
  if (gc > last) gc = last;
  off = (uint32_t)((col0 + gc * 8) * 2);
}

template <bool QK, int KS>
__device__ __forceinline__ BgDma<KS> bg_dma(const BGemm& g, int i0, int j0, int wave, int lane) {
  using B = Bg<KS>;
  BgDma<KS> d;
#pragma unroll
  for (int q = 0; q < B::LP; ++q) mn_src<BG_TI>((4 * q + wave) * 64 + lane, i0, g.I, d.pr[q], d.pc[q]);
  if (QK) {
#pragma unroll
    for (int q = 0; q < B::LQ; ++q) {
      const int row = B::QRPL * (4 * q + wave) + lane / B::QCPR;
      const int c = (lane % B::QCPR) ^ k_swz<B::QROWB>(row);
      int j = j0 + row;
      if (j >= g.J) j = g.J - 1;
      d.qr[q] = 0;
      d.qc[q] = (uint32_t)((int64_t)(j - j0) * g.ldq + c * 16);
    }
  } else {
#pragma unroll
    for (int q = 0; q < B::LQ; ++q) mn_src<BG_TJ>((4 * q + wave) * 64 + lane, j0, g.J, d.qr[q], d.qc[q]);
  }
  return d;
}

// Stage whose reduction rows start at rs (rows past rlim are clamped to it)
// into the ring slot at LDS address `slot`.
template <bool QK, int KS>
__device__ __forceinline__ void bg_issue(const BGemm& g, const BgDma<KS>& d, const uint8_t* qtile, int64_t rs,
                                         int rlim, uint32_t slot, int wave) {
  using B = Bg<KS>;
  const uint8_t* ps = g.p + rs * g.ldp;
  const uint32_t ldp = (uint32_t)g.ldp;
#pragma unroll
  for (int q = 0; q < B::LP; ++q)
    dma16(ps, (uint32_t)min(d.pr[q], rlim) * ldp + d.pc[q], slot + (4 * q + wave) * 1024);
  if (QK) {
    const uint8_t* qs = qtile + rs * 2;
#pragma unroll
    for (int q = 0; q < B::LQ; ++q) dma16(qs, d.qc[q], slot + B::PB + (4 * q + wave) * 1024);
  } else {
    const uint8_t* qs = g.q + rs * g.ldq;
    const uint32_t ldq = (uint32_t)g.ldq;
#pragma unroll
    for (int q = 0; q < B::LQ; ++q)
      dma16(qs, (uint32_t)min(d.qr[q], rlim) * ldq + d.qc[q], slot + B::PB + (4 * q + wave) * 1024);
  }
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// One MFMA operand fragment (32 columns x 16 reduction values) of an MN-major
// stage: two transpose reads, 4 rows apart.
__device__ __forceinline__ bf16x8_t tr_frag(uint32_t addr, int rp) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)addr);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(addr + 4 * rp));
  const i16x4_t v0 = lo, v1 = hi;
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Zero the values of a fragment whose reduction index (kbase + e) >= rem.
__device__ __forceinline__ bf16x8_t mask_tail(bf16x8_t f, int kbase, int rem) {
  u32x4_t u = __builtin_bit_cast(u32x4_t, f);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = kbase + 2 * w < rem ? 0x0000FFFFu : 0u;
    const uint32_t hi = kbase + 2 * w + 1 < rem ? 0xFFFF0000u : 0u;
    u[w] &= lo | hi;
  }
  return __builtin_bit_cast(bf16x8_t, u);
}

// Lane-constant parts of the fragment addresses (bytes from the stage base).
struct BgFrag {
  uint32_t p[BG_BI];  // P block ib, row group of this lane, swizzled segment
  uint32_t q[BG_BJ];  // Q block jb
};

template <bool QK, int KS>
__device__ __forceinline__ BgFrag bg_frag(int wi, int wj, int lane) {
  using B = Bg<KS>;
  BgFrag f;
  const int g = lane >> 4, s = lane & 15;
  const int rsub = 8 * (g >> 1) + (s >> 2);         // row inside a 16-row step
  const int cin = 32 * (g & 1) + 8 * (s & 3);        // byte inside the 64-byte segment
#pragma unroll
  for (int ib = 0; ib < BG_BI; ++ib)
    f.p[ib] = rsub * BG_RPP + (((BG_BI * wi + ib) ^ mn_swz<BG_RPP>(rsub)) << 6) + cin;
#pragma unroll
  for (int jb = 0; jb < BG_BJ; ++jb) {
    if (QK) {
      const int row = 64 * wj + 32 * jb + (lane & 31);
      f.q[jb] = B::PB + row * B::QROWB;  // chunk added per step
    } else {
      f.q[jb] = B::PB + rsub * BG_RPQ + (((BG_BJ * wj + jb) ^ mn_swz<BG_RPQ>(rsub)) << 6) + cin;
    }
  }
  return f;
}

template <bool QK, int KS, bool TAIL>
__device__ __forceinline__ void bg_mma(f32x16_t (&acc)[BG_BI][BG_BJ], uint32_t cur, const BgFrag& f, int lane,
                                       int rem) {
  using B = Bg<KS>;
  const int half = lane >> 5;
  bf16x8_t a[B::NJS][BG_BI], b[B::NJS][BG_BJ];
#pragma unroll
  for (int js = 0; js < B::NJS; ++js) {
#pragma unroll
    for (int ib = 0; ib < BG_BI; ++ib) a[js][ib] = tr_frag(cur + f.p[ib] + 16 * js * BG_RPP, BG_RPP);
#pragma unroll
    for (int jb = 0; jb < BG_BJ; ++jb) {
      if (QK) {
        // fragment rows 64 wj + 32 jb + lane%32: the swizzle key is lane%32's
        const int c = (2 * js + half) ^ k_swz<B::QROWB>(lane & 31);
        b[js][jb] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
            (uintptr_t)(cur + f.q[jb] + (c << 4)));
      } else {
        b[js][jb] = tr_frag(cur + f.q[jb] + 16 * js * BG_RPQ, BG_RPQ);
      }
    }
  }
  // keep every fragment read of the stage ahead of its MFMAs: the later k16
  // steps' reads then complete under the first step's MFMAs (the default
  // schedule interleaves each read right before its use)
  __builtin_amdgcn_sched_barrier(0);
  if (TAIL) {
#pragma unroll
    for (int js = 0; js < B::NJS; ++js) {
      const int kb = 16 * js + 8 * half;
#pragma unroll
      for (int ib = 0; ib < BG_BI; ++ib) a[js][ib] = mask_tail(a[js][ib], kb, rem);
      if (!QK) {
#pragma unroll
        for (int jb = 0; jb < BG_BJ; ++jb) b[js][jb] = mask_tail(b[js][jb], kb, rem);
      }
    }
  }
#pragma unroll
  for (int js = 0; js < B::NJS; ++js)
#pragma unroll
    for (int jb = 0; jb < BG_BJ; ++jb)
#pragma unroll
      for (int ib = 0; ib < BG_BI; ++ib)
        acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[js][ib], b[js][jb], acc[ib][jb], 0, 0, 0);
}

// acc[ib][jb] lane l, register r: i = i0 + 96 wi + 32 ib + 8 (r/4) + 4 (l/32) + r%4,
// j = j0 + 64 wj + 32 jb + l%32. fp32: 4 consecutive i per lane (16 bytes).
// bf16: lanes l and l^32 trade one 4-value group (v_permlane32_swap) so each
// lane stores 8 consecutive i (16 bytes) and each row j receives 32
// contiguous bytes per store instruction.
template <bool F32>
__device__ __forceinline__ void bg_store(const BGemm& g, const f32x16_t (&acc)[BG_BI][BG_BJ], int z, int i0,
                                         int j0, int wi, int wj, int lane) {
  const int half = lane >> 5;
  const int64_t zoff = (int64_t)z * g.J * g.I;
#pragma unroll
  for (int jb = 0; jb < BG_BJ; ++jb) {
    const int j = j0 + 64 * wj + 32 * jb + (lane & 31);
    const bool jok = j < g.J;
#pragma unroll
    for (int ib = 0; ib < BG_BI; ++ib) {
      const int ib0 = i0 + 32 * (BG_BI * wi + ib);
      const f32x16_t& A = acc[ib][jb];
      if (F32) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int i = ib0 + 8 * grp + 4 * half;
          if (jok && i < g.I)
            *reinterpret_cast<float4*>(static_cast<float*>(g.out) + zoff + (int64_t)j * g.I + i) =
                make_float4(A[4 * grp], A[4 * grp + 1], A[4 * grp + 2], A[4 * grp + 3]);
        }
      } else {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          // groups 2pp (i = 16pp + 4half + 0..3) and 2pp+1 (i = 16pp + 8 + 4half + 0..3)
          const uint32_t a0 = pack_bf16x2(A[8 * pp + 0], A[8 * pp + 1]);
          const uint32_t a1 = pack_bf16x2(A[8 * pp + 2], A[8 * pp + 3]);
          const uint32_t b0 = pack_bf16x2(A[8 * pp + 4], A[8 * pp + 5]);
          const uint32_t b1 = pack_bf16x2(A[8 * pp + 6], A[8 * pp + 7]);
          // lower lane: own a, partner's a; upper lane: partner's b, own b
          const u32x2_t s0 = swap_halves(a0, b0), s1 = swap_halves(a1, b1);
          const u32x4_t o = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
          const int i = ib0 + 16 * pp + 8 * half;
          if (jok && i < g.I)
            *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(g.out) + zoff + (int64_t)j * g.I + i) = o;
        }
      }
    }
  }
}

template <bool QK, int KS, bool F32>
__global__ __launch_bounds__(BG_THREADS) __attribute__((amdgpu_waves_per_eu(BG_WG_PER_CU, BG_WG_PER_CU)))
void bgemm_kernel(BGemm g) {
  using B = Bg<KS>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[B::STAGES * B::SB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  const uint32_t ring = lds_u32(lds);

  BgGrid gr;
  gr.ti = (g.I + BG_TI - 1) / BG_TI;
  gr.tj = (g.J + BG_TJ - 1) / BG_TJ;
  gr.per = gr.ti * gr.tj;
  gr.total = gr.per * g.splits;
  const BgFrag fr = bg_frag<QK, KS>(wi, wj, lane);

  int u = blockIdx.x;
  if (u >= gr.total) return;
  int z, ti, tj;
  bg_coords(gr, u, z, ti, tj);
  int i0 = ti * BG_TI, j0 = tj * BG_TJ;
  int64_t r0 = (int64_t)z * g.sps * KS;
  int64_t r1 = min(g.R, r0 + (int64_t)g.sps * KS);
  int nk = (int)((r1 - r0 + KS - 1) / KS);
  BgDma<KS> dp = bg_dma<QK, KS>(g, i0, j0, wave, lane);
  const uint8_t* qt = g.q + (int64_t)j0 * g.ldq;  // K-major Q: the tile's first row

  // stage kt of the current tile (clamped to the last one) into slot s
  auto issue = [&](int kt, int slot_kt) {
    const int k = kt < nk ? kt : nk - 1;
    const int64_t rs = r0 + (int64_t)k * KS;
    const int rlim = (int)min((int64_t)(KS - 1), r1 - 1 - rs);
    bg_issue<QK, KS>(g, dp, qt, rs, rlim, ring + (uint32_t)(slot_kt % B::STAGES) * B::SB, wave);
  };

#pragma unroll
  for (int s = 0; s < B::STAGES - 1; ++s) issue(s, s);

  for (;;) {
    f32x16_t acc[BG_BI][BG_BJ];
#pragma unroll
    for (int a = 0; a < BG_BI; ++a)
#pragma unroll
      for (int b = 0; b < BG_BJ; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int rem = (int)(r1 - r0 - (int64_t)(nk - 1) * KS);  // rows of the last stage
    const int nfull = rem == KS ? nk : nk - 1;
    // Full stages in a loop with one code path (a second MFMA path inside the
    // loop makes the compiler copy every accumulator at the merge).
    for (int kt = 0; kt < nfull; ++kt) {
      vm_wait<(B::STAGES - 2) * B::LPS>();
      barrier();
      // slot (kt + STAGES - 1) % STAGES was read in iteration kt - 1, and every
      // wave has passed the barrier since
      issue(kt + B::STAGES - 1, kt + B::STAGES - 1);
      bg_mma<QK, KS, false>(acc, ring + (uint32_t)(kt % B::STAGES) * B::SB, fr, lane, KS);
    }
    if (nfull < nk) {
      // partial last stage: no further stage to issue (the wait below drains all)
      vm_wait<(B::STAGES - 2) * B::LPS>();
      barrier();
      bg_mma<QK, KS, true>(acc, ring + (uint32_t)(nfull % B::STAGES) * B::SB, fr, lane, rem);
    }

    // drain this tile's DMA (including the clamped stages issued past its
    // end) and let every wave finish reading the ring; store the tile, then
    // start the next one
    vm_wait<0>();
    barrier();
    bg_store<F32>(g, acc, z, i0, j0, wi, wj, lane);
    u += gridDim.x;
    if (u >= gr.total) break;
    bg_coords(gr, u, z, ti, tj);
    i0 = ti * BG_TI;
    j0 = tj * BG_TJ;
    r0 = (int64_t)z * g.sps * KS;
    r1 = min(g.R, r0 + (int64_t)g.sps * KS);
    nk = (int)((r1 - r0 + KS - 1) / KS);
    dp = bg_dma<QK, KS>(g, i0, j0, wave, lane);
    qt = g.q + (int64_t)j0 * g.ldq;
#pragma unroll
    for (int s = 0; s < B::STAGES - 1; ++s) issue(s, s);
  }
}

int bg_grid(const BGemm& g, int cus) {
  const int64_t tiles = (int64_t)((g.I + BG_TI - 1) / BG_TI) * ((g.J + BG_TJ - 1) / BG_TJ) * g.splits;
  int64_t n = (int64_t)(cus > 0 ? cus : 256) * BG_WG_PER_CU;
  n -= n % 8;
  if (n < 8) n = 8;
  return (int)(tiles < n ? tiles : n);
}

// Sum of the fp32 partials of the reduction splits, in split order, rounded
// once to the output type (bf16, or fp32 with F32OUT).
template <bool F32OUT>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int splits,
                                                          int64_t n4, void* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int z = 1; z < splits; ++z) {
      const float4 v = reinterpret_cast<const float4*>(part + (int64_t)z * n4 * 4)[i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if (F32OUT)
      reinterpret_cast<float4*>(out)[i] = s;
    else
      reinterpret_cast<uint2*>(out)[i] = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
  }
}

// n4 groups of four values; the grid is capped and strided.
hipError_t launch_split_reduce(const float* part, int splits, int64_t n4, void* out, bool f32out,
                               hipStream_t stream) {
  const dim3 grid((unsigned)std::min<int64_t>((n4 + 255) / 256, (int64_t)1 << 20));
  if (f32out)
    hipLaunchKernelGGL(split_reduce_kernel<true>, grid, dim3(256), 0, stream, part, splits, n4, out);
  else
    hipLaunchKernelGGL(split_reduce_kernel<false>, grid, dim3(256), 0, stream, part, splits, n4, out);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

hipError_t zero_fill(void* p, size_t bytes, hipStream_t s) {
  // every caller passes a whole number of 4-byte words (N is a multiple of 32)
  if (!p || bytes == 0) return hipSuccess;
  const int64_t words = (int64_t)(bytes / 4);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<int64_t>((words + 255) / 256, 4096)), dim3(256), 0,
                     s, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qup_bwd(const BwdParams& p, const BwdPlan& pl, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(p.workspace);
  if (p.T == 0) {
    hipError_t e = zero_fill(p.dw, (size_t)p.N * p.K * (p.dw_fp32 ? 4 : 2), stream);
    if (e != hipSuccess) return e;
    return p.use_bias ? zero_fill(p.db, (size_t)p.N * 2, stream) : hipSuccess;
  }
  float* db_part = p.use_bias ? reinterpret_cast<float*>(ws + pl.db_off) : nullptr;
  {
    dim3 grid((p.N + IR_COLS - 1) / IR_COLS, (unsigned)std::min(pl.db_row_chunks, 65535));
    hipLaunchKernelGGL(inv_rope_kernel, grid, dim3(IR_THREADS), 0, stream, p, pl.ir_rows,
                       (int64_t)pl.db_row_chunks, db_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.use_bias) {
    hipError_t e = launch_db_reduce(db_part, pl.db_row_chunks, p.N, p.db, stream);
    if (e != hipSuccess) return e;
  }
  const int cus = device_cu_count();
  if (p.dx) {
    // dX[t][k] = sum_n W[n][k] dq_pre[t][n]; the reduction length N is a
    // multiple of 32, as a K-major Q requires
    BGemm g{};
    g.p = reinterpret_cast<const uint8_t*>(p.w);
    g.ldp = (int64_t)p.K * 2;
    g.q = reinterpret_cast<const uint8_t*>(p.dq_pre);
    g.ldq = (int64_t)p.N * 2;
    g.I = p.K;
    g.J = (int)p.T;
    g.R = p.N;
    const int ks = dx_stage_depth(p.N);
    const int stages = p.N / ks;
    g.splits = pl.dx_splits;
    g.sps = (stages + g.splits - 1) / g.splits;
    const bool split = g.splits > 1;
    g.out = split ? static_cast<void*>(ws + pl.dx_off) : static_cast<void*>(p.dx);
    const dim3 grid(bg_grid(g, cus));
    if (ks == 64) {
      if (split) hipLaunchKernelGGL((bgemm_kernel<true, 64, true>), grid, dim3(BG_THREADS), 0, stream, g);
      else hipLaunchKernelGGL((bgemm_kernel<true, 64, false>), grid, dim3(BG_THREADS), 0, stream, g);
    } else {
      if (split) hipLaunchKernelGGL((bgemm_kernel<true, 32, true>), grid, dim3(BG_THREADS), 0, stream, g);
      else hipLaunchKernelGGL((bgemm_kernel<true, 32, false>), grid, dim3(BG_THREADS), 0, stream, g);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (split) {
      e = launch_split_reduce(static_cast<const float*>(g.out), g.splits, p.T * p.K / 4, p.dx, false, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (p.dw) {
    // dW[n][k] = sum_t X[t][k] dq_pre[t][n]
    BGemm g{};
    g.p = reinterpret_cast<const uint8_t*>(p.x);
    g.ldp = (int64_t)p.K * 2;
    g.q = reinterpret_cast<const uint8_t*>(p.dq_pre);
    g.ldq = (int64_t)p.N * 2;
    g.I = p.K;
    g.J = p.N;
    g.R = p.T;
    const int stages = (int)((p.T + 63) / 64);
    g.splits = pl.dw_splits;
    g.sps = (stages + g.splits - 1) / g.splits;
    // split: fp32 partials [splits][N][K] in the workspace, summed below
    const bool split = g.splits > 1;
    g.out = split ? static_cast<void*>(ws + pl.dw_off) : p.dw;
    if (split || p.dw_fp32)
      hipLaunchKernelGGL((bgemm_kernel<false, 64, true>), dim3(bg_grid(g, cus)), dim3(BG_THREADS), 0, stream, g);
    else
      hipLaunchKernelGGL((bgemm_kernel<false, 64, false>), dim3(bg_grid(g, cus)), dim3(BG_THREADS), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (split) {
      e = launch_split_reduce(static_cast<const float*>(g.out), g.splits, (int64_t)p.N * p.K / 4, p.dw,
                              p.dw_fp32 != 0, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// MXFP8 backward: each product's operands quantized along its reduction axis
// (the forward page's mxfp8 projection carried into the backward page's
// linear backward), then the forward kernel's MXFP8 main loop in its plain
// product form:
//   dX[t][k] = sum_n Qrow(dq_pre)[t][n] Qcol(W)[n][k]  ("tokens" t, "rows" k)
//   dW[n][k] = sum_t Qcol(dq_pre)[t][n] Qcol(X)[t][k]  ("tokens" n, "rows" k)
// Column-quantized operands are stored transposed (reduction axis
// contiguous), so both products read two K-major operands; the token axis is
// zero-padded to a multiple of 128 (one MXFP8 stage).
// ---------------------------------------------------------------------------
hipError_t launch_qup_bwd_mx(const BwdParams& p, const MxBwdPlan& pl, int fp8_mfma, hipStream_t stream) {
  if (p.T == 0) return launch_qup_bwd(p, pl.base, stream);  // zero dW and db
  uint8_t* ws = static_cast<uint8_t*>(p.workspace);
  const int64_t T = p.T;
  const int N = p.N, K = p.K;
  // one pass over dq: dq_pre, its quantizations along n (the dX operand) and
  // along t (the dW operand, transposed), and the db partials of 128-row
  // bands; the pass assumes whole 128-column tiles and bands
  if (N % MXB_COLS != 0 || pl.Tp % MXB_ROWS != 0 || pl.base.ir_rows != MXB_ROWS) return hipErrorInvalidValue;
  float* db_part = p.use_bias ? reinterpret_cast<float*>(ws + pl.base.db_off) : nullptr;
  const int col_tiles = N / MXB_COLS;
  hipLaunchKernelGGL(inv_rope_mx_kernel, dim3((unsigned)(pl.Tp / MXB_ROWS * col_tiles)), dim3(256), 0, stream, p,
                     pl.Tp, db_part, p.dx ? ws + pl.dq_rows : nullptr, p.dx ? ws + pl.dq_rows_sc : nullptr,
                     p.dw ? ws + pl.dq_t : nullptr, p.dw ? ws + pl.dq_t_sc : nullptr, col_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.use_bias) {
    if ((e = launch_db_reduce(db_part, pl.base.db_row_chunks, N, p.db, stream))) return e;
  }
  if (p.dx) {
    if ((e = launch_mxfp8_quantize_t(p.w, N, K, K, N, ws + pl.w_t, ws + pl.w_t_sc, stream))) return e;
    FwdParams g{};
    g.x = ws + pl.dq_rows;
    g.xs = ws + pl.dq_rows_sc;
    g.w = ws + pl.w_t;
    g.ws = ws + pl.w_t_sc;
    g.T = T;
    g.K = N;
    g.N = K;
    g.H = 1;
    g.D = K;
    g.d_nope = K;
    g.B = 1;
    g.S = (int)T;
    g.mx_fp8_mfma = fp8_mfma;
    g.k_splits = pl.dx_splits;
    const bool split = pl.dx_splits > 1;
    g.out_f32 = split;
    g.split_stride = (int64_t)T * K * 4;
    g.out = split ? static_cast<void*>(ws + pl.dx_part) : static_cast<void*>(p.dx);
    if ((e = launch_mx_gemm(g, stream))) return e;
    if (split) {
      if ((e = launch_split_reduce(reinterpret_cast<const float*>(ws + pl.dx_part), pl.dx_splits, T * K / 4, p.dx,
                                   false, stream)))
        return e;
    }
  }
  if (p.dw) {
    if ((e = launch_mxfp8_quantize_t(p.x, T, K, K, pl.Tp, ws + pl.x_t, ws + pl.x_t_sc, stream))) return e;
    FwdParams g{};
    g.x = ws + pl.dq_t;
    g.xs = ws + pl.dq_t_sc;
    g.w = ws + pl.x_t;
    g.ws = ws + pl.x_t_sc;
    g.T = N;
    g.K = (int)pl.Tp;
    g.N = K;
    g.H = 1;
    g.D = K;
    g.d_nope = K;
    g.B = 1;
    g.S = N;
    g.mx_fp8_mfma = fp8_mfma;
    g.k_splits = 1;
    g.out_f32 = p.dw_fp32;
    g.out = p.dw;
    if ((e = launch_mx_gemm(g, stream))) return e;
  }
  return hipSuccess;
}

}  // namespace mla
