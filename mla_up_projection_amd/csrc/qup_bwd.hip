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
//   db_reduce_kernel: db[n] = sum over chunks, in chunk order.
//   gemm_kernel     : C[m, n] = sum_r A(m, r) B(n, r) on bf16 MFMA; an
//                     operand whose reduction axis is strided in memory
//                     (W for dX; dq_pre and X for dW) is loaded as 8 x 8
//                     blocks and transposed in registers on its way into LDS.
//   dX = dq_pre W       : A = dq_pre (r contiguous), B(k, r) = W[r, k]
//   dW = dq_pre^T X     : A(n, t) = dq_pre[t, n], B(k, t) = X[t, k]
//   split_reduce_kernel: ordered sum of the dX reduction splits -> bf16.
// No floating-point atomics anywhere: results are run-to-run deterministic.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

// ---------------------------------------------------------------------------
// Inverse RoPE + db partials
// ---------------------------------------------------------------------------
constexpr int IR_THREADS = 128;
constexpr int IR_COLS = IR_THREADS * 8;  // columns per workgroup
constexpr int IR_ROWS = 64;              // token rows per workgroup

__global__ __launch_bounds__(IR_THREADS) void inv_rope_kernel(BwdParams p, float* __restrict__ db_part) {
  __shared__ int s_pos[IR_ROWS];
  const int64_t r0 = (int64_t)blockIdx.y * IR_ROWS;
  const int rows = (int)min((int64_t)IR_ROWS, p.T - r0);
  const TokenMap tm{p.fmt, p.B, p.S, p.cu, p.nseq};
  for (int i = threadIdx.x; i < rows; i += IR_THREADS) {
    int pos, b, s;
    token_coords(tm, r0 + i, pos, b, s);
    s_pos[i] = pos;
  }
  __syncthreads();
  const int n0 = blockIdx.x * IR_COLS + threadIdx.x * 8;
  if (n0 >= p.N) return;
  const uint16_t* __restrict__ dq = p.dq;
  uint16_t* __restrict__ dq_pre = p.dq_pre;
  const float* __restrict__ cos_t = p.cos;
  const float* __restrict__ sin_t = p.sin;
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
  float sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // Rows in batches of RB: all loads of a batch are issued before any store,
  // so RB 16-byte loads per lane are in flight at once.
  constexpr int RB = 8;
  for (int i0 = 0; i0 < rows; i0 += RB) {
    u32x4_t g[RB];
    float cs[RB][4], sn[RB][4];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int i = i0 + j < rows ? i0 + j : rows - 1;
      g[j] = *reinterpret_cast<const u32x4_t*>(dq + (r0 + i) * p.N + n0);
      if (any_rot) {
        const int pos = s_pos[i];
        const bool pos_ok = pos >= 0 && pos < p.rope_rows;
        const int64_t trow = (int64_t)(pos_ok ? pos : 0) * p.rope_pairs;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          cs[j][k] = rot[k] ? cos_t[trow + pi[k]] : 1.0f;
          sn[j][k] = rot[k] ? sin_t[trow + pi[k]] : 0.0f;
          if (!pos_ok) cs[j][k] = sn[j][k] = __builtin_nanf("");
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
        if (any_rot && rot[k]) {
          const float c = cs[j][k], s = sn[j][k];
          const float na = a * c + b * s;
          const float nb = b * c - a * s;
          a = na;
          b = nb;
        }
        sum[2 * k] += a;
        sum[2 * k + 1] += b;
        o[k] = pack_bf16x2(a, b);
      }
      *reinterpret_cast<u32x4_t*>(dq_pre + (r0 + i0 + j) * p.N + n0) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  }
  if (db_part) {
    float* dst = db_part + (int64_t)blockIdx.y * p.N + n0;
    reinterpret_cast<float4*>(dst)[0] = make_float4(sum[0], sum[1], sum[2], sum[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(sum[4], sum[5], sum[6], sum[7]);
  }
}

// db[n] = sum of the per-chunk partials, in chunk order: 8 lanes per column
// each add every 8th chunk, then the 8 partial sums are added in lane order.
constexpr int DBR_COLS = 32;
__global__ __launch_bounds__(256) void db_reduce_kernel(const float* __restrict__ part, int chunks,
                                                       int N, uint16_t* __restrict__ db) {
  __shared__ float red[8][DBR_COLS];
  const int c = threadIdx.x % DBR_COLS;
  const int g = threadIdx.x / DBR_COLS;
  const int n = blockIdx.x * DBR_COLS + c;
  float s = 0.0f;
  if (n < N)
    for (int k = g; k < chunks; k += 8) s += part[(int64_t)k * N + n];
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && n < N) {
    float t = red[0][c];
#pragma unroll
    for (int q = 1; q < 8; ++q) t += red[q][c];
    db[n] = (uint16_t)f32_to_bf16_bits(t);
  }
}

// ---------------------------------------------------------------------------
// Generic bf16 MFMA GEMM, C[m, n] = sum_r A(m, r) * B(n, r).
// Tile 256 (m) x 128 (n) x 64 (r), 4 waves in 2 x 2, wave tile 128 x 64.
// MFMA rows are n, columns m (D = C^T block), so a lane owns 4 consecutive
// n of one m: 8-byte (bf16) or 16-byte (fp32) stores.
// ---------------------------------------------------------------------------
constexpr int G_BM = 256;
constexpr int G_BN = 128;
constexpr int G_ROW = 128;  // bytes per LDS row per stage (64 bf16 of r)
constexpr int G_THREADS = 256;
constexpr int G_A_STAGE = G_BM * G_ROW;
constexpr int G_STAGE = (G_BM + G_BN) * G_ROW;  // 49152
constexpr int G_LDS = 2 * G_STAGE;

__device__ __forceinline__ int g_off(int r, int c) { return r * G_ROW + ((c ^ (r & 7)) << 4); }

struct GemmArgs {
  const uint16_t* a;
  int64_t lda;  // element stride of A's slow axis
  const uint16_t* b;
  int64_t ldb;
  int M, Nc;
  int64_t R;
  int64_t r_per_split;
  void* c;      // [splits][M][Nc]
  int out_f32;
};

// Operand staging for one stage: rows x 64 of the reduction axis.
// K-major (reduction contiguous): rows*8 16-byte chunks, ROWS*8/256 per thread.
// MN-major (rows contiguous): (rows/8) x 8 blocks of 8x8, one per thread.
template <int ROWS, bool KMAJOR>
struct OperandStage {
  static constexpr int NCH = KMAJOR ? ROWS * 8 / G_THREADS : 8;
  u32x4_t v[NCH];
};

template <int ROWS, bool KMAJOR>
__device__ __forceinline__ void op_load(OperandStage<ROWS, KMAJOR>& st, const uint16_t* __restrict__ base,
                                        int64_t ld, int row0, int rows_valid, int64_t r0, int64_t r_end,
                                        int tid) {
  if (KMAJOR) {
    const int c = tid & 7;
    const int64_t r = r0 + c * 8;
#pragma unroll
    for (int i = 0; i < st.NCH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      if (row < rows_valid && r < r_end)
        st.v[i] = *reinterpret_cast<const u32x4_t*>(base + (int64_t)(row0 + row) * ld + r);
      else
        st.v[i] = u32x4_t{0, 0, 0, 0};
    }
  } else {
    constexpr int MBLK = ROWS / 8;
    const int mb = tid % MBLK;
    const int rb = tid / MBLK;
    const bool active = rb < 8;
    const int row = 8 * mb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t r = r0 + 8 * rb + j;
      if (active && row < rows_valid && r < r_end)
        st.v[j] = *reinterpret_cast<const u32x4_t*>(base + r * ld + row0 + row);
      else
        st.v[j] = u32x4_t{0, 0, 0, 0};
    }
  }
}

template <int ROWS, bool KMAJOR>
__device__ __forceinline__ void op_store(const OperandStage<ROWS, KMAJOR>& st, uint8_t* lds, int tid) {
  if (KMAJOR) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < st.NCH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4_t*>(lds + g_off(row, c)) = st.v[i];
    }
  } else {
    constexpr int MBLK = ROWS / 8;
    const int mb = tid % MBLK;
    const int rb = tid / MBLK;
    if (rb >= 8) return;
    // st.v[j] holds 8 values of rows 8mb..8mb+7 at reduction index 8rb+j;
    // out[i] gathers the 8 reduction values of row 8mb+i.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int w = i >> 1;
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = st.v[2 * q][w];
        const uint32_t hi = st.v[2 * q + 1][w];
        o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      *reinterpret_cast<u32x4_t*>(lds + g_off(8 * mb + i, rb)) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  }
}

template <bool A_KMAJOR, bool B_KMAJOR>
__global__ __launch_bounds__(G_THREADS) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[G_LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int half = lane >> 5;

  const int tiles_m = (g.M + G_BM - 1) / G_BM;
  const int tiles_n = (g.Nc + G_BN - 1) / G_BN;
  const int total = tiles_m * tiles_n;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  const int tm = id % tiles_m;
  const int tn = id / tiles_m;
  const int m0 = tm * G_BM;
  const int n0 = tn * G_BN;
  const int64_t r_begin = (int64_t)blockIdx.z * g.r_per_split;
  int64_t r_end = r_begin + g.r_per_split;
  if (r_end > g.R) r_end = g.R;
  const int nk = (int)((r_end - r_begin + 63) / 64);
  const int m_valid = g.M - m0;
  const int n_valid = g.Nc - n0;

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  OperandStage<G_BM, A_KMAJOR> sa;
  OperandStage<G_BN, B_KMAJOR> sb;
  const uint16_t* abase = g.a;
  op_load<G_BM, A_KMAJOR>(sa, abase, g.lda, m0, m_valid, r_begin, r_end, tid);
  op_load<G_BN, B_KMAJOR>(sb, g.b, g.ldb, n0, n_valid, r_begin, r_end, tid);
  op_store<G_BM, A_KMAJOR>(sa, lds, tid);
  op_store<G_BN, B_KMAJOR>(sb, lds + G_A_STAGE, tid);
  __syncthreads();

  const int arow0 = wm * 128 + (lane & 31);  // m rows (MFMA columns)
  const int brow0 = wn * 64 + (lane & 31);   // n rows (MFMA rows)
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t rn = r_begin + (int64_t)(kt + 1) * 64;
      op_load<G_BM, A_KMAJOR>(sa, abase, g.lda, m0, m_valid, rn, r_end, tid);
      op_load<G_BN, B_KMAJOR>(sb, g.b, g.ldb, n0, n_valid, rn, r_end, tid);
    }
    const uint8_t* cur = lds + (kt & 1) * G_STAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = 2 * j + half;
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8_t*>(cur + g_off(arow0 + 32 * mb, ch));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bfr[nb] = *reinterpret_cast<const bf16x8_t*>(cur + G_A_STAGE + g_off(brow0 + 32 * nb, ch));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[nb][mb], 0, 0, 0);
    }
    if (more) {
      uint8_t* nxt = lds + ((kt + 1) & 1) * G_STAGE;
      op_store<G_BM, A_KMAJOR>(sa, nxt, tid);
      op_store<G_BN, B_KMAJOR>(sb, nxt + G_A_STAGE, tid);
    }
    __syncthreads();
  }

  // acc[nb][mb] lane l, reg r: n = n0 + wn*64 + 32nb + 8(r/4) + 4half + r%4,
  // m = m0 + wm*128 + 32mb + lane%32.
  const int64_t split_off = (int64_t)blockIdx.z * g.M * g.Nc;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + 32 * mb + (lane & 31);
      if (m >= g.M) continue;
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int n = n0 + wn * 64 + 32 * nb + 8 * grp + 4 * half;
        if (n >= g.Nc) continue;
        const float v0 = acc[nb][mb][4 * grp + 0], v1 = acc[nb][mb][4 * grp + 1];
        const float v2 = acc[nb][mb][4 * grp + 2], v3 = acc[nb][mb][4 * grp + 3];
        const int64_t idx = split_off + (int64_t)m * g.Nc + n;
        if (g.out_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(g.c) + idx) = make_float4(v0, v1, v2, v3);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c) + idx) =
              make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        }
      }
    }
}

__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int splits,
                                                          int64_t n4, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 s = reinterpret_cast<const float4*>(part)[i];
  for (int z = 1; z < splits; ++z) {
    const float4 v = reinterpret_cast<const float4*>(part + (int64_t)z * n4 * 4)[i];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  reinterpret_cast<uint2*>(out)[i] = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
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

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

BwdPlan plan_bwd(int64_t T, int N, int K, bool use_bias, bool want_dx) {
  BwdPlan pl{};
  pl.db_row_chunks = (int)((T + IR_ROWS - 1) / IR_ROWS);
  pl.db_off = 0;
  pl.db_bytes = use_bias ? align256((size_t)pl.db_row_chunks * N * 4) : 0;
  pl.dx_splits = 1;
  if (want_dx && T > 0) {
    const int64_t tiles = ((T + G_BM - 1) / G_BM) * ((K + G_BN - 1) / G_BN);
    int64_t s = (640 + tiles - 1) / tiles;
    const int64_t max_by_len = N / 1024;
    if (s > max_by_len) s = max_by_len;
    if (s > 8) s = 8;
    if (s < 1) s = 1;
    pl.dx_splits = (int)s;
  }
  pl.dx_off = pl.db_bytes;
  pl.dx_bytes = pl.dx_splits > 1 ? align256((size_t)pl.dx_splits * T * K * 4) : 0;
  pl.total = pl.db_bytes + pl.dx_bytes;
  return pl;
}

hipError_t launch_qup_bwd(const BwdParams& p, const BwdPlan& pl, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(p.workspace);
  if (p.T == 0) {
    hipError_t e = zero_fill(p.dw, (size_t)p.N * p.K * (p.dw_fp32 ? 4 : 2), stream);
    if (e != hipSuccess) return e;
    return p.use_bias ? zero_fill(p.db, (size_t)p.N * 2, stream) : hipSuccess;
  }
  float* db_part = p.use_bias ? reinterpret_cast<float*>(ws + pl.db_off) : nullptr;
  {
    dim3 grid((p.N + IR_COLS - 1) / IR_COLS, pl.db_row_chunks);
    hipLaunchKernelGGL(inv_rope_kernel, grid, dim3(IR_THREADS), 0, stream, p, db_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.use_bias) {
    hipLaunchKernelGGL(db_reduce_kernel, dim3((p.N + DBR_COLS - 1) / DBR_COLS), dim3(256), 0, stream, db_part,
                       pl.db_row_chunks, p.N, p.db);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.dx) {
    GemmArgs g{};
    g.a = p.dq_pre;
    g.lda = p.N;
    g.b = p.w;
    g.ldb = p.K;
    g.M = (int)p.T;
    g.Nc = p.K;
    g.R = p.N;
    const int64_t per = (((int64_t)p.N + pl.dx_splits - 1) / pl.dx_splits + 63) / 64 * 64;
    g.r_per_split = per;
    const bool split = pl.dx_splits > 1;
    g.c = split ? static_cast<void*>(ws + pl.dx_off) : static_cast<void*>(p.dx);
    g.out_f32 = split ? 1 : 0;
    const int tiles = ((g.M + G_BM - 1) / G_BM) * ((g.Nc + G_BN - 1) / G_BN);
    hipLaunchKernelGGL((gemm_kernel<true, false>), dim3(tiles, 1, pl.dx_splits), dim3(G_THREADS), 0,
                       stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (split) {
      const int64_t n4 = p.T * p.K / 4;
      hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                         static_cast<const float*>(g.c), pl.dx_splits, n4, p.dx);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (p.dw) {
    GemmArgs g{};
    g.a = p.dq_pre;
    g.lda = p.N;
    g.b = p.x;
    g.ldb = p.K;
    g.M = p.N;
    g.Nc = p.K;
    g.R = p.T;
    g.r_per_split = p.T;
    g.c = p.dw;
    g.out_f32 = p.dw_fp32;
    const int tiles = ((g.M + G_BM - 1) / G_BM) * ((g.Nc + G_BN - 1) / G_BN);
    hipLaunchKernelGGL((gemm_kernel<false, false>), dim3(tiles, 1, 1), dim3(G_THREADS), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
