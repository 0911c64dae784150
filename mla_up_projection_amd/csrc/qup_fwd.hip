// Fused MLA query up-projection forward for gfx950:
//   Q^T tile = W_tile * X_tile^T on MFMA (bf16 32x32x16, or the scaled FP8
//   32x32x64 for MXFP8 operands), then a register-level epilogue: bias,
//   RoPE/YaRN rotation of each head's rope slice, per-32 amax, E8M0 scale,
//   E4M3 encode (or bf16), BHSD store with scales laid out like the data.
// Pages: "Add support for fused Q Up-Proj GEMM/RoPE/Quant." (description,
// flowchart: GEMM + RoPE + MXFP8 quantization in one kernel, 16-bit or MXFP8
// projection, BHSD scale transpose); "Fix fused MLA YaRN RoPE query kernel
// corrupting upstream tensor in-place" (the rotation is out of place: the
// accumulator is rotated in registers, no intermediate q exists).
//
// Tile: 192 rows of N (six 32-row blocks; a block never straddles a head
// because D is a multiple of 32) x 256 tokens, 4 waves in a 2 x 2 grid, each
// wave 96 rows x 128 tokens = 3 x 4 MFMA blocks. The MFMA row axis is N
// (W is the A operand), so in the 32x32 accumulator layout a lane holds
// runs of 4 consecutive head-dim elements of one token: RoPE pairs are
// lane-local and a 32-element scale block is split between lanes l and
// l^32 (one xor-shuffle for its amax).
#include <utility>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int TILE_N = 192;
constexpr int TILE_T = 256;
constexpr int ROW_BYTES = 128;            // bytes of one tile row per LDS stage
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr int WBLK_N = 3;                 // 32-row blocks per wave
constexpr int WBLK_T = 4;                 // 32-token blocks per wave
constexpr int X_STAGE = TILE_T * ROW_BYTES;
constexpr int W_STAGE = TILE_N * ROW_BYTES;
constexpr int STAGE = X_STAGE + W_STAGE;  // 57344 bytes
constexpr int LDS_BYTES = 2 * STAGE;      // double buffered
constexpr int X_CHUNKS = TILE_T * 8 / NTHREADS;   // 16-byte chunks per thread
constexpr int W_CHUNKS = TILE_N * 8 / NTHREADS;

// LDS address of 16-byte chunk c of row r: chunks are xor-swizzled with the
// row's low 3 bits so that 8 lanes reading one chunk column of 8 rows hit
// 8 distinct bank groups.
__device__ __forceinline__ int lds_off(int r, int c) { return r * ROW_BYTES + ((c ^ (r & 7)) << 4); }

// Grid position -> (token tile, n tile). Workgroups are dispatched round
// robin over the 8 XCDs; consecutive ids on one XCD are given the same
// W tile and successive token tiles so they share the W rows in that XCD's
// L2 while walking X.
__device__ __forceinline__ void tile_of(int g, int tiles_t, int tiles_n, int& tt, int& tn) {
  const int total = tiles_t * tiles_n;
  int id = g;
  if ((total & 7) == 0) id = (g & 7) * (total >> 3) + (g >> 3);
  tt = id % tiles_t;
  tn = id / tiles_t;
}

struct Staging {
  u32x4_t x[X_CHUNKS];
  u32x4_t w[W_CHUNKS];
};

// Global -> registers for one LDS stage: 128 bytes of every tile row,
// starting at byte column kb0 of X and W rows (row pitch row_bytes).
__device__ __forceinline__ void load_stage(Staging& st, const uint8_t* __restrict__ xb,
                                           const uint8_t* __restrict__ wb, int64_t t0, int n0,
                                           int64_t T, int N, int64_t row_bytes, int64_t kb0,
                                           int tid) {
  const int c = tid & 7;
  const bool kin = kb0 + c * 16 < row_bytes;
#pragma unroll
  for (int i = 0; i < X_CHUNKS; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int64_t t = t0 + r;
    if (kin && t < T)
      st.x[i] = *reinterpret_cast<const u32x4_t*>(xb + t * row_bytes + kb0 + c * 16);
    else
      st.x[i] = u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < W_CHUNKS; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int n = n0 + r;
    if (kin && n < N)
      st.w[i] = *reinterpret_cast<const u32x4_t*>(wb + (int64_t)n * row_bytes + kb0 + c * 16);
    else
      st.w[i] = u32x4_t{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void store_stage(const Staging& st, uint8_t* lds, int tid) {
  const int c = tid & 7;
#pragma unroll
  for (int i = 0; i < X_CHUNKS; ++i) {
    const int r = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4_t*>(lds + lds_off(r, c)) = st.x[i];
  }
#pragma unroll
  for (int i = 0; i < W_CHUNKS; ++i) {
    const int r = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4_t*>(lds + X_STAGE + lds_off(r, c)) = st.w[i];
  }
}

// ---------------------------------------------------------------------------
// Fused epilogue for one 32 (n) x 32 (token) accumulator block.
// acc[r] holds row 8*(r/4) + 4*(lane/32) + r%4 of the block, token lane%32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void epilogue_block(const FwdParams& p, const TokenMap& tm,
                                               const f32x16_t& acc, int n_blk, int64_t t,
                                               int lane) {
  const int half = lane >> 5;
  const bool tok_ok = t < p.T;
  const int h = n_blk / p.D;
  const int d_blk = n_blk - h * p.D;
  int pos = 0, b = 0, s = 0;
  if (tok_ok) token_coords(tm, t, pos, b, s);

  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = acc[r];

  if (p.bias) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = n_blk + 8 * (r >> 2) + 4 * half + (r & 3);
      v[r] += bf16_bits_to_f32(p.bias[n]);
    }
  }
  if (d_blk + 32 > p.d_nope && p.d_rope > 0) {
    const bool pos_ok = tok_ok && pos >= 0 && pos < p.rope_rows;
    const int64_t trow = (int64_t)(pos_ok ? pos : 0) * p.rope_pairs;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int d = d_blk + 8 * (r >> 2) + 4 * half + (r & 3);
      if (d >= p.d_nope) {
        const int i = (d - p.d_nope) >> 1;
        float c = p.cos[trow + i];
        float sn = p.sin[trow + i];
        if (!pos_ok) c = sn = __builtin_nanf("");
        const float a = v[r], bb = v[r + 1];
        v[r] = a * c - bb * sn;
        v[r + 1] = a * sn + bb * c;
      }
    }
  }

  const int64_t row = ((int64_t)b * p.H + h) * p.S + s;  // BHSD (b, h, s)
  if (p.out_mx) {
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = max(m, abs_bits(v[r]));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    uint32_t P[4];
    uint32_t sc;
    if (m >= 0x7F800000u) {
      P[0] = P[1] = P[2] = P[3] = 0x7F7F7F7Fu;
      sc = 0xFF;
    } else {
      const int E = mx_block_exp(m);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        P[g] = e4m3_encode(v[4 * g + 0], E) | (e4m3_encode(v[4 * g + 1], E) << 8) |
               (e4m3_encode(v[4 * g + 2], E) << 16) | (e4m3_encode(v[4 * g + 3], E) << 24);
      }
      sc = (uint32_t)(E + 127);
    }
    // Lanes l and l+32 swap two 4-row groups so each ends up with 16
    // consecutive rows: lower lane rows 0..15, upper lane rows 16..31.
    const uint32_t s0 = half ? P[0] : P[2];
    const uint32_t s1 = half ? P[1] : P[3];
    const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32);
    const uint32_t r1 = (uint32_t)__shfl_xor((int)s1, 32);
    u32x4_t o = half ? u32x4_t{r0, P[2], r1, P[3]} : u32x4_t{P[0], r0, P[1], r1};
    if (tok_ok) {
      uint8_t* dst = static_cast<uint8_t*>(p.out) + row * p.D + d_blk + 16 * half;
      *reinterpret_cast<u32x4_t*>(dst) = o;
      if (half == 0) p.out_scales[row * (p.D / 32) + d_blk / 32] = (uint8_t)sc;
    }
  } else {
    uint32_t P[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      P[2 * g] = pack_bf16x2(v[4 * g + 0], v[4 * g + 1]);
      P[2 * g + 1] = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
    }
    uint32_t snd[4], rcv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) snd[k] = half ? P[k] : P[4 + k];
#pragma unroll
    for (int k = 0; k < 4; ++k) rcv[k] = (uint32_t)__shfl_xor((int)snd[k], 32);
    u32x4_t o0, o1;
    if (half) {
      o0 = u32x4_t{rcv[0], rcv[1], P[4], P[5]};
      o1 = u32x4_t{rcv[2], rcv[3], P[6], P[7]};
    } else {
      o0 = u32x4_t{P[0], P[1], rcv[0], rcv[1]};
      o1 = u32x4_t{P[2], P[3], rcv[2], rcv[3]};
    }
    if (tok_ok) {
      uint16_t* dst = static_cast<uint16_t*>(p.out) + row * p.D + d_blk + 16 * half;
      reinterpret_cast<u32x4_t*>(dst)[0] = o0;
      reinterpret_cast<u32x4_t*>(dst)[1] = o1;
    }
  }
}

// The epilogue body is too large for the loop unroller, and a runtime index
// into the accumulator array would place it in scratch memory; a fold over a
// compile-time index sequence keeps every accumulator access constant.
template <int I>
__device__ __forceinline__ void epilogue_one(const FwdParams& p, const TokenMap& tm,
                                             const f32x16_t (&acc)[WBLK_N][WBLK_T], int n_wave,
                                             int64_t t_lane, int lane) {
  constexpr int nb = I / WBLK_T;
  constexpr int tb = I % WBLK_T;
  const int n_blk = n_wave + 32 * nb;
  if (n_blk < p.N) epilogue_block(p, tm, acc[nb][tb], n_blk, t_lane + 32 * tb, lane);
}

template <int... Is>
__device__ __forceinline__ void epilogue_all(const FwdParams& p, const TokenMap& tm,
                                             const f32x16_t (&acc)[WBLK_N][WBLK_T], int n_wave,
                                             int64_t t_lane, int lane, std::integer_sequence<int, Is...>) {
  (epilogue_one<Is>(p, tm, acc, n_wave, t_lane, lane), ...);
}

enum { MODE_BF16 = 0, MODE_MX_EXACT = 1, MODE_MX_FP8 = 2 };

// MXFP8 operands, exact mode: per LDS stage of 64 K-values, each thread
// loads 16-byte runs of E4M3 codes (16 K-values of one row, inside one
// 32-block), converts them to bf16 with the block's E8M0 scale folded in
// (v_cvt_scalef32_pk_bf16_fp8: code * 2^(scale-127), exact whenever the
// result is a bf16 normal), and stores two bf16 chunks, so the stage has the
// layout of the bf16 path. E4M3 values have 4 significant bits, so products
// of two are exact in fp32 and the bf16 MFMA accumulates them in fp32.
constexpr int MXE_X = TILE_T * 4 / NTHREADS;  // 16-byte code runs per thread
constexpr int MXE_W = TILE_N * 4 / NTHREADS;

struct MxStaging {
  u32x4_t x[MXE_X];
  u32x4_t w[MXE_W];
  uint32_t xs[MXE_X];
  uint32_t ws[MXE_W];
};

__device__ __forceinline__ void load_stage_mx(MxStaging& st, const FwdParams& p, int64_t t0, int n0,
                                              int kt, int tid) {
  const int c16 = tid & 3;
  const int kb = 64 * kt + 16 * c16;  // first K index of this run
  const int kblocks = p.K / 32;
  const uint8_t* xb = static_cast<const uint8_t*>(p.x);
  const uint8_t* wb = static_cast<const uint8_t*>(p.w);
#pragma unroll
  for (int i = 0; i < MXE_X; ++i) {
    const int r = (tid >> 2) + 64 * i;
    const int64_t t = t0 + r;
    if (t < p.T) {
      st.x[i] = *reinterpret_cast<const u32x4_t*>(xb + t * p.K + kb);
      st.xs[i] = p.xs[t * kblocks + (kb >> 5)];
    } else {
      st.x[i] = u32x4_t{0, 0, 0, 0};
      st.xs[i] = 127;
    }
  }
#pragma unroll
  for (int i = 0; i < MXE_W; ++i) {
    const int r = (tid >> 2) + 64 * i;
    const int n = n0 + r;
    if (n < p.N) {
      st.w[i] = *reinterpret_cast<const u32x4_t*>(wb + (int64_t)n * p.K + kb);
      st.ws[i] = p.ws[(int64_t)n * kblocks + (kb >> 5)];
    } else {
      st.w[i] = u32x4_t{0, 0, 0, 0};
      st.ws[i] = 127;
    }
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t codes, float scale) {
  const bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, HI);
  return __builtin_bit_cast(uint32_t, v);
}

// 2^(e8m0 - 127) as a float (byte 0 gives the float32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

__device__ __forceinline__ void store_run(uint8_t* lds, int r, int c16, const u32x4_t& v, uint32_t sbyte) {
  const float sc = e8m0_to_f32(sbyte);
  const u32x4_t lo = u32x4_t{cvt2<false>(v[0], sc), cvt2<true>(v[0], sc), cvt2<false>(v[1], sc),
                             cvt2<true>(v[1], sc)};
  const u32x4_t hi = u32x4_t{cvt2<false>(v[2], sc), cvt2<true>(v[2], sc), cvt2<false>(v[3], sc),
                             cvt2<true>(v[3], sc)};
  *reinterpret_cast<u32x4_t*>(lds + lds_off(r, 2 * c16)) = lo;
  *reinterpret_cast<u32x4_t*>(lds + lds_off(r, 2 * c16 + 1)) = hi;
}

__device__ __forceinline__ void store_stage_mx(const MxStaging& st, uint8_t* lds, int tid) {
  const int c16 = tid & 3;
#pragma unroll
  for (int i = 0; i < MXE_X; ++i) store_run(lds, (tid >> 2) + 64 * i, c16, st.x[i], st.xs[i]);
#pragma unroll
  for (int i = 0; i < MXE_W; ++i) store_run(lds + X_STAGE, (tid >> 2) + 64 * i, c16, st.w[i], st.ws[i]);
}

// bf16 MFMA over one LDS stage (64 K-values): 4 steps of k16.
__device__ __forceinline__ void mma_stage_bf16(f32x16_t (&acc)[WBLK_N][WBLK_T], const uint8_t* cur,
                                               int arow0, int brow0, int half) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = 2 * j + half;
    bf16x8_t a[WBLK_N], bv[WBLK_T];
#pragma unroll
    for (int nb = 0; nb < WBLK_N; ++nb)
      a[nb] = *reinterpret_cast<const bf16x8_t*>(cur + X_STAGE + lds_off(arow0 + 32 * nb, ch));
#pragma unroll
    for (int tb = 0; tb < WBLK_T; ++tb)
      bv[tb] = *reinterpret_cast<const bf16x8_t*>(cur + lds_off(brow0 + 32 * tb, ch));
#pragma unroll
    for (int nb = 0; nb < WBLK_N; ++nb)
#pragma unroll
      for (int tb = 0; tb < WBLK_T; ++tb)
        acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[nb], bv[tb], acc[nb][tb], 0, 0, 0);
  }
}

template <int MODE>
__device__ __forceinline__ void run_tile(const FwdParams& p, uint8_t* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1;  // which 96-row half of the N tile
  const int wt = wave & 1;   // which 128-token half of the token tile
  const int tiles_t = (int)((p.T + TILE_T - 1) / TILE_T);
  const int tiles_n = (p.N + TILE_N - 1) / TILE_N;
  int tt, tn;
  tile_of(blockIdx.x, tiles_t, tiles_n, tt, tn);
  const int64_t t0 = (int64_t)tt * TILE_T;
  const int n0 = tn * TILE_N;

  f32x16_t acc[WBLK_N][WBLK_T];
#pragma unroll
  for (int i = 0; i < WBLK_N; ++i)
#pragma unroll
    for (int j = 0; j < WBLK_T; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragment rows of this lane inside the tile.
  const int arow0 = wn * 96 + (lane & 31);   // + 32*nb
  const int brow0 = wt * 128 + (lane & 31);  // + 32*tb
  const int half = lane >> 5;

  if (MODE == MODE_MX_EXACT) {
    const int nk = p.K / 64;
    MxStaging st;
    load_stage_mx(st, p, t0, n0, 0, tid);
    store_stage_mx(st, lds, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load_stage_mx(st, p, t0, n0, kt + 1, tid);
      mma_stage_bf16(acc, lds + (kt & 1) * STAGE, arow0, brow0, half);
      if (more) store_stage_mx(st, lds + ((kt + 1) & 1) * STAGE, tid);
      __syncthreads();
    }
  } else {
    constexpr bool FP8 = MODE == MODE_MX_FP8;
    const int64_t row_bytes = FP8 ? (int64_t)p.K : (int64_t)p.K * 2;
    const int nk = (int)((row_bytes + ROW_BYTES - 1) / ROW_BYTES);
    const uint8_t* xb = static_cast<const uint8_t*>(p.x);
    const uint8_t* wb = static_cast<const uint8_t*>(p.w);

    // FP8 MFMA: E8M0 scales of this lane's rows for the current stage (4
    // blocks of 32 along K), pre-shifted so byte 0 / byte 2 serve MFMA step
    // 0 / 1 (lane half h supplies the scale of K-block h of each step).
    const int kblocks = p.K / 32;
    uint32_t xsc[WBLK_T], wsc[WBLK_N], xsc_n[WBLK_T], wsc_n[WBLK_N];
    auto load_scales = [&](int kt, uint32_t* xs_out, uint32_t* ws_out) {
#pragma unroll
      for (int tb = 0; tb < WBLK_T; ++tb) {
        const int64_t t = t0 + brow0 + 32 * tb;
        uint32_t v = 0;
        if (t < p.T) {
          const uint8_t* s = p.xs + t * kblocks + 4 * kt;
          v = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16) | ((uint32_t)s[3] << 24);
        }
        xs_out[tb] = v >> (8 * half);
      }
#pragma unroll
      for (int nb = 0; nb < WBLK_N; ++nb) {
        const int n = n0 + arow0 + 32 * nb;
        uint32_t v = 0;
        if (n < p.N) {
          const uint8_t* s = p.ws + (int64_t)n * kblocks + 4 * kt;
          v = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16) | ((uint32_t)s[3] << 24);
        }
        ws_out[nb] = v >> (8 * half);
      }
    };

    Staging st;
    load_stage(st, xb, wb, t0, n0, p.T, p.N, row_bytes, 0, tid);
    if (FP8) load_scales(0, xsc, wsc);
    store_stage(st, lds, tid);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) {
        load_stage(st, xb, wb, t0, n0, p.T, p.N, row_bytes, (int64_t)(kt + 1) * ROW_BYTES, tid);
        if (FP8) load_scales(kt + 1, xsc_n, wsc_n);
      }
      const uint8_t* cur = lds + (kt & 1) * STAGE;
      if (!FP8) {
        mma_stage_bf16(acc, cur, arow0, brow0, half);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // 2 steps of k64 per 128-byte stage
          // Scaled FP8 32x32x64 operand: lane (row, half) holds 16 bytes of
          // K-block 0 (k = 16*half .. +15) in its first four registers and 16
          // bytes of K-block 1 (k = 32 + 16*half .. +15) in the last four; the
          // E8M0 scale of (row, block b) is taken from lane row + 32*b.
          const int ch = 4 * j + half;
          i32x8_t a[WBLK_N], bv[WBLK_T];
#pragma unroll
          for (int nb = 0; nb < WBLK_N; ++nb) {
            const int r = arow0 + 32 * nb;
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(cur + X_STAGE + lds_off(r, ch));
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(cur + X_STAGE + lds_off(r, ch + 2));
            a[nb] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          }
#pragma unroll
          for (int tb = 0; tb < WBLK_T; ++tb) {
            const int r = brow0 + 32 * tb;
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(cur + lds_off(r, ch));
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(cur + lds_off(r, ch + 2));
            bv[tb] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          }
#pragma unroll
          for (int nb = 0; nb < WBLK_N; ++nb)
#pragma unroll
            for (int tb = 0; tb < WBLK_T; ++tb) {
              if (j == 0)
                acc[nb][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[nb], bv[tb], acc[nb][tb], 0, 0, 0, (int)wsc[nb], 0, (int)xsc[tb]);
              else
                acc[nb][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[nb], bv[tb], acc[nb][tb], 0, 0, 2, (int)wsc[nb], 2, (int)xsc[tb]);
            }
        }
      }
      if (more) {
        store_stage(st, lds + ((kt + 1) & 1) * STAGE, tid);
        if (FP8) {
#pragma unroll
          for (int tb = 0; tb < WBLK_T; ++tb) xsc[tb] = xsc_n[tb];
#pragma unroll
          for (int nb = 0; nb < WBLK_N; ++nb) wsc[nb] = wsc_n[nb];
        }
      }
      __syncthreads();
    }
  }

  const TokenMap tm{p.fmt, p.B, p.S, p.cu, p.nseq};
  epilogue_all(p, tm, acc, n0 + wn * 96, t0 + wt * 128 + (lane & 31), lane,
               std::make_integer_sequence<int, WBLK_N * WBLK_T>{});
}

template <int MODE>
__global__ __launch_bounds__(NTHREADS) void qup_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  run_tile<MODE>(p, lds);
}

int grid_of(const FwdParams& p) {
  const int64_t tiles_t = (p.T + TILE_T - 1) / TILE_T;
  const int64_t tiles_n = (p.N + TILE_N - 1) / TILE_N;
  return (int)(tiles_t * tiles_n);
}

}  // namespace

hipError_t launch_qup_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(qup_fwd_kernel<MODE_BF16>, dim3(grid_of(p)), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_qup_fwd_mx(const FwdParams& p, hipStream_t stream) {
  if (p.mx_fp8_mfma)
    hipLaunchKernelGGL(qup_fwd_kernel<MODE_MX_FP8>, dim3(grid_of(p)), dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(qup_fwd_kernel<MODE_MX_EXACT>, dim3(grid_of(p)), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
