// Fused MLA query up-projection forward for gfx950:
//   Q^T tile = W_tile * X_tile^T on MFMA, then a register-level epilogue:
//   bias, RoPE/YaRN rotation of each head's rope slice, per-32 amax, E8M0
//   scale, E4M3 encode (or bf16), BHSD store with scales laid out like the
//   data.
// Pages: "Add support for fused Q Up-Proj GEMM/RoPE/Quant." (description,
// flowchart: GEMM + RoPE + MXFP8 quantization in one kernel, 16-bit or MXFP8
// projection, BHSD scale transpose); "Fix fused MLA YaRN RoPE query kernel
// corrupting upstream tensor in-place" (the rotation is out of place: the
// accumulator is rotated in registers, no intermediate q exists).
//
// Work decomposition (two independent 256-thread workgroups per CU, persistent,
// so each SIMD runs one wave of each: one workgroup's barriers, LDS round trips
// and epilogue are covered by the other's MFMAs):
//   * tile = 128 tokens x 192 rows of N (one DeepSeek-V3 head); the 4 waves
//     form 2 x 2, each owning 64 tokens x 96 rows = 2 x 3 blocks of the
//     32x32 MFMA (96 fp32 accumulators per lane; 5 fragment reads per 6
//     MFMAs). The MFMA row axis is N (W is the A operand), so a lane holds
//     runs of 4 consecutive head-dim elements of one token: RoPE pairs are
//     lane-local and a 32-element scale block is split between lanes l and
//     l^32 (one xor-shuffle for its amax).
//   * K streams through an LDS ring of row slices (128 bytes per row and
//     stage in 2 slots; 64 bytes in 4 slots for bf16 with K % 64 == 32),
//     filled by direct global->LDS DMA (global_load_lds_dwordx4) issued
//     STAGES-1 stages ahead; each wave counts its own outstanding loads with
//     s_waitcnt vmcnt and one s_barrier per stage publishes the slot. The
//     only other vector-memory loads in the loop are the MXFP8 operand
//     scales, one dword per row for a pair of stages.
//   * After the last stage of a tile, the first stages of the workgroup's
//     next tile are put in flight before the epilogue runs.
//   * Tiles are ordered so that the 64 workgroups resident on one XCD share
//     W and X slices in that XCD's L2.
#include <utility>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int TILE_T = FWD_TILE_T;         // 128 tokens
constexpr int TILE_N = FWD_TILE_N;         // 192 rows of N: one DeepSeek-V3 head (D = 192)
constexpr int NTHREADS = 256;
constexpr int WBLK_N = 3;                 // 32-row blocks of N per wave (96 rows)
constexpr int WBLK_T = 2;                 // 32-token blocks per wave (64 tokens)
constexpr int WAVES_N = TILE_N / (32 * WBLK_N);  // waves along N (2); along T: 2
static_assert(WAVES_N * (TILE_T / (32 * WBLK_T)) == NTHREADS / 64, "2 x 2 waves");
static_assert(WBLK_N == 3, "packed scale stores below are written for 3 blocks per wave");
constexpr int WG_PER_CU = 2;              // two independent workgroups per CU
constexpr int ROPE_ROW_BYTES = 128;       // LDS-staged table rows: 32 fp32 pairs (d_rope = 64)
constexpr int ROPE_TAB_HALF = TILE_T * ROPE_ROW_BYTES;  // cos rows, then sin rows (32 KB in all)

// LDS-staged table rows: 16-byte chunk c of token row r sits at chunk
// position c ^ rope_swz(r), so the 32 rows one half-wave reads in the
// epilogue spread over the banks.
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

enum { MODE_BF16 = 0, MODE_MX_EXACT = 1, MODE_MX_FP8 = 2, MODE_BF16_R64 = 3 };
enum { EPI_MLA = 0, EPI_PLAIN = 1 };  // fused RoPE/quantize/BHSD epilogue, or a plain row-major store

// Stage layout per mode: a ring slot holds ROWB bytes of each of the tile's
// TILE_T X rows and TILE_N W rows. 128-byte row slices (whole cache lines per
// request: 64 bf16 or 128 E4M3 K-values) in a 2-slot ring, except BF16 with
// K % 64 == 32, which uses 64-byte slices in 4 slots. Every mode takes 80 KB
// of LDS; E4M3 operand scales travel in registers (see StageScales).
template <int MODE>
struct Tile {
  static constexpr bool MX = MODE == MODE_MX_EXACT || MODE == MODE_MX_FP8;
  static constexpr int ROWB = MODE == MODE_BF16_R64 ? 64 : 128;
  static constexpr int KPS = MX ? ROWB : ROWB / 2;  // K-values per stage
  static constexpr int STAGES = MODE == MODE_BF16_R64 ? 4 : 2;
  static constexpr int XSB = TILE_T * ROWB;         // X part of a slot
  static constexpr int WSB = TILE_N * ROWB;         // W part of a slot
  static constexpr int SB = XSB + WSB;
  static constexpr int LQX = XSB / 4096;            // X DMA loads (1 KB) per wave per stage
  static constexpr int LQW = WSB / 4096;
  static constexpr int LPS = LQX + LQW;
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int RPL = 1024 / ROWB;           // rows per 1 KB wave load
};

// Chunk swizzle: 16-byte chunk c of row r is stored at c ^ swz(r), so the 16
// lanes of one LDS pass of a fragment read (16 consecutive rows, one chunk)
// hit distinct bank groups: (r >> 2) & 3 for 64-byte rows (four chunks),
// (r >> 1) & 7 for 128-byte rows (eight chunks; odd rows sit in the other
// half of the banks).
template <int ROWB>
__device__ __forceinline__ int swz(int r) { return ROWB == 64 ? (r >> 2) & 3 : (r >> 1) & 7; }
template <int ROWB>
__device__ __forceinline__ int roff(int r, int c) { return r * ROWB + ((c ^ swz<ROWB>(r)) << 4); }


// ---------------------------------------------------------------------------
// Fused epilogue for one 32 (n) x 32 (token) accumulator block.
// acc[r] holds row 8*(r/4) + 4*(lane/32) + r%4 of the block, token lane%32.
// ---------------------------------------------------------------------------
// The tile's cos/sin rows staged in LDS (see stage_rope_rows): `on` is
// wave-uniform, `addr` the LDS byte address of the cos rows.
struct RopeTab {
  bool on;
  uint32_t addr;
};

struct TokInfo {
  bool ok;      // token row < T
  int pos;      // RoPE position
  int64_t row;  // BHSD row of head 0: (b*H)*S + s; head h adds h*S
};

// t: this lane's token, in the wave's run of 32 consecutive tokens starting at
// t - (lane & 31).
__device__ __forceinline__ TokInfo tok_info(const FwdParams& p, const TokenMap& tm, int64_t t, int lane) {
  TokInfo ti{t < p.T, 0, 0};
  if (ti.ok) {
    int b, s;
    const int base = (int)t - (lane & 31);
    token_coords_run(tm, t, base, base + 31, ti.pos, b, s);
    ti.row = (int64_t)b * p.H * p.S + s;
  }
  return ti;
}

// Rotation of the pair (a, b) by the angle with cosine c and sine s, as
// (a c - b s, a s + b c): each output is one rounded product and one fused
// multiply-add, written out so the rounding does not depend on how the
// compiler contracts the surrounding code.
__device__ __forceinline__ float rot_lo(float a, float b, float c, float s) { return __builtin_fmaf(a, c, -(b * s)); }
__device__ __forceinline__ float rot_hi(float a, float b, float c, float s) { return __builtin_fmaf(a, s, b * c); }

// One 32 (n) x 32 (token) block: bias, rotation, quantization, store.
// Returns the block's E8M0 scale byte (MXFP8 output), which the caller
// stores; `store_scale` makes this function store it itself instead. `tab`
// is the tile's cos/sin rows staged in LDS (see stage_rope_rows) or null, and
// `tok` this lane's token row inside the tile.
__device__ __forceinline__ uint32_t epilogue_block(const FwdParams& p, const TokInfo& ti, const f32x16_t& acc,
                                                   int n_blk, int lane, bool store_scale, RopeTab tab,
                                                   int tok) {
  const int half = lane >> 5;
  const int h = n_blk / p.D;
  const int d_blk = n_blk - h * p.D;

  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = acc[r];

  if (p.bias) {
    // rows 8g + 4 half + 0..3 of this lane: 4 consecutive bf16 (8 bytes, N % 32 == 0)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n_blk + 8 * g + 4 * half);
      v[4 * g] += bf16_bits_to_f32(bb.x & 0xFFFFu);
      v[4 * g + 1] += bf16_bits_to_f32(bb.x >> 16);
      v[4 * g + 2] += bf16_bits_to_f32(bb.y & 0xFFFFu);
      v[4 * g + 3] += bf16_bits_to_f32(bb.y >> 16);
    }
  }
  if (d_blk + 32 > p.d_nope && p.d_rope > 0) {
    const bool pos_ok = ti.ok && ti.pos >= 0 && ti.pos < p.rope_rows;
    const int64_t trow = (int64_t)(pos_ok ? ti.pos : 0) * p.rope_pairs;
    const float nan = __builtin_nanf("");
    // Rows 4g + {0,1} and 4g + {2,3} of this lane are table pairs i, i+1.
    if (d_blk >= p.d_nope && ((p.d_nope | p.rope_pairs) & 3) == 0) {
      // Whole block inside the rope slice (uniform branch): pair index
      // i = i0 + 4g with i0 even, so each group is one 8-byte cos and one
      // 8-byte sin load, all eight issued before any use.
      const int i0 = ((d_blk - p.d_nope) >> 1) + 2 * half;
      float2 cc[4], ss[4];
      if (tab.on) {
        // pair i0 + 4g is chunk i0 / 4 + g, bytes 8 half .. +7 of it; LDS
        // reads (ds_read_b64) by address, so they neither count against nor
        // wait for the vector-memory loads in flight (the next tile's DMA)
        const uint32_t row = tab.addr + (uint32_t)(tok * ROPE_ROW_BYTES + 8 * half);
        const int sw = rope_swz(tok);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t c = (uint32_t)(((i0 >> 2) + g) ^ sw);
          cc[g] = lds_read_f2(row + 16 * c);
          ss[g] = lds_read_f2(row + ROPE_TAB_HALF + 16 * c);
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          cc[g] = *reinterpret_cast<const float2*>(p.cos + trow + i0 + 4 * g);
          ss[g] = *reinterpret_cast<const float2*>(p.sin + trow + i0 + 4 * g);
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float c0 = pos_ok ? cc[g].x : nan, c1 = pos_ok ? cc[g].y : nan;
        const float s0 = pos_ok ? ss[g].x : nan, s1 = pos_ok ? ss[g].y : nan;
        const float a0 = v[4 * g], b0 = v[4 * g + 1], a1 = v[4 * g + 2], b1 = v[4 * g + 3];
        v[4 * g] = rot_lo(a0, b0, c0, s0);
        v[4 * g + 1] = rot_hi(a0, b0, c0, s0);
        v[4 * g + 2] = rot_lo(a1, b1, c1, s1);
        v[4 * g + 3] = rot_hi(a1, b1, c1, s1);
      }
    } else {
      // block straddling the nope/rope boundary, or unaligned table rows
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = d_blk + 8 * g + 4 * half;
        if (d >= p.d_nope) {
          const int i = (d - p.d_nope) >> 1;
          const float c0 = pos_ok ? p.cos[trow + i] : nan, c1 = pos_ok ? p.cos[trow + i + 1] : nan;
          const float s0 = pos_ok ? p.sin[trow + i] : nan, s1 = pos_ok ? p.sin[trow + i + 1] : nan;
          const float a0 = v[4 * g], b0 = v[4 * g + 1], a1 = v[4 * g + 2], b1 = v[4 * g + 3];
          v[4 * g] = rot_lo(a0, b0, c0, s0);
          v[4 * g + 1] = rot_hi(a0, b0, c0, s0);
          v[4 * g + 2] = rot_lo(a1, b1, c1, s1);
          v[4 * g + 3] = rot_hi(a1, b1, c1, s1);
        }
      }
    }
  }

  const int64_t row = ti.row + (int64_t)h * p.S;  // BHSD (b, h, s)
  uint32_t sc = 0;
  if (p.out_mx) {
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = max(m, abs_bits(v[r]));
    const u32x2_t mm = swap_halves(m, m);
    m = max(mm[0], mm[1]);  // amax over both halves of the block
    uint32_t P[4];
    if (m >= 0x7F800000u) {
      P[0] = P[1] = P[2] = P[3] = 0x7F7F7F7Fu;
      sc = 0xFF;
    } else {
      const int E = mx_block_exp(m);
#pragma unroll
      for (int g = 0; g < 4; ++g) P[g] = e4m3_pack4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], E);
      sc = (uint32_t)(E + 127);
    }
    // Lanes l and l+32 trade two 4-row groups so each ends up with 16
    // consecutive rows: lower lane rows 0..15, upper lane rows 16..31.
    const u32x2_t o01 = swap_halves(P[0], P[2]);
    const u32x2_t o23 = swap_halves(P[1], P[3]);
    if (ti.ok) {
      uint8_t* dst = static_cast<uint8_t*>(p.out) + row * p.D + d_blk + 16 * half;
      *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{o01[0], o01[1], o23[0], o23[1]};
      if (store_scale && half == 0) p.out_scales[row * (p.D / 32) + d_blk / 32] = (uint8_t)sc;
    }
  } else {
    uint32_t P[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      P[2 * g] = pack_bf16x2(v[4 * g + 0], v[4 * g + 1]);
      P[2 * g + 1] = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
    }
    // lower lane: rows 0..7 then 8..15; upper lane: rows 16..23 then 24..31
    u32x2_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = swap_halves(P[k], P[4 + k]);
    if (ti.ok) {
      uint16_t* dst = static_cast<uint16_t*>(p.out) + row * p.D + d_blk + 16 * half;
      reinterpret_cast<u32x4_t*>(dst)[0] = u32x4_t{r[0][0], r[1][0], r[0][1], r[1][1]};
      reinterpret_cast<u32x4_t*>(dst)[1] = u32x4_t{r[2][0], r[3][0], r[2][1], r[3][1]};
    }
  }
  return sc;
}

// The epilogue body is too large for the loop unroller, and a runtime index
// into the accumulator array would place it in scratch memory; folds over
// compile-time index sequences keep every accumulator access constant.
template <int TB, int NB>
__device__ __forceinline__ void epilogue_one(const FwdParams& p, const TokInfo& ti,
                                             const f32x16_t (&acc)[WBLK_N][WBLK_T], int n0, int lane,
                                             bool packed, uint32_t (&sc)[WBLK_N], RopeTab tab, int tok) {
  const int n_blk = n0 + 32 * NB;
  // one block at a time: interleaving blocks would hold several blocks'
  // temporaries live next to the accumulators
  __builtin_amdgcn_sched_barrier(0);
  sc[NB] = n_blk < p.N ? epilogue_block(p, ti, acc[NB][TB], n_blk, lane, !packed, tab, tok) : 0u;
}

template <int TB, int... NBs>
__device__ __forceinline__ void epilogue_tok(const FwdParams& p, const TokenMap& tm,
                                             const f32x16_t (&acc)[WBLK_N][WBLK_T], int n0, int64_t t_lane,
                                             int lane, RopeTab tab, int tok0,
                                             std::integer_sequence<int, NBs...>) {
  const TokInfo ti = tok_info(p, tm, t_lane + 32 * TB, lane);
  // When the tile is exactly one head, the head's D/32 scale bytes of this
  // token are contiguous: store them as 16-bit pairs, right after the token
  // row's codes, instead of one byte per block.
  const bool packed = p.out_mx && p.D == TILE_N;
  uint32_t sc[WBLK_N];
  (epilogue_one<TB, NBs>(p, ti, acc, n0, lane, packed, sc, tab, tok0 + 32 * TB), ...);
  if (packed && ti.ok && lane < 32) {
    // this wave's 3 scale bytes of the token's head: one 16-bit and one byte store
    const int64_t row = ti.row + (int64_t)(n0 / p.D) * p.S;
    uint8_t* dst = p.out_scales + row * (TILE_N / 32) + (n0 % p.D) / 32;
    if ((reinterpret_cast<uintptr_t>(dst) & 1) == 0) {
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(sc[0] | (sc[1] << 8));
      dst[2] = (uint8_t)sc[2];
    } else {
      dst[0] = (uint8_t)sc[0];
      *reinterpret_cast<uint16_t*>(dst + 1) = (uint16_t)(sc[1] | (sc[2] << 8));
    }
  }
}

template <int... TBs>
__device__ __forceinline__ void epilogue_all(const FwdParams& p, const TokenMap& tm,
                                             const f32x16_t (&acc)[WBLK_N][WBLK_T], int n0, int64_t t_lane,
                                             int lane, RopeTab tab, int tok0,
                                             std::integer_sequence<int, TBs...>) {
  (epilogue_tok<TBs>(p, tm, acc, n0, t_lane, lane, tab, tok0, std::make_integer_sequence<int, WBLK_N>{}), ...);
}

// t_lane: this lane's first token; tok0: its row inside the tile (for tab).
__device__ __forceinline__ void epilogue_tile(const FwdParams& p, const TokenMap& tm,
                                              const f32x16_t (&acc)[WBLK_N][WBLK_T], int n0, int64_t t_lane,
                                              int lane, RopeTab tab, int tok0) {
  epilogue_all(p, tm, acc, n0, t_lane, lane, tab, tok0, std::make_integer_sequence<int, WBLK_T>{});
}

// The tile's cos and sin table rows (d_rope = 64: the first 32 pairs of
// each row, 128 bytes) DMA'd into a free ring slot: [cos rows of the 128
// tokens][sin rows], row r at r * 128. Wave load j = 4q + wave fills rows
// 8j .. 8j + 7 of both tables; lane i writes row 8j + i / 8, chunk position
// i % 8. Positions outside the table (and rows past T) read row 0; the
// epilogue turns those tokens into NaN as it does for direct table loads.
__device__ __forceinline__ void stage_rope_rows(const FwdParams& p, const TokenMap& tm, int64_t t0,
                                                uint32_t dst, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 4 * q + wave;
    const int r = 8 * j + (lane >> 3);
    int64_t t = t0 + r;
    if (t >= p.T) t = p.T - 1;
    // the wave's run: rows 8j .. 8j + 7 (clamped like t)
    const int run0 = (int)min(t0 + 8 * j, p.T - 1), run1 = (int)min(t0 + 8 * j + 7, p.T - 1);
    int pos, b, s;
    token_coords_run(tm, t, run0, run1, pos, b, s);
    if (pos < 0 || pos >= p.rope_rows) pos = 0;
    const uint32_t off = (uint32_t)pos * (uint32_t)(p.rope_pairs * 4) + (uint32_t)(((lane & 7) ^ rope_swz(r)) * 16);
    dma16(p.cos, off, dst + j * 1024);
    dma16(p.sin, off, dst + ROPE_TAB_HALF + j * 1024);
  }
}

// ---------------------------------------------------------------------------
// Tile scheduling.
// ---------------------------------------------------------------------------
struct TileGrid {
  int tiles_t, tiles_n, total;
};

// Tile u -> (token tile, n tile). Workgroup g runs on XCD g % 8 and takes
// tiles g, g + G, g + 2G, ... (G a multiple of 8), so every tile of one XCD
// has u % 8 == xcd; v = xcd * (total / 8) + u / 8 gives each XCD a contiguous
// run of v. v is then decoded in groups of 8 token tiles: 64 consecutive v
// (one round of the XCD's 64 resident workgroups) cover 8 token tiles x 8 n
// tiles, whose K slices the XCD's L2 serves to all 64 at once.
constexpr int GROUP_T = 8;
__device__ __forceinline__ void tile_coords(const TileGrid& g, int u, int& tt, int& tn) {
  int v = u;
  if ((g.total & 7) == 0) v = (u & 7) * (g.total >> 3) + (u >> 3);
  const int per_group = GROUP_T * g.tiles_n;
  const int first_t = (v / per_group) * GROUP_T;
  const int rows = min(g.tiles_t - first_t, GROUP_T);
  const int w = v % per_group;
  tt = first_t + w % rows;
  tn = w / rows;
}


// Per-lane DMA source offsets of one tile (rows clamped into the matrix so
// that partial tiles never read out of bounds; clamped rows only feed
// accumulators the epilogue discards). Wave load q of wave w fills rows
// RPL (4q + w) .. +RPL-1 of the slot; lane i takes row i / CPR and the source
// chunk whose swizzled place is chunk i % CPR.
template <int MODE>
struct DmaPlan {
  uint32_t xo[Tile<MODE>::LQX];
  uint32_t wo[Tile<MODE>::LQW];
};

template <int MODE>
__device__ __forceinline__ DmaPlan<MODE> dma_plan(const FwdParams& p, int64_t t0, int n0, int wave, int lane,
                                                  int row_bytes) {
  using TL = Tile<MODE>;
  DmaPlan<MODE> d;
  const int ci = lane % TL::CPR;
#pragma unroll
  for (int q = 0; q < TL::LQX; ++q) {
    const int r = TL::RPL * (4 * q + wave) + lane / TL::CPR;
    int64_t t = t0 + r;
    if (t >= p.T) t = p.T - 1;
    d.xo[q] = (uint32_t)(t * row_bytes + ((ci ^ swz<TL::ROWB>(r)) << 4));
  }
#pragma unroll
  for (int q = 0; q < TL::LQW; ++q) {
    const int r = TL::RPL * (4 * q + wave) + lane / TL::CPR;
    int n = n0 + r;
    if (n >= p.N) n = p.N - 1;
    d.wo[q] = (uint32_t)((int64_t)n * row_bytes + ((ci ^ swz<TL::ROWB>(r)) << 4));
  }
  return d;
}

// Stage `kt` of the tile (K slice kt, clamped to the last one) into ring
// slot `slot_kt % STAGES`.
template <int MODE>
__device__ __forceinline__ void issue_stage(const DmaPlan<MODE>& d, const uint8_t* xb, const uint8_t* wb,
                                            int kt, int nk, int slot_kt, uint32_t ring, int wave) {
  using TL = Tile<MODE>;
  const uint32_t slot = ring + (uint32_t)(slot_kt % TL::STAGES) * TL::SB;
  const int64_t kb = (int64_t)(kt < nk ? kt : nk - 1) * TL::ROWB;
#pragma unroll
  for (int q = 0; q < TL::LQX; ++q) dma16(xb + kb, d.xo[q], slot + (4 * q + wave) * 1024);
#pragma unroll
  for (int q = 0; q < TL::LQW; ++q) dma16(wb + kb, d.wo[q], slot + TL::XSB + (4 * q + wave) * 1024);
}

// Four E4M3 codes -> four bf16 (two dwords), each times 2^(scale - 127).
__device__ __forceinline__ u32x2_t cvt4(uint32_t codes, float scale) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, true);
  return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// 2^(e8m0 - 127) as a float (byte 0 gives the float32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

__device__ __forceinline__ void frag_mx_exact(const uint8_t* rowp, int c, int r, float scale, bf16x8_t& f0,
                                              bf16x8_t& f1) {
  // 16 codes of chunk c of this 128-byte row slice -> two bf16x8 fragments
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(rowp + ((c ^ swz<128>(r)) << 4));
  const u32x2_t q0 = cvt4(v[0], scale), q1 = cvt4(v[1], scale);
  const u32x2_t q2 = cvt4(v[2], scale), q3 = cvt4(v[3], scale);
  f0 = __builtin_bit_cast(bf16x8_t, u32x4_t{q0[0], q0[1], q1[0], q1[1]});
  f1 = __builtin_bit_cast(bf16x8_t, u32x4_t{q2[0], q2[1], q3[0], q3[1]});
}

// MXFP8 operand scales of one stage for this lane's fragment rows: the four
// E8M0 bytes of K blocks 4k .. 4k+3 of W rows arow0 + 32 nb and of X rows
// brow0 + 32 tb (one dword per row and stage, K % 128 == 0). In the FP8 MFMA
// mode only the two bytes this lane passes are kept, in bytes 0 and 1 (see
// mma_stage).
struct StageScales {
  uint32_t w[WBLK_N];
  uint32_t x[WBLK_T];
};
struct ScaleRows {  // byte offset of each row's scales (rows clamped into the matrix)
  int64_t w[WBLK_N];
  int64_t x[WBLK_T];
};

__device__ __forceinline__ ScaleRows scale_rows(const FwdParams& p, int64_t t0, int n0, int arow0, int brow0,
                                                int kt0) {
  ScaleRows sr;
  const int kb = p.K / 32;
  const int64_t k4 = 4 * (int64_t)kt0;  // 4 scale bytes per 128-value stage
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) {
    int n = n0 + arow0 + 32 * nb;
    if (n >= p.N) n = p.N - 1;
    sr.w[nb] = (int64_t)n * kb + k4;
  }
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) {
    int64_t t = t0 + brow0 + 32 * tb;
    if (t >= p.T) t = p.T - 1;
    sr.x[tb] = t * kb + k4;
  }
  return sr;
}

// Scales travel in pairs of stages: for pair j, the lane in wave half h
// loads the dword of stage 2j + h of each of its rows (the two halves hold
// the same rows), and one half-swap gives every lane both stages' dwords.
// That is half the load instructions and cache-line visits of one dword per
// lane and stage, in the same registers.
__device__ __forceinline__ StageScales load_pair(const FwdParams& p, const ScaleRows& sr, int j, int nk,
                                                 int half) {
  int kt = 2 * j + half;
  if (kt > nk - 1) kt = nk - 1;
  const int k4 = 4 * kt;
  StageScales sc;
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) sc.w[nb] = *reinterpret_cast<const uint32_t*>(p.ws + sr.w[nb] + k4);
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) sc.x[tb] = *reinterpret_cast<const uint32_t*>(p.xs + sr.x[tb] + k4);
  return sc;
}

// The pair's dwords in use: s[0] for the even stage, s[1] for the odd one.
// FP8 MFMA mode packs the bytes the lane passes (blocks h and 2 + h of each
// stage, h the wave half) into s[0]: even stage in bytes 0-1, odd in 2-3.
struct PairScales {
  StageScales s[2];
};

template <bool FP8>
__device__ __forceinline__ PairScales unpack_pair(const StageScales& raw, int half) {
  PairScales ps;
  const uint32_t sel = half ? 0x07050301u : 0x06040200u;
  const auto one = [&](uint32_t v, uint32_t& e, uint32_t& o) {
    const u32x2_t t = swap_halves(v, v);  // {stage 2j, stage 2j + 1} in every lane
    if (FP8) {
      e = __builtin_amdgcn_perm(t[1], t[0], sel);
      o = 0;
    } else {
      e = t[0];
      o = t[1];
    }
  };
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) one(raw.w[nb], ps.s[0].w[nb], ps.s[1].w[nb]);
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) one(raw.x[tb], ps.s[0].x[tb], ps.s[1].x[tb]);
  return ps;
}

// FP8 MFMA mode: scales in groups of four stages. For group j the lane in
// wave half h loads the two dwords of stages 4j + 2h and 4j + 2h + 1 of each
// row (one 8-byte load; two dword loads, each clamped, for a group that runs
// past the last stage), two half-swaps give every lane all four stages, and
// the bytes the lane passes (blocks h and 2 + h of each stage) pack into two
// dwords: stages 4j, 4j + 1 in the first, 4j + 2, 4j + 3 in the second. A
// quarter of the load instructions of one dword per lane and stage.
struct QuadScales {
  uint32_t w[WBLK_N][2];
  uint32_t x[WBLK_T][2];
};
// Exact mode: both wave halves pass all four bytes of a stage, so the four
// stages' dwords are kept as loaded.
struct QuadScales4 {
  uint32_t w[WBLK_N][4];
  uint32_t x[WBLK_T][4];
};

__device__ __forceinline__ QuadScales load_quad(const FwdParams& p, const ScaleRows& sr, int j, int nk, int half) {
  QuadScales q;
  const int kt = 4 * j + 2 * half;
  if (4 * j + 3 < nk) {
    const int k4 = 4 * kt;
    const auto ld8 = [](const uint8_t* a, uint32_t (&o)[2]) {
      u32x2_t v;  // 8 bytes at a 4-byte aligned address: one global_load_dwordx2
      __builtin_memcpy(&v, a, 8);
      o[0] = v[0];
      o[1] = v[1];
    };
#pragma unroll
    for (int nb = 0; nb < WBLK_N; ++nb) ld8(p.ws + sr.w[nb] + k4, q.w[nb]);
#pragma unroll
    for (int tb = 0; tb < WBLK_T; ++tb) ld8(p.xs + sr.x[tb] + k4, q.x[tb]);
  } else {
    const int ka = 4 * min(kt, nk - 1), kb = 4 * min(kt + 1, nk - 1);
#pragma unroll
    for (int nb = 0; nb < WBLK_N; ++nb) {
      q.w[nb][0] = *reinterpret_cast<const uint32_t*>(p.ws + sr.w[nb] + ka);
      q.w[nb][1] = *reinterpret_cast<const uint32_t*>(p.ws + sr.w[nb] + kb);
    }
#pragma unroll
    for (int tb = 0; tb < WBLK_T; ++tb) {
      q.x[tb][0] = *reinterpret_cast<const uint32_t*>(p.xs + sr.x[tb] + ka);
      q.x[tb][1] = *reinterpret_cast<const uint32_t*>(p.xs + sr.x[tb] + kb);
    }
  }
  return q;
}

__device__ __forceinline__ QuadScales unpack_quad(const QuadScales& raw, int half) {
  QuadScales q;
  const uint32_t sel = half ? 0x07050301u : 0x06040200u;
  const auto one = [&](const uint32_t (&r)[2], uint32_t (&o)[2]) {
    const u32x2_t t0 = swap_halves(r[0], r[0]);  // stages 4j, 4j + 2
    const u32x2_t t1 = swap_halves(r[1], r[1]);  // stages 4j + 1, 4j + 3
    o[0] = __builtin_amdgcn_perm(t1[0], t0[0], sel);
    o[1] = __builtin_amdgcn_perm(t1[1], t0[1], sel);
  };
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) one(raw.w[nb], q.w[nb]);
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) one(raw.x[tb], q.x[tb]);
  return q;
}

__device__ __forceinline__ QuadScales4 unpack_quad4(const QuadScales& raw) {
  QuadScales4 q;
  const auto one = [&](const uint32_t (&r)[2], uint32_t (&o)[4]) {
    const u32x2_t t0 = swap_halves(r[0], r[0]);  // stages 4j, 4j + 2
    const u32x2_t t1 = swap_halves(r[1], r[1]);  // stages 4j + 1, 4j + 3
    o[0] = t0[0];
    o[1] = t1[0];
    o[2] = t0[1];
    o[3] = t1[1];
  };
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) one(raw.w[nb], q.w[nb]);
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) one(raw.x[tb], q.x[tb]);
  return q;
}

__device__ __forceinline__ StageScales quad4_stage(const QuadScales4& q, int kt) {
  const bool hi = (kt >> 1) & 1, odd = kt & 1;
  StageScales sc;
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) {
    const uint32_t a = odd ? q.w[nb][1] : q.w[nb][0], b = odd ? q.w[nb][3] : q.w[nb][2];
    sc.w[nb] = hi ? b : a;
  }
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) {
    const uint32_t a = odd ? q.x[tb][1] : q.x[tb][0], b = odd ? q.x[tb][3] : q.x[tb][2];
    sc.x[tb] = hi ? b : a;
  }
  return sc;
}

__device__ __forceinline__ StageScales quad_stage(const QuadScales& q, int kt) {
  // a select of two named values and a shift (a runtime index into the
  // pair would put the arrays in scratch memory)
  const bool hi = (kt >> 1) & 1;
  const int sh = 16 * (kt & 1);
  StageScales sc;
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) {
    const uint32_t a = q.w[nb][0], b = q.w[nb][1];
    sc.w[nb] = (hi ? b : a) >> sh;
  }
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) {
    const uint32_t a = q.x[tb][0], b = q.x[tb][1];
    sc.x[tb] = (hi ? b : a) >> sh;
  }
  return sc;
}

// Scales of stage kt of the current pair.
template <bool FP8>
__device__ __forceinline__ StageScales stage_scales(const PairScales& ps, int kt) {
  const bool odd = kt & 1;
  StageScales sc;
#pragma unroll
  for (int nb = 0; nb < WBLK_N; ++nb) sc.w[nb] = FP8 ? ps.s[0].w[nb] >> (odd ? 16 : 0) : (odd ? ps.s[1].w[nb] : ps.s[0].w[nb]);
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) sc.x[tb] = FP8 ? ps.s[0].x[tb] >> (odd ? 16 : 0) : (odd ? ps.s[1].x[tb] : ps.s[0].x[tb]);
  return sc;
}

template <int MODE>
__device__ __forceinline__ void mma_stage(f32x16_t (&acc)[WBLK_N][WBLK_T], const uint8_t* cur,
                                          const StageScales& sc, int arow0, int brow0, int half) {
  using TL = Tile<MODE>;
  if (!TL::MX) {
    // all fragments of the stage's k16 steps first, so the later steps' LDS
    // reads are in flight while the first step's MFMAs run
    constexpr int NJS = TL::KPS / 16;
    bf16x8_t a[NJS][WBLK_N], b[NJS][WBLK_T];
#pragma unroll
    for (int j = 0; j < NJS; ++j) {
#pragma unroll
      for (int nb = 0; nb < WBLK_N; ++nb)
        a[j][nb] = *reinterpret_cast<const bf16x8_t*>(cur + TL::XSB + roff<TL::ROWB>(arow0 + 32 * nb, 2 * j + half));
#pragma unroll
      for (int tb = 0; tb < WBLK_T; ++tb)
        b[j][tb] = *reinterpret_cast<const bf16x8_t*>(cur + roff<TL::ROWB>(brow0 + 32 * tb, 2 * j + half));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead
#pragma unroll
    for (int j = 0; j < NJS; ++j)
#pragma unroll
      for (int tb = 0; tb < WBLK_T; ++tb)
#pragma unroll
        for (int nb = 0; nb < WBLK_N; ++nb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][nb], b[j][tb], acc[nb][tb], 0, 0, 0);
  } else if (MODE == MODE_MX_EXACT) {
    // E4M3 expanded exactly to bf16 (code * 2^(scale-127)) per fragment; the
    // bf16 MFMA then multiplies exactly and accumulates in fp32. K is walked
    // in a permuted but identical order for both operands: for K-block jb of
    // the slice, lane half h reads the whole 16-byte chunk 2 jb + h, whose
    // first and last 8 codes feed two k16 steps.
#pragma unroll
    for (int jb = 0; jb < TL::KPS / 32; ++jb) {
      const int c = 2 * jb + half;
      bf16x8_t a0[WBLK_N], a1[WBLK_N], b0[WBLK_T], b1[WBLK_T];
#pragma unroll
      for (int nb = 0; nb < WBLK_N; ++nb) {
        const int r = arow0 + 32 * nb;
        frag_mx_exact(cur + TL::XSB + r * TL::ROWB, c, r, e8m0_to_f32((sc.w[nb] >> (8 * jb)) & 0xFFu),
                      a0[nb], a1[nb]);
      }
#pragma unroll
      for (int tb = 0; tb < WBLK_T; ++tb) {
        const int r = brow0 + 32 * tb;
        frag_mx_exact(cur + r * TL::ROWB, c, r, e8m0_to_f32((sc.x[tb] >> (8 * jb)) & 0xFFu), b0[tb], b1[tb]);
      }
#pragma unroll
      for (int nb = 0; nb < WBLK_N; ++nb)
#pragma unroll
        for (int tb = 0; tb < WBLK_T; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[nb], b0[tb], acc[nb][tb], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < WBLK_N; ++nb)
#pragma unroll
        for (int tb = 0; tb < WBLK_T; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[nb], b1[tb], acc[nb][tb], 0, 0, 0);
    }
  } else {
    // Scaled FP8 32x32x64, two per 128-value slice (s = 0, 1): lane
    // (row, half) holds 16 bytes of K-block 2s (k = 64 s + 16 half .. +15) in
    // its first four registers and 16 bytes of K-block 2s+1 (k = 64 s + 32 +
    // 16 half .. +15) in the last four; the E8M0 scale of (row, block b) is
    // taken from lane row + 32 b, byte 0, so each lane passes the scale of
    // block 2s + half of its row.
#pragma unroll
    for (int st = 0; st < TL::KPS / 64; ++st) {
      i32x8_t a[WBLK_N], b[WBLK_T];
      uint32_t sa[WBLK_N], sb[WBLK_T];
      const int sh = 8 * st;  // packed: this lane's block 2 st + half
#pragma unroll
      for (int nb = 0; nb < WBLK_N; ++nb) {
        const int r = arow0 + 32 * nb;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(cur + TL::XSB + roff<128>(r, 4 * st + half));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(cur + TL::XSB + roff<128>(r, 4 * st + 2 + half));
        a[nb] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sa[nb] = (sc.w[nb] >> sh) & 0xFFu;
      }
#pragma unroll
      for (int tb = 0; tb < WBLK_T; ++tb) {
        const int r = brow0 + 32 * tb;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(cur + roff<128>(r, 4 * st + half));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(cur + roff<128>(r, 4 * st + 2 + half));
        b[tb] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sb[tb] = (sc.x[tb] >> sh) & 0xFFu;
      }
#pragma unroll
      for (int nb = 0; nb < WBLK_N; ++nb)
#pragma unroll
        for (int tb = 0; tb < WBLK_T; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[nb], b[tb], acc[nb][tb], 0, 0, 0, (int)sa[nb], 0, (int)sb[tb]);
    }
  }
}

// Plain row-major store of one 32 x 32 block, out[t][n] with row stride N,
// bf16 or fp32 (no bias, no rotation): the product form the MXFP8 backward
// uses. Lanes l and l^32 trade 4-row groups so that each lane owns 16
// consecutive n (lower lane rows 0..15, upper 16..31).
__device__ __forceinline__ void plain_block(const FwdParams& p, uint8_t* out, int64_t t, bool ok,
                                            const f32x16_t& acc, int n_blk, int lane) {
  const int half = lane >> 5;
  if (p.out_f32) {
    u32x2_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      // by value: a bit cast of a vector element lvalue reads element 0 here
      r[j] = swap_halves(__float_as_uint(acc[j]), __float_as_uint(acc[8 + j]));
    if (ok) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (t * p.N + n_blk + 16 * half) * 4);
      dst[0] = u32x4_t{r[0][0], r[1][0], r[2][0], r[3][0]};
      dst[1] = u32x4_t{r[0][1], r[1][1], r[2][1], r[3][1]};
      dst[2] = u32x4_t{r[4][0], r[5][0], r[6][0], r[7][0]};
      dst[3] = u32x4_t{r[4][1], r[5][1], r[6][1], r[7][1]};
    }
  } else {
    uint32_t P[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      P[2 * g] = pack_bf16x2(acc[4 * g + 0], acc[4 * g + 1]);
      P[2 * g + 1] = pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3]);
    }
    u32x2_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = swap_halves(P[k], P[4 + k]);
    if (ok) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (t * p.N + n_blk + 16 * half) * 2);
      dst[0] = u32x4_t{r[0][0], r[1][0], r[0][1], r[1][1]};
      dst[1] = u32x4_t{r[2][0], r[3][0], r[2][1], r[3][1]};
    }
  }
}

__device__ __forceinline__ void plain_tile(const FwdParams& p, uint8_t* out,
                                           const f32x16_t (&acc)[WBLK_N][WBLK_T], int n0, int64_t t_lane,
                                           int lane) {
#pragma unroll
  for (int tb = 0; tb < WBLK_T; ++tb) {
    const int64_t t = t_lane + 32 * tb;
#pragma unroll
    for (int nb = 0; nb < WBLK_N; ++nb) {
      const int n_blk = n0 + 32 * nb;
      if (n_blk < p.N) plain_block(p, out, t, t < p.T, acc[nb][tb], n_blk, lane);
    }
  }
}

// Work unit u -> tile and K range. The fused forward runs every tile over
// the whole K; the plain product form may split K into p.k_splits ranges of
// equal stage counts (unit u: range u / tiles, tile u % tiles), each range
// writing its own fp32 partial output.
struct Unit {
  int tt, tn;   // token tile, n tile
  int kt0, nk;  // first stage and stage count
  int split;
};
template <int EPI>
__device__ __forceinline__ Unit unit_coords(const TileGrid& g, const FwdParams& p, int u, int nk_all) {
  Unit w;
  if (EPI == EPI_PLAIN) {
    w.split = u / g.total;
    const int per = (nk_all + p.k_splits - 1) / p.k_splits;
    w.kt0 = w.split * per;
    w.nk = min(per, nk_all - w.kt0);
    tile_coords(g, u - w.split * g.total, w.tt, w.tn);
  } else {
    w.split = 0;
    w.kt0 = 0;
    w.nk = nk_all;
    tile_coords(g, u, w.tt, w.tn);
  }
  return w;
}

// TAB: the tile's cos/sin rows are staged in LDS for the epilogue (a
// compile-time choice, so that instantiation has no global table loads whose
// waits would also wait for the next tile's DMA in flight).
template <int MODE, int EPI, bool TAB = false>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(WG_PER_CU, WG_PER_CU)))
void qup_fwd_kernel(FwdParams p) {
  using TL = Tile<MODE>;
  constexpr bool MX = TL::MX;
  constexpr int KPS = TL::KPS;
  constexpr int STAGES = TL::STAGES;
  constexpr int RING = TL::SB * STAGES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RING];
  static_assert(STAGES != 2 || 2 * ROPE_TAB_HALF <= TL::SB, "table rows must fit one slot");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int wn = wave % WAVES_N, wt = wave / WAVES_N;
  const int arow0 = 32 * WBLK_N * wn + (lane & 31);  // 96 of the tile's N rows
  const int brow0 = 32 * WBLK_T * wt + (lane & 31);  // and 64 of its tokens

  const TileGrid grid{(int)((p.T + TILE_T - 1) / TILE_T), (p.N + TILE_N - 1) / TILE_N, 0};
  const TileGrid g{grid.tiles_t, grid.tiles_n, grid.tiles_t * grid.tiles_n};
  const int row_bytes = MX ? p.K : 2 * p.K;
  const int nk_all = p.K / KPS;
  const int units = EPI == EPI_PLAIN ? g.total * p.k_splits : g.total;
  const uint32_t ring = lds_u32(lds);
  const TokenMap tm{p.fmt, p.B, p.S, p.cu, p.nseq};

  int u = blockIdx.x;
  if (u >= units) return;
  Unit un_ = unit_coords<EPI>(g, p, u, nk_all);
  int64_t t0 = (int64_t)un_.tt * TILE_T;
  int n0 = un_.tn * TILE_N;
  int nk = un_.nk;
  // operand bases at the unit's first stage (stage indices below are relative)
  const uint8_t* xb = static_cast<const uint8_t*>(p.x) + (int64_t)un_.kt0 * TL::ROWB;
  const uint8_t* wb = static_cast<const uint8_t*>(p.w) + (int64_t)un_.kt0 * TL::ROWB;
  DmaPlan<MODE> dp = dma_plan<MODE>(p, t0, n0, wave, lane, row_bytes);
  ScaleRows sr{};
  StageScales sc_raw{}, sc_cur{};
  PairScales sc_pair{};
  QuadScales q_raw{}, q_cur{};  // FP8 MFMA mode: packed bytes
  QuadScales4 q4_cur{};         // exact mode: whole dwords
  // groups of four stages, except the exact mode's fused forward, which has
  // no registers to spare for them (pairs there)
  constexpr bool QUAD = MODE == MODE_MX_FP8 || (MODE == MODE_MX_EXACT && EPI == EPI_PLAIN);
  if (MX) sr = scale_rows(p, t0, n0, arow0, brow0, un_.kt0);
  // stage s of the current tile lives in slot (sb + s) % STAGES; each tile
  // starts where the previous one's stage sequence (nk + STAGES - 1 issued
  // stages) left off
  int sb = 0;
  // With two slots, the last iteration's spare load (past the last stage)
  // brings the tile's cos/sin rows instead, so they land during the last
  // stage's MFMAs rather than after the loop, and the epilogue reads them
  // with LDS reads that never wait for the next tile's DMA.
  constexpr bool tab_lds = TAB;
  static_assert(!TAB || (STAGES == 2 && EPI == EPI_MLA), "table staging uses the spare slot of a 2-slot ring");
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue_stage<MODE>(dp, xb, wb, s, nk, sb + s, ring, wave);
  if (QUAD)
    q_raw = load_quad(p, sr, 0, nk, half);
  else if (MX)
    sc_raw = load_pair(p, sr, 0, nk, half);  // MX: STAGES == 2

  for (;;) {
    f32x16_t acc[WBLK_N][WBLK_T];
#pragma unroll
    for (int i = 0; i < WBLK_N; ++i)
#pragma unroll
      for (int j = 0; j < WBLK_T; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int kt = 0; kt < nk; ++kt) {
      vm_wait<(STAGES - 2) * TL::LPS>();
      barrier();
      // Always issue (past the last stage the source clamps to it) so every
      // iteration has the same number of loads in flight; slot
      // (kt + STAGES - 1) % STAGES was read in iteration kt - 1 and every
      // wave has passed the barrier since.
      if (tab_lds && kt == nk - 1)
        stage_rope_rows(p, tm, t0, ring + (uint32_t)((sb + nk) % STAGES) * TL::SB, wave, lane);
      else
        issue_stage<MODE>(dp, xb, wb, kt + STAGES - 1, nk, sb + kt + STAGES - 1, ring, wave);
      if (QUAD) {
        // group kt / 4 arrived (the wait above covers all vector loads); the
        // next group goes out with stage kt + 1's DMA
        if ((kt & 3) == 0) {
          if (MODE == MODE_MX_FP8)
            q_cur = unpack_quad(q_raw, half);
          else
            q4_cur = unpack_quad4(q_raw);
          q_raw = load_quad(p, sr, kt / 4 + 1, nk, half);
        }
        sc_cur = MODE == MODE_MX_FP8 ? quad_stage(q_cur, kt) : quad4_stage(q4_cur, kt);
      } else if (MX) {
        // the same in pairs of stages
        if ((kt & 1) == 0) {
          sc_pair = unpack_pair<MODE == MODE_MX_FP8>(sc_raw, half);
          sc_raw = load_pair(p, sr, kt / 2 + 1, nk, half);
        }
        sc_cur = stage_scales<MODE == MODE_MX_FP8>(sc_pair, kt);
      }
      mma_stage<MODE>(acc, lds + ((sb + kt) % STAGES) * TL::SB, sc_cur, arow0, brow0, half);
    }

    // Next tile of this workgroup: start its first stages before the
    // epilogue of the current one.
    const int un = u + gridDim.x;
    const bool more = un < units;
    const int64_t t0c = t0;
    const int n0c = n0;
    const int split_c = un_.split;
    const RopeTab tab{tab_lds, ring + (uint32_t)((sb + nk) % STAGES) * TL::SB};
    sb = (sb + nk + STAGES - 1) % STAGES;  // the next tile's stage 0 avoids the table's slot
    vm_wait<0>();
    barrier();
    if (more) {
      un_ = unit_coords<EPI>(g, p, un, nk_all);
      t0 = (int64_t)un_.tt * TILE_T;
      n0 = un_.tn * TILE_N;
      nk = un_.nk;
      xb = static_cast<const uint8_t*>(p.x) + (int64_t)un_.kt0 * TL::ROWB;
      wb = static_cast<const uint8_t*>(p.w) + (int64_t)un_.kt0 * TL::ROWB;
      dp = dma_plan<MODE>(p, t0, n0, wave, lane, row_bytes);
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) issue_stage<MODE>(dp, xb, wb, s, nk, sb + s, ring, wave);
      if (MX) {
        sr = scale_rows(p, t0, n0, arow0, brow0, un_.kt0);
        if (QUAD)
          q_raw = load_quad(p, sr, 0, nk, half);
        else
          sc_raw = load_pair(p, sr, 0, nk, half);
      }
    }
    if (EPI == EPI_PLAIN)
      plain_tile(p, static_cast<uint8_t*>(p.out) + (int64_t)split_c * p.split_stride, acc,
                 n0c + 32 * WBLK_N * wn, t0c + 32 * WBLK_T * wt + (lane & 31), lane);
    else
      epilogue_tile(p, tm, acc, n0c + 32 * WBLK_N * wn, t0c + 32 * WBLK_T * wt + (lane & 31), lane, tab,
                    32 * WBLK_T * wt + (lane & 31));
    if (!more) break;
    u = un;
  }
}

}  // namespace

int fwd_grid(const FwdParams& p, int num_cus) {
  const int64_t tiles = ((p.T + TILE_T - 1) / TILE_T) * ((p.N + TILE_N - 1) / TILE_N);
  int64_t g = (int64_t)num_cus * WG_PER_CU;
  if (g % 8) g -= g % 8;
  if (g < 8) g = 8;
  return (int)(tiles < g ? tiles : g);
}


namespace {
// Table rows can be staged in LDS when the rope slice is 64 wide (the first
// 32 pairs of a row, 128 bytes), rows start 16-byte aligned and every row
// offset fits the 32-bit DMA offset.
bool rope_rows_fit_lds(const FwdParams& p) {
  const auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  return p.d_rope == 64 && p.rope_pairs % 4 == 0 && p.rope_rows > 0 && a16(p.cos) && a16(p.sin) &&
         (int64_t)p.rope_rows * p.rope_pairs * 4 <= (int64_t)UINT32_MAX;
}
}  // namespace

hipError_t launch_qup_fwd_bf16(const FwdParams& p_in, hipStream_t stream) {
  FwdParams p = p_in;
  p.rope_lds = rope_rows_fit_lds(p);
  const dim3 grid(fwd_grid(p, device_cu_count()));
  if (p.K % 64 == 0) {
    if (p.rope_lds)
      hipLaunchKernelGGL((qup_fwd_kernel<MODE_BF16, EPI_MLA, true>), grid, dim3(NTHREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((qup_fwd_kernel<MODE_BF16, EPI_MLA>), grid, dim3(NTHREADS), 0, stream, p);
  } else
    hipLaunchKernelGGL((qup_fwd_kernel<MODE_BF16_R64, EPI_MLA>), grid, dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_qup_fwd_mx(const FwdParams& p_in, hipStream_t stream) {
  FwdParams p = p_in;
  p.rope_lds = rope_rows_fit_lds(p);
  const dim3 grid(fwd_grid(p, device_cu_count()));
  if (p.mx_fp8_mfma) {
    if (p.rope_lds)
      hipLaunchKernelGGL((qup_fwd_kernel<MODE_MX_FP8, EPI_MLA, true>), grid, dim3(NTHREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((qup_fwd_kernel<MODE_MX_FP8, EPI_MLA>), grid, dim3(NTHREADS), 0, stream, p);
  } else {
    if (p.rope_lds)
      hipLaunchKernelGGL((qup_fwd_kernel<MODE_MX_EXACT, EPI_MLA, true>), grid, dim3(NTHREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((qup_fwd_kernel<MODE_MX_EXACT, EPI_MLA>), grid, dim3(NTHREADS), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const FwdParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)mx_gemm_tiles(p.T, p.N) * p.k_splits;
  int64_t g = (int64_t)device_cu_count() * WG_PER_CU;
  if (g % 8) g -= g % 8;
  if (g < 8) g = 8;
  const dim3 grid((unsigned)(units < g ? units : g));
  if (p.mx_fp8_mfma)
    hipLaunchKernelGGL((qup_fwd_kernel<MODE_MX_FP8, EPI_PLAIN>), grid, dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL((qup_fwd_kernel<MODE_MX_EXACT, EPI_PLAIN>), grid, dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
