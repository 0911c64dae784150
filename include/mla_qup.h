/*
 * mla_qup.h -- C ABI of the MI355X (gfx950) fused MLA query up-projection.
 *
 * The operation, as the pages state it:
 *   - forward: "Add support for fused Q Up-Proj GEMM/RoPE/Quant."
 *     (TransformerEngine pull request), description and flowchart: the Q
 *     up-projection GEMM of DeepSeek-V3's MLA fused with the RoPE that
 *     follows it and with MXFP8 quantization of the query; 16-bit or MXFP8
 *     projection; inputs are the activation, the weight and RoPE cos/sin;
 *     file table: BHSD layout with transposed scales.
 *   - backward: "Add a backwards linear function to be used with the fused
 *     mla q up-proj" (TransformerEngine pull request), summary and sequence
 *     diagram: inverse RoPE on the query-output gradient, then the linear
 *     backward for input and weight gradients; review comment "BF16 bias
 *     gradient remains missing": with use_bias the bias gradient is due.
 *   - "Fix fused MLA YaRN RoPE query kernel corrupting upstream tensor
 *     in-place" (Megatron-LM pull request): YaRN RoPE on q, sbhd and thd
 *     token formats, the input must not be modified (Changes; review
 *     thread), and the cos/sin table must be wide enough for the rope
 *     dimension (Problem).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The
 *     library never allocates, frees or retains them, and keeps no state
 *     between calls apart from a read-only cache of device properties.
 *   - Inputs are const and never written. Outputs must not overlap any
 *     input, any other output or the workspace (else MLA_EALIAS).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). All work
 *     is enqueued asynchronously on it; nothing synchronizes.
 *   - Arguments are validated on the host before anything is enqueued. On
 *     any error status nothing is enqueued and nothing is written.
 *     MLA_EDEVICE means the HIP runtime refused a launch; faults inside a
 *     kernel surface at the caller's next synchronization, as usual in HIP.
 *   - bf16 tensors are passed as raw 16-bit storage; tensors read with
 *     16-byte vector loads must be 16-byte aligned (stated per argument).
 *   - T = 0 tokens is valid: the forward enqueues nothing; the backward
 *     writes zeros to dw and db (sums over no tokens) and nothing else.
 */
#ifndef MLA_QUP_H
#define MLA_QUP_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mla_status;
enum {
  MLA_OK = 0,
  MLA_EINVAL = 1,        /* NULL required pointer, bad size/shape, misalignment */
  MLA_EROPE_TABLE = 2,   /* cos/sin table narrower than d_rope/2 pairs, or fewer
                            rows than the largest position + 1 */
  MLA_EALIAS = 3,        /* an output overlaps an input, output or workspace */
  MLA_EUNSUPPORTED = 4,  /* valid combination this library does not implement */
  MLA_EDEVICE = 5,       /* the HIP runtime reported an error at launch */
  MLA_EWORKSPACE = 6,    /* workspace NULL or smaller than required */
  MLA_ESCRATCH = 7       /* mla_qup_bwd_noalloc: the call needs more than the
                            library's static scratch (MLA_BWD_SCRATCH_BYTES) */
};

enum { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP32 = 1, MLA_DTYPE_MXFP8 = 2 };

/* Token formats: rows of X (and of dQ) are tokens.
 *   BSHD: row t = b*S + s, position s.
 *   SBHD: row t = s*B + b, position s.
 *   THD : sequences packed back to back; cu_seqlens[j] is the first row of
 *         sequence j; position = t - cu_seqlens[j] (restarts per sequence).
 * The BHSD output of the forward is [B, H, S, D]; for THD it is
 * [1, H, T, D], token t at s = t. */
enum { MLA_FMT_BSHD = 0, MLA_FMT_SBHD = 1, MLA_FMT_THD = 2 };

typedef struct {
  int32_t fmt;                 /* MLA_FMT_* */
  int32_t B, S;                /* BSHD/SBHD: batch and sequence length, T = B*S.
                                  THD: ignored */
  int64_t T;                   /* number of token rows */
  const int32_t* cu_seqlens;   /* THD: device int32[nseq + 1], cu[0] = 0,
                                  nondecreasing, cu[nseq] = T. Else NULL */
  int32_t nseq;                /* THD: number of sequences (>= 1) */
  int32_t max_seqlen;          /* THD: host-side bound on every sequence length;
                                  the table must have >= max_seqlen rows. A
                                  token whose position is still beyond the
                                  table gets NaN in its rotated elements
                                  (never an out-of-bounds read) */
} mla_tokens;

/* YaRN frequency scaling (YaRN, Peng et al. 2023, NTK-by-parts; ramp linear
 * in the pair index between floor(corr(beta_fast)) and ceil(corr(beta_slow)),
 * corr(n) = d*ln(L/(2*pi*n))/(2*ln(base)), clamped to [0, d-1]).
 * theta'_i = theta_i*(1 - r_i) + theta_i/factor*r_i; cos and sin are
 * multiplied by mscale. */
typedef struct {
  double factor;        /* > 0 */
  int32_t orig_max_pos; /* original context length L, > 0 */
  double beta_fast;     /* > 0 */
  double beta_slow;     /* > 0 */
  double mscale;        /* multiplier of cos and sin */
} mla_yarn;

/* RoPE table: cos[p*pairs + i], sin[p*pairs + i], fp32, device, each
 * 16-byte aligned (the inverse-RoPE kernel reads four pairs with one 16-byte
 * load, the forward epilogue two with one 8-byte load). Forward page,
 * flowchart: "RoPE cos/sin" is an input of the fused up-projection; YaRN-fix
 * page, Problem: the table must cover the rope width and every position. */
typedef struct {
  const float* cos;
  const float* sin;
  int32_t rows;    /* positions covered: 0 .. rows-1 */
  int32_t pairs;   /* row stride in elements; must be >= d_rope/2 */
} mla_rope;

/* Build the RoPE table: for p < rows, i < d_rope/2,
 *   cos[p*(d_rope/2)+i] = m*cos(p*theta'_i), sin[...] = m*sin(p*theta'_i),
 * theta_i = base^(-2i/d_rope), computed in double and rounded to float.
 * yarn == NULL: plain RoPE (theta' = theta, m = 1).
 * Forward page flowchart: "RoPE cos/sin" is an input of the fused
 * up-projection. cos, sin: device float[rows*d_rope/2], 4-byte aligned.
 * Errors: MLA_EINVAL for NULL tables, rows < 1, d_rope < 2 or odd,
 * base <= 1, or invalid yarn fields. */
MLA_API mla_status rope_cache_build(float* cos, float* sin, int32_t rows, int32_t d_rope,
                            double base, const mla_yarn* yarn, void* stream);

/* MXFP8-quantize a row-major matrix along its rows (blocks of 32 consecutive
 * elements of a row). Forward page, file table and review thread: the
 * separable MXFP8 quantization used for the MXFP8 projection operands.
 * Per block (OCP Microscaling Formats v1.0): amax = max|x|;
 * E = clamp(floor(log2 amax) - 8, -127, 127) (E = -127 when amax = 0);
 * scale byte E + 127; element = E4M3 round-to-nearest-even of x*2^-E,
 * saturated to +-448, sign of zero kept. A block holding NaN or Inf gets
 * scale 0xFF and codes 0x7F.
 *   x      : device, x_dtype MLA_DTYPE_BF16 or MLA_DTYPE_FP32, element (r, c)
 *            at x[r*ld + c]; 16-byte aligned, ld*elemsize a multiple of 16.
 *   rows, cols: rows >= 0, cols > 0 and a multiple of 32, rows * cols <= 2^36;
 *               ld >= cols.
 *   codes  : device uint8[rows*cols] (row-major, stride cols), 8-byte aligned.
 *   scales : device uint8[rows*cols/32] (row-major, stride cols/32).
 * Errors: MLA_EINVAL, MLA_EALIAS. */
MLA_API mla_status mxfp8_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                          int64_t ld, uint8_t* codes, uint8_t* scales, void* stream);

/* MXFP8-quantize a row-major bf16 matrix along its COLUMNS (blocks of 32
 * consecutive rows of a column) and store the result transposed, the blocked
 * axis contiguous: the operand layout of a product that reduces over the
 * matrix's rows. Used by mla_qup_bwd_mxfp8 for W, x and dq_pre (the forward
 * page's mxfp8 projection carried into the backward page's linear backward;
 * each operand is quantized along its product's reduction axis). Same block
 * rule as mxfp8_quantize; rows r in [rows, rows_pad) count as zeros.
 *   x       : device bf16, element (r, c) at x[r*ld + c]; 16-byte aligned,
 *             ld a multiple of 8.
 *   rows >= 0; cols > 0, a multiple of 8, at most 4194240; ld >= cols;
 *   rows_pad >= rows, a multiple of 32.
 *   codes_t : device uint8[cols*rows_pad], element (c, r) at
 *             codes_t[c*rows_pad + r]; 16-byte aligned.
 *   scales_t: device uint8[cols*rows_pad/32], block (c, r/32) at
 *             scales_t[c*(rows_pad/32) + r/32].
 * Errors: MLA_EINVAL, MLA_EALIAS. */
MLA_API mla_status mxfp8_quantize_t(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                    int64_t rows_pad, uint8_t* codes_t, uint8_t* scales_t,
                                    void* stream);

/* Forward: Q = X W^T (+ bias), RoPE on pairs (2i, 2i+1) of each head's rope
 * slice (head layout [nope | rope], D = d_nope + d_rope, N = H*D), written
 * out of place in BHSD, as BF16 or MXFP8 (one E8M0 scale per 32 elements
 * along head_dim, scales laid out [B, H, S, D/32] like the data).
 * The fp32 accumulator is rotated and quantized without an intermediate
 * 16-bit rounding. */
typedef struct {
  const void* x;            /* BF16 [T, K] or MXFP8 codes [T, K]; 16-B aligned */
  const uint8_t* x_scales;  /* MXFP8: [T, K/32] E8M0, 4-B aligned; else NULL */
  int32_t x_dtype;          /* MLA_DTYPE_BF16 or MLA_DTYPE_MXFP8 */
  const void* w;            /* BF16 [N, K] or MXFP8 codes [N, K]; 16-B aligned */
  const uint8_t* w_scales;  /* MXFP8: [N, K/32], 4-B aligned; else NULL */
  int32_t w_dtype;          /* must equal x_dtype */
  const void* bias;         /* bf16 [N] added before the rotation, or NULL;
                               8-B aligned */
  int32_t K;                /* q_lora_rank; > 0, multiple of 32 (MXFP8: of 128) */
  int32_t H;                /* heads, > 0 */
  int32_t d_nope;           /* >= 0, even */
  int32_t d_rope;           /* >= 0, even; D = d_nope + d_rope a multiple of 32 */
  mla_tokens tokens;
  mla_rope rope;            /* required when d_rope > 0 */
  int32_t out_dtype;        /* MLA_DTYPE_BF16 or MLA_DTYPE_MXFP8 */
  void* out;                /* BHSD; bf16 or uint8 codes; 16-B aligned */
  uint8_t* out_scales;      /* MXFP8: BHSD [.., D/32]; else NULL */
  int32_t flags;            /* 0 or MLA_FWD_FP8_MFMA */
} mla_qup_fwd_args;

/* MXFP8 projection precision. By default (flags = 0) the E4M3 operands are
 * expanded exactly to bf16 (code * 2^(scale-127)) and multiplied on the bf16
 * MFMA with fp32 accumulation, so the result is the fp32-accumulated product.
 * With MLA_FWD_FP8_MFMA they go to the scaled FP8 MFMA instead, at twice the
 * peak rate; on gfx950 that instruction sums the products of one K-step in a
 * narrower fixed-point window (products far below the largest one lose
 * bits), so results deviate from fp32 accumulation by up to ~1e-2 of the
 * output RMS on MX-scaled data. Ignored for bf16 operands. */
enum { MLA_FWD_FP8_MFMA = 1 };

/* The fused forward. Forward page, description: the Q up-projection GEMM
 * with the RoPE that follows it and MXFP8 quantization of the query in one
 * kernel, BF16 or MXFP8 projection; flowchart: X, W and RoPE cos/sin in,
 * MXFP8 Q with BHSD scale transpose out; YaRN-fix page, Changes: YaRN RoPE
 * on q in sbhd and thd formats, the input left unmodified.
 * Ownership: every pointer is caller-owned device memory; inputs are read
 * only; out and out_scales are written completely (every element of the
 * [B, H, S, D] output).
 * Errors: MLA_EINVAL, MLA_EROPE_TABLE, MLA_EALIAS, MLA_EUNSUPPORTED
 * (x_dtype != w_dtype, or X or W spanning more than 4 GiB: the kernel
 * addresses their rows with 32-bit offsets), MLA_EDEVICE. */
MLA_API mla_status mla_qup_fwd(const mla_qup_fwd_args* args, void* stream);

/* Backward:
 *   dq_pre = inverse RoPE of dq (pairs (a, b) -> (a c + b s, -a s + b c),
 *            the transpose of the forward rotation; nope elements copied),
 *   dx = dq_pre W,  dw = dq_pre^T x,  db = sum over tokens of dq_pre.
 * Accumulation is fp32; dq_pre is stored as bf16 and the GEMMs read that
 * bf16 copy; db sums the fp32 values before that rounding. Results are
 * deterministic (no floating-point atomics). */
typedef struct {
  const void* dq;           /* bf16 [T, H, D] token-major; 16-B aligned */
  const void* x;            /* bf16 [T, K] saved forward input; 16-B aligned */
  const void* w;            /* bf16 [N, K]; 16-B aligned */
  int32_t K, H, d_nope, d_rope;   /* as in the forward */
  mla_tokens tokens;
  mla_rope rope;
  void* dq_pre;             /* out: bf16 [T, N]; 16-B aligned (required) */
  void* dx;                 /* out: bf16 [T, K], or NULL to skip; 16-B aligned */
  void* dw;                 /* out: [N, K] in dw_dtype, or NULL to skip; 16-B aligned */
  int32_t dw_dtype;         /* MLA_DTYPE_BF16 or MLA_DTYPE_FP32 */
  int32_t use_bias;         /* 0 or 1 */
  void* db;                 /* out: bf16 [N]; required iff use_bias */
  void* workspace;          /* device scratch, >= mla_qup_bwd_workspace_size()
                               bytes, 256-B aligned; NULL allowed if that is 0 */
  size_t workspace_bytes;
} mla_qup_bwd_args;

/* Workspace bytes mla_qup_bwd needs for these arguments (0 if none). Backward
 * page, review comment on the missing bias gradient and sequence diagram
 * (linear backward for input and weight gradients): the workspace holds the
 * partial sums of those reductions. It contains the db
 * partial sums when use_bias, and the fp32 partials of dX or dW when their
 * reduction is split (long N for dX; few heads and many tokens for dW), so it
 * depends on which of dx, dw and db are requested: query it with the same
 * arguments as the call. Reads the shape fields and whether dx / dw are NULL,
 * never dereferences pointers. Returns 0 for invalid shapes. */
MLA_API size_t mla_qup_bwd_workspace_size(const mla_qup_bwd_args* args);

/* The backward. Backward page, summary and sequence diagram: the RoPE
 * backward turns the query-output gradient into the pre-RoPE projection
 * gradient, then the linear backward gives the input and weight gradients;
 * review comment: with use_bias the bias gradient is produced. YaRN-fix
 * page, review thread: the weight gradient is dy^T x with x the saved input.
 * Ownership: caller-owned device memory; dq, x, w and the table are read
 * only; dq_pre, dx, dw, db and the workspace are written.
 * Errors: MLA_EINVAL, MLA_EROPE_TABLE, MLA_EALIAS, MLA_EWORKSPACE,
 * MLA_EDEVICE. */
MLA_API mla_status mla_qup_bwd(const mla_qup_bwd_args* args, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, results and errors as mla_qup_bwd, except that
 * `workspace` and `workspace_bytes` are ignored: the partial sums live in a
 * static device array of MLA_BWD_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends (looked up once per device, with the
 * stream's device current). When the workspace plan of mla_qup_bwd does not
 * fit, dX and dW are computed without reduction splits (no split partials);
 * if the db partials alone (ceil(T/64) * N * 4 bytes at most) still do not
 * fit: MLA_ESCRATCH. Calls that overlap on one GPU (several streams or host
 * threads) race on that one array: serialize them. The array keeps the last
 * call's contents; nothing in it needs to start at zero. Allocates nothing.
 * Errors: as mla_qup_bwd (never MLA_EWORKSPACE), plus MLA_ESCRATCH, and
 * MLA_EINVAL when the stream belongs to a device other than the current one. */
#define MLA_BWD_SCRATCH_BYTES ((size_t)64 << 20)
MLA_API mla_status mla_qup_bwd_noalloc(const mla_qup_bwd_args* args, void* stream);

/* MXFP8 backward: the forward page's "mxfp8 projection" carried into the
 * backward page's linear backward. Same arguments, outputs and dq_pre / db
 * as mla_qup_bwd; the two products take MXFP8 operands, each quantized
 * along its product's reduction axis (OCP MX: blocks of 32, E8M0 scale,
 * E4M3 round-to-nearest-even, saturating) from the stored bf16 dq_pre and
 * the bf16 x and W:
 *   dx = deq(Q_along_n(dq_pre)) . deq(Q_along_n(W))        (reduction over n)
 *   dw = deq(Q_along_t(dq_pre))^T . deq(Q_along_t(x))      (reduction over t)
 * The token axis is zero-padded for the blocks along t. Accumulation fp32.
 *   fp8_mfma: 0 = products on exact bf16 MFMA of the dequantized operands,
 *             1 = the scaled FP8 MFMA (its internal precision is lower).
 * Extra shape limits: N = H*D a multiple of 128, K a multiple of 32, and
 * T*N, N*ceil128(T), K*N, K*ceil128(T) each below 2^32 (else MLA_EUNSUPPORTED).
 * Workspace: mla_qup_bwd_mxfp8_workspace_size() bytes (quantized operands
 * and dX split partials), 256-B aligned.
 * Errors: as mla_qup_bwd, plus MLA_EUNSUPPORTED. */
MLA_API size_t mla_qup_bwd_mxfp8_workspace_size(const mla_qup_bwd_args* args);
MLA_API mla_status mla_qup_bwd_mxfp8(const mla_qup_bwd_args* args, int32_t fp8_mfma, void* stream);

/* KV side of the attention inputs. YaRN-fix page, Solution: the KV rotary
 * writes fresh key and value outputs (nothing in place); forward page,
 * flowchart: the key and the value each go through an MXFP8 quantization
 * into the same BHSD scale layout as the query. Per token t and head h, with
 * kv[t, h] = [k_nope | v] and one rope slice k_pe[t] shared by all heads:
 *   key[t, h]   = [k_nope[t, h] | rotate(k_pe[t], pos_t)],  D_k = d_nope + d_rope
 *   value[t, h] = v[t, h],                                 D_v = d_v
 * rotated like the query (pairs (2i, 2i+1), (a, b) -> (a c - b s, a s + b c),
 * fp32 from the bf16 inputs, quantized without a 16-bit rounding in between).
 * A position with no table row gives NaN rope elements (an MXFP8 block
 * holding one: scale 0xFF, codes 0x7F). */
typedef struct {
  const void* kv;           /* bf16 [T, H, d_nope + d_v] token-major; 16-B aligned */
  const void* k_pe;         /* bf16 [T, d_rope]; 16-B aligned */
  int32_t H, d_nope, d_rope, d_v;   /* H >= 1; each >= 0 and a multiple of 8;
                                       d_rope <= 256; D_k + D_v > 0 */
  mla_tokens tokens;
  mla_rope rope;            /* as the forward's (only read when d_rope > 0) */
  int32_t out_dtype;        /* MLA_DTYPE_BF16 or MLA_DTYPE_MXFP8 (then D_k and
                               D_v multiples of 32) */
  void* key;                /* out: BHSD [B, H, S, D_k], bf16 or E4M3 codes; 16-B aligned */
  void* key_scales;         /* out (MXFP8): E8M0 [B, H, S, D_k/32] */
  void* value;              /* out: BHSD [B, H, S, D_v]; 16-B aligned */
  void* value_scales;       /* out (MXFP8): E8M0 [B, H, S, D_v/32] */
} mla_kv_args;

/* Errors: MLA_EINVAL, MLA_EROPE_TABLE, MLA_EALIAS, MLA_EDEVICE;
 * MLA_EUNSUPPORTED when T*H*(D_k + D_v)/8 exceeds 2^31 - 1. */
MLA_API mla_status mla_kv_rope(const mla_kv_args* args, void* stream);

/* Static string naming a status code. */
MLA_API const char* mla_status_str(mla_status status);

#ifdef __cplusplus
}
#endif
#endif /* MLA_QUP_H */
