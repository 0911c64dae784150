"""Plain, slow CPU oracle for the fused MLA query up-projection.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do. It shares no code with the HIP library.

Every step is the plain definition, in float64, in the order the pages state
it. The pages (three pull-request pages) are cited by title and section:

  [FWD]  "Add support for fused Q Up-Proj GEMM/RoPE/Quant."
         (TransformerEngine) -- description, Greptile summary, file table,
         flowchart.
  [BWD]  "Add a backwards linear function to be used with the fused mla q
         up-proj" (TransformerEngine) -- Greptile summary, sequence diagram,
         review comment "BF16 bias gradient remains missing".
  [YQ]   "Fix fused MLA YaRN RoPE query kernel corrupting upstream tensor
         in-place" (Megatron-LM) -- What does this PR do, Problem, Solution,
         Changes, review thread.

Where the pages name a format or a method without defining it, the oracle
follows the public definition and names it:

  [OCP-FP8]  OCP 8-bit Floating Point Specification (OFP8): E4M3 encoding
             (bias 7, no infinities, S.1111.111 is NaN, max normal 448).
  [OCP-MX]   OCP Microscaling Formats (MX) v1.0: E8M0 scale, block of 32,
             shared exponent floor(log2 amax) - emax_elem, elements
             quantized with round-to-nearest-even and saturation.
  [ROPE]     RoFormer (Su et al.): rotary position embedding, general form,
             theta_i = base^(-2i/d).
  [YARN]     YaRN (Peng et al., 2023): NTK-by-parts interpolation, in the
             correction-range form used by the MLA YaRN RoPE the [YQ] page
             works on (ramp linear in the pair index between
             floor(corr(beta_fast)) and ceil(corr(beta_slow))).

Precision: arithmetic is float64. Where a floating-point value decides an
integer (the E8M0 scale from the block amax, the E4M3 code), the decision is
taken on the float32 value, the precision the GPU kernel computes in; the
float64 result is rounded once to float32 before that point.

Parity pins: every function here is pinned by tests marked "not gpu"
(closed forms, invariants, library special cases, brute force). No function
is parity-unpinned.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

FMT_BSHD = 0
FMT_SBHD = 1
FMT_THD = 2


# ---------------------------------------------------------------------------
# bf16 storage: decode by definition (the upper 16 bits of a float32),
# encode with torch's CPU round-to-nearest-even cast.
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64. A bf16 is the top half of a float32."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_f64(t) -> np.ndarray:
    """A CPU torch tensor (bf16 / fp32) or numpy array -> float64 numpy."""
    if isinstance(t, torch.Tensor):
        if t.dtype == torch.bfloat16:
            return bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy().view(np.uint16))
        return t.detach().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


# ---------------------------------------------------------------------------
# E4M3 (OCP FP8) and E8M0 (OCP MX) -- [FWD, description: "MXFP8
# quantization"]; element and scale formats per [OCP-FP8], [OCP-MX].
# ---------------------------------------------------------------------------
def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes, from the bit fields [OCP-FP8].

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    Exponent 0 is subnormal: m/8 * 2^-6. S.1111.111 is NaN; no infinities.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = math.nan
        elif exp == 0:
            vals[code] = sign * (man / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


_E4M3 = e4m3_decode_table()
# Non-negative finite codes 0x00..0x7E are increasing in value, so a code's
# index in this array is the code itself.
_E4M3_POS = _E4M3[:0x7F].copy()
E4M3_MAX = 448.0


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 code to each finite y, ties to the even code [OCP-MX].

    Nearest is searched among the 127 non-negative finite codes; a magnitude
    above 448 has 448 as its nearest finite code, which is the saturation the
    MX conversion asks for. The tie-break picks the code whose mantissa LSB is
    0 (the even code index). The sign bit is copied, so -0.0 -> 0x80.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.searchsorted(_E4M3_POS, a, side="left")
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = np.abs(_E4M3_POS[hi] - a)
    d_lo = np.abs(a - _E4M3_POS[lo])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code |= (np.signbit(y).astype(np.uint8) << 7)
    return code


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(code, dtype=np.uint8)]


def e8m0_decode(scale: np.ndarray) -> np.ndarray:
    """E8M0 byte -> 2^(byte-127); 0xFF is NaN [OCP-MX]."""
    s = np.asarray(scale, dtype=np.int64)
    out = np.ldexp(1.0, s - 127).astype(np.float64)
    return np.where(s == 0xFF, math.nan, out)


def floor_log2(a: np.ndarray) -> np.ndarray:
    """Exact floor(log2 a) for a > 0, from frexp (a = m * 2^e, m in [0.5,1))."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1


def mxfp8_quantize_blocks(v: np.ndarray):
    """MXFP8-quantize along the last axis in blocks of 32 [OCP-MX].

    v holds float32 values (any float array; it is rounded to float32 first,
    the precision in which the GPU takes the same decisions). For each block:
      amax = max |v_j|;
      E = -127 if amax == 0, else clamp(floor(log2 amax) - 8, -127, 127)
          (8 = exponent of the largest E4M3 normal, 448 = 1.75 * 2^8);
      scale byte = E + 127;
      code_j = nearest finite E4M3 to v_j * 2^-E, ties to even, saturating.
    A block holding a NaN or an infinity gets scale 0xFF and codes 0x7F.
    Returns (codes uint8 [..., n], scales uint8 [..., n/32]).
    """
    v32 = np.asarray(v, dtype=np.float32)
    n = v32.shape[-1]
    if n % 32:
        raise ValueError("last axis must be a multiple of 32")
    blk = v32.astype(np.float64).reshape(v32.shape[:-1] + (n // 32, 32))
    finite = np.isfinite(blk).all(axis=-1)
    safe = np.where(finite[..., None], blk, 0.0)
    amax = np.abs(safe).max(axis=-1)
    e = np.where(amax > 0, floor_log2(np.where(amax > 0, amax, 1.0)) - 8, -127)
    E = np.clip(e, -127, 127)
    scaled = np.ldexp(safe, -E[..., None])
    codes = e4m3_encode(scaled)
    codes = np.where(finite[..., None], codes, np.uint8(0x7F)).astype(np.uint8)
    scales = np.where(finite, E + 127, 0xFF).astype(np.uint8)
    return codes.reshape(v32.shape), scales


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code value * 2^(scale-127), per block of 32 along the last axis [OCP-MX]."""
    c = np.asarray(codes)
    n = c.shape[-1]
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (n // 32, 32))
    return (vals * e8m0_decode(scales)[..., None]).reshape(c.shape)


# ---------------------------------------------------------------------------
# RoPE / YaRN table -- [FWD, flowchart: "RoPE cos/sin" is an input of the
# fused up-projection]; [YQ, title and Problem: the YaRN RoPE applied to q,
# and the cos/sin width that must cover the rope dimension].
# ---------------------------------------------------------------------------
@dataclass
class Yarn:
    factor: float          # context scaling factor s
    orig_max_pos: int      # original context length L
    beta_fast: float       # rotation count where interpolation starts
    beta_slow: float       # rotation count where interpolation is complete
    mscale: float = 1.0    # multiplier folded into cos and sin


def rope_theta(d_rope: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d_rope), i < d_rope/2 [ROPE]."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    return base ** (-2.0 * i / d_rope)


def yarn_correction_dim(n_rot: float, d_rope: int, base: float, orig_max_pos: int) -> float:
    """Pair index (continuous) whose wavelength fits n_rot times in L [YARN].

    theta_i * L = 2*pi*n_rot with theta_i = base^(-2i/d) gives
    i = d * ln(L / (2*pi*n_rot)) / (2 ln base).
    """
    return d_rope * math.log(orig_max_pos / (n_rot * 2.0 * math.pi)) / (2.0 * math.log(base))


def yarn_ramp(d_rope: int, base: float, y: Yarn) -> np.ndarray:
    """r_i in [0,1]: 0 keeps theta_i, 1 divides it by the factor [YARN]."""
    low = max(math.floor(yarn_correction_dim(y.beta_fast, d_rope, base, y.orig_max_pos)), 0)
    high = min(math.ceil(yarn_correction_dim(y.beta_slow, d_rope, base, y.orig_max_pos)), d_rope - 1)
    span = (high - low) if high != low else 0.001
    i = np.arange(d_rope // 2, dtype=np.float64)
    return np.clip((i - low) / span, 0.0, 1.0)


def yarn_theta(d_rope: int, base: float, y: Yarn) -> np.ndarray:
    """theta'_i = theta_i * (1 - r_i) + (theta_i / s) * r_i [YARN]."""
    th = rope_theta(d_rope, base)
    r = yarn_ramp(d_rope, base, y)
    return th * (1.0 - r) + (th / y.factor) * r


def rope_table(rows: int, d_rope: int, base: float, yarn: Yarn | None = None):
    """cos/sin tables [rows, d_rope/2] float32: m*cos(p*theta'_i), m*sin(p*theta'_i).

    Computed in float64 and rounded once to float32. m = 1 without YaRN.
    """
    th = yarn_theta(d_rope, base, yarn) if yarn is not None else rope_theta(d_rope, base)
    m = float(yarn.mscale) if yarn is not None else 1.0
    ang = np.arange(rows, dtype=np.float64)[:, None] * th[None, :]
    return (m * np.cos(ang)).astype(np.float32), (m * np.sin(ang)).astype(np.float32)


# ---------------------------------------------------------------------------
# Token formats -- [YQ, Changes: tests parameterized over sbhd and thd];
# [FWD, review: "SBHD/BSHD"]. Tokens are the rows of X.
# ---------------------------------------------------------------------------
def token_coords(fmt: int, T: int, B: int = 1, S: int | None = None, cu_seqlens=None):
    """For each token row t of X: (position, b, s) of its BHSD destination.

    BSHD: t = b*S + s;  SBHD: t = s*B + b;  both with position s.
    THD:  sequences packed back to back, cu_seqlens[j] = first token of
          sequence j; position = t - cu_seqlens[j] (reset per sequence);
          destination (0, h, t) of a [1, H, T, D] output.
    """
    t = np.arange(T, dtype=np.int64)
    if fmt == FMT_BSHD:
        b, s = t // S, t % S
        return s, b, s
    if fmt == FMT_SBHD:
        s, b = t // B, t % B
        return s, b, s
    if fmt == FMT_THD:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        j = np.searchsorted(cu, t, side="right") - 1
        return t - cu[j], np.zeros_like(t), t
    raise ValueError("unknown token format")


def out_shape(fmt: int, T: int, H: int, D: int, B: int = 1, S: int | None = None):
    if fmt == FMT_THD:
        return (1, H, T, D)
    return (B, H, S, D)


# ---------------------------------------------------------------------------
# Forward -- [FWD, description and flowchart]: Q = X W^T (16-bit or MXFP8
# projection), RoPE on the rope slice of each head, MXFP8 quantization;
# [YQ, Problem]: q = linear_q_up_proj(x) then a zero-copy view [T, H, D];
# [YQ, Solution / review thread]: the rotation writes a fresh output and never
# modifies its input.
# ---------------------------------------------------------------------------
def rope_rotate(q: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray,
                d_nope: int, d_rope: int, inverse: bool = False) -> np.ndarray:
    """Rotate pairs (2i, 2i+1) of each head's rope slice, out of place.

    q: float64 [T, H, D] with D = d_nope + d_rope; per head the first d_nope
    elements pass through, the rope slice starts at d_nope. With c, s =
    cos[pos, i], sin[pos, i]:
      forward  (a, b) -> (a*c - b*s, a*s + b*c)      [ROPE]
      inverse  (a, b) -> (a*c + b*s, -a*s + b*c)     the adjoint (transpose),
               used on the gradient [BWD, sequence diagram: RoPE backward].
    """
    out = np.array(q, dtype=np.float64, copy=True)
    if d_rope == 0:
        return out
    c = cos[pos].astype(np.float64)[:, None, :]
    s = sin[pos].astype(np.float64)[:, None, :]
    a = q[:, :, d_nope + 0:d_nope + d_rope:2]
    b = q[:, :, d_nope + 1:d_nope + d_rope:2]
    if not inverse:
        out[:, :, d_nope + 0:d_nope + d_rope:2] = a * c - b * s
        out[:, :, d_nope + 1:d_nope + d_rope:2] = a * s + b * c
    else:
        out[:, :, d_nope + 0:d_nope + d_rope:2] = a * c + b * s
        out[:, :, d_nope + 1:d_nope + d_rope:2] = -a * s + b * c
    return out


def qup_forward_f64(x: np.ndarray, w: np.ndarray, bias, H: int, d_nope: int, d_rope: int,
                    pos: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Pre-quantization query in float64, [T, H, D].

    x [T, K], w [N = H*D, K] as float64 values; bias [N] or None, added to the
    projection before the rotation (the linear's own bias,
    [BWD, review comment on use_bias]).
    """
    D = d_nope + d_rope
    T = x.shape[0]
    q = x @ w.T
    if bias is not None:
        q = q + np.asarray(bias, dtype=np.float64)[None, :]
    return rope_rotate(q.reshape(T, H, D), pos, cos, sin, d_nope, d_rope)


def to_bhsd(q_thd: np.ndarray, b: np.ndarray, s: np.ndarray, shape) -> np.ndarray:
    """Scatter token-major [T, H, X] rows to [B, H, S, X] (BHSD)."""
    out = np.zeros(shape[:3] + (q_thd.shape[-1],), dtype=q_thd.dtype)
    out[b, :, s, :] = q_thd
    return out


@dataclass
class FwdResult:
    q32: np.ndarray          # float32 [T, H, D], token-major, pre-quantization
    out: np.ndarray          # BHSD: bf16 bits (uint16) or E4M3 codes (uint8)
    scales: np.ndarray | None  # BHSD [.., D/32] E8M0 bytes (MXFP8 output)


def qup_forward(x, w, *, H, d_nope, d_rope, cos, sin, fmt=FMT_BSHD, B=1, S=None,
                cu_seqlens=None, bias=None, x_scales=None, w_scales=None,
                out_dtype="mxfp8") -> FwdResult:
    """The fused forward, plain: GEMM, bias, RoPE, then BF16 or MXFP8 BHSD.

    x: bf16 tensor [T, K] or, with x_scales, E4M3 codes uint8 [T, K] with E8M0
    scales [T, K/32] (MXFP8 projection path, [FWD, description: "supports
    both 16-bit projection and mxfp8 projection"]); w likewise [N, K].
    The MXFP8 operands enter the product as code * 2^(scale - 127) exactly.
    Output is laid out BHSD, its scales [B, H, S, D/32] follow the same
    layout ([FWD, file table: "BHSD scale-transpose"]).
    """
    xf = mxfp8_dequantize(x, x_scales) if x_scales is not None else to_f64(x)
    wf = mxfp8_dequantize(w, w_scales) if w_scales is not None else to_f64(w)
    T = xf.shape[0]
    D = d_nope + d_rope
    if S is None:
        S = T // B
    pos, b, s = token_coords(fmt, T, B, S, cu_seqlens)
    bf = to_f64(bias) if bias is not None else None
    q = qup_forward_f64(xf, wf, bf, H, d_nope, d_rope, pos, cos, sin)
    q32 = q.astype(np.float32)
    shape = out_shape(fmt, T, H, D, B, S)
    if out_dtype == "bf16":
        return FwdResult(q32, to_bhsd(f32_to_bf16_bits(q32), b, s, shape), None)
    codes, scales = mxfp8_quantize_blocks(q32)
    return FwdResult(q32, to_bhsd(codes, b, s, shape), to_bhsd(scales, b, s, shape))


# ---------------------------------------------------------------------------
# Backward -- [BWD, Greptile summary and sequence diagram]: the query-output
# gradient goes through the RoPE backward to the pre-RoPE projection
# gradient, then the linear backward gives the input and weight gradients;
# [YQ, review thread]: the weight gradient is dw = dy^T x with x the linear's
# saved input; [BWD, review comment]: with use_bias the bias gradient must
# be produced.
# ---------------------------------------------------------------------------
@dataclass
class BwdResult:
    dq_pre: np.ndarray   # float64 [T, N]
    dx: np.ndarray       # float64 [T, K]
    dw: np.ndarray       # float64 [N, K]
    db: np.ndarray       # float64 [N]


def qup_backward(dq, x, w, *, H, d_nope, d_rope, cos, sin, fmt=FMT_BSHD, B=1, S=None,
                 cu_seqlens=None) -> BwdResult:
    """dq [T, H, D] (token-major), saved input x [T, K], weight w [N, K].

    dq_pre = inverse RoPE of dq;  dX = dq_pre W;  dW = dq_pre^T X;
    db = sum over tokens of dq_pre.
    """
    dqf = to_f64(dq)
    xf = to_f64(x)
    wf = to_f64(w)
    T = dqf.shape[0]
    if S is None:
        S = T // B
    pos, _, _ = token_coords(fmt, T, B, S, cu_seqlens)
    dq_pre = rope_rotate(dqf.reshape(T, H, d_nope + d_rope), pos, cos, sin,
                         d_nope, d_rope, inverse=True).reshape(T, -1)
    return BwdResult(dq_pre, dq_pre @ wf, dq_pre.T @ xf, dq_pre.sum(axis=0))


# ---------------------------------------------------------------------------
# MXFP8 backward -- the "mxfp8 projection" of [FWD, description] carried into
# the linear backward that [BWD, Greptile summary] routes the pre-RoPE
# gradient through. The pages name no further detail; the reading taken is
# the MXFP8 training recipe of the library the pages extend: every operand of
# a product is quantized along that product's reduction axis [OCP-MX], from
# the stored bf16 dq_pre and the bf16 x and W:
#   dX = deq(Q_rows(dq_pre)) . deq(Q_cols(W))     (reduction over n)
#   dW = deq(Q_cols(dq_pre))^T . deq(Q_cols(x))   (reduction over tokens)
#   db = sum over tokens of dq_pre (unquantized, as in the bf16 backward).
# Q_rows blocks 32 consecutive elements of a row, Q_cols 32 consecutive rows
# of a column; the token axis is zero-padded to a multiple of 32.
# ---------------------------------------------------------------------------
def mxfp8_quantize_columns(v: np.ndarray):
    """MXFP8-quantize along the first axis: blocks of 32 consecutive rows of
    each column [OCP-MX], rows zero-padded to a multiple of 32. The result is
    returned transposed, the blocked axis contiguous: codes uint8 [C, Rp] and
    scales uint8 [C, Rp/32]."""
    v32 = np.asarray(v, dtype=np.float32)
    R, C = v32.shape
    Rp = -(-R // 32) * 32
    vp = np.zeros((Rp, C), dtype=np.float32)
    vp[:R] = v32
    return mxfp8_quantize_blocks(np.ascontiguousarray(vp.T))


@dataclass
class MxBwdResult:
    dq_pre: np.ndarray       # float64 [T, N], before the bf16 store
    dq_pre_bf16: np.ndarray  # uint16 [T, N], the stored copy the operands come from
    dx: np.ndarray           # float64 [T, K]
    dw: np.ndarray           # float64 [N, K]
    db: np.ndarray           # float64 [N]
    dq_rows: tuple           # (codes [T, N], scales [T, N/32])
    dq_cols_t: tuple         # (codes [N, Tp], scales [N, Tp/32])
    w_cols_t: tuple          # (codes [K, N], scales [K, N/32])
    x_cols_t: tuple          # (codes [K, Tp], scales [K, Tp/32])


def qup_backward_mxfp8(dq, x, w, *, H, d_nope, d_rope, cos, sin, fmt=FMT_BSHD, B=1, S=None,
                       cu_seqlens=None) -> MxBwdResult:
    """The backward with MXFP8 operands (see the section comment above).

    dq_pre is the inverse RoPE of dq, stored as bf16 (rounded once to float32,
    the kernel's precision, then to bf16); both products read that copy.
    """
    r = qup_backward(dq, x, w, H=H, d_nope=d_nope, d_rope=d_rope, cos=cos, sin=sin, fmt=fmt,
                     B=B, S=S, cu_seqlens=cu_seqlens)
    bits = f32_to_bf16_bits(r.dq_pre.astype(np.float32))
    dqp = bf16_bits_to_f64(bits)
    rows = mxfp8_quantize_blocks(dqp)
    dq_t = mxfp8_quantize_columns(dqp)
    w_t = mxfp8_quantize_columns(to_f64(w))
    x_t = mxfp8_quantize_columns(to_f64(x))
    dx = mxfp8_dequantize(*rows) @ mxfp8_dequantize(*w_t).T
    dw = mxfp8_dequantize(*dq_t) @ mxfp8_dequantize(*x_t).T
    return MxBwdResult(r.dq_pre, bits, dx, dw, r.db, rows, dq_t, w_t, x_t)


# ---------------------------------------------------------------------------
# KV side -- [FWD, flowchart]: the key and the value each go through MXFP8
# quantization and the same BHSD scale layout as the query before the fused
# attention; [YQ, Solution]: the KV rotary kernel writes fresh key and value
# outputs (nothing in place). The pages do not spell out the KV rotary
# itself; the reading taken is the MLA one the [YQ] page works on: per
# token, the up-projected kv row holds per head [k_nope | v], and one rope
# slice k_pe per token, shared by every head, is rotated with the query's
# table and placed after each head's k_nope:
#   key[t, h]   = [k_nope[t, h] | rope(k_pe[t], pos_t)]
#   value[t, h] = v[t, h]
# The rotated values are float32 (from bf16 inputs) and quantized without
# an intermediate 16-bit rounding, like the query.
# ---------------------------------------------------------------------------
@dataclass
class KvResult:
    key64: np.ndarray            # float64 [T, H, d_nope + d_rope], token-major, exact
    key32: np.ndarray            # float32 [T, H, d_nope + d_rope], token-major
    value32: np.ndarray          # float32 [T, H, d_v]
    key: np.ndarray              # BHSD bf16 bits or E4M3 codes
    key_scales: np.ndarray | None
    value: np.ndarray
    value_scales: np.ndarray | None


def kv_rope(kv, k_pe, *, H, d_nope, d_rope, d_v, cos, sin, fmt=FMT_BSHD, B=1, S=None,
            cu_seqlens=None, out_dtype="mxfp8") -> KvResult:
    """kv: bf16 [T, H, d_nope + d_v]; k_pe: bf16 [T, d_rope]."""
    kvf = to_f64(kv)
    pe = to_f64(k_pe)
    T = kvf.shape[0]
    if S is None:
        S = T // B
    pos, b, s = token_coords(fmt, T, B, S, cu_seqlens)
    rot = rope_rotate(pe.reshape(T, 1, d_rope), pos, cos, sin, 0, d_rope)[:, 0, :]
    key = np.concatenate([kvf[:, :, :d_nope], np.broadcast_to(rot[:, None, :], (T, H, d_rope))], axis=2)
    val = kvf[:, :, d_nope:d_nope + d_v]
    k32, v32 = key.astype(np.float32), val.astype(np.float32)
    outs = []
    for a32, D in ((k32, d_nope + d_rope), (v32, d_v)):
        shape = out_shape(fmt, T, H, D, B, S)
        if out_dtype == "bf16":
            outs += [to_bhsd(f32_to_bf16_bits(a32), b, s, shape), None]
        else:
            codes, scales = mxfp8_quantize_blocks(a32)
            outs += [to_bhsd(codes, b, s, shape), to_bhsd(scales, b, s, shape)]
    return KvResult(key, k32, v32, *outs)
