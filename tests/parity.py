"""Comparison rules between the HIP path and the CPU oracle.

BF16 outputs : max |g - r| / max(|r|, 1e-3 RMS(r)) <= 2e-2 and
               mean |g - r| <= 1e-3 RMS(r), on bf16-decoded values.
MXFP8 outputs: E8M0 scales bit-exact, E4M3 codes bit-exact except at most
               0.1 % of elements one code apart. A difference is accepted only
               where float32 accumulation order can explain it: the oracle's
               float64 value lies within the float32 forward-error bound of
               the rounding boundary between the two codes (or, for a scale,
               of the power of two that separates the two exponents).
Gradients    : relative Frobenius error <= 1e-2.

The error bound of a float32 dot product of length K summed in any order is
gamma_K * sum_k |x_k w_k|, gamma_K = K u / (1 - K u), u = 2^-24 (Higham,
Accuracy and Stability of Numerical Algorithms, section 3.1); the rotation
adds at most a few roundings of its products, and everything is doubled.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as o

U = 2.0 ** -24


def fwd_reference_rows(x, w, bias, rows, *, H, d_nope, d_rope, cos, sin, pos, x_scales=None,
                       w_scales=None):
    """Oracle pre-quantization values (float64) and their float32 error bound
    for the token rows `rows` of X. pos: positions of every token row."""
    xf = o.mxfp8_dequantize(x, x_scales) if x_scales is not None else o.to_f64(x)
    wf = o.mxfp8_dequantize(w, w_scales) if w_scales is not None else o.to_f64(w)
    xs = xf[rows]
    K = xs.shape[1]
    D = d_nope + d_rope
    bf = o.to_f64(bias) if bias is not None else None
    q64 = o.qup_forward_f64(xs, wf, bf, H, d_nope, d_rope, pos[rows], cos, sin)
    gamma = K * U / (1 - K * U)
    mag = np.abs(xs) @ np.abs(wf).T
    lin = xs @ wf.T
    if bf is not None:
        mag = mag + np.abs(bf)[None, :]
        lin = lin + bf[None, :]
    B = (gamma * mag + 2 * U * np.abs(lin)).reshape(len(rows), H, D)
    lin = lin.reshape(len(rows), H, D)
    if d_rope:
        c = np.abs(cos[pos[rows]].astype(np.float64))[:, None, :]
        s = np.abs(sin[pos[rows]].astype(np.float64))[:, None, :]
        a, b = lin[..., d_nope::2], lin[..., d_nope + 1::2]
        Ba, Bb = B[..., d_nope::2].copy(), B[..., d_nope + 1::2].copy()
        rot = 4 * U * (np.abs(a) * c + np.abs(b) * s) + U * (np.abs(a) + np.abs(b))
        B[..., d_nope::2] = c * Ba + s * Bb + rot
        B[..., d_nope + 1::2] = s * Ba + c * Bb + rot
    return q64, 2.0 * B + U * np.abs(q64)


def check_bf16(g_bits: np.ndarray, r_bits: np.ndarray, what: str = "bf16"):
    g = o.bf16_bits_to_f64(g_bits)
    r = o.bf16_bits_to_f64(r_bits)
    assert np.isfinite(g).all(), f"{what}: non-finite values in the GPU output"
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    rel = err / np.maximum(np.abs(r), 1e-3 * rms)
    assert rel.max() <= 2e-2, f"{what}: max rel {rel.max():.3e} at {np.unravel_index(rel.argmax(), rel.shape)}"
    assert err.mean() <= 1e-3 * rms, f"{what}: mean abs {err.mean():.3e} vs RMS {rms:.3e}"
    return {"max_rel": float(rel.max()), "mean_abs_over_rms": float(err.mean() / rms),
            "exact_frac": float((g_bits == r_bits).mean())}


def check_mx(g_codes, g_scales, q64, bound, what: str = "mxfp8"):
    """g_codes [..., D] uint8, g_scales [..., D/32]; q64/bound [..., D] float64
    (oracle value before its float32 rounding, and its error bound)."""
    r_codes, r_scales = o.mxfp8_quantize_blocks(q64.astype(np.float32))
    shp = q64.shape[:-1] + (q64.shape[-1] // 32, 32)
    # scales
    smis = g_scales != r_scales
    excluded = np.zeros(shp[:-1], bool)
    if smis.any():
        idx = np.argwhere(smis)
        blk64 = np.abs(q64.reshape(shp))
        bnd = bound.reshape(shp)
        for i in idx:
            i = tuple(i)
            eg, er = int(g_scales[i]) - 127, int(r_scales[i]) - 127
            amax = blk64[i].max()
            j = blk64[i].argmax()
            edge = 2.0 ** (max(eg, er) + 8)
            ok = abs(eg - er) == 1 and abs(amax - edge) <= bnd[i][j] + 1e-300
            assert ok, f"{what}: scale mismatch at block {i}: gpu {eg} oracle {er}, amax {amax!r}"
            excluded[i] = True
    # codes
    cmis = (g_codes != r_codes) & ~np.repeat(excluded, 32, axis=-1).reshape(q64.shape)
    n_mis = int(cmis.sum())
    frac = n_mis / g_codes.size
    assert frac <= 1e-3, f"{what}: {n_mis} code mismatches ({frac:.2e})"
    if n_mis:
        gc, rc = g_codes[cmis].astype(np.int64), r_codes[cmis].astype(np.int64)
        # codes as signed steps on the E4M3 number line (+0 and -0 are both step 0,
        # and differ only by the sign of a value that rounds to zero)
        step = lambda c: np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
        assert (np.abs(step(gc) - step(rc)) <= 1).all(), f"{what}: code differs by more than 1 step"
        E = np.repeat(r_scales.astype(np.int64) - 127, 32, axis=-1).reshape(q64.shape)[cmis]
        mid = (o.e4m3_decode(gc) + o.e4m3_decode(rc)) / 2 * np.ldexp(1.0, E)
        dist = np.abs(q64[cmis] - mid)
        assert (dist <= bound[cmis]).all(), (
            f"{what}: code flip not explained by accumulation order "
            f"(max dist/bound {np.max(dist / bound[cmis]):.2f})")
    return {"scale_mismatch_blocks": int(excluded.sum()), "code_mismatches": n_mis,
            "code_mismatch_frac": frac}


def frob_rel(g: np.ndarray, r: np.ndarray) -> float:
    return float(np.linalg.norm(g - r) / np.linalg.norm(r))


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()
