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
                       w_scales=None, abs_w=None):
    """Oracle pre-quantization values (float64) and their float32 error bound
    for the token rows `rows` of X. pos: positions of every token row. x and
    w may be given already as float64 arrays (then abs_w, |w|, may be too)."""
    xf = o.mxfp8_dequantize(x, x_scales) if x_scales is not None else o.to_f64(x)
    wf = o.mxfp8_dequantize(w, w_scales) if w_scales is not None else o.to_f64(w)
    xs = xf[rows]
    K = xs.shape[1]
    D = d_nope + d_rope
    bf = o.to_f64(bias) if bias is not None else None
    q64 = o.qup_forward_f64(xs, wf, bf, H, d_nope, d_rope, pos[rows], cos, sin)
    gamma = K * U / (1 - K * U)
    mag = np.abs(xs) @ (abs_w if abs_w is not None else np.abs(wf)).T
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


def mx_stats(g_codes, g_scales, q64, bound):
    """Counts of the MXFP8 comparison without any assertion (summable over
    chunks with merge_stats). g_codes [..., D] uint8, g_scales [..., D/32];
    q64 / bound [..., D] float64 (oracle value before its float32 rounding,
    and its float32 error bound).

    scale_adjudicated: blocks whose scale differs by one where the oracle's
    amax lies within the bound of the power of two between the two exponents;
    scale_unexplained: every other scale difference. Code flips are counted
    outside mismatched blocks; flip_gt1 counts codes more than one step
    apart, flip_unexplained one-step flips beyond the bound of their rounding
    boundary; max_dist_over_bound is the largest distance to that boundary
    over the bound among the flips."""
    r_codes, r_scales = o.mxfp8_quantize_blocks(q64.astype(np.float32))
    shp = q64.shape[:-1] + (q64.shape[-1] // 32, 32)
    smis = g_scales != r_scales
    adjudicated = np.zeros(shp[:-1], bool)
    unexplained = 0
    if smis.any():
        blk64 = np.abs(q64.reshape(shp))
        bnd = bound.reshape(shp)
        for i in np.argwhere(smis):
            i = tuple(i)
            eg, er = int(g_scales[i]) - 127, int(r_scales[i]) - 127
            j = blk64[i].argmax()
            edge = 2.0 ** (max(eg, er) + 8)
            if abs(eg - er) == 1 and abs(blk64[i][j] - edge) <= bnd[i][j] + 1e-300:
                adjudicated[i] = True
            else:
                unexplained += 1
    skip = np.repeat(smis, 32, axis=-1).reshape(q64.shape)
    cmis = (g_codes != r_codes) & ~skip
    n_mis = int(cmis.sum())
    gt1 = unexpl = 0
    worst = worst_gt1 = 0.0
    if n_mis:
        gc, rc = g_codes[cmis].astype(np.int64), r_codes[cmis].astype(np.int64)
        # codes as signed steps on the E4M3 number line (+0 and -0 are both step 0,
        # and differ only by the sign of a value that rounds to zero)
        step = lambda c: np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
        one = np.abs(step(gc) - step(rc)) <= 1
        gt1 = int((~one).sum())
        E = np.repeat(r_scales.astype(np.int64) - 127, 32, axis=-1).reshape(q64.shape)[cmis]
        mid = (o.e4m3_decode(gc) + o.e4m3_decode(rc)) / 2 * np.ldexp(1.0, E)
        ratio = np.abs(q64[cmis] - mid) / bound[cmis]
        unexpl = int(((ratio > 1) & one).sum())
        worst = float(ratio[one].max()) if one.any() else 0.0
        if gt1:
            # how far the GPU's decoded value lies from the oracle's, in bounds
            gval = o.e4m3_decode(gc) * np.ldexp(1.0, E)
            worst_gt1 = float((np.abs(gval - q64[cmis]) / bound[cmis])[~one].max())
    return {"blocks": int(np.prod(shp[:-1])), "elements": int(g_codes.size),
            "scale_adjudicated": int(adjudicated.sum()), "scale_unexplained": unexplained,
            "code_flips": n_mis, "flip_gt1": gt1, "flip_unexplained": unexpl,
            "max_dist_over_bound": worst, "max_gt1_err_over_bound": worst_gt1}


def merge_stats(parts):
    out = {}
    for st in parts:
        for k, v in st.items():
            out[k] = max(out.get(k, 0.0), v) if k.startswith("max_") else out.get(k, 0) + v
    return out


def assert_mx_bar(st, what: str = "mxfp8"):
    """The MXFP8 parity bar on merged statistics. Scales bit-exact, except
    a scale one apart at a power-of-two boundary within the float32 bound,
    at most one such block per million (and at least one allowed); codes
    bit-exact except at most 0.1 % one step apart, every flip explained by
    the float32 bound, and each adjudicated block's 32 codes counted against
    that 0.1 %."""
    assert st["scale_unexplained"] == 0, f"{what}: {st['scale_unexplained']} unexplained scale mismatches"
    assert st["scale_adjudicated"] <= max(1, st["blocks"] // 10 ** 6), f"{what}: {st}"
    frac = (st["code_flips"] + 32 * st["scale_adjudicated"]) / st["elements"]
    assert frac <= 1e-3, f"{what}: code mismatches {frac:.2e} of the elements"
    assert st["flip_gt1"] == 0, f"{what}: a code differs by more than one step"
    assert st["flip_unexplained"] == 0, (
        f"{what}: code flip not explained by accumulation order "
        f"(max dist/bound {st['max_dist_over_bound']:.2f})")
    st["code_mismatch_frac"] = frac
    return st


def check_mx(g_codes, g_scales, q64, bound, what: str = "mxfp8"):
    return assert_mx_bar(mx_stats(g_codes, g_scales, q64, bound), what)


def parallel_chunks(fn, n, chunk, workers=16):
    """fn(lo, hi) over [0, n) in chunks on a thread pool (numpy releases the
    GIL in the heavy steps); BLAS limited to one thread per worker."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    spans = [(lo, min(lo + chunk, n)) for lo in range(0, n, chunk)]
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(lambda sp: fn(*sp), spans))


# Guard bands: an output allocated inside sentinel-filled margins, so that a
# write outside its extent is caught.
GUARD_BYTES = 1 << 16
GUARD_FILL = 0xA5


class Guarded:
    def __init__(self, shape, dtype, fill_bits=None, device="cuda"):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * esz
        self.raw = torch.full((GUARD_BYTES + n + GUARD_BYTES,), GUARD_FILL, dtype=torch.uint8, device=device)
        inner = self.raw[GUARD_BYTES:GUARD_BYTES + n]
        if fill_bits is not None:
            inner.fill_(fill_bits)
        self.t = inner.view(dtype).view(shape)

    def check(self, what="output"):
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[self.raw.numel() - GUARD_BYTES:]
        assert bool((head == GUARD_FILL).all()), f"{what}: write before the start of the buffer"
        assert bool((tail == GUARD_FILL).all()), f"{what}: write past the end of the buffer"


def frob_rel(g: np.ndarray, r: np.ndarray) -> float:
    return float(np.linalg.norm(g - r) / np.linalg.norm(r))


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()
