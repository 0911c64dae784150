"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked values of the formats' definitions (tests/golden/, each file cites
its source), library special cases (torch's float8 cast), closed forms of the
rotation, invariants, and brute force on tiny inputs. CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as o
from mla_up_projection_amd import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line


# ---------------------------------------------------------------- E4M3 ----
def test_e4m3_decode_table_matches_torch_float8():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = o.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # Only S.1111.111 is NaN; 448 is the largest finite value.
    assert [c for c in range(256) if math.isnan(got[c])] == [0x7F, 0xFF]
    assert np.nanmax(got) == 448.0


def test_e4m3_hand_worked_values():
    for row in _rows("e4m3_values.txt"):
        val, code = row.split()[:2]
        got = int(o.e4m3_encode(np.array([float(val)]))[0])
        assert got == int(code, 16), (val, hex(got), code)


@pytest.mark.parametrize("E", [-127, -8, 0, 7])
def test_e4m3_exhaustive_bf16_against_torch_cast(E):
    """All 65536 bf16 patterns times 2^-E: the oracle's nearest-code search
    equals torch's round-to-nearest-even cast after clamping to +-448."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = o.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    y = np.ldexp(v[fin], -E)
    got = o.e4m3_encode(y)
    yc = np.clip(y, -448.0, 448.0)
    # float32 holds every clamped value exactly except those far below the
    # smallest E4M3 subnormal, which round to (signed) zero on both sides.
    ref = torch.from_numpy(yc.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


# ---------------------------------------------------------------- E8M0 ----
def test_e8m0_hand_worked_scales():
    for row in _rows("e8m0_scales.txt"):
        amax, byte = row.split()[:2]
        a = np.float32(float(amax))
        blk = np.zeros((1, 32), np.float32)
        blk[0, 5] = a
        blk[0, 6] = -a / np.float32(4)
        _, sc = o.mxfp8_quantize_blocks(blk)
        assert int(sc[0, 0]) == int(byte, 16), (amax, hex(int(sc[0, 0])), byte)


def test_mx_hand_worked_blocks():
    blocks, cur = {}, None
    for row in _rows("mx_blocks.txt"):
        f = row.split()
        if f[0] == "block":
            cur = blocks.setdefault(f[1], {"v": np.zeros(32, np.float32),
                                           "c": np.zeros(32, np.uint8)})
        elif f[0] == "scale":
            cur["s"] = int(f[1], 16)
        else:
            i = int(f[0])
            cur["v"][i] = np.float32(float(f[1]))
            cur["c"][i] = int(f[2], 16)
    assert len(blocks) == 4
    for name, b in blocks.items():
        codes, sc = o.mxfp8_quantize_blocks(b["v"][None, :])
        assert int(sc[0, 0]) == b["s"], name
        assert np.array_equal(codes[0], b["c"]), (name, codes[0])


def test_mx_nonfinite_block():
    v = np.ones((2, 64), np.float32)
    v[0, 3] = np.nan
    v[1, 40] = np.inf
    codes, sc = o.mxfp8_quantize_blocks(v)
    assert sc[0, 0] == 0xFF and sc[0, 1] == 0x77
    assert sc[1, 0] == 0x77 and sc[1, 1] == 0xFF
    assert (codes[0, :32] == 0x7F).all() and (codes[1, 32:] == 0x7F).all()
    assert (codes[0, 32:] == 0x78).all()


def _e4m3_ulp(y):
    a = np.abs(y)
    e = np.where(a >= 2.0 ** -6, o.floor_log2(np.where(a > 0, a, 1.0)), -6)
    return np.ldexp(1.0, e - 3)


def test_mx_quantizer_invariants_random():
    """dequant(quant(v)) within half an E4M3 ulp (scaled), saturation exact,
    and 256 <= amax * 2^-E < 512 for every block with an unclamped scale."""
    rng = np.random.default_rng(11)
    v = (rng.standard_normal((512, 192)) * 0.784).astype(np.float32)
    v[::7] *= np.float32(1e-30)      # deep small range: scale near its clamp
    v[::11] *= np.float32(1e20)
    codes, sc = o.mxfp8_quantize_blocks(v)
    E = sc.astype(np.int64) - 127
    blk = v.astype(np.float64).reshape(512, 6, 32)
    amax = np.abs(blk).max(-1)
    r = np.ldexp(amax, -E)
    unclamped = E > -127
    assert ((r[unclamped] >= 256) & (r[unclamped] < 512)).all()
    y = np.ldexp(blk, -E[..., None])
    deq = o.mxfp8_dequantize(codes, sc).reshape(512, 6, 32)
    sat = np.abs(y) > 464
    assert np.array_equal(np.abs(np.ldexp(deq, -E[..., None]))[sat], np.full(sat.sum(), 448.0))
    err = np.abs(np.ldexp(deq, -E[..., None]) - y)
    assert (err[~sat] <= 0.5 * _e4m3_ulp(y[~sat])).all()
    assert sat.any()


def test_mx_dequantize_values():
    codes = np.zeros((1, 32), np.uint8)
    codes[0, :3] = [0x38, 0x7E, 0xB8]
    assert o.mxfp8_dequantize(codes, np.array([[0x7F]], np.uint8))[0, :3].tolist() == [1.0, 448.0, -1.0]
    assert o.mxfp8_dequantize(codes, np.array([[0x80]], np.uint8))[0, :3].tolist() == [2.0, 896.0, -2.0]
    assert o.mxfp8_dequantize(codes, np.array([[0x77]], np.uint8))[0, 1] == 1.75


def test_bf16_roundtrip_values():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7, -2.5, 3.0e38], np.float32)
    got = o.bf16_bits_to_f64(o.f32_to_bf16_bits(v))
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6).
    assert got.tolist()[:5] == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5]
    assert abs(got[5] / 3.0e38 - 1) < 2 ** -8


# ---------------------------------------------------------------- RoPE ----
def test_theta_closed_forms():
    for row in _rows("rope_values.txt"):
        f = row.split()
        if f[0] == "theta":
            d, i, val = int(f[1]), int(f[2]), float(f[3])
            assert o.rope_theta(d, 10000.0)[i] == pytest.approx(val, rel=1e-14)


def test_table_closed_forms():
    for row in _rows("rope_values.txt"):
        f = row.split()
        if f[0] == "table":
            d, p, i, c, s = int(f[1]), int(f[2]), int(f[3]), float(f[4]), float(f[5])
            cos, sin = o.rope_table(p + 1, d, 10000.0)
            assert cos.dtype == np.float32
            assert abs(cos[p, i] - c) <= 6e-8 and abs(sin[p, i] - s) <= 6e-8, (d, p, i)


def _rand_q(T, H, D, seed=0):
    return np.random.default_rng(seed).standard_normal((T, H, D))


def test_rope_direction_counterclockwise():
    cos, sin = o.rope_table(2, 16, 10000.0)
    q = np.zeros((1, 1, 32))
    q[0, 0, 16] = 1.0          # pair 0 of the rope slice = (1, 0)
    q[0, 0, 19] = 1.0          # pair 1 = (0, 1)
    out = o.rope_rotate(q, np.array([1]), cos, sin, 16, 16)
    assert out[0, 0, 16] == pytest.approx(0.5403023058681398, abs=6e-8)
    assert out[0, 0, 17] == pytest.approx(0.8414709848078965, abs=6e-8)
    th1 = 0.31622776601683794
    assert out[0, 0, 18] == pytest.approx(-math.sin(th1), abs=6e-8)
    assert out[0, 0, 19] == pytest.approx(math.cos(th1), abs=6e-8)
    assert np.array_equal(out[0, 0, :16], q[0, 0, :16])


def test_rope_position_zero_is_identity():
    cos, sin = o.rope_table(4, 64, 10000.0)
    q = _rand_q(5, 3, 192)
    out = o.rope_rotate(q, np.zeros(5, np.int64), cos, sin, 128, 64)
    assert np.array_equal(out, q)


def test_rope_inverse_after_forward_and_norm():
    cos, sin = o.rope_table(4096, 64, 10000.0)
    q = _rand_q(64, 4, 192)
    pos = np.random.default_rng(1).integers(0, 4096, 64)
    f = o.rope_rotate(q, pos, cos, sin, 128, 64)
    back = o.rope_rotate(f, pos, cos, sin, 128, 64, inverse=True)
    # the float32 table has cos^2 + sin^2 = 1 within ~1.2e-7
    assert np.max(np.abs(back - q)) <= 3e-7 * np.max(np.abs(q))
    assert np.array_equal(f[..., :128], q[..., :128])
    n0 = np.linalg.norm(q[..., 128:], axis=-1)
    n1 = np.linalg.norm(f[..., 128:], axis=-1)
    assert np.max(np.abs(n1 / n0 - 1)) < 2e-7


def test_rope_composition_and_relative_position():
    cos, sin = o.rope_table(300, 64, 10000.0)
    q = _rand_q(1, 1, 64, 3)
    k = _rand_q(1, 1, 64, 4)
    a, b = 37, 121
    ra = o.rope_rotate(q, np.array([a]), cos, sin, 0, 64)
    rab = o.rope_rotate(ra, np.array([b]), cos, sin, 0, 64)
    r_sum = o.rope_rotate(q, np.array([a + b]), cos, sin, 0, 64)
    assert np.max(np.abs(rab - r_sum)) < 2e-6
    dots = []
    for m in (0, 50, 170):
        qm = o.rope_rotate(q, np.array([m + 20]), cos, sin, 0, 64)
        kn = o.rope_rotate(k, np.array([m + 5]), cos, sin, 0, 64)
        dots.append(float((qm * kn).sum()))
    assert max(dots) - min(dots) < 1e-5 * max(abs(d) for d in dots)


# ---------------------------------------------------------------- YaRN ----
def _yarn_golden():
    return {r.split()[0]: float(r.split()[1]) for r in _rows("yarn_c4.txt")}


def test_yarn_correction_range_hand_worked():
    g = _yarn_golden()
    assert o.yarn_correction_dim(32, 64, 1e4, 4096) == pytest.approx(g["corr_fast"], abs=1e-3)
    assert o.yarn_correction_dim(1, 64, 1e4, 4096) == pytest.approx(g["corr_slow"], abs=1e-3)
    y = o.Yarn(40.0, 4096, 32.0, 1.0, 1.0)
    r = o.yarn_ramp(64, 1e4, y)
    low, high = int(g["low"]), int(g["high"])
    assert (r[:low + 1] == 0).all() and (r[high:] == 1).all()
    steps = np.diff(r[low:high + 1])
    assert np.allclose(steps, 1.0 / (high - low), rtol=0, atol=1e-15)
    ratio = o.yarn_theta(64, 1e4, y) / o.rope_theta(64, 1e4)
    assert np.allclose(ratio[:low + 1], 1.0, rtol=0, atol=1e-15)
    assert np.allclose(ratio[high:], 1.0 / 40.0, rtol=1e-15)


def test_yarn_factor_one_is_plain_rope():
    c0, s0 = o.rope_table(512, 64, 1e4)
    c1, s1 = o.rope_table(512, 64, 1e4, o.Yarn(1.0, 4096, 32.0, 1.0, 1.0))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_yarn_interpolated_pairs_equal_rope_at_scaled_position():
    # beta_fast 600 -> corr 0.07 -> low 0; beta_slow 366 -> corr 0.50 -> high 1:
    # pair 0 kept, every other pair divided by the factor (pure interpolation).
    y = o.Yarn(4.0, 4096, 600.0, 366.0, 1.0)
    r = o.yarn_ramp(16, 1e4, y)
    assert r[0] == 0 and (r[1:] == 1).all()
    cy, sy = o.rope_table(4 * 50 + 1, 16, 1e4, y)
    cp, sp = o.rope_table(51, 16, 1e4)
    p = np.arange(51)
    assert np.max(np.abs(cy[4 * p, 1:] - cp[p, 1:])) <= 1.2e-7
    assert np.max(np.abs(sy[4 * p, 1:] - sp[p, 1:])) <= 1.2e-7
    assert np.array_equal(cy[:51, 0], cp[:, 0])


def test_yarn_mscale_multiplies_table():
    c1, s1 = o.rope_table(64, 64, 1e4, o.Yarn(40.0, 4096, 32.0, 1.0, 1.0))
    c2, s2 = o.rope_table(64, 64, 1e4, o.Yarn(40.0, 4096, 32.0, 1.0, 2.0))
    assert np.array_equal(c2, 2 * c1) and np.array_equal(s2, 2 * s1)


# ----------------------------------------------------------- positions ----
def test_token_coords_hand_worked():
    fmts = {"BSHD": o.FMT_BSHD, "SBHD": o.FMT_SBHD, "THD": o.FMT_THD}
    for row in _rows("token_positions.txt"):
        head, pos, b, s = [p.split() for p in row.split("|")]
        fmt, B, S, cu = head[0], int(head[1]), int(head[2]), head[3]
        cu = None if cu == "-" else [int(c) for c in cu.split(",")]
        T = B * S if cu is None else cu[-1]
        gp, gb, gs = o.token_coords(fmts[fmt], T, B, S, cu)
        assert gp.tolist() == [int(x) for x in pos], fmt
        assert gb.tolist() == [int(x) for x in b], fmt
        assert gs.tolist() == [int(x) for x in s], fmt


def test_thd_lengths_recipe():
    w = syn.workload("thd_yarn_fwd")
    assert sum(w.lengths) == 16384
    assert all(512 <= n <= 4096 for n in w.lengths[:-1]) and 1 <= w.lengths[-1] <= 4096


# ------------------------------------------------------ forward: GEMM -----
def test_forward_one_hot_selects_weight_columns():
    """Row t of X is e_{k(t)}; at position 0 the query is W[:, k(t)]: catches a
    transposed operand or a wrong head/element placement."""
    T, K, H, dn, dr = 6, 64, 2, 16, 16
    D = dn + dr
    ks = [0, 5, 17, 63, 32, 9]
    x = torch.zeros(T, K, dtype=torch.bfloat16)
    for t, k in enumerate(ks):
        x[t, k] = 1.0
    w = syn.normal_bf16((H * D, K), 1.0, 5)
    cos, sin = o.rope_table(1, dr, 1e4)
    res = o.qup_forward(x, w, H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin,
                        fmt=o.FMT_BSHD, B=T, S=1, out_dtype="bf16")
    wf = o.to_f64(w)
    for t, k in enumerate(ks):
        assert np.array_equal(res.q32[t].reshape(-1), wf[:, k].astype(np.float32))
        for h in range(H):
            got = o.bf16_bits_to_f64(res.out[t, h, 0])
            assert np.array_equal(got, wf[h * D:(h + 1) * D, k])


def test_forward_bhsd_placement_exact():
    """q[t, n] = (t+1) * n / 4096 exactly, then checked at [b, h, s, d] for
    b-major and s-major token orders."""
    B, S, H, D, K = 2, 32, 2, 32, 32
    T = B * S
    x = torch.zeros(T, K, dtype=torch.float32)
    x[:, 0] = (torch.arange(T) + 1).float() / 64
    w = torch.zeros(H * D, K, dtype=torch.float32)
    w[:, 0] = torch.arange(H * D).float() / 64
    x, w = x.to(torch.bfloat16), w.to(torch.bfloat16)
    cos, sin = o.rope_table(S, 0, 1e4)
    for fmt in (o.FMT_BSHD, o.FMT_SBHD):
        res = o.qup_forward(x, w, H=H, d_nope=D, d_rope=0, cos=cos, sin=sin,
                            fmt=fmt, B=B, S=S, out_dtype="bf16")
        assert res.out.shape == (B, H, S, D)
        for b in range(B):
            for s in range(S):
                t = b * S + s if fmt == o.FMT_BSHD else s * B + b
                for h in range(H):
                    got = o.bf16_bits_to_f64(res.out[b, h, s])
                    want = (t + 1) * (h * D + np.arange(D)) / 4096.0
                    assert np.array_equal(res.q32[t, h], want.astype(np.float32))
                    want16 = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).double().numpy()
                    assert np.array_equal(got, want16)


def test_forward_brute_force_tiny():
    """Scalar loops over a tiny case: sum over k, bias, then the rotation of
    each pair with math.cos / math.sin of pos * base^(-2i/d)."""
    T, K, H, dn, dr = 3, 32, 2, 16, 16
    D = dn + dr
    x = syn.normal_bf16((T, K), 1.0, 21)
    w = syn.normal_bf16((H * D, K), 0.2, 22)
    bias = syn.normal_bf16((H * D,), 0.5, 23)
    cos, sin = o.rope_table(8, dr, 1e4)
    pos = [0, 5, 7]
    xf, wf, bf = o.to_f64(x), o.to_f64(w), o.to_f64(bias)
    got = o.qup_forward_f64(xf, wf, bf, H, dn, dr, np.array(pos), cos, sin)
    for t in range(T):
        for h in range(H):
            lin = [sum(xf[t, k] * wf[h * D + d, k] for k in range(K)) + bf[h * D + d] for d in range(D)]
            for d in range(dn):
                assert got[t, h, d] == pytest.approx(lin[d], abs=1e-12)
            for i in range(dr // 2):
                ang = pos[t] * 10000.0 ** (-2.0 * i / dr)
                c, s = float(np.float32(math.cos(ang))), float(np.float32(math.sin(ang)))
                a, b = lin[dn + 2 * i], lin[dn + 2 * i + 1]
                assert got[t, h, dn + 2 * i] == pytest.approx(a * c - b * s, abs=1e-12)
                assert got[t, h, dn + 2 * i + 1] == pytest.approx(a * s + b * c, abs=1e-12)


def test_forward_without_rope_is_plain_gemm_integers():
    # small integers: every product and sum is exact in any precision
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.integers(-3, 4, (16, 64)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.integers(-3, 4, (64, 64)).astype(np.float32)).to(torch.bfloat16)
    cos, sin = o.rope_table(16, 0, 1e4)
    res = o.qup_forward(x, w, H=2, d_nope=32, d_rope=0, cos=cos, sin=sin, fmt=o.FMT_BSHD,
                        B=1, S=16, out_dtype="bf16")
    xi = x.float().numpy().astype(np.int64)
    wi = w.float().numpy().astype(np.int64)
    ref = (xi @ wi.T).reshape(16, 2, 32)
    assert np.array_equal(res.q32.astype(np.int64), ref)


def test_mxfp8_projection_operands_enter_exactly():
    """X and W given as MXFP8 codes + scales: the product sees code * 2^(s-127)."""
    T, K, H, D = 4, 64, 1, 32
    xc = np.full((T, K), 0x38, np.uint8)            # 1.0
    xs = np.full((T, K // 32), 0x7F, np.uint8)      # * 2^0
    xs[:, 1] = 0x80                                 # second K-block * 2
    wc = np.full((H * D, K), 0x30, np.uint8)        # 0.5
    ws = np.full((H * D, K // 32), 0x7E, np.uint8)  # * 2^-1 -> 0.25
    cos, sin = o.rope_table(T, 0, 1e4)
    res = o.qup_forward(xc, wc, x_scales=xs, w_scales=ws, H=H, d_nope=D, d_rope=0,
                        cos=cos, sin=sin, B=1, S=T, out_dtype="bf16")
    # 32 * (1 * 0.25) + 32 * (2 * 0.25) = 24
    assert (res.q32 == 24.0).all()


# ------------------------------------------------------------ backward ----
def _tiny_case(seed=0):
    w = syn.workload("tiny")
    x = o.to_f64(syn.normal_bf16((w.T, w.K), 1.0, seed))
    W = o.to_f64(syn.normal_bf16((w.N, w.K), 0.125, seed + 1))
    b = o.to_f64(syn.normal_bf16((w.N,), 0.1, seed + 2))
    cos, sin = o.rope_table(w.T, w.d_rope, 1e4)
    pos = np.arange(w.T)
    return w, x, W, b, cos, sin, pos


def test_backward_matches_finite_differences():
    """The map is linear in X, W and b, so central differences are exact up to
    rounding: <G, f(X+E) - f(X-E)> / 2 = <dX, E> and likewise for W and b."""
    w, x, W, b, cos, sin, pos = _tiny_case()
    f = lambda x_, W_, b_: o.qup_forward_f64(x_, W_, b_, w.H, w.d_nope, w.d_rope, pos, cos, sin)
    rng = np.random.default_rng(9)
    G = rng.standard_normal((w.T, w.H, w.D))
    Gt = torch.from_numpy(G.astype(np.float32))
    r = o.qup_backward(Gt, torch.from_numpy(x.astype(np.float32)), torch.from_numpy(W.astype(np.float32)),
                       H=w.H, d_nope=w.d_nope, d_rope=w.d_rope, cos=cos, sin=sin, B=1, S=w.T)
    G = o.to_f64(Gt)
    for _ in range(3):
        Ex, EW, Eb = rng.standard_normal(x.shape), rng.standard_normal(W.shape), rng.standard_normal(b.shape)
        fd = ((f(x + Ex, W, b) - f(x - Ex, W, b)) * G.reshape(w.T, w.H, w.D)).sum() / 2
        assert fd == pytest.approx((r.dx * Ex).sum(), rel=1e-9)
        fd = ((f(x, W + EW, b) - f(x, W - EW, b)) * G.reshape(w.T, w.H, w.D)).sum() / 2
        assert fd == pytest.approx((r.dw * EW).sum(), rel=1e-9)
        fd = ((f(x, W, b + Eb) - f(x, W, b - Eb)) * G.reshape(w.T, w.H, w.D)).sum() / 2
        assert fd == pytest.approx((r.db * Eb).sum(), rel=1e-9)


def test_backward_full_jacobian_small():
    """Explicit Jacobian of the forward in X on a small case, column by column."""
    T, K, H, dn, dr = 3, 8, 1, 2, 4
    D = dn + dr
    rng = np.random.default_rng(2)
    x = rng.standard_normal((T, K))
    W = rng.standard_normal((H * D, K))
    cos, sin = o.rope_table(T, dr, 1e4)
    pos = np.arange(T)
    f = lambda x_: o.qup_forward_f64(x_, W, None, H, dn, dr, pos, cos, sin).reshape(-1)
    J = np.zeros((T * H * D, T * K))
    for j in range(T * K):
        e = np.zeros(T * K)
        e[j] = 1.0
        J[:, j] = f(x + e.reshape(T, K)) - f(x)
    G = rng.standard_normal(T * H * D)
    r = o.qup_backward(torch.from_numpy(G.reshape(T, H, D)), torch.from_numpy(x), torch.from_numpy(W),
                       H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, B=1, S=T)
    assert np.allclose(r.dx.reshape(-1), J.T @ G, rtol=1e-10, atol=1e-10)


def test_oracle_leaves_inputs_untouched():
    w, x, W, b, cos, sin, pos = _tiny_case()
    xt = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    Wt = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16)
    x0, W0 = xt.clone(), Wt.clone()
    o.qup_forward(xt, Wt, H=w.H, d_nope=w.d_nope, d_rope=w.d_rope, cos=cos, sin=sin, B=1, S=w.T)
    assert torch.equal(xt.view(torch.int16), x0.view(torch.int16))
    assert torch.equal(Wt.view(torch.int16), W0.view(torch.int16))


# ------------------------------------------------------ MXFP8 backward ----
def test_mx_columns_hand_worked():
    # [OCP-MX] worked by hand: 33 rows (padded to 64), two columns.
    # column 0 = [2^20, 1 x 31, 3]: block 0 amax 2^20 -> E = 20 - 8 = 12, 2^20 -> 256 = code 0x78,
    # 1 * 2^-12 is below half the smallest E4M3 subnormal (2^-9) -> 0; block 1 = [3, 0 x 31]
    # -> E = 1 - 8 = -7, 3 * 2^7 = 384 = 1.5 * 2^8 -> code 0x7C. Column 1 = ones: E = -8,
    # 1 -> 256 = 0x78; its second block holds one 1 and padding zeros.
    v = np.ones((33, 2))
    v[0, 0] = 2.0 ** 20
    v[32, 0] = 3.0
    codes, scales = o.mxfp8_quantize_columns(v)
    assert codes.shape == (2, 64) and scales.shape == (2, 2)
    assert codes[0, 0] == 0x78 and not codes[0, 1:32].any()
    assert codes[0, 32] == 0x7C and not codes[0, 33:].any()
    assert (codes[1, :33] == 0x78).all() and not codes[1, 33:].any()
    assert scales.tolist() == [[12 + 127, -7 + 127], [-8 + 127, -8 + 127]]


def _mx_bwd(dq, x, w, H, dn, dr, T, seed=0):
    cos, sin = o.rope_table(T, max(dr, 2), 10000.0) if dr else (np.ones((T, 1)), np.zeros((T, 1)))
    return o.qup_backward_mxfp8(torch.from_numpy(dq.astype(np.float32)).to(torch.bfloat16),
                                torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16),
                                torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16),
                                H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin)


def test_mx_backward_exact_when_representable():
    # Every block's amax in [4, 7] gives E = -6, and k * 64 (|k| <= 7) is an E4M3 value:
    # quantization is lossless, so the products equal the plain ones. T = 40 exercises the
    # zero-padded token blocks.
    rng = np.random.default_rng(5)
    T, H, D, K = 40, 2, 32, 64
    pick = lambda *s: rng.choice([-7, -6, -5, -4, 4, 5, 6, 7], size=s).astype(np.float64)
    dq, x, w = pick(T, H * D), pick(T, K), pick(H * D, K)
    r = _mx_bwd(dq.reshape(T, H, D), x, w, H, D, 0, T)
    assert np.array_equal(r.dx, dq @ w)
    assert np.array_equal(r.dw, dq.T @ x)
    assert np.array_equal(r.db, dq.sum(axis=0))


def test_mx_backward_orientation_hand_worked():
    # dq (32 x 32, one head without rope): dq[0,0] = 2^20, the rest of row 0 is 1, the
    # rest of column 0 is 2, everything else 1. Row quantization (dX operand) flushes the
    # ones of token 0 (1 * 2^-12 -> 0) and keeps every other row exactly; column
    # quantization (dW operand) flushes the twos of column 0 (2 * 2^-12 -> 0) and keeps
    # every other column. W = 2 I and x = 3 I then expose each quantized operand.
    T = N = K = 32
    dq = np.ones((T, N))
    dq[1:, 0] = 2.0
    dq[0, 0] = 2.0 ** 20
    w = 2.0 * np.eye(N, K)
    x = 3.0 * np.eye(T, K)
    r = _mx_bwd(dq.reshape(T, 1, N), x, w, 1, N, 0, T)
    ex = 2.0 * dq
    ex[0, 1:] = 0.0
    ew = 3.0 * dq.T
    ew[0, 1:] = 0.0
    assert np.array_equal(r.dx, ex)
    assert np.array_equal(r.dw, ew)


def test_mx_backward_power_of_two_scaling():
    # Scaling by a power of two moves every block exponent and nothing else.
    rng = np.random.default_rng(6)
    T, H, dn, dr, K = 48, 2, 32, 32, 64
    D = dn + dr
    dq = rng.standard_normal((T, H, D))
    x = rng.standard_normal((T, K))
    w = rng.standard_normal((H * D, K))
    a = _mx_bwd(dq, x, w, H, dn, dr, T)
    b = _mx_bwd(dq * 8.0, x, w, H, dn, dr, T)
    c = _mx_bwd(dq, x * 0.25, w, H, dn, dr, T)
    assert np.array_equal(b.dx, 8.0 * a.dx) and np.array_equal(b.dw, 8.0 * a.dw)
    assert np.array_equal(c.dw, 0.25 * a.dw) and np.array_equal(c.dx, a.dx)


def test_mx_backward_within_quantization_bound():
    # Each quantized operand element is within 2^-4 of its value relative (E4M3, 3 mantissa
    # bits, round to nearest) plus 2^(E-10) absolute (half the subnormal step of its block);
    # the products' error is bounded by the sum of those terms. Also a gross check that
    # the MXFP8 products track the unquantized ones.
    rng = np.random.default_rng(7)
    T, H, dn, dr, K = 64, 2, 32, 32, 96
    D = dn + dr
    dq = rng.standard_normal((T, H, D))
    x = rng.standard_normal((T, K))
    w = rng.standard_normal((H * D, K)) * 0.05
    r = _mx_bwd(dq, x, w, H, dn, dr, T)
    a = o.bf16_bits_to_f64(r.dq_pre_bf16)
    xf = o.to_f64(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
    wf = o.to_f64(torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16))

    def err(v, scales_along_rows):  # per-element bound, scales broadcast over their block
        s = o.e8m0_decode(scales_along_rows)
        return 2.0 ** -4 * np.abs(v) + np.repeat(s, 32, axis=-1)[..., :v.shape[-1]] * 2.0 ** -10
    ea = err(a, r.dq_rows[1])
    ew = err(wf.T, r.w_cols_t[1]).T
    bound_dx = ea @ np.abs(wf) + np.abs(a) @ ew + ea @ ew
    assert (np.abs(r.dx - a @ wf) <= bound_dx * (1 + 1e-12)).all()
    eat = err(a.T, r.dq_cols_t[1][:, :T // 32 + (T % 32 > 0)])
    ex = err(xf.T, r.x_cols_t[1]).T
    bound_dw = eat @ np.abs(xf) + np.abs(a.T) @ ex + eat @ ex
    assert (np.abs(r.dw - a.T @ xf) <= bound_dw * (1 + 1e-12)).all()
    rel = np.linalg.norm(r.dx - a @ wf) / np.linalg.norm(a @ wf)
    assert 1e-4 < rel < 0.05


def test_mx_backward_quantizes_the_stored_bf16_copy():
    # The operands are quantized from dq_pre as stored (bf16), not from its exact value.
    # Pick g_a, g_b so that v = c g_a + s g_b (inverse rotation at position 1, pair 0)
    # lies in (1.0625, 1.0625 + 2^-9): bf16 rounds v down to 1.0625 exactly. The block
    # amax is in [1, 2), so E = -8 and the E4M3 grid near 1.0625 * 256 = 272 has step 32:
    # 272 is a tie between 256 (code 0x78) and 288 (0x79), broken to even -> 0x78; the
    # unrounded v would round up to 0x79.
    T, H, dn, dr, K = 2, 1, 32, 32, 32
    cos, sin = o.rope_table(T, dr, 10000.0)
    c, s = float(np.float32(cos[1, 0])), float(np.float32(sin[1, 0]))
    grid = o.bf16_bits_to_f64(np.arange(0x3F00, 0x3FC0, dtype=np.uint16))  # 0.5 .. 1.5
    va = grid[:, None] * c + grid[None, :] * s
    i, j = np.argwhere((va > 1.0625) & (va < 1.0625 + 2.0 ** -9))[0]
    ga, gb = grid[i], grid[j]
    assert abs(-ga * s + gb * c) < 2.0
    dq = np.zeros((T, H, dn + dr))
    dq[1, 0, dn] = ga
    dq[1, 0, dn + 1] = gb
    x = np.ones((T, K))
    w = np.ones((H * (dn + dr), K))
    r = _mx_bwd(dq, x, w, H, dn, dr, T)
    assert o.bf16_bits_to_f64(r.dq_pre_bf16[1:2, dn:dn + 1])[0, 0] == 1.0625
    assert r.dq_rows[1][1, dn // 32] == 127 - 8
    assert r.dq_rows[0][1, dn] == 0x78


# ------------------------------------------------------------ KV side ----
def _kv_inputs(T, H, dn, dr, dv, seed):
    rng = np.random.default_rng(seed)
    kv = torch.from_numpy(rng.standard_normal((T, H, dn + dv)).astype(np.float32)).to(torch.bfloat16)
    pe = torch.from_numpy(rng.standard_normal((T, dr)).astype(np.float32)).to(torch.bfloat16)
    return kv, pe


def test_kv_rope_passthrough_broadcast_and_closed_form():
    # bf16 output: k_nope and v pass through bit for bit, every head carries the same
    # rotated slice, position 0 is the identity, and at position p pair i is the closed
    # form (a cos(p theta_i) - b sin(p theta_i), a sin(p theta_i) + b cos(p theta_i)).
    T, H, dn, dr, dv = 5, 3, 32, 16, 32
    kv, pe = _kv_inputs(T, H, dn, dr, dv, 11)
    cos, sin = o.rope_table(T, dr, 10000.0)
    r = o.kv_rope(kv, pe, H=H, d_nope=dn, d_rope=dr, d_v=dv, cos=cos, sin=sin, out_dtype="bf16")
    kvb = kv.view(torch.int16).numpy().view(np.uint16)
    key = r.key[0].transpose(1, 0, 2)      # [T, H, D] from BHSD with B = 1
    val = r.value[0].transpose(1, 0, 2)
    assert np.array_equal(key[:, :, :dn], kvb[:, :, :dn])
    assert np.array_equal(val, kvb[:, :, dn:])
    assert all(np.array_equal(key[:, h, dn:], key[:, 0, dn:]) for h in range(H))
    peb = pe.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(key[0, 0, dn:], peb[0])
    p, i = 3, 2
    th = 10000.0 ** (-2 * i / dr)
    a, b_ = o.to_f64(pe)[p, 2 * i], o.to_f64(pe)[p, 2 * i + 1]
    want = (a * math.cos(p * th) - b_ * math.sin(p * th), a * math.sin(p * th) + b_ * math.cos(p * th))
    got = r.key32[p, 1, dn + 2 * i:dn + 2 * i + 2]
    assert np.allclose(got, want, rtol=1e-6, atol=1e-7)
    # the rotated values are kept at float32 (no 16-bit rounding before quantization)
    rope32 = r.key32[1:, 0, dn:]
    assert (o.bf16_bits_to_f64(o.f32_to_bf16_bits(rope32)) != rope32).any()


def test_kv_rope_mxfp8_blocks_and_bhsd_placement():
    # MXFP8: key blocks of 32 along its head dim (one here spans k_nope and the rope
    # slice), value blocks likewise; SBHD token order lands token t = s B + b at [b, :, s].
    B, S, H, dn, dr, dv = 2, 3, 2, 16, 48, 64
    T = B * S
    kv, pe = _kv_inputs(T, H, dn, dr, dv, 12)
    cos, sin = o.rope_table(S, dr, 10000.0)
    r = o.kv_rope(kv, pe, H=H, d_nope=dn, d_rope=dr, d_v=dv, cos=cos, sin=sin, fmt=o.FMT_SBHD,
                  B=B, S=S)
    assert r.key.shape == (B, H, S, dn + dr) and r.key_scales.shape == (B, H, S, 2)
    assert r.value.shape == (B, H, S, dv) and r.value_scales.shape == (B, H, S, 2)
    t = 1 * B + 1   # s = 1, b = 1
    for h in range(H):
        blk = r.key32[t, h, :32]
        e = o.floor_log2(np.abs(blk).max()) - 8
        assert r.key_scales[1, h, 1, 0] == e + 127
        deq = o.mxfp8_dequantize(r.key[1, h, 1], r.key_scales[1, h, 1])
        assert np.all(np.abs(deq[:32] - blk) <= 2.0 ** -4 * np.abs(blk) + 2.0 ** (e - 10))
    # the value is the kv tail, untouched before quantization
    assert np.array_equal(r.value32, o.to_f64(kv)[:, :, dn:].astype(np.float32))
