"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Small cases compare every output element; the five named workloads run at
their full sizes in the same launch configuration the benchmark times, and
the oracle checks sampled token rows (plus full-size properties: input bytes
unchanged, run-to-run bit identity, every output element written).
"""
import numpy as np
import pytest
import torch

import mla_up_projection_amd as m
import oracle as o
from mla_up_projection_amd import synthetic as syn
from parity import (Guarded, assert_mx_bar, bits16, check_bf16, check_mx, frob_rel, fwd_reference_rows,
                    merge_stats, mx_stats, parallel_chunks, u8)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _dev(t):
    return t.to(DEV)


def rope_tables(rows, d_rope, base=1e4, yarn=None):
    """GPU table from rope_cache_build, oracle table from the oracle."""
    pairs = max(d_rope // 2, 1)
    cos = torch.empty(rows, pairs, dtype=torch.float32, device=DEV)
    sin = torch.empty_like(cos)
    if d_rope:
        m.rope_cache_build(cos, sin, d_rope, base, yarn)
    oy = o.Yarn(*yarn) if yarn is not None else None
    oc, os_ = o.rope_table(rows, d_rope, base, oy)
    return cos, sin, oc, os_


def run_fwd(x, w, *, H, dn, dr, out_mx, fmt=m.FMT_BSHD, B=1, S=None, cu=None, max_seqlen=None,
            yarn=None, bias=None, x_scales=None, w_scales=None, rows=None):
    """Run the GPU forward; returns (out, scales, oracle tables). Outputs are
    prefilled with a NaN pattern so unwritten elements are visible."""
    T = x.shape[0]
    D = dn + dr
    if S is None:
        S = T // B
    max_pos = max_seqlen if fmt == m.FMT_THD else S
    cos, sin, oc, os_ = rope_tables(rows or max_pos, dr, yarn=yarn)
    shape = o.out_shape(fmt, T, H, D, B, S)
    # prefilled so unwritten elements show, inside sentinel margins
    if out_mx:
        go = Guarded(shape, torch.uint8, 0x7F)
        gs = Guarded(shape[:3] + (D // 32,), torch.uint8, 0xFF)
        out, sc = go.t, gs.t
    else:
        go, gs = Guarded(shape, torch.bfloat16, 0xFF), None   # 0xFFFF: NaN
        out, sc = go.t, None
    m.mla_qup_fwd(x, w, out, H=H, d_nope=dn, d_rope=dr, cos=cos if dr else None,
                  sin=sin if dr else None, x_scales=x_scales, w_scales=w_scales, bias=bias,
                  out_scales=sc, fmt=fmt, B=B, S=S, cu_seqlens=cu, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    go.check("out")
    if gs is not None:
        gs.check("out_scales")
    return out, sc, oc, os_


# ------------------------------------------------------------ rope table ----
@pytest.mark.parametrize("rows,d,yarn", [(64, 16, None), (4096, 64, None),
                                         (4096, 64, (40.0, 4096, 32.0, 1.0, 1.0)),
                                         (300, 64, (40.0, 4096, 32.0, 1.0, 1.3688))])
def test_rope_cache_matches_oracle(rows, d, yarn):
    cos, sin, oc, os_ = rope_tables(rows, d, yarn=yarn)
    for g, r in ((cos.cpu().numpy(), oc), (sin.cpu().numpy(), os_)):
        ulp = np.abs(g.view(np.int32).astype(np.int64) - r.view(np.int32).astype(np.int64))
        # both round a float64 cos/sin to float32; libm and device math may
        # differ in the last double bit, which moves a float32 rounding at most
        # one step, and rarely
        assert ulp.max() <= 1 and (ulp > 0).mean() <= 1e-3


# --------------------------------------------------------- mxfp8_quantize ----
def test_mxfp8_quantize_bf16_exhaustive_bitexact():
    """All 65536 bf16 patterns, in 2048 blocks of 32 (blocks holding NaN or Inf
    become 0xFF / 0x7F), plus a shuffled copy for mixed-magnitude blocks."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    perm = np.random.default_rng(5).permutation(65536)
    allb = np.concatenate([bits, bits[perm]]).reshape(-1, 256)
    x = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16)
    xd = _dev(x)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    scales = torch.empty(x.shape[0], x.shape[1] // 32, dtype=torch.uint8, device=DEV)
    m.mxfp8_quantize(xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = o.mxfp8_quantize_blocks(o.to_f64(x).astype(np.float32))
    assert np.array_equal(u8(scales), rs)
    assert np.array_equal(u8(codes), rc)


def test_mxfp8_quantize_fp32_special_values_and_stride():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((96, 192)) * 0.784).astype(np.float32)
    v[1, :32] = 0.0
    v[2, :32] = -0.0
    v[3, :32] = np.float32(1e-40) * rng.standard_normal(32).astype(np.float32)  # subnormals
    v[4, 32:64] = np.float32(3e38)
    v[5, 5] = np.nan
    v[6, 70] = -np.inf
    # exact E4M3 ties after scaling by 2^-E (amax 448 gives E = 0)
    v[7, :6] = [448.0, 17.0, 19.0, 0.0029296875, 0.0009765625, -0.0048828125]
    v[8, :32] = np.float32(2.0 ** -130)   # amax float32-subnormal: E clamps to -127
    base = np.zeros((96, 256), np.float32)
    base[:, :192] = v
    xd = _dev(torch.from_numpy(base))[:, :192]     # row stride 256 > cols
    codes = torch.empty(96, 192, dtype=torch.uint8, device=DEV)
    scales = torch.empty(96, 6, dtype=torch.uint8, device=DEV)
    m.mxfp8_quantize(xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = o.mxfp8_quantize_blocks(v)
    assert np.array_equal(u8(scales), rs)
    assert np.array_equal(u8(codes), rc)


# ------------------------------------------------------------- forward ------
def full_compare_fwd(x, w, *, H, dn, dr, fmt=m.FMT_BSHD, B=1, S=None, cu=None, max_seqlen=None,
                     yarn=None, bias=None, mx_in=False):
    T, K = x.shape
    S = S if S is not None else T // B
    xs = ws = xq = wq = None
    xd, wd = _dev(x), _dev(w)
    if mx_in:
        xq = torch.empty(T, K, dtype=torch.uint8, device=DEV)
        xs = torch.empty(T, K // 32, dtype=torch.uint8, device=DEV)
        wq = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
        ws = torch.empty(w.shape[0], K // 32, dtype=torch.uint8, device=DEV)
        m.mxfp8_quantize(xd, xq, xs)
        m.mxfp8_quantize(wd, wq, ws)
        xd, wd = xq, wq
    cud = _dev(cu) if cu is not None else None
    bd_ = _dev(bias) if bias is not None else None
    res = {}
    for out_mx in (False, True):
        out, sc, oc, os_ = run_fwd(xd, wd, H=H, dn=dn, dr=dr, out_mx=out_mx, fmt=fmt, B=B, S=S,
                                   cu=cud, max_seqlen=max_seqlen, yarn=yarn, bias=bd_,
                                   x_scales=xs, w_scales=ws)
        # oracle: quantizes X and W itself on the MXFP8 path
        if mx_in:
            oxq, oxs = o.mxfp8_quantize_blocks(o.to_f64(x).astype(np.float32))
            owq, ows = o.mxfp8_quantize_blocks(o.to_f64(w).astype(np.float32))
            assert np.array_equal(u8(xq), oxq) and np.array_equal(u8(xs), oxs)
            ox, ow = oxq, owq
        else:
            ox, ow, oxs, ows = x, w, None, None
        pos, bb, ss = o.token_coords(fmt, T, B, S, cu.numpy() if cu is not None else None)
        rows = np.arange(T)
        q64, bound = fwd_reference_rows(ox, ow, bias, rows, H=H, d_nope=dn, d_rope=dr, cos=oc,
                                        sin=os_, pos=pos, x_scales=oxs if mx_in else None,
                                        w_scales=ows if mx_in else None)
        g = out.cpu()
        g_rows = g[bb, :, ss, :]                  # [T, H, D] token-major
        if out_mx:
            g_sc = sc.cpu()[bb, :, ss, :]
            res["mx"] = check_mx(g_rows.numpy(), g_sc.numpy(), q64, bound)
            print("\nmx", res["mx"], flush=True)
            # every element written: BHSD has no slot outside the token rows
            assert g.numel() == g_rows.numel() and sc.numel() == g_sc.numel()
        else:
            r_bits = o.f32_to_bf16_bits(q64.astype(np.float32))
            res["bf16"] = check_bf16(bits16(g_rows), r_bits)
    return res


def test_fwd_tiny_workload():
    w = syn.workload("tiny")
    full_compare_fwd(w.x(), w.w(), H=w.H, dn=w.d_nope, dr=w.d_rope, B=1, S=w.T)


@pytest.mark.parametrize("fmt,B,S", [(m.FMT_BSHD, 1, 333), (m.FMT_SBHD, 3, 111), (m.FMT_BSHD, 3, 111)])
def test_fwd_ragged_multi_tile(fmt, B, S):
    """T = 333 (two token tiles, ragged), N = 960 (five N tiles), K = 256, bias."""
    T, K, H = B * S, 256, 5
    x = syn.normal_bf16((T, K), 1.0, 10)
    w = syn.normal_bf16((H * 192, K), 0.05, 11)
    bias = syn.normal_bf16((H * 192,), 0.3, 12)
    full_compare_fwd(x, w, H=H, dn=128, dr=64, fmt=fmt, B=B, S=S, bias=bias)


@pytest.mark.parametrize("dn,dr,H", [(32, 0, 3), (0, 64, 2), (16, 16, 7)])
def test_fwd_head_layouts(dn, dr, H):
    T, K = 200, 96
    x = syn.normal_bf16((T, K), 1.0, 20)
    w = syn.normal_bf16((H * (dn + dr), K), 0.1, 21)
    full_compare_fwd(x, w, H=H, dn=dn, dr=dr, B=1, S=T)


def test_fwd_thd_yarn_small():
    lengths = [100, 37, 200, 1]
    cu = syn.cu_seqlens_of(lengths)
    T, K, H = sum(lengths), 128, 3
    x = syn.normal_bf16((T, K), 1.0, 30)
    w = syn.normal_bf16((H * 192, K), 0.05, 31)
    full_compare_fwd(x, w, H=H, dn=128, dr=64, fmt=m.FMT_THD, cu=cu, max_seqlen=max(lengths),
                     yarn=(40.0, 4096, 32.0, 1.0, 1.0))


def test_fwd_thd_many_short_and_empty_sequences():
    """Sequences of 0 to 5 tokens among longer ones, across two token tiles:
    32-token runs that hold several sequence starts (and empty sequences), so
    every token must restart its position at its own sequence's start."""
    lengths = [1, 0, 3, 5, 0, 2, 31, 33, 1, 1, 1, 64, 7, 0, 0, 4, 2, 2, 2, 2, 40, 1, 3, 0]
    cu = syn.cu_seqlens_of(lengths)
    T, K, H = sum(lengths), 128, 2
    x = syn.normal_bf16((T, K), 1.0, 32)
    w = syn.normal_bf16((H * 192, K), 0.05, 33)
    full_compare_fwd(x, w, H=H, dn=128, dr=64, fmt=m.FMT_THD, cu=cu, max_seqlen=max(lengths))


def test_fwd_mxfp8_projection_small():
    T, K, H = 300, 256, 3
    x = syn.normal_bf16((T, K), 1.0, 40)
    w = syn.normal_bf16((H * 192, K), 0.02, 41)
    full_compare_fwd(x, w, H=H, dn=128, dr=64, B=1, S=T, mx_in=True)


def test_fwd_mxfp8_projection_long_k():
    """K = 4096 (operand scales stream with each stage, so K has no limit
    beyond the 32-bit row offsets); ragged token tile."""
    T, K, H = 96, 4096, 2
    x = syn.normal_bf16((T, K), 1.0, 44)
    w = syn.normal_bf16((H * 192, K), 0.02, 45)
    full_compare_fwd(x, w, H=H, dn=128, dr=64, B=1, S=T, mx_in=True)


@pytest.mark.parametrize("fp8_mfma,K", [(False, 512), (True, 512), (False, 2176), (True, 2176)])
def test_fwd_mxfp8_operands_narrow_codes_random_scales(fp8_mfma, K):
    """MXFP8 X and W given directly: every code has exponent field 7 (values
    +-1..1.875), scales vary per 32-block. Products then never differ by more
    than 2^4, so the result is exact up to fp32 summation: this isolates the
    operand/scale layout of the scaled MFMA from its dot-product precision."""
    T, H, D = 256, 2, 192
    rng = np.random.default_rng(80)
    def codes(shape):
        return ((rng.integers(0, 2, shape) << 7) | (7 << 3) | rng.integers(0, 8, shape)).astype(np.uint8)
    xc, wc = codes((T, K)), codes((H * D, K))
    xs = rng.integers(118, 136, (T, K // 32)).astype(np.uint8)
    ws = rng.integers(112, 130, (H * D, K // 32)).astype(np.uint8)
    cos, sin, oc, os_ = rope_tables(T, 64)
    out = torch.full((1, H, T, D), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    m.mla_qup_fwd(_dev(torch.from_numpy(xc)), _dev(torch.from_numpy(wc)), out, H=H, d_nope=128,
                  d_rope=64, cos=cos, sin=sin, x_scales=_dev(torch.from_numpy(xs)),
                  w_scales=_dev(torch.from_numpy(ws)), B=1, S=T, fp8_mfma=fp8_mfma)
    torch.cuda.synchronize()
    pos = np.arange(T)
    q64, bound = fwd_reference_rows(xc, wc, None, pos, H=H, d_nope=128, d_rope=64, cos=oc, sin=os_,
                                    pos=pos, x_scales=xs, w_scales=ws)
    g = o.bf16_bits_to_f64(bits16(out[0].transpose(0, 1)))
    r = o.bf16_bits_to_f64(o.f32_to_bf16_bits(q64.astype(np.float32)))
    # g and r are bf16 roundings (half a step, 2^-8 relative, each) of values
    # within the fp32 accumulation bound of the exact result
    lim = 2.0 ** -7 * np.abs(q64) + 1.01 * bound + 1e-30
    ratio = np.abs(g - r) / lim
    print(f"\nnarrow codes K={K} fp8_mfma={fp8_mfma}: worst |g-r| / bound = {ratio.max():.3g}")
    assert (ratio <= 1).all()


def test_fwd_fp8_mfma_mode_accuracy():
    """Opt-in scaled-FP8-MFMA mode on MX-quantized DeepSeek-V3-like operands.
    Its dot products are summed in the instruction's narrower fixed-point
    window, so the bar is a relative Frobenius error of 1e-2 on the bf16
    output (the deviation is printed) rather than the MXFP8 code bar."""
    T, K, H = 512, 1536, 4
    x = syn.normal_bf16((T, K), 1.0, 0)
    w = syn.normal_bf16((H * 192, K), 0.02, 1)
    xq = torch.empty(T, K, dtype=torch.uint8, device=DEV)
    xs = torch.empty(T, K // 32, dtype=torch.uint8, device=DEV)
    wq = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
    ws = torch.empty(w.shape[0], K // 32, dtype=torch.uint8, device=DEV)
    m.mxfp8_quantize(_dev(x), xq, xs)
    m.mxfp8_quantize(_dev(w), wq, ws)
    cos, sin, oc, os_ = rope_tables(T, 64)
    out = torch.empty(1, H, T, 192, dtype=torch.bfloat16, device=DEV)
    m.mla_qup_fwd(xq, wq, out, H=H, d_nope=128, d_rope=64, cos=cos, sin=sin, x_scales=xs,
                  w_scales=ws, B=1, S=T, fp8_mfma=True)
    torch.cuda.synchronize()
    pos = np.arange(T)
    q64, _ = fwd_reference_rows(u8(xq), u8(wq), None, pos, H=H, d_nope=128, d_rope=64, cos=oc,
                                sin=os_, pos=pos, x_scales=u8(xs), w_scales=u8(ws))
    g = o.bf16_bits_to_f64(bits16(out[0].transpose(0, 1)))
    rms = np.sqrt((q64 ** 2).mean())
    rel = frob_rel(g, q64)
    print(f"\nfp8-mfma mode: rel Frobenius {rel:.3e}, max abs err / RMS {np.abs(g - q64).max() / rms:.3e}")
    assert rel <= 1e-2


def _at_offset(t, offset):
    """A device copy of t starting `offset` bytes past a 256-byte boundary."""
    t = t.contiguous()
    nb = t.numel() * t.element_size()
    buf = torch.zeros(nb + 512, dtype=torch.uint8, device=DEV)
    view = buf[offset:offset + nb].view(t.dtype).view(t.shape)
    view.copy_(t.to(DEV))
    assert view.data_ptr() % 256 == offset
    return view


def test_fwd_and_bwd_at_minimum_alignment():
    """Arguments at the smallest alignment the C ABI admits: x, w, out and
    dq / dq_pre / dx / dw 16 bytes past a 256-byte boundary, the bias 8 bytes
    past one, cos / sin 16 bytes past one (the widest vector loads the
    kernels issue on them). Results against the oracle."""
    T, K, H, dn, dr = 333, 256, 3, 128, 64
    D, N = dn + dr, H * (dn + dr)
    x = syn.normal_bf16((T, K), 1.0, 140)
    w = syn.normal_bf16((N, K), 0.05, 141)
    bias = syn.normal_bf16((N,), 0.3, 142)
    cos, sin, oc, os_ = rope_tables(T, dr)
    c16, s16 = _at_offset(cos, 16), _at_offset(sin, 16)
    xd, wd, bd_ = _at_offset(x, 16), _at_offset(w, 16), _at_offset(bias, 8)
    out = _at_offset(torch.zeros(1, H, T, D, dtype=torch.uint8), 16)
    sc = _at_offset(torch.zeros(1, H, T, D // 32, dtype=torch.uint8), 16)
    outb = _at_offset(torch.zeros(1, H, T, D, dtype=torch.bfloat16), 16)
    kw = dict(H=H, d_nope=dn, d_rope=dr, cos=c16, sin=s16, bias=bd_, B=1, S=T)
    m.mla_qup_fwd(xd, wd, out, out_scales=sc, **kw)
    m.mla_qup_fwd(xd, wd, outb, **kw)
    torch.cuda.synchronize()
    pos, bb, ss = o.token_coords(o.FMT_BSHD, T, 1, T)
    q64, bound = fwd_reference_rows(x, w, bias, np.arange(T), H=H, d_nope=dn, d_rope=dr, cos=oc,
                                    sin=os_, pos=pos)
    check_mx(u8(out)[0].transpose(1, 0, 2), u8(sc)[0].transpose(1, 0, 2), q64, bound, "min-align mx")
    check_bf16(bits16(outb)[0].transpose(1, 0, 2), o.f32_to_bf16_bits(q64.astype(np.float32)),
               "min-align bf16")
    dq = syn.normal_bf16((T, H, D), 1e-3, 143)
    dqd = _at_offset(dq, 16)
    dq_pre = _at_offset(torch.zeros(T, N, dtype=torch.bfloat16), 16)
    dx = _at_offset(torch.zeros(T, K, dtype=torch.bfloat16), 16)
    dw = _at_offset(torch.zeros(N, K, dtype=torch.bfloat16), 16)
    db = _at_offset(torch.zeros(N, dtype=torch.bfloat16), 2)
    bkw = dict(H=H, d_nope=dn, d_rope=dr, cos=c16, sin=s16, dx=dx, dw=dw, db=db, use_bias=True, B=1, S=T)
    nbytes = m.mla_qup_bwd_workspace_size(dqd, xd, wd, dq_pre, **bkw)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    m.mla_qup_bwd(dqd, xd, wd, dq_pre, workspace=ws if nbytes else None, **bkw)
    torch.cuda.synchronize()
    r = o.qup_backward(dq, x, w, H=H, d_nope=dn, d_rope=dr, cos=oc, sin=os_, S=T)
    check_bf16(bits16(dq_pre), o.f32_to_bf16_bits(r.dq_pre.astype(np.float32)), "min-align dq_pre")
    assert frob_rel(o.to_f64(dx.cpu()), r.dx) <= 1e-2
    assert frob_rel(o.to_f64(dw.cpu()), r.dw) <= 1e-2
    assert frob_rel(o.to_f64(db.cpu()), r.db) <= 1e-2


def test_fwd_zero_tokens_enqueues_nothing():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(1, 2, 0, 32, dtype=torch.bfloat16, device=DEV)
    cu = torch.zeros(2, dtype=torch.int32, device=DEV)
    cos = torch.ones(4, 8, device=DEV)
    m.mla_qup_fwd(x, w, out, H=2, d_nope=16, d_rope=16, cos=cos, sin=cos, fmt=m.FMT_THD,
                  cu_seqlens=cu, max_seqlen=1)
    torch.cuda.synchronize()


def test_fwd_position_beyond_table_is_nan_not_a_read():
    """A THD sequence longer than the max_seqlen the caller promised: the
    kernel's own bound check turns the rotated elements of positions past the
    table into NaN (MXFP8: scale 0xFF) instead of reading past it."""
    lengths = [40, 30]
    cu = _dev(syn.cu_seqlens_of(lengths))
    T, K, H = 70, 64, 1
    x = _dev(syn.normal_bf16((T, K), 1.0, 50))
    w = _dev(syn.normal_bf16((64, K), 0.1, 51))
    cos = torch.empty(32, 16, device=DEV)
    sin = torch.empty_like(cos)
    m.rope_cache_build(cos, sin, 32, 1e4)
    out = torch.empty(1, 2, T, 32, dtype=torch.uint8, device=DEV)   # H=2 heads of 32
    sc = torch.empty(1, 2, T, 1, dtype=torch.uint8, device=DEV)
    m.mla_qup_fwd(x, w, out, H=2, d_nope=0, d_rope=32, cos=cos, sin=sin, out_scales=sc,
                  fmt=m.FMT_THD, cu_seqlens=cu, max_seqlen=32)
    torch.cuda.synchronize()
    s = sc.cpu()[0, :, :, 0]
    pos = np.array(list(range(40)) + list(range(30)))
    assert (s[:, pos >= 32] == 0xFF).all() and (s[:, pos < 32] != 0xFF).all()


def test_fwd_position_beyond_table_is_nan_with_a_64_wide_rope_slice():
    """The same with heads of 128 + 64 (the table rows of a tile are staged
    in LDS on this path): rows past the table give NaN rope blocks only."""
    lengths = [40, 30]
    cu = _dev(syn.cu_seqlens_of(lengths))
    T, K, H, dn, dr = 70, 64, 1, 128, 64
    x = _dev(syn.normal_bf16((T, K), 1.0, 52))
    w = _dev(syn.normal_bf16((H * (dn + dr), K), 0.1, 53))
    cos = torch.empty(32, dr // 2, device=DEV)
    sin = torch.empty_like(cos)
    m.rope_cache_build(cos, sin, dr, 1e4)
    out = torch.empty(1, H, T, dn + dr, dtype=torch.uint8, device=DEV)
    sc = torch.empty(1, H, T, (dn + dr) // 32, dtype=torch.uint8, device=DEV)
    m.mla_qup_fwd(x, w, out, H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, out_scales=sc,
                  fmt=m.FMT_THD, cu_seqlens=cu, max_seqlen=32)
    torch.cuda.synchronize()
    s = sc.cpu()[0, 0]                       # [T, 6]: blocks 0..3 nope, 4..5 rope
    pos = np.array(list(range(40)) + list(range(30)))
    assert (s[pos >= 32][:, 4:] == 0xFF).all() and (s[pos < 32][:, 4:] != 0xFF).all()
    assert (s[:, :4] != 0xFF).all()


# ------------------------------------------------------------ backward ------
def run_bwd(dq, x, w, *, H, dn, dr, fmt=m.FMT_BSHD, B=1, S=None, cu=None, max_seqlen=None,
            use_bias=True, dw_fp32=False, yarn=None, mx=None, want=("dx", "dw")):
    """mx: None for the bf16 backward, else the fp8_mfma flag of the MXFP8 one."""
    T, K = x.shape
    N = H * (dn + dr)
    S = S if S is not None else T // B
    max_pos = max_seqlen if fmt == m.FMT_THD else S
    cos, sin, oc, os_ = rope_tables(max_pos, dr, yarn=yarn)
    dqd, xd, wd = _dev(dq), _dev(x), _dev(w)
    # every output and the workspace inside sentinel margins (out-of-bounds writes)
    guards = {"dq_pre": Guarded((T, N), torch.bfloat16)}
    if "dx" in want:
        guards["dx"] = Guarded((T, K), torch.bfloat16)
    if "dw" in want:
        guards["dw"] = Guarded((N, K), torch.float32 if dw_fp32 else torch.bfloat16)
    if use_bias:
        guards["db"] = Guarded((N,), torch.bfloat16)
    out = {k: (guards[k].t if k in guards else None) for k in ("dq_pre", "dx", "dw", "db")}
    dq_pre = out["dq_pre"]
    kw = dict(H=H, d_nope=dn, d_rope=dr, cos=cos if dr else None, sin=sin if dr else None,
              dx=out["dx"], dw=out["dw"], db=out["db"], use_bias=use_bias, fmt=fmt, B=B, S=S,
              cu_seqlens=_dev(cu) if cu is not None else None, max_seqlen=max_seqlen)
    if mx is None:
        nbytes = m.mla_qup_bwd_workspace_size(dqd, xd, wd, dq_pre, **kw)
    else:
        nbytes = m.mla_qup_bwd_mxfp8_workspace_size(dqd, xd, wd, dq_pre, **kw)
    if nbytes:
        guards["workspace"] = Guarded((nbytes,), torch.uint8)
    ws = guards["workspace"].t if nbytes else None
    if mx is None:
        m.mla_qup_bwd(dqd, xd, wd, dq_pre, workspace=ws, **kw)
    else:
        m.mla_qup_bwd_mxfp8(dqd, xd, wd, dq_pre, fp8_mfma=mx, workspace=ws, **kw)
    torch.cuda.synchronize()
    for k, g in guards.items():
        g.check(k)
    return dict(out, oc=oc, os=os_)


def test_bwd_small_against_oracle():
    T, K, H = 333, 256, 5
    x = syn.normal_bf16((T, K), 1.0, 60)
    w = syn.normal_bf16((H * 192, K), 0.02, 61)
    dq = syn.normal_bf16((T, H, 192), 1e-3, 62)
    for dw_fp32 in (False, True):
        g = run_bwd(dq, x, w, H=H, dn=128, dr=64, S=T, dw_fp32=dw_fp32)
        r = o.qup_backward(dq, x, w, H=H, d_nope=128, d_rope=64, cos=g["oc"], sin=g["os"], S=T)
        check_bf16(bits16(g["dq_pre"]), o.f32_to_bf16_bits(r.dq_pre.astype(np.float32)), "dq_pre")
        assert frob_rel(o.to_f64(g["dx"].cpu()), r.dx) <= 1e-2
        assert frob_rel(o.to_f64(g["dw"].cpu()), r.dw) <= 1e-2
        assert frob_rel(o.to_f64(g["db"].cpu()), r.db) <= 1e-2


@pytest.mark.parametrize("T", [1000, 2000])
def test_bwd_dw_token_splits(T):
    """Few heads, many tokens: dW has 3 x 1 output tiles, so its token
    reduction is split (2 splits of 8 stages at T = 1000, 4 at T = 2000; the
    last split ends in a partial stage) and the fp32 partials are summed in
    split order, into bf16 and into fp32 dW."""
    K, H = 192, 2
    x = syn.normal_bf16((T, K), 1.0, 63)
    w = syn.normal_bf16((H * 192, K), 0.02, 64)
    dq = syn.normal_bf16((T, H, 192), 1e-3, 65)
    for dw_fp32 in (False, True):
        g = run_bwd(dq, x, w, H=H, dn=128, dr=64, S=T, dw_fp32=dw_fp32)
        r = o.qup_backward(dq, x, w, H=H, d_nope=128, d_rope=64, cos=g["oc"], sin=g["os"], S=T)
        check_bf16(bits16(g["dq_pre"]), o.f32_to_bf16_bits(r.dq_pre.astype(np.float32)), "dq_pre")
        assert frob_rel(o.to_f64(g["dx"].cpu()), r.dx) <= 1e-2
        assert frob_rel(o.to_f64(g["dw"].cpu()), r.dw) <= 1e-2
        assert frob_rel(o.to_f64(g["db"].cpu()), r.db) <= 1e-2


def test_bwd_dw_token_splits_thd_dw_only():
    """dW alone (no dX, no bias: the split partials start the workspace) over a
    packed THD batch with YaRN, T = 1500: 24 stages of 64 tokens in 3 splits of
    8, sequence starts inside the splits, and a partial last stage."""
    lengths = [700, 1, 333, 466]
    cu = syn.cu_seqlens_of(lengths)
    T, K, H = sum(lengths), 192, 2
    x = syn.normal_bf16((T, K), 1.0, 66)
    w = syn.normal_bf16((H * 192, K), 0.02, 67)
    dq = syn.normal_bf16((T, H, 192), 1e-3, 68)
    yarn = (40.0, 4096, 32.0, 1.0, 1.0)
    for dw_fp32 in (False, True):
        g = run_bwd(dq, x, w, H=H, dn=128, dr=64, fmt=m.FMT_THD, cu=cu, max_seqlen=max(lengths),
                    use_bias=False, yarn=yarn, want=("dw",), dw_fp32=dw_fp32)
        r = o.qup_backward(dq, x, w, H=H, d_nope=128, d_rope=64, cos=g["oc"], sin=g["os"],
                           fmt=o.FMT_THD, cu_seqlens=cu.numpy())
        check_bf16(bits16(g["dq_pre"]), o.f32_to_bf16_bits(r.dq_pre.astype(np.float32)), "dq_pre")
        assert frob_rel(o.to_f64(g["dw"].cpu()), r.dw) <= 1e-2


def test_bwd_thd_yarn_no_bias():
    lengths = [64, 129, 7]
    cu = syn.cu_seqlens_of(lengths)
    T, K, H = sum(lengths), 192, 2
    x = syn.normal_bf16((T, K), 1.0, 70)
    w = syn.normal_bf16((H * 192, K), 0.02, 71)
    dq = syn.normal_bf16((T, H, 192), 1e-3, 72)
    yarn = (40.0, 4096, 32.0, 1.0, 1.0)
    g = run_bwd(dq, x, w, H=H, dn=128, dr=64, fmt=m.FMT_THD, cu=cu, max_seqlen=129,
                use_bias=False, yarn=yarn)
    r = o.qup_backward(dq, x, w, H=H, d_nope=128, d_rope=64, cos=g["oc"], sin=g["os"],
                       fmt=o.FMT_THD, cu_seqlens=cu.numpy())
    check_bf16(bits16(g["dq_pre"]), o.f32_to_bf16_bits(r.dq_pre.astype(np.float32)), "dq_pre")
    assert frob_rel(o.to_f64(g["dx"].cpu()), r.dx) <= 1e-2
    assert frob_rel(o.to_f64(g["dw"].cpu()), r.dw) <= 1e-2


def test_bwd_dx_only_and_dw_only():
    """Only dX, then only dW: the separate-launch paths (both together share
    one launch)."""
    T, K, H = 301, 320, 3
    x = syn.normal_bf16((T, K), 1.0, 80)
    w = syn.normal_bf16((H * 192, K), 0.02, 81)
    dq = syn.normal_bf16((T, H, 192), 1e-3, 82)
    N = H * 192
    cos, sin, oc, os_ = rope_tables(T, 64)
    r = o.qup_backward(dq, x, w, H=H, d_nope=128, d_rope=64, cos=oc, sin=os_, S=T)
    dqd, xd, wd = _dev(dq), _dev(x), _dev(w)
    for want in ("dx", "dw"):
        dq_pre = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
        dx = torch.empty(T, K, dtype=torch.bfloat16, device=DEV) if want == "dx" else None
        dw = torch.empty(N, K, dtype=torch.float32, device=DEV) if want == "dw" else None
        kw = dict(H=H, d_nope=128, d_rope=64, cos=cos, sin=sin, dx=dx, dw=dw, db=None,
                  use_bias=False, B=1, S=T)
        nbytes = m.mla_qup_bwd_workspace_size(dqd, xd, wd, dq_pre, **kw)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
        m.mla_qup_bwd(dqd, xd, wd, dq_pre, workspace=ws if nbytes else None, **kw)
        torch.cuda.synchronize()
        if want == "dx":
            assert frob_rel(o.to_f64(dx.cpu()), r.dx) <= 1e-2
        else:
            assert frob_rel(o.to_f64(dw.cpu()), r.dw) <= 1e-2


def test_bwd_width_not_multiple_of_64():
    """N = 96 (3 heads x 16+16): the dX reduction runs in 32-value stages."""
    T, K, H = 150, 96, 3
    x = syn.normal_bf16((T, K), 1.0, 90)
    w = syn.normal_bf16((H * 32, K), 0.1, 91)
    dq = syn.normal_bf16((T, H, 32), 1e-2, 92)
    g = run_bwd(dq, x, w, H=H, dn=16, dr=16, S=T)
    r = o.qup_backward(dq, x, w, H=H, d_nope=16, d_rope=16, cos=g["oc"], sin=g["os"], S=T)
    check_bf16(bits16(g["dq_pre"]), o.f32_to_bf16_bits(r.dq_pre.astype(np.float32)), "dq_pre")
    assert frob_rel(o.to_f64(g["dx"].cpu()), r.dx) <= 1e-2
    assert frob_rel(o.to_f64(g["dw"].cpu()), r.dw) <= 1e-2
    assert frob_rel(o.to_f64(g["db"].cpu()), r.db) <= 1e-2


def test_bwd_sbhd():
    """SBHD token order (t = s*B + b): positions s for the inverse rotation."""
    B, S, K, H = 3, 77, 128, 2
    T = B * S
    x = syn.normal_bf16((T, K), 1.0, 95)
    w = syn.normal_bf16((H * 192, K), 0.02, 96)
    dq = syn.normal_bf16((T, H, 192), 1e-3, 97)
    g = run_bwd(dq, x, w, H=H, dn=128, dr=64, fmt=m.FMT_SBHD, B=B, S=S)
    r = o.qup_backward(dq, x, w, H=H, d_nope=128, d_rope=64, cos=g["oc"], sin=g["os"],
                       fmt=o.FMT_SBHD, B=B, S=S)
    check_bf16(bits16(g["dq_pre"]), o.f32_to_bf16_bits(r.dq_pre.astype(np.float32)), "dq_pre")
    assert frob_rel(o.to_f64(g["dx"].cpu()), r.dx) <= 1e-2
    assert frob_rel(o.to_f64(g["dw"].cpu()), r.dw) <= 1e-2
    assert frob_rel(o.to_f64(g["db"].cpu()), r.db) <= 1e-2


def test_bwd_zero_tokens_zeroes_dw_db():
    K, H = 64, 2
    x = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, K, dtype=torch.bfloat16, device=DEV)
    dq = torch.empty(0, H, 32, dtype=torch.bfloat16, device=DEV)
    dq_pre = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    dw = torch.full((64, K), 7.0, dtype=torch.bfloat16, device=DEV)
    db = torch.full((64,), 7.0, dtype=torch.bfloat16, device=DEV)
    cos = torch.ones(4, 8, device=DEV)
    cu = torch.zeros(2, dtype=torch.int32, device=DEV)
    m.mla_qup_bwd(dq, x, w, dq_pre, H=H, d_nope=16, d_rope=16, cos=cos, sin=cos, dw=dw, db=db,
                  use_bias=True, fmt=m.FMT_THD, cu_seqlens=cu, max_seqlen=1)
    torch.cuda.synchronize()
    assert (dw.float() == 0).all() and (db.float() == 0).all()


# ------------------------------------------------------- MXFP8 backward ----
def test_mxfp8_quantize_t_bitexact():
    """Column quantization with a transposed store: 200 rows padded to 224
    (a partial 128-row tile), special values, bit for bit against the oracle."""
    R, C, Rp = 200, 96, 224
    x = syn.normal_bf16((R, C), 1.0, 150).clone()
    x[0:32, 3] = 0.0                            # an all-zero block
    x[40, 5] = float("nan")                     # a NaN block
    x[70, 6] = float("inf")                     # an infinite block
    x[100, 7] = 3.0e38                          # saturates its block's other codes to 0
    x[130:162, 8] = 2.0 ** -130                 # subnormal-range block
    codes = torch.full((C, Rp), 0xAA, dtype=torch.uint8, device=DEV)
    scales = torch.full((C, Rp // 32), 0xAA, dtype=torch.uint8, device=DEV)
    m.mxfp8_quantize_t(_dev(x), codes, scales)
    torch.cuda.synchronize()
    rc, rs = o.mxfp8_quantize_columns(o.to_f64(x))
    assert rc.shape == (C, Rp)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


def test_mxfp8_quantize_t_more_row_tiles_than_one_grid_column_holds():
    """8,388,648 rows padded to 8,388,672: 65,537 tiles of 128 rows, past the
    launch's cap on the grid along the rows, so a workgroup quantizes two
    tiles; every code and scale against the oracle."""
    R, C = (1 << 23) + 40, 16
    Rp = (R + 31) // 32 * 32
    x = syn.normal_bf16((R, C), 1.0, 151)
    codes = torch.full((C, Rp), 0xAA, dtype=torch.uint8, device=DEV)
    scales = torch.full((C, Rp // 32), 0xAA, dtype=torch.uint8, device=DEV)
    m.mxfp8_quantize_t(_dev(x), codes, scales)
    torch.cuda.synchronize()
    rc, rs = o.mxfp8_quantize_columns(o.to_f64(x))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


def _check_mx_bwd(g, r, what, fp8_mfma=False):
    """The dequantized operand products are exact in float32, so the only
    error against the oracle is float32 accumulation (far below 1e-6 here),
    the output rounding (bf16: at most 2^-9 relative per element, so a
    relative Frobenius error below 2^-9), the scaled FP8 MFMA's lower internal
    precision in that mode (bounded at 1e-3), and the rare operand code that
    differs because dq_pre's bf16 store rounded a float32 value the oracle
    holds in float64 (one E4M3 step on one element)."""
    check_bf16(bits16(g["dq_pre"]), r.dq_pre_bf16, f"{what} dq_pre")
    out = {}
    for k in ("dx", "dw"):
        if g[k] is not None:
            out[k] = frob_rel(o.to_f64(g[k].cpu()), getattr(r, k))
            if g[k].dtype == torch.float32:
                lim = 1e-3 if fp8_mfma else 1e-6
            else:
                lim = 2.0 ** -9 * 1.1 + (1e-3 if fp8_mfma else 0.0)
            assert out[k] <= lim, (what, k, out[k], lim)
    if g["db"] is not None:
        assert frob_rel(o.to_f64(g["db"].cpu()), r.db) <= 1e-2
    print(f"\n{what}: rel Frobenius {out}", flush=True)


@pytest.mark.parametrize("fp8_mfma", [False, True])
def test_bwd_mxfp8_small_against_oracle(fp8_mfma):
    """T = 333 (tokens padded to 384 for the blocks along t), N = 384, K = 256."""
    T, K, H = 333, 256, 2
    x = syn.normal_bf16((T, K), 1.0, 160)
    w = syn.normal_bf16((H * 192, K), 0.02, 161)
    dq = syn.normal_bf16((T, H, 192), 1e-3, 162)
    for dw_fp32 in (False, True):
        g = run_bwd(dq, x, w, H=H, dn=128, dr=64, S=T, dw_fp32=dw_fp32, mx=fp8_mfma)
        r = o.qup_backward_mxfp8(dq, x, w, H=H, d_nope=128, d_rope=64, cos=g["oc"], sin=g["os"], S=T)
        _check_mx_bwd(g, r, f"mx bwd fp8_mfma={fp8_mfma} dw_fp32={dw_fp32}", fp8_mfma)
    # the MXFP8 backward's fused pass over dq rotates exactly as the bf16
    # backward's inverse RoPE: the same dq_pre, bit for bit (ragged last band)
    g16 = run_bwd(dq, x, w, H=H, dn=128, dr=64, S=T)
    assert np.array_equal(bits16(g16["dq_pre"]), bits16(g["dq_pre"]))


def test_bwd_mxfp8_thd_dx_only_then_dw_only():
    lengths = [64, 129, 7]
    cu = syn.cu_seqlens_of(lengths)
    T, K, H = sum(lengths), 96, 2
    x = syn.normal_bf16((T, K), 1.0, 170)
    w = syn.normal_bf16((H * 64, K), 0.05, 171)
    dq = syn.normal_bf16((T, H, 64), 1e-2, 172)
    yarn = (40.0, 4096, 32.0, 1.0, 1.0)
    for want in (("dx",), ("dw",)):
        g = run_bwd(dq, x, w, H=H, dn=32, dr=32, fmt=m.FMT_THD, cu=cu, max_seqlen=129,
                    use_bias=False, yarn=yarn, mx=False, want=want, dw_fp32=True)
        r = o.qup_backward_mxfp8(dq, x, w, H=H, d_nope=32, d_rope=32, cos=g["oc"], sin=g["os"],
                                 fmt=o.FMT_THD, cu_seqlens=cu.numpy())
        _check_mx_bwd(g, r, f"mx bwd thd {want}")


@pytest.mark.parametrize("want", [("dx",), ("dw",), ("dx", "dw")])
def test_bwd_mxfp8_sbhd_yarn_bias(want):
    """SBHD tokens (3 sequences of 111: three bands, the last ragged), a YaRN
    table and the bias gradient through the MXFP8 backward's fused pass, with
    dX only, dW only and both."""
    B, S, K, H = 3, 111, 128, 2
    T = B * S
    x = syn.normal_bf16((T, K), 1.0, 175)
    w = syn.normal_bf16((H * 192, K), 0.03, 176)
    dq = syn.normal_bf16((T, H, 192), 1e-2, 177)
    yarn = (40.0, 64, 32.0, 1.0, 1.0)
    g = run_bwd(dq, x, w, H=H, dn=128, dr=64, fmt=m.FMT_SBHD, B=B, S=S, use_bias=True, yarn=yarn,
                mx=False, want=want)
    r = o.qup_backward_mxfp8(dq, x, w, H=H, d_nope=128, d_rope=64, cos=g["oc"], sin=g["os"],
                             fmt=o.FMT_SBHD, B=B, S=S)
    _check_mx_bwd(g, r, f"mx bwd sbhd yarn bias {want}")


def test_bwd_position_beyond_table_is_nan_in_both_backwards():
    """A THD sequence longer than the max_seqlen the caller promised, in the
    backward: both the bf16 backward and the MXFP8 one's fused pass (a whole
    128-row band and a ragged one) turn the rotated columns of positions past
    the table into NaN, leave the other columns finite, and agree bit for bit
    on dq_pre."""
    lengths = [150, 30]
    cu = _dev(syn.cu_seqlens_of(lengths))
    T, K, H, dn, dr = 180, 64, 2, 32, 32
    N = H * (dn + dr)
    x = _dev(syn.normal_bf16((T, K), 1.0, 180))
    w = _dev(syn.normal_bf16((N, K), 0.1, 181))
    dq = _dev(syn.normal_bf16((T, H, dn + dr), 1e-2, 182))
    cos = torch.empty(64, dr // 2, device=DEV)
    sin = torch.empty_like(cos)
    m.rope_cache_build(cos, sin, dr, 1e4)
    pres = []
    for mx in (None, False):
        dq_pre = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
        dx = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
        dw = torch.empty(N, K, dtype=torch.float32, device=DEV)
        kw = dict(H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, dx=dx, dw=dw, use_bias=False,
                  fmt=m.FMT_THD, cu_seqlens=cu, max_seqlen=64)
        if mx is None:
            n = m.mla_qup_bwd_workspace_size(dq, x, w, dq_pre, **kw)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
            m.mla_qup_bwd(dq, x, w, dq_pre, workspace=ws if n else None, **kw)
        else:
            n = m.mla_qup_bwd_mxfp8_workspace_size(dq, x, w, dq_pre, **kw)
            ws = torch.empty(n, dtype=torch.uint8, device=DEV)
            m.mla_qup_bwd_mxfp8(dq, x, w, dq_pre, fp8_mfma=mx, workspace=ws, **kw)
        torch.cuda.synchronize()
        pres.append(dq_pre.float().cpu().numpy().reshape(T, H, dn + dr))
    pos = np.array(list(range(150)) + list(range(30)))
    for d in pres:
        assert np.isnan(d[pos >= 64][:, :, dn:]).all()
        assert np.isfinite(d[pos < 64]).all() and np.isfinite(d[:, :, :dn]).all()
    assert np.array_equal(pres[0].view(np.uint32), pres[1].view(np.uint32))


def test_whole_path_replays_bit_identically_from_a_graph():
    """Graph capture, for serving and training loops that replay a recorded
    step: the fused forward (MXFP8 BHSD out), the allocation-free backward, the
    MXFP8 backward (caller's workspace, allocated before capture) and the KV
    side recorded in one HIP graph. The library makes no allocation, memset or
    synchronising call on these paths, so capture succeeds; every replay, with
    eager work and synchronisations between replays, is bit-identical to the
    eager calls."""
    T, K, H, dn, dr, dv = 640, 256, 4, 128, 64, 128
    N = H * (dn + dr)
    x = _dev(syn.normal_bf16((T, K), 1.0, 190))
    w = _dev(syn.normal_bf16((N, K), 0.05, 191))
    dq = _dev(syn.normal_bf16((T, H, dn + dr), 1e-2, 192))
    kv = _dev(syn.normal_bf16((T, H, dn + dv), 1.0, 193))
    pe = _dev(syn.normal_bf16((T, dr), 1.0, 194))
    cos = torch.empty(T, dr // 2, device=DEV)
    sin = torch.empty_like(cos)
    m.rope_cache_build(cos, sin, dr, 1e4)
    u8 = dict(dtype=torch.uint8, device=DEV)
    b16 = dict(dtype=torch.bfloat16, device=DEV)

    def bufs():
        return dict(out=torch.empty(1, H, T, dn + dr, **u8), sc=torch.empty(1, H, T, (dn + dr) // 32, **u8),
                    dq_pre=torch.empty(T, N, **b16), dx=torch.empty(T, K, **b16), dw=torch.empty(N, K, **b16),
                    db=torch.empty(N, **b16), mdq_pre=torch.empty(T, N, **b16), mdx=torch.empty(T, K, **b16),
                    mdw=torch.empty(N, K, **b16), key=torch.empty(1, H, T, dn + dr, **u8),
                    ksc=torch.empty(1, H, T, (dn + dr) // 32, **u8), val=torch.empty(1, H, T, dv, **u8),
                    vsc=torch.empty(1, H, T, dv // 32, **u8))

    rope = dict(H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, B=1, S=T)
    probe = bufs()
    nws = m.mla_qup_bwd_mxfp8_workspace_size(dq, x, w, probe["mdq_pre"], dx=probe["mdx"], dw=probe["mdw"], **rope)
    ws = torch.empty(nws, **u8)

    def run(b):
        m.mla_qup_fwd(x, w, b["out"], out_scales=b["sc"], **rope)
        m.mla_qup_bwd_noalloc(dq, x, w, b["dq_pre"], dx=b["dx"], dw=b["dw"], db=b["db"], use_bias=True, **rope)
        m.mla_qup_bwd_mxfp8(dq, x, w, b["mdq_pre"], dx=b["mdx"], dw=b["mdw"], workspace=ws, fp8_mfma=False,
                            **rope)
        m.mla_kv_rope(kv, pe, b["key"], b["val"], d_v=dv, key_scales=b["ksc"], value_scales=b["vsc"], **rope)

    ref = bufs()
    run(ref)  # eager (also the allocation-free entry point's one-time set-up)
    torch.cuda.synchronize()
    got = bufs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(got)
    for rep in range(3):
        for t in got.values():
            t.view(torch.uint8).fill_(0xA5 ^ rep)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k].view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
    assert torch.isfinite(ref["dx"].float()).all() and torch.isfinite(ref["mdw"].float()).all()


def test_bwd_more_token_bands_than_one_grid_column_holds():
    """4,196,000 tokens (4196 sequences of 1000) of one 64-wide head: 65,563
    inverse-RoPE bands of 64 rows, more than the launch's grid extent along
    the bands (65,535), so workgroups take several bands each, the last one
    ragged. dq_pre on rows from each end and around the grid's wrap, and db
    over every token, against the oracle."""
    B, S, K, H, dn, dr = 4196, 1000, 32, 1, 32, 32
    T, N = B * S, H * (dn + dr)
    print(f"\nbackward T={T} N={N}: running", flush=True)
    dq = syn.normal_bf16((T, H, dn + dr), 1e-2, 200)
    x = _dev(syn.normal_bf16((T, K), 1.0, 201))
    w = _dev(syn.normal_bf16((N, K), 0.1, 202))
    cos, sin, oc, os_ = rope_tables(S, dr)
    dqd = _dev(dq)
    dq_pre = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    dw = torch.empty(N, K, dtype=torch.float32, device=DEV)
    db = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    kw = dict(H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, dw=dw, db=db, use_bias=True, B=B, S=S)
    n = m.mla_qup_bwd_workspace_size(dqd, x, w, dq_pre, **kw)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    m.mla_qup_bwd(dqd, x, w, dq_pre, workspace=ws, **kw)
    torch.cuda.synchronize()
    pos = np.arange(T, dtype=np.int64) % S
    # db over every token, in chunks of the oracle's inverse rotation
    ref_db = np.zeros(N)
    dqf = o.to_f64(dq)
    for c0 in range(0, T, 1 << 20):
        c1 = min(T, c0 + (1 << 20))
        ref_db += o.rope_rotate(dqf[c0:c1], pos[c0:c1], oc, os_, dn, dr, inverse=True).reshape(c1 - c0, N).sum(0)
    assert frob_rel(o.to_f64(db.cpu()), ref_db) <= 1e-2
    rows = np.concatenate([np.arange(0, 256), np.arange(65535 * 64 - 256, 65535 * 64 + 256), np.arange(T - 256, T)])
    ref = o.rope_rotate(dqf[rows], pos[rows], oc, os_, dn, dr, inverse=True).reshape(len(rows), N)
    got = dq_pre[torch.from_numpy(rows).to(DEV)]
    check_bf16(bits16(got), o.f32_to_bf16_bits(ref.astype(np.float32)), "dq_pre")
    assert torch.isfinite(dw).all()


def test_bwd_mxfp8_zero_tokens_zeroes_dw_db():
    K, H = 64, 2
    x = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(128, K, dtype=torch.bfloat16, device=DEV)
    dq = torch.empty(0, H, 64, dtype=torch.bfloat16, device=DEV)
    dq_pre = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    dw = torch.full((128, K), 7.0, dtype=torch.bfloat16, device=DEV)
    db = torch.full((128,), 7.0, dtype=torch.bfloat16, device=DEV)
    cos = torch.ones(4, 16, device=DEV)
    cu = torch.zeros(2, dtype=torch.int32, device=DEV)
    m.mla_qup_bwd_mxfp8(dq, x, w, dq_pre, H=H, d_nope=32, d_rope=32, cos=cos, sin=cos, dw=dw, db=db,
                        use_bias=True, fmt=m.FMT_THD, cu_seqlens=cu, max_seqlen=1)
    torch.cuda.synchronize()
    assert (dw.float() == 0).all() and (db.float() == 0).all()


# ------------------------------------------------ full-size named workloads --
# Every output element is compared: the oracle runs over chunks of token rows
# on a thread pool. Full-size properties are checked too: inputs unchanged,
# run-to-run bit identity, every output written, no write outside the outputs.
FULL_CHUNK = 128


def _hash(t):
    return hash(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())


def _fwd_full_size_run(wl, fp8_mfma=False):
    """Run one named forward workload at full size (the benchmark's launch
    configuration), twice, with guarded outputs; returns what the oracle
    comparison needs."""
    x, w = wl.x(), wl.w()
    T, K = x.shape
    xd, wd = _dev(x), _dev(w)
    cu = wl.cu_seqlens()
    cud = _dev(cu) if cu is not None else None
    max_pos = wl.max_pos
    cos, sin, oc, os_ = rope_tables(max_pos, wl.d_rope, yarn=wl.yarn)
    hx, hw, hc = _hash(xd), _hash(wd), _hash(cos)
    xs = ws = None
    ref = dict(x=o.to_f64(x), w=o.to_f64(w))
    if wl.mx_weight:
        xq = torch.empty(T, K, dtype=torch.uint8, device=DEV)
        xs = torch.empty(T, K // 32, dtype=torch.uint8, device=DEV)
        wq = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
        ws = torch.empty(w.shape[0], K // 32, dtype=torch.uint8, device=DEV)
        m.mxfp8_quantize(xd, xq, xs)
        m.mxfp8_quantize(wd, wq, ws)
        torch.cuda.synchronize()
        oxq, oxs = o.mxfp8_quantize_blocks(ref["x"].astype(np.float32))
        owq, ows = o.mxfp8_quantize_blocks(ref["w"].astype(np.float32))
        assert np.array_equal(u8(xs), oxs) and np.array_equal(u8(ws), ows)
        assert np.array_equal(u8(xq), oxq) and np.array_equal(u8(wq), owq)
        ref = dict(x=o.mxfp8_dequantize(oxq, oxs), w=o.mxfp8_dequantize(owq, ows))
        xin, win = xq, wq
    else:
        xin, win = xd, wd
    shape = o.out_shape(wl.fmt, T, wl.H, wl.D, wl.B, wl.S)
    outs = []
    for rep in range(2):
        go = Guarded(shape, torch.uint8, 0x7F)
        gs = Guarded(shape[:3] + (wl.D // 32,), torch.uint8, 0xFF)
        m.mla_qup_fwd(xin, win, go.t, H=wl.H, d_nope=wl.d_nope, d_rope=wl.d_rope, cos=cos, sin=sin,
                      x_scales=xs, w_scales=ws, out_scales=gs.t, fmt=wl.fmt, B=wl.B, S=wl.S,
                      cu_seqlens=cud, max_seqlen=max_pos, fp8_mfma=fp8_mfma)
        torch.cuda.synchronize()
        go.check("out")
        gs.check("out_scales")
        outs.append((go.t, gs.t))
    # determinism and completeness (finite inputs never give 0xFF scales)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert not (outs[0][1] == 0xFF).any()
    # inputs untouched, byte for byte
    assert _hash(xd) == hx and _hash(wd) == hw and _hash(cos) == hc
    pos, bb, ss = o.token_coords(wl.fmt, T, wl.B, wl.S, cu.numpy() if cu is not None else None)
    return dict(out=u8(outs[0][0]), sc=u8(outs[0][1]), ref=ref, oc=oc, os=os_, pos=pos, bb=bb, ss=ss)


def _fwd_full_size_stats(wl, r):
    """mx_stats over every token row, in parallel chunks."""
    xf, wf = r["ref"]["x"], r["ref"]["w"]
    awf = np.abs(wf)

    def one(lo, hi):
        rows = np.arange(lo, hi)
        q64, bound = fwd_reference_rows(xf, wf, None, rows, H=wl.H, d_nope=wl.d_nope, d_rope=wl.d_rope,
                                        cos=r["oc"], sin=r["os"], pos=r["pos"], abs_w=awf)
        g = r["out"][r["bb"][rows], :, r["ss"][rows], :]
        gs = r["sc"][r["bb"][rows], :, r["ss"][rows], :]
        return mx_stats(g, gs, q64, bound)

    return merge_stats(parallel_chunks(one, xf.shape[0], FULL_CHUNK))


@pytest.mark.parametrize("name", ["dsv3_fwd_bf16w", "dsv3_fwd_mxfp8w", "thd_yarn_fwd"])
def test_fwd_full_size(name):
    """The three full-size forward workloads (the MXFP8 projection in its
    default exact mode), every output element against the oracle at the
    MXFP8 bar."""
    wl = syn.workload(name)
    print(f"\n{name}: running", flush=True)
    r = _fwd_full_size_run(wl)
    st = assert_mx_bar(_fwd_full_size_stats(wl, r), name)
    print(f"{name}: {st}", flush=True)


def test_fwd_full_size_mxfp8_projection_on_fp8_mfma():
    """The MXFP8 projection at full size (T = 8192) on the scaled FP8 MFMA,
    every element against the oracle. The instruction sums each K-step's
    products in a narrower fixed-point window than float32, so its output is
    held to its measured deviation, not to the MXFP8 bar: scales and codes
    are compared, every flip is at most one code step, and the flip and
    scale-mismatch rates stay within the measured figures."""
    wl = syn.workload("dsv3_fwd_mxfp8w")
    print("\ndsv3_fwd_mxfp8w on FP8 MFMA: running", flush=True)
    r = _fwd_full_size_run(wl, fp8_mfma=True)
    st = _fwd_full_size_stats(wl, r)
    flips = st["code_flips"] / st["elements"]
    smis = (st["scale_adjudicated"] + st["scale_unexplained"]) / st["blocks"]
    gt1 = st["flip_gt1"] / st["elements"]
    print(f"dsv3_fwd_mxfp8w fp8_mfma: {st}; code flip fraction {flips:.3e}, more than one step "
          f"{gt1:.3e}, scale mismatch fraction {smis:.3e}", flush=True)
    # the measured deviation (deterministic for these seeded inputs), with a
    # margin for a reordered reduction
    assert flips <= 1.2e-3, flips
    assert gt1 <= 6e-5, gt1
    assert smis <= 1.2e-5 and st["scale_unexplained"] == 0, st
    assert st["flip_unexplained"] == 0, st


def test_bwd_full_size():
    """DeepSeek-V3 backward at full size, every element: dq_pre by the BF16
    rule, dX, dW and db by relative Frobenius error, with guarded outputs."""
    wl = syn.workload("dsv3_bwd")
    x, w, dq = wl.x(), wl.w(), wl.dq()
    T, K, N = wl.T, wl.K, wl.N
    print("\ndsv3_bwd: running", flush=True)
    g = run_bwd(dq, x, w, H=wl.H, dn=wl.d_nope, dr=wl.d_rope, S=wl.S, use_bias=True)
    pos, _, _ = o.token_coords(o.FMT_BSHD, T, 1, T)
    dq_pre = o.rope_rotate(o.to_f64(dq), pos, g["oc"], g["os"], wl.d_nope, wl.d_rope, inverse=True).reshape(T, N)
    gq = bits16(g["dq_pre"])
    st = parallel_chunks(lambda lo, hi: check_bf16(gq[lo:hi], o.f32_to_bf16_bits(dq_pre[lo:hi].astype(np.float32)),
                                                   "dq_pre"), T, 256)
    print(f"dq_pre worst max_rel {max(c['max_rel'] for c in st):.3e}", flush=True)
    wf, xf = o.to_f64(w), o.to_f64(x)
    ex = frob_rel(o.to_f64(g["dx"].cpu()), dq_pre @ wf)
    ew = frob_rel(o.to_f64(g["dw"].cpu()), dq_pre.T @ xf)
    eb = frob_rel(o.to_f64(g["db"].cpu()), dq_pre.sum(0))
    print(f"dsv3_bwd: dx {ex:.2e} dw {ew:.2e} db {eb:.2e}", flush=True)
    assert ex <= 1e-2 and ew <= 1e-2 and eb <= 1e-2


SAMPLE = 96


def sample_rows(T, seed=123):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, T // 2, T - 2, T - 1], rng.integers(0, T, SAMPLE)]))
    return rows


def test_bwd_tp8_shard_sampled():
    """One rank's share under 8-way head parallelism at DeepSeek-V3 size: the
    first 16 heads (N = 3072), T = 4096, K = 1536, in the launch configuration
    the benchmark times (dW in 2 token splits). Sampled dX and dW rows, all of
    db."""
    wl = syn.workload("dsv3_bwd")
    Hs = wl.H // 8
    T, K, D = wl.T, wl.K, wl.D
    Ns = Hs * D
    x = wl.x()
    w = wl.w()[:Ns].contiguous()
    dq = wl.dq().reshape(T, wl.H, D)[:, :Hs].contiguous()
    g = run_bwd(dq, x, w, H=Hs, dn=wl.d_nope, dr=wl.d_rope, S=wl.S, use_bias=True)
    pos, _, _ = o.token_coords(o.FMT_BSHD, T, 1, T)
    dq_pre = o.rope_rotate(o.to_f64(dq), pos, g["oc"], g["os"], wl.d_nope, wl.d_rope,
                           inverse=True).reshape(T, Ns)
    rows = sample_rows(T)
    check_bf16(bits16(g["dq_pre"][torch.from_numpy(rows).to(DEV)]),
               o.f32_to_bf16_bits(dq_pre[rows].astype(np.float32)), "dq_pre")
    wf, xf = o.to_f64(w), o.to_f64(x)
    assert frob_rel(o.to_f64(g["dx"][torch.from_numpy(rows).to(DEV)].cpu()), dq_pre[rows] @ wf) <= 1e-2
    nrows = sample_rows(Ns, seed=7)
    assert frob_rel(o.to_f64(g["dw"][torch.from_numpy(nrows).to(DEV)].cpu()), dq_pre[:, nrows].T @ xf) <= 1e-2
    assert frob_rel(o.to_f64(g["db"].cpu()), dq_pre.sum(0)) <= 1e-2


def test_bwd_mxfp8_full_size_sampled():
    """DeepSeek-V3 backward with MXFP8 operands, both MFMA modes; sampled dX
    rows and dW rows against the oracle's steps (the row and column
    quantizers and the dequantized products)."""
    wl = syn.workload("dsv3_bwd")
    x, w, dq = wl.x(), wl.w(), wl.dq()
    T, K, N = wl.T, wl.K, wl.N
    pos, _, _ = o.token_coords(o.FMT_BSHD, T, 1, T)
    rows, nrows = sample_rows(T), sample_rows(N, seed=7)
    ref = None
    for fp8 in (False, True):
        g = run_bwd(dq, x, w, H=wl.H, dn=wl.d_nope, dr=wl.d_rope, S=wl.S, use_bias=True, mx=fp8)
        if ref is None:
            dq_pre = o.rope_rotate(o.to_f64(dq), pos, g["oc"], g["os"], wl.d_nope, wl.d_rope,
                                   inverse=True).reshape(T, N)
            dqp = o.bf16_bits_to_f64(o.f32_to_bf16_bits(dq_pre.astype(np.float32)))
            wq = o.mxfp8_dequantize(*o.mxfp8_quantize_columns(o.to_f64(w)))      # [K, N]
            xq = o.mxfp8_dequantize(*o.mxfp8_quantize_columns(o.to_f64(x)))      # [K, Tp]
            dx_ref = o.mxfp8_dequantize(*o.mxfp8_quantize_blocks(dqp[rows])) @ wq.T
            dqc = o.mxfp8_dequantize(*o.mxfp8_quantize_columns(dqp[:, nrows]))   # [n, Tp]
            dw_ref = dqc @ xq.T
            ref = (dx_ref, dw_ref, dq_pre.sum(0))
            del dq_pre, dqp, wq, xq, dqc
        ri = torch.from_numpy(rows).to(DEV)
        ni = torch.from_numpy(nrows).to(DEV)
        ex = frob_rel(o.to_f64(g["dx"][ri].cpu()), ref[0])
        ew = frob_rel(o.to_f64(g["dw"][ni].cpu()), ref[1])
        print(f"\nmx bwd dsv3 fp8_mfma={fp8}: dx {ex:.2e} dw {ew:.2e}", flush=True)
        lim = 2.0 ** -9 * 1.1 + (1e-3 if fp8 else 0.0)
        assert ex <= lim and ew <= lim
        assert frob_rel(o.to_f64(g["db"].cpu()), ref[2]) <= 1e-2


# ------------------------------------------------------------ KV side ------
U32 = 2.0 ** -24


def kv_bound(pe64, cos, sin, pos, H, dn, dv):
    """float32 error bound of the rotated key elements (two products and a sum
    per element, doubled); the k_nope and value elements are exact copies."""
    T, dr = pe64.shape
    a, b = np.abs(pe64[:, 0::2]), np.abs(pe64[:, 1::2])
    c, s = np.abs(cos[pos].astype(np.float64)), np.abs(sin[pos].astype(np.float64))
    e = 8 * U32 * (a + b) * (c + s)
    rot = np.repeat(e, 2, axis=1)
    key = np.concatenate([np.zeros((T, H, dn)), np.broadcast_to(rot[:, None, :], (T, H, dr))], axis=2)
    return key


def run_kv(kv, pe, *, H, dn, dr, dv, mx, fmt=m.FMT_BSHD, B=1, S=None, cu=None, max_seqlen=None,
           cos=None, sin=None):
    T = kv.shape[0]
    S = S if S is not None else T // B
    Bo, So = (1, T) if fmt == m.FMT_THD else (B, S)
    dt = torch.uint8 if mx else torch.bfloat16
    key = torch.empty(Bo, H, So, dn + dr, dtype=dt, device=DEV)
    val = torch.empty(Bo, H, So, dv, dtype=dt, device=DEV)
    ks = torch.empty(Bo, H, So, (dn + dr) // 32, dtype=torch.uint8, device=DEV) if mx else None
    vs = torch.empty(Bo, H, So, dv // 32, dtype=torch.uint8, device=DEV) if mx else None
    m.mla_kv_rope(_dev(kv), _dev(pe), key, val, H=H, d_nope=dn, d_rope=dr, d_v=dv, cos=cos, sin=sin,
                  key_scales=ks, value_scales=vs, fmt=fmt, B=B, S=S,
                  cu_seqlens=_dev(cu) if cu is not None else None, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return key, val, ks, vs


# the last case has a partial group of heads (64 + 6) and a partial chunk of
# tokens (13 = 3 x 4 + 1) in the kernel's work split
@pytest.mark.parametrize("fmt,B,S,lengths,H", [(m.FMT_BSHD, 1, 333, None, 3), (m.FMT_SBHD, 3, 77, None, 3),
                                               (m.FMT_THD, 1, None, [64, 129, 7], 3),
                                               (m.FMT_BSHD, 1, 13, None, 70)])
def test_kv_rope_against_oracle(fmt, B, S, lengths, H):
    dn, dr, dv = 128, 64, 128
    cu = syn.cu_seqlens_of(lengths) if lengths else None
    T = sum(lengths) if lengths else B * S
    max_pos = max(lengths) if lengths else S
    kv = syn.normal_bf16((T, H, dn + dv), 1.0, 180)
    pe = syn.normal_bf16((T, dr), 1.0, 181)
    cos, sin, oc, os_ = rope_tables(max_pos, dr)
    okw = dict(H=H, d_nope=dn, d_rope=dr, d_v=dv, cos=oc, sin=os_, fmt=fmt, B=B, S=S,
               cu_seqlens=cu.numpy() if cu is not None else None)
    gkw = dict(H=H, dn=dn, dr=dr, dv=dv, fmt=fmt, B=B, S=S, cu=cu, max_seqlen=max_pos, cos=cos, sin=sin)
    # bf16 outputs: k_nope and value are copies (bit-exact), the rope slice within bf16 rounding
    key, val, _, _ = run_kv(kv, pe, mx=False, **gkw)
    r = o.kv_rope(kv, pe, out_dtype="bf16", **okw)
    kb, vb = bits16(key), bits16(val)
    assert np.array_equal(vb, r.value)
    assert np.array_equal(kb[..., :dn], r.key[..., :dn])
    check_bf16(kb, r.key, "kv key bf16")
    # MXFP8 outputs
    key, val, ks, vs = run_kv(kv, pe, mx=True, **gkw)
    r = o.kv_rope(kv, pe, **okw)
    pos, bb, ss = o.token_coords(fmt, T, B, S if S else T, okw["cu_seqlens"])
    bnd = kv_bound(o.to_f64(pe), oc, os_, pos, H, dn, dv)
    g = key.cpu().numpy()[bb, :, ss, :]          # back to token-major [T, H, D]
    gs = ks.cpu().numpy()[bb, :, ss, :]
    stats = check_mx(g, gs, r.key64, 2 * bnd + U32 * np.abs(r.key64), "kv key mxfp8")
    assert np.array_equal(val.cpu().numpy(), r.value) and np.array_equal(vs.cpu().numpy(), r.value_scales)
    print(f"\nkv {fmt}: {stats}", flush=True)


def test_kv_rope_dsv3_sampled():
    """DeepSeek-V3 KV side: T = 4096, 128 heads of [128 k_nope | 128 v], a 64-wide
    shared rope slice, MXFP8 outputs; sampled tokens against the oracle (the
    sampled rows as a batch of one sequence of positions `rows`, with the
    table re-indexed to those positions)."""
    T, H, dn, dr, dv = 4096, 128, 128, 64, 128
    kv = syn.normal_bf16((T, H, dn + dv), 1.0, 190)
    pe = syn.normal_bf16((T, dr), 1.0, 191)
    cos, sin, oc, os_ = rope_tables(T, dr)
    key, val, ks, vs = run_kv(kv, pe, H=H, dn=dn, dr=dr, dv=dv, mx=True, S=T, cos=cos, sin=sin)
    rows = sample_rows(T)
    n = len(rows)
    r = o.kv_rope(kv[rows], pe[rows], H=H, d_nope=dn, d_rope=dr, d_v=dv, cos=oc[rows], sin=os_[rows],
                  B=1, S=n)
    bnd = kv_bound(o.to_f64(pe[rows]), oc[rows], os_[rows], np.arange(n), H, dn, dv)
    ri = torch.from_numpy(rows).to(DEV)
    g = key[0][:, ri, :].permute(1, 0, 2).cpu().numpy()
    gs = ks[0][:, ri, :].permute(1, 0, 2).cpu().numpy()
    stats = check_mx(g, gs, r.key64, 2 * bnd + U32 * np.abs(r.key64), "kv dsv3 key")
    assert np.array_equal(val[0][:, ri, :].cpu().numpy(), r.value[0])
    assert np.array_equal(vs[0][:, ri, :].cpu().numpy(), r.value_scales[0])
    print(f"\nkv dsv3: {stats}", flush=True)


def test_kv_rope_bf16_widths_not_multiple_of_32():
    """bf16 output with k_nope 24, rope 16, value 40 (8-element units)."""
    T, H, dn, dr, dv = 100, 2, 24, 16, 40
    kv = syn.normal_bf16((T, H, dn + dv), 1.0, 200)
    pe = syn.normal_bf16((T, dr), 1.0, 201)
    cos, sin, oc, os_ = rope_tables(T, dr)
    key, val, _, _ = run_kv(kv, pe, H=H, dn=dn, dr=dr, dv=dv, mx=False, S=T, cos=cos, sin=sin)
    r = o.kv_rope(kv, pe, H=H, d_nope=dn, d_rope=dr, d_v=dv, cos=oc, sin=os_, S=T, out_dtype="bf16")
    kb = bits16(key)
    assert np.array_equal(bits16(val), r.value)
    assert np.array_equal(kb[..., :dn], r.key[..., :dn])
    check_bf16(kb, r.key, "kv key bf16 narrow")


@pytest.mark.parametrize("fp8_mfma", [False, True])
def test_bwd_mxfp8_split_reduction_small(fp8_mfma):
    """One dX tile and eight 128-value stages: the reduction over n is split in
    two (fp32 partials summed in order), on a shape the oracle does whole."""
    T, K, H, dn, dr = 128, 192, 8, 64, 64
    x = syn.normal_bf16((T, K), 1.0, 210)
    w = syn.normal_bf16((H * (dn + dr), K), 0.05, 211)
    dq = syn.normal_bf16((T, H, dn + dr), 1e-2, 212)
    g = run_bwd(dq, x, w, H=H, dn=dn, dr=dr, S=T, mx=fp8_mfma, dw_fp32=True)
    r = o.qup_backward_mxfp8(dq, x, w, H=H, d_nope=dn, d_rope=dr, cos=g["oc"], sin=g["os"], S=T)
    _check_mx_bwd(g, r, f"mx bwd split fp8_mfma={fp8_mfma}", fp8_mfma)


def test_bwd_and_kv_leave_inputs_untouched_and_repeat_bit_identically():
    """The backward (bf16 and MXFP8) and the KV side write fresh outputs only:
    every input is byte-identical afterwards, and a second run gives the same
    bits (no floating-point atomics)."""
    T, K, H, dn, dr, dv = 256, 128, 4, 64, 64, 64
    x = _dev(syn.normal_bf16((T, K), 1.0, 220))
    w = _dev(syn.normal_bf16((H * (dn + dr), K), 0.05, 221))
    dq = _dev(syn.normal_bf16((T, H, dn + dr), 1e-2, 222))
    kv = _dev(syn.normal_bf16((T, H, dn + dv), 1.0, 223))
    pe = _dev(syn.normal_bf16((T, dr), 1.0, 224))
    cos, sin, _, _ = rope_tables(T, dr)
    before = [_hash(t) for t in (x, w, dq, kv, pe, cos, sin)]
    N = H * (dn + dr)

    def run():
        outs = []
        for mx in (None, False, True):
            dq_pre = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
            dx = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
            dw = torch.empty(N, K, dtype=torch.float32, device=DEV)
            db = torch.empty(N, dtype=torch.bfloat16, device=DEV)
            kw = dict(H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, dx=dx, dw=dw, db=db, use_bias=True,
                      B=1, S=T)
            if mx is None:
                ws = torch.empty(max(m.mla_qup_bwd_workspace_size(dq, x, w, dq_pre, **kw), 1),
                                 dtype=torch.uint8, device=DEV)
                m.mla_qup_bwd(dq, x, w, dq_pre, workspace=ws, **kw)
            else:
                ws = torch.empty(m.mla_qup_bwd_mxfp8_workspace_size(dq, x, w, dq_pre, **kw), dtype=torch.uint8,
                                 device=DEV)
                m.mla_qup_bwd_mxfp8(dq, x, w, dq_pre, workspace=ws, fp8_mfma=mx, **kw)
            outs += [dq_pre, dx, dw, db]
        key = torch.empty(1, H, T, dn + dr, dtype=torch.uint8, device=DEV)
        ks = torch.empty(1, H, T, (dn + dr) // 32, dtype=torch.uint8, device=DEV)
        val = torch.empty(1, H, T, dv, dtype=torch.uint8, device=DEV)
        vs = torch.empty(1, H, T, dv // 32, dtype=torch.uint8, device=DEV)
        m.mla_kv_rope(kv, pe, key, val, H=H, d_nope=dn, d_rope=dr, d_v=dv, cos=cos, sin=sin, key_scales=ks,
                      value_scales=vs, B=1, S=T)
        torch.cuda.synchronize()
        return [_hash(t) for t in outs + [key, ks, val, vs]]

    first, second = run(), run()
    assert first == second
    assert [_hash(t) for t in (x, w, dq, kv, pe, cos, sin)] == before


@pytest.mark.parametrize("dn,dr,H", [(128, 64, 2), (32, 32, 3)])
def test_fwd_epilogue_bit_exact_on_exactly_representable_values(dn, dr, H):
    """Inputs whose every pre-quantization value is exact in float32 in any
    summation order: small-integer X and W (each W row scaled by its own power
    of two, so blocks get different exponents), an integer bias, and a cos/sin
    table of quarter turns only (c, s in {0, +-1}), passed in by the caller.
    The GPU's float32 values then equal the oracle's, so the fused epilogue's
    rotation, E8M0 scales, E4M3 codes and bf16 rounding must match the oracle
    bit for bit, with no accumulation-order allowance. dr = 64 takes the path
    that stages the table rows in LDS; 32 reads the table directly."""
    T, K = 200, 128
    D = dn + dr
    N = H * D
    rng = np.random.default_rng(230 + dr)
    xf = rng.integers(-3, 4, (T, K)).astype(np.float32)
    wf = (rng.integers(-3, 4, (N, K)) * np.exp2(rng.integers(-4, 5, (N, 1)))).astype(np.float32)
    bf = (rng.integers(-40, 41, (N,)) * 0.25).astype(np.float32)
    x, w, bias = (torch.from_numpy(a).to(torch.bfloat16) for a in (xf, wf, bf))
    quarter = rng.integers(0, 4, (T, dr // 2))
    oc = np.choose(quarter, [1.0, 0.0, -1.0, 0.0]).astype(np.float32)
    os_ = np.choose(quarter, [0.0, 1.0, 0.0, -1.0]).astype(np.float32)
    cos, sin = torch.from_numpy(oc).to(DEV), torch.from_numpy(os_).to(DEV)
    for out_dtype in ("mxfp8", "bf16"):
        mx = out_dtype == "mxfp8"
        out = torch.empty(1, H, T, D, dtype=torch.uint8 if mx else torch.bfloat16, device=DEV)
        sc = torch.empty(1, H, T, D // 32, dtype=torch.uint8, device=DEV) if mx else None
        m.mla_qup_fwd(_dev(x), _dev(w), out, H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, bias=_dev(bias),
                      out_scales=sc, B=1, S=T)
        torch.cuda.synchronize()
        r = o.qup_forward(x, w, H=H, d_nope=dn, d_rope=dr, cos=oc, sin=os_, B=1, S=T, bias=bias,
                          out_dtype=out_dtype)
        if mx:
            assert np.array_equal(sc.cpu().numpy(), r.scales)
            assert np.array_equal(out.cpu().numpy(), r.out)
        else:
            assert np.array_equal(bits16(out), r.out)
