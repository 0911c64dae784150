"""The C ABI without a GPU: the library loads, exports every function that
include/mla_qup.h declares, and every validation error is returned before
anything is enqueued (fake device addresses are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import mla_up_projection_amd as m
from mla_up_projection_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bd.LIB_PATH):
        from mla_up_projection_amd import build
        build.build()
    return bd.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mla_qup.h")).read()
    return sorted(set(re.findall(r"MLA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(bd.FUNCTIONS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in range(8):
        assert m.mla_status_str(code).startswith("MLA_")
    assert "unknown" in m.mla_status_str(99)


def test_struct_layouts_match_c(tmp_path):
    """sizeof/offsetof of every ABI struct as gcc lays it out == the ctypes mirror."""
    structs = [bd.mla_tokens, bd.mla_yarn, bd.mla_rope, bd.mla_qup_fwd_args, bd.mla_qup_bwd_args,
               bd.mla_kv_args]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mla_qup.h"', "int main(void){"]
    for s in structs:
        lines.append(f'printf("{s.__name__} %zu\\n", sizeof({s.__name__}));')
        for f, _ in s._fields_:
            lines.append(f'printf("{s.__name__}.{f} %zu\\n", offsetof({s.__name__}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for s in structs:
        assert int(out[s.__name__]) == ctypes.sizeof(s), s.__name__
        for f, _ in s._fields_:
            assert int(out[f"{s.__name__}.{f}"]) == getattr(s, f).offset, (s.__name__, f)


# Fake, 256-byte-aligned, far-apart device addresses: validation only compares
# and aligns them.
BASE = 0x7F0000000000
def addr(i, off=0):
    return BASE + i * (1 << 36) + off


def fwd_args(**over):
    a = bd.mla_qup_fwd_args()
    T, K, H, dn, dr = 256, 1536, 4, 128, 64
    a.x, a.x_dtype = addr(1), bd.DTYPE_BF16
    a.w, a.w_dtype = addr(2), bd.DTYPE_BF16
    a.K, a.H, a.d_nope, a.d_rope = K, H, dn, dr
    a.tokens.fmt, a.tokens.B, a.tokens.S, a.tokens.T = bd.FMT_BSHD, 1, T, T
    a.rope.cos, a.rope.sin, a.rope.rows, a.rope.pairs = addr(3), addr(4), T, dr // 2
    a.out_dtype, a.out, a.out_scales = bd.DTYPE_MXFP8, addr(5), addr(6)
    for k, v in over.items():
        obj = a
        *path, last = k.split("__")
        for p in path:
            obj = getattr(obj, p)
        setattr(obj, last, v)
    return a


def fwd(L, **over):
    return L.mla_qup_fwd(ctypes.byref(fwd_args(**over)), None)


@pytest.mark.parametrize("over,code", [
    (dict(K=0), bd.MLA_EINVAL),
    (dict(K=100), bd.MLA_EINVAL),
    (dict(H=0), bd.MLA_EINVAL),
    (dict(d_rope=63), bd.MLA_EINVAL),
    (dict(d_nope=120), bd.MLA_EINVAL),                    # D = 184 not a multiple of 32
    (dict(tokens__B=2), bd.MLA_EINVAL),                   # B*S != T
    (dict(tokens__fmt=7), bd.MLA_EINVAL),
    (dict(x=0), bd.MLA_EINVAL),
    (dict(out=0), bd.MLA_EINVAL),
    (dict(out_scales=0), bd.MLA_EINVAL),
    (dict(x=addr(1, 8)), bd.MLA_EINVAL),                  # misaligned
    (dict(out_dtype=9), bd.MLA_EINVAL),
    (dict(x_dtype=bd.DTYPE_MXFP8), bd.MLA_EUNSUPPORTED),  # MXFP8 x with BF16 w
    (dict(rope__pairs=31), bd.MLA_EROPE_TABLE),           # table narrower than d_rope/2
    (dict(rope__rows=255), bd.MLA_EROPE_TABLE),           # no row for position 255
    (dict(rope__cos=0), bd.MLA_EINVAL),
    (dict(out=addr(1, 4096)), bd.MLA_EALIAS),             # output inside x
    (dict(out_scales=addr(5, 64)), bd.MLA_EALIAS),        # scales inside out
    (dict(out=addr(3)), bd.MLA_EALIAS),                   # output over the cos table
    (dict(rope__cos=addr(3, 4)), bd.MLA_EINVAL),          # table 4-B aligned: 16 needed
    (dict(rope__sin=addr(4, 8)), bd.MLA_EINVAL),
    (dict(bias=addr(11, 2)), bd.MLA_EINVAL),              # bias 2-B aligned: 8 needed
    (dict(bias=addr(11, 4)), bd.MLA_EINVAL),
])
def test_fwd_validation(L, over, code):
    assert fwd(L, **over) == code


def test_fwd_validation_mx_and_thd(L):
    mx = dict(x_dtype=bd.DTYPE_MXFP8, w_dtype=bd.DTYPE_MXFP8)
    assert fwd(L, **mx) == bd.MLA_EINVAL                          # scales missing
    assert fwd(L, **mx, x_scales=addr(7), w_scales=addr(8), K=1600) == bd.MLA_EINVAL  # K % 128
    # operand scales are read as dwords: 4-byte alignment
    assert fwd(L, **mx, x_scales=addr(7, 2), w_scales=addr(8)) == bd.MLA_EINVAL
    assert fwd(L, **mx, x_scales=addr(7), w_scales=addr(8, 1)) == bd.MLA_EINVAL
    thd = dict(tokens__fmt=bd.FMT_THD, tokens__cu_seqlens=addr(9), tokens__nseq=2,
               tokens__max_seqlen=200)
    assert fwd(L, **{**thd, "tokens__nseq": 0}) == bd.MLA_EINVAL
    assert fwd(L, **{**thd, "tokens__cu_seqlens": 0}) == bd.MLA_EINVAL
    assert fwd(L, **{**thd, "rope__rows": 199}) == bd.MLA_EROPE_TABLE
    assert fwd(L, **{**thd, "out": addr(9, 0)}) == bd.MLA_EALIAS
    # zero tokens: valid, nothing enqueued (no GPU needed)
    assert fwd(L, tokens__T=0, tokens__S=0, tokens__B=1) == bd.MLA_EINVAL  # S < 1
    assert fwd(L, **{**thd, "tokens__T": 0}) == bd.MLA_OK
    # the table check runs before the zero-token return: 16-byte aligned
    # tables are accepted, 4- and 8-byte aligned ones are not
    assert fwd(L, **{**thd, "tokens__T": 0, "rope__cos": addr(3, 16), "rope__sin": addr(4, 48)}) == bd.MLA_OK
    assert fwd(L, **{**thd, "tokens__T": 0, "rope__cos": addr(3, 8)}) == bd.MLA_EINVAL


def bwd_args(**over):
    a = bd.mla_qup_bwd_args()
    T, K, H, dn, dr = 256, 1536, 4, 128, 64
    a.dq, a.x, a.w = addr(1), addr(2), addr(3)
    a.K, a.H, a.d_nope, a.d_rope = K, H, dn, dr
    a.tokens.fmt, a.tokens.B, a.tokens.S, a.tokens.T = bd.FMT_BSHD, 1, T, T
    a.rope.cos, a.rope.sin, a.rope.rows, a.rope.pairs = addr(4), addr(5), T, dr // 2
    a.dq_pre, a.dx, a.dw, a.dw_dtype = addr(6), addr(7), addr(8), bd.DTYPE_BF16
    a.use_bias, a.db = 1, addr(9)
    a.workspace, a.workspace_bytes = addr(10), 1 << 30
    for k, v in over.items():
        obj = a
        *path, last = k.split("__")
        for p in path:
            obj = getattr(obj, p)
        setattr(obj, last, v)
    return a


def test_bwd_workspace_size(L):
    a = bwd_args()
    need = L.mla_qup_bwd_workspace_size(ctypes.byref(a))
    assert need > 0 and need % 256 == 0
    b = bwd_args(use_bias=0, dx=0)
    assert L.mla_qup_bwd_workspace_size(ctypes.byref(b)) == 0
    assert L.mla_qup_bwd_workspace_size(ctypes.byref(bwd_args(K=10))) == 0


def test_bwd_workspace_holds_dw_token_splits(L):
    # H = 2 (N = 384), K = 192: 3 dW output tiles. T = 1000 is 16 token stages
    # of 64 (2 splits of 8), T = 1500 is 24 (3 of 8), T = 2000 is 32 (4 of 8):
    # fp32 partials [splits, N, K] in the workspace, none when dW is not
    # requested.
    N, K = 384, 192
    for T, s in ((1000, 2), (1500, 3), (2000, 4)):
        kw = dict(H=2, K=K, tokens__T=T, tokens__S=T, rope__rows=T, use_bias=0, dx=0)
        assert L.mla_qup_bwd_workspace_size(ctypes.byref(bwd_args(**kw))) == s * N * K * 4
        assert L.mla_qup_bwd_workspace_size(ctypes.byref(bwd_args(**kw, dw=0))) == 0
    # 16 heads (one rank of 8-way head parallelism), T = 4096: 192 tiles, 2 splits
    kw = dict(H=16, tokens__T=4096, tokens__S=4096, rope__rows=4096, use_bias=0, dx=0)
    assert L.mla_qup_bwd_workspace_size(ctypes.byref(bwd_args(**kw))) == 2 * 3072 * 1536 * 4
    # all 128 heads: 1536 tiles fill the chip, no split
    kw = dict(H=128, tokens__T=4096, tokens__S=4096, rope__rows=4096, use_bias=0, dx=0)
    assert L.mla_qup_bwd_workspace_size(ctypes.byref(bwd_args(**kw))) == 0


def test_bwd_workspace_db_bands(L):
    # db partials: one fp32 column-sum row per token band of the inverse-RoPE
    # grid, whose band is the most rows (64, 32, 16 or 8) that still give 1536
    # workgroups of 1024 columns. 128 heads (24 column blocks), T = 4096: 64-row
    # bands; 16 heads (3 column blocks): 8-row bands.
    for H, band in ((128, 64), (16, 8)):
        kw = dict(H=H, tokens__T=4096, tokens__S=4096, rope__rows=4096, dx=0, dw=0)
        assert L.mla_qup_bwd_workspace_size(ctypes.byref(bwd_args(**kw))) == (4096 // band) * H * 192 * 4


@pytest.mark.parametrize("over,code", [
    (dict(db=0), bd.MLA_EINVAL),                 # use_bias without a db buffer
    (dict(use_bias=2), bd.MLA_EINVAL),
    (dict(dq_pre=0), bd.MLA_EINVAL),
    (dict(dw_dtype=bd.DTYPE_MXFP8), bd.MLA_EINVAL),
    (dict(workspace=0), bd.MLA_EWORKSPACE),
    (dict(workspace_bytes=1024), bd.MLA_EWORKSPACE),
    (dict(workspace=addr(10, 16)), bd.MLA_EINVAL),
    (dict(rope__pairs=16), bd.MLA_EROPE_TABLE),
    (dict(dx=addr(1, 512)), bd.MLA_EALIAS),      # dx inside dq
    (dict(dw=addr(6, 1024)), bd.MLA_EALIAS),     # dw inside dq_pre
    (dict(db=addr(10, 4096)), bd.MLA_EALIAS),    # db inside the workspace
    (dict(rope__cos=addr(4, 4)), bd.MLA_EINVAL),  # table rows read 16 bytes at a time
    (dict(rope__sin=addr(5, 8)), bd.MLA_EINVAL),
])
def test_bwd_validation(L, over, code):
    assert L.mla_qup_bwd(ctypes.byref(bwd_args(**over)), None) == code


def test_bwd_noalloc_validation(L):
    """The allocation-free backward validates like mla_qup_bwd (its workspace
    arguments are ignored) and refuses, with its own status, a call whose db
    partials exceed the static scratch."""
    nows = dict(workspace=0, workspace_bytes=0)
    assert L.mla_qup_bwd_noalloc(ctypes.byref(bwd_args(**nows, db=0)), None) == bd.MLA_EINVAL
    assert L.mla_qup_bwd_noalloc(ctypes.byref(bwd_args(**nows, rope__pairs=16)), None) == bd.MLA_EROPE_TABLE
    assert L.mla_qup_bwd_noalloc(ctypes.byref(bwd_args(**nows, dx=addr(1, 512))), None) == bd.MLA_EALIAS
    # 2^20 tokens x 768 columns: db partials of 16384 bands x 768 x 4 B = 48 MiB fit;
    # 128 heads (N = 24576): 1.5 GiB do not
    big = dict(nows, tokens__T=1 << 20, tokens__S=1 << 20, rope__rows=1 << 20, H=128)
    assert L.mla_qup_bwd_noalloc(ctypes.byref(bwd_args(**big)), None) == bd.MLA_ESCRATCH
    assert "MLA_BWD_SCRATCH_BYTES" in m.mla_status_str(bd.MLA_ESCRATCH)


def test_bwd_mxfp8_workspace_and_validation(L):
    # T = 256, N = 4 * 192 = 768, K = 1536: db partials (one column-sum row per
    # 128-token band, the band of the fused pass over dq), then the quantized
    # operands, each 256-byte aligned (all of these sizes already are); dX needs
    # no split here (16 tiles, 6 stages of 128).
    T, N, K = 256, 768, 1536
    db_part = (T // 128) * N * 4
    expect = db_part + T * N + T * N // 32 + N * T + N * T // 32 + K * N + K * N // 32 \
        + K * T + K * T // 32
    assert L.mla_qup_bwd_mxfp8_workspace_size(ctypes.byref(bwd_args())) == expect
    assert L.mla_qup_bwd_mxfp8_workspace_size(ctypes.byref(bwd_args(use_bias=0))) == expect - db_part
    # N = 3 * 192 = 576 is not a multiple of 128
    assert L.mla_qup_bwd_mxfp8_workspace_size(ctypes.byref(bwd_args(H=3))) == 0
    assert L.mla_qup_bwd_mxfp8(ctypes.byref(bwd_args(H=3)), 0, None) == bd.MLA_EUNSUPPORTED
    assert L.mla_qup_bwd_mxfp8(ctypes.byref(bwd_args()), 2, None) == bd.MLA_EINVAL
    small = L.mla_qup_bwd_workspace_size(ctypes.byref(bwd_args()))
    assert L.mla_qup_bwd_mxfp8(ctypes.byref(bwd_args(workspace_bytes=small)), 0, None) == bd.MLA_EWORKSPACE
    assert L.mla_qup_bwd_mxfp8(ctypes.byref(bwd_args(db=addr(10, 4096))), 1, None) == bd.MLA_EALIAS


def test_quantize_t_validation(L):
    q = L.mxfp8_quantize_t
    assert q(addr(1), 40, 60, 64, 64, addr(2), addr(3), None) == bd.MLA_EINVAL    # cols % 8
    assert q(addr(1), 40, 64, 60, 64, addr(2), addr(3), None) == bd.MLA_EINVAL    # ld < cols
    assert q(addr(1), 40, 64, 68, 64, addr(2), addr(3), None) == bd.MLA_EINVAL    # ld % 8
    assert q(addr(1), 40, 64, 64, 48, addr(2), addr(3), None) == bd.MLA_EINVAL    # rows_pad % 32
    assert q(addr(1), 40, 64, 64, 32, addr(2), addr(3), None) == bd.MLA_EINVAL    # rows_pad < rows
    assert q(addr(1, 8), 40, 64, 64, 64, addr(2), addr(3), None) == bd.MLA_EINVAL  # x alignment
    assert q(addr(1), 40, 64, 64, 64, addr(1, 256), addr(3), None) == bd.MLA_EALIAS
    assert q(addr(1), 0, 64, 64, 0, 0, 0, None) == bd.MLA_OK


def kv_args(**over):
    a = bd.mla_kv_args()
    T, H, dn, dr, dv = 256, 4, 128, 64, 128
    a.kv, a.k_pe = addr(1), addr(2)
    a.H, a.d_nope, a.d_rope, a.d_v = H, dn, dr, dv
    a.tokens.fmt, a.tokens.B, a.tokens.S, a.tokens.T = bd.FMT_BSHD, 1, T, T
    a.rope.cos, a.rope.sin, a.rope.rows, a.rope.pairs = addr(3), addr(4), T, dr // 2
    a.out_dtype = bd.DTYPE_MXFP8
    a.key, a.key_scales, a.value, a.value_scales = addr(5), addr(6), addr(7), addr(8)
    for k, v in over.items():
        obj = a
        *path, last = k.split("__")
        for p in path:
            obj = getattr(obj, p)
        setattr(obj, last, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(H=0), bd.MLA_EINVAL),
    (dict(d_nope=12), bd.MLA_EINVAL),                   # not a multiple of 8
    (dict(d_nope=0, d_rope=0, d_v=0), bd.MLA_EINVAL),
    (dict(d_v=48), bd.MLA_EINVAL),                      # MXFP8 needs whole 32-blocks
    (dict(out_dtype=7), bd.MLA_EINVAL),
    (dict(rope__pairs=16), bd.MLA_EROPE_TABLE),
    (dict(rope__rows=100), bd.MLA_EROPE_TABLE),
    (dict(k_pe=0), bd.MLA_EINVAL),
    (dict(key_scales=0), bd.MLA_EINVAL),
    (dict(kv=addr(1, 8)), bd.MLA_EINVAL),               # alignment
    (dict(key=addr(1, 1024)), bd.MLA_EALIAS),            # key inside kv
    (dict(value=addr(5, 4096)), bd.MLA_EALIAS),          # value inside key
    (dict(value_scales=addr(2, 64)), bd.MLA_EALIAS),     # scales inside k_pe
    (dict(tokens__T=0, tokens__S=1, tokens__B=1), bd.MLA_EINVAL),  # B*S != T
    (dict(rope__cos=addr(3, 4)), bd.MLA_EINVAL),         # tables 16-byte aligned
])
def test_kv_rope_validation(L, over, code):
    assert L.mla_kv_rope(ctypes.byref(kv_args(**over)), None) == code


def test_kv_rope_zero_tokens_and_bf16_widths(L):
    thd = dict(tokens__fmt=bd.FMT_THD, tokens__cu_seqlens=addr(9), tokens__nseq=1,
               tokens__max_seqlen=8, tokens__T=0)
    assert L.mla_kv_rope(ctypes.byref(kv_args(**thd)), None) == bd.MLA_OK
    # bf16 output needs only multiples of 8
    assert L.mla_kv_rope(ctypes.byref(kv_args(**thd, out_dtype=bd.DTYPE_BF16, d_v=40)), None) == bd.MLA_OK


def test_rope_and_quantize_validation(L):
    y = bd.mla_yarn(40.0, 4096, 32.0, 1.0, 1.0)
    assert L.rope_cache_build(None, addr(2), 16, 64, 1e4, None, None) == bd.MLA_EINVAL
    assert L.rope_cache_build(addr(1), addr(2), 16, 63, 1e4, None, None) == bd.MLA_EINVAL
    assert L.rope_cache_build(addr(1), addr(2), 16, 64, 1.0, None, None) == bd.MLA_EINVAL
    bad = bd.mla_yarn(0.0, 4096, 32.0, 1.0, 1.0)
    assert L.rope_cache_build(addr(1), addr(2), 16, 64, 1e4, ctypes.byref(bad), None) == bd.MLA_EINVAL
    assert L.rope_cache_build(addr(1), addr(1, 64), 16, 64, 1e4, ctypes.byref(y), None) == bd.MLA_EALIAS
    assert L.mxfp8_quantize(addr(1), bd.DTYPE_MXFP8, 4, 64, 64, addr(2), addr(3), None) == bd.MLA_EINVAL
    assert L.mxfp8_quantize(addr(1), bd.DTYPE_BF16, 4, 48, 48, addr(2), addr(3), None) == bd.MLA_EINVAL
    assert L.mxfp8_quantize(addr(1), bd.DTYPE_BF16, 4, 64, 60, addr(2), addr(3), None) == bd.MLA_EINVAL
    assert L.mxfp8_quantize(addr(1), bd.DTYPE_BF16, 4, 64, 64, addr(1, 64), addr(3), None) == bd.MLA_EALIAS
    assert L.mxfp8_quantize(addr(1), bd.DTYPE_BF16, 0, 64, 64, 0, 0, None) == bd.MLA_OK


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIB_PATH", "/nonexistent/libmlaqup.so")
    with pytest.raises(RuntimeError, match="missing"):
        bd.lib()


# ------------------------------------------------- binding argument checks --
# The binding checks every tensor before a pointer crosses the C ABI, which
# cannot tell a host address or a short buffer from a good one. "meta" tensors
# stand in for device tensors here (no GPU, no data).
@pytest.fixture
def meta(monkeypatch):
    monkeypatch.setattr(bd, "DEVICE_TYPE", "meta")
    return lambda *shape, dt=torch.bfloat16, dev="meta": torch.empty(*shape, dtype=dt, device=dev)


def _fwd_kw(t, T=64, K=64, H=2, dn=16, dr=16):
    D = dn + dr
    return dict(x=t(T, K), w=t(H * D, K), out=t(1, H, T, D, dt=torch.uint8),
                out_scales=t(1, H, T, D // 32, dt=torch.uint8), cos=t(T, dr // 2, dt=torch.float32),
                sin=t(T, dr // 2, dt=torch.float32), H=H, d_nope=dn, d_rope=dr, B=1, S=T)


def test_binding_rejects_host_cu_seqlens(meta):
    kw = _fwd_kw(meta)
    kw.update(fmt=bd.FMT_THD, S=None, max_seqlen=64)
    cu_host = torch.tensor([0, 30, 64], dtype=torch.int32)          # built on the CPU
    x, w, out = kw.pop("x"), kw.pop("w"), kw.pop("out")
    with pytest.raises(ValueError, match="cu_seqlens is on cpu"):
        m.mla_qup_fwd(x, w, out, cu_seqlens=cu_host, **kw)
    # an int64 cu_seqlens on the device is refused too (the kernels read int32)
    with pytest.raises(ValueError, match="cu_seqlens has dtype torch.int64"):
        m.mla_qup_fwd(x, w, out, cu_seqlens=meta(3, dt=torch.int64), **kw)


@pytest.mark.parametrize("name,shape,dt", [
    ("out", (1, 2, 63, 32), torch.uint8),         # one token row short
    ("out_scales", (1, 2, 64, 0), torch.uint8),
    ("w", (63, 64), torch.bfloat16),              # fewer than H*D rows
    ("w", (64, 64), torch.float16),               # wrong dtype
    ("cos", (64, 8), torch.float16),
])
def test_binding_rejects_undersized_or_mistyped_fwd_tensors(meta, name, shape, dt):
    kw = _fwd_kw(meta)
    kw[name] = meta(*shape, dt=dt)
    if name == "cos":
        kw["sin"] = meta(*shape, dt=dt)
    x, w, out = kw.pop("x"), kw.pop("w"), kw.pop("out")
    with pytest.raises(ValueError, match=name):
        m.mla_qup_fwd(x, w, out, **kw)


def test_binding_rejects_host_tensor_and_mixed_devices(meta):
    kw = _fwd_kw(meta)
    x, w, out = kw.pop("x"), kw.pop("w"), kw.pop("out")
    with pytest.raises(ValueError, match="x is on cpu"):
        m.mla_qup_fwd(torch.empty(64, 64, dtype=torch.bfloat16), w, out, **kw)
    with pytest.raises(ValueError, match="not contiguous|contiguous"):
        m.mla_qup_fwd(meta(64, 128)[:, ::2], w, out, **kw)


@pytest.mark.parametrize("name,shape,dt", [
    ("dq_pre", (64, 63), torch.bfloat16),
    ("dx", (64, 32), torch.bfloat16),
    ("dw", (64, 64), torch.float16),
    ("db", (32,), torch.bfloat16),
    ("workspace", (16,), torch.float32),
])
def test_binding_rejects_bad_bwd_tensors(meta, name, shape, dt):
    T, K, H, dn, dr = 64, 64, 2, 16, 16
    N = H * (dn + dr)
    args = dict(dq=meta(T, H, dn + dr), x=meta(T, K), w=meta(N, K), dq_pre=meta(T, N))
    kw = dict(H=H, d_nope=dn, d_rope=dr, cos=meta(T, dr // 2, dt=torch.float32),
              sin=meta(T, dr // 2, dt=torch.float32), dx=meta(T, K), dw=meta(N, K), db=meta(N),
              use_bias=True, workspace=meta(1024, dt=torch.uint8), B=1, S=T)
    tgt = args if name in args else kw
    tgt[name] = meta(*shape, dt=dt)
    with pytest.raises(ValueError, match=name):
        m.mla_qup_bwd(args["dq"], args["x"], args["w"], args["dq_pre"], **kw)


def test_binding_rejects_bad_quantize_and_kv_tensors(meta):
    x = meta(8, 64)
    with pytest.raises(ValueError, match="codes"):
        m.mxfp8_quantize(x, meta(8, 63, dt=torch.uint8), meta(8, 2, dt=torch.uint8))
    with pytest.raises(ValueError, match="scales"):
        m.mxfp8_quantize(x, meta(8, 64, dt=torch.uint8), meta(8, 1, dt=torch.uint8))
    with pytest.raises(ValueError, match="x is on cpu"):
        m.mxfp8_quantize(torch.empty(8, 64, dtype=torch.bfloat16), meta(8, 64, dt=torch.uint8),
                         meta(8, 2, dt=torch.uint8))
    with pytest.raises(ValueError, match="codes_t"):
        m.mxfp8_quantize_t(x, meta(64, 16, dt=torch.uint8), meta(64, 1, dt=torch.uint8), rows_pad=32)
    T, H, dn, dr, dv = 16, 2, 32, 32, 32
    kv, pe = meta(T, H, dn + dv), meta(T, dr)
    key, val = meta(1, H, T, dn + dr, dt=torch.uint8), meta(1, H, T, dv, dt=torch.uint8)
    tab = dict(cos=meta(T, dr // 2, dt=torch.float32), sin=meta(T, dr // 2, dt=torch.float32))
    with pytest.raises(ValueError, match="value_scales"):
        m.mla_kv_rope(kv, pe, key, val, H=H, d_nope=dn, d_rope=dr, d_v=dv, key_scales=meta(1, H, T, 2, dt=torch.uint8),
                      value_scales=meta(1, H, T, 2, dt=torch.uint8), B=1, S=T, **tab)
    with pytest.raises(ValueError, match="rope_cache_build"):
        m.rope_cache_build(meta(T, 16, dt=torch.float32), meta(T, 16, dt=torch.float32), 64)
