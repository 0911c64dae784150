"""The allocation-free backward (mla_qup_bwd_noalloc) against the workspace
backward (mla_qup_bwd) on the GPU: two calls in a row, the second smaller, so
the second runs on scratch that still holds the first call's partials. The
outputs must be bit-identical (same plan, same kernels, same summation
order)."""
import numpy as np
import pytest
import torch

import mla_up_projection_amd as m
from mla_up_projection_amd import synthetic as syn

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(T, H, K, seed, use_bias=True):
    dn, dr = 128, 64
    N = H * (dn + dr)
    x = syn.normal_bf16((T, K), 1.0, seed).to(DEV)
    w = syn.normal_bf16((N, K), 0.02, seed + 1).to(DEV)
    dq = syn.normal_bf16((T, H, dn + dr), 1e-3, seed + 2).to(DEV)
    cos = torch.empty(T, dr // 2, dtype=torch.float32, device=DEV)
    sin = torch.empty_like(cos)
    m.rope_cache_build(cos, sin, dr, 1e4)
    return x, w, dq, cos, sin, dict(H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, use_bias=use_bias, B=1, S=T)


def _outs(T, N, K, use_bias):
    return dict(dq_pre=torch.full((T, N), 7.0, dtype=torch.bfloat16, device=DEV),
                dx=torch.full((T, K), 7.0, dtype=torch.bfloat16, device=DEV),
                dw=torch.full((N, K), 7.0, dtype=torch.bfloat16, device=DEV),
                db=torch.full((N,), 7.0, dtype=torch.bfloat16, device=DEV) if use_bias else None)


def test_bwd_noalloc_matches_workspace_backward_twice():
    # DeepSeek-V3 shape first (db partials and dX split partials: 56.6 MB of the
    # 64 MiB scratch), then a smaller ragged call
    for T, H, K, seed in ((4096, 128, 1536, 300), (333, 3, 256, 310)):
        print(f"\nnoalloc backward T={T} H={H} K={K}", flush=True)
        x, w, dq, cos, sin, kw = _case(T, H, K, seed)
        N = H * 192
        ref = _outs(T, N, K, True)
        nbytes = m.mla_qup_bwd_workspace_size(dq, x, w, ref["dq_pre"], dx=ref["dx"], dw=ref["dw"], db=ref["db"], **kw)
        assert nbytes <= m.binding.MLA_BWD_SCRATCH_BYTES
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
        m.mla_qup_bwd(dq, x, w, ref["dq_pre"], dx=ref["dx"], dw=ref["dw"], db=ref["db"],
                      workspace=ws if nbytes else None, **kw)
        got = _outs(T, N, K, True)
        m.mla_qup_bwd_noalloc(dq, x, w, got["dq_pre"], dx=got["dx"], dw=got["dw"], db=got["db"], **kw)
        torch.cuda.synchronize()
        for k in ("dq_pre", "dx", "dw", "db"):
            assert torch.equal(got[k].view(torch.int16), ref[k].view(torch.int16)), k
        assert torch.isfinite(got["dx"].float()).all()


def test_bwd_noalloc_refuses_more_than_its_scratch():
    # 2^16 tokens x 128 heads: db partials of 1024 bands x 24576 x 4 B = 100 MB
    T, H, K = 1 << 16, 128, 32
    x = torch.zeros(T, K, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(H * 192, K, dtype=torch.bfloat16, device=DEV)
    dq = torch.zeros(T, H, 192, dtype=torch.bfloat16, device=DEV)
    cos = torch.ones(T, 32, device=DEV)
    o = _outs(T, H * 192, K, True)
    with pytest.raises(m.MlaError) as e:
        m.mla_qup_bwd_noalloc(dq, x, w, o["dq_pre"], dx=o["dx"], dw=o["dw"], db=o["db"], H=H, d_nope=128,
                              d_rope=64, cos=cos, sin=cos, use_bias=True, B=1, S=T)
    assert e.value.status == m.binding.MLA_ESCRATCH
    # nothing was written
    assert (o["db"].float() == 7.0).all()
