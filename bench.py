#!/usr/bin/env python3
"""Benchmark of the fused MLA query up-projection on one MI355X.

One step = the whole hot path over one batch at DeepSeek-V3 shape
(T=4096 tokens, q_lora_rank K=1536, 128 heads of 128+64):
  rope_cache_build (4096 x 32 table)
  -> mla_qup_fwd: GEMM + RoPE + MXFP8 quantization, BHSD output, BF16 weight
  -> mla_qup_bwd: inverse RoPE, db, dX, dW (bias gradient on).
Throughput is the step's GEMM FLOPs (2TNK forward + 4TNK backward) over the
step time, in TFLOP/s. Inputs are seeded synthetic tensors, resident in HBM
before the timed region. The MXFP8-projection path (quantize + forward at
T=8192) and the MXFP8 quantizer are timed in separate legs after the timed
region. The CPU oracle is timed on a bounded token sample of the same step.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
METRIC = "fused Q-up-proj fwd/bwd TFLOP/s and % MFMA peak at DeepSeek-V3 shape, 1 GPU"
# Where each MXFP8-projection leg stands against the MXFP8 parity bar (every
# element of the T = 8192 workload compared with the oracle in the GPU tests).
C2_PARITY = {
    "exact_bf16_mfma": "green: meets the MXFP8 bar (2.1e-6 code flips, 0 scale mismatches)",
    "fp8_mfma": "not green: measured deviation above the MXFP8 bar (9.9e-4 code flips, "
                "3.8e-5 of codes more than one step off, 7e-6 of scales one step off)",
}
# sources compiled into the fused forward kernel (its traffic summary is tied to them)
FWD_KERNEL_SRCS = [os.path.join(ROOT, "mla_up_projection_amd", "csrc", f)
                   for f in ("qup_fwd.hip", "device_common.h", "internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qup_fwd_bf16_dsv3_traffic.md")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--legs-reps", type=int, default=20)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def fwd_kernel_sha256() -> str:
    h = hashlib.sha256()
    for f in FWD_KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def fwd_traffic():
    """HBM bytes per launch of the fused forward from the committed counter
    summary, or None if it is absent or was taken on another kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    if not m_bytes or not m_src:
        return None
    if fwd_kernel_sha256() != m_src.group(1):
        return None
    return float(m_bytes.group(1))


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operation runs on a single GPU; sharding it across GPUs is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mla_up_projection_amd as m
    from mla_up_projection_amd import synthetic as syn

    if not os.path.exists(m.LIB_PATH):
        from mla_up_projection_amd import build
        build.build()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    wf = syn.workload("dsv3_fwd_bf16w")
    wb = syn.workload("dsv3_bwd")
    T, K, H, dn, dr = wf.T, wf.K, wf.H, wf.d_nope, wf.d_rope
    D, N = wf.D, wf.N

    # ---- inputs resident in HBM ----
    x = wf.x().to(dev)
    w = wf.w().to(dev)
    dq = wb.dq().to(dev)
    cos = torch.empty(wf.S, dr // 2, dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    out = torch.empty(1, H, T, D, dtype=torch.uint8, device=dev)
    out_sc = torch.empty(1, H, T, D // 32, dtype=torch.uint8, device=dev)
    dq_pre = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
    db = torch.empty(N, dtype=torch.bfloat16, device=dev)
    bkw = dict(H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, dx=dx, dw=dw, db=db, use_bias=True,
               B=1, S=T)
    ws_bytes = m.mla_qup_bwd_workspace_size(dq, x, w, dq_pre, **bkw)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        m.rope_cache_build(cos, sin, dr, 10000.0)
        if ev is not None:
            ev[0].record(stream)
        m.mla_qup_fwd(x, w, out, H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, out_scales=out_sc,
                      B=1, S=T)
        if ev is not None:
            ev[1].record(stream)
        m.mla_qup_bwd(dq, x, w, dq_pre, workspace=ws, **bkw)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    fwd_each = np.array([e[0].elapsed_time(e[1]) for e in evs])
    bwd_each = np.array([e[1].elapsed_time(e[2]) for e in evs])
    fwd_ms = float(np.mean(fwd_each))

    def pct(a):
        return {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
                "p90_ms": float(np.percentile(a, 90))}

    flops_fwd = 2.0 * T * N * K
    flops_bwd = 4.0 * T * N * K
    tflops = (flops_fwd + flops_bwd) / (ms_step * 1e-3) / 1e12
    fwd_tflops = flops_fwd / (fwd_ms * 1e-3) / 1e12
    bwd_ms = ms_step - fwd_ms

    # ---- separate legs (after the timed region) ----
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    parts = {"qup_fwd_bf16_dsv3": {"ms": fwd_ms, "tflops": fwd_tflops,
                                   "pct_bf16_peak": 100 * fwd_tflops / BF16_PEAK_TFLOPS, **pct(fwd_each)},
             "qup_bwd_dsv3": {"ms": bwd_ms, "tflops": flops_bwd / (bwd_ms * 1e-3) / 1e12,
                              "events_mean_ms": float(np.mean(bwd_each)), **pct(bwd_each)}}
    R = args.legs_reps
    # MXFP8 projection path, T = 8192 (2 x 4096)
    w2 = syn.workload("dsv3_fwd_mxfp8w")
    x2 = w2.x().to(dev)
    xq = torch.empty(w2.T, K, dtype=torch.uint8, device=dev)
    xs = torch.empty(w2.T, K // 32, dtype=torch.uint8, device=dev)
    wq = torch.empty(N, K, dtype=torch.uint8, device=dev)
    wsc = torch.empty(N, K // 32, dtype=torch.uint8, device=dev)
    m.mxfp8_quantize(w, wq, wsc)
    out2 = torch.empty(w2.B, H, w2.S, D, dtype=torch.uint8, device=dev)
    out2_sc = torch.empty(w2.B, H, w2.S, D // 32, dtype=torch.uint8, device=dev)
    # a 9 us kernel is shorter than one Python call: time R calls captured in
    # one HIP graph, and check the replayed output against the eager one. The
    # calls rotate over copies of X totalling more than the 256 MB Infinity
    # Cache, so each call reads its input from HBM.
    m.mxfp8_quantize(x2, xq, xs)
    torch.cuda.synchronize()
    xq_ref, xs_ref = xq.clone(), xs.clone()
    x2s = [x2] + [x2.clone() for _ in range(int(300e6 // (x2.numel() * 2)))]
    qg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(qg):
        for i in range(R):
            m.mxfp8_quantize(x2s[i % len(x2s)], xq, xs)
    q_ms = timed(qg.replay, 3) / R
    if not (torch.equal(xq, xq_ref) and torch.equal(xs, xs_ref)):
        raise RuntimeError("mxfp8_quantize: graph replay differs from the eager call")
    del x2s, qg
    q_bytes = w2.T * K * (2 + 1 + 1 / 32)
    parts["mxfp8_quantize_x_8192x1536"] = {"ms": q_ms, "gbs": q_bytes / (q_ms * 1e-3) / 1e9,
                                           "pct_hbm_peak": 100 * q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    f2 = 2.0 * w2.T * N * K
    for mode, fp8 in (("exact_bf16_mfma", False), ("fp8_mfma", True)):
        ms2 = timed(lambda: m.mla_qup_fwd(xq, wq, out2, H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin,
                                          x_scales=xs, w_scales=wsc, out_scales=out2_sc, B=w2.B,
                                          S=w2.S, fp8_mfma=fp8), R)
        tf = f2 / (ms2 * 1e-3) / 1e12
        parts[f"qup_fwd_mxfp8w_dsv3_{mode}"] = {
            "ms": ms2, "tflops": tf, "pct_bf16_peak": 100 * tf / BF16_PEAK_TFLOPS,
            "pct_fp8_peak": 100 * tf / FP8_PEAK_TFLOPS, "parity": C2_PARITY[mode]}
    del x2, xq, wq, out2
    # MXFP8 backward at the same shape: operands quantized along each product's
    # reduction axis (quantization passes included), both MFMA modes
    mws_bytes = m.mla_qup_bwd_mxfp8_workspace_size(dq, x, w, dq_pre, **bkw)
    mws = torch.empty(mws_bytes, dtype=torch.uint8, device=dev)
    for mode, fp8 in (("exact_bf16_mfma", False), ("fp8_mfma", True)):
        msb = timed(lambda: m.mla_qup_bwd_mxfp8(dq, x, w, dq_pre, workspace=mws, fp8_mfma=fp8, **bkw), R)
        tfb = flops_bwd / (msb * 1e-3) / 1e12
        parts[f"qup_bwd_mxfp8_dsv3_{mode}"] = {"ms": msb, "tflops": tfb,
                                              "pct_bf16_peak": 100 * tfb / BF16_PEAK_TFLOPS,
                                              "pct_fp8_peak": 100 * tfb / FP8_PEAK_TFLOPS}
    del mws
    # packed variable-length (THD) YaRN forward, 16384 tokens, BF16 weight, MXFP8 out
    w4 = syn.workload("thd_yarn_fwd")
    x4 = w4.x().to(dev)
    cu4 = w4.cu_seqlens().to(dev)
    cos4 = torch.empty(w4.max_pos, dr // 2, dtype=torch.float32, device=dev)
    sin4 = torch.empty_like(cos4)
    m.rope_cache_build(cos4, sin4, dr, 10000.0, yarn=w4.yarn)
    out4 = torch.empty(1, H, w4.T, D, dtype=torch.uint8, device=dev)
    out4_sc = torch.empty(1, H, w4.T, D // 32, dtype=torch.uint8, device=dev)
    ms4 = timed(lambda: m.mla_qup_fwd(x4, w, out4, H=H, d_nope=dn, d_rope=dr, cos=cos4, sin=sin4,
                                      out_scales=out4_sc, fmt=m.FMT_THD, cu_seqlens=cu4,
                                      max_seqlen=w4.max_pos), R)
    tf4 = w4.flops_fwd() / (ms4 * 1e-3) / 1e12
    parts["qup_fwd_thd_yarn_16384"] = {"ms": ms4, "tflops": tf4, "pct_bf16_peak": 100 * tf4 / BF16_PEAK_TFLOPS,
                                       "sequences": len(w4.lengths)}
    del x4, out4
    # KV side at DeepSeek-V3: 128 heads of [128 k_nope | 128 v], 64-wide shared
    # rope slice, MXFP8 key and value in BHSD (one HBM pass)
    dv = 128
    kvin = syn.normal_bf16((T, H, dn + dv), 1.0, 190).to(dev)
    kpe = syn.normal_bf16((T, dr), 1.0, 191).to(dev)
    kkey = torch.empty(1, H, T, dn + dr, dtype=torch.uint8, device=dev)
    kks = torch.empty(1, H, T, (dn + dr) // 32, dtype=torch.uint8, device=dev)
    kval = torch.empty(1, H, T, dv, dtype=torch.uint8, device=dev)
    kvs = torch.empty(1, H, T, dv // 32, dtype=torch.uint8, device=dev)
    ms_kv = timed(lambda: m.mla_kv_rope(kvin, kpe, kkey, kval, H=H, d_nope=dn, d_rope=dr, d_v=dv,
                                        cos=cos, sin=sin, key_scales=kks, value_scales=kvs, B=1, S=T), R)
    kv_bytes = T * H * (dn + dv) * 2 + T * dr * 2 + T * H * (dn + dr + dv) * (1 + 1 / 32)
    parts["kv_rope_mxfp8_dsv3"] = {"ms": ms_kv, "gbs": kv_bytes / (ms_kv * 1e-3) / 1e9,
                                   "pct_hbm_peak": 100 * kv_bytes / (ms_kv * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del kvin, kpe, kkey, kks, kval, kvs
    # one rank's share under 8-way head (tensor) parallelism: the first 16
    # heads of W (N = 3072), the same 4096 tokens, forward and backward
    Hs = H // 8
    Ns = Hs * D
    w_s = w[:Ns]
    dq_s = dq.reshape(T, H, D)[:, :Hs].contiguous()
    out_s = torch.empty(1, Hs, T, D, dtype=torch.uint8, device=dev)
    out_s_sc = torch.empty(1, Hs, T, D // 32, dtype=torch.uint8, device=dev)
    dq_pre_s = torch.empty(T, Ns, dtype=torch.bfloat16, device=dev)
    bkw_s = dict(H=Hs, d_nope=dn, d_rope=dr, cos=cos, sin=sin,
                 dx=torch.empty(T, K, dtype=torch.bfloat16, device=dev),
                 dw=torch.empty(Ns, K, dtype=torch.bfloat16, device=dev),
                 db=torch.empty(Ns, dtype=torch.bfloat16, device=dev), use_bias=True, B=1, S=T)
    ws_s = torch.empty(max(m.mla_qup_bwd_workspace_size(dq_s, x, w_s, dq_pre_s, **bkw_s), 1),
                       dtype=torch.uint8, device=dev)
    ms_fs = timed(lambda: m.mla_qup_fwd(x, w_s, out_s, H=Hs, d_nope=dn, d_rope=dr, cos=cos, sin=sin,
                                        out_scales=out_s_sc, B=1, S=T), R)
    ms_bs = timed(lambda: m.mla_qup_bwd(dq_s, x, w_s, dq_pre_s, workspace=ws_s, **bkw_s), R)
    f_s = 2.0 * T * Ns * K
    parts["qup_tp8_shard_16_heads"] = {
        "fwd_ms": ms_fs, "fwd_tflops": f_s / (ms_fs * 1e-3) / 1e12,
        "bwd_ms": ms_bs, "bwd_tflops": 2 * f_s / (ms_bs * 1e-3) / 1e12}
    del dq_s, out_s, out_s_sc, dq_pre_s, bkw_s, ws_s
    # context: the vendor library GEMM (torch -> hipBLASLt) on the same three
    # products, bf16 out, with no epilogue and no inverse RoPE
    dq2 = dq.reshape(T, N)
    lib = {}
    for name, fn in (("fwd_x_wT", lambda: torch.nn.functional.linear(x, w)),
                     ("dx_dq_w", lambda: torch.mm(dq2, w)),
                     ("dw_dqT_x", lambda: torch.mm(dq2.t(), x))):
        lib[name + "_ms"] = timed(fn, R)
    parts["context_library_gemm_bf16"] = lib
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        parts["calib_copy_bytes"] = n

    traffic = fwd_traffic()
    roofline = {"bound": "mfma", "kernel": "qup_fwd_kernel<bf16> (fused GEMM+RoPE+MXFP8)",
                "achieved": fwd_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": fwd_tflops / BF16_PEAK_TFLOPS, "traffic": traffic}

    # ---- CPU oracle on a bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_sample_tokens, x, w, dq, dn, dr, H)

    line = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "pct_bf16_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "config": {"workload": "DeepSeek-V3 MLA q up-projection step: rope table + fused forward "
                               "(BF16 weight, MXFP8 BHSD out) + backward (inverse RoPE, dX, dW, db)",
                   "T": T, "K": K, "H": H, "d_nope": dn, "d_rope": dr, "seq": "1x4096",
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "parts": parts,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(ts, x, w, dq, dn, dr, H):
    """The oracle, as it stands, on the first `ts` tokens of the step's
    workload: forward (GEMM, RoPE, MXFP8) and backward for those tokens."""
    import numpy as np
    import oracle as o
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    xs, wc, dqs = x[:ts].cpu(), w.cpu(), dq[:ts].cpu()
    cos, sin = o.rope_table(4096, dr, 1e4)
    K = xs.shape[1]
    N = wc.shape[0]
    t0 = time.perf_counter()
    o.qup_forward(xs, wc, H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, B=1, S=ts)
    o.qup_backward(dqs, xs, wc, H=H, d_nope=dn, d_rope=dr, cos=cos, sin=sin, B=1, S=ts)
    dt = time.perf_counter() - t0
    flops = 6.0 * ts * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "seconds": dt, "cpu_model": cpu_model, "cores_available": len(os.sched_getaffinity(0)),
            "threads": f"{blas} threads in the float64 matrix products (the BLAS pool); "
                       "every other step of the oracle runs on one thread",
            "sample": f"first {ts} of 4096 tokens of the step (forward + backward, all 128 heads), "
                      "float64 numpy"}


if __name__ == "__main__":
    main()
