"""Seeded synthetic inputs for the fused MLA query up-projection.

This module holds none of the method's arithmetic: it only draws seeded
normal numbers (numpy PCG64), stores them as bf16 (round to nearest even,
torch's CPU cast) and draws packed-sequence lengths. The tests, the benchmark
and the smoke check use it to feed the same host tensors to the GPU library
and to the CPU oracle.

Shapes follow DeepSeek-V3's MLA query up-projection (q_lora_rank 1536, 128
heads, 128 no-position + 64 rotary dims per head), the model the forward page
("Add support for fused Q Up-Proj GEMM/RoPE/Quant.", description) names.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

FMT_BSHD = 0
FMT_SBHD = 1
FMT_THD = 2


def normal_bf16(shape, sigma: float, seed: int) -> torch.Tensor:
    """float32 N(0, sigma) from default_rng(seed), rounded to bf16 (CPU tensor)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(sigma)
    return torch.from_numpy(a).to(torch.bfloat16)


def thd_lengths(total: int, lo: int, hi: int, seed: int) -> list[int]:
    """Sequence lengths uniform in [lo, hi] from default_rng(seed), drawn until
    they cover `total` tokens; the last one is cut so the sum is exactly total."""
    rng = np.random.default_rng(seed)
    out: list[int] = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out


def cu_seqlens_of(lengths) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return torch.from_numpy(cu)


@dataclass
class Workload:
    name: str
    T: int
    K: int
    H: int
    d_nope: int
    d_rope: int
    fmt: int = FMT_BSHD
    B: int = 1
    S: int = 0
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    dq_sigma: float = 1e-3
    seeds: dict = field(default_factory=lambda: {"x": 0, "w": 1, "dq": 2, "bias": 3})
    base: float = 10000.0
    yarn: tuple | None = None        # (factor, orig_max_pos, beta_fast, beta_slow, mscale)
    lengths: list | None = None      # THD sequence lengths
    mx_weight: bool = False          # MXFP8 projection path (X and W quantized along K)
    out_dtype: str = "mxfp8"
    use_bias: bool = False
    backward: bool = False

    @property
    def D(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def N(self) -> int:
        return self.H * self.D

    @property
    def max_pos(self) -> int:
        if self.fmt == FMT_THD:
            return max(self.lengths)
        return self.S

    def x(self) -> torch.Tensor:
        return normal_bf16((self.T, self.K), self.x_sigma, self.seeds["x"])

    def w(self) -> torch.Tensor:
        return normal_bf16((self.N, self.K), self.w_sigma, self.seeds["w"])

    def dq(self) -> torch.Tensor:
        return normal_bf16((self.T, self.H, self.D), self.dq_sigma, self.seeds["dq"])

    def bias(self) -> torch.Tensor:
        return normal_bf16((self.N,), 0.1, self.seeds["bias"])

    def cu_seqlens(self) -> torch.Tensor | None:
        return cu_seqlens_of(self.lengths) if self.fmt == FMT_THD else None

    def flops_fwd(self) -> float:
        return 2.0 * self.T * self.N * self.K

    def flops_bwd(self) -> float:
        return 4.0 * self.T * self.N * self.K


def workload(name: str) -> Workload:
    """The five workloads: a tiny forward and four at DeepSeek-V3 shape."""
    if name == "tiny":
        # T=64, K=64, 2 heads of 16+16, W ~ N(0, 1/sqrt(64)), positions 0..63.
        return Workload("tiny", T=64, K=64, H=2, d_nope=16, d_rope=16, S=64,
                        x_sigma=1.0, w_sigma=0.125, out_dtype="mxfp8")
    if name == "dsv3_fwd_bf16w":
        return Workload("dsv3_fwd_bf16w", T=4096, K=1536, H=128, d_nope=128, d_rope=64, S=4096)
    if name == "dsv3_fwd_mxfp8w":
        return Workload("dsv3_fwd_mxfp8w", T=8192, K=1536, H=128, d_nope=128, d_rope=64,
                        B=2, S=4096, mx_weight=True)
    if name == "dsv3_bwd":
        return Workload("dsv3_bwd", T=4096, K=1536, H=128, d_nope=128, d_rope=64, S=4096,
                        use_bias=True, backward=True)
    if name == "thd_yarn_fwd":
        lengths = thd_lengths(16384, 512, 4096, seed=7)
        return Workload("thd_yarn_fwd", T=16384, K=1536, H=128, d_nope=128, d_rope=64,
                        fmt=FMT_THD, S=16384, lengths=lengths,
                        yarn=(40.0, 4096, 32.0, 1.0, 1.0))
    raise KeyError(name)


WORKLOADS = ("tiny", "dsv3_fwd_bf16w", "dsv3_fwd_mxfp8w", "dsv3_bwd", "thd_yarn_fwd")
