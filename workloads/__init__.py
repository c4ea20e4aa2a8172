"""Seeded synthetic attention inputs shared by the tests, the bench and the oracle checks.

This module only draws random numbers and arranges them into tensors. It holds no
step of the quantized-attention method (no scaling, rounding or reduction of the
method), so the HIP path and the CPU oracle can both be fed from it without
sharing any of the method's arithmetic.

Workloads stand in for the attention layers of the diffusion transformers that the
pages time end to end (no weights or prompts are available here):

* ``flux_like``: a 1024x1024 Flux image is 64x64 latent patches plus 512 text
  tokens, N = 4608 (apatero page "TeaCache和SageAttention优化实现更快的AI图像生成",
  section on Flux performance).
* ``video``: 21 latent frames of 30x52 patches, N = 32760, the shape class of the
  video models timed on the apatero page and of the 864x480 MiniMax H3 clip on the
  juejin page "MiniMax H3 接入 SageAttention 实测加速" (section 七).
* ``sweep8k``/``sweep16k``/``stress``: the 8K/16K/65K token lengths at which the
  sd114.wiki page on ComfyUI-sol-attn ("核心亮点" item 1) times its INT8 kernel.

Distributions: Q and V are standard normal. K is standard normal plus a per-head,
per-channel bias drawn from N(0, 3^2) and shared by all tokens (the channel-wise
offset that K smoothing is meant to remove). ``outliers`` channels per head are
then multiplied, bias and noise together, by 20.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "get"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    outliers: int = 0          # outlier K channels per head, scaled x20
    seed: int = 0

    @property
    def ops(self) -> float:
        """Operation count of one attention call: 4*B*H*N^2*d (both products)."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=2, N=256, d=64),
    "flux_like": Workload("flux_like", B=1, H=24, N=4608, d=128),
    "sweep8k": Workload("sweep8k", B=1, H=24, N=8192, d=128),
    "sweep16k": Workload("sweep16k", B=1, H=24, N=16384, d=128),
    "video": Workload("video", B=1, H=40, N=32760, d=128),
    "stress": Workload("stress", B=1, H=24, N=65536, d=128, outliers=4),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def make_qkv(w: Workload, dtype=torch.bfloat16):
    """Return (q, k, v) as CPU tensors of shape [B, N, H, d] (the layout a DiT qkv
    projection yields), drawn from ``torch.Generator('cpu').manual_seed(w.seed)`` in
    the fixed order Q, V, K-noise, K-bias, outlier channel picks."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    shape = (w.B, w.N, w.H, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    bias = torch.randn((w.H, w.d), generator=g, dtype=torch.float32) * 3.0
    k += bias
    if w.outliers:
        for h in range(w.H):
            idx = torch.randperm(w.d, generator=g)[: w.outliers]
            k[:, :, h, idx] *= 20.0
    return q.to(dtype), k.to(dtype), v.to(dtype)
