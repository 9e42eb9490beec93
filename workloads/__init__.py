"""Seeded synthetic workloads for the Diffuser attention-diffusion path.

This module holds only workload descriptions and seeded input generators. It
contains none of the method's arithmetic and is the one module that both the
HIP path's callers and the oracle's callers share.

The five workloads stand in for the pages' settings: the headline shape is the
continued-MLM configuration of the Diffuser reading notes (section 3.1:
length 4096, 12 heads of width 64, window / global / random budget 64, K=5,
alpha=0.1); the 16384-token one stands in for long-document inputs (TriviaQA
documents average about 11.6K tokens, ImageNet-64 sequences are 12,288 long,
section 3.1-3.2). No dataset is read: Q, K, V are iid normal draws.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    d: int
    dtype: str               # "f32" or "bf16" (storage); accumulation is fp32
    radius: int
    global_idx: tuple
    num_random: int
    num_graphs: int          # 1 (shared by every (b, h)) or B (one per batch element)
    K: int = 5
    alpha: float = 0.1
    causal: bool = False
    data_seed: int = 0
    graph_seed: int = 0
    scale: float = 1.0       # multiplies the N(0, 1) draws

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def describe(self) -> str:
        g = len(self.global_idx)
        return (f"{self.name}: B={self.B} H={self.H} n={self.n} d={self.d} {self.dtype} "
                f"r={self.radius} g={g} R={self.num_random} graphs={self.num_graphs} "
                f"K={self.K} alpha={self.alpha} causal={int(self.causal)}")


def evenly_spaced(n: int, g: int) -> tuple:
    """g global positions floor(k*n/g), k < g."""
    return tuple((k * n) // g for k in range(g))


def _cfg(c, **kw):
    return Workload(data_seed=2000 + c, graph_seed=1000 + c, **kw)


WORKLOADS = {
    # 1 batch, 1 head, n=512, d=64, fp32; globals {0, 256}; 8 random per token.
    "small_f32": _cfg(1, name="small_f32", B=1, H=1, n=512, d=64, dtype="f32", radius=32,
                      global_idx=(0, 256), num_random=8, num_graphs=1),
    # batch 32, 8 heads, n=1024, d=32, bf16, N(0,1)/sqrt(2); 16 evenly spaced globals.
    "batch_bf16": _cfg(2, name="batch_bf16", B=32, H=8, n=1024, d=32, dtype="bf16",
                       radius=32, global_idx=evenly_spaced(1024, 16), num_random=16,
                       num_graphs=1, scale=2 ** -0.5),
    # headline: batch 8, 12 heads, n=4096, d=64, bf16; globals = first 64 positions;
    # 64 random per token, one graph per batch element.
    "mlm4096_bf16": _cfg(3, name="mlm4096_bf16", B=8, H=12, n=4096, d=64, dtype="bf16",
                         radius=64, global_idx=tuple(range(64)), num_random=64,
                         num_graphs=8),
    # long document: batch 1, 12 heads, n=16384, d=64, bf16; 128 evenly spaced globals.
    "long16k_bf16": _cfg(4, name="long16k_bf16", B=1, H=12, n=16384, d=64, dtype="bf16",
                         radius=128, global_idx=evenly_spaced(16384, 128), num_random=128,
                         num_graphs=1),
    # sweep base: batch 4, 8 heads, n=8192, d=64, fp32; 32 evenly spaced globals.
    "sweep8192_f32": _cfg(5, name="sweep8192_f32", B=4, H=8, n=8192, d=64, dtype="f32",
                          radius=64, global_idx=evenly_spaced(8192, 32), num_random=128,
                          num_graphs=1),
}

HEADLINE = "mlm4096_bf16"


def sweep_variants() -> List[Workload]:
    """The n=8192 fp32 sweep: random budget {0,32,128} x K {1,3,5,10} x
    alpha {0.05,0.1,0.3} x {bidirectional, causal}."""
    base = WORKLOADS["sweep8192_f32"]
    out = []
    for causal in (False, True):
        for R in (0, 32, 128):
            for K in (1, 3, 5, 10):
                for a in (0.05, 0.1, 0.3):
                    out.append(replace(base, name=f"sweep8192_f32_R{R}_K{K}_a{a}_c{int(causal)}",
                                       num_random=R, K=K, alpha=a, causal=causal))
    return out


def make_qkv(w: Workload, device: str = "cpu", B: Optional[int] = None):
    """Q, K, V of shape [B, H, n, d] from torch.randn on a CPU generator seeded
    with w.data_seed, drawn in the order Q, K, V, scaled, then cast to the
    storage dtype with round-to-nearest-even."""
    B = w.B if B is None else B
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.data_seed)
    out = []
    for _ in range(3):
        x = torch.randn(B, w.H, w.n, w.d, generator=gen, dtype=torch.float32)
        if w.scale != 1.0:
            x = x * w.scale
        out.append(x.to(w.torch_dtype).to(device))
    return tuple(out)


def make_tensor(shape, seed: int, dtype=torch.float32, scale: float = 1.0, device="cpu"):
    """One seeded N(0, scale^2) tensor (used by the small randomized cases)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randn(*shape, generator=gen, dtype=torch.float32) * scale
    return x.to(dtype).to(device)
