"""The five synthetic KV workloads the codec is measured and tested on.

Shapes follow the model families named on the pages: Llama-7B (the 622 MB -> 176 MB
example in the gptget.net summary of CacheGen, "Key Results"), Llama-3-8B (the
compression table in "Guide to CacheGen", Evaluation) and Llama-3-70B (the size
formula examples in "Guide to CacheGen", Problem).  Bin counts are per layer,
finer for early layers ("Guide to CacheGen", Solution pillar 1).

Pure data: no codec arithmetic lives here.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple


@dataclass(frozen=True)
class GenSpec:
    """Recipe of the synthetic generator (see synth.py)."""
    rho: float                 # AR(1) coefficient along tokens, same for every channel
    heavy_tail: bool           # False: Gaussian innovations; True: Student-t(3), unit variance
    outlier_frac: float        # fraction of channels whose scale is multiplied
    outlier_mult: float        # the multiplier
    seed: int = 0


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    H_kv: int
    d: int
    S: int
    group: int                 # anchor interval G
    chunk: int                 # tokens per chunk (one stream per (layer, K/V, channel, chunk))
    bins: Tuple[int, ...]      # per-layer bin count N_l
    gen: GenSpec
    levels: Tuple[Tuple[int, ...], ...] = field(default=())  # extra bin schedules (streamed case)

    @property
    def C(self) -> int:
        return self.H_kv * self.d

    @property
    def raw_bytes(self) -> int:
        # 2 (K and V) * L * H_kv * d * S * sizeof(fp16)
        return 2 * self.L * self.H_kv * self.d * self.S * 2

    @property
    def n_chunks(self) -> int:
        return -(-self.S // self.chunk)


def tiered(L: int, tiers: List[Tuple[int, int]]) -> Tuple[int, ...]:
    """Expand [(n_layers, bins), ...] into a per-layer tuple; the last tier fills up."""
    out: List[int] = []
    for n, b in tiers:
        out.extend([b] * n)
    if len(out) < L:
        out.extend([tiers[-1][1]] * (L - len(out)))
    return tuple(out[:L])


_GAUSS = GenSpec(rho=0.9, heavy_tail=False, outlier_frac=0.02, outlier_mult=20.0, seed=0)
_HEAVY = GenSpec(rho=0.85, heavy_tail=True, outlier_frac=0.01, outlier_mult=30.0, seed=0)

TINY = Workload("tiny", L=2, H_kv=2, d=64, S=256, group=10, chunk=256,
                bins=(8, 8), gen=_GAUSS)
LLAMA7B = Workload("llama7b", L=32, H_kv=32, d=128, S=1216, group=10, chunk=256,
                   bins=tiered(32, [(8, 32), (8, 16), (16, 8)]), gen=_GAUSS)
LLAMA3_8B = Workload("llama3_8b", L=32, H_kv=8, d=128, S=32768, group=10, chunk=1024,
                     bins=tiered(32, [(8, 32), (8, 16), (16, 8)]), gen=_HEAVY)
LLAMA3_70B = Workload("llama3_70b", L=80, H_kv=8, d=128, S=32768, group=10, chunk=1536,
                      bins=tiered(80, [(20, 32), (20, 16), (40, 8)]), gen=_HEAVY)
LLAMA3_70B_131K = Workload(
    "llama3_70b_131k", L=80, H_kv=8, d=128, S=131072, group=10, chunk=1536,
    bins=tiered(80, [(20, 32), (20, 16), (40, 8)]), gen=_HEAVY,
    levels=(tiered(80, [(20, 32), (20, 16), (40, 8)]),
            tiered(80, [(20, 16), (20, 8), (40, 4)]),
            tiered(80, [(20, 8), (20, 4), (40, 2)])))

ALL = {w.name: w for w in (TINY, LLAMA7B, LLAMA3_8B, LLAMA3_70B, LLAMA3_70B_131K)}
