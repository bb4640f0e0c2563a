"""Named workload shapes.

The full-size shapes follow the pages' workloads: a lightning-indexer decode
at 128K context with an fp8 K-index and a 576-wide latent KV ("XM-Sparse"
blog: 2,048 selected entries per layer, 4,096-token hot buffer), a 64-token
block-sparse decode over two layers that share one selection ("MiniMax-M3"
PR), and a Fathom bit-plane scan at one million tokens.  The small shapes are
the same methods at sizes the CPU oracle finishes in seconds; they span
several tiles and end in ragged tails.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "dot" | "lightning" | "block" | "fathom"
    B: int
    n: int               # cached tokens per request (capacity)
    k: int               # selected units per row (tokens, or blocks)
    idx_heads: int       # index query heads
    idx_dim: int         # index key / query dim
    hq: int              # attention query heads
    hkv: int             # attention KV heads
    d_qk: int
    d_v: int
    dtype: str = "bf16"  # attention / index query dtype ("f32" or "bf16")
    block: int = 1       # selection unit in tokens
    page: int = 0        # paged latent KV page size (0 = contiguous)
    budget: int = 0      # Fathom bits per key per KV head
    layers: int = 1      # layers sharing one selection
    hot: int = 0         # hot-buffer tokens per request (0 = all KV in HBM)
    miss_rate: float = 0.0
    seq_lens: tuple | None = None  # per-request valid lengths (None = all n)
    seed: int = 0
    meta: dict = field(default_factory=dict, compare=False)

    @property
    def mla(self) -> bool:
        return self.kind == "lightning"

    @property
    def sm_scale(self) -> float:
        """The softmax scale of the workload's attention: 1/sqrt(d_qk) (the
        fp32 workload states 1/sqrt(128); the latent workloads take the
        same rule over the 576-wide query/key rows)."""
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def n_units(self) -> int:
        return (self.n + self.block - 1) // self.block

    def valid(self, b: int) -> int:
        return self.n if self.seq_lens is None else self.seq_lens[b]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _w(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS: dict[str, Workload] = {}


def _reg(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


# --- full-size shapes -------------------------------------------------------
TINY_FP32 = _reg(_w(name="tiny_fp32", kind="dot", B=1, n=8192, k=256,
                    idx_heads=8, idx_dim=128, hq=8, hkv=1, d_qk=128, d_v=128,
                    dtype="f32", seed=1001))
LIGHTNING_128K = _reg(_w(name="lightning_128k", kind="lightning", B=32,
                         n=131072, k=2048, idx_heads=64, idx_dim=128, hq=128,
                         hkv=1, d_qk=576, d_v=512, page=64, seed=1002))
BLOCK_80K = _reg(_w(name="block_sparse_80k", kind="block", B=16, n=81920,
                    k=32, idx_heads=8, idx_dim=128, hq=64, hkv=8, d_qk=128,
                    d_v=128, block=64, layers=2, seed=1003))
FATHOM_1M = _reg(_w(name="fathom_1m", kind="fathom", B=1, n=1048576, k=2048,
                    idx_heads=32, idx_dim=128, hq=32, hkv=8, d_qk=128,
                    d_v=128, budget=92, seed=1004))
HOT_16K = _reg(_w(name="hot_16k", kind="lightning", B=241, n=16384, k=2048,
                  idx_heads=64, idx_dim=128, hq=128, hkv=1, d_qk=576,
                  d_v=512, hot=4096, miss_rate=0.2, seed=1005))
HOT_128K = _reg(_w(name="hot_128k", kind="lightning", B=109, n=131072,
                   k=2048, idx_heads=64, idx_dim=128, hq=128, hkv=1,
                   d_qk=576, d_v=512, hot=4096, miss_rate=0.2, seed=1006))

# --- small shapes for element-by-element parity -----------------------------
TINY_FP32_SMALL = _reg(TINY_FP32.with_(name="tiny_fp32_small", B=3, n=3000,
                                       k=256, seq_lens=(3000, 2049, 200),
                                       seed=2001))
LIGHTNING_SMALL = _reg(LIGHTNING_128K.with_(name="lightning_small", B=3,
                                            n=5000, k=512,
                                            seq_lens=(5000, 4097, 300),
                                            seed=2002))
BLOCK_SMALL = _reg(BLOCK_80K.with_(name="block_sparse_small", B=3, n=4100,
                                   k=8, seq_lens=(4100, 2050, 300),
                                   seed=2003))
FATHOM_SMALL = _reg(FATHOM_1M.with_(name="fathom_small", B=2, n=20000,
                                    k=300, seq_lens=(20000, 9001),
                                    seed=2004))
HOT_SMALL = _reg(HOT_16K.with_(name="hot_small", B=3, n=6000, k=512,
                               hot=1024, seq_lens=(6000, 5000, 2500),
                               seed=2005))


def get(name: str) -> Workload:
    return WORKLOADS[name]
