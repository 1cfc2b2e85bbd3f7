"""Seeded synthetic workloads for the Ulysses rank-share attention path.

This module is shared by the tests, the benchmark and the CPU oracle's
callers. It holds shapes, seeds and random draws only: no step of the
attention or permute arithmetic lives here.

Workloads (the shapes come from the pages' long-context runs: a 120,000-token
Qwen3-8B-like run sharded 8 ways over the sequence, and a 131,072-token
packed-document run, see "feat(dspark): add Ulysses sequence parallel
training", Accuracy Test, and "GLM-5.2 131k context parallelism", Purpose):

  name        S        P  full model     per rank   d    dtype  passes
  tiny        512      2  8 Q / 4 KV     4 Q / 2 KV 64   fp32   fwd+bwd
  s8k         8192     8  32 Q / 8 KV    4 Q / 1 KV 128  bf16   fwd
  s32k        32768    8  32 Q / 8 KV    4 Q / 1 KV 128  bf16   fwd+bwd
  s120k       120000   8  32 Q / 8 KV    4 Q / 1 KV 128  bf16   fwd+bwd
  s120k_pad   119999   8  (padded to 120000; padded keys masked)
  thd131k     131072   2  32 Q / 8 KV    16 Q / 4 KV 128 bf16   fwd+bwd,
              packed documents, block-diagonal causal mask

Recipe: every tensor is drawn at the full model's sequence-major shape
[S, H, d] with numpy's ``default_rng([cfg, variant, tensor])``
``standard_normal(dtype=float32)``; bf16 workloads then round that to bf16
(round-to-nearest-even, torch's ``.to(torch.bfloat16)``). ``cfg`` is the
0-based workload index (tiny=0, s8k=1, s32k=2, s120k=3, thd131k=4),
``variant`` is 1 for the 119,999-token case and 0 otherwise, ``tensor`` is
0=Q, 1=K, 2=V, 3=dO, 4=document lengths, 9=row sample.
"""
from __future__ import annotations

import dataclasses

import numpy as np

Q, K, V, DO, DOCS, ROWS = 0, 1, 2, 3, 4, 9


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: int
    variant: int
    s: int            # real sequence length (tokens)
    p: int            # Ulysses degree simulated on one GPU
    hq_full: int      # query heads of the full model
    hkv_full: int     # key/value heads of the full model
    d: int            # head dimension
    dtype: str        # "fp32" or "bf16"
    backward: bool    # whether the workload runs the backward pass
    thd: bool = False # packed documents (block-diagonal causal mask)

    @property
    def s_pad(self) -> int:
        return self.p * (-(-self.s // self.p))

    @property
    def hq(self) -> int:
        return self.hq_full // self.p

    @property
    def hkv(self) -> int:
        return self.hkv_full // self.p

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 0, 0, 512, 2, 8, 4, 64, "fp32", True),
        Workload("s8k", 1, 0, 8192, 8, 32, 8, 128, "bf16", False),
        Workload("s32k", 2, 0, 32768, 8, 32, 8, 128, "bf16", True),
        Workload("s120k", 3, 0, 120000, 8, 32, 8, 128, "bf16", True),
        Workload("s120k_pad", 3, 1, 119999, 8, 32, 8, 128, "bf16", True),
        Workload("thd131k", 4, 0, 131072, 2, 32, 8, 128, "bf16", True, thd=True),
    ]
}


def rng(cfg: int, variant: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([cfg, variant, tensor])


def normal_f32(cfg: int, variant: int, tensor: int, shape) -> np.ndarray:
    """N(0,1) float32 draw for one tensor of one workload."""
    return rng(cfg, variant, tensor).standard_normal(tuple(shape), dtype=np.float32)


def tensor(w: Workload, which: int, heads: int | None = None, s: int | None = None):
    """Full-model, sequence-major input tensor [S, H, d] as a torch CPU tensor.

    ``which`` is Q, K, V or DO. The dtype is the workload's (fp32 or bf16).
    ``heads`` defaults to the full model's head count for that tensor.
    """
    import torch

    if heads is None:
        heads = w.hq_full if which in (Q, DO) else w.hkv_full
    s = w.s if s is None else s
    x = torch.from_numpy(normal_f32(w.cfg, w.variant, which, (s, heads, w.d)))
    if w.dtype == "bf16":
        x = x.to(torch.bfloat16)
    return x


def doc_lengths(total: int, lo: int = 2048, hi: int = 32768,
                cfg: int = 4, variant: int = 0) -> list[int]:
    """Seeded document lengths for a packed (THD) sequence.

    Draws integers uniform in [lo, hi] one at a time until they reach
    ``total``; the last draw is cut to the remainder, so it may be shorter
    than ``lo``.
    """
    g = rng(cfg, variant, DOCS)
    out: list[int] = []
    acc = 0
    while acc < total:
        x = int(g.integers(lo, hi, endpoint=True))
        x = min(x, total - acc)
        out.append(x)
        acc += x
    return out


def cu_seqlens(lengths) -> np.ndarray:
    """Prefix offsets [0, L0, L0+L1, ...] as int32."""
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def index_sample(n: int, seed, n_uniform: int = 1024, edge: int = 64, boundaries=(),
                 lo: int = 0) -> np.ndarray:
    """Sorted distinct indexes in [lo, n): the first and last ``edge``, +-2
    around every boundary inside the range, and ``n_uniform`` seeded uniform
    draws from ``np.random.default_rng(seed)``."""
    idx = set(range(lo, min(lo + edge, n)))
    idx.update(range(max(lo, n - edge), n))
    for b in boundaries:
        idx.update(i for i in range(b - 2, b + 3) if lo <= i < n)
    g = np.random.default_rng(seed)
    idx.update(int(i) for i in g.integers(lo, n, size=n_uniform))
    return np.array(sorted(idx), dtype=np.int64)


def sample_boundaries(w: Workload) -> list[int]:
    """Slice boundaries of the rank's share and, for packed documents, the
    document boundaries: the positions the full-size samples straddle."""
    b = [r * (w.s_pad // w.p) for r in range(1, w.p)]
    if w.thd:
        b += [int(c) for c in cu_seqlens(doc_lengths(w.s))[1:-1]]
    return sorted(set(b))


def row_sample(w: Workload, n_uniform: int = 1024, edge: int = 64,
               boundaries=None) -> np.ndarray:
    """Rows (and the same set as keys) checked at full size: both ends, both
    sides of every slice or document boundary, and seeded uniform rows
    (seed [cfg, variant, 9])."""
    if boundaries is None:
        boundaries = sample_boundaries(w)
    return index_sample(w.s_pad, [w.cfg, w.variant, ROWS], n_uniform, edge, boundaries)
