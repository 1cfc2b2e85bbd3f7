"""Oracle: the Ulysses layout transform, by index definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "feat(dspark): add Ulysses sequence parallel training", Modifications.
Inputs are sharded and padded across the sequence-parallel group, and separate
Q/K/V all-to-alls turn each rank's sequence slice (all heads) into the full
sequence restricted to that rank's heads; head counts must divide the Ulysses
degree. Readings taken where the page is silent:
  * padding goes at the global tail before sharding, so every slice has
    S_pad / P rows (only the last slice holds padding);
  * padded rows are zero;
  * rank r owns the contiguous head block [r*H/P, (r+1)*H/P).

On one device the P ranks' packs followed by the all-to-all compose into one
map, X[S_real, H, d] -> Y[P, S_pad, H/P, d]:
    Y[r, s, h, :] = X[s, r*H/P + h, :]   for s < S_real
    Y[r, s, h, :] = 0                    for S_real <= s < S_pad
and the unpack (reverse all-to-all followed by each rank's unpack) is its
inverse on the real rows. Both are bit copies, so the oracle works on any
numpy dtype (bf16 is handled as its raw uint16 bits).
"""
from __future__ import annotations

import numpy as np


def padded_len(s_real: int, p: int) -> int:
    """Smallest multiple of the Ulysses degree p that holds s_real rows."""
    if p < 1 or s_real < 0:
        raise ValueError("p must be >= 1 and s_real >= 0")
    return p * ((s_real + p - 1) // p)


def pad_pack_seq2head(x: np.ndarray, p: int) -> np.ndarray:
    """[S_real, H, d] -> [P, S_pad, H/P, d], zero rows at the global tail."""
    s_real, h, d = x.shape
    if h % p != 0:
        raise ValueError("head count must be divisible by the Ulysses degree")
    hp = h // p
    s_pad = padded_len(s_real, p)
    y = np.zeros((p, s_pad, hp, d), dtype=x.dtype)
    for r in range(p):
        y[r, :s_real] = x[:, r * hp:(r + 1) * hp, :]
    return y


def unpack_head2seq(y: np.ndarray, s_real: int) -> np.ndarray:
    """[P, S_pad, H/P, d] -> [S_real, H, d]; padded rows are dropped."""
    p, s_pad, hp, d = y.shape
    if s_real > s_pad:
        raise ValueError("s_real exceeds the padded length")
    x = np.empty((s_real, p * hp, d), dtype=y.dtype)
    for r in range(p):
        x[:, r * hp:(r + 1) * hp, :] = y[r, :s_real]
    return x
