"""Plain fp64 CPU oracle for the Ulysses rank-share hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with
the HIP library (no kernels, headers, helpers or tables) and imports nothing
from the product package.

Contents
  permute    pad + pack (sequence-sharded -> head-sharded) and its inverse,
             written out from their index definitions.
  attention  exact grouped-query attention forward (textbook softmax over
             materialised score rows) and its closed-form backward, with the
             causal, key-padding and packed-document masks; attention between
             a query interval and a key interval (global positions), the
             log-sum-exp merge of partial results, and the per-interval
             backward contributions.

Pins (see tests/test_oracle_*.py): a hand-derived worked example
(tests/golden), torch's float64 scaled_dot_product_attention with autograd
on the CPU, central finite differences, closed forms (first row, K = 0,
V = const, padded query), the sequence-parallel invariant (pack, per-rank
attention, unpack equals full-model attention), a brute-force simulated
all-to-all for the pack, and the exact gradient identities.
"""
from .permute import padded_len, pad_pack_seq2head, unpack_head2seq
from .attention import (
    doc_of,
    allowed_keys,
    attn_fwd,
    attn_bwd,
    attn_fwd_rows,
    attn_bwd_rows,
    attn_bwd_keys,
    attn_fwd_partial,
    attn_bwd_partial,
    lse_merge,
)

__all__ = [
    "padded_len",
    "pad_pack_seq2head",
    "unpack_head2seq",
    "doc_of",
    "allowed_keys",
    "attn_fwd",
    "attn_bwd",
    "attn_fwd_rows",
    "attn_bwd_rows",
    "attn_bwd_keys",
    "attn_fwd_partial",
    "attn_bwd_partial",
    "lse_merge",
]
