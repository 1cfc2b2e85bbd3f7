"""Writes the stored expected dK / dV values of the full-size GPU parity tests
(tests/golden/full_size_keys/*.npz).

At 120K tokens and more, dK and dV of a key early in the sequence depend on
the LSE and D of every later row, so the oracle needs a whole forward pass
(about 15 TFLOP in fp64) per workload: minutes on a host, too slow to repeat
in every GPU test run. This script runs it once. It calls only the fp64
oracle (oracle/) and the seeded input generator (workloads/): no value comes
from the GPU library.

For each case the keys are the full-size sample (the first and last 64
positions, +-2 around every slice, ring-block and document boundary, and 1024
seeded uniform positions: the same set as the sampled query rows), and the
values are oracle.attn_bwd_keys over the case's query rows, with the sums
of the absolute values of each element's terms (AdK, AdV: the per-element
rounding bound of the bf16 path is derived from them). The oracle runs in
fp64; the stored dK / dV are rounded to float32 (a relative 6e-8, far below
the 2e-2 / 2e-3 bars) and AdK / AdV to float16 (bounds, needed to 3 digits).
Each file also holds a SHA-256 of the bf16 input bits, which the GPU test
checks before comparing.

Cases (the GPU tests build the same inputs):
  s32k, s120k, s120k_pad,    rank 0's share of the workload after the pack
  thd131k                    (full attention, all rows);
  usp_u2r4_120k              one GPU of Ulysses 2 x Ring 4 at S = 120000:
                             Q/K/V/dO heads of Ulysses group 0 (16 Q / 4 KV),
                             contributions of the last ring rank's rows
                             [90000, 120000) only.

Usage: python tests/golden/make_full_size_keys.py [case ...]   (8 processes)
"""
from __future__ import annotations

import hashlib
import multiprocessing as mp
import os
import sys
import time

os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")
os.environ.setdefault("OMP_NUM_THREADS", "1")
os.environ.setdefault("MKL_NUM_THREADS", "1")

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "full_size_keys")
USP_U, USP_R = 2, 4

_SHARED = {}


def bits(t):
    import torch
    return t.contiguous().view(torch.int16).numpy()


def fingerprint(arrays_bits) -> str:
    h = hashlib.sha256()
    for a in arrays_bits:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def case_inputs(name):
    """(bf16 bit arrays of Q, K, V, dO as the GPU test builds them, sequence
    length s, s_valid, cu_seqlens or None, scale, key sample, query interval)."""
    import torch
    if name == "usp_u2r4_120k":
        w = workloads.WORKLOADS["s120k"]
        xb = []
        for t in (workloads.Q, workloads.K, workloads.V, workloads.DO):
            full = workloads.tensor(w, t)
            xb.append(bits(full[:, : full.shape[1] // USP_U]))
            del full
        blk = w.s // USP_R
        keys = workloads.index_sample(w.s, [w.cfg, 7, 9], 1024, 64, [blk, 2 * blk, 3 * blk])
        return xb, w.s, w.s, None, w.scale, keys, ((USP_R - 1) * blk, w.s)
    w = workloads.WORKLOADS[name]
    cu = workloads.cu_seqlens(workloads.doc_lengths(w.s)).tolist() if w.thd else None
    xb = []
    for t in (workloads.Q, workloads.K, workloads.V, workloads.DO):
        x = workloads.tensor(w, t)
        xb.append(oracle.pad_pack_seq2head(bits(x), w.p)[0])
        del x
    return xb, w.s_pad, w.s, cu, w.scale, workloads.row_sample(w), (0, w.s_pad)


def _f64(b):
    import torch
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.bfloat16).double().numpy()


def _work(interval):
    a, b = interval
    sh = _SHARED
    return oracle.attn_bwd_keys(sh["q"], sh["k"], sh["v"], sh["do"], sh["keys"], sh["scale"],
                                sh["s_valid"], sh["cu"], True, q_lo=a, q_hi=b, with_abs=True)


def make(name, procs=8):
    t0 = time.time()
    xb, s, s_valid, cu, scale, keys, (qa, qb) = case_inputs(name)
    _SHARED.update(q=_f64(xb[0]), k=_f64(xb[1]), v=_f64(xb[2]), do=_f64(xb[3]), keys=keys,
                   scale=scale, s_valid=s_valid, cu=cu)
    # row intervals of about equal causal work, summed in order afterwards
    edges = np.unique(np.round(np.sqrt(np.linspace(qa * qa, qb * qb, 4 * procs + 1))).astype(int))
    edges[0], edges[-1] = qa, qb
    intervals = list(zip(edges[:-1].tolist(), edges[1:].tolist()))
    with mp.get_context("fork").Pool(procs) as pool:
        parts = pool.map(_work, intervals, chunksize=1)
    dk, dv, adk, adv = (np.zeros_like(parts[0][i]) for i in range(4))
    for a, b, c, e in parts:
        dk += a
        dv += b
        adk += c
        adv += e
    os.makedirs(OUT, exist_ok=True)
    path = os.path.join(OUT, f"{name}.npz")
    np.savez_compressed(path, keys=keys, dk=dk.astype(np.float32), dv=dv.astype(np.float32),
                        adk=adk.astype(np.float16), adv=adv.astype(np.float16),
                        inputs_sha256=np.array(fingerprint(xb)), q_lo=qa, q_hi=qb,
                        s_valid=s_valid)
    print(f"{name}: {len(keys)} keys, rows [{qa}, {qb}), {time.time() - t0:.0f} s -> {path}",
          flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or ["s32k", "s120k", "s120k_pad", "thd131k", "usp_u2r4_120k"]
    for n in names:
        make(n)
