"""The oracle's output on every row of a named workload, for the full-size
parity tests.

    python tests/_oracle_full.py NAME OUT.npy [WORKERS]

Regenerates the workload from its seed (workloads.make_problem is
deterministic), stores the new tokens with the oracle's cache write, and runs
the oracle on every (sequence, query token, head) row, split by sequence over
WORKERS processes.  The result, float64 [num_seqs * q_len, num_q_heads,
head_dim], goes to OUT.npy.  It runs as a child process of the GPU test so
that the worker processes never share state with the one that drives the GPU.

Test infrastructure: it imports the oracle and the input generators only.
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import workloads as wl  # noqa: E402
from _gpu import host_caches_after_write, reference_rows  # noqa: E402

_P = _KC = _VC = None


def _rows_of(bs):
    p = _P
    rows = [(b, j, h) for b in bs for j in range(p.q_len) for h in range(p.num_q_heads)]
    return reference_rows(p, rows, _KC, _VC)


def full_output(name: str, workers: int) -> np.ndarray:
    global _P, _KC, _VC
    _P = wl.make_problem(name)
    _KC, _VC = host_caches_after_write(_P)
    p = _P
    # balance the pool by context length: longest sequences first, dealt round-robin
    order = sorted(range(p.num_seqs), key=lambda b: -int(p.context_lens[b]))
    chunks = [order[i::workers * 4] for i in range(workers * 4)]
    chunks = [c for c in chunks if c]
    if workers > 1:
        import multiprocessing as mp

        with mp.get_context("fork").Pool(workers) as pool:
            parts = pool.map(_rows_of, chunks)
    else:
        parts = [_rows_of(c) for c in chunks]
    out = np.empty((p.num_seqs * p.q_len, p.num_q_heads, p.head_dim), dtype=np.float64)
    for bs, part in zip(chunks, parts):
        part = part.reshape(len(bs), p.q_len, p.num_q_heads, p.head_dim)
        for i, b in enumerate(bs):
            out[b * p.q_len:(b + 1) * p.q_len] = part[i]
    return out


if __name__ == "__main__":
    name, path = sys.argv[1], sys.argv[2]
    workers = int(sys.argv[3]) if len(sys.argv) > 3 else 1
    np.save(path, full_output(name, workers))
