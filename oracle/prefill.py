"""Chunked-prefill attention over the paged cache, for the oracle (test infrastructure only).

A long prompt is cut into chunks (for example 512 tokens) that are processed
one per engine step ("Chapter 18: Speculative Decoding and Serving
Optimizations", arunshar.com, section 18.2.1, on chunking long prefills; "LLM
serving: KV cache, batching, paged attention and quantization",
learn.mohebi.ai, section 3.6; "07 - Inference", lourdhu02.github.io, section
2.4).  Each chunk's keys and values go into the cache, and every token of the
chunk attends to the whole cached prefix and to the chunk's earlier tokens;
the result equals a single prefill of the whole prompt (the lab check the
last page names).

Readings:

* one call holds sequences with different numbers of new tokens, given by
  query_start[S + 1] (sequence b owns query rows query_start[b] ..
  query_start[b + 1] - 1): a prefill chunk, or a single decode token;
* context_lens counts the new tokens; new token i of sequence b sits at
  position L_b - n_b + i and sees positions 0 .. L_b - n_b + i (the causal
  mask of the decode oracle, with a per-sequence q_len);
* a row that sees no position (L_b < n_b) is 0, the library's contract.
"""

from __future__ import annotations

import numpy as np

from .attention import BLOCK_SIZE, attend_row, gather_sequence, kv_head_of, to_f64


def visible_count(context_len: int, n_new: int, i: int) -> int:
    """Positions new token i of a sequence with n_new new tokens and context_len cached tokens
    (the new ones included) may see: 0 .. context_len - n_new + i."""
    return context_len - n_new + i + 1


def query_counts(query_start) -> np.ndarray:
    qs = np.asarray(query_start, dtype=np.int64)
    return qs[1:] - qs[:-1]


def query_row(query_start, b: int, i: int) -> int:
    """Row of q (and of the output) holding new token i of sequence b."""
    return int(query_start[b]) + i


def paged_prefill_rows(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype, rows,
                       block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Attention for the listed (b, i, h) rows (new token i of sequence b, query head h),
    [len(rows), d] float64.  q is [query_start[-1], n_h, d]."""
    qs = np.asarray(query_start, dtype=np.int64)
    n = query_counts(qs)
    n_h, d = q.shape[1], q.shape[2]
    n_kv = k_cache.shape[2]
    assert q.shape[0] == qs[-1] and n_h % n_kv == 0 and (n >= 0).all()
    G = n_h // n_kv
    scale64 = float(np.float32(scale))
    out = np.empty((len(rows), d), dtype=np.float64)
    cache = {}
    for r, (b, i, h) in enumerate(rows):
        L = int(context_lens[b])
        g = kv_head_of(h, G)
        if (b, g) not in cache:
            K = to_f64(gather_sequence(k_cache, block_tables[b], L, block_size)[:, g, :], dtype)
            V = to_f64(gather_sequence(v_cache, block_tables[b], L, block_size)[:, g, :], dtype)
            cache[(b, g)] = (K, V)
        K, V = cache[(b, g)]
        visible = visible_count(L, int(n[b]), i)
        if visible <= 0:
            out[r] = 0.0
            continue
        out[r] = attend_row(to_f64(q[query_row(qs, b, i), h], dtype), K[:visible], V[:visible], scale64)
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype,
                  block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Full output [query_start[-1], n_h, d] in float64."""
    n = query_counts(query_start)
    n_h = q.shape[1]
    rows = [(b, i, h) for b in range(len(n)) for i in range(int(n[b])) for h in range(n_h)]
    flat = paged_prefill_rows(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype, rows,
                              block_size)
    return flat.reshape(q.shape[0], n_h, q.shape[2])
