"""Tree-mask verify for the oracle (test infrastructure only).

Speculative decoding with Medusa heads samples several candidates per future
position and checks them as a tree in one forward pass of the target model;
the pages' example is a complete binary tree over 4 levels, 15 nodes
("Chapter 18: Speculative Decoding and Serving Optimizations", arunshar.com,
section 18.1.2, the passage on tree-based speculative decoding for Medusa).
The candidates are verified under a tree attention mask ("07 - Inference",
lourdhu02.github.io, section 3.4, the table of drafters, Medusa row).

Readings (the pages fix no layout):

* a tree of T nodes is given by parents[j] for j = 0 .. T-1, with
  parents[j] < j (nodes numbered from the root towards the leaves) and -1 for
  a node that hangs directly on the committed context (the root);
* the T nodes' keys and values sit in the cache at the sequence's last T
  positions, node j at position L - T + j, where the context length L counts
  them, as the q_len new tokens of a causal verify do;
* node j attends to every position before the tree and to the tree nodes on
  its own path to the root, itself included: never to a sibling or to another
  branch.  A chain (parents[j] = j - 1) is then the causal verify of
  "07 - Inference", section 3;
* the library's contract for a parent outside [-1, j) (not a tree): the walk
  towards the root stops there, as at -1.
"""

from __future__ import annotations

import numpy as np

from .attention import BLOCK_SIZE, _check, attend_row, gather_sequence, kv_head_of, to_f64


def path_to_root(parents, j: int) -> list:
    """Node j and its ancestors, from j up to the root (walk parents while they point to an earlier node)."""
    path = [j]
    cur = j
    while True:
        p = int(parents[cur])
        if p < 0 or p >= cur:
            return path
        path.append(p)
        cur = p


def visible_positions(context_len: int, parents, j: int) -> np.ndarray:
    """Cache positions node j attends to, ascending: the context before the tree, then its path to the root."""
    T = len(parents)
    base = context_len - T
    tree = sorted(base + a for a in path_to_root(parents, j))
    pos = list(range(max(base, 0))) + [p for p in tree if 0 <= p < context_len]
    return np.array(pos, dtype=np.int64)


def paged_tree_decode_rows(q, k_cache, v_cache, block_tables, context_lens, parents, scale, dtype, rows,
                           block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Tree-mask attention for the listed (b, j, h) rows, [len(rows), d] float64.

    q is [num_seqs * T, n_h, d] (node j of sequence b is row b * T + j); parents
    is [num_seqs, T] (one tree per sequence).  Paging and attention are those
    of attention.paged_decode_rows; only the set of visible positions differs.
    """
    parents = np.asarray(parents)
    T = parents.shape[1]
    S, n_h, n_kv, d, G = _check(q, k_cache, v_cache, block_tables, context_lens, T)
    scale64 = float(np.float32(scale))
    out = np.empty((len(rows), d), dtype=np.float64)
    cache = {}
    for i, (b, j, h) in enumerate(rows):
        L = int(context_lens[b])
        g = kv_head_of(h, G)
        if (b, g) not in cache:
            K = to_f64(gather_sequence(k_cache, block_tables[b], L, block_size)[:, g, :], dtype)
            V = to_f64(gather_sequence(v_cache, block_tables[b], L, block_size)[:, g, :], dtype)
            cache[(b, g)] = (K, V)
        K, V = cache[(b, g)]
        vis = visible_positions(L, parents[b], j)
        if len(vis) == 0:  # the library's contract: a row that sees no position is 0
            out[i] = 0.0
            continue
        out[i] = attend_row(to_f64(q[b * T + j, h], dtype), K[vis], V[vis], scale64)
    return out


def paged_tree_decode(q, k_cache, v_cache, block_tables, context_lens, parents, scale, dtype,
                      block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Full output [num_seqs * T, n_h, d] in float64."""
    parents = np.asarray(parents)
    S, T = parents.shape
    n_h, d = q.shape[1], q.shape[2]
    rows = [(b, j, h) for b in range(S) for j in range(T) for h in range(n_h)]
    flat = paged_tree_decode_rows(q, k_cache, v_cache, block_tables, context_lens, parents, scale, dtype, rows,
                                  block_size)
    return flat.reshape(S * T, n_h, d)
