"""Pins of the tree-mask verify oracle (oracle/tree.py).

Independent routes:
* dense attention with torch's scaled_dot_product_attention in float64 over
  contiguous K/V, under a boolean mask built from node labels: every node is
  the string of branch choices from the root, and node i is visible to node j
  exactly when i's label is a prefix of j's (the tree attention of Medusa,
  "Chapter 18: Speculative Decoding and Serving Optimizations", arunshar.com,
  section 18.1.2; "07 - Inference", lourdhu02.github.io, section 3.4);
* the pages' 15-node complete binary tree, whose ancestor rule has a closed
  form in heap numbering, with an exact count probe (identical keys, one-hot
  values) that reveals every node's visible set and its size (depth + 1);
* a chain reduces exactly to the causal verify oracle;
* a node's output does not move when a node off its path changes.
Each planted mistake (below) fails at least one of them.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import tree as ot
from _pins import build_paged, torch_widen


def trie(T, rng, roots=1):
    """A random tree as labels (tuples of branch choices) and the parent array they imply."""
    labels = [(r,) for r in range(roots)]
    while len(labels) < T:
        i = int(rng.integers(0, len(labels)))
        labels.append(labels[i] + (len(labels),))
    labels = labels[:T]
    index = {lab: k for k, lab in enumerate(labels)}
    parents = np.array([index[lab[:-1]] if len(lab) > 1 else -1 for lab in labels], np.int32)
    return labels, parents


def prefix_mask(labels):
    T = len(labels)
    return np.array([[labels[j][:len(labels[i])] == labels[i] for i in range(T)] for j in range(T)])


def heap_parents(T):
    return np.array([-1] + [(j - 1) // 2 for j in range(1, T)], np.int32)


def heap_mask(T):
    """Complete binary tree in heap numbering (1-based n = j + 1): node i is on node j's path
    to the root exactly when the binary digits of i + 1 begin those of j + 1."""
    m = np.zeros((T, T), bool)
    for j in range(T):
        for i in range(T):
            a, b = i + 1, j + 1
            shift = b.bit_length() - a.bit_length()
            m[j, i] = shift >= 0 and (b >> shift) == a
    return m


def sdpa_tree(P, masks, scale):
    """Dense float64 attention per sequence with context columns visible and tree columns from masks[b]."""
    T = masks[0].shape[0]
    S = len(P["context_lens"])
    n_h, n_kv = P["q"].shape[1], P["k_cache"].shape[2]
    G = n_h // n_kv
    q_all = torch_widen(P["q"], P["dtype"])
    outs = []
    for b in range(S):
        L = int(P["context_lens"][b])
        Q = q_all[b * T:(b + 1) * T].permute(1, 0, 2)[None]
        K = torch.from_numpy(P["Ks"][b]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        V = torch.from_numpy(P["Vs"][b]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        mask = torch.ones(T, L, dtype=torch.bool)
        mask[:, L - T:] = torch.from_numpy(masks[b])
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=float(np.float32(scale)))
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


def run_tree(P, parents, scale):
    return oracle.paged_tree_decode(P["q"], P["k_cache"], P["v_cache"], P["block_tables"], P["context_lens"],
                                    parents, scale, P["dtype"])


# ---------------------------------------------------------------------------
# the pins


def pin_random_tries(seed=0, T=9, lens=(9, 20, 47), dtype="bf16", roots=1, tol=1e-12):
    rng = np.random.default_rng(seed)
    P = build_paged(seed, list(lens), 4, 2, 16, T, dtype)
    trees = [trie(T, rng, roots) for _ in lens]
    parents = np.stack([p for _, p in trees])
    ref = sdpa_tree(P, [prefix_mask(lab) for lab, _ in trees], 0.31)
    return bool(np.max(np.abs(run_tree(P, parents, 0.31) - ref)) <= tol)


def pin_binary15_sdpa(dtype="f32"):
    T = 15
    P = build_paged(5, [T, 31, 64], 8, 2, 16, T, dtype)
    parents = np.tile(heap_parents(T), (3, 1))
    ref = sdpa_tree(P, [heap_mask(T)] * 3, 0.25)
    return bool(np.max(np.abs(run_tree(P, parents, 0.25) - ref)) <= 1e-12)


def pin_binary15_counts():
    """Keys all zero (every score 0), value column c of position t is 1 when c == t: out[c] is
    1 / (visible count) on the visible positions and 0 elsewhere, exactly."""
    T, L, d = 15, 40, 40
    P = build_paged(6, [L], 2, 1, d, T, "f32")
    k = np.zeros_like(P["k_cache"])
    v = np.zeros_like(P["v_cache"])
    for t in range(L):
        blk = P["block_tables"][0, t // 16]
        v[blk, t % 16, 0, t] = 1.0
    out = oracle.paged_tree_decode(P["q"], k, v, P["block_tables"], P["context_lens"],
                                   heap_parents(T)[None], 0.5, "f32")
    hm = heap_mask(T)
    ok = True
    for j in range(T):
        depth = int(hm[j].sum()) - 1
        ok &= depth == (j + 1).bit_length() - 1  # depth of heap node j: floor(log2(j + 1))
        seen = np.zeros(L, bool)
        seen[:L - T] = True
        seen[L - T:] = hm[j]
        n = int(seen.sum())
        want = np.where(seen, 1.0 / n, 0.0)
        for h in range(2):
            ok &= bool(np.array_equal(out[j, h], want))
    return ok


def pin_chain_is_causal(dtype="bf16"):
    T = 5
    P = build_paged(7, [5, 18, 33], 4, 2, 16, T, dtype)
    chain = np.tile(np.arange(-1, T - 1, dtype=np.int32), (3, 1))
    causal = oracle.paged_decode(P["q"], P["k_cache"], P["v_cache"], P["block_tables"], P["context_lens"], 0.4, T,
                                 dtype)
    return bool(np.array_equal(run_tree(P, chain, 0.4), causal))


def pin_off_path_nodes_do_not_matter():
    """Changing the keys and values of node 4 (heap numbering: parent 1, children 9 and 10)
    leaves every node outside node 4's subtree bit-for-bit unchanged and moves the subtree."""
    T = 15
    P = build_paged(8, [30], 2, 1, 16, T, "f32")
    parents = heap_parents(T)[None]
    a = run_tree(P, parents, 0.3)
    k, v = P["k_cache"].copy(), P["v_cache"].copy()
    t = 30 - T + 4
    blk = P["block_tables"][0, t // 16]
    k[blk, t % 16] += 1.0
    v[blk, t % 16] -= 2.0
    b = oracle.paged_tree_decode(P["q"], k, v, P["block_tables"], P["context_lens"], parents, 0.3, "f32")
    off_path = [0, 1, 3, 7, 8, 2, 5, 6]  # node 4's path is 4 -> 1 -> 0; its subtree is 9, 10
    moved = [4, 9, 10]
    return bool(all(np.array_equal(a[j], b[j]) for j in off_path) and
                all(not np.array_equal(a[j], b[j]) for j in moved))


def pin_forest_and_star(dtype="bf16"):
    """Several roots (a forest), and the star: every node a root seeing the context and itself."""
    ok = pin_random_tries(seed=3, T=12, lens=(12, 30), dtype=dtype, roots=3)
    star_labels = [(r,) for r in range(6)]
    P = build_paged(9, [6, 21], 4, 1, 16, 6, dtype)
    parents = np.full((2, 6), -1, np.int32)
    ref = sdpa_tree(P, [prefix_mask(star_labels)] * 2, 0.3)
    return ok and bool(np.max(np.abs(run_tree(P, parents, 0.3) - ref)) <= 1e-12)


PINS = {
    "random_tries_bf16": lambda: pin_random_tries(dtype="bf16"),
    "random_tries_f32_deep": lambda: pin_random_tries(seed=1, T=16, lens=(16, 17, 50), dtype="f32"),
    "binary15_sdpa": pin_binary15_sdpa,
    "binary15_counts": pin_binary15_counts,
    "chain_is_causal": pin_chain_is_causal,
    "off_path_nodes": pin_off_path_nodes_do_not_matter,
    "forest_and_star": pin_forest_and_star,
}


def failing_pins():
    return [name for name, pin in PINS.items() if not pin()]


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    assert PINS[name]()


def test_trie_parents_are_a_tree():
    labels, parents = trie(20, np.random.default_rng(1), roots=2)
    assert all(-1 <= p < j for j, p in enumerate(parents))
    assert [len(oracle.path_to_root(parents, j)) for j in range(20)] == [len(lab) for lab in labels]


def test_non_tree_parent_stops_the_walk():
    """The library's contract for parents outside [-1, j): the walk stops there."""
    parents = np.array([-1, 0, 5, 1, 3, -7], np.int32)
    assert oracle.path_to_root(parents, 2) == [2]
    assert oracle.path_to_root(parents, 4) == [4, 3, 1, 0]
    assert oracle.path_to_root(parents, 5) == [5]
    assert list(oracle.visible_positions(10, parents, 4)) == [0, 1, 2, 3, 4, 5, 7, 8]


# ---------------------------------------------------------------------------
# planted mistakes: every one must fail at least one pin

_true_path = ot.path_to_root


def _path_without_self(parents, j):
    return _true_path(parents, j)[1:]


def _path_without_root(parents, j):
    p = _true_path(parents, j)
    return p[:-1] if len(p) > 1 else p


def _causal_positions(L, parents, j):
    T = len(parents)
    return np.arange(L - T + j + 1)


def _tree_at_front(L, parents, j):
    T = len(parents)
    return np.array(sorted(set(range(T, L)) | set(_true_path(parents, j))), np.int64)


def _no_context(L, parents, j):
    T = len(parents)
    return np.array(sorted(L - T + a for a in _true_path(parents, j)), np.int64)


def _siblings_too(L, parents, j):
    T = len(parents)
    path = set(_true_path(parents, j))
    sib = {k for k in range(T) if parents[k] == parents[j]}
    return np.array(list(range(L - T)) + sorted(L - T + a for a in path | sib), np.int64)


MUTATIONS = {
    "path_without_self": ("path_to_root", _path_without_self),
    "path_without_root": ("path_to_root", _path_without_root),
    "causal_instead_of_tree": ("visible_positions", _causal_positions),
    "tree_at_front_of_context": ("visible_positions", _tree_at_front),
    "context_not_visible": ("visible_positions", _no_context),
    "siblings_visible": ("visible_positions", _siblings_too),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ot, attr, fn)
    assert failing_pins(), f"no pin fails with {name} planted"
