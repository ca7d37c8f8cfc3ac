"""The parity gates reject wrong answers (CPU).

A gate that a wrong kernel passes proves nothing, so each gate used by the
GPU tests (tests/_gpu.py parity: elementwise |gpu - ref| <= atol + rtol |ref|
plus relative L2 over the compared rows) is shown here to reject three
plausible failures, computed with the oracle itself on rows of every
workload's shape: an all-zero output, the wrong GQA map (query head h reading
KV head h mod n_kv instead of h // G), and, where contexts are short enough
for one token to matter (up to about 2,300 tokens at d = 128), a context one
token short.  The workloads keep their head shapes and length ranges with
fewer sequences, so the CPU suite stays fast.

The per-row gate of the full-size tests (parity(..., rows=True): relative L2
of every output row against the oracle's) is shown to reject a piece of a cut
sequence lost or merged twice, and one lost block of 16 tokens, in a single
row among many, and to accept an exact re-partitioning of the same rows.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import parity, widen
from oracle import attention as oa
from oracle import tree as ot


def shape_of(name, **kw):
    spec = wl.CONFIGS[name]
    few = {"tiny-f32": {}, "llama3-8b-decode": dict(num_seqs=6, num_blocks=None),
           "llama3-70b-decode": dict(num_seqs=6), "long-split": dict(num_seqs=1, lens=("fixed", (40000,)),
                                                                      max_len=40960),
           "spec-verify": dict(num_seqs=4), "tree-verify": dict(num_seqs=3)}[name]
    return wl.make_problem(spec.with_(**{**few, **kw}))


def rows_of(p, n=12, seed=0):
    rng = np.random.default_rng(seed)
    S, Q, H = p.num_seqs, p.q_len, p.num_q_heads
    return sorted({(int(rng.integers(0, S)), int(rng.integers(0, Q)), int(rng.integers(0, H))) for _ in range(n)})


def reference(p, rows):
    if p.parents is not None:
        return oracle.paged_tree_decode_rows(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.parents,
                                             p.scale, p.dtype, rows)
    return oracle.paged_decode_rows(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, p.q_len,
                                    p.dtype, rows)


NAMES = ["tiny-f32", "llama3-8b-decode", "llama3-70b-decode", "long-split", "spec-verify", "tree-verify"]


@pytest.mark.parametrize("name", NAMES)
def test_gate_rejects_zeros_and_wrong_gqa_map(name, monkeypatch):
    p = shape_of(name)
    rows = rows_of(p)
    ref = reference(p, rows)
    assert parity(ref, ref, p.dtype)["ok"]  # the oracle against itself passes
    assert not parity(np.zeros_like(ref), ref, p.dtype)["ok"], "an all-zero output passes the gate"
    if p.num_kv_heads > 1 and p.spec.group > 1:
        wrong_map = lambda h, group: h % p.num_kv_heads  # noqa: E731
        monkeypatch.setattr(oa, "kv_head_of", wrong_map)
        monkeypatch.setattr(ot, "kv_head_of", wrong_map)
        wrong = reference(p, rows)
        monkeypatch.undo()
        assert not parity(wrong, ref, p.dtype)["ok"], "the h mod n_kv head map passes the gate"


@pytest.mark.parametrize("name,max_len", [("tiny-f32", 48), ("llama3-8b-decode", 2304)])
def test_gate_rejects_a_context_one_token_short(name, max_len, monkeypatch):
    p = shape_of(name)
    short = [b for b in range(p.num_seqs) if p.context_lens[b] <= max_len]
    if not short:  # make one: the shortest of the workload's range
        p = shape_of(name, lens=("fixed", tuple(min(int(x), max_len) for x in p.context_lens)))
        short = list(range(p.num_seqs))
    rows = [(b, 0, h) for b in short for h in range(0, p.num_q_heads, max(1, p.num_q_heads // 4))]
    ref = reference(p, rows)
    monkeypatch.setattr(oa, "visible_tokens", lambda L, q_len, j: L - q_len + j)
    wrong = reference(p, rows)
    monkeypatch.undo()
    assert not parity(wrong, ref, p.dtype)["ok"], "a context one token short passes the gate"


# The full-size tests (tests/_gpu.py check_full_size_every_row) compare every row of every
# schedule with the oracle.  What they must catch: a piece of a cut sequence lost or merged
# twice (a balanced merge or pa_reduce mistake), or one block of 16 tokens lost, even in one
# row of thousands.  Simulated here with the oracle's own partials and merge on rows of the
# 8B layer's shape, rounded to bf16 as the GPU outputs are.
def _rows_through_partials(p, rows, partition_size, edit=None):
    from oracle import attention as oa

    G = p.spec.group
    out = []
    for (b, j, h) in rows:
        L = int(p.context_lens[b])
        g = oa.kv_head_of(h, G)
        K = oa.to_f64(oa.gather_sequence(p.k_cache, p.block_tables[b], L)[:, g], p.dtype)
        V = oa.to_f64(oa.gather_sequence(p.v_cache, p.block_tables[b], L)[:, g], p.dtype)
        qv = oa.to_f64(p.q[b * p.q_len + j, h], p.dtype)
        ms, ls, accs = oa.partition_partials(qv, K, V, float(np.float32(p.scale)),
                                             oa.visible_tokens(L, p.q_len, j), L, partition_size)
        if edit is not None:
            ms, ls, accs = edit(ms, ls, accs)
        out.append(oa.merge_partials(ms, ls, accs))
    return widen(wl.round_to_bf16_bits(np.asarray(out, dtype=np.float32)), "bf16")


def _drop(k):
    return lambda ms, ls, accs: (np.delete(ms, k), np.delete(ls, k), np.delete(accs, k, axis=0))


def _double(k):
    return lambda ms, ls, accs: (np.append(ms, ms[k]), np.append(ls, ls[k]), np.vstack([accs, accs[k:k + 1]]))


@pytest.mark.parametrize("mistake", ["piece_lost", "piece_doubled", "block_lost"])
def test_row_gate_rejects_one_row_with_a_lost_or_doubled_piece(mistake):
    p = shape_of("llama3-8b-decode")
    rows = rows_of(p, n=16, seed=1)
    ref = reference(p, rows)
    exact = _rows_through_partials(p, rows, 512)
    # an exact partitioning of the same rows, rounded to bf16, passes
    assert parity(exact, ref, p.dtype, rows=True)["ok"]
    assert parity(_rows_through_partials(p, rows, 1024), ref, p.dtype, rows=True)["ok"]
    # the mistake in every row is caught by every gate; in one row only by the per-row gate
    if mistake == "piece_lost":
        bad = _rows_through_partials(p, rows, 512, _drop(1))
    elif mistake == "piece_doubled":
        bad = _rows_through_partials(p, rows, 512, _double(1))
    else:
        bad = _rows_through_partials(p, rows, 16, _drop(3))
    assert not parity(bad, ref, p.dtype, rows=True)["ok"], mistake
    for i in range(len(rows)):
        one = exact.copy()
        one[i] = bad[i]
        # embedded among 2,048 exact rows (the 8B layer's output), as in the full-size tests
        big_ref = np.concatenate([ref, np.repeat(ref, 128, axis=0)])
        big = np.concatenate([one, np.repeat(exact, 128, axis=0)])
        assert not parity(big, big_ref, p.dtype, rows=True)["ok"], (mistake, i)
