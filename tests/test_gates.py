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
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import parity
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
