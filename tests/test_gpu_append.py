"""pa_decode_append (the new tokens' cache write and the decode in one launch)
on the GPU.

Gates: the caches after the call are bit-exact against the oracle's
cache_write with the slots the pages' append rule gives (new token j of
sequence b at position L_b - q_len + j, through b's block table); the output
(or the partials pa_reduce merges) is bit-identical to pa_cache_write followed
by pa_decode, which the other suites pin to the oracle, and sampled rows are
checked against the oracle directly.  Covered: every schedule (one pass,
partitions with pa_reduce, balanced), the vector-ALU and matrix-core kernels,
fp32 and bf16, new tokens straddling a block boundary whose two blocks are
read by different workgroups, contexts shorter than q_len, a new token's block
outside the pool, and the full 8B decode and speculative-verify workloads.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import DeviceProblem, host_caches_after_write, parity, reference_rows, sample_rows, to_host, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def appended_slots(p):
    """The append rule: new token j of sequence b goes to position L_b - q_len + j of b's
    blocks; a position before 0, or a block id outside the pool, stores nothing (-1)."""
    slots = []
    for b in range(p.num_seqs):
        L = int(p.context_lens[b])
        for j in range(p.q_len):
            pos = L - p.q_len + j
            phys = int(p.block_tables[b, pos // 16]) if pos >= 0 else -1
            slots.append(phys * 16 + pos % 16 if 0 <= phys < p.num_blocks else -1)
    return np.array(slots, dtype=np.int64)


def fused(p, ps):
    import paged_kv_attention_decode_amd as pa

    d = DeviceProblem(p)
    ws = pa.new_workspace(d.q, d.k_cache, d.block_tables, p.q_len, ps) if ps != 0 else None
    r = pa.decode_append(d.q, d.new_k, d.new_v, d.k_cache, d.v_cache, d.block_tables, d.context_lens, float(p.scale),
                         p.q_len, ps, out=d.out if ps <= 0 else None, workspace=ws)
    if ps > 0:
        pa.reduce(d.out, r, d.context_lens, p.q_len, p.max_blocks_per_seq, ps)
    torch.cuda.synchronize()
    return d


def separate(p, ps):
    d = DeviceProblem(p)
    d.step(ps)
    torch.cuda.synchronize()
    return d


def check(p, ps, what, n_rows=24, skip_seqs=()):
    assert p.new_k is not None
    a, b = separate(p, ps), fused(p, ps)
    ka, kb = to_host(a.k_cache), to_host(b.k_cache)
    va, vb = to_host(a.v_cache), to_host(b.v_cache)
    # the caches: what the oracle's cache write stores at the appended slots, bit for bit
    kc, vc = oracle.cache_write(p.k_cache, p.v_cache, p.new_k, p.new_v, appended_slots(p))
    assert np.array_equal(kb.view(np.uint8), np.ascontiguousarray(kc).view(np.uint8)), f"{what}: K cache"
    assert np.array_equal(vb.view(np.uint8), np.ascontiguousarray(vc).view(np.uint8)), f"{what}: V cache"
    assert np.array_equal(ka.view(np.uint8), kb.view(np.uint8)) and np.array_equal(va.view(np.uint8), vb.view(np.uint8))
    # the output: bit-identical to the two calls, and the oracle on sampled rows
    oa, ob = to_host(a.out), to_host(b.out)
    assert np.array_equal(oa.view(np.uint8), ob.view(np.uint8)), f"{what}: output differs from cache_write + decode"
    # rows that see no position are zeros (the contract); the oracle is asked about the others
    seen = lambda b, j: int(p.context_lens[b]) - p.q_len + j + 1 > 0  # noqa: E731
    for bb in range(p.num_seqs):
        for j in range(p.q_len):
            if not seen(bb, j):
                assert not widen(ob, p.dtype)[bb * p.q_len + j].any(), f"{what}: row {bb},{j} sees nothing"
    rows = [r for r in sample_rows(p, n_rows) if seen(r[0], r[1]) and r[0] not in skip_seqs]
    hk, hv = host_caches_after_write(p)
    ref = reference_rows(p, rows, hk, hv)
    out = widen(ob, p.dtype)
    r = parity(np.stack([out[bb * p.q_len + j, h] for (bb, j, h) in rows]), ref, p.dtype, rows=True)
    assert r["ok"], f"{what}: {r}"


def spec(dtype="bf16", G=4, d=128, q_len=1, n_kv=2, S=9, lens=None, seed=0, **kw):
    lens = lens or ("uniform", q_len, 700)
    return wl.Spec(name="append", dtype=dtype, num_seqs=S, num_q_heads=G * n_kv, num_kv_heads=n_kv, head_dim=d,
                   lens=lens, max_len=720, q_len=q_len, write_new_tokens=True, seed=seed, **kw)


CASES = [dict(dtype="bf16", G=4, d=128, q_len=1),   # vector ALU, 4 rows
         dict(dtype="bf16", G=8, d=128, q_len=5),   # matrix cores, 40 rows
         dict(dtype="bf16", G=2, d=64, q_len=8),    # matrix cores, 16 rows, 8 new tokens
         dict(dtype="f32", G=2, d=64, q_len=2),     # fp32
         dict(dtype="f32", G=1, d=128, q_len=8)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['dtype']}-G{c['G']}-d{c['d']}-q{c['q_len']}")
def test_append_matches_write_then_decode(case):
    p = wl.make_problem(spec(seed=3 + case["G"] + case["q_len"], **case))
    for ps in (0, 48, 512, -1):
        say(f"append {case} partition={ps}")
        check(p, ps, f"{case} ps={ps}")


def test_append_tokens_straddling_blocks_of_different_workgroups():
    """Contexts of 1-7 tokens past a block boundary with 8 new tokens: the new tokens
    fall in two blocks.  With fewer blocks than balanced ranges every block is its own
    range, so the two blocks are stored and read by two different workgroups."""
    lens = tuple(16 * k + r for k, r in ((1, 3), (2, 1), (2, 7), (1, 5), (3, 2)))
    p = wl.make_problem(spec(G=4, d=128, q_len=8, n_kv=2, S=len(lens), lens=("fixed", lens), seed=7))
    for ps in (0, 16, -1):
        check(p, ps, f"straddle ps={ps}")


def test_append_short_contexts_and_blocks_outside_the_pool():
    """Contexts shorter than q_len (positions before 0 are not stored) and a sequence
    whose last block id lies outside the pool (its new tokens are not stored and the
    block reads as zeros), as pa_cache_write skips such slots."""
    p = wl.make_problem(spec(G=8, d=64, q_len=8, n_kv=1, S=5, lens=("fixed", (8, 8, 40, 200, 8)), seed=9))
    p.context_lens[0], p.context_lens[1] = 3, 1  # fewer tokens than new ones
    p.block_tables[3, (int(p.context_lens[3]) - 1) // 16] = p.num_blocks + 5
    p.slot_mapping = appended_slots(p)  # the two calls skip the same tokens
    for ps in (0, 16, -1):
        # sequence 3 reads a block outside the pool, which the oracle cannot gather: it is
        # covered by the bitwise agreement with the two calls
        check(p, ps, f"short/outside ps={ps}", n_rows=40, skip_seqs=(3,))


@pytest.mark.parametrize("name", ["llama3-8b-decode", "spec-verify"])
def test_append_full_size(name):
    import bench

    p = wl.make_problem(name)
    assert np.array_equal(appended_slots(p), p.slot_mapping)
    ps = bench.partition_for(p)
    say(f"{name}: append, partition {ps}")
    check(p, ps, name, n_rows=64)
