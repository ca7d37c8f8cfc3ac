"""Parity of pa_decode_tree (tree-mask verify) with the fp64 oracle, on the GPU.

Gate: the bf16 tolerance |gpu - ref| <= 2e-2 + 1e-2 |ref| and relative L2
<= 5e-3 against oracle.paged_tree_decode on the same seeded inputs, for every
schedule (one pass, partitions + pa_reduce, balanced), tree shapes from a
single node to 64 nodes (complete binary, random, forests, chains) and ragged
context lengths; exact invariants (a chain equals pa_decode's causal verify
bit for bit, nodes off a changed node's subtree do not move, physical block
ids do not matter, NaN in rows never read does not leak).
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import check_full_size_every_row, DeviceProblem, host_caches_after_write, parity, reference_full, reference_rows, sample_rows, to_dev
from _gpu import to_host, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    import paged_kv_attention_decode_amd as pa

    pa.load_library()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run(p, partition_size):
    d = DeviceProblem(p)
    out = d.step(partition_size)
    torch.cuda.synchronize()
    return d, widen(to_host(out), p.dtype)


def assert_parity(got, ref, what):
    r = parity(got, ref, "bf16")
    assert r["ok"], f"{what}: {r}"
    return r


def small(G=4, d=128, T=15, tree="binary", n_kv=2, S=7, lens=None, seed=0, **kw):
    lens = lens or ("uniform", T, 700)
    return wl.Spec(name="tree-small", dtype="bf16", num_seqs=S, num_q_heads=G * n_kv, num_kv_heads=n_kv,
                   head_dim=d, lens=lens, max_len=720, q_len=T, tree=tree, write_new_tokens=True, seed=seed, **kw)


CASES = [dict(G=4, d=128, T=15, tree="binary"),     # the pages' 15-node tree on the 8B shape: 60 rows
         dict(G=8, d=128, T=7, tree="binary"),      # 56 rows
         dict(G=2, d=64, T=16, tree="random"),      # 32 rows
         dict(G=1, d=128, T=9, tree="random"),      # 9 rows, one tile
         dict(G=1, d=128, T=64, tree="random"),     # the most nodes: 64 rows
         dict(G=3, d=128, T=13, tree="random"),     # 39 rows, three tiles
         dict(G=1, d=64, T=1, tree="binary"),       # a single node: plain decode
         dict(G=4, d=64, T=3, tree="random")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"G{c['G']}-d{c['d']}-T{c['T']}-{c['tree']}")
def test_small_tree(case):
    p = wl.make_problem(small(seed=11 + case["G"] + case["T"], **case))
    ref = reference_full(p)
    for ps in (0, 16, 48, 512, -1):
        say(f"tree decode {case} partition={ps} lens={p.context_lens.tolist()}")
        _, got = run(p, ps)
        assert_parity(got, ref, f"partition {ps}")


def test_tree_sweep_of_lengths():
    """Every context length T .. T + 40 (block boundaries, the tree straddling blocks)."""
    T = 15
    lens = tuple(range(T, T + 41))
    p = wl.make_problem(small(G=4, T=T, n_kv=1, S=len(lens), lens=("fixed", lens), seed=3))
    ref = reference_full(p)
    for ps in (0, 16, -1):
        say(f"tree sweep ps={ps}")
        _, got = run(p, ps)
        assert_parity(got, ref, f"sweep ps={ps}")


@pytest.mark.parametrize("ps", [0, 32, -1])
def test_chain_equals_causal_verify_bitwise(ps):
    """parents[j] = j - 1 is the causal verify: pa_decode_tree and pa_decode agree bit for bit."""
    import paged_kv_attention_decode_amd as pa

    spec = small(G=8, T=5, tree="", seed=21)
    p = wl.make_problem(spec)
    d = DeviceProblem(p)
    causal = to_host(d.step(ps)).copy()
    chain = torch.from_numpy(np.tile(np.arange(-1, 4, dtype=np.int32), (p.num_seqs, 1))).cuda()
    if ps > 0:
        ws = pa.decode_tree(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, chain, float(p.scale), ps)
        out = pa.reduce(torch.empty_like(d.q), ws, d.context_lens, 5, p.max_blocks_per_seq, ps)
    else:
        ws = pa.new_workspace(d.q, d.k_cache, d.block_tables, 5, ps) if ps < 0 else None
        out = pa.decode_tree(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, chain, float(p.scale), ps,
                             workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), causal)


def test_off_subtree_nodes_do_not_move():
    """New K/V for node 4 of the binary tree change nodes 4, 9, 10 and no other node's output."""
    p = wl.make_problem(small(G=4, T=15, S=5, seed=23).with_(write_new_tokens=False))
    d = DeviceProblem(p)
    a = to_host(d.step(0, write=False)).copy()
    rng = np.random.default_rng(5)
    for b in range(p.num_seqs):
        pos = int(p.context_lens[b]) - 15 + 4
        blk = int(p.block_tables[b, pos // 16])
        row = wl.round_to_bf16_bits(rng.standard_normal((p.num_kv_heads, p.head_dim)).astype(np.float32))
        d.k_cache[blk, pos % 16] = to_dev(row, "bf16")
        d.v_cache[blk, pos % 16] = to_dev(row[::-1].copy(), "bf16")
    b_ = to_host(d.step(0, write=False))
    torch.cuda.synchronize()
    for b in range(p.num_seqs):
        for j in range(15):
            same = np.array_equal(a[b * 15 + j], b_[b * 15 + j])
            assert same == (j not in (4, 9, 10)), (b, j)


def test_non_tree_parents_follow_the_contract():
    """Parents outside [-1, j) end a node's path, as the oracle's contract says."""
    p = wl.make_problem(small(G=4, T=8, tree="random", S=3, seed=29))
    par = p.parents.copy()
    par[0, 3] = 3      # itself
    par[0, 5] = 7      # a later node
    par[1, 6] = -5     # below -1
    par[2, 7] = 1000   # far out of range
    p.parents = par
    ref = reference_full(p)
    for ps in (0, -1):
        _, got = run(p, ps)
        assert_parity(got, ref, f"non-tree parents ps={ps}")


@pytest.mark.parametrize("ps", [0, 64, -1])
def test_tree_permutation_invariant_and_repeatable(ps):
    p = wl.make_problem(small(G=4, T=15, seed=31))
    _, a = run(p, ps)
    q = wl.permute_physical(p, 7)
    _, b = run(q, ps)
    _, c = run(p, ps)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_tree_poisoned_unread_rows():
    spec = small(G=4, T=15, seed=37)
    clean = wl.make_problem(spec)
    dirty = wl.make_problem(spec.with_(poison=True, pad="garbage"))
    for ps in (0, 64, -1):
        _, a = run(clean, ps)
        _, b = run(dirty, ps)
        assert np.isfinite(b).all()
        assert np.array_equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G,T,tree", [(4, 15, "binary"), (1, 9, "random"), (3, 13, "random")])
def test_tree_scores_rising_far_past_the_first_block(G, T, tree, d):
    """Keys grow by 0.2 per position in one dimension (queries 4 there, scale
    1/8), so weights relative to a wave's first block exceed 2^64 and the tree
    kernel must take its exact two-pass path, in every schedule; the tree's
    own nodes sit on the ramp too."""
    spec = small(G=G, d=d, T=T, tree=tree, n_kv=1, S=3, lens=("fixed", (1000, 700, 40)), seed=59).with_(
        write_new_tokens=False, max_len=1024, scale=0.125)
    p = wl.make_problem(spec)
    bits = lambda x: wl.round_to_bf16_bits(np.array([x], dtype=np.float32))[0]
    p.q[:] = 0
    p.k_cache[:] = 0
    p.q[:, :, 0] = bits(4.0)
    for b, L in enumerate(p.context_lens):
        for t in range(int(L)):
            p.k_cache[p.block_tables[b, t // 16], t % 16, 0, 0] = bits(0.2 * t)
    ref = reference_full(p)
    for ps in (0, 512, -1):
        say(f"tree ramp G={G} T={T} {tree} d={d} ps={ps}")
        _, got = run(p, ps)
        assert np.isfinite(got).all()
        assert_parity(got, ref, f"tree ramp ps={ps}")


def test_tree_verify_full_size_every_row():
    """Every output row of the full tree-verify workload, in the schedule bench.py times and in the
    others, against the oracle (stated tolerance, relative L2, and relative L2 per row)."""
    check_full_size_every_row("tree-verify", say)
