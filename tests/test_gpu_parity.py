"""Parity of the HIP path with the fp64 oracle, through the C ABI, on the GPU.

Gates (elementwise, on every compared output):
  fp32: |gpu - ref| <= 2e-3, and ||gpu - ref|| / ||ref|| <= 1e-5
  bf16: |gpu - ref| <= 2e-2 + 1e-2 |ref|, and ||gpu - ref|| / ||ref|| <= 5e-3
cache writes: bit-exact.  Invariants that must hold bit for bit: physical block
permutation, batch composition, run-to-run repetition, unread rows poisoned
with NaN, future tokens of a verify row.
"""

import os
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import DeviceProblem, check_full_size_every_row, host_caches_after_write, parity, sample_rows, to_dev, to_host, widen

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


def run(p: wl.Problem, partition_size: int, write: bool = True):
    d = DeviceProblem(p)
    out = d.step(partition_size, write)
    torch.cuda.synchronize()
    return d, widen(to_host(out), p.dtype)


def full_reference(p: wl.Problem):
    kc, vc = host_caches_after_write(p)
    return oracle.paged_decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, p.q_len, p.dtype)


def assert_parity(got, ref, dtype, what, **kw):
    r = parity(got, ref, dtype, **kw)
    assert r["ok"], f"{what}: {r}"
    return r


# ---------------------------------------------------------------------------
# pa_cache_write: bit-exact


@pytest.mark.parametrize("dtype,n_kv,d", [("bf16", 8, 128), ("f32", 2, 64), ("bf16", 1, 64), ("f32", 3, 128)])
def test_cache_write_bit_exact(dtype, n_kv, d):
    rng = np.random.default_rng(hash((dtype, n_kv, d)) % 2**32)
    NB, T = 37, 29
    bits = np.uint16 if dtype == "bf16" else np.uint32
    kc = rng.integers(0, np.iinfo(bits).max, size=(NB, 16, n_kv, d), dtype=bits, endpoint=True)
    vc = rng.integers(0, np.iinfo(bits).max, size=(NB, 16, n_kv, d), dtype=bits, endpoint=True)
    k = rng.integers(0, np.iinfo(bits).max, size=(T, n_kv, d), dtype=bits, endpoint=True)
    v = rng.integers(0, np.iinfo(bits).max, size=(T, n_kv, d), dtype=bits, endpoint=True)
    slots = rng.choice(NB * 16, size=T, replace=False).astype(np.int64)
    slots[3] = -1
    slots[7] = -5
    slots[11] = NB * 16 + 3  # outside the pool: skipped
    view = (lambda a: a) if dtype == "bf16" else (lambda a: a.view(np.float32))
    say(f"cache_write {dtype} n_kv={n_kv} d={d} T={T}")
    dk, dv = to_dev(view(k), dtype), to_dev(view(v), dtype)
    dkc, dvc = to_dev(view(kc), dtype), to_dev(view(vc), dtype)
    import paged_kv_attention_decode_amd as pa

    pa.cache_write(dk, dv, dkc, dvc, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    keep = (slots >= 0) & (slots < NB * 16)
    ek, ev = oracle.cache_write(kc, vc, k[keep], v[keep], slots[keep])
    gk = to_host(dkc).view(bits)
    gv = to_host(dvc).view(bits)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


# ---------------------------------------------------------------------------
# small problems, full output


def test_tiny_f32_config():
    p = wl.make_problem("tiny-f32")
    say("tiny-f32")
    _, got = run(p, 0)
    assert_parity(got, full_reference(p), "f32", "tiny-f32")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("q_len,n_h,n_kv", [(1, 8, 2), (5, 2, 2), (2, 8, 2)])
def test_length_sweep_f32(d, q_len, n_h, n_kv):
    """Every context length 1..48 crossed with block boundaries, fp32 inputs, 1e-5."""
    lens = tuple(range(max(1, q_len), 49))
    spec = wl.Spec(name="sweep", dtype="f32", num_seqs=len(lens), num_q_heads=n_h, num_kv_heads=n_kv, head_dim=d,
                   lens=("fixed", lens), max_len=64, q_len=q_len, seed=d + q_len)
    p = wl.make_problem(spec)
    for ps in (0, 16, 32, -1):
        say(f"sweep f32 d={d} q_len={q_len} heads={n_h}/{n_kv} partition={ps}")
        _, got = run(p, ps)
        assert_parity(got, full_reference(p), "f32", f"sweep ps={ps}", atol=1e-5)


SMALL_BF16 = [
    dict(G=1, d=128, q_len=1), dict(G=2, d=128, q_len=1), dict(G=4, d=128, q_len=1), dict(G=8, d=128, q_len=1),
    dict(G=4, d=64, q_len=1), dict(G=8, d=64, q_len=1), dict(G=4, d=128, q_len=2), dict(G=1, d=128, q_len=5),
    dict(G=3, d=128, q_len=1),
    # 8 to 64 rows per KV head: the matrix-core kernel, 1 to 4 row tiles
    dict(G=8, d=128, q_len=2), dict(G=2, d=128, q_len=5), dict(G=8, d=128, q_len=5), dict(G=8, d=64, q_len=5),
    dict(G=5, d=128, q_len=7), dict(G=16, d=128, q_len=4), dict(G=16, d=64, q_len=4), dict(G=12, d=128, q_len=5),
    # the longest causal verify the ABI takes (q_len 8): 64 rows, and 8 rows of one head
    dict(G=8, d=128, q_len=8), dict(G=1, d=64, q_len=8),
]


@pytest.mark.parametrize("case", SMALL_BF16, ids=lambda c: f"G{c['G']}-d{c['d']}-q{c['q_len']}")
def test_small_bf16(case):
    G, d, q_len = case["G"], case["d"], case["q_len"]
    spec = wl.Spec(name="small", dtype="bf16", num_seqs=7, num_q_heads=2 * G, num_kv_heads=2, head_dim=d,
                   lens=("uniform", max(1, q_len), 700), max_len=720, q_len=q_len, write_new_tokens=True,
                   seed=17 + G + d + q_len)
    p = wl.make_problem(spec)
    ref = full_reference(p)
    for ps in (0, 16, 48, 512, -1):
        say(f"small bf16 G={G} d={d} q_len={q_len} partition={ps} lens={p.context_lens.tolist()}")
        _, got = run(p, ps)
        assert_parity(got, ref, "bf16", f"partition {ps}")


def test_many_sequences_single_block():
    spec = wl.Spec(name="short", dtype="bf16", num_seqs=300, num_q_heads=32, num_kv_heads=8, head_dim=128,
                   lens=("uniform", 1, 16), max_len=16, seed=5)
    p = wl.make_problem(spec)
    say("300 sequences of 1..16 tokens")
    for ps in (0, -1):
        _, got = run(p, ps)
        assert_parity(got, full_reference(p), "bf16", f"short ps={ps}")


# ---------------------------------------------------------------------------
# invariants, bit for bit

INV_SPEC = wl.Spec(name="inv", dtype="bf16", num_seqs=6, num_q_heads=16, num_kv_heads=4, head_dim=128,
                   lens=("uniform", 2, 900), max_len=960, q_len=2, seed=23)


# 40 rows per KV head (8 query heads per KV head, 5 query tokens)
INV_SPEC_WIDE = INV_SPEC.with_(num_q_heads=32, num_kv_heads=4, q_len=5, lens=("uniform", 5, 900), seed=29)
# 64 rows per KV head (8 query tokens): four row tiles, whose one-pass and
# partition schedules stage V in LDS
INV_SPEC_64 = INV_SPEC.with_(num_q_heads=32, num_kv_heads=4, q_len=8, lens=("uniform", 8, 900), seed=41)
INV_SPECS = {"rows8": INV_SPEC, "rows40": INV_SPEC_WIDE, "rows64": INV_SPEC_64}


@pytest.mark.parametrize("rows", list(INV_SPECS))
@pytest.mark.parametrize("ps", [0, 64, -1])
def test_physical_permutation_is_bitwise_invariant(ps, rows):
    p = wl.make_problem(INV_SPECS[rows])
    say(f"permutation ps={ps}")
    _, a = run(p, ps)
    _, b = run(wl.permute_physical(p, 99), ps)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("ps", [0, 64, -1])
def test_cache_placement_is_bitwise_invariant(ps):
    """The pools in one allocation as pa_kv_cache_layout places them (what DeviceProblem
    uses) and in two separate allocations give the same bits; the layout's views are
    disjoint, 2 KiB-aligned for K and one head slice off for V."""
    p = wl.make_problem(INV_SPEC_WIDE)
    say(f"placement ps={ps}")
    d = DeviceProblem(p)
    kc, vc = d.k_cache, d.v_cache
    nbytes = kc.numel() * kc.element_size()
    slice_ = p.spec.head_dim * kc.element_size()
    assert kc.data_ptr() % 2048 == 0 and (vc.data_ptr() - kc.data_ptr()) % 2048 == slice_
    assert vc.data_ptr() >= kc.data_ptr() + nbytes
    a = to_host(d.step(ps, write=False).clone())
    d.k_cache, d.v_cache = kc.clone(), vc.clone()  # separate allocations, same contents
    assert d.k_cache.data_ptr() != kc.data_ptr()
    b = to_host(d.step(ps, write=False).clone())
    torch.cuda.synchronize()
    assert np.array_equal(a, b)
    assert np.array_equal(to_host(d.k_cache), to_host(kc)) and np.array_equal(to_host(d.v_cache), to_host(vc))


@pytest.mark.parametrize("rows", list(INV_SPECS))
@pytest.mark.parametrize("ps", [0, 64])
def test_repeatable_and_batch_independent(ps, rows):
    p = wl.make_problem(INV_SPECS[rows])
    ql = p.q_len
    say(f"repeat / batch ps={ps} rows={p.spec.group * ql}")
    d = DeviceProblem(p)
    o1 = to_host(d.step(ps).clone())
    o2 = to_host(d.step(ps).clone())
    assert np.array_equal(o1, o2)
    # sequence 3 alone
    b = 3
    one = wl.Problem(spec=p.spec.with_(num_seqs=1), context_lens=p.context_lens[b:b + 1].copy(),
                     block_tables=p.block_tables[b:b + 1].copy(), q=p.q[b * ql:(b + 1) * ql].copy(),
                     k_cache=p.k_cache, v_cache=p.v_cache, scale=p.scale)
    _, alone = run(one, ps)
    assert np.array_equal(widen(o1[b * ql:(b + 1) * ql], "bf16"), alone)


@pytest.mark.parametrize("rows", list(INV_SPECS))
def test_unread_rows_poisoned_and_garbage_padding(rows):
    spec = INV_SPECS[rows]
    clean = wl.make_problem(spec)
    dirty = wl.make_problem(spec.with_(poison=True, pad="garbage"))
    for ps in (0, 64, -1):
        say(f"poison ps={ps}")
        _, a = run(clean, ps)
        _, b = run(dirty, ps)
        assert np.isfinite(b).all()
        assert np.array_equal(a, b)


@pytest.mark.parametrize("q_len,n_h", [(2, 8), (5, 32)], ids=["rows4", "rows40"])
def test_future_tokens_do_not_change_earlier_verify_rows(q_len, n_h):
    spec = INV_SPEC.with_(q_len=q_len, num_q_heads=n_h, num_kv_heads=4, lens=("uniform", q_len, 900))
    p = wl.make_problem(spec)
    _, base = run(p, 0)
    q = wl.make_problem(spec)
    for b in range(q.num_seqs):
        t = int(q.context_lens[b]) - 1  # visible to the last query token only
        q.k_cache[q.block_tables[b, t // 16], t % 16] = np.uint16(0x4100)
        q.v_cache[q.block_tables[b, t // 16], t % 16] = np.uint16(0xC100)
    _, pert = run(q, 0)
    early = [b * q_len + j for b in range(p.num_seqs) for j in range(q_len - 1)]
    last = [b * q_len + q_len - 1 for b in range(p.num_seqs)]
    assert np.array_equal(base[early], pert[early])
    assert not np.array_equal(base[last], pert[last])


def test_values_all_one_give_exactly_one():
    p = wl.make_problem(INV_SPEC)
    p.v_cache[:] = np.uint16(0x3F80)
    for ps in (0, 64, -1):
        _, got = run(p, ps)
        assert np.all(got == 1.0), ps


@pytest.mark.parametrize("n_h", [8, 16, 64], ids=["rows4", "rows8", "rows32"])
def test_one_token_context_returns_v_exactly(n_h):
    spec = wl.Spec(name="one", dtype="bf16", num_seqs=5, num_q_heads=n_h, num_kv_heads=2, head_dim=128,
                   lens=("fixed", (1, 1, 1, 1, 1)), max_len=16, seed=3)
    p = wl.make_problem(spec)
    G = n_h // 2
    for ps in (0, -1):
        _, got = run(p, ps)
        for b in range(5):
            for h in range(n_h):
                expect = widen(p.v_cache[p.block_tables[b, 0], 0, h // G], "bf16")
                assert np.array_equal(got[b, h], expect), (ps, b, h)


@pytest.mark.parametrize("q_len,L", [(1, 300), (5, 77), (1, 20000)])
def test_identical_keys_count_probe_fp32(q_len, L):
    """All keys equal, V[t, c] = 1 where c == t mod d: each output is an exact count / (p + 1)."""
    d = 128
    lens = (L, L - 1, max(q_len, L // 3))
    spec = wl.Spec(name="count", dtype="f32", num_seqs=3, num_q_heads=1, num_kv_heads=1, head_dim=d,
                   lens=("fixed", lens), max_len=L + 16, q_len=q_len, seed=8)
    p = wl.make_problem(spec)
    p.k_cache[:] = np.float32(0.25)
    p.v_cache[:] = 0
    for b, Lb in enumerate(lens):
        for t in range(Lb):
            p.v_cache[p.block_tables[b, t // 16], t % 16, 0, t % d] = 1.0
    for ps in (0, 512, -1):
        say(f"count probe q_len={q_len} L={L} ps={ps}")
        _, got = run(p, ps)
        for b, Lb in enumerate(lens):
            for j in range(q_len):
                pos = Lb - q_len + j
                expect = np.array([len(range(c, pos + 1, d)) for c in range(d)]) / (pos + 1)
                np.testing.assert_allclose(got[b * q_len + j, 0], expect, rtol=2e-6, atol=0)


COUNT_SHAPES = [  # (GQA group, q_len, context lengths, partition sizes): the workloads' kernel paths
    (4, 1, (2304, 2303, 700), (0, -1)),      # 8B decode: vector ALUs
    (8, 1, (2304, 1000, 33), (0, -1)),       # 70B decode: matrix cores, one tile
    (8, 5, (2304, 1029, 77), (0, -1)),       # verify: matrix cores, three tiles
    (4, 1, (131072,), (0, 512)),             # long context: partitions + pa_reduce
]


@pytest.mark.parametrize("G,q_len,lens,parts", COUNT_SHAPES, ids=["8b", "70b", "verify", "long"])
def test_identical_keys_count_probe_bf16(G, q_len, lens, parts):
    """bf16 at the workloads' shapes: all keys equal, V[t, c] = 1 where c == t mod d.  Every
    weight is exactly 1, so each output is count / (p + 1): in one pass the bf16 rounding
    of one fp32 division, bit for bit; the split and balanced merges of normalized partials
    stay within one bf16 unit in the last place."""
    d, n_kv = 128, 2
    spec = wl.Spec(name="count16", dtype="bf16", num_seqs=len(lens), num_q_heads=G * n_kv, num_kv_heads=n_kv,
                   head_dim=d, lens=("fixed", lens), max_len=max(lens) + 16, q_len=q_len, seed=9)
    p = wl.make_problem(spec)
    p.k_cache[:] = np.uint16(0x3E80)  # 0.25
    p.v_cache[:] = 0
    for b, Lb in enumerate(lens):
        t = np.arange(Lb)
        blk = p.block_tables[b, t // 16]
        for g in range(n_kv):
            p.v_cache[blk, t % 16, g, t % d] = np.uint16(0x3F80)
    expect = np.zeros((len(lens) * q_len, d), dtype=np.float32)
    for b, Lb in enumerate(lens):
        for j in range(q_len):
            pos = Lb - q_len + j
            counts = np.array([len(range(c, pos + 1, d)) for c in range(d)], dtype=np.float32)
            expect[b * q_len + j] = counts / np.float32(pos + 1)
    expect_bits = wl.round_to_bf16_bits(expect)
    for ps in parts:
        say(f"bf16 count probe G={G} q_len={q_len} lens={lens} ps={ps}")
        d_ = DeviceProblem(p)
        out = to_host(d_.step(ps, write=False))
        for h in range(spec.num_q_heads):
            if ps == 0:
                assert np.array_equal(out[:, h], expect_bits), (ps, h)
            else:
                np.testing.assert_allclose(widen(out[:, h], "bf16"), widen(expect_bits, "bf16"), rtol=2 ** -7, atol=0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype,q_len,n_h", [("f32", 1, 2), ("f32", 2, 2), ("bf16", 1, 2), ("bf16", 2, 2),
                                             ("bf16", 5, 2), ("bf16", 5, 8), ("bf16", 8, 8)])
def test_scores_rising_far_past_the_first_block(dtype, q_len, n_h, d):
    """Scores grow by ~0.1 per position (scale 1/8 at both head sizes), so
    weights relative to a wave's first block exceed 2^64 and every kernel
    variant (vector ALU and matrix core up to four row tiles, the last with V
    staged in LDS, d 64 and 128) must take its exact
    two-pass path, in each schedule."""
    spec = wl.Spec(name="ramp", dtype=dtype, num_seqs=3, num_q_heads=n_h, num_kv_heads=1, head_dim=d,
                   lens=("fixed", (1000, 700, 40)), max_len=1024, q_len=q_len, seed=31, scale=0.125)
    p = wl.make_problem(spec)
    p.q[:] = 0
    p.k_cache[:] = 0
    one = np.float32(4.0)
    p.q[:, :, 0] = wl.round_to_bf16_bits(np.array([one]))[0] if dtype == "bf16" else one
    for b, L in enumerate(p.context_lens):
        for t in range(int(L)):
            val = np.float32(0.2 * t)
            p.k_cache[p.block_tables[b, t // 16], t % 16, 0, 0] = (
                wl.round_to_bf16_bits(np.array([val]))[0] if dtype == "bf16" else val)
    ref = full_reference(p)
    for ps in (0, 512, -1):
        say(f"ramp {dtype} d={d} q_len={q_len} heads={n_h} ps={ps}")
        _, got = run(p, ps)
        assert_parity(got, ref, dtype, f"ramp ps={ps}")


def test_balanced_is_repeatable_and_reuses_its_workspace():
    """Run-to-run bitwise determinism of the balanced split, whose cut pieces are
    merged by whichever workgroup arrives last; the workspace counters must be
    back at zero after every call."""
    p = wl.make_problem(INV_SPEC.with_(num_seqs=40, lens=("uniform", 2, 3000), max_len=3008))
    d = DeviceProblem(p)
    outs = [to_host(d.step(-1).clone()) for _ in range(4)]
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)
    counters = to_host(d.workspace[:4 * p.num_seqs * p.num_kv_heads].clone())
    assert not counters.any()
    assert_parity(widen(outs[0], "bf16"), full_reference(p), "bf16", "balanced")


def test_balanced_with_empty_and_tiny_contexts():
    """Zero-length contexts get zero rows; ranges that start and end inside one block."""
    spec = wl.Spec(name="empty", dtype="bf16", num_seqs=9, num_q_heads=8, num_kv_heads=2, head_dim=128,
                   lens=("fixed", (1, 40, 1, 3, 900, 1, 16, 17, 1)), max_len=912, seed=13)
    p = wl.make_problem(spec)
    ref = full_reference(p)
    p0 = wl.Problem(**{**p.__dict__})
    p0.context_lens = p.context_lens.copy()
    p0.context_lens[[0, 2, 5]] = 0
    for prob, want_zero in ((p, []), (p0, [0, 2, 5])):
        _, got = run(prob, -1)
        keep = [b for b in range(9) if b not in want_zero]
        assert_parity(got[keep], ref[keep], "bf16", "balanced rows")
        assert np.all(got[want_zero] == 0)


@pytest.mark.parametrize("num_seqs", [4096, 4097], ids=["balanced-max", "one-pass-fallback"])
def test_balanced_batch_size_limit(num_seqs):
    """The balanced mode's prefix table holds 4096 sequences; one more falls back to one pass.
    Either way the result matches the oracle on sampled rows."""
    spec = wl.Spec(name="wide-batch", dtype="bf16", num_seqs=num_seqs, num_q_heads=4, num_kv_heads=2, head_dim=64,
                   lens=("uniform", 1, 40), max_len=48, seed=41)
    p = wl.make_problem(spec)
    say(f"{num_seqs} sequences, balanced")
    _, got = run(p, -1)
    assert np.isfinite(got).all()
    rows = sample_rows(p, 64)
    ref = oracle.paged_decode_rows(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, p.q_len,
                                   p.dtype, rows)
    assert_parity(np.stack([got[b * p.q_len + j, h] for (b, j, h) in rows]), ref, "bf16", f"{num_seqs} sequences")


def test_balanced_kv_head_limit_falls_back():
    """More than 1024 KV heads: the balanced request runs as one pass, still exact to the oracle."""
    spec = wl.Spec(name="many-heads", dtype="bf16", num_seqs=3, num_q_heads=1025, num_kv_heads=1025, head_dim=64,
                   lens=("fixed", (5, 20, 33)), max_len=48, seed=43)
    p = wl.make_problem(spec)
    say("1025 KV heads, balanced")
    _, got = run(p, -1)
    rows = [(b, 0, h) for b in range(3) for h in (0, 1, 511, 1023, 1024)]
    ref = oracle.paged_decode_rows(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, p.q_len,
                                   p.dtype, rows)
    assert_parity(np.stack([got[b, h] for (b, _, h) in rows]), ref, "bf16", "1025 KV heads")


# ---------------------------------------------------------------------------
# the full-size workloads, in the launch configuration bench.py times

FULL = ["llama3-8b-decode", "llama3-70b-decode", "long-split", "spec-verify"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_row(name):
    """Every output row of the full workload, in the schedule bench.py times and in the
    others, against the oracle: the stated tolerance, relative L2 over the output, and
    relative L2 per row (which a lost or doubled piece of a cut sequence, or one lost
    block, fails; tests/test_gates.py)."""
    check_full_size_every_row(name, say)


def test_concurrent_calls_on_two_streams_with_their_own_workspaces():
    """Two balanced decodes of different batches, launched on two streams at once, each with
    its own workspace (the contract only forbids sharing one): each equals, bit for bit, the
    same call made alone."""
    import torch

    import paged_kv_attention_decode_amd as pa

    probs = [wl.make_problem(INV_SPEC.with_(num_seqs=n, lens=("uniform", 2, 3000), max_len=3008, seed=s))
             for n, s in ((40, 11), (33, 12))]
    devs = [DeviceProblem(p) for p in probs]
    alone = [to_host(d.step(-1).clone()) for d in devs]
    outs = [torch.empty_like(d.q) for d in devs]
    wss = [pa.new_workspace(d.q, d.k_cache, d.block_tables, p.q_len, -1) for d, p in zip(devs, probs)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        for d, p, o, ws, st in zip(devs, probs, outs, wss, streams):
            with torch.cuda.stream(st):
                pa.decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, float(p.scale), p.q_len, -1,
                          out=o, workspace=ws)
        torch.cuda.synchronize()
        for a, o in zip(alone, outs):
            assert np.array_equal(a, to_host(o))
