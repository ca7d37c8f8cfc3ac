"""Parity of pa_prefill (chunked prefill over the paged cache) with the fp64 oracle, on the GPU.

Gate: the bf16 tolerance |gpu - ref| <= 2e-2 + 1e-2 |ref| and relative L2
<= 5e-3 against oracle.paged_prefill on the same seeded inputs (the new
tokens' K/V written by pa_cache_write first), over mixes of prefill chunks,
single decode tokens and empty entries, GQA groups 1-8, head_dim 64/128,
chunks that span several 256-row workgroups with ragged tails; exact
properties: a prompt fed in chunks gives the rows of a single prefill bit for
bit, physical block ids do not matter, NaN in rows never read does not leak,
malformed query_start entries leave their rows untouched.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import host_caches_after_write, parity, to_dev, to_host, widen

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


class Dev:
    """A prefill problem in HBM: caches with the new tokens written by pa_cache_write."""

    def __init__(self, p: wl.Problem):
        import paged_kv_attention_decode_amd as pa

        self.p = p
        self.q = to_dev(p.q, p.dtype)
        self.k = to_dev(p.k_cache, p.dtype)
        self.v = to_dev(p.v_cache, p.dtype)
        self.tables = torch.from_numpy(p.block_tables).cuda()
        self.lens = torch.from_numpy(p.context_lens).cuda()
        self.qs = torch.from_numpy(p.query_start).cuda()
        if p.new_k is not None:
            pa.cache_write(to_dev(p.new_k, p.dtype), to_dev(p.new_v, p.dtype), self.k, self.v,
                           torch.from_numpy(p.slot_mapping).cuda())

    def run(self, out=None, query_start=None, max_q_len=None):
        import paged_kv_attention_decode_amd as pa

        p = self.p
        mq = int(p.q_counts.max()) if max_q_len is None else max_q_len
        o = pa.prefill(self.q, self.k, self.v, self.tables, self.lens, self.qs if query_start is None else query_start,
                       float(p.scale), mq, out=out)
        torch.cuda.synchronize()
        return o


def spec(counts, lens, G=4, d=128, n_kv=2, seed=0, **kw):
    return wl.Spec(name="prefill-small", dtype="bf16", num_seqs=len(counts), num_q_heads=G * n_kv, num_kv_heads=n_kv,
                   head_dim=d, lens=("fixed", tuple(lens)), max_len=max(lens) + 16, new_tokens=("fixed", tuple(counts)),
                   write_new_tokens=True, seed=seed, **kw)


def reference(p):
    kc, vc = host_caches_after_write(p)
    return oracle.paged_prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start, p.scale, p.dtype)


def check(p, what):
    got = widen(to_host(Dev(p).run()), "bf16")
    r = parity(got, reference(p), "bf16")
    assert r["ok"], f"{what}: {r}"
    return got


CASES = [
    dict(counts=(40, 1, 200, 0, 33), lens=(40, 300, 520, 7, 33), G=4, d=128),  # from scratch, decode, deep chunk
    dict(counts=(64, 64, 1, 1), lens=(64, 700, 65, 9), G=8, d=128),
    dict(counts=(129, 17), lens=(400, 17), G=1, d=128),                       # waves without rows
    dict(counts=(300, 17), lens=(420, 17), G=1, d=128),                       # rows cross workgroups
    dict(counts=(96, 5, 50), lens=(96, 250, 170), G=4, d=64),
    dict(counts=(31, 100), lens=(47, 333), G=3, d=128),                       # a group that does not divide 32
    dict(counts=(16, 16, 16), lens=(16, 32, 48), G=2, d=64),                  # block-aligned
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"G{c['G']}-d{c['d']}-n{'_'.join(map(str, c['counts']))}")
def test_small_prefill(case):
    c = dict(case)
    p = wl.make_problem(spec(seed=sum(c["counts"]) % 97, **c))
    say(f"prefill {case}")
    check(p, str(case))


def test_chunked_equals_single_prefill_bitwise():
    """A 300-token prompt in one call, and in chunks of 128, 100 and 72 over three calls (each
    call's cache holding the earlier chunks): identical rows."""
    import paged_kv_attention_decode_amd as pa

    prompt = 300
    p = wl.make_problem(spec((prompt,), (prompt,), G=4, seed=3))
    d = Dev(p)
    whole = to_host(d.run()).copy()
    pieces = []
    start = 0
    for size in (128, 100, 72):
        end = start + size
        out = pa.prefill(d.q[start:end].contiguous(), d.k, d.v, d.tables, torch.tensor([end], dtype=torch.int32,
                         device="cuda"), torch.tensor([0, size], dtype=torch.int32, device="cuda"), float(p.scale), size)
        torch.cuda.synchronize()
        pieces.append(to_host(out))
        start = end
    assert np.array_equal(np.concatenate(pieces), whole)


def test_permutation_invariant_and_repeatable():
    p = wl.make_problem(spec((70, 1, 150), (300, 44, 150), G=4, seed=5))
    a = to_host(Dev(p).run())
    b = to_host(Dev(wl.permute_physical(p, 3)).run())
    c = to_host(Dev(p).run())
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_poisoned_unread_rows():
    s = spec((70, 1, 150), (300, 44, 150), G=4, seed=7)
    a = to_host(Dev(wl.make_problem(s)).run())
    b = to_host(Dev(wl.make_problem(s.with_(poison=True, pad="garbage"))).run())
    assert np.isfinite(widen(b, "bf16")).all()
    assert np.array_equal(a, b)


def test_malformed_query_start_leaves_rows_untouched():
    """Entries whose range is negative or longer than max_q_len are skipped; the others are computed."""
    p = wl.make_problem(spec((20, 30, 10), (40, 60, 10), G=4, seed=9))
    d = Dev(p)
    ref = reference(p)
    sentinel = torch.full_like(d.q, 7.0)
    # sequence 1: rows 20 .. 10 (a negative range); sequence 2: 50 rows, more than max_q_len = 30
    bad = torch.tensor([0, 20, 10, 60], dtype=torch.int32, device="cuda")
    out = widen(to_host(d.run(out=sentinel.clone(), query_start=bad, max_q_len=30)), "bf16")
    r = parity(out[:20], ref[:20], "bf16")
    assert r["ok"], r
    assert (out[20:] == 7.0).all()
    # the true starts with max_q_len = 20: sequence 1 (30 new tokens) is skipped, 0 and 2 computed
    out2 = widen(to_host(d.run(out=sentinel.clone(), max_q_len=20)), "bf16")
    assert parity(out2[:20], ref[:20], "bf16")["ok"]
    assert (out2[20:50] == 7.0).all()
    assert parity(out2[50:], ref[50:], "bf16")["ok"]


def test_chunked_prefill_full_size_sampled_rows():
    p = wl.make_problem("chunked-prefill")
    say(f"chunked-prefill: lens {p.context_lens.tolist()}")
    d = Dev(p)
    out = widen(to_host(d.run()), "bf16")
    assert np.isfinite(out).all()
    kc, vc = host_caches_after_write(p)
    rng = np.random.default_rng(0)
    rows = []
    for b in range(p.num_seqs):
        n = int(p.q_counts[b])
        for i in sorted({0, n - 1, *rng.integers(0, n, size=6).tolist()}):
            rows.append((b, i, int(rng.integers(0, p.num_q_heads))))
    ref = oracle.paged_prefill_rows(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start, p.scale, p.dtype,
                                    rows)
    got = np.stack([out[int(p.query_start[b]) + i, h] for (b, i, h) in rows])
    r = parity(got, ref, "bf16")
    say(f"chunked-prefill: {r}")
    assert r["ok"], r


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_scores_rising_far_past_the_first_block(d):
    """Keys grow along the context (0.3 per position in one dimension, queries
    4 sqrt(d / 64) there), so a row's late weights exceed its reference from
    step 0 by about 2^150, past the fp32 range: only the exact two-sweep path,
    which the overflow flag must trigger, gives finite results.  The new tokens
    continue the ramp through pa_cache_write."""
    p = wl.make_problem(spec((40, 1, 300), (700, 500, 300), G=2, d=d, n_kv=1, seed=33))
    bits = lambda x: wl.round_to_bf16_bits(np.array([x], dtype=np.float32))[0]
    p.q[:] = 0
    p.k_cache[:] = 0
    p.new_k[:] = 0
    p.q[:, :, 0] = bits(4.0 * np.sqrt(d / 64.0))
    for b in range(len(p.context_lens)):
        L, n = int(p.context_lens[b]), int(p.q_counts[b])
        base = L - n
        for t in range(base):
            p.k_cache[p.block_tables[b, t // 16], t % 16, 0, 0] = bits(0.3 * t)
        for i in range(n):
            p.new_k[int(p.query_start[b]) + i, 0, 0] = bits(0.3 * (base + i))
    say(f"prefill ramp d={d}")
    check(p, f"ramp d={d}")
