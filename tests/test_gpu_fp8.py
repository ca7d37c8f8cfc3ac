"""Parity of the fp8 (E4M3) KV-cache path with the fp64 oracle, on the GPU.

Gates: cache writes bit-exact (the codes are integers decided from the fp32
quotient on both sides); decode outputs within the bf16 gate
|gpu - ref| <= 2e-2 + 1e-2 |ref| and relative L2 <= 5e-3 against the oracle
over the same codes and scales (the dequantized keys and values are exact on
both sides, so the tolerance covers only the bf16 query/weights/output).
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import check_full_size_every_row, DeviceProblem, host_caches_after_write, parity, reference_full, reference_rows, sample_rows, to_host, widen

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


def run(p, partition_size, write=True):
    d = DeviceProblem(p)
    out = d.step(partition_size, write)
    torch.cuda.synchronize()
    return d, widen(to_host(out), p.dtype)


def assert_parity(got, ref, what, **kw):
    r = parity(got, ref, "bf16", **kw)
    assert r["ok"], f"{what}: {r}"
    return r


def small(G=4, d=128, q_len=1, n_kv=2, S=7, lens=None, seed=0, **kw):
    lens = lens or ("uniform", q_len, 700)
    return wl.Spec(name="fp8-small", dtype="bf16", num_seqs=S, num_q_heads=G * n_kv, num_kv_heads=n_kv, head_dim=d,
                   lens=lens, max_len=720, q_len=q_len, write_new_tokens=True, kv="fp8", seed=seed, **kw)


# ---------------------------------------------------------------------------
# pa_cache_write_fp8: bit-exact


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("n_kv,d", [(8, 128), (2, 64), (3, 128)])
def test_cache_write_fp8_bit_exact(src, n_kv, d):
    import paged_kv_attention_decode_amd as pa

    rng = np.random.default_rng(n_kv * 10 + d)
    NB, T = 24, 37
    kc = rng.integers(0, 256, size=(NB, 16, n_kv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(NB, 16, n_kv, d)).astype(np.uint8)
    k = (rng.standard_normal((T, n_kv, d)) * 2.0).astype(np.float32)
    v = (rng.standard_normal((T, n_kv, d)) * 2.0).astype(np.float32)
    k[0, 0, :4] = [1e4, -1e4, 0.0, -0.0]  # saturation and signed zero
    if src == "bf16":
        k, v = wl.round_to_bf16_bits(k), wl.round_to_bf16_bits(v)
    slots = rng.permutation(NB * 16)[:T].astype(np.int64)
    slots[5] = -1
    slots[11] = NB * 16 + 3  # outside the pool: skipped
    ks = wl.fp8_scales(n_kv, "k")
    vs = wl.fp8_scales(n_kv, "v")
    say(f"fp8 cache write src={src} n_kv={n_kv} d={d}")
    kd, vd = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    valid = slots.copy()
    valid[11] = -1  # the oracle raises on out-of-pool slots; the library skips them
    pa.cache_write_fp8(dev(k), dev(v), kd, vd, torch.from_numpy(slots).cuda(), torch.from_numpy(ks).cuda(),
                       torch.from_numpy(vs).cuda())
    torch.cuda.synchronize()
    rk, rv = oracle.cache_write_fp8(kc, vc, k, v, valid, ks, vs, src)
    assert np.array_equal(kd.cpu().numpy(), rk)
    assert np.array_equal(vd.cpu().numpy(), rv)
    assert rk.reshape(-1, n_kv, d)[slots[0], 0, 0] == 0x7E and rk.reshape(-1, n_kv, d)[slots[0], 0, 1] == 0xFE


# ---------------------------------------------------------------------------
# decode


CASES = [dict(G=4, d=128, q_len=1), dict(G=1, d=128, q_len=1), dict(G=8, d=128, q_len=1), dict(G=4, d=64, q_len=1),
         dict(G=8, d=128, q_len=5), dict(G=8, d=64, q_len=5), dict(G=16, d=128, q_len=4), dict(G=2, d=128, q_len=2)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"G{c['G']}-d{c['d']}-q{c['q_len']}")
def test_small_fp8(case):
    p = wl.make_problem(small(seed=31 + case["G"] + case["d"] + case["q_len"], **case))
    ref = reference_full(p)
    for ps in (0, 16, 48, 512, -1):
        say(f"fp8 decode {case} partition={ps} lens={p.context_lens.tolist()}")
        _, got = run(p, ps)
        assert_parity(got, ref, f"partition {ps}")


def test_fp8_sweep_of_lengths():
    """Every context length 1..48 (block boundaries, ragged tails) at 8 and 40 rows."""
    for G, q_len in ((8, 1), (8, 5)):
        lens = tuple(range(q_len, 49))
        spec = small(G=G, q_len=q_len, d=128, n_kv=1, S=len(lens), lens=("fixed", lens), seed=3)
        p = wl.make_problem(spec)
        ref = reference_full(p)
        for ps in (0, 16, -1):
            say(f"fp8 sweep G={G} q_len={q_len} ps={ps}")
            _, got = run(p, ps)
            assert_parity(got, ref, f"sweep ps={ps}")


@pytest.mark.parametrize("ps", [0, 64, -1])
def test_fp8_permutation_invariant_and_repeatable(ps):
    spec = small(G=4, q_len=2, seed=41)
    p = wl.make_problem(spec)
    _, a = run(p, ps)
    _, b = run(wl.permute_physical(p, 5), ps)
    _, c = run(p, ps)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_fp8_poisoned_unread_codes():
    spec = small(G=8, q_len=5, seed=43)
    clean = wl.make_problem(spec)
    dirty = wl.make_problem(spec.with_(poison=True, pad="garbage"))
    for ps in (0, 64, -1):
        _, a = run(clean, ps)
        _, b = run(dirty, ps)
        assert np.isfinite(b).all()
        assert np.array_equal(a, b)


def test_fp8_one_token_returns_scaled_v():
    spec = small(G=4, q_len=1, S=5, lens=("fixed", (1, 1, 1, 1, 1)), seed=47).with_(write_new_tokens=False)
    p = wl.make_problem(spec)
    _, got = run(p, 0)
    table = oracle.e4m3_table()
    for b in range(5):
        for h in range(p.num_q_heads):
            g = h // p.spec.group
            want = table[p.v_cache[p.block_tables[b, 0], 0, g]] * float(p.v_scale[g])
            np.testing.assert_allclose(got[b, h], want, rtol=2 ** -8, atol=0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G,q_len", [(4, 1), (8, 5)])
def test_fp8_scores_rising_far_past_the_first_block(G, q_len, d):
    """Key codes grow along the context in one dimension (to 7 after the
    per-head scale; queries 256 there), so weights relative to a wave's first
    block exceed 2^64 even within one 512-token partition and the fp8 kernel
    must take its exact two-pass path, in every schedule."""
    spec = small(G=G, d=d, q_len=q_len, n_kv=2, S=3, lens=("fixed", (1000, 700, 40)), seed=53).with_(
        write_new_tokens=False, max_len=1024)
    p = wl.make_problem(spec)
    p.q[:] = 0
    p.q[:, :, 0] = wl.round_to_bf16_bits(np.array([256.0], dtype=np.float32))[0]
    vals = np.zeros(p.k_cache.shape, dtype=np.float32)
    for b, L in enumerate(p.context_lens):
        for t in range(int(L)):
            vals[p.block_tables[b, t // 16], t % 16, :, 0] = 7.0 * t / 1000.0
    p.k_cache[:] = wl.to_fp8_codes(wl.round_to_bf16_bits(vals), p.k_scale)
    ref = reference_full(p)
    for ps in (0, 512, -1):
        say(f"fp8 ramp G={G} q_len={q_len} d={d} ps={ps}")
        _, got = run(p, ps)
        assert np.isfinite(got).all()
        assert_parity(got, ref, f"fp8 ramp ps={ps}")


def test_fp8_full_size_every_row():
    """Every output row of the full llama3-8b-decode-fp8kv workload, in the schedule bench.py times and in the
    others, against the oracle (stated tolerance, relative L2, and relative L2 per row)."""
    check_full_size_every_row("llama3-8b-decode-fp8kv", say)
