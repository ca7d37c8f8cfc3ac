"""Pools beyond 4 GiB: the byte offset of a high physical block needs 64 bits.

A compact problem is copied into the high end of a large pool, every other block
from the top, with its block tables, new-token slots and copy mapping renumbered.
At 8 KV heads and d 128 a block of one cache is 32 KiB in bf16 (16 KiB in fp8), so
block 131,072 (262,144) starts at 4 GiB; the pools here hold 150,000 (300,000)
blocks, 4.9 GB per cache, and every block the problem uses lies past 4 GiB.  The
rest of the pool is never written and never read.

On the large pool:
* pa_cache_write (bf16 and fp8) stores exactly what the oracle's write stores;
* pa_decode (bf16 and fp8) in one pass, 512-token partitions + pa_reduce and
  balanced matches the oracle on the compact problem (the dtype's gate);
* pa_prefill matches the oracle likewise;
* pa_copy_blocks between two positions past 4 GiB is bit-exact.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import DeviceProblem, host_caches_after_write, parity, reference_full, to_dev, to_host, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_KV, D = 8, 128
FOUR_GIB = 1 << 32


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    import paged_kv_attention_decode_amd as pa

    pa.load_library()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def big_ids(n_compact: int, nb_big: int, block_bytes: int) -> np.ndarray:
    """Compact block i -> large-pool block nb_big - 1 - 2 i, all past 4 GiB."""
    ids = nb_big - 1 - 2 * np.arange(n_compact, dtype=np.int64)
    assert ids.min() * block_bytes > FOUR_GIB
    return ids


def to_big(cache, ids: np.ndarray, nb_big: int):
    big = torch.empty((nb_big,) + tuple(cache.shape[1:]), dtype=cache.dtype, device="cuda")
    big[torch.from_numpy(ids).cuda()] = cache
    return big


def on_big_pool(p: wl.Problem, nb_big: int):
    """p resident in HBM with its blocks at the high ids of an nb_big-block pool."""
    d = DeviceProblem(p)
    block_bytes = d.k_cache[0].numel() * d.k_cache.element_size()
    ids = big_ids(p.k_cache.shape[0], nb_big, block_bytes)
    d.k_cache = to_big(d.k_cache, ids, nb_big)
    d.v_cache = to_big(d.v_cache, ids, nb_big)
    d.block_tables = torch.from_numpy(ids[p.block_tables].astype(np.int32)).cuda()
    if p.slot_mapping is not None:
        slots = ids[p.slot_mapping // 16] * 16 + p.slot_mapping % 16
        d.slots = torch.from_numpy(slots.astype(np.int64)).cuda()
    torch.cuda.synchronize()
    return d, ids


KINDS = {
    "bf16": dict(nb_big=150_000, kv="same"),
    "fp8": dict(nb_big=300_000, kv="fp8"),
}


@pytest.mark.parametrize("kind", sorted(KINDS))
def test_write_decode_and_copy_beyond_4gib(kind):
    import paged_kv_attention_decode_amd as pa

    k = KINDS[kind]
    spec = wl.Spec(name="big-pool", dtype="bf16", num_seqs=4, num_q_heads=32, num_kv_heads=N_KV, head_dim=D,
                   lens=("fixed", (300, 517, 64, 1000)), max_len=1024, write_new_tokens=True, kv=k["kv"], seed=21)
    p = wl.make_problem(spec)
    say(f"{kind}: {k['nb_big']}-block pool, {p.k_cache.shape[0]} blocks used")
    d, ids = on_big_pool(p, k["nb_big"])
    ref = reference_full(p)
    kc, vc = host_caches_after_write(p)
    for ps in (0, 512, -1):
        d.workspace = None
        got = widen(to_host(d.step(ps).clone()), p.dtype)
        r = parity(got, ref, p.dtype)
        say(f"{kind}: partition {ps}: {r}")
        assert r["ok"], (kind, ps, r)
    # the write, at its slots in the large pool
    blk, off = ids[p.slot_mapping // 16], p.slot_mapping % 16
    bt, ot = torch.from_numpy(blk).cuda(), torch.from_numpy(off).cuda()
    assert np.array_equal(to_host(d.k_cache[bt, ot]), kc[p.slot_mapping // 16, p.slot_mapping % 16])
    assert np.array_equal(to_host(d.v_cache[bt, ot]), vc[p.slot_mapping // 16, p.slot_mapping % 16])
    # copy every used block to the free block just below it (also past 4 GiB)
    mapping = torch.from_numpy(np.stack([ids, ids - 1], axis=1)).cuda()
    pa.copy_blocks(d.k_cache, d.v_cache, d.k_cache, d.v_cache, mapping)
    src, dst = torch.from_numpy(ids).cuda(), torch.from_numpy(ids - 1).cuda()
    assert torch.equal(d.k_cache[dst], d.k_cache[src]) and torch.equal(d.v_cache[dst], d.v_cache[src])
    del d
    torch.cuda.empty_cache()


def test_prefill_beyond_4gib():
    import paged_kv_attention_decode_amd as pa

    counts, lens = (40, 1, 90), (300, 517, 90)
    spec = wl.Spec(name="big-prefill", dtype="bf16", num_seqs=3, num_q_heads=32, num_kv_heads=N_KV, head_dim=D,
                   lens=("fixed", lens), max_len=max(lens) + 16, new_tokens=("fixed", counts),
                   write_new_tokens=True, seed=22)
    p = wl.make_problem(spec)
    d, _ = on_big_pool(p, KINDS["bf16"]["nb_big"])
    pa.cache_write(d.new_k, d.new_v, d.k_cache, d.v_cache, d.slots)
    qs = torch.from_numpy(p.query_start).cuda()
    got = widen(to_host(pa.prefill(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, qs, float(p.scale),
                                   int(p.q_counts.max()))), "bf16")
    kc, vc = host_caches_after_write(p)
    ref = oracle.paged_prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start, p.scale, p.dtype)
    r = parity(got, ref, "bf16")
    say(f"prefill: {r}")
    assert r["ok"], r
    del d
    torch.cuda.empty_cache()
