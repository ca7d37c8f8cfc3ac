"""pa_copy_blocks on the GPU: bit-exact against the oracle for bf16, fp32 and
fp8 pools, within one pool (copy-on-write) and between pools (swapping),
with out-of-pool pairs skipped; and a copy-on-write step end to end through
the cache write and the decode."""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from _gpu import parity, to_dev, to_host, widen

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


def pool(rng, NB, n_kv, d, kind):
    shape = (NB, 16, n_kv, d)
    if kind == "fp8":
        return rng.integers(0, 256, size=shape).astype(np.uint8)
    x = rng.standard_normal(shape).astype(np.float32)
    return wl.round_to_bf16_bits(x) if kind == "bf16" else x


@pytest.mark.parametrize("kind", ["bf16", "f32", "fp8"])
@pytest.mark.parametrize("same_pool", [True, False], ids=["copy-on-write", "swap"])
def test_copy_blocks_bit_exact(kind, same_pool):
    import paged_kv_attention_decode_amd as pa

    rng = np.random.default_rng(7)
    n_kv, d = 8, 128
    sk, sv = pool(rng, 40, n_kv, d, kind), pool(rng, 40, n_kv, d, kind)
    if same_pool:
        dk, dv = sk, sv
        ids = rng.permutation(40)
        mapping = np.stack([ids[:12], ids[12:24]], axis=1)  # sources and destinations disjoint
    else:
        dk, dv = pool(rng, 25, n_kv, d, kind), pool(rng, 25, n_kv, d, kind)
        mapping = np.stack([rng.permutation(40)[:15], rng.permutation(25)[:15]], axis=1)
    mapping = np.concatenate([mapping, [[-1, 3], [2, 999], [45, 0]]]).astype(np.int64)  # skipped pairs
    say(f"copy blocks kind={kind} same_pool={same_pool}")
    src_k, src_v = to_dev(sk, "x"), to_dev(sv, "x")
    dst_k, dst_v = (src_k, src_v) if same_pool else (to_dev(dk, "x"), to_dev(dv, "x"))
    pa.copy_blocks(src_k, src_v, dst_k, dst_v, torch.from_numpy(mapping).cuda())
    torch.cuda.synchronize()
    rk, rv = oracle.copy_blocks(sk, sv, dk, dv, mapping)
    assert np.array_equal(to_host(dst_k), rk)
    assert np.array_equal(to_host(dst_v), rv)


def test_copy_on_write_then_decode():
    """Two sequences share their last block; the second gets a private copy of
    it, writes its new token there and decodes: the GPU path equals the oracle
    doing the same steps, and the first sequence's output does not move."""
    import paged_kv_attention_decode_amd as pa

    rng = np.random.default_rng(9)
    n_kv, d, n_h, NB = 2, 128, 8, 10
    k, v = pool(rng, NB, n_kv, d, "bf16"), pool(rng, NB, n_kv, d, "bf16")
    tables = np.array([[4, 7, 0], [4, 7, 0]], np.int32)
    q = wl.round_to_bf16_bits(rng.standard_normal((2, n_h, d)).astype(np.float32))
    new_k = wl.round_to_bf16_bits(rng.standard_normal((1, n_kv, d)).astype(np.float32))
    new_v = wl.round_to_bf16_bits(rng.standard_normal((1, n_kv, d)).astype(np.float32))
    L = 27
    # oracle: copy block 7 -> 9 for sequence 1, point its table there, write its token at position 27
    ok, ov = oracle.copy_blocks(k, v, k, v, [(7, 9)])
    t2 = tables.copy()
    t2[1, 1] = 9
    ok, ov = oracle.cache_write(ok, ov, new_k, new_v, np.array([9 * 16 + 11], np.int64))
    lens = np.array([L, L + 1], np.int32)
    ref = oracle.paged_decode(q, ok, ov, t2, lens, 0.0883883461356163, 1, "bf16")
    # GPU
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    pa.copy_blocks(kd, vd, kd, vd, torch.tensor([[7, 9]], dtype=torch.int64, device="cuda"))
    pa.cache_write(to_dev(new_k, "bf16"), to_dev(new_v, "bf16"), kd, vd,
                   torch.tensor([9 * 16 + 11], dtype=torch.int64, device="cuda"))
    out = pa.decode(to_dev(q, "bf16"), kd, vd, torch.from_numpy(t2).cuda(), torch.from_numpy(lens).cuda(),
                    0.0883883461356163, 1, 0)
    torch.cuda.synchronize()
    got = widen(to_host(out), "bf16")
    r = parity(got, ref, "bf16")
    assert r["ok"], r
    assert np.array_equal(to_host(kd)[7], k[7])  # the shared block is untouched


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_swap_out_to_pinned_host_and_back(kind):
    """Blocks go out to a pinned host pool and come back into other device
    blocks, bit-exact against the oracle doing the same two copies."""
    import paged_kv_attention_decode_amd as pa

    rng = np.random.default_rng(11)
    n_kv, d = 4, 128
    gk, gv = pool(rng, 30, n_kv, d, kind), pool(rng, 30, n_kv, d, kind)
    hk, hv = pool(rng, 12, n_kv, d, kind), pool(rng, 12, n_kv, d, kind)
    out_map = np.stack([rng.permutation(30)[:9], rng.permutation(12)[:9]], axis=1).astype(np.int64)
    back_ids = rng.permutation(30)
    back_map = np.stack([out_map[:, 1], back_ids[:9]], axis=1).astype(np.int64)
    say(f"swap via pinned host kind={kind}")
    dk, dv = to_dev(gk, "x"), to_dev(gv, "x")
    host_k, host_v = to_dev(hk, "x", "cpu").pin_memory(), to_dev(hv, "x", "cpu").pin_memory()
    assert host_k.is_pinned() and host_v.is_pinned()
    pa.copy_blocks(dk, dv, host_k, host_v, torch.from_numpy(out_map).cuda())  # swap out
    torch.cuda.synchronize()
    ok, ov = oracle.copy_blocks(gk, gv, hk, hv, out_map)
    assert np.array_equal(to_host(host_k), ok)
    assert np.array_equal(to_host(host_v), ov)
    pa.copy_blocks(host_k, host_v, dk, dv, torch.from_numpy(back_map).cuda())  # swap in
    torch.cuda.synchronize()
    rk, rv = oracle.copy_blocks(ok, ov, gk, gv, back_map)
    assert np.array_equal(to_host(dk), rk)
    assert np.array_equal(to_host(dv), rv)


def test_pageable_host_memory_is_refused():
    """The library launches nothing on memory the GPU cannot reach."""
    import ctypes

    import paged_kv_attention_decode_amd as pa

    lib = pa.load_library()
    dev = torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16, device="cuda")
    pageable = np.zeros((4, 16, 2, 64), np.uint16)
    mapping = torch.tensor([[0, 1]], dtype=torch.int64, device="cuda")
    hp = ctypes.c_void_p(pageable.ctypes.data)
    dp = ctypes.c_void_p(dev.data_ptr())
    st = lib.pa_copy_blocks(dp, dp, hp, hp, ctypes.c_void_p(mapping.data_ptr()), 1, 4, 4, 4096, None)
    assert st == 6, pa.status_string(st)
    st = lib.pa_copy_blocks(hp, hp, dp, dp, ctypes.c_void_p(mapping.data_ptr()), 1, 4, 4, 4096, None)
    assert st == 6, pa.status_string(st)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        pa.copy_blocks(dev, dev, torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16), torch.zeros(4, 16, 2, 64,
                       dtype=torch.bfloat16), mapping)
