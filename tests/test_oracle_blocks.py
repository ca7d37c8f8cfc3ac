"""Pins of the block-copy oracle: the copy seen through attention (copy-on-
write keeps the sharing sequence's output and gives the writer its own block),
a swap out and back is the identity, and untouched blocks keep their bits."""

import numpy as np

import oracle
import workloads as wl


def _pool(seed, NB=12, n_kv=2, d=16):
    rng = np.random.default_rng(seed)
    k = wl.round_to_bf16_bits(rng.standard_normal((NB, 16, n_kv, d)).astype(np.float32))
    v = wl.round_to_bf16_bits(rng.standard_normal((NB, 16, n_kv, d)).astype(np.float32))
    return k, v


def test_copied_blocks_equal_their_sources_bit_for_bit():
    k, v = _pool(0)
    k2, v2 = _pool(1)
    mapping = [(3, 7), (0, 1), (11, 0), (5, 12), (-1, 2)]  # the last two fall outside a pool: skipped
    ok, ov = oracle.copy_blocks(k, v, k2, v2, mapping)
    for s, d in [(3, 7), (0, 1), (11, 0)]:
        assert np.array_equal(ok[d], k[s]) and np.array_equal(ov[d], v[s])
    for d in set(range(12)) - {7, 1, 0}:
        assert np.array_equal(ok[d], k2[d]) and np.array_equal(ov[d], v2[d])


def test_swap_out_and_back_is_the_identity():
    k, v = _pool(2)
    swap_k = np.zeros((5, *k.shape[1:]), k.dtype)
    swap_v = np.zeros_like(swap_k)
    out = [(4, 0), (9, 1), (2, 2)]
    sk, sv = oracle.copy_blocks(k, v, swap_k, swap_v, out)
    wiped_k, wiped_v = k.copy(), v.copy()
    wiped_k[[4, 9, 2]] = 0
    wiped_v[[4, 9, 2]] = 0
    bk, bv = oracle.copy_blocks(sk, sv, wiped_k, wiped_v, [(d, s) for s, d in out])
    assert np.array_equal(bk, k) and np.array_equal(bv, v)


def test_copy_on_write_seen_through_attention():
    """Two sequences share their last, partly filled block.  Copy it for the
    second one, point its table at the copy and write its new token there: the
    first sequence's output is unchanged and the second one sees its token."""
    rng = np.random.default_rng(4)
    n_kv, d, n_h = 2, 16, 4
    k, v = _pool(3, NB=8, n_kv=n_kv, d=d)
    L = 20  # blocks 0..1, the second holding tokens 16..19
    tables = np.array([[5, 2, 0], [5, 2, 0]], np.int32)
    lens = np.array([L, L], np.int32)
    q = wl.round_to_bf16_bits(rng.standard_normal((2, n_h, d)).astype(np.float32))
    before = oracle.paged_decode(q, k, v, tables, lens, 0.25, 1, "bf16")
    assert np.array_equal(before[0], oracle.paged_decode(q[:1], k, v, tables[:1], lens[:1], 0.25, 1, "bf16")[0])
    # copy-on-write of block 2 into free block 6 for sequence 1, then append its token at position 20
    k1, v1 = oracle.copy_blocks(k, v, k, v, [(2, 6)])
    tables[1, 1] = 6
    new_k = wl.round_to_bf16_bits(rng.standard_normal((1, n_kv, d)).astype(np.float32))
    new_v = wl.round_to_bf16_bits(rng.standard_normal((1, n_kv, d)).astype(np.float32))
    k2, v2 = oracle.cache_write(k1, v1, new_k, new_v, np.array([6 * 16 + 4], np.int64))
    lens2 = np.array([L, L + 1], np.int32)
    after = oracle.paged_decode(q, k2, v2, tables, lens2, 0.25, 1, "bf16")
    assert np.array_equal(after[0], before[0])  # the sharer's block was not touched
    assert np.array_equal(k2[2], k[2])
    # the writer's output is attention over its 20 shared tokens plus its own new one
    rows = [(1, 0, h) for h in range(n_h)]
    got = oracle.paged_decode_rows(q, k2, v2, tables, lens2, 0.25, 1, "bf16", rows)
    K = oracle.to_f64(np.concatenate([k[5], k[2, :4], new_k]), "bf16")
    V = oracle.to_f64(np.concatenate([v[5], v[2, :4], new_v]), "bf16")
    for h in range(n_h):
        s = 0.25 * (K[:, h // 2] @ oracle.to_f64(q[1, h], "bf16"))
        w = np.exp(s - s.max())
        np.testing.assert_allclose(got[h], (w / w.sum()) @ V[:, h // 2], rtol=0, atol=1e-12)


def test_planted_mistake_swapped_pair_is_caught():
    k, v = _pool(5)
    k2, v2 = _pool(6)
    ok, _ = oracle.copy_blocks(k, v, k2, v2, [(3, 7)])
    wrong = k2.copy()
    wrong[3] = k[7]  # source and destination swapped
    assert not np.array_equal(ok, wrong)
