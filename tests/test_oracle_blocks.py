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


def test_worked_example_four_samples_of_a_thousand_token_prompt():
    """The parallel-sampling exercise of "LLM serving: KV cache, batching, paged
    attention and quantization" (learn.mohebi.ai, section 8 "Check yourself",
    question 4): 4 samples share a 1000-token prompt
    in ceil(1000/16) = 63 blocks (62 full, one holding 8 tokens) with reference
    count 4.  Each writes its first new token into the shared last block: the
    first three writers get a private copy, the last finds the count at 1 and
    writes in place, for 66 blocks in all.  Played here with reference counts
    and the oracle's copy and cache write; each sample then sees the 1000
    shared tokens plus its own token, and nothing else."""
    rng = np.random.default_rng(12)
    n_kv, d, prompt, S = 1, 16, 1000, 4
    NB = 80
    k = wl.round_to_bf16_bits(rng.standard_normal((NB, 16, n_kv, d)).astype(np.float32))
    v = wl.round_to_bf16_bits(rng.standard_normal((NB, 16, n_kv, d)).astype(np.float32))
    n_blocks = -(-prompt // 16)
    assert n_blocks == 63 and prompt - 62 * 16 == 8
    free = list(range(n_blocks, NB))
    refs = {b: S for b in range(n_blocks)}
    tables = np.tile(np.arange(n_blocks, dtype=np.int32), (S, 1))
    new_k = wl.round_to_bf16_bits(rng.standard_normal((S, n_kv, d)).astype(np.float32))
    new_v = wl.round_to_bf16_bits(rng.standard_normal((S, n_kv, d)).astype(np.float32))
    kk, vv = k, v
    for s in range(S):
        last = int(tables[s, -1])
        if refs[last] > 1:  # shared: copy before writing
            mine = free.pop(0)
            kk, vv = oracle.copy_blocks(kk, vv, kk, vv, [(last, mine)])
            refs[last] -= 1
            refs[mine] = 1
            tables[s, -1] = mine
        kk, vv = oracle.cache_write(kk, vv, new_k[s:s + 1], new_v[s:s + 1],
                                    np.array([int(tables[s, -1]) * 16 + prompt % 16], np.int64))
    assert len(refs) == 66 and sum(1 for c in refs.values() if c == S) == 62
    assert refs[n_blocks - 1] == 1  # the last writer kept the original block
    lens = np.full(S, prompt + 1, np.int32)
    q = wl.round_to_bf16_bits(rng.standard_normal((S, 2, d)).astype(np.float32))
    got = oracle.paged_decode(q, kk, vv, tables, lens, 0.25, 1, "bf16")
    K0 = oracle.to_f64(k.reshape(-1, n_kv, d)[:prompt, 0], "bf16")
    V0 = oracle.to_f64(v.reshape(-1, n_kv, d)[:prompt, 0], "bf16")
    for s in range(S):
        K = np.concatenate([K0, oracle.to_f64(new_k[s, 0], "bf16")[None]])
        V = np.concatenate([V0, oracle.to_f64(new_v[s, 0], "bf16")[None]])
        for h in range(2):
            sc = 0.25 * (K @ oracle.to_f64(q[s, h], "bf16"))
            w = np.exp(sc - sc.max())
            np.testing.assert_allclose(got[s, h], (w / w.sum()) @ V, rtol=0, atol=1e-12)
