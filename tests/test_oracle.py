"""The oracle against what the pages and the mathematics fix (CPU only).

Pins:
* brute force: torch SDPA (float64) on contiguous K/V placed into blocks token
  by token, GQA by repeat_interleave, causal mask aligned to the context end;
* closed forms: one-token context returns V; identical keys give an exact
  token count; two tokens give v0 + sigmoid(s1 - s0)(v1 - v0);
* invariants: physical-block permutation, rows of softmax weights summing to
  1, split/merge equal to the unsplit result, future tokens not changing a
  verify row, unread rows poisoned with NaN not changing anything, GQA equal
  to MHA with replicated KV heads;
* the cache write: rows land at their slots, everything else keeps its bits;
* planted mistakes: each plausible error in an oracle step fails some pin.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa
import workloads as wl
import _pins as pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    dict(lens=(1, 16, 17, 40), n_h=4, n_kv=2, d=16, q_len=1),
    dict(lens=(5, 15, 16, 33), n_h=8, n_kv=2, d=32, q_len=5),
    dict(lens=(2, 48, 49), n_h=3, n_kv=3, d=8, q_len=2),
    dict(lens=(7,), n_h=8, n_kv=1, d=64, q_len=7),
])
def test_matches_sdpa_bruteforce(dtype, shape):
    assert pins.pin_sdpa(seed=11, dtype=dtype, **shape)


def test_permutation_invariance_is_exact():
    assert pins.pin_permutation(dtype="bf16", q_len=1)
    assert pins.pin_permutation(dtype="f32", q_len=3)


def test_one_token_context_returns_v():
    assert pins.pin_one_token("f32")
    assert pins.pin_one_token("bf16")


@pytest.mark.parametrize("q_len", [1, 5])
def test_identical_keys_give_exact_counts(q_len):
    got, expect = pins.count_probe([5, 16, 17, 70, 129], 8, 2, 16, q_len)
    assert np.max(np.abs(got - expect)) <= 1e-12
    # the plain "mean of V" statement: with identical keys every visible value row has weight 1/(p+1)
    P = pins.build_paged(9, [9, 20], 2, 1, 8, 1, "f32")
    P["k_cache"][:] = 0.5
    got = pins.run_oracle(P, 1.0)
    for b in range(2):
        np.testing.assert_allclose(got[b, 0], P["Vs"][b][:, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_two_token_closed_form():
    assert pins.pin_two_token_closed_form()


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(0)
    for n in (1, 2, 17, 1000):
        s = rng.standard_normal(n) * 10
        p = oracle.softmax_weights(s)
        assert abs(p.sum() - 1.0) <= 1e-12
        assert np.all(p >= 0)
    # large positive scores must not overflow
    p = oracle.softmax_weights(np.array([1000.0, 999.0]))
    assert np.isfinite(p).all() and abs(p.sum() - 1) <= 1e-15


@pytest.mark.parametrize("partition_size", [16, 32, 48, 512])
@pytest.mark.parametrize("q_len", [1, 5])
def test_split_merge_equals_full(partition_size, q_len):
    P = pins.build_paged(5, [5, 31, 32, 33, 97], 4, 2, 16, q_len, "bf16")
    full = pins.run_oracle(P, 0.3)
    split = oracle.paged_decode_split(P["q"], P["k_cache"], P["v_cache"], P["block_tables"],
                                      P["context_lens"], 0.3, q_len, "bf16", partition_size)
    assert np.max(np.abs(full - split)) <= 1e-12


def test_single_partition_is_identity():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((20, 8))
    V = rng.standard_normal((20, 8))
    q = rng.standard_normal(8)
    ms, ls, accs = oracle.partition_partials(q, K, V, 0.5, 20, 20, 64)
    assert ms.shape == (1,)
    np.testing.assert_array_equal(oracle.merge_partials(ms, ls, accs), accs[0] / ls[0])


def test_fully_masked_partition_has_zero_weight():
    # the last partition holds only tokens a row may not see yet
    rng = np.random.default_rng(4)
    K = rng.standard_normal((34, 8))
    V = rng.standard_normal((34, 8))
    q = rng.standard_normal(8)
    ms, ls, accs = oracle.partition_partials(q, K, V, 0.5, 32, 34, 16)
    assert ls[2] == 0 and ms[2] == -np.inf
    ref = oracle.attend_row(q, K[:32], V[:32], 0.5)
    assert np.max(np.abs(oracle.merge_partials(ms, ls, accs) - ref)) <= 1e-13


def test_future_tokens_do_not_change_verify_rows():
    q_len = 5
    P = pins.build_paged(8, [21, 40], 4, 2, 16, q_len, "bf16")
    base = pins.run_oracle(P, 0.2)
    for j in range(q_len):
        Q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in P.items()}
        for b, L in enumerate(P["context_lens"]):
            for t in range(int(L) - q_len + j + 1, int(L)):
                blk = Q["block_tables"][b, t // 16]
                Q["k_cache"][blk, t % 16] = np.uint16(0x4000)  # 2.0
                Q["v_cache"][blk, t % 16] = np.uint16(0xC000)  # -2.0
        out = pins.run_oracle(Q, 0.2)
        for b in range(2):
            for jj in range(j + 1):
                np.testing.assert_array_equal(out[b * q_len + jj], base[b * q_len + jj])


def test_unread_rows_are_never_read():
    spec = wl.Spec(name="t", dtype="bf16", num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=16,
                   lens=("fixed", (3, 16, 17, 45)), max_len=64, q_len=2, seed=5)
    clean = wl.make_problem(spec)
    dirty = wl.make_problem(spec.with_(poison=True, pad="garbage"))
    a = oracle.paged_decode(clean.q, clean.k_cache, clean.v_cache, clean.block_tables, clean.context_lens,
                            clean.scale, 2, "bf16")
    # padding of the clean tables is valid-but-wrong ids; the dirty tables hold huge ids
    b = oracle.paged_decode(dirty.q, dirty.k_cache, dirty.v_cache, dirty.block_tables, dirty.context_lens,
                            dirty.scale, 2, "bf16")
    assert np.isfinite(b).all()
    np.testing.assert_array_equal(a, b)


def test_gqa_equals_replicated_mha():
    P = pins.build_paged(12, [9, 33], 8, 2, 16, 1, "f32")
    gqa = pins.run_oracle(P, 0.3)
    mha = dict(P)
    mha["k_cache"] = np.repeat(P["k_cache"], 4, axis=2)
    mha["v_cache"] = np.repeat(P["v_cache"], 4, axis=2)
    np.testing.assert_array_equal(pins.run_oracle(mha, 0.3), gqa)


def test_cache_write_places_rows_and_keeps_the_rest():
    assert pins.pin_cache_write()


def test_cache_write_f32_keeps_nan_payload_bits():
    kc = np.zeros((2, 16, 1, 4), dtype=np.float32)
    vc = np.zeros_like(kc)
    k = np.array([[[1.0, -0.0, np.inf, 0.0]]], dtype=np.float32)
    k.view(np.uint32)[0, 0, 3] = 0x7FC01234  # a NaN with a payload
    v = -k
    kc2, vc2 = oracle.cache_write(kc, vc, k, v, np.array([17]))
    assert np.array_equal(kc2.view(np.uint32)[1, 1], k.view(np.uint32)[0])
    assert np.array_equal(vc2.view(np.uint32)[1, 1], v.view(np.uint32)[0])


def test_cache_write_rejects_out_of_pool_slot():
    kc = np.zeros((2, 16, 1, 4), dtype=np.uint16)
    with pytest.raises(IndexError):
        oracle.cache_write(kc, kc, kc[0, :1], kc[0, :1], np.array([32]))


def test_write_then_attend_sees_new_tokens():
    spec = wl.Spec(name="t", dtype="bf16", num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                   lens=("fixed", (6, 16, 40)), max_len=48, q_len=5, write_new_tokens=True, seed=2)
    p = wl.make_problem(spec)
    kc, vc = oracle.cache_write(p.k_cache, p.v_cache, p.new_k, p.new_v, p.slot_mapping)
    for b in range(3):
        L = int(p.context_lens[b])
        K = oracle.gather_sequence(kc, p.block_tables[b], L)
        V = oracle.gather_sequence(vc, p.block_tables[b], L)
        np.testing.assert_array_equal(K[L - 5:], p.new_k[b * 5:(b + 1) * 5])
        np.testing.assert_array_equal(V[L - 5:], p.new_v[b * 5:(b + 1) * 5])


def test_bf16_widening_is_exact():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0x0001, 0x4049], dtype=np.uint16)
    expect = [0.0, -0.0, 1.0, -1.0, np.inf, 2.0 ** -133, 3.140625]
    got = oracle.to_f64(bits, "bf16")
    assert list(got) == expect


# ---------------------------------------------------------------------------
# golden sizing values printed on the pages


def _golden():
    with open(os.path.join(HERE, "golden", "kv_sizing.json")) as f:
        return json.load(f)


def test_kv_bytes_per_token_match_pages():
    for row in _golden()["per_token"]:
        got = wl.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"], row["bytes_per_value"])
        assert got == row["bytes"], row["cite"]


def test_kv_bytes_per_block_match_pages():
    for row in _golden()["per_block"]:
        got = wl.kv_bytes_per_block(row["block_tokens"], row["layers"], row["kv_heads"], row["head_dim"],
                                    row["bytes_per_value"])
        assert got == row["bytes"], row["cite"]


def test_block_counts_match_pages():
    g = _golden()
    for row in g["blocks_for_tokens"]:
        assert oa.block_count(row["tokens"], row["block_tokens"]) == row["blocks"], row["cite"]
    w = g["max_waste_tokens"]
    bs = w["block_tokens"]
    assert max(bs * oa.block_count(n, bs) - n for n in range(1, 10 * bs)) == w["waste"]


def test_algorithmic_bytes_follow_the_per_token_formula():
    p = wl.make_problem(wl.Spec(name="t", dtype="bf16", num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                                lens=("fixed", (6, 16, 40)), max_len=48, seed=2))
    ab = wl.algorithmic_bytes(p)
    assert ab["kv_logical"] == int(p.context_lens.sum()) * wl.kv_bytes_per_token(1, 2, 16, 2)


# ---------------------------------------------------------------------------
# planted mistakes: every one must fail at least one pin


def test_pins_pass_on_the_oracle():
    assert pins.failing_pins() == []


MUTATIONS = {
    "gqa_modulo_map": ("kv_head_of", lambda h, group: h % 2),
    "context_off_by_one": ("visible_tokens", lambda L, q_len, j: L - q_len + j),
    "no_causal_mask": ("visible_tokens", lambda L, q_len, j: L),
    "mask_top_left": ("visible_tokens", lambda L, q_len, j: j + 1),
    "block_index_not_translated": (
        "gather_sequence",
        lambda cache, row, L, bs=16: np.concatenate([cache[i] for i in range(-(-L // bs))], axis=0)[:L]),
    "unnormalized_weights": ("softmax_weights", lambda s: np.exp(s - s.max())),
    "dropped_scale": ("attend_row", lambda q, K, V, scale: oa.softmax_weights(K @ q) @ V),
    "inverted_scale": ("attend_row", lambda q, K, V, scale: oa.softmax_weights((K @ q) / scale) @ V),
    "bf16_wrong_shift": (
        "to_f64",
        lambda a, dtype: ((np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32)
                          .astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float32).astype(np.float64))),
    "merge_without_rescale": (
        "merge_partials",
        lambda ms, ls, accs: accs[ls > 0].sum(axis=0) / ls[ls > 0].sum()),
    "cache_write_block_row_swapped": (
        "cache_write", None),  # filled in below
}


def _swapped_cache_write(k_cache, v_cache, k, v, slot_mapping, block_size=16):
    kc, vc = k_cache.copy(), v_cache.copy()
    NB = kc.shape[0]
    for t, s in enumerate(slot_mapping):
        if s < 0:
            continue
        kc[s % NB, s // NB % block_size] = k[t]  # block and row taken the wrong way round
        vc[s % NB, s // NB % block_size] = v[t]
    return kc, vc


MUTATIONS["cache_write_block_row_swapped"] = ("cache_write", _swapped_cache_write)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert pins.failing_pins(), f"no pin fails with {name} planted"
