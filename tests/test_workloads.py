"""Seeded generator sanity (CPU only): reproducible, well-formed block tables and slots."""

import numpy as np
import pytest

import workloads as wl


SMALL = wl.Spec(name="s", dtype="bf16", num_seqs=5, num_q_heads=8, num_kv_heads=2, head_dim=16,
                lens=("uniform", 5, 90), max_len=96, q_len=5, write_new_tokens=True, shared_prefix_blocks=0, seed=3)


def test_reproducible():
    a = wl.make_problem(SMALL)
    b = wl.make_problem(SMALL)
    for name in ("context_lens", "block_tables", "q", "k_cache", "v_cache", "new_k", "new_v", "slot_mapping"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))


def test_fill_normal_independent_of_threads(monkeypatch):
    a = wl.fill_normal((3, 1 << 21), "bf16", 7, 2)
    monkeypatch.setattr(wl, "_threads", lambda: 1)
    b = wl.fill_normal((3, 1 << 21), "bf16", 7, 2)
    np.testing.assert_array_equal(a, b)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], dtype=np.float32)
    got = wl.bf16_bits_to_f32(wl.round_to_bf16_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5], dtype=np.float32))


def test_blocks_distinct_and_in_range():
    p = wl.make_problem(SMALL)
    used = []
    for b in range(p.num_seqs):
        nb = -(-int(p.context_lens[b]) // 16)
        used.extend(p.block_tables[b, :nb].tolist())
    assert len(used) == len(set(used))
    assert min(used) >= 0 and max(used) < p.num_blocks


def test_slots_unique_and_at_the_newest_positions():
    p = wl.make_problem(SMALL)
    assert len(set(p.slot_mapping.tolist())) == len(p.slot_mapping)
    for b in range(p.num_seqs):
        L = int(p.context_lens[b])
        for j in range(p.q_len):
            pos = L - p.q_len + j
            s = int(p.slot_mapping[b * p.q_len + j])
            assert s // 16 == p.block_tables[b, pos // 16] and s % 16 == pos % 16


def test_shared_prefix_layout():
    spec = SMALL.with_(lens=("uniform", 40, 90), shared_prefix_blocks=2)
    p = wl.make_problem(spec)
    assert (p.block_tables[:, :2] == p.block_tables[0, :2]).all()
    private = set()
    for b in range(p.num_seqs):
        nb = -(-int(p.context_lens[b]) // 16)
        row = p.block_tables[b, 2:nb].tolist()
        assert not (set(row) & private) and not (set(row) & set(p.block_tables[0, :2].tolist()))
        private |= set(row)
    assert all(s // 16 not in set(p.block_tables[0, :2].tolist()) for s in p.slot_mapping.tolist())


def test_named_configs_shapes():
    c = wl.CONFIGS
    assert [c[n].dtype for n in wl.CONFIG_ORDER] == ["f32", "bf16", "bf16", "bf16", "bf16"]
    assert c["llama3-8b-decode"].max_blocks_per_seq == 256
    assert c["llama3-70b-decode"].max_blocks_per_seq == 512
    assert c["long-split"].max_blocks_per_seq == 8192
    assert c["spec-verify"].group == 8 and c["spec-verify"].q_len == 5
    p = wl.make_problem("tiny-f32")
    assert p.context_lens.tolist() == [17, 40] and p.num_blocks == 16 and p.scale == np.float32(0.125)


def test_lognormal_lengths_have_the_stated_mean():
    spec = wl.CONFIGS["llama3-70b-decode"]
    rng = np.random.default_rng(0)
    lens = np.concatenate([wl.draw_lens(spec.with_(num_seqs=4096), rng) for _ in range(8)])
    assert lens.min() >= 16 and lens.max() <= 8192
    assert 900 < lens.mean() < 1100


def test_permute_physical_moves_rows_with_ids():
    p = wl.make_problem(SMALL)
    q = wl.permute_physical(p, 1)
    for b in range(p.num_seqs):
        nb = -(-int(p.context_lens[b]) // 16)
        np.testing.assert_array_equal(p.k_cache[p.block_tables[b, :nb]], q.k_cache[q.block_tables[b, :nb]])
    np.testing.assert_array_equal(p.k_cache.reshape(-1, 2, 16)[p.slot_mapping],
                                  q.k_cache.reshape(-1, 2, 16)[q.slot_mapping])
