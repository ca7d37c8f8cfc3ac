"""pa_decode_balanced_noalloc (the balanced decode on the library's fixed
scratch, for callers that cannot allocate) against pa_decode with
PA_BALANCED and a workspace of the caller's.

Both run the same kernels with the same schedule, so the outputs must agree
bit for bit: on the 8B layer's decode workload, then on a smaller batch of
another head shape (the scratch keeps the first call's contents, and the
arrival counters must have been left at zero), then on the first workload
again.  Sizes beyond the scratch are refused before anything is launched.
"""

import numpy as np
import pytest

import workloads as wl
from _gpu import DeviceProblem, parity, reference_rows, host_caches_after_write, sample_rows, to_host, widen

pytestmark = pytest.mark.gpu


def _both(p):
    import paged_kv_attention_decode_amd as pa

    d = DeviceProblem(p)
    want = to_host(d.step(-1).clone())  # cache write + balanced decode with a workspace
    got = pa.decode_balanced_noalloc(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, float(p.scale),
                                     p.q_len)
    return want, to_host(got)


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    big = wl.make_problem("llama3-8b-decode")
    small = wl.make_problem(wl.Spec(name="noalloc-small", dtype="bf16", num_seqs=37, num_q_heads=16, num_kv_heads=2,
                                    head_dim=64, lens=("uniform", 1, 700), max_len=768, seed=5))
    for i, p in enumerate((big, small, big)):
        want, got = _both(p)
        print(f"call {i}: {p.spec.name} S={p.num_seqs} d={p.head_dim} rows/KV head={p.spec.group * p.q_len}",
              flush=True)
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"call {i} differs from pa_decode"
        # and the oracle on sampled rows, as every decode is checked
        rows = sample_rows(p, 16, seed=i)
        kc, vc = host_caches_after_write(p)
        ref = reference_rows(p, rows, kc, vc)
        out = widen(got, p.dtype)
        r = parity(np.stack([out[b * p.q_len + j, h] for (b, j, h) in rows]), ref, p.dtype, rows=True)
        assert r["ok"], (i, r)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    import torch

    import paged_kv_attention_decode_amd as pa

    # 32 rows per KV head at head_dim 128 need 2048 pieces * 32 rows * 130 floats > 32 MiB
    p = wl.make_problem(wl.Spec(name="noalloc-big", dtype="bf16", num_seqs=4, num_q_heads=32, num_kv_heads=1,
                                head_dim=128, lens=("uniform", 1, 64), max_len=64, seed=6))
    assert pa.decode_workspace_size(4, 1, 32, 1, 128, p.max_blocks_per_seq, pa.PA_BALANCED) > 32 << 20
    d = DeviceProblem(p)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.decode_balanced_noalloc(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, float(p.scale), 1)
    assert e.value.status == 7 and "PA_ERR_SCRATCH" in str(e.value)
    torch.cuda.synchronize()
