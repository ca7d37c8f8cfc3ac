"""Pins of the chunked-prefill oracle (oracle/prefill.py).

Independent routes:
* torch's scaled_dot_product_attention in float64 on contiguous K/V per
  sequence, with the causal mask aligned to the end of the context
  (tril with diagonal L - n), sequences of different new-token counts in one
  call;
* chunking does not change the result: the rows of one prefill over a whole
  prompt equal, bit for bit, those of the same prompt fed in chunks, each
  chunk's call seeing the earlier chunks in the cache (the lab check named in
  "07 - Inference", lourdhu02.github.io, section 2.4);
* equal new-token counts reduce to the causal decode oracle, one new token
  to plain decode, and a mixed batch equals its sequences run one by one.
Each planted mistake (below) fails at least one of them.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import prefill as op
from _pins import build_paged, torch_widen
from workloads import round_to_bf16_bits

BS = 16


def varlen(seed, lens, counts, n_h=4, n_kv=2, d=16, dtype="bf16"):
    """Paged caches per build_paged, and a q of sum(counts) rows."""
    P = build_paged(seed, list(lens), n_h, n_kv, d, 1, dtype)
    rng = np.random.default_rng(seed + 1000)
    x = rng.standard_normal((int(sum(counts)), n_h, d)).astype(np.float32)
    P["q"] = round_to_bf16_bits(x) if dtype == "bf16" else x
    P["query_start"] = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return P


def run(P, scale):
    return oracle.paged_prefill(P["q"], P["k_cache"], P["v_cache"], P["block_tables"], P["context_lens"],
                                P["query_start"], scale, P["dtype"])


def sdpa_varlen(P, scale):
    qs = P["query_start"]
    n_h, n_kv = P["q"].shape[1], P["k_cache"].shape[2]
    G = n_h // n_kv
    q_all = torch_widen(P["q"], P["dtype"])
    outs = []
    for b, L in enumerate(P["context_lens"]):
        L, n = int(L), int(qs[b + 1] - qs[b])
        if n == 0:
            continue
        Q = q_all[qs[b]:qs[b + 1]].permute(1, 0, 2)[None]
        K = torch.from_numpy(P["Ks"][b]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        V = torch.from_numpy(P["Vs"][b]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=float(np.float32(scale)))
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


# ---------------------------------------------------------------------------
# the pins


def pin_sdpa_varlen(dtype="bf16"):
    P = varlen(0, lens=(40, 17, 64, 5, 33), counts=(40, 1, 23, 5, 0), dtype=dtype)
    return bool(np.max(np.abs(run(P, 0.3) - sdpa_varlen(P, 0.3))) <= 1e-12)


def pin_chunked_equals_single_prefill(prompt=100, chunk=32, dtype="bf16"):
    """One call over the whole prompt (n = L = prompt) against ceil(prompt / chunk) calls,
    call k holding tokens [k chunk, min((k + 1) chunk, prompt)) with L = the end of its chunk."""
    P = varlen(1, lens=(prompt,), counts=(prompt,), dtype=dtype)
    whole = run(P, 0.25)
    pieces = []
    for s in range(0, prompt, chunk):
        e = min(s + chunk, prompt)
        Pk = dict(P, q=P["q"][s:e], context_lens=np.array([e], np.int32),
                  query_start=np.array([0, e - s], np.int32))
        pieces.append(run(Pk, 0.25))
    return bool(np.array_equal(np.concatenate(pieces), whole))


def pin_equal_counts_is_causal_decode():
    P = varlen(2, lens=(9, 30, 47), counts=(5, 5, 5))
    dec = oracle.paged_decode(P["q"], P["k_cache"], P["v_cache"], P["block_tables"], P["context_lens"], 0.4, 5,
                              "bf16")
    one = varlen(3, lens=(9, 30, 47), counts=(1, 1, 1))
    dec1 = oracle.paged_decode(one["q"], one["k_cache"], one["v_cache"], one["block_tables"], one["context_lens"],
                               0.4, 1, "bf16")
    return bool(np.array_equal(run(P, 0.4), dec) and np.array_equal(run(one, 0.4), dec1))


def pin_mixed_batch_is_its_sequences():
    """A decode token, two chunks and an empty entry in one call equal the sequences run alone."""
    counts = (1, 12, 0, 20)
    P = varlen(4, lens=(50, 12, 7, 45), counts=counts)
    together = run(P, 0.35)
    qs = P["query_start"]
    alone = []
    for b, n in enumerate(counts):
        if n == 0:
            continue
        Pb = dict(P, q=P["q"][qs[b]:qs[b + 1]], block_tables=P["block_tables"][b:b + 1],
                  context_lens=P["context_lens"][b:b + 1], query_start=np.array([0, n], np.int32))
        alone.append(run(Pb, 0.35))
    return bool(np.array_equal(np.concatenate(alone), together))


def pin_rows_before_the_context_are_zero():
    """L < n: the first n - L new tokens would sit before position 0 and see nothing."""
    P = varlen(5, lens=(3,), counts=(6,), dtype="f32")
    out = run(P, 0.5)
    K, V = P["Ks"][0], P["Vs"][0]
    ok = bool(np.array_equal(out[:3], np.zeros_like(out[:3])))
    for i in range(3, 6):  # token i at position i - 3 sees positions 0 .. i - 3
        for h in range(4):
            s = 0.5 * (K[:i - 2, h // 2] @ oracle.to_f64(P["q"][i, h], "f32"))
            w = np.exp(s - s.max())
            ok &= bool(np.allclose(out[i, h], (w / w.sum()) @ V[:i - 2, h // 2], rtol=0, atol=1e-12))
    return ok


PINS = {
    "sdpa_varlen_bf16": pin_sdpa_varlen,
    "sdpa_varlen_f32": lambda: pin_sdpa_varlen("f32"),
    "chunked_equals_single": pin_chunked_equals_single_prefill,
    "chunked_equals_single_ragged": lambda: pin_chunked_equals_single_prefill(prompt=77, chunk=16, dtype="f32"),
    "equal_counts_is_causal_decode": pin_equal_counts_is_causal_decode,
    "mixed_batch": pin_mixed_batch_is_its_sequences,
    "rows_before_context": pin_rows_before_the_context_are_zero,
}


def failing_pins():
    """Pins that do not hold; a pin that raises (an index out of range) does not hold either."""
    bad = []
    for name, pin in PINS.items():
        try:
            ok = pin()
        except (IndexError, ValueError, AssertionError):
            ok = False
        if not ok:
            bad.append(name)
    return bad


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    assert PINS[name]()


# ---------------------------------------------------------------------------
# planted mistakes: every one must fail at least one pin

_true_visible = op.visible_count
_true_row = op.query_row

MUTATIONS = {
    "visible_off_by_one": ("visible_count", lambda L, n, i: _true_visible(L, n, i) - 1),
    "mask_top_left": ("visible_count", lambda L, n, i: i + 1),
    "no_causal_mask": ("visible_count", lambda L, n, i: L),
    "row_offset_ignored": ("query_row", lambda qs, b, i: i),
    "row_offset_of_next_sequence": ("query_row", lambda qs, b, i: int(qs[min(b + 1, len(qs) - 1)]) + i - 1),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(op, attr, fn)
    assert failing_pins(), f"no pin fails with {name} planted"
