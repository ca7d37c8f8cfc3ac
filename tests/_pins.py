"""Pins for the oracle: checks against things other than the oracle itself.

Each pin returns True when the oracle agrees with an independent route:
torch's scaled_dot_product_attention on contiguous K/V built token by token
from the block-table definition, closed forms, or exact invariants.  The same
pins are re-run with mistakes planted in the oracle (tests/test_oracle.py)
to show that each plausible mistake fails at least one of them.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import attention as oa
from workloads import bf16_bits_to_f32, round_to_bf16_bits

BS = 16


def build_paged(seed, lens, n_h, n_kv, d, q_len, dtype, extra_blocks=3):
    """Draw contiguous per-sequence K/V, then place token t of sequence b in row
    t % 16 of physical block table[b][t // 16] (the block-table definition).

    Returns the paged arrays plus the contiguous float64 K/V and q used by SDPA.
    """
    rng = np.random.default_rng(seed)
    S = len(lens)
    nblk = [-(-L // BS) for L in lens]
    NB = sum(nblk) + extra_blocks
    MB = max(nblk) + 1
    perm = rng.permutation(NB)
    tables = rng.integers(0, NB, size=(S, MB)).astype(np.int32)  # padding: valid but wrong ids
    cur = 0
    for b in range(S):
        tables[b, :nblk[b]] = perm[cur:cur + nblk[b]]
        cur += nblk[b]

    def draw(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        if dtype == "bf16":
            bits = round_to_bf16_bits(x)
            return bits, bf16_bits_to_f32(bits).astype(np.float64)
        return x, x.astype(np.float64)

    store_dt = np.uint16 if dtype == "bf16" else np.float32
    k_cache = np.zeros((NB, BS, n_kv, d), dtype=store_dt)
    v_cache = np.zeros((NB, BS, n_kv, d), dtype=store_dt)
    fill_k, _ = draw((NB, BS, n_kv, d))
    fill_v, _ = draw((NB, BS, n_kv, d))
    k_cache[:] = fill_k
    v_cache[:] = fill_v
    Ks, Vs = [], []
    for b, L in enumerate(lens):
        kb, kb64 = draw((L, n_kv, d))
        vb, vb64 = draw((L, n_kv, d))
        for t in range(L):
            blk = tables[b, t // BS]
            k_cache[blk, t % BS] = kb[t]
            v_cache[blk, t % BS] = vb[t]
        Ks.append(kb64)
        Vs.append(vb64)
    q, q64 = draw((S * q_len, n_h, d))
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables,
                context_lens=np.asarray(lens, dtype=np.int32), q_len=q_len, dtype=dtype,
                q64=q64, Ks=Ks, Vs=Vs)


def torch_widen(a, dtype):
    """Independent widening through torch's own bf16 type."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)


def sdpa_reference(P, scale):
    """Dense attention per sequence with torch SDPA in float64, GQA by repeat_interleave,
    and a causal mask aligned to the end of the context (the new tokens are the last q_len)."""
    q_len = P["q_len"]
    S = len(P["context_lens"])
    n_h = P["q"].shape[1]
    n_kv = P["k_cache"].shape[2]
    G = n_h // n_kv
    outs = []
    q_all = torch_widen(P["q"], P["dtype"])
    for b in range(S):
        L = int(P["context_lens"][b])
        Q = q_all[b * q_len:(b + 1) * q_len].permute(1, 0, 2)[None]  # [1, n_h, q_len, d]
        K = torch.from_numpy(P["Ks"][b]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        V = torch.from_numpy(P["Vs"][b]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        mask = torch.ones(q_len, L, dtype=torch.bool).tril(diagonal=L - q_len)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=float(np.float32(scale)))
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


def run_oracle(P, scale):
    return oracle.paged_decode(P["q"], P["k_cache"], P["v_cache"], P["block_tables"], P["context_lens"],
                               scale, P["q_len"], P["dtype"])


# ---------------------------------------------------------------------------
# the pins


def pin_sdpa(seed=0, lens=(1, 16, 17, 40), n_h=4, n_kv=2, d=16, q_len=1, dtype="f32", scale=0.37, tol=1e-12):
    P = build_paged(seed, list(lens), n_h, n_kv, d, q_len, dtype)
    ref = sdpa_reference(P, scale)
    got = run_oracle(P, scale)
    return bool(np.max(np.abs(got - ref)) <= tol)


def pin_permutation(seed=1, dtype="bf16", q_len=1):
    from workloads import make_problem, permute_physical, Spec

    spec = Spec(name="perm", dtype=dtype, num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                lens=("fixed", (5, 33, 48)), max_len=64, q_len=q_len, seed=seed)
    p = make_problem(spec)
    p2 = permute_physical(p, seed + 100)
    a = oracle.paged_decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, p.q_len, dtype)
    b = oracle.paged_decode(p2.q, p2.k_cache, p2.v_cache, p2.block_tables, p2.context_lens, p2.scale, p2.q_len, dtype)
    return bool(np.array_equal(a, b))


def pin_one_token(dtype="f32"):
    P = build_paged(2, [1, 1], 4, 2, 16, 1, dtype)
    got = run_oracle(P, 0.25)
    ok = True
    for b in range(2):
        for h in range(4):
            ok &= bool(np.array_equal(got[b, h], P["Vs"][b][0, h // 2]))
    return ok


def count_probe(lens, n_h, n_kv, d, q_len, dtype="bf16"):
    """Identical keys, V[t, g, c] = 1 if c == t mod d else 0: the output is an exact token count."""
    P = build_paged(3, list(lens), n_h, n_kv, d, q_len, dtype)
    one = np.uint16(0x3F80) if dtype == "bf16" else np.float32(1.0)
    zero = np.zeros((), dtype=P["k_cache"].dtype)
    NB = P["k_cache"].shape[0]
    P["k_cache"][:] = P["k_cache"][0, 0, 0, 0]  # every key row identical
    P["v_cache"][:] = zero
    for b, L in enumerate(lens):
        for t in range(L):
            blk = P["block_tables"][b, t // BS]
            P["v_cache"][blk, t % BS, :, t % d] = one
    del NB
    got = run_oracle(P, 0.1)
    expect = np.zeros_like(got)
    for b, L in enumerate(lens):
        for j in range(q_len):
            p = L - q_len + j
            counts = np.array([len(range(c, p + 1, d)) for c in range(d)], dtype=np.float64)
            expect[b * q_len + j] = counts / (p + 1)
    return got, expect


def pin_count_probe(q_len=5):
    got, expect = count_probe([5, 16, 37, 70], 4, 2, 16, q_len)
    return bool(np.max(np.abs(got - expect)) <= 1e-12)


def pin_two_token_closed_form():
    """L = 2 with keys along one axis: out = v0 + sigmoid(s1 - s0) (v1 - v0)."""
    d = 8
    P = build_paged(4, [2], 1, 1, d, 1, "f32")
    P["q"][:] = 0
    P["q"][0, 0, 0] = 2.0
    P["Ks"][0][:] = 0
    for t, x in enumerate((0.5, -1.25)):
        P["Ks"][0][t, 0, 0] = x
        P["k_cache"][P["block_tables"][0, 0], t, 0, :] = 0
        P["k_cache"][P["block_tables"][0, 0], t, 0, 0] = x
    scale = 0.75
    s0, s1 = scale * 2.0 * 0.5, scale * 2.0 * -1.25
    sig = 1.0 / (1.0 + np.exp(-(s1 - s0)))
    v0, v1 = P["Vs"][0][0, 0], P["Vs"][0][1, 0]
    expect = v0 + sig * (v1 - v0)
    got = run_oracle(P, scale)[0, 0]
    return bool(np.max(np.abs(got - expect)) <= 1e-14)


def pin_split(q_len=5, partition_size=32):
    P = build_paged(5, [5, 31, 32, 33, 97], 4, 2, 16, q_len, "bf16")
    full = run_oracle(P, 0.3)
    split = oracle.paged_decode_split(P["q"], P["k_cache"], P["v_cache"], P["block_tables"], P["context_lens"],
                                      0.3, P["q_len"], "bf16", partition_size)
    return bool(np.max(np.abs(full - split)) <= 1e-12)


def pin_cache_write():
    rng = np.random.default_rng(6)
    NB, n_kv, d = 9, 2, 8
    kc = rng.integers(0, 1 << 16, size=(NB, BS, n_kv, d), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(NB, BS, n_kv, d), dtype=np.uint16)
    T = 7
    k = rng.integers(0, 1 << 16, size=(T, n_kv, d), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(T, n_kv, d), dtype=np.uint16)
    blocks = rng.permutation(NB)[:T]
    rows = rng.integers(0, BS, size=T)
    slots = (blocks * BS + rows).astype(np.int64)
    slots[3] = -1
    kc2, vc2 = oracle.cache_write(kc, vc, k, v, slots)
    ok = True
    touched = np.zeros((NB, BS), dtype=bool)
    for t in range(T):
        if t == 3:
            continue
        ok &= bool(np.array_equal(kc2[blocks[t], rows[t]], k[t])) and bool(np.array_equal(vc2[blocks[t], rows[t]], v[t]))
        touched[blocks[t], rows[t]] = True
    ok &= bool(np.array_equal(kc2[~touched], kc[~touched])) and bool(np.array_equal(vc2[~touched], vc[~touched]))
    return ok


FAST_PINS = {
    "sdpa_f32_q1": lambda: pin_sdpa(dtype="f32", q_len=1),
    "sdpa_bf16_q5": lambda: pin_sdpa(seed=7, lens=(5, 16, 33), n_h=8, n_kv=2, dtype="bf16", q_len=5),
    "permutation": pin_permutation,
    "one_token": pin_one_token,
    "count_probe": pin_count_probe,
    "two_token": pin_two_token_closed_form,
    "split": pin_split,
    "cache_write": pin_cache_write,
}


def failing_pins():
    bad = []
    for name, fn in FAST_PINS.items():
        try:
            if not fn():
                bad.append(name)
        except Exception:  # a crash is a failed pin as well
            bad.append(name)
    return bad


__all__ = ["build_paged", "sdpa_reference", "run_oracle", "FAST_PINS", "failing_pins", "count_probe", "oa"]
