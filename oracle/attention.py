"""Plain, slow, fp64 paged decode attention (test infrastructure only).

Conventions (the pages leave these open; the readings are listed with the
design notes of the repository):

* q and out are [num_seqs * q_len, num_q_heads, head_dim]; query token j of
  sequence b is row b * q_len + j.
* context_lens counts the q_len new tokens, so query token j sits at absolute
  position L - q_len + j and sees positions 0 .. L - q_len + j.
* query head h reads key/value head h // (num_q_heads // num_kv_heads).
* scale is the fp32 value the kernels receive, upcast exactly.
* bf16 inputs arrive as uint16 bit patterns and are widened exactly.

Every function is written for clarity, not speed: one query row at a time,
one matrix-vector product for the scores and one for the weighted sum.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 16


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64 (bf16 is the upper half of an fp32 bit pattern)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kv_head_of(h: int, group: int) -> int:
    """Grouped-query attention: consecutive groups of `group` query heads share a KV head.

    The pages say only that n_h / n_kv query heads share one key/value head
    (learn.mohebi.ai lesson 13, section 3 notation; "07 - Inference",
    lourdhu02.github.io, section 1); contiguous groups are the reading taken.
    """
    return h // group


def visible_tokens(context_len: int, q_len: int, j: int) -> int:
    """How many tokens query token j may attend to under the causal mask among the q_len newest.

    The target scores every draft position in one pass under a causal mask
    ("LLM serving: continuous batching & PagedAttention", systemcraft.online,
    section 8, item 1; "07 - Inference", lourdhu02.github.io, section 3).
    context_len counts the new tokens, which are written before attention.
    """
    return context_len - q_len + j + 1


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, context_len: int,
                    block_size: int = BLOCK_SIZE) -> np.ndarray:
    """The sequence's tokens in logical order, [context_len, n_kv, d], storage dtype.

    Logical token t lives in row t % block_size of physical block
    table_row[t // block_size]; table entries past the last used block are
    never looked at.  Logical block i holds tokens 16i .. 16i+15 and the
    kernel follows the block table one block at a time (learn.mohebi.ai
    lesson 13, section 3.5).
    """
    nblk = -(-context_len // block_size)
    blocks = [cache[int(table_row[i])] for i in range(nblk)]
    return np.concatenate(blocks, axis=0)[:context_len]


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """softmax over a 1-D score vector (max subtracted for range, normalized by the sum).

    The plain definition that the online softmax reproduces exactly
    ("07 - Inference", lourdhu02.github.io, section 5.1).
    """
    m = scores.max()
    w = np.exp(scores - m)
    return w / w.sum()


def attend_row(q_vec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query row: softmax(scale * K q) weighted sum of V.  K, V are [n, d] float64.

    Decode attention per query head: q^T K over the cached keys, then the
    weighted sum of the values (learn.mohebi.ai lesson 13, section 3.3, proof
    step 4).  The scale is an explicit argument; the pages do not print it.
    """
    s = scale * (K @ q_vec)
    p = softmax_weights(s)
    return p @ V


def _check(q, k_cache, v_cache, block_tables, context_lens, q_len):
    S = block_tables.shape[0]
    n_h, d = q.shape[1], q.shape[2]
    n_kv = k_cache.shape[2]
    assert q.shape[0] == S * q_len, "q must hold q_len rows per sequence"
    assert k_cache.shape == v_cache.shape and k_cache.shape[3] == d
    assert n_h % n_kv == 0, "query heads must be a multiple of KV heads"
    assert len(context_lens) == S
    return S, n_h, n_kv, d, n_h // n_kv


class _SeqCache:
    """Per-sequence gathered K/V, widened to fp64 one KV head at a time."""

    def __init__(self, k_cache, v_cache, block_tables, context_lens, dtype, block_size):
        self.k_cache, self.v_cache = k_cache, v_cache
        self.tables, self.lens = block_tables, context_lens
        self.dtype, self.bs = dtype, block_size
        self._b = None
        self._heads = {}

    def head(self, b: int, g: int):
        if self._b != b:
            L = int(self.lens[b])
            self._Kb = gather_sequence(self.k_cache, self.tables[b], L, self.bs)
            self._Vb = gather_sequence(self.v_cache, self.tables[b], L, self.bs)
            self._b, self._heads = b, {}
        if g not in self._heads:
            self._heads[g] = (to_f64(self._Kb[:, g, :], self.dtype), to_f64(self._Vb[:, g, :], self.dtype))
        return self._heads[g]


def paged_decode_rows(q, k_cache, v_cache, block_tables, context_lens, scale, q_len, dtype, rows,
                      block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Attention output for the listed (b, j, h) rows only, [len(rows), d] float64.

    Plain attention over the block-table-gathered keys and values: paging only
    changes where a token is stored (learn.mohebi.ai lesson 13, section 3.5),
    so each row is attend_row over its visible prefix.
    """
    S, n_h, n_kv, d, G = _check(q, k_cache, v_cache, block_tables, context_lens, q_len)
    scale64 = float(np.float32(scale))
    seqs = _SeqCache(k_cache, v_cache, block_tables, context_lens, dtype, block_size)
    out = np.empty((len(rows), d), dtype=np.float64)
    for i, (b, j, h) in enumerate(rows):
        L = int(context_lens[b])
        n = visible_tokens(L, q_len, j)
        K, V = seqs.head(b, kv_head_of(h, G))
        qv = to_f64(q[b * q_len + j, h], dtype)
        out[i] = attend_row(qv, K[:n], V[:n], scale64)
    return out


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale, q_len, dtype,
                 block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Full output [num_seqs * q_len, num_q_heads, head_dim] in float64 (every row of paged_decode_rows)."""
    S, n_h, n_kv, d, G = _check(q, k_cache, v_cache, block_tables, context_lens, q_len)
    rows = [(b, j, h) for b in range(S) for j in range(q_len) for h in range(n_h)]
    flat = paged_decode_rows(q, k_cache, v_cache, block_tables, context_lens, scale, q_len, dtype, rows,
                             block_size)
    return flat.reshape(S * q_len, n_h, d)


# ---------------------------------------------------------------------------
# split context (FlashDecoding): partials per partition, then the merge


def partition_partials(q_vec, K, V, scale: float, n_visible: int, context_len: int, partition_size: int):
    """Partials (m, l, acc) of one query row for partitions [p*ps, (p+1)*ps) of [0, context_len).

    FlashDecoding: chunks of the context each give a partial (m, l, acc)
    ("07 - Inference", lourdhu02.github.io, section 5.3).

    m is the partition's largest score, l the sum of exp(score - m), acc the
    exp(score - m)-weighted sum of its value rows.  Tokens past n_visible are
    masked; a partition with no visible token gives (-inf, 0, 0).
    """
    P = -(-context_len // partition_size)
    d = V.shape[1]
    ms = np.full(P, -np.inf)
    ls = np.zeros(P)
    accs = np.zeros((P, d))
    for p in range(P):
        lo = p * partition_size
        hi = min(lo + partition_size, n_visible)
        if hi <= lo:
            continue
        s = scale * (K[lo:hi] @ q_vec)
        m = s.max()
        w = np.exp(s - m)
        ms[p], ls[p], accs[p] = m, w.sum(), w @ V[lo:hi]
    return ms, ls, accs


def merge_partials(ms: np.ndarray, ls: np.ndarray, accs: np.ndarray) -> np.ndarray:
    """Combine partials with the online-softmax rescaling: every partition is
    rescaled to the global maximum M by exp(m_p - M), then sum(acc) / sum(l)
    ("07 - Inference", lourdhu02.github.io, sections 5.1 and 5.3: the merge
    uses the same rescaling rule and is exact)."""
    live = ls > 0
    M = ms[live].max()
    f = np.where(live, np.exp(np.where(live, ms, M) - M), 0.0)
    return (f[:, None] * accs).sum(axis=0) / (f * ls).sum()


def paged_decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, q_len, dtype,
                       partition_size: int, rows=None, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Same result as paged_decode, computed through per-partition partials and the merge
    ("07 - Inference", lourdhu02.github.io, section 5.3)."""
    S, n_h, n_kv, d, G = _check(q, k_cache, v_cache, block_tables, context_lens, q_len)
    scale64 = float(np.float32(scale))
    if rows is None:
        rows = [(b, j, h) for b in range(S) for j in range(q_len) for h in range(n_h)]
        shape = (S * q_len, n_h, d)
    else:
        shape = (len(rows), d)
    seqs = _SeqCache(k_cache, v_cache, block_tables, context_lens, dtype, block_size)
    out = np.empty((len(rows), d))
    for i, (b, j, h) in enumerate(rows):
        L = int(context_lens[b])
        K, V = seqs.head(b, kv_head_of(h, G))
        qv = to_f64(q[b * q_len + j, h], dtype)
        ms, ls, accs = partition_partials(qv, K, V, scale64, visible_tokens(L, q_len, j), L, partition_size)
        out[i] = merge_partials(ms, ls, accs)
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# slot-mapped write of new tokens


def cache_write(k_cache, v_cache, k, v, slot_mapping, block_size: int = BLOCK_SIZE):
    """Copies of the caches with token t's K/V rows stored at flat slot slot_mapping[t].

    A slot is physical_block * block_size + row; a negative slot means the
    token is not stored.  The rows are copied as raw bits.  New tokens are
    appended in place into the sequence's current block ("LLM Inference
    Serving", systeminternals.dev, the passage on the block manager), and
    logical block i covers tokens 16i .. 16i+15 (learn.mohebi.ai lesson 13,
    section 3.5).
    """
    NB = k_cache.shape[0]
    kc = k_cache.copy()
    vc = v_cache.copy()
    unit = np.uint16 if kc.dtype == np.uint16 else np.uint32
    kf = kc.view(unit).reshape(NB * block_size, *kc.shape[2:])
    vf = vc.view(unit).reshape(NB * block_size, *vc.shape[2:])
    kin = np.ascontiguousarray(k).view(unit)
    vin = np.ascontiguousarray(v).view(unit)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        if slot >= NB * block_size:
            raise IndexError(f"slot {slot} outside a pool of {NB} blocks")
        kf[slot] = kin[t]
        vf[slot] = vin[t]
    return kc, vc


def block_count(context_len: int, block_size: int = BLOCK_SIZE) -> int:
    """Blocks a context of context_len tokens occupies (learn.mohebi.ai lesson 13, section 3.5)."""
    return int(math.ceil(context_len / block_size))
