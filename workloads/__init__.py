"""Seeded synthetic inputs for paged KV-cache decode attention.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It draws random numbers, rounds them to the storage type,
assigns physical blocks and builds slot mappings.  It contains none of the
attention arithmetic: no scores, no softmax, no gathers through the block
table, no scatter of new tokens.

The workload shapes follow the pages' description of a paged KV cache
("LLM Inference Serving", systeminternals.dev: per layer K and V are each
stored as [num_blocks, block_size, num_kv_heads, head_dim]; the block size is
16 tokens) and of the block table ("LLM serving: KV cache, batching, paged
attention and quantization", learn.mohebi.ai, section 3.5: logical block i
holds tokens 16i..16i+15 and maps to any physical block).

Every array is reproducible from (spec, seed) alone.  Large arrays are drawn in
fixed-size chunks whose seeds derive from (seed, stream, chunk index), so the
values do not depend on how many threads fill them.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
BF16_QNAN_BITS = np.uint16(0x7FC0)
F32_QNAN = np.float32("nan")

# stream ids for the derived seeds of the large arrays
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_NEWK, _STREAM_NEWV = 1, 2, 3, 4, 5
_CHUNK = 1 << 22  # values per independently seeded chunk


# ----------------------------------------------------------------------------
# storage-type helpers (input preparation, not part of the method)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns by round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_normal(shape, dtype: str, seed: int, stream: int) -> np.ndarray:
    """N(0,1) draws in fp32, stored as fp32 ("f32") or bf16 bits ("bf16")."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def work(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        if hi <= lo:
            return
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        tmp = np.empty(hi - lo, dtype=np.float32)
        g.standard_normal(out=tmp, dtype=np.float32)
        if dtype == "f32":
            out[lo:hi] = tmp
        else:
            out[lo:hi] = round_to_bf16_bits(tmp)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# specs


@dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic paged-decode workload.

    lens: ("fixed", (l0, l1, ...)) | ("uniform", lo, hi) | ("lognormal", mu, sigma, lo, hi)
    num_blocks: physical pool size; None -> shared + ceil(1.25 * sum of private blocks)
    max_len: the largest context the block table must hold (sets max_blocks_per_seq)
    """

    name: str
    dtype: str  # "f32" | "bf16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lens: tuple
    max_len: int
    q_len: int = 1
    num_blocks: Optional[int] = None
    shared_prefix_blocks: int = 0
    write_new_tokens: bool = False
    partition_size: int = 0
    seed: int = 0
    scale: Optional[float] = None  # None -> fp32(1/sqrt(head_dim))
    pad: str = "valid"  # block-table padding: "valid" random in-range ids | "garbage"
    poison: bool = False  # NaN in cache rows never read (unused blocks, rows >= L)
    kv: str = "same"  # cache element type: "same" as dtype | "fp8" (E4M3 codes with per-head scales; dtype bf16)
    tree: str = ""  # q_len > 1: "" causal chain | "binary" complete binary tree (heap numbering) | "random"
    # prefill: new tokens per sequence, () -> q_len each | ("fixed", (n_0, ...)) | ("chunk", C) -> min(C, L_b)
    new_tokens: tuple = ()
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return (self.max_len + BLOCK_SIZE - 1) // BLOCK_SIZE

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


CONFIGS = {
    "tiny-f32": Spec(
        name="tiny-f32", dtype="f32", num_seqs=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
        lens=("fixed", (17, 40)), max_len=48, num_blocks=16, seed=0,
        description="2 sequences (17, 40 tokens), 4 q heads / 2 kv heads, d=64, fp32, 16-block pool",
    ),
    "llama3-8b-decode": Spec(
        name="llama3-8b-decode", dtype="bf16", num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        lens=("uniform", 512, 4096), max_len=4096, num_blocks=20000, write_new_tokens=True, seed=1,
        description="Llama-3-8B-shaped layer: 32/8 heads, d=128, bf16, batch 64, L~U[512,4096], 20k-block pool, 64 new tokens written",
    ),
    "llama3-70b-decode": Spec(
        name="llama3-70b-decode", dtype="bf16", num_seqs=256, num_q_heads=64, num_kv_heads=8, head_dim=128,
        lens=("lognormal", math.log(1024.0) - 0.5, 1.0, 16, 8192), max_len=8192, seed=2,
        description="Llama-3-70B-shaped layer: 64/8 heads, d=128, bf16, batch 256, L lognormal mean 1024 clipped to [16,8192]",
    ),
    "long-split": Spec(
        name="long-split", dtype="bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
        lens=("uniform", 32768, 131072), max_len=131072, partition_size=512, seed=3,
        description="long contexts: 32/8 heads, d=128, bf16, batch 8, L~U[32768,131072], 512-token partitions + reduce",
    ),
    "spec-verify": Spec(
        name="spec-verify", dtype="bf16", num_seqs=128, num_q_heads=64, num_kv_heads=8, head_dim=128,
        lens=("uniform", 1024, 4096), max_len=4096, q_len=5, shared_prefix_blocks=32, write_new_tokens=True, seed=4,
        description="speculative verify: 4 drafts + 1 = 5 query tokens, causal among them, 64/8 heads, d=128, bf16, batch 128, L~U[1024,4096], 32 shared prefix blocks, 640 new tokens written",
    ),
}

CONFIG_ORDER = ["tiny-f32", "llama3-8b-decode", "llama3-70b-decode", "long-split", "spec-verify"]

# Beyond the five workloads: tree verify on the Llama-3-8B-shaped layer (Medusa's
# 15-node complete binary tree, branching 2 over 4 levels, under a tree mask)
CONFIGS["tree-verify"] = Spec(
    name="tree-verify", dtype="bf16", num_seqs=128, num_q_heads=32, num_kv_heads=8, head_dim=128,
    lens=("uniform", 1024, 4096), max_len=4096, q_len=15, tree="binary", shared_prefix_blocks=32,
    write_new_tokens=True, seed=5,
    description="tree verify: a 15-node complete binary tree of candidates per sequence under a tree mask, 32/8 "
                "heads, d=128, bf16, batch 128, L~U[1024,4096], 32 shared prefix blocks, 1920 new tokens written")

# chunked prefill on the Llama-3-8B-shaped layer: a 2,048-token step budget of four
# 512-token prompt chunks, each at a different depth of its prompt
CONFIGS["chunked-prefill"] = Spec(
    name="chunked-prefill", dtype="bf16", num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
    lens=("chunks", 512, 16), max_len=8192, new_tokens=("chunk", 512), write_new_tokens=True, seed=6,
    description="chunked prefill: 4 prompt chunks of 512 tokens (a 2,048-token step), chunk k of its prompt "
                "(k ~ U{0..15}) over a cache of 512 k earlier tokens, causal within the chunk, 32/8 heads, d=128, "
                "bf16, the chunks' K/V written first")

# the Llama-3-8B-shaped layer over an fp8 (E4M3) cache
CONFIGS["llama3-8b-decode-fp8kv"] = CONFIGS["llama3-8b-decode"].with_(
    name="llama3-8b-decode-fp8kv", kv="fp8",
    description="the llama3-8b-decode layer with an fp8 (E4M3) KV cache, per-head scales, 64 new tokens quantized "
                "by pa_cache_write_fp8")


# ----------------------------------------------------------------------------
# problems


@dataclass
class Problem:
    spec: Spec
    context_lens: np.ndarray  # int32 [S]; counts the q_len newest tokens
    block_tables: np.ndarray  # int32 [S, max_blocks_per_seq]
    q: np.ndarray  # [S*q_len, n_h, d]  float32 or uint16 (bf16 bits)
    k_cache: np.ndarray  # [NB, 16, n_kv, d]  (before new tokens are written)
    v_cache: np.ndarray
    scale: np.float32
    new_k: Optional[np.ndarray] = None  # [T, n_kv, d]
    new_v: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # int64 [T]
    k_scale: Optional[np.ndarray] = None  # fp8 caches: float32 [n_kv]
    v_scale: Optional[np.ndarray] = None
    parents: Optional[np.ndarray] = None  # tree verify: int32 [S, q_len], parents[b, j] in [-1, j)
    query_start: Optional[np.ndarray] = None  # prefill: int32 [S + 1], sequence b owns q rows qs[b] .. qs[b+1]-1
    extra: dict = field(default_factory=dict)

    # convenience views of the spec
    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def num_seqs(self) -> int:
        return self.spec.num_seqs

    @property
    def q_len(self) -> int:
        return self.spec.q_len

    @property
    def num_q_heads(self) -> int:
        return self.spec.num_q_heads

    @property
    def num_kv_heads(self) -> int:
        return self.spec.num_kv_heads

    @property
    def head_dim(self) -> int:
        return self.spec.head_dim

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def partition_size(self) -> int:
        return self.spec.partition_size

    @property
    def q_counts(self) -> np.ndarray:
        """New tokens (query rows per head) of each sequence."""
        if self.query_start is not None:
            return (self.query_start[1:] - self.query_start[:-1]).astype(np.int64)
        return np.full(self.num_seqs, self.q_len, dtype=np.int64)

    def as_float32(self, a: np.ndarray) -> np.ndarray:
        return a if self.dtype == "f32" else bf16_bits_to_f32(a)


def draw_lens(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lens[0]
    S = spec.num_seqs
    if kind == "fixed":
        vals = np.asarray(spec.lens[1], dtype=np.int64)
        assert vals.size == S, "fixed lens must list one length per sequence"
        lens = vals
    elif kind == "uniform":
        lo, hi = spec.lens[1], spec.lens[2]
        lens = rng.integers(lo, hi, size=S, endpoint=True)
    elif kind == "chunks":
        chunk, max_chunks = spec.lens[1], spec.lens[2]
        lens = chunk * (rng.integers(0, max_chunks, size=S) + 1)
    elif kind == "lognormal":
        mu, sigma, lo, hi = spec.lens[1:5]
        lens = np.clip(np.rint(rng.lognormal(mu, sigma, size=S)), lo, hi).astype(np.int64)
    else:
        raise ValueError(f"unknown length distribution {kind!r}")
    assert lens.min() >= 1 and lens.max() <= spec.max_len
    return lens.astype(np.int32)


FP8_NAN_CODE = np.uint8(0x7F)


def fp8_scales(n_kv: int, which: str) -> np.ndarray:
    """Per-head scales of a synthetic fp8 cache: 1/64 to 1.25/64 (K) and 1/48 to 1.25/48 (V)
    across the heads, so that N(0,1) data spans most of the +-448 code range and every head
    has its own scale."""
    base = 1.0 / 64 if which == "k" else 1.0 / 48
    return (base * (1.0 + 0.25 * np.arange(n_kv) / max(1, n_kv - 1))).astype(np.float32)


def to_fp8_codes(bits_bf16: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E4M3 codes of bf16 data divided by the per-head scale (last-but-one axis is the
    head), through torch's float8_e4m3fn cast after clamping to +-448: a library
    conversion that prepares synthetic cache contents (the oracle and the kernels
    each quantize new tokens with their own code)."""
    import torch

    x = torch.from_numpy(np.ascontiguousarray(bits_bf16).view(np.int16)).view(torch.bfloat16).to(torch.float32)
    s = torch.from_numpy(scale.astype(np.float32))[:, None]
    return (x / s).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def tree_parents(spec: Spec) -> Optional[np.ndarray]:
    """Parent arrays [S, q_len] of a tree-verify workload (None for the causal chain).

    "binary": node j's parent is (j - 1) // 2, the root -1 (heap numbering);
    "random": node j >= 1 hangs on a uniformly drawn earlier node, node 0 and,
    with probability 1/8, any later node on the context (a forest)."""
    if not spec.tree:
        return None
    S, T = spec.num_seqs, spec.q_len
    if spec.tree == "binary":
        row = np.array([-1] + [(j - 1) // 2 for j in range(1, T)], dtype=np.int32)
        return np.tile(row, (S, 1))
    if spec.tree == "random":
        rng = np.random.default_rng((spec.seed, 7001))
        par = np.full((S, T), -1, dtype=np.int32)
        for j in range(1, T):
            par[:, j] = rng.integers(0, j, size=S)
            par[rng.random(S) < 0.125, j] = -1
        return par
    raise ValueError(f"unknown tree {spec.tree!r}")


def new_token_counts(spec: Spec, lens: np.ndarray) -> np.ndarray:
    """New tokens of each sequence: q_len each, or the prefill spec's counts."""
    S = spec.num_seqs
    if not spec.new_tokens:
        return np.full(S, spec.q_len, dtype=np.int64)
    kind = spec.new_tokens[0]
    if kind == "fixed":
        counts = np.asarray(spec.new_tokens[1], dtype=np.int64)
        assert counts.size == S, "fixed new_tokens must list one count per sequence"
        return counts
    if kind == "chunk":
        return np.minimum(np.int64(spec.new_tokens[1]), lens.astype(np.int64))
    raise ValueError(f"unknown new_tokens {kind!r}")


def make_problem(spec: Spec) -> Problem:
    """Draw every input of one workload from spec.seed."""
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if spec.kv == "fp8":
        assert spec.dtype == "bf16", "fp8 caches go with bf16 queries"
        p = make_problem(spec.with_(kv="same", poison=False))
        p.spec = spec
        p.k_scale = fp8_scales(spec.num_kv_heads, "k")
        p.v_scale = fp8_scales(spec.num_kv_heads, "v")
        p.k_cache = to_fp8_codes(p.k_cache, p.k_scale)
        p.v_cache = to_fp8_codes(p.v_cache, p.v_scale)
        if spec.poison:
            poison_unread(spec, p.context_lens, p.block_tables, p.k_cache, p.v_cache)
        return p
    rng = np.random.default_rng(spec.seed)
    S, bs = spec.num_seqs, BLOCK_SIZE
    lens = draw_lens(spec, rng)
    counts = new_token_counts(spec, lens)
    assert (lens >= counts).all(), "every context must hold its newest tokens"
    nblk = (lens.astype(np.int64) + bs - 1) // bs
    shared = spec.shared_prefix_blocks
    if shared:
        assert (lens.astype(np.int64) - counts).min() >= shared * bs, "new tokens must land past the shared prefix"
    private = nblk - shared
    if spec.num_blocks is None:
        NB = shared + int(math.ceil(1.25 * float(private.sum())))
    else:
        NB = spec.num_blocks
    assert NB >= shared + int(private.sum()), "pool too small for the assigned blocks"

    # block assignment: a seeded permutation of the pool, handed out in sequence order
    perm = rng.permutation(NB).astype(np.int32)
    MB = spec.max_blocks_per_seq
    tables = np.empty((S, MB), dtype=np.int32)
    if spec.pad == "valid":
        tables[:] = rng.integers(0, NB, size=(S, MB), dtype=np.int32)
    elif spec.pad == "garbage":
        tables[:] = np.int32(0x7FFFFFF0)
    else:
        raise ValueError(spec.pad)
    cursor = shared
    for b in range(S):
        tables[b, :shared] = perm[:shared]
        n = int(private[b])
        tables[b, shared:shared + n] = perm[cursor:cursor + n]
        cursor += n

    n_kv, d = spec.num_kv_heads, spec.head_dim
    starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    q = fill_normal((int(starts[-1]), spec.num_q_heads, d), spec.dtype, spec.seed, _STREAM_Q)
    k_cache = fill_normal((NB, bs, n_kv, d), spec.dtype, spec.seed, _STREAM_K)
    v_cache = fill_normal((NB, bs, n_kv, d), spec.dtype, spec.seed, _STREAM_V)

    new_k = new_v = slots = None
    if spec.write_new_tokens:
        T = int(starts[-1])
        new_k = fill_normal((T, n_kv, d), spec.dtype, spec.seed, _STREAM_NEWK)
        new_v = fill_normal((T, n_kv, d), spec.dtype, spec.seed, _STREAM_NEWV)
        slots = np.empty(T, dtype=np.int64)
        for b in range(S):
            for j in range(int(counts[b])):
                pos = int(lens[b]) - int(counts[b]) + j
                slots[starts[b] + j] = int(tables[b, pos // bs]) * bs + pos % bs

    if spec.poison:
        poison_unread(spec, lens, tables, k_cache, v_cache)

    scale = np.float32(1.0 / math.sqrt(d)) if spec.scale is None else np.float32(spec.scale)
    return Problem(spec=spec, context_lens=lens, block_tables=tables, q=q, k_cache=k_cache, v_cache=v_cache,
                   scale=scale, new_k=new_k, new_v=new_v, slot_mapping=slots, parents=tree_parents(spec),
                   query_start=starts.astype(np.int32) if spec.new_tokens else None)


def poison_unread(spec: Spec, lens, tables, k_cache, v_cache) -> None:
    """Write NaN into every cache row that a correct kernel never reads."""
    bs = BLOCK_SIZE
    nan = FP8_NAN_CODE if spec.kv == "fp8" else (BF16_QNAN_BITS if spec.dtype == "bf16" else F32_QNAN)
    used = np.zeros(k_cache.shape[0], dtype=bool)
    for b in range(len(lens)):
        nb = (int(lens[b]) + bs - 1) // bs
        used[tables[b, :nb]] = True
    k_cache[~used] = nan
    v_cache[~used] = nan
    for b in range(len(lens)):
        L = int(lens[b])
        nb = (L + bs - 1) // bs
        tail = L - (nb - 1) * bs
        if tail < bs:
            last = tables[b, nb - 1]
            k_cache[last, tail:] = nan
            v_cache[last, tail:] = nan


def permute_physical(problem: Problem, seed: int) -> Problem:
    """The same logical problem with every physical block moved to a new id.

    Pool contents move with their ids, and block tables and slots are rewritten,
    so every sequence still sees the same tokens in the same logical order.
    """
    NB = problem.num_blocks
    rng = np.random.default_rng(seed)
    new_id = rng.permutation(NB).astype(np.int64)  # old id -> new id
    k = np.empty_like(problem.k_cache)
    v = np.empty_like(problem.v_cache)
    k[new_id] = problem.k_cache
    v[new_id] = problem.v_cache
    tables = problem.block_tables.astype(np.int64)
    in_range = (tables >= 0) & (tables < NB)
    tables = np.where(in_range, new_id[np.clip(tables, 0, NB - 1)], tables).astype(np.int32)
    slots = None
    if problem.slot_mapping is not None:
        s = problem.slot_mapping
        slots = new_id[s // BLOCK_SIZE] * BLOCK_SIZE + s % BLOCK_SIZE
    return replace(problem, k_cache=k, v_cache=v, block_tables=tables, slot_mapping=slots)


def algorithmic_bytes(problem: Problem) -> dict:
    """KV and Q bytes one decode call must read: each KV row once per (sequence, kv head).

    'unique' counts physical rows once when sequences share prefix blocks.
    """
    esz = 4 if problem.dtype == "f32" else 2
    kv_esz = 1 if problem.spec.kv == "fp8" else esz
    row = problem.num_kv_heads * problem.head_dim * kv_esz  # one token's K (or V) over all kv heads
    logical_tokens = int(problem.context_lens.astype(np.int64).sum())
    shared_tokens = problem.spec.shared_prefix_blocks * BLOCK_SIZE
    unique_tokens = logical_tokens - max(0, problem.num_seqs - 1) * shared_tokens if shared_tokens else logical_tokens
    n_q = int(problem.q_counts.sum())
    q_bytes = n_q * problem.num_q_heads * problem.head_dim * esz
    return {
        "kv_logical": 2 * logical_tokens * row,
        "kv_unique": 2 * unique_tokens * row,
        "q": q_bytes,
        "out": q_bytes,
        "tokens": n_q,
    }


def attention_flops(problem: Problem) -> int:
    """Multiply-adds x 2 of the visible (query row, position) pairs: q.k and p.v, 2 d flops each.

    New token i of sequence b sees L_b - n_b + i + 1 positions (at least 0)."""
    total = 0
    for L, n in zip(problem.context_lens.astype(np.int64), problem.q_counts):
        i = np.arange(int(n), dtype=np.int64)
        total += int(np.maximum(int(L) - int(n) + i + 1, 0).sum())
    return total * problem.num_q_heads * 4 * problem.head_dim


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_value: int) -> int:
    """K and V bytes per token: 2 * layers * kv_heads * head_dim * bytes (the pages' KV sizing)."""
    return 2 * layers * kv_heads * head_dim * bytes_per_value


def kv_bytes_per_block(block_tokens: int, layers: int, kv_heads: int, head_dim: int, bytes_per_value: int) -> int:
    return block_tokens * kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_value)
