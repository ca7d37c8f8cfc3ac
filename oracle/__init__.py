"""CPU fp64 oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

What it computes, and which passage each step follows:

* Paging is an indirection only.  A sequence's block table maps logical block
  i (tokens 16i..16i+15) to a physical block id; the attention reads keys and
  values one block at a time through it ("LLM serving: KV cache, batching,
  paged attention and quantization", learn.mohebi.ai, section 3.5).  Per layer
  K and V are each stored as [num_blocks, block_size, num_kv_heads, head_dim]
  ("LLM Inference Serving", systeminternals.dev, the passage on the per-layer
  cache shape).
* Decode attention: every query head computes q^T K over its sequence's keys
  and a softmax-weighted sum of the values (learn.mohebi.ai, section 3.3,
  proof step 4); with grouped-query attention n_h/n_kv query heads share one
  key/value head (learn.mohebi.ai, section 3, notation).
* Verify: the target scores all K+1 positions of prefix + drafts in one pass
  under a causal mask ("07 - Inference", lourdhu02.github.io, section 3, the
  verify step; systemcraft.online, section 8.1).
* The online softmax and the FlashDecoding split/merge are exact, so the
  plain softmax is the reference; the split path (partials (m, l, acc) merged
  by the online-softmax rescaling rule) is written out as well
  (lourdhu02.github.io "07 - Inference", sections 5.1 and 5.3).

* fp8 KV cache (oracle/fp8.py): keys and values stored as E4M3 codes with a
  per-head scale, products in higher precision ("LLM serving: KV cache,
  batching, paged attention and quantization", learn.mohebi.ai, section 3.7;
  "07 - Inference", lourdhu02.github.io, section 4.3).

* Block copies for copy-on-write and swapping (oracle/blocks.py): whole
  blocks as raw bytes (learn.mohebi.ai, section 3.5; arunshar.com, section
  18.2.2).

* Tree-mask verify (oracle/tree.py): the candidates of a draft tree are
  scored in one pass, each node seeing the context and its own path to the
  root ("Chapter 18: Speculative Decoding and Serving Optimizations",
  arunshar.com, section 18.1.2; "07 - Inference", lourdhu02.github.io,
  section 3.4).

* Chunked prefill (oracle/prefill.py): sequences with different numbers of
  new tokens in one call, each new token seeing the cached prefix and the
  earlier new tokens ("Chapter 18: Speculative Decoding and Serving
  Optimizations", arunshar.com, section 18.2.1; "LLM serving: KV cache,
  batching, paged attention and quantization", learn.mohebi.ai, section 3.6;
  "07 - Inference", lourdhu02.github.io, section 2.4).

Parity of individual output elements is pinned by the tests in
tests/test_oracle.py, tests/test_oracle_fp8.py, tests/test_oracle_blocks.py
tests/test_oracle_tree.py and tests/test_oracle_prefill.py (brute-force SDPA, closed forms, torch's float8
type, the pages' worked figures, invariants).
"""

from .attention import (  # noqa: F401
    BLOCK_SIZE,
    attend_row,
    cache_write,
    gather_sequence,
    kv_head_of,
    merge_partials,
    paged_decode,
    paged_decode_rows,
    paged_decode_split,
    partition_partials,
    softmax_weights,
    to_f64,
    visible_tokens,
)
from .blocks import copy_blocks  # noqa: F401
from .fp8 import (  # noqa: F401
    cache_write_fp8,
    e4m3_decode,
    e4m3_encode,
    e4m3_table,
    paged_decode_fp8,
    paged_decode_fp8_rows,
    quantize,
)
from .tree import paged_tree_decode, paged_tree_decode_rows, path_to_root, visible_positions  # noqa: F401
from .prefill import paged_prefill, paged_prefill_rows, query_counts, query_row, visible_count  # noqa: F401
