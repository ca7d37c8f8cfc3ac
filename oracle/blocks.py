"""Block copies for copy-on-write and swapping (test infrastructure only).

A physical block shared by several sequences carries a reference count;
before a sequence writes into a block whose count is above one it gets a
private copy ("LLM serving: KV cache, batching, paged attention and
quantization", learn.mohebi.ai, section 3.5, sharing and copy-on-write).  A
paused sequence's blocks can be swapped out of GPU memory and back
("Chapter 18: Speculative Decoding and Serving Optimizations", arunshar.com,
section 18.2.2, on CPU swap).  Both are copies of whole blocks: the K and V
rows of all 16 slots of every KV head, as raw bytes.

Reading: a mapping is a list of (source id, destination id) pairs; pairs
whose ids fall outside their pools are skipped; the destinations are distinct
and no destination is also a source in the same call (otherwise the result
would depend on the order of the copies).
"""

from __future__ import annotations

import numpy as np


def copy_blocks(src_k, src_v, dst_k, dst_v, mapping):
    """Copies of the destination caches [NB_dst, 16, n_kv, d] after copying block
    src of the source caches to block dst for every (src, dst) in mapping."""
    out_k, out_v = dst_k.copy(), dst_v.copy()
    nb_src, nb_dst = src_k.shape[0], dst_k.shape[0]
    for s, d in np.asarray(mapping, dtype=np.int64).reshape(-1, 2):
        if 0 <= s < nb_src and 0 <= d < nb_dst:
            out_k[d] = src_k[s]
            out_v[d] = src_v[s]
    return out_k, out_v
