/*
 * pa.h - paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Operations:
 *
 *   pa_cache_write  store the K/V rows of new tokens into their cache slots;
 *   pa_decode       attention of the newest q_len tokens of every sequence over
 *                   its paged KV cache: in one pass, work-balanced across the
 *                   GPU, or as per-partition partials (split context);
 *   pa_reduce       merge the partials of a split pa_decode into the output;
 *   pa_decode_append
 *                   pa_cache_write of the new tokens and pa_decode in one launch;
 *   pa_cache_write_fp8, pa_decode_fp8
 *                   the same over a KV cache of fp8 (E4M3) codes with one
 *                   scale per KV head;
 *   pa_decode_tree  verify a tree of draft tokens under a tree mask;
 *   pa_prefill      chunked prefill: new tokens of varying count per sequence;
 *   pa_copy_blocks  copy whole blocks (copy-on-write, swapping);
 *   pa_kv_cache_layout
 *                   where to place the K and V pools of one layer in one
 *                   allocation (a host-side query; launches nothing).
 *
 * Sources of the definitions (the web pages this library implements):
 *   - per layer, K and V are each stored as [num_blocks, block_size,
 *     num_kv_heads, head_dim] ("LLM Inference Serving", systeminternals.dev,
 *     the passage on the per-layer cache shape);
 *   - a sequence's block table maps logical block i (tokens 16i .. 16i+15) to
 *     a physical block id; the kernel follows the table and reads keys and
 *     values one block at a time ("LLM serving: KV cache, batching, paged
 *     attention and quantization", learn.mohebi.ai, section 3.5);
 *   - a generated token is appended in place in the last block while it has
 *     room (systeminternals.dev, the Sequence / block_table sketch);
 *   - decode attention: q^T K, softmax, weighted sum of V per query head;
 *     n_h / n_kv query heads share one KV head (learn.mohebi.ai, section 3.3
 *     and the notation of section 3);
 *   - speculative verify scores all K+1 positions in one pass under a causal
 *     mask ("07 - Inference", lourdhu02.github.io, section 3);
 *   - split context: chunks produce partials (m, l, acc) that a second small
 *     kernel merges with the online-softmax rescaling rule (lourdhu02.github.io,
 *     section 5.3 "Decode attention and FlashDecoding");
 *   - an fp8 KV cache stores keys and values in 8 bits while the products run
 *     in higher precision, halving the KV bytes read per step
 *     (learn.mohebi.ai, section 3.7, the table of quantization schemes); E4M3,
 *     largest magnitude 448, is the fp8 format for inference, with per-tensor,
 *     per-channel or per-block scales (lourdhu02.github.io, section 4.3);
 *   - tree verification: the candidates of a draft tree are checked in one
 *     pass under a tree attention mask ("Chapter 18: Speculative Decoding
 *     and Serving Optimizations", arunshar.com, section 18.1.2;
 *     lourdhu02.github.io, section 3.4);
 *   - chunked prefill: a long prompt processed in chunks over several steps,
 *     each chunk attending to the cached prefix (arunshar.com, section
 *     18.2.1; learn.mohebi.ai, section 3.6; lourdhu02.github.io, section 2.4);
 *   - copy-on-write of shared blocks and swapping of paused sequences
 *     (learn.mohebi.ai, section 3.5; arunshar.com, section 18.2.2).
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or synchronizes; it enqueues kernels on `stream`
 *     (a hipStream_t; NULL means the default stream) and returns.
 *   - Tensors are dense, row-major, and 16-byte aligned.
 *   - dtype selects the element type of q, out, k, v and the caches:
 *     PA_F32 (IEEE binary32) or PA_BF16 (bfloat16).  Arithmetic is fp32.
 *   - block_size must be 16; head_dim must be 64 or 128.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid argument returns an error status and launches nothing.
 *   - Values that live in device memory (context lengths, block ids, slots)
 *     cannot be checked on the host without a synchronization.  The kernels
 *     never access memory out of bounds because of them: a slot outside the
 *     pool is skipped, a block id outside [0, num_blocks) contributes no
 *     tokens, a context length is clamped to max_blocks_per_seq * block_size.
 *     Such values are still caller errors and give unspecified results.
 *   - Stateless and re-entrant; no global state.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  PA_ERR_UNSUPPORTED = 3, /* valid but not implemented (head_dim, block_size, rows per KV head, dtype) */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than pa_decode_workspace_size() */
  PA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  PA_ERR_MEMORY = 6,      /* a buffer is not memory the GPU can access (e.g. pageable host memory) */
  PA_ERR_SCRATCH = 7      /* pa_decode_balanced_noalloc: the call needs more than its fixed scratch */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* partition_size value selecting the work-balanced mode of pa_decode */
#define PA_BALANCED (-1)

/*
 * pa_cache_write - write the K and V rows of new tokens into the paged caches.
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim]  new keys / values
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim]
 *   v_cache
 *   slot_mapping  int64 [num_tokens]: slot = physical_block * block_size + row.
 *                 A negative slot skips the token; a slot >= num_blocks *
 *                 block_size is skipped as well (caller error).  Two tokens with
 *                 the same slot is a caller error (which one lands is unspecified).
 *
 * The rows are copied as raw bits (bit-exact, NaN payloads included); nothing
 * else in the caches changes.  num_tokens == 0 is valid and launches nothing.
 */
pa_status pa_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                         void* stream);

/*
 * pa_decode - paged attention of the q_len newest tokens of each sequence.
 *
 *   out           [num_seqs * q_len, num_q_heads, head_dim], dtype.  Written when
 *                 partition_size is 0 or PA_BALANCED; untouched by a split call
 *                 (may be NULL then).
 *   q             [num_seqs * q_len, num_q_heads, head_dim], dtype.  Row
 *                 b * q_len + j is query token j of sequence b.
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim], dtype
 *   v_cache
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; entry i of row b is the
 *                 physical block holding tokens i*block_size .. +block_size-1 of
 *                 sequence b.  Entries at or past ceil(L_b / block_size) are never read.
 *   context_lens  int32 [num_seqs]; L_b counts the q_len new tokens, which must
 *                 already be in the cache.  Query token j sits at position
 *                 L_b - q_len + j and attends to positions 0 .. L_b - q_len + j
 *                 (causal among the new tokens; all L_b positions when q_len == 1).
 *                 A query row with no visible position gets zeros.
 *   scale         softmax scale applied to q.k (typically 1/sqrt(head_dim)).
 *   q_len         1 .. 8 new tokens per sequence.
 *   num_q_heads   a multiple of num_kv_heads; query head h reads KV head
 *                 h / (num_q_heads / num_kv_heads).  Rows per KV head
 *                 (num_q_heads / num_kv_heads) * q_len must be <= 8 for PA_F32 and
 *                 <= 64 for PA_BF16.
 *   partition_size
 *                 0: one pass, one workgroup per (KV head, sequence); writes out.
 *                 PA_BALANCED (-1): writes out; the (sequence, block) work is
 *                 cut into equal ranges, each taken by one workgroup per KV head,
 *                 so ragged context lengths keep every compute unit equally busy
 *                 and the heads of a token row are read together; a
 *                 (sequence, head) cut between ranges is merged inside the call
 *                 with the rescaling rule, in a fixed order.  Needs a workspace
 *                 whose first 4 * num_seqs * num_kv_heads bytes are zero before
 *                 the first such call; every balanced call leaves them zero, so
 *                 one workspace serves any number of calls.  Batches of more than
 *                 4096 sequences, or more than 1024 KV heads, fall back to the
 *                 one-pass mode.
 *                 Otherwise a positive multiple of block_size: the context is
 *                 split into partitions [p*partition_size, (p+1)*partition_size),
 *                 and for every query row the partition's partial result is
 *                 written to the workspace; pa_reduce then produces out.
 *   workspace     device buffer of at least pa_decode_workspace_size(...) bytes
 *                 for the same partition_size (only used, and only required,
 *                 when partition_size != 0).  Its contents are private to the
 *                 library; a workspace used by a split call must be zeroed again
 *                 before it serves a balanced call.  Calls sharing one workspace
 *                 must not overlap in time.
 *
 * Results are bitwise deterministic from run to run and independent of the
 * physical block ids.  In the one-pass and split modes a sequence's result
 * also does not depend on the other sequences of the batch; in PA_BALANCED
 * mode the cut points follow the whole batch's context lengths, so a
 * sequence's result may differ in the last bits with the batch around it.
 * With bf16, the softmax weights are rounded to bf16 before the weighted sum
 * of V, and the row sums add the same rounded weights: 8 or more rows per KV
 * head run on the matrix cores, fewer on the vector ALUs (two tokens per
 * v_dot2_f32_bf16).  fp32 keeps the weights in fp32.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale, int32_t q_len,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                    int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                    void* stream);

/*
 * pa_decode_append - pa_cache_write of the batch's new tokens and pa_decode
 * over them, in one launch.
 *
 * A generated token's key and value are appended in place in its sequence's
 * last block ("LLM Inference Serving", systeminternals.dev, the Sequence /
 * block_table sketch), and are written before attention reads them ("07 -
 * Inference", lourdhu02.github.io, section 3, speculative verify).  Launching
 * the store and the attention as one kernel removes a launch per step (the
 * pages name launch overhead as what fusing small kernels saves: lourdhu02,
 * sections 2.6 and 5.4).
 *
 *   new_k, new_v  [num_seqs * q_len, num_kv_heads, head_dim], dtype; row
 *                 b * q_len + j is new token j of sequence b, whose position is
 *                 L_b - q_len + j.  It is stored at slot
 *                 16 * block_tables[b][pos / 16] + pos % 16 of k_cache /
 *                 v_cache (a position below 0, or a block id outside
 *                 [0, num_blocks), is skipped, as pa_cache_write skips a slot
 *                 outside the pool).
 *   k_cache, v_cache  written (the new rows) and read.
 * Every other argument, the schedules, the workspace and the results are those
 * of pa_decode (PA_F32 or PA_BF16).  After the call the caches hold exactly
 * what pa_cache_write with those slots would have stored, and out (or the
 * partials for pa_reduce) is bit for bit what pa_decode computes after it.
 * The new tokens of one sequence must not share a slot with another
 * sequence's tokens or with any position read by the call.
 */
pa_status pa_decode_append(void* out, const void* q, const void* new_k, const void* new_v, void* k_cache,
                           void* v_cache, const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t q_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                           void* stream);

/*
 * pa_decode_balanced_noalloc - pa_decode with partition_size PA_BALANCED and no
 * workspace argument, for callers that cannot allocate memory (code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that
 * forbid it).
 *
 * Arguments, layouts and results are those of pa_decode; the call computes
 * bit for bit what pa_decode computes with PA_BALANCED.  The balanced mode's
 * counters and partial results live in a fixed 32 MiB array of device memory
 * inside the library (one per GPU, held until the process ends), so the call
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine.
 * The first call on a device looks the array up and clears it with a kernel
 * on the given stream.  Every call on a GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and must not
 * be made.
 *
 * Returns PA_ERR_SCRATCH, launching nothing, when the call would need more
 * than 32 MiB, i.e. when pa_decode_workspace_size(..., PA_BALANCED) exceeds
 * 33554432 bytes (with head_dim 128, up to 31 rows per KV head fit, fewer when
 * num_seqs * num_kv_heads is above about 130,000); PA_ERR_HIP when the array
 * cannot be looked up; the errors of pa_decode otherwise.
 */
pa_status pa_decode_balanced_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t q_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_blocks, int32_t block_size,
                                     int32_t max_blocks_per_seq, pa_dtype dtype, void* stream);

/*
 * pa_decode_workspace_size - bytes of workspace pa_decode needs for partition_size.
 *
 * Split (partition_size > 0): with P = ceil(max_blocks_per_seq * block_size /
 * partition_size) partitions and R = num_seqs * q_len * num_q_heads query rows,
 * fp32 max_logits[R][P], exp_sums[R][P] and partial outputs [R][P][head_dim].
 * Balanced (PA_BALANCED): int32 arrival counters [num_seqs * num_kv_heads], then
 * fp32 partials for 2 * 1024 pieces of (num_q_heads / num_kv_heads) * q_len rows
 * of head_dim + 2 values.  Each region is 256-byte aligned.  Returns 0 for
 * partition_size 0, invalid sizes, or a partition_size that is neither.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t partition_size);

/*
 * pa_reduce - merge the per-partition partials of a split pa_decode into out.
 *
 * The arguments must repeat those of the pa_decode (pa_decode_fp8,
 * pa_decode_tree with q_len = tree_size, up to 64) call that filled the
 * workspace (same shapes, partition_size, context_lens), on the same stream or
 * after it.  For each query row: M = max over partitions of m_p,
 * w_p = l_p * 2^(m_p - M), out = sum_p w_p * o_p / sum_p w_p, over the
 * partitions that hold at least one position the row may see.
 */
pa_status pa_reduce(void* out, const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                    int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size, pa_dtype dtype,
                    void* stream);

/* A static, human-readable description of a status code. */
/*
 * fp8 KV cache.  The caches hold OCP E4M3 codes (one byte per value: sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7F/0xFF are
 * NaN; largest finite magnitude 448) in the same [num_blocks, block_size,
 * num_kv_heads, head_dim] layout.  Each KV head g has an fp32 scale for K and
 * one for V: code c of head g stands for decode(c) * scale[g].  Per-tensor
 * scaling is the case of equal scales.
 *
 * pa_cache_write_fp8 - quantize the K and V rows of new tokens into their slots.
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim] of dtype (PA_F32 or PA_BF16).
 *   k_cache,      uint8 [num_blocks, block_size, num_kv_heads, head_dim] codes.
 *   v_cache
 *   slot_mapping  int64 [num_tokens] as for pa_cache_write (negative = skip;
 *                 slots outside the pool are skipped).
 *   k_scale,      fp32 [num_kv_heads] device arrays, positive and finite.
 *   v_scale
 *
 * Each value x of head g becomes the E4M3 code nearest to the fp32 quotient
 * x / scale[g] (one correctly rounded fp32 division), ties to the even
 * mantissa, after clamping the quotient to [-448, 448]; a NaN becomes 0x7F.
 * Deterministic and bit-exact.
 */
pa_status pa_cache_write_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, const float* k_scale, const float* v_scale,
                             int32_t num_tokens, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                             int32_t head_dim, pa_dtype dtype, void* stream);

/*
 * pa_decode_fp8 - pa_decode over an fp8 KV cache.
 *
 * Arguments as pa_decode, with k_cache and v_cache holding E4M3 codes and
 * k_scale, v_scale the per-head fp32 scales; dtype (the type of q and out)
 * must be PA_BF16; rows per KV head up to 64.  The keys and values are decoded
 * to bf16 exactly (every E4M3 value is a bf16 value) and multiplied on the
 * matrix cores with fp32 accumulation; the K scale is folded into the score
 * scale and the V scale into the final normalization.  The workspace, the
 * partition sizes, PA_BALANCED and pa_reduce work as for pa_decode (the
 * partials are in the output's units, so pa_reduce merges them unchanged).
 */
pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables, const int32_t* context_lens, float scale,
                        int32_t q_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                        void* stream);

/*
 * pa_decode_tree - verify a tree of draft tokens in one pass (tree attention).
 *
 * Speculative decoding with several candidates per position checks them as a
 * tree in a single forward pass of the target model, e.g. a complete binary
 * tree of 15 nodes over 4 levels ("Chapter 18: Speculative Decoding and
 * Serving Optimizations", arunshar.com, section 18.1.2, tree-based
 * verification for Medusa), under a tree attention mask ("07 - Inference",
 * lourdhu02.github.io, section 3.4).
 *
 *   tree_size     T = 1 .. 64 nodes per sequence; they take the place of the
 *                 q_len new tokens of pa_decode: node j of sequence b is query
 *                 row b * T + j, its key and value are already in the cache at
 *                 position L_b - T + j, and context_lens counts the T nodes.
 *   tree_parents  int32 [num_seqs, T] device array: the parent node of node j,
 *                 an earlier node (0 <= parent < j), or -1 for a node that
 *                 hangs directly on the context (a root; several roots form a
 *                 forest).  Node j attends to every position before the tree
 *                 and to the nodes on its own path to the root, itself
 *                 included; never to its siblings or other branches.  A chain
 *                 (parent j - 1) gives pa_decode's causal verify.  A parent
 *                 outside [-1, j) ends the node's path there, as -1 does.
 *   dtype         PA_BF16 (q, out and the caches); rows per KV head
 *                 (num_q_heads / num_kv_heads) * T up to 64.  Runs on the
 *                 matrix cores like bf16 pa_decode with 8 or more rows.
 *
 * Every other argument, the workspace, the partition modes, PA_BALANCED and
 * pa_reduce (called with q_len = T) are those of pa_decode.
 */
pa_status pa_decode_tree(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, const int32_t* tree_parents,
                         float scale, int32_t tree_size, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, pa_dtype dtype, void* stream);

/*
 * pa_prefill - attention of the new tokens of sequences with different
 * numbers of them: chunked prefill, optionally mixed with decode tokens.
 *
 * A long prompt is processed in chunks (for example 512 tokens) over several
 * engine steps, a step filling a token budget with decode tokens and prefill
 * chunks ("Chapter 18: Speculative Decoding and Serving Optimizations",
 * arunshar.com, section 18.2.1; "LLM serving: KV cache, batching, paged
 * attention and quantization", learn.mohebi.ai, section 3.6; "07 -
 * Inference", lourdhu02.github.io, section 2.4).  Each new token attends to
 * every cached token before it and to the earlier new tokens of its sequence,
 * so a prompt run in chunks gives the same result as in one piece.
 *
 *   out, q        [num_q_tokens, num_q_heads, head_dim] bf16.  Sequence b owns
 *                 rows query_start[b] .. query_start[b + 1] - 1, its n_b new
 *                 tokens in order.
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim] bf16, with
 *   v_cache       the new tokens' K/V already written (pa_cache_write).
 *   block_tables, as for pa_decode; context_lens[b] = L_b counts the n_b new
 *   context_lens  tokens: new token i sits at position L_b - n_b + i and sees
 *                 positions 0 .. L_b - n_b + i.  A row with no visible position
 *                 (L_b < n_b) gets zeros.
 *   query_start   int32 [num_seqs + 1] device array, nondecreasing, from 0 to
 *                 num_q_tokens.  A sequence with n_b = 0 is skipped; one whose
 *                 range is negative, longer than max_q_len or outside
 *                 [0, num_q_tokens) is skipped too, its rows left untouched.
 *   max_q_len     an upper bound of every n_b (1 .. 2^20); sizes the grid.
 *                 PA_ERR_UNSUPPORTED when max_q_len * (num_q_heads /
 *                 num_kv_heads) or the number of workgroups, ceil(that / 256)
 *                 * num_kv_heads * num_seqs, exceeds 2^31 - 1.
 *   dtype         PA_BF16.  head_dim 64 or 128, block_size 16.
 *
 * Each workgroup owns 256 query rows (new token x query head of one KV head's
 * group) and walks the sequence's blocks up to the last position those rows
 * see, staging each block once in LDS for its eight waves; the products run on
 * the matrix cores with fp32 accumulation, the softmax weights rounded to bf16
 * for P V as in pa_decode.  No workspace; results are bitwise deterministic
 * and do not depend on the other sequences of the call.
 */
pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                     float scale, int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                     int32_t max_blocks_per_seq, pa_dtype dtype, void* stream);

/*
 * pa_copy_blocks - copy whole KV blocks, for copy-on-write and swapping.
 *
 * Before a sequence writes into a block that other sequences share, it gets a
 * private copy ("LLM serving: KV cache, batching, paged attention and
 * quantization", learn.mohebi.ai, section 3.5, sharing and copy-on-write); a
 * paused sequence's blocks can be swapped out and back ("Chapter 18:
 * Speculative Decoding and Serving Optimizations", arunshar.com, section
 * 18.2.2).  For every pair p, block block_mapping[2p] of the source caches is
 * copied to block block_mapping[2p + 1] of the destination caches, K and V,
 * as raw bytes (any element type: bf16, fp32 or fp8 codes).
 *
 *   src_k, src_v  caches of src_num_blocks blocks of block_bytes each
 *                 ([num_blocks, block_size, num_kv_heads, head_dim] of any type).
 *   dst_k, dst_v  caches of dst_num_blocks blocks (may be src_k, src_v).
 *                 Each of the four may be device memory or pinned host memory
 *                 (hipHostMalloc), so one call swaps blocks out to host DRAM or
 *                 back in over the host link.  The library asks the runtime
 *                 about each pointer (hipPointerGetAttributes) and returns
 *                 PA_ERR_MEMORY, launching nothing, for memory the GPU cannot
 *                 access (pageable host memory).  Host buffers must not be
 *                 touched by the host until the stream has passed the copy.
 *   block_mapping int64 [num_pairs, 2] device array of (source, destination) ids;
 *                 pairs with an id outside its pool are skipped.  Destinations
 *                 must be distinct and no destination may be a source of the
 *                 same call (then the copies do not depend on their order).
 *   block_bytes   a positive multiple of 16 (bytes of one block of K, or of V).
 */
pa_status pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int64_t* block_mapping, int32_t num_pairs, int32_t src_num_blocks,
                         int32_t dst_num_blocks, int64_t block_bytes, void* stream);

/*
 * pa_kv_cache_layout - placement of one layer's K and V pools in one allocation.
 *
 * The pools keep the per-layer shape [num_blocks, block_size, num_kv_heads,
 * head_dim] ("LLM Inference Serving", systeminternals.dev, the passage on the
 * per-layer cache shape); this query only says where the V pool starts.  K
 * sits at byte 0 of an allocation whose base the caller aligns to 2 KiB; V
 * starts at *v_offset, the K pool's size rounded up to 2 KiB plus one head
 * slice (head_dim * elem_bytes, rounded up to 128 bytes, modulo 2 KiB).
 *
 * Why: on MI355X, reads of the slices that sit at some offsets within each
 * 1 KiB of the address space complete more slowly than the others.  With the
 * pools back to back, K and V of a KV head sit at the same offsets, so the
 * decode workgroups of two heads stream two slow slices per token while the
 * others stream none, and those workgroups set the launch's length.  Moving V
 * by one slice puts the slow K and slow V slices on different heads (measured
 * on the one-pass decode of 64 sequences of 512..4096 tokens, 8 KV heads of
 * 128: 111 us to 106 us in bf16, 60 us to 55 us with fp8 codes).  Every entry
 * point accepts any placement; this one is faster, not required.
 *
 *   num_blocks    blocks of each pool, > 0.
 *   block_size    16.
 *   num_kv_heads, head_dim
 *                 > 0.
 *   elem_bytes    bytes of one cache element: 1 (fp8 codes), 2 (bf16) or 4 (fp32).
 *   total_bytes   out: bytes of the allocation holding both pools.
 *   v_offset      out: byte offset of the V pool in it (a multiple of 128).
 *
 * PA_ERR_NULL for a NULL output, PA_ERR_SHAPE for a size out of range,
 * PA_ERR_UNSUPPORTED for another block_size or a size past 2^62 bytes.
 */
pa_status pa_kv_cache_layout(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                             int32_t elem_bytes, int64_t* total_bytes, int64_t* v_offset);

const char* pa_status_string(pa_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
