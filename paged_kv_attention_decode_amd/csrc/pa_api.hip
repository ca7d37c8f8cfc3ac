// C ABI of the paged-attention library: argument validation, kernel choice,
// launch.  Declarations and contracts are in include/pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_kernels.h"
#include "pa_prefill.h"

namespace {

constexpr int kBlock = 16;
constexpr size_t kAlign = 256;
constexpr int kMaxRowsF32 = 8;
constexpr int kMaxRowsBF16 = 64;
constexpr int kMaxRowsValu = 8;  // the vector-ALU kernel's limit
constexpr int kMaxQLen = 8;       // new tokens per sequence, causal
constexpr int kMaxTreeNodes = 64; // tree nodes per sequence (one bit each in a row's path mask)
constexpr int kMaxPrefillTokens = 1 << 20;  // new tokens of one sequence in one pa_prefill call
// bf16 with at least this many rows per KV head runs on the matrix cores
#ifndef PA_MFMA_MIN_ROWS
#define PA_MFMA_MIN_ROWS 8
#endif
constexpr int kMfmaMinRows = PA_MFMA_MIN_ROWS;
static_assert(kMfmaMinRows <= kMaxRowsValu + 1, "every row count needs a kernel");

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct WsLayout {
  size_t m_off, l_off, o_off, total;  // partitions
  size_t cnt_off, piece_off;           // balanced
  int parts;
};


// partition_size > 0: max_logits[R][P], exp_sums[R][P], partial outputs [R][P][D] (R = rows, P = partitions)
// partition_size == PA_BALANCED: counters int32[S * n_kv], pieces [2 * kBalancedMaxWGs][rows per KV head][D + 2]
bool workspace_layout(int32_t S, int32_t q_len, int32_t n_h, int32_t n_kv, int32_t D, int32_t MB, int32_t bs,
                      int32_t ps, WsLayout* w) {
  if (S < 0 || q_len <= 0 || n_h <= 0 || n_kv <= 0 || n_h % n_kv != 0 || D <= 0 || MB <= 0 || bs <= 0) return false;
  *w = WsLayout{};
  if (ps == PA_BALANCED) {
    const size_t rows_kv = (size_t)(n_h / n_kv) * q_len;
    w->cnt_off = 0;
    w->piece_off = align_up((size_t)S * n_kv * sizeof(int32_t));
    w->total = w->piece_off + align_up(2 * (size_t)pa::kBalancedMaxWGs * rows_kv * (D + 2) * sizeof(float));
    return true;
  }
  if (ps <= 0 || ps % bs != 0) return false;
  const size_t ctx = (size_t)MB * bs;
  const size_t parts = (ctx + ps - 1) / ps;
  if (parts > 0x7fffffff) return false;
  const size_t rows = (size_t)S * q_len * n_h;
  const size_t stats = align_up(rows * parts * sizeof(float));
  w->parts = (int)parts;
  w->m_off = 0;
  w->l_off = stats;
  w->o_off = 2 * stats;
  w->total = 2 * stats + align_up(rows * parts * (size_t)D * sizeof(float));
  return true;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// The address a kernel uses for p: p itself for device or managed memory, the
// mapped device address for pinned host memory; false for anything else
// (pageable or unknown memory), which a kernel must never touch.
bool gpu_address(const void* p, const void** out) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error the failed query leaves
    return false;
  }
  switch (a.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
      *out = p;
      return true;
    case hipMemoryTypeHost:
      if (!a.devicePointer) return false;
      *out = a.devicePointer;
      return true;
    default:
      return false;
  }
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: sizes inconsistent, out of range, or a pointer not 16-byte aligned";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: head_dim must be 64 or 128, block_size 16, rows per KV head <= 8 (fp32) or "
             "<= 64 (bf16), dtype PA_F32 or PA_BF16";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing, misaligned or smaller than pa_decode_workspace_size()";
    case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime reported an error at launch";
    case PA_ERR_MEMORY: return "PA_ERR_MEMORY: a buffer is not memory the GPU can access";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: pa_decode_balanced_noalloc needs more than its fixed 32 MiB scratch for these sizes "
             "(use pa_decode with a workspace)";
  }
  return "unknown pa_status";
}

int32_t pa_version(void) { return 10000; }

pa_status pa_cache_write(const void* k, const void* v, void* k_cache, void* v_cache, const int64_t* slot_mapping,
                         int32_t num_tokens, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, pa_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_SHAPE;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlock || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_SHAPE;
  const size_t esz = dtype == PA_F32 ? 4 : 2;
  const size_t row_bytes = (size_t)num_kv_heads * head_dim * esz;
  if (row_bytes / 16 > 0x7fffffff || 2 * (row_bytes / 16) * (size_t)num_tokens / 256 > 0x7fffffff)
    return PA_ERR_SHAPE;
  pa::CacheWriteParams p;
  p.k = k;
  p.v = v;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.slots = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_blocks = num_blocks;
  p.row_chunks = (int)(row_bytes / 16);
  return from_hip(pa::launch_cache_write(p, static_cast<hipStream_t>(stream)));
}

pa_status pa_cache_write_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, const float* k_scale, const float* v_scale,
                             int32_t num_tokens, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                             int32_t head_dim, pa_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_SHAPE;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlock || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale) return PA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_SHAPE;
  const size_t row_codes = (size_t)num_kv_heads * head_dim;
  if (row_codes / 16 > 0x7fffffff || 2 * (row_codes / 16) * (size_t)num_tokens / 256 > 0x7fffffff) return PA_ERR_SHAPE;
  pa::CacheWriteFp8Params p;
  p.k = k;
  p.v = v;
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.slots = slot_mapping;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.num_tokens = num_tokens;
  p.num_blocks = num_blocks;
  p.head_dim = head_dim;
  p.row_chunks = (int)(row_codes / 16);
  p.in_f32 = dtype == PA_F32;
  return from_hip(pa::launch_cache_write_fp8(p, static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int64_t* block_mapping, int32_t num_pairs, int32_t src_num_blocks,
                         int32_t dst_num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16 != 0)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 0x7fffffff / 2) return PA_ERR_UNSUPPORTED;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PA_ERR_NULL;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v)) return PA_ERR_SHAPE;
  const void *sk, *sv, *dk, *dv, *map;
  if (!gpu_address(src_k, &sk) || !gpu_address(src_v, &sv) || !gpu_address(dst_k, &dk) ||
      !gpu_address(dst_v, &dv) || !gpu_address(block_mapping, &map))
    return PA_ERR_MEMORY;
  pa::CopyBlocksParams p;
  p.src_k = sk;
  p.src_v = sv;
  p.dst_k = const_cast<void*>(dk);
  p.dst_v = const_cast<void*>(dv);
  p.mapping = static_cast<const int64_t*>(map);
  p.num_pairs = num_pairs;
  p.src_blocks = src_num_blocks;
  p.dst_blocks = dst_num_blocks;
  p.block_chunks = block_bytes / 16;
  return from_hip(pa::launch_copy_blocks(p, static_cast<hipStream_t>(stream)));
}

pa_status pa_kv_cache_layout(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                             int32_t elem_bytes, int64_t* total_bytes, int64_t* v_offset) {
  if (!total_bytes || !v_offset) return PA_ERR_NULL;
  if (num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4))
    return PA_ERR_SHAPE;
  if (block_size != kBlock) return PA_ERR_UNSUPPORTED;
  constexpr long long kPeriod = 2048, kLine = 128, kMax = 1LL << 62;
  const long long row = (long long)num_kv_heads * head_dim * elem_bytes;  // < 2^35
  if (num_blocks > kMax / (block_size * row) / 3) return PA_ERR_UNSUPPORTED;
  const long long pool = num_blocks * block_size * row;
  const long long slice = ((long long)head_dim * elem_bytes + kLine - 1) / kLine * kLine % kPeriod;
  *v_offset = (pool + kPeriod - 1) / kPeriod * kPeriod + slice;
  *total_bytes = *v_offset + pool;
  return PA_OK;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t partition_size) {
  WsLayout w;
  if (!workspace_layout(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                        partition_size, &w))
    return 0;
  return w.total;
}

namespace {

// pa_decode, pa_decode_fp8 and pa_decode_tree: validation, workspace, schedule and launch
pa_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, bool fp8, bool tree, const int32_t* parents, const void* new_k,
                      const void* new_v, const int32_t* block_tables, const int32_t* context_lens, float scale, int32_t q_len,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, pa_dtype dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if ((fp8 || tree) && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlock || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || q_len < 1 || q_len > (tree ? kMaxTreeNodes : kMaxQLen) || num_q_heads <= 0 ||
      num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      (partition_size < 0 && partition_size != PA_BALANCED) || (partition_size > 0 && partition_size % kBlock != 0))
    return PA_ERR_SHAPE;
  if (num_seqs > 65535 || num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  const int rows = group * q_len;
  if (rows > (dtype == PA_F32 ? kMaxRowsF32 : kMaxRowsBF16)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  const bool split = partition_size > 0;
  const bool balanced = partition_size == PA_BALANCED;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || (!split && !out)) return PA_ERR_NULL;
  if (fp8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (tree && !parents) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || (out && !aligned16(out))) return PA_ERR_SHAPE;
  const bool append = new_k || new_v;
  if (append && (!new_k || !new_v)) return PA_ERR_NULL;
  if (append && (!aligned16(new_k) || !aligned16(new_v))) return PA_ERR_SHAPE;

  pa::DecodeParams p = {};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.parents = tree ? parents : nullptr;
  p.new_k = append ? new_k : nullptr;
  p.new_v = append ? new_v : nullptr;
  p.append_row_bytes = append ? head_dim * (dtype == PA_F32 ? 4 : 2) : 0;
  p.tables = block_tables;
  p.lens = context_lens;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.q_len = q_len;
  p.group = group;
  p.n_h = num_q_heads;
  p.n_kv = num_kv_heads;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.mode = pa::kSinglePass;
  p.part_blocks = 0;
  p.num_parts = 1;
  p.num_wgs = 0;
  if (split || balanced) {
    WsLayout w;
    if (!workspace_layout(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                          partition_size, &w))
      return PA_ERR_SHAPE;
    if (!workspace) return PA_ERR_WORKSPACE;
    if (workspace_bytes < w.total || !aligned16(workspace)) return PA_ERR_WORKSPACE;
    char* base = static_cast<char*>(workspace);
    if (split) {
      p.mode = pa::kPartitions;
      p.ws_m = reinterpret_cast<float*>(base + w.m_off);
      p.ws_l = reinterpret_cast<float*>(base + w.l_off);
      p.ws_o = reinterpret_cast<float*>(base + w.o_off);
      p.part_blocks = partition_size / kBlock;
      p.num_parts = w.parts;
    } else if (num_seqs <= pa::kBalancedMaxSeqs && num_kv_heads <= pa::kBalancedMaxWGs) {
      p.mode = pa::kBalanced;
      p.counters = reinterpret_cast<int*>(base + w.cnt_off);
      p.pieces = reinterpret_cast<float*>(base + w.piece_off);
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8) return from_hip(pa::launch_decode_mfma_fp8(p, head_dim, rows, s));
  if (tree) return from_hip(pa::launch_decode_mfma_tree(p, head_dim, rows, s));
  if (dtype == PA_BF16 && rows >= kMfmaMinRows) return from_hip(pa::launch_decode_mfma(p, head_dim, rows, s));
  return from_hip(pa::launch_decode_valu(p, dtype == PA_F32 ? pa::kF32 : pa::kBF16, head_dim, rows, s));
}

// ---- pa_decode_balanced_noalloc: the balanced decode with a fixed scratch.
// The balanced mode's counters and pieces live in this array instead of a
// caller's workspace.  Host code never passes the array's name to a kernel
// (in host code it is only a stand-in for the device symbol): the device
// address comes from hipGetSymbolAddress, once per device, and is kept here.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words(uint4* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// this device's copy of the array; the first call on a device clears it (a
// kernel on the caller's stream, ahead of the decode)
pa_status scratch_of_current_device(char** out, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_HIP;
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, s, static_cast<uint4*>(ptr),
                       kNoAllocScratchBytes / sizeof(uint4));
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

pa_status pa_decode_balanced_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t q_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_blocks, int32_t block_size,
                                     int32_t max_blocks_per_seq, pa_dtype dtype, void* stream) {
  WsLayout w;
  if (num_seqs > 0 && workspace_layout(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                       block_size, PA_BALANCED, &w) &&
      w.total > kNoAllocScratchBytes)
    return PA_ERR_SCRATCH;  // more than the fixed scratch holds
  char* ws = nullptr;
  if (num_seqs > 0) {
    const pa_status st = scratch_of_current_device(&ws, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
  return decode_impl(out, q, k_cache, v_cache, nullptr, nullptr, false, false, nullptr, nullptr, nullptr, block_tables,
                     context_lens, scale, q_len, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, PA_BALANCED, ws, kNoAllocScratchBytes, dtype, stream);
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale, int32_t q_len,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, pa_dtype dtype, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, nullptr, nullptr, false, false, nullptr, nullptr, nullptr, block_tables,
                     context_lens, scale, q_len, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, partition_size, workspace, workspace_bytes, dtype, stream);
}

pa_status pa_decode_append(void* out, const void* q, const void* new_k, const void* new_v, void* k_cache,
                           void* v_cache, const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t q_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                           void* stream) {
  if (num_seqs > 0 && (!new_k || !new_v)) return PA_ERR_NULL;
  return decode_impl(out, q, k_cache, v_cache, nullptr, nullptr, false, false, nullptr, new_k, new_v, block_tables,
                     context_lens, scale, q_len, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     block_size, max_blocks_per_seq, partition_size, workspace, workspace_bytes, dtype, stream);
}

pa_status pa_decode_tree(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, const int32_t* tree_parents,
                         float scale, int32_t tree_size, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, pa_dtype dtype, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, nullptr, nullptr, false, true, tree_parents, nullptr, nullptr,
                     block_tables, context_lens, scale, tree_size, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     block_size, max_blocks_per_seq, partition_size, workspace, workspace_bytes, dtype, stream);
}

pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables, const int32_t* context_lens, float scale,
                        int32_t q_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                        void* stream) {
  return decode_impl(out, q, k_cache, v_cache, k_scale, v_scale, true, false, nullptr, nullptr, nullptr, block_tables,
                     context_lens, scale, q_len, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, partition_size, workspace, workspace_bytes, dtype, stream);
}

pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                     float scale, int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                     int32_t max_blocks_per_seq, pa_dtype dtype, void* stream) {
  if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlock || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_tokens < 0 || max_q_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (num_seqs > 65535 || num_kv_heads > 65535 || max_q_len > kMaxPrefillTokens) return PA_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * kBlock > 0x7fffffffLL) return PA_ERR_SHAPE;
  {
    // the kernel indexes query rows and its workgroups with 32-bit ints
    const long long rows = (long long)max_q_len * (num_q_heads / num_kv_heads);
    const long long chunks = (rows + pa::kPrefillRowsPerWG - 1) / pa::kPrefillRowsPerWG;
    if (rows > 0x7fffffffLL || chunks * num_kv_heads * num_seqs > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0 || num_q_tokens == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_SHAPE;
  pa::PrefillParams p;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.tables = block_tables;
  p.lens = context_lens;
  p.qstart = query_start;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.group = num_q_heads / num_kv_heads;
  p.n_h = num_q_heads;
  p.n_kv = num_kv_heads;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.max_q_len = max_q_len;
  p.num_q_tokens = num_q_tokens;
  p.num_seqs = num_seqs;
  return from_hip(pa::launch_prefill(p, head_dim, static_cast<hipStream_t>(stream)));
}

pa_status pa_reduce(void* out, const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                    int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size, pa_dtype dtype,
                    void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlock || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || q_len < 1 || q_len > kMaxTreeNodes || num_q_heads <= 0 || max_blocks_per_seq <= 0 ||
      partition_size <= 0 || partition_size % kBlock != 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_SHAPE;
  WsLayout w;
  if (!workspace_layout(num_seqs, q_len, num_q_heads, 1, head_dim, max_blocks_per_seq, block_size, partition_size,
                        &w))
    return PA_ERR_SHAPE;
  if (!workspace) return PA_ERR_WORKSPACE;
  if (workspace_bytes < w.total || !aligned16(workspace)) return PA_ERR_WORKSPACE;
  if ((size_t)num_seqs * q_len * num_q_heads > 0x7fffffff) return PA_ERR_SHAPE;
  const char* base = static_cast<const char*>(workspace);
  pa::ReduceParams p;
  p.out = out;
  p.ws_m = reinterpret_cast<const float*>(base + w.m_off);
  p.ws_l = reinterpret_cast<const float*>(base + w.l_off);
  p.ws_o = reinterpret_cast<const float*>(base + w.o_off);
  p.lens = context_lens;
  p.q_len = q_len;
  p.n_h = num_q_heads;
  p.max_blocks = max_blocks_per_seq;
  p.part_blocks = partition_size / kBlock;
  p.num_parts = w.parts;
  p.num_seqs = num_seqs;
  return from_hip(pa::launch_reduce(p, dtype == PA_F32 ? pa::kF32 : pa::kBF16, head_dim,
                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"
