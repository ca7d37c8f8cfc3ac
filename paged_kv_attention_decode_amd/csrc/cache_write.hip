// Slot-mapped write of new K/V rows into the paged caches.
//
// A new token is appended in place in its sequence's last block
// ("LLM Inference Serving", systeminternals.dev, the Sequence / block_table
// sketch); its flat slot is physical_block * 16 + row, logical block i
// holding tokens 16i .. 16i+15 ("LLM serving: KV cache, batching, paged
// attention and quantization", section 3.5).  One token's K (or V) row over
// all KV heads is contiguous in both the input [T, n_kv, D] and the cache
// [NB, 16, n_kv, D], so each thread copies one 16-byte chunk of one row as raw
// bits.  Slots that are negative or outside the pool are skipped.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void cache_write_kernel(CacheWriteParams a) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t per_tok = 2 * (size_t)a.row_chunks;
  if (idx >= per_tok * (size_t)a.num_tokens) return;
  const size_t t = idx / per_tok;
  const size_t rem = idx - t * per_tok;
  const bool is_v = rem >= (size_t)a.row_chunks;
  const size_t chunk = is_v ? rem - a.row_chunks : rem;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= (int64_t)a.num_blocks * kBlockTokens) return;
  const uint4* src = static_cast<const uint4*>(is_v ? a.v : a.k) + t * a.row_chunks + chunk;
  uint4* dst = static_cast<uint4*>(is_v ? a.v_cache : a.k_cache) + (size_t)slot * a.row_chunks + chunk;
  *dst = *src;
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s) {
  const size_t threads = 2 * (size_t)p.row_chunks * p.num_tokens;
  const size_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
