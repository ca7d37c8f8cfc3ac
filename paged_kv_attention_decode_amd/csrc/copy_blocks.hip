// Whole-block copies of the K and V caches, for copy-on-write of shared blocks
// ("LLM serving: KV cache, batching, paged attention and quantization",
// section 3.5) and for swapping a paused sequence's blocks out and back
// ("Chapter 18: Speculative Decoding and Serving Optimizations", section
// 18.2.2).  Grid (pairs, 2): each workgroup copies the K (y = 0) or V (y = 1)
// block of one pair with 16-byte loads and stores, every thread a strided set
// of chunks; pairs with an id outside its pool are skipped.  The stores are
// non-temporal: the copies are not read back soon, and streaming them past
// the caches took 2048 random 32 KiB block pairs from 56.0-56.7 to 41.8 us
// (three alternating runs; 42.2-42.5 with 4 chunks in flight per thread
// instead of 8, while 8 with ordinary stores took 83 us).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // chunks in flight per thread (a whole 32 KiB block at 256 threads)

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyBlocksParams a) {
  const int pair = blockIdx.x;
  const int64_t s = a.mapping[2 * (size_t)pair], d = a.mapping[2 * (size_t)pair + 1];
  if (s < 0 || s >= a.src_blocks || d < 0 || d >= a.dst_blocks) return;
  const uint4* __restrict__ src =
      static_cast<const uint4*>(blockIdx.y ? a.src_v : a.src_k) + (size_t)s * (size_t)a.block_chunks;
  uint4* __restrict__ dst = static_cast<uint4*>(blockIdx.y ? a.dst_v : a.dst_k) + (size_t)d * (size_t)a.block_chunks;
  for (int64_t c0 = threadIdx.x; c0 < a.block_chunks; c0 += (int64_t)kThreads * kUnroll) {
    uint4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + (int64_t)u * kThreads;
      if (c < a.block_chunks) x[u] = src[c];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + (int64_t)u * kThreads;
      if (c < a.block_chunks)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x[u]), reinterpret_cast<u32x4_t*>(&dst[c]));
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t s) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)p.num_pairs, 2), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
