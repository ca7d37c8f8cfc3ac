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

// ---- fp8 (E4M3) caches: quantize while writing
//
// A KV cache of fp8 codes halves the bytes every decode step reads ("LLM
// serving: KV cache, batching, paged attention and quantization", section 3.7,
// the table of quantization schemes); E4M3 (largest magnitude 448) is the fp8
// format for inference ("07 - Inference", lourdhu02.github.io, section 4.3).
// Each thread writes one 16-byte chunk of codes (16 values of one head): the
// fp32 quotient x / scale[head] (an IEEE division), clamped to +-448 so that
// the conversion saturates instead of producing NaN, converted with
// round-to-nearest-even by v_cvt_pk_fp8_f32; a NaN input becomes 0x7F.

__device__ __forceinline__ uint32_t fp8_pair(float x0, float x1, float scale) {
  const float q0 = x0 / scale, q1 = x1 / scale;
  const float c0 = fminf(fmaxf(q0, -448.0f), 448.0f), c1 = fminf(fmaxf(q1, -448.0f), 448.0f);
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0u, false) & 0xFFFFu;
  if (q0 != q0) w = (w & 0xFF00u) | 0x7Fu;
  if (q1 != q1) w = (w & 0x00FFu) | 0x7F00u;
  return w;
}

__global__ __launch_bounds__(kThreads) void cache_write_fp8_kernel(CacheWriteFp8Params a) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t per_tok = 2 * (size_t)a.row_chunks;
  if (idx >= per_tok * (size_t)a.num_tokens) return;
  const size_t t = idx / per_tok;
  const size_t rem = idx - t * per_tok;
  const bool is_v = rem >= (size_t)a.row_chunks;
  const size_t chunk = is_v ? rem - a.row_chunks : rem;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= (int64_t)a.num_blocks * kBlockTokens) return;
  const int head = (int)(chunk * 16 / a.head_dim);
  const float scale = (is_v ? a.v_scale : a.k_scale)[head];
  float x[16];
  const size_t elem0 = t * (size_t)a.row_chunks * 16 + chunk * 16;  // first input element
  if (a.in_f32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(is_v ? a.v : a.k) + elem0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = src[i];
      x[4 * i] = f.x;
      x[4 * i + 1] = f.y;
      x[4 * i + 2] = f.z;
      x[4 * i + 3] = f.w;
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(is_v ? a.v : a.k) + elem0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 u = src[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = bf16_lo(w[j]);
        x[8 * i + 2 * j + 1] = bf16_hi(w[j]);
      }
    }
  }
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    out[i] = fp8_pair(x[4 * i], x[4 * i + 1], scale) | (fp8_pair(x[4 * i + 2], x[4 * i + 3], scale) << 16);
  uint4* dst = reinterpret_cast<uint4*>((is_v ? a.v_cache : a.k_cache) + (size_t)slot * a.row_chunks * 16) + chunk;
  *dst = make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace

hipError_t launch_cache_write_fp8(const CacheWriteFp8Params& p, hipStream_t s) {
  const size_t threads = 2 * (size_t)p.row_chunks * p.num_tokens;
  const size_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cache_write_fp8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s) {
  const size_t threads = 2 * (size_t)p.row_chunks * p.num_tokens;
  const size_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
