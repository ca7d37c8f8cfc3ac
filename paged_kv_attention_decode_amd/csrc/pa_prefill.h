// Host/device interface of the chunked-prefill kernel (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct PrefillParams {
  void* out;              // [num_q_tokens, n_h, D] bf16
  const void* q;          // [num_q_tokens, n_h, D] bf16
  const void* k_cache;    // [NB, 16, n_kv, D] bf16
  const void* v_cache;
  const int32_t* tables;  // [S, MB]
  const int32_t* lens;    // [S], new tokens included
  const int32_t* qstart;  // [S + 1], sequence b owns q rows qstart[b] .. qstart[b + 1] - 1
  float scale_log2;       // softmax scale * log2(e)
  int group, n_h, n_kv, num_blocks, max_blocks;
  int max_q_len, num_q_tokens, num_seqs;
};

// query rows (new token x head of the GQA group) per workgroup
constexpr int kPrefillRowsPerWG = 256;

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t s);

}  // namespace pa
