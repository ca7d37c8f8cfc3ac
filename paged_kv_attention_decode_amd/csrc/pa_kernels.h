// Internal launch interface between the C ABI (pa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum ElemType { kF32 = 0, kBF16 = 1 };

// How a decode call divides the work among workgroups.
enum DecodeMode {
  kSinglePass = 0,  // one workgroup per (KV head, sequence); writes out
  kPartitions = 1,  // one workgroup per (partition, KV head, sequence); writes partials for pa_reduce
  kBalanced = 2,    // equal block ranges of the flattened (sequence, KV head, block) list; writes out
};

// largest batch the balanced mode handles (its block prefix over the sequences lives in LDS)
constexpr int kBalancedMaxSeqs = 4096;
// most workgroups of a balanced launch (the workspace holds two pieces per workgroup)
constexpr int kBalancedMaxWGs = 1024;

// most workgroups per compute unit in a balanced launch: more ranges than two
// per CU measured slower (70B layer: 234 us at three per CU against 221 us)
constexpr int kBalancedMaxPerCU = 2;

// Workgroups of a balanced launch: as many as stay resident together
// (resident_per_cu per compute unit, the kernel's occupancy, at most
// kBalancedMaxPerCU), so that no range waits for a second round; a whole
// number of ranges of n_kv workgroups, at least one, at most kBalancedMaxWGs
// (n_kv <= kBalancedMaxWGs is checked before).
inline int balanced_workgroups(int resident_per_cu, int n_kv) {
  if (resident_per_cu > kBalancedMaxPerCU) resident_per_cu = kBalancedMaxPerCU;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus <= 0)
    cus = 256;
  if (resident_per_cu < 1) resident_per_cu = 1;
  int ranges = resident_per_cu * cus / n_kv;
  if (ranges < 1) ranges = 1;
  if ((long long)ranges * n_kv > kBalancedMaxWGs) ranges = kBalancedMaxWGs / n_kv;
  return ranges * n_kv;
}

// workgroups of `kernel` (threads each) one compute unit keeps resident
template <class Kernel>
int resident_per_cu(Kernel kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

// One-pass launches: the pairing stride for decode_pairing in pa_schedule.h,
// or 0 for plain longest first.  The hardware hands workgroups out in launch
// order, one per compute unit first, so workgroups k and k + CUs share a CU
// when at least two fit on one.  When the whole grid (S * n_kv workgroups)
// fits in two per CU, the first CUs / n_kv sequence slots
// take the longest sequences and the rest are dealt shortest first, so that
// each CU pairs a long sequence with a short one (longest processing time
// first over the two slots) instead of the first and the CUs / n_kv-th
// longest.  Larger grids run in rounds, where launch order in descending
// length already balances.
inline int one_pass_pairing(int resident_per_cu, int num_seqs, int n_kv) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus <= 0)
    return 0;
  const long long wgs = (long long)num_seqs * n_kv;
  if (resident_per_cu < 2 || cus % n_kv != 0 || wgs <= cus || wgs > 2LL * cus) return 0;
  return cus / n_kv;
}

struct DecodeParams {
  void* out;             // [S*q_len, n_h, D] (single pass and balanced)
  const void* q;         // [S*q_len, n_h, D]
  const void* k_cache;   // [NB, 16, n_kv, D]
  const void* v_cache;
  const int32_t* tables; // [S, MB]
  const int32_t* lens;   // [S]
  float* ws_m;           // partitions: [S*q_len*n_h, P]
  float* ws_l;           // partitions: [S*q_len*n_h, P]
  float* ws_o;           // partitions: [S*q_len*n_h, P, D]
  int* counters;         // balanced: [S * n_kv] arrival counters, zero between calls
  float* pieces;         // balanced: [2 * num_wgs][rows_per_kv][D + 2] partial (m, l, o) per row
  const float* k_scale;  // fp8 caches: [n_kv] per-head scales (null otherwise)
  const float* v_scale;
  const int32_t* parents;  // tree verify: [S, q_len] parent of each node (null: causal among the new tokens)
  // append (pa_decode_append): the new tokens' K and V rows [S*q_len, n_kv, D],
  // stored at their positions before they are read (null: nothing to store)
  const void* new_k;
  const void* new_v;
  int append_row_bytes;  // bytes of one (token, head) row of K or V
  float scale_log2;      // softmax scale * log2(e)
  int q_len, group, n_h, n_kv, num_blocks, max_blocks;
  int mode;              // DecodeMode
  int part_blocks;       // partitions: blocks per partition
  int num_parts;         // partitions: partition stride of the workspace
  int num_wgs;           // balanced: workgroups in the grid (set by the launcher)
  int pair_stride;       // one pass: one_pass_pairing's stride (0: longest first)
  int num_seqs;
};

struct ReduceParams {
  void* out;
  const float* ws_m;
  const float* ws_l;
  const float* ws_o;
  const int32_t* lens;
  int q_len, n_h, max_blocks, part_blocks, num_parts, num_seqs;
};

struct CacheWriteParams {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const int64_t* slots;
  int num_tokens, num_blocks, row_chunks;  // row_chunks = 16-byte chunks per token row (n_kv * D * esize / 16)
};

struct CacheWriteFp8Params {
  const void* k;  // [T, n_kv, D] of fp32 or bf16
  const void* v;
  uint8_t* k_cache;  // [NB, 16, n_kv, D] E4M3 codes
  uint8_t* v_cache;
  const int64_t* slots;
  const float* k_scale;  // [n_kv]
  const float* v_scale;
  int num_tokens, num_blocks, head_dim;
  int row_chunks;  // 16-code chunks per token row (n_kv * D / 16)
  int in_f32;      // input dtype: 1 fp32, 0 bf16
};

struct CopyBlocksParams {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int64_t* mapping;  // [num_pairs, 2] (source, destination)
  int num_pairs;
  int64_t src_blocks, dst_blocks;
  int64_t block_chunks;  // 16-byte chunks per block
};

// rows_per_kv = group * q_len (already validated)
hipError_t launch_decode_valu(const DecodeParams& p, ElemType t, int head_dim, int rows_per_kv, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, int rows_per_kv, hipStream_t s);
hipError_t launch_decode_mfma_fp8(const DecodeParams& p, int head_dim, int rows_per_kv, hipStream_t s);
hipError_t launch_decode_mfma_tree(const DecodeParams& p, int head_dim, int rows_per_kv, hipStream_t s);
hipError_t launch_reduce(const ReduceParams& p, ElemType t, int head_dim, hipStream_t s);
hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s);
hipError_t launch_cache_write_fp8(const CacheWriteFp8Params& p, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t s);

}  // namespace pa
