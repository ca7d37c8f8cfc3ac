// Merge of split-context partials (FlashDecoding's second kernel).
//
// For each query row the split pa_decode stored, per partition p, the largest
// score m_p (log2 units), the weight sum l_p = sum 2^(s - m_p) and the
// normalized partial output o_p.  The merge rescales every partition to the
// global maximum with the online-softmax rule ("07 - Inference",
// lourdhu02.github.io, section 5.3):
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// A partition in which the row sees no position has l_p = 0 and weight 0.
//
// One workgroup of 256 threads per query row: every thread owns 4 columns of
// one partition slot; the slots stride over the partitions and are summed in
// a fixed order at the end, so the result is deterministic.  A slot's loads of
// kBatch partitions are all issued before any is used (one memory round trip
// per batch, not per partition).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceParams a) {
  constexpr int TPR = D / 4;             // threads per partial row (4 columns each)
  constexpr int SLOTS = kThreads / TPR;  // partitions in flight per pass
  __shared__ float s_red[kThreads / 64];
  __shared__ float4 s_acc[SLOTS][TPR];
  __shared__ float s_w[SLOTS];

  const int tid = threadIdx.x;
  const size_t rr = blockIdx.x;  // (b * q_len + j) * n_h + h
  const int b = (int)(rr / ((size_t)a.q_len * a.n_h));
  int L = a.lens[b];
  const int Lmax = a.max_blocks * kBlockTokens;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

  const float* __restrict__ m = a.ws_m + rr * a.num_parts;
  const float* __restrict__ l = a.ws_l + rr * a.num_parts;
  const float4* __restrict__ o = reinterpret_cast<const float4*>(a.ws_o + rr * a.num_parts * D);

  // M: each thread's partitions, then the wave, then the waves (max is exact in any order)
  float M = kNegInf;
  for (int p = tid; p < nparts; p += kThreads) M = fmaxf(M, m[p]);
  M = wave_max(M);
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = s_red[0];
#pragma unroll
  for (int u = 1; u < kThreads / 64; ++u) M = fmaxf(M, s_red[u]);

  const int slot = tid / TPR, cg = tid % TPR;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.0f;
  if (M != kNegInf) {
    for (int p0 = slot; p0 < nparts; p0 += SLOTS * kBatch) {
      float mm[kBatch], ll[kBatch];
      float4 x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = p0 + SLOTS * u;
        mm[u] = kNegInf;
        ll[u] = 0.0f;
        x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p < nparts) {
          mm[u] = m[p];
          ll[u] = l[p];
          x[u] = o[(size_t)p * TPR + cg];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (p0 + SLOTS * u < nparts) {
          const float f = ll[u] * fast_exp2(mm[u] - M);
          acc.x = fmaf(f, x[u].x, acc.x);
          acc.y = fmaf(f, x[u].y, acc.y);
          acc.z = fmaf(f, x[u].z, acc.z);
          acc.w = fmaf(f, x[u].w, acc.w);
          wsum += f;
        }
      }
    }
  }
  s_acc[slot][cg] = acc;
  if (cg == 0) s_w[slot] = wsum;
  __syncthreads();

  if (tid < TPR) {
    float4 t = s_acc[0][tid];
    float wt = s_w[0];
#pragma unroll
    for (int u = 1; u < SLOTS; ++u) {
      const float4 x = s_acc[u][tid];
      t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
      wt += s_w[u];
    }
    const float inv_ok = wt > 0.0f ? 1.0f : 0.0f;
    float res[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = inv_ok != 0.0f ? res[e] / wt : 0.0f;
    if constexpr (sizeof(T) == 4) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + rr * D) + tid;
      *dst = make_float4(res[0], res[1], res[2], res[3]);
    } else {
      uint2 packed;
      packed.x = f32_to_bf16_bits(res[0]) | (f32_to_bf16_bits(res[1]) << 16);
      packed.y = f32_to_bf16_bits(res[2]) | (f32_to_bf16_bits(res[3]) << 16);
      *(reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + rr * D) + tid) = packed;
    }
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, ElemType t, int head_dim, hipStream_t s) {
  const size_t rows = (size_t)p.num_seqs * p.q_len * p.n_h;
  dim3 grid((unsigned)rows), block(kThreads);
  if (t == kF32) {
    if (head_dim == 64) hipLaunchKernelGGL((reduce_kernel<float, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((reduce_kernel<float, 128>), grid, block, 0, s, p);
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((reduce_kernel<uint16_t, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((reduce_kernel<uint16_t, 128>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace pa
