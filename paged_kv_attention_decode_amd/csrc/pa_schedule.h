// How a decode launch divides (sequence, KV head, block) work among its
// workgroups, and where each workgroup's result goes.  Shared by the decode
// kernels; each kernel supplies an "attender" object:
//
//   static constexpr int kThreads, kD;
//   void  run(int b, int g, int L, int lo, int hi);  // blocks [lo, hi) of sequence b, KV head g;
//                                                   // all threads; ends with a barrier
//   float result(int r, int c, float& M, float& l);  // merged row r, column c: the normalized
//                                                   // output, its max M (log2 units) and sum l
//   void  store(size_t idx, float x);                // out[idx] = x in the output type
//
// Modes:
//   single pass  one workgroup per (KV head, sequence) over the whole context;
//   partitions   one workgroup per (partition, KV head, sequence); the partial
//                (m, l, o) of every query row goes to the workspace for pa_reduce
//                (FlashDecoding's split, "07 - Inference", lourdhu02.github.io,
//                section 5.3);
//   balanced     the flattened list of (sequence, KV head, block) work is cut into
//                equal contiguous ranges, one per workgroup, so every workgroup
//                (and every CU) streams the same number of blocks whatever the
//                context lengths.  A (sequence, head) that one range covers whole
//                is written directly; one cut between ranges leaves a partial
//                (m, l, o) per piece, and the last workgroup to finish a piece
//                (an arrival counter per (sequence, head)) merges the pieces in
//                their fixed order with the same rescaling rule and resets the
//                counter, so results do not depend on arrival order.
#pragma once

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

__device__ __forceinline__ int clamped_len(const DecodeParams& a, int b) {
  const int L = a.lens[b];
  const int Lmax = a.max_blocks * kBlockTokens;
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

__device__ __forceinline__ int blocks_of(int L) { return (L + kBlockTokens - 1) / kBlockTokens; }

// stores and loads that are coherent across the whole device (all XCDs)
__device__ __forceinline__ void coherent_store(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// output row of query row r = j * group + hh of sequence b, KV head g
__device__ __forceinline__ size_t out_row(const DecodeParams& a, int b, int g, int r) {
  const int j = r / a.group, hh = r % a.group;
  return ((size_t)b * a.q_len + j) * a.n_h + (size_t)g * a.group + hh;
}

template <class Attn>
__device__ void write_final(const DecodeParams& a, Attn& at, int b, int g) {
  const int rows = a.group * a.q_len;
  for (int idx = threadIdx.x; idx < rows * Attn::kD; idx += Attn::kThreads) {
    const int r = idx / Attn::kD, c = idx % Attn::kD;
    float M, l;
    const float res = at.result(r, c, M, l);
    at.store(out_row(a, b, g, r) * Attn::kD + c, res);
  }
}

template <class Attn>
__device__ void write_zeros(const DecodeParams& a, Attn& at, int b, int g) {
  const int rows = a.group * a.q_len;
  for (int idx = threadIdx.x; idx < rows * Attn::kD; idx += Attn::kThreads) {
    const int r = idx / Attn::kD, c = idx % Attn::kD;
    at.store(out_row(a, b, g, r) * Attn::kD + c, 0.0f);
  }
}

// ---- single pass and partitions: grid (partitions or 1, n_kv, num_seqs)

template <class Attn>
__device__ void drive_fixed(const DecodeParams& a, Attn& at) {
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = clamped_len(a, b);
  const int nblk = blocks_of(L);
  if (a.mode == kSinglePass) {
    if (nblk == 0) {
      write_zeros(a, at, b, g);
      return;
    }
    at.run(b, g, L, 0, nblk);
    write_final(a, at, b, g);
    return;
  }
  const int lo = part * a.part_blocks;
  if (lo >= nblk) return;  // no token in this partition; pa_reduce never reads it
  at.run(b, g, L, lo, min(lo + a.part_blocks, nblk));
  const int rows = a.group * a.q_len;
  for (int idx = threadIdx.x; idx < rows * Attn::kD; idx += Attn::kThreads) {
    const int r = idx / Attn::kD, c = idx % Attn::kD;
    float M, l;
    const float res = at.result(r, c, M, l);
    const size_t pi = out_row(a, b, g, r) * a.num_parts + part;
    a.ws_o[pi * Attn::kD + c] = res;
    if (c == 0) {
      a.ws_m[pi] = M;
      a.ws_l[pi] = l;
    }
  }
}

// ---- balanced: grid (num_wgs)

// the workgroup whose range holds flat block x: largest w with floor(w T / W) <= x
__device__ __forceinline__ int range_of(long long x, long long T, int W) {
  return (int)(((x + 1) * W + T - 1) / T) - 1;
}

template <class Attn>
__device__ void drive_balanced(const DecodeParams& a, Attn& at) {
  __shared__ int s_prefix[kBalancedMaxSeqs + 1];  // blocks of sequences before b
  __shared__ int s_scan[Attn::kThreads];
  __shared__ int s_last;
  const int S = a.num_seqs, W = a.num_wgs, wid = blockIdx.x, tid = threadIdx.x;
  constexpr int NT = Attn::kThreads;

  // block prefix over the sequences (contexts clamped like everywhere else)
  const int per = (S + NT - 1) / NT;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < S) sum += blocks_of(clamped_len(a, b));
  }
  s_scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? s_scan[tid - 1] : 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < S) {
      s_prefix[b] = run;
      run += blocks_of(clamped_len(a, b));
    }
  }
  if (tid == NT - 1) s_prefix[S] = s_scan[NT - 1];
  __syncthreads();

  // sequences with an empty context: zero rows, spread over the workgroups
  for (int b = wid; b < S; b += W) {
    if (s_prefix[b + 1] == s_prefix[b]) {
      for (int g = 0; g < a.n_kv; ++g) write_zeros(a, at, b, g);
    }
  }

  const long long T = (long long)a.n_kv * s_prefix[S];
  if (T == 0) return;
  // ranges [floor(w T / Wr), floor((w + 1) T / Wr)); with Wr <= T none is empty,
  // so the pieces of a cut (sequence, head) come from consecutive workgroups
  const int Wr = T < W ? (int)T : W;
  if (wid >= Wr) return;
  const long long B0 = (long long)wid * T / Wr, B1 = (long long)(wid + 1) * T / Wr;

  // the sequence holding flat block B0: largest b with n_kv * prefix[b] <= B0
  const int X = (int)(B0 / a.n_kv);
  int lo = 0, hi = S;  // invariant: prefix[lo] <= X < prefix[hi] (prefix[S] > X since B0 < T)
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (s_prefix[mid] <= X) lo = mid;
    else hi = mid;
  }
  int b = lo;
  int nb = s_prefix[b + 1] - s_prefix[b];
  int g = (int)((B0 - (long long)a.n_kv * s_prefix[b]) / nb);
  const int rows = a.group * a.q_len;
  const size_t piece_stride = (size_t)rows * (Attn::kD + 2);

  while (true) {
    const long long seg0 = (long long)a.n_kv * s_prefix[b] + (long long)g * nb;  // flat index of block 0
    const long long seg1 = seg0 + nb;
    const int blo = (int)((B0 > seg0 ? B0 : seg0) - seg0);
    const int bhi = (int)((B1 < seg1 ? B1 : seg1) - seg0);
    at.run(b, g, clamped_len(a, b), blo, bhi);
    if (blo == 0 && bhi == nb) {
      write_final(a, at, b, g);
    } else {
      // a piece: store the partial, then the last arrival merges all pieces
      const int slot = seg0 > B0 ? 2 * wid + 1 : 2 * wid;
      float* mine = a.pieces + (size_t)slot * piece_stride;
      // The partial goes out with device-coherent stores (written through to
      // the point of coherence of all XCDs) and every wave waits for them
      // before the barrier, so the arrival below is ordered after them without
      // writing back or invalidating a whole L2 (release/acquire fences at
      // device scope do that, which costs far more than the kernel's work).
      for (int idx = tid; idx < rows * Attn::kD; idx += NT) {
        const int r = idx / Attn::kD, c = idx % Attn::kD;
        float M, l;
        const float res = at.result(r, c, M, l);
        coherent_store(mine + (size_t)r * (Attn::kD + 2) + c, res);
        if (c == 0) {
          coherent_store(mine + (size_t)r * (Attn::kD + 2) + Attn::kD, M);
          coherent_store(mine + (size_t)r * (Attn::kD + 2) + Attn::kD + 1, l);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
      __syncthreads();
      const int first = range_of(seg0, T, Wr), last = range_of(seg1 - 1, T, Wr);
      const int npieces = last - first + 1;
      if (tid == 0) {
        int* cnt = a.counters + (size_t)b * a.n_kv + g;
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int is_last = old == npieces - 1;
        if (is_last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = is_last;
      }
      __syncthreads();
      if (s_last) {
        // the other pieces, read with device-coherent loads (past any stale cache line)
        for (int idx = tid; idx < rows * Attn::kD; idx += NT) {
          const int r = idx / Attn::kD, c = idx % Attn::kD;
          float M = kNegInf;
          for (int k = 0; k < npieces; ++k) {
            const int w2 = first + k;
            const int sl = (k == 0 && seg0 > (long long)w2 * T / Wr) ? 2 * w2 + 1 : 2 * w2;
            M = fmaxf(M, coherent_load(a.pieces + (size_t)sl * piece_stride + (size_t)r * (Attn::kD + 2) + Attn::kD));
          }
          float o = 0.0f, l = 0.0f;
          if (M != kNegInf) {
            for (int k = 0; k < npieces; ++k) {
              const int w2 = first + k;
              const int sl = (k == 0 && seg0 > (long long)w2 * T / Wr) ? 2 * w2 + 1 : 2 * w2;
              const float* pc = a.pieces + (size_t)sl * piece_stride + (size_t)r * (Attn::kD + 2);
              const float f = coherent_load(pc + Attn::kD + 1) * fast_exp2(coherent_load(pc + Attn::kD) - M);
              o += f * coherent_load(pc + c);
              l += f;
            }
          }
          at.store(out_row(a, b, g, r) * Attn::kD + c, l > 0.0f ? o / l : 0.0f);
        }
      }
      __syncthreads();
    }
    if (seg1 >= B1) break;
    // next (sequence, head) with blocks
    if (++g == a.n_kv) {
      g = 0;
      do {
        ++b;
      } while (s_prefix[b + 1] == s_prefix[b]);
      nb = s_prefix[b + 1] - s_prefix[b];
    }
  }
}

}  // namespace pa
