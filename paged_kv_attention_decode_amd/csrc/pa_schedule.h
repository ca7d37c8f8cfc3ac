// How a decode launch divides (sequence, KV head, block) work among its
// workgroups, and where each workgroup's result goes.  Shared by the decode
// kernels; each kernel supplies an "attender" object:
//
//   static constexpr int kThreads, kD;
//   void  run(int b, int g, int L, int lo, int hi);  // blocks [lo, hi) of sequence b, KV head g;
//                                                   // all threads; ends with a barrier
//   float result(int r, int c, float& M, float& l);  // merged row r, column c: the normalized
//                                                   // output, its max M (log2 units) and sum l
//   void  result8(int r, int c0, float (&x)[8]);     // result() of columns c0 .. c0 + 7
//   void  store8(size_t idx, const float (&x)[8]);   // out[idx .. idx + 7] = x
//   void  store(size_t idx, float x);                // out[idx] = x in the output type
//
// Modes:
//   single pass  one workgroup per (KV head, sequence) over the whole context;
//   partitions   one workgroup per (partition, KV head, sequence); the partial
//                (m, l, o) of every query row goes to the workspace for pa_reduce
//                (FlashDecoding's split, "07 - Inference", lourdhu02.github.io,
//                section 5.3);
//   balanced     the flattened list of (sequence, block) work is cut into equal
//                contiguous ranges; each range goes to num_kv_heads adjacent
//                workgroups, one per KV head, so every workgroup (and every CU)
//                streams the same number of blocks whatever the context lengths,
//                and the heads of one token row are read close together in time
//                (one DRAM page instead of num_kv_heads scattered visits).  A
//                (sequence, head) that one range covers whole is written
//                directly; one cut between ranges leaves a partial (m, l, o) per
//                piece, and the last workgroup to finish a piece (an arrival
//                counter per (sequence, head)) merges the pieces in their fixed
//                order with the same rescaling rule and resets the counter, so
//                results do not depend on arrival order.
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

// the merged output rows, 8 columns per thread and step (one 16-byte store of bf16)
template <class Attn>
__device__ void write_final(const DecodeParams& a, Attn& at, int b, int g) {
  constexpr int CV = Attn::kD / 8;
  const int rows = a.group * a.q_len;
  for (int idx = threadIdx.x; idx < rows * CV; idx += Attn::kThreads) {
    const int r = idx / CV, c0 = 8 * (idx % CV);
    float x[8];
    at.result8(r, c0, x);
    at.store8(out_row(a, b, g, r) * Attn::kD + c0, x);
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

// largest batch whose one-pass launch runs the longest sequences first
constexpr int kLongestFirstMaxSeqs = 256;

// The sequence of rank z in descending block count (ties by index).  The
// hardware hands out workgroups in launch order; when the grid needs more
// than one round of resident workgroups, starting the longest sequences first
// keeps a long one from starting last and running alone at the end (longest
// processing time first).  Every workgroup ranks the whole batch in LDS, which
// costs O(S^2 / threads) compares, so only batches up to
// kLongestFirstMaxSeqs are reordered.
template <int NT>
__device__ int sequence_of_rank(const DecodeParams& a, int z) {
  __shared__ int s_blocks[kLongestFirstMaxSeqs];
  __shared__ int s_pick;
  const int S = a.num_seqs;
  for (int i = threadIdx.x; i < S; i += NT) s_blocks[i] = blocks_of(clamped_len(a, i));
  __syncthreads();
  for (int c = threadIdx.x; c < S; c += NT) {
    const int mine = s_blocks[c];
    int rank = 0;
    for (int i = 0; i < S; ++i) {
      const int o = s_blocks[i];
      rank += (o > mine) | ((o == mine) & (i < c));
    }
    if (rank == z) s_pick = c;
  }
  __syncthreads();
  return s_pick;
}

// pa_decode_append: before a workgroup reads blocks [blo, bhi) of sequence b
// for KV head g, it stores the new tokens that fall in them.  New token j of
// sequence b sits at position L - q_len + j, in slot 16 * table[b][pos / 16] +
// pos % 16 (the sequence's own block table: tokens are appended in place);
// positions before 0 and blocks outside the pool are skipped.  Each (block,
// KV head) slice is read by exactly one wave in every schedule: wave w of the
// workgroup owning the block reads blocks blo + w + NW k.  That wave stores
// the new tokens of its blocks here, before it issues any load, and a wave's
// memory operations reach memory in the order it issues them, so its loads
// see the stores without a wait, a barrier, or any other wave involved.
template <int NT>
__device__ void append_new_tokens(const DecodeParams& a, int b, int g, int L, int blo, int bhi) {
  constexpr int NW = NT / 64;
  const int first = L - a.q_len;  // position of new token 0
  const int blk0 = (first < 0 ? 0 : first) / kBlockTokens, blk1 = (L - 1) / kBlockTokens;
  if (L <= 0 || blk1 < blo || blk0 >= bhi) return;  // no new token in these blocks (wave-uniform)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunks = a.append_row_bytes / 16;
  const size_t tok_bytes = (size_t)a.n_kv * a.append_row_bytes;
  for (int idx = lane; idx < a.q_len * 2 * chunks; idx += 64) {
    const int j = idx / (2 * chunks), kv = (idx / chunks) & 1, c = idx % chunks;
    const int pos = first + j;
    if (pos < 0) continue;
    const int blk = pos / kBlockTokens;
    if (blk < blo || blk >= bhi || (blk - blo) % NW != w) continue;  // another wave's block
    const int phys = a.tables[(size_t)b * a.max_blocks + blk];
    if ((unsigned)phys >= (unsigned)a.num_blocks) continue;
    const char* src = static_cast<const char*>(kv ? a.new_v : a.new_k) +
                      ((size_t)(b * a.q_len + j) * a.n_kv + g) * a.append_row_bytes + 16 * c;
    char* dst = static_cast<char*>(const_cast<void*>(kv ? a.v_cache : a.k_cache)) +
                ((size_t)phys * kBlockTokens + pos % kBlockTokens) * tok_bytes + (size_t)g * a.append_row_bytes + 16 * c;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

// the length rank a one-pass workgroup slot takes: slots below the pairing
// stride P take ranks 0 .. P - 1 (the longest), the others the remaining
// ranks shortest first (S - 1 down to P), so that slot z and its CU partner
// z + P hold ranks z and S - 1 - z (one_pass_pairing in pa_kernels.h)
__device__ __forceinline__ int decode_pairing(const DecodeParams& a, int z) {
  const int P = a.pair_stride;
  return (P > 0 && z >= P) ? a.num_seqs - 1 + P - z : z;
}

template <class Attn>
__device__ void drive_fixed(const DecodeParams& a, Attn& at) {
  const int part = blockIdx.x, g = blockIdx.y;
  const int b = a.mode == kSinglePass && a.num_seqs <= kLongestFirstMaxSeqs
                    ? sequence_of_rank<Attn::kThreads>(a, decode_pairing(a, (int)blockIdx.z))
                    : (int)blockIdx.z;
  const int L = clamped_len(a, b);
  const int nblk = blocks_of(L);
  if (a.mode == kSinglePass) {
    if (nblk == 0) {
      write_zeros(a, at, b, g);
      return;
    }
    if (a.new_k && !Attn::defers_append(a)) append_new_tokens<Attn::kThreads>(a, b, g, L, 0, nblk);
    at.run(b, g, L, 0, nblk);
    write_final(a, at, b, g);
    return;
  }
  const int lo = part * a.part_blocks;
  if (lo >= nblk) return;  // no token in this partition; pa_reduce never reads it
  if (a.new_k && !Attn::defers_append(a))
    append_new_tokens<Attn::kThreads>(a, b, g, L, lo, min(lo + a.part_blocks, nblk));
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

// How T blocks are cut into W equal contiguous ranges
// [floor(r T / W), floor((r + 1) T / W)); with W <= T none is empty.
struct Ranges {
  long long T;
  int W;
  __device__ Ranges(long long T_, int W_) : T(T_), W(W_) {}
  __device__ long long start(int r) const { return (long long)r * T / W; }
  __device__ int of(long long x) const { return range_of(x, T, W); }  // the range holding block x
};

// The last arrival's merge of the npieces partials of (sequence b, head g), in
// range order: the loads of a batch of pieces are all issued before any is
// used (each goes past the caches to the point of coherence, so one at a time
// would cost a full memory round trip per piece).
template <class Attn, class SlotOf>
__device__ void merge_pieces(const DecodeParams& a, Attn& at, int b, int g, int first, int npieces,
                             bool first_at_end, SlotOf slot_of) {
  constexpr int kBatch = 8;
  const int rows = a.group * a.q_len;
  const size_t piece_stride = (size_t)rows * (Attn::kD + 2);
  for (int idx = threadIdx.x; idx < rows * Attn::kD; idx += Attn::kThreads) {
    const int r = idx / Attn::kD, c = idx % Attn::kD;
    const size_t off = (size_t)r * (Attn::kD + 2);
    float M = kNegInf;
    for (int k0 = 0; k0 < npieces; k0 += kBatch) {
      float m[kBatch], l[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        m[u] = kNegInf;
        l[u] = 0.0f;
        if (k0 + u < npieces) {
          const float* pc = a.pieces + slot_of(first + k0 + u, k0 + u == 0 && first_at_end) * piece_stride + off;
          m[u] = coherent_load(pc + Attn::kD);
          l[u] = coherent_load(pc + Attn::kD + 1);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (l[u] > 0.0f) M = fmaxf(M, m[u]);  // a piece where the row sees nothing carries no weight
    }
    float o = 0.0f, lsum = 0.0f;
    if (M != kNegInf) {
      for (int k0 = 0; k0 < npieces; k0 += kBatch) {
        float m[kBatch], l[kBatch], x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          m[u] = kNegInf;
          l[u] = 0.0f;
          x[u] = 0.0f;
          if (k0 + u < npieces) {
            const float* pc = a.pieces + slot_of(first + k0 + u, k0 + u == 0 && first_at_end) * piece_stride + off;
            m[u] = coherent_load(pc + Attn::kD);
            l[u] = coherent_load(pc + Attn::kD + 1);
            x[u] = coherent_load(pc + c);
          }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float f = l[u] > 0.0f ? l[u] * fast_exp2(m[u] - M) : 0.0f;
          o += f * x[u];
          lsum += f;
        }
      }
    }
    at.store(out_row(a, b, g, r) * Attn::kD + c, lsum > 0.0f ? o / lsum : 0.0f);
  }
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

  // ranges over the (sequence, block) list, one workgroup per (range, KV head)
  const int n_kv = a.n_kv;
  const long long T = s_prefix[S];
  const int Wh = W / n_kv;  // ranges
  if (T == 0 || wid >= Wh * n_kv) return;
  // ranges [floor(r T / Wr), floor((r + 1) T / Wr)); with Wr <= T none is empty,
  // so the pieces of a cut sequence come from consecutive ranges
  const int Wr = T < Wh ? (int)T : Wh;
  const int rid = wid / n_kv, g = wid % n_kv;
  if (rid >= Wr) return;
  const Ranges rg(T, Wr);
  const long long B0 = rg.start(rid), B1 = rg.start(rid + 1);

  // the sequence holding flat block B0: largest b with prefix[b] <= B0
  int lo = 0, hi = S;  // invariant: prefix[lo] <= B0 < prefix[hi] (prefix[S] > B0 since B0 < T)
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (s_prefix[mid] <= B0) lo = mid;
    else hi = mid;
  }
  int b = lo;
  const int rows = a.group * a.q_len;
  const size_t piece_stride = (size_t)rows * (Attn::kD + 2);
  // piece slots: two per workgroup, the one at its range's start and the one at its end
  auto slot_of = [&](int r, bool at_end) { return (size_t)(2 * (r * n_kv + g) + (at_end ? 1 : 0)); };

  // a piece's arrival: wait until this workgroup's stores are complete, count
  // it, and let the last of its pieces merge them all
  auto arrive = [&](int bb, long long seg0, long long seg1) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __syncthreads();
    const int first = rg.of(seg0), last = rg.of(seg1 - 1);
    const int npieces = last - first + 1;
    if (tid == 0) {
      int* cnt = a.counters + (size_t)bb * n_kv + g;
      const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int is_last = old == npieces - 1;
      if (is_last) {
        __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the merge's loads come after every other piece's arrival: an
        // agent-scope acquire (an invalidate of this CU's caches, cheap, and
        // a compiler barrier), which the workgroup barrier below extends to
        // the other threads
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      s_last = is_last;
    }
    __syncthreads();
    if (s_last) merge_pieces(a, at, bb, g, first, npieces, seg0 > rg.start(first), slot_of);
    __syncthreads();
  };

  // the sequence holding flat block B1 - 1 (the range's last)
  int b_last = b;
  {
    int l2 = b, h2 = S;  // prefix[l2] <= B1 - 1 < prefix[h2]
    while (h2 - l2 > 1) {
      const int mid = (l2 + h2) / 2;
      if (s_prefix[mid] <= B1 - 1) l2 = mid;
      else h2 = mid;
    }
    b_last = l2;
  }

  // one sequence's share of the range: written out when whole, published as a piece when cut
  auto one = [&](int bb) {
    const long long seg0 = s_prefix[bb], seg1 = s_prefix[bb + 1];
    const int nb = (int)(seg1 - seg0);
    const int blo = (int)((B0 > seg0 ? B0 : seg0) - seg0);
    const int bhi = (int)((B1 < seg1 ? B1 : seg1) - seg0);
    if (a.new_k && !Attn::defers_append(a)) append_new_tokens<NT>(a, bb, g, clamped_len(a, bb), blo, bhi);
    at.run(bb, g, clamped_len(a, bb), blo, bhi);
    if (blo == 0 && bhi == nb) {
      write_final(a, at, bb, g);
    } else {
      // a piece: its partial goes out with device-coherent stores (written
      // through to the point of coherence of all XCDs) and its arrival is
      // ordered after them by waiting for the stores, not by a device-scope
      // release fence, which would write back a whole L2.  Arriving at once
      // (rather than at the range's end) keeps the round trips in the middle
      // of the range, where the CU's other workgroup keeps the memory busy.
      float* mine = a.pieces + slot_of(rid, seg0 > B0) * piece_stride;
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
      arrive(bb, seg0, seg1);
    }
  };

  // Order: the cut piece at the range's end first, then the one at its
  // start, then the whole sequences between.  A cut sequence's two pieces
  // are then both done early by their workgroups, so the publication round
  // trips and the last arrival's merge overlap streaming instead of adding to
  // every workgroup's tail, which ends on plain writes.
  // (one call site, so the attention body is instantiated once)
  const bool end_cut = b_last != b && s_prefix[b_last + 1] > B1;
  int phase = end_cut ? 0 : 1, cur = b;
  while (true) {
    int bb;
    if (phase == 0) {  // the end piece
      bb = b_last;
      phase = 1;
    } else if (phase == 1) {  // the first sequence
      bb = b;
      phase = 2;
    } else if (phase == 2) {  // the sequences between, skipping empty contexts
      do {
        ++cur;
      } while (cur < b_last && s_prefix[cur + 1] == s_prefix[cur]);
      if (cur >= b_last) {
        phase = 3;
        continue;
      }
      bb = cur;
    } else if (phase == 3 && b_last != b && !end_cut) {  // the last sequence, whole or cut at the start
      bb = b_last;
      phase = 4;
    } else {
      break;
    }
    one(bb);
  }
}

}  // namespace pa
