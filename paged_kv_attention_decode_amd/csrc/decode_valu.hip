// Paged decode attention on the vector ALUs, for up to 8 query rows per KV head.
//
// What is computed (see include/pa.h): for every sequence b, KV head g and
// query row r = j * group + hh (query token j, head h = g * group + hh),
//   out = sum_t softmax_t(scale * q . k_t) v_t   over visible positions t,
// reading K and V through the block table one 16-token block at a time
// ("LLM serving: KV cache, batching, paged attention and quantization",
// section 3.5), with one load of each K/V row serving every query row of the
// GQA group (section 3.3, intensity n_h / n_kv).
//
// Work decomposition: one workgroup of 4 waves per (partition, KV head,
// sequence).  The partition's blocks are dealt to the waves round-robin.
//
// Lane layouts inside a wave (bf16, head_dim 128; other shapes scale alike):
//   scores  4 lanes per token, 16 tokens = one block per pass; each lane owns
//           4 of the 16 sixteen-byte chunks of the token's row and dots them
//           with the same chunks of every query row (v_dot2_f32_bf16), then a
//           quad DPP reduction leaves the full score in all 4 lanes.
//   values  16 lanes per token, 4 tokens per pass, 4 passes per block; each
//           lane owns one chunk (8 columns) and accumulates p * v for every
//           query row.  The weights p move from the score layout to the value
//           layout through a 16 x rows LDS tile.
// Both loads are 16 bytes per lane; the four lanes (scores) or sixteen lanes
// (values) of a token read contiguous bytes of its row.
//
// Online softmax (lourdhu02.github.io "07 - Inference", section 5.1: running
// max m, running sum l, rescaled accumulator; normalized once at the end,
// section 5.2).  Scores are kept in log2 units (scale * log2 e folded in) so
// the exponential is v_exp_f32.  The running max is only raised when a score
// exceeds it by more than kRescaleSlack, a wave-uniform test (ballot); below
// that the weights stay <= 2^kRescaleSlack and no rescale is needed.  The
// result is the same softmax: numerator and denominator carry the same factor.
//
// The partition's partial (m, l, acc) per wave is merged across the 4 waves in
// LDS; a split call stores the normalized partial and (m, l) for pa_reduce
// (section 5.3 "Decode attention and FlashDecoding"), a single pass writes
// the output.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr float kRescaleSlack = 8.0f;
// buffer descriptor word 3 for the gfx9 family (raw 32-bit access, no swizzle)
constexpr int kBufferWord3 = 0x00020000;

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;
};

template <typename T>
__device__ __forceinline__ void store_out(T* dst, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* dst, float x) { *dst = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* dst, float x) { *dst = (uint16_t)f32_to_bf16_bits(x); }

template <typename T, int D, int R>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(DecodeParams a) {
  constexpr bool kBF16 = sizeof(T) == 2;
  constexpr int EPC = Elem<T>::kPer16B;  // elements per 16-byte chunk
  constexpr int NC = D / EPC;            // chunks per head row
  constexpr int NCK = NC / 4;            // score layout: chunks per lane
  constexpr int TPV = 64 / NC;           // value layout: tokens per pass
  constexpr int NV = kBlockTokens / TPV; // value layout: passes per block
  static_assert(NC % 4 == 0 && 64 % NC == 0 && kBlockTokens % TPV == 0, "unsupported head layout");

  __shared__ float s_p[kWaves][kBlockTokens][R];
  __shared__ float s_m[kWaves][R];
  __shared__ float s_l[kWaves][R];
  __shared__ float s_acc[kWaves][R][D];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const bool split = a.part_blocks > 0;

  int L = a.lens[b];
  const int Lmax = a.max_blocks * kBlockTokens;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
  const int pb = split ? a.part_blocks : nblk;
  const int blk_begin = part * pb;
  const int blk_end = min(blk_begin + pb, nblk);
  const int rows = a.group * a.q_len;

  const T* __restrict__ qp = static_cast<const T*>(a.q);
  T* __restrict__ op = static_cast<T*>(a.out);

  if (blk_begin >= nblk) {
    // split: the partition holds no token and pa_reduce never reads it.
    // single pass with an empty context: every row is zero.
    if (!split) {
      for (int idx = threadIdx.x; idx < rows * D; idx += kWaves * 64) {
        const int r = idx / D, c = idx % D;
        const int j = r / a.group, hh = r % a.group;
        const size_t orow = ((size_t)b * a.q_len + j) * a.n_h + (size_t)g * a.group + hh;
        store_out<T>(op + orow * D + c, 0.0f);
      }
    }
    return;
  }

  // ---- per-row constants and the query rows in registers (score layout) ----
  const int tk = lane >> 2;  // token of this lane in the score layout
  const int kq = lane & 3;   // chunk phase of this lane in the score layout
  const int vch = lane % NC; // chunk of this lane in the value layout
  const int tv = lane / NC;  // token phase of this lane in the value layout

  int vis[R];
  uint4 qv[R][NCK];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = r / a.group, hh = r % a.group;
    vis[r] = r < rows ? L - a.q_len + j + 1 : 0;
#pragma unroll
    for (int c = 0; c < NCK; ++c) qv[r][c] = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      const T* qrow = qp + (((size_t)b * a.q_len + j) * a.n_h + (size_t)g * a.group + hh) * D;
#pragma unroll
      for (int c = 0; c < NCK; ++c) qv[r][c] = *reinterpret_cast<const uint4*>(qrow + (kq + 4 * c) * EPC);
    }
  }

  float mref[R], lsum[R], acc[R][EPC];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    mref[r] = kNegInf;
    lsum[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[r][e] = 0.0f;
  }

  // K/V rows are read with buffer loads: the descriptor (wave-uniform) points at
  // one physical block, the per-lane byte offsets never change.  A descriptor
  // with no records makes every load of an invalid or past-the-end block
  // return zeros without touching memory, so the next block's loads can be
  // issued unconditionally and the wait counts stay exact.
  const uint32_t tok_bytes = (uint32_t)a.n_kv * D * sizeof(T);
  const uint32_t blk_bytes = tok_bytes * kBlockTokens;
  const uint32_t head_off = (uint32_t)g * D * sizeof(T);
  const uint32_t k_off = (uint32_t)tk * tok_bytes + head_off + (uint32_t)kq * 16;
  const uint32_t v_off = (uint32_t)tv * tok_bytes + head_off + (uint32_t)vch * 16;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const int32_t* __restrict__ table = a.tables + (size_t)b * a.max_blocks;
  const float scale_log2 = a.scale_log2;

  // this wave's blocks: blk_begin + w + kWaves * k
  const int n_mine = (blk_end - blk_begin - w + kWaves - 1) / kWaves;

  for (int k0 = 0; k0 < n_mine; k0 += 64) {
    const int cnt = min(64, n_mine - k0);
    const int ids = lane < cnt ? table[blk_begin + w + kWaves * (k0 + lane)] : 0;

    auto issue = [&](int kk, uint4(&kb)[NCK], uint4(&vb)[NV], int& lblk, bool& ok) {
      const int phys = __builtin_amdgcn_readlane(ids, kk < cnt ? kk : 0);
      ok = kk < cnt && (unsigned)phys < (unsigned)a.num_blocks;
      lblk = blk_begin + w + kWaves * (k0 + kk);
      const size_t boff = ok ? (size_t)phys * blk_bytes : 0;
      const uint32_t nrec = ok ? blk_bytes : 0u;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + boff), (short)0, (int)nrec, kBufferWord3);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + boff), (short)0, (int)nrec, kBufferWord3);
#pragma unroll
      for (int c = 0; c < NCK; ++c)
        kb[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off + 64 * c, 0, 0));
#pragma unroll
      for (int i = 0; i < NV; ++i)
        vb[i] = __builtin_bit_cast(uint4,
                                   __builtin_amdgcn_raw_buffer_load_b128(vr, v_off, i * TPV * tok_bytes, 0));
    };

    auto compute = [&](const uint4(&kb)[NCK], const uint4(&vb)[NV], int lblk, bool ok) {
      // scores of this lane's token for every row, log2 units
      float s[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float x = 0.0f;
#pragma unroll
        for (int c = 0; c < NCK; ++c) {
          if constexpr (kBF16) {
            x = dot2_bf16(qv[r][c].x, kb[c].x, x);
            x = dot2_bf16(qv[r][c].y, kb[c].y, x);
            x = dot2_bf16(qv[r][c].z, kb[c].z, x);
            x = dot2_bf16(qv[r][c].w, kb[c].w, x);
          } else {
            x = fmaf(__builtin_bit_cast(float, qv[r][c].x), __builtin_bit_cast(float, kb[c].x), x);
            x = fmaf(__builtin_bit_cast(float, qv[r][c].y), __builtin_bit_cast(float, kb[c].y), x);
            x = fmaf(__builtin_bit_cast(float, qv[r][c].z), __builtin_bit_cast(float, kb[c].z), x);
            x = fmaf(__builtin_bit_cast(float, qv[r][c].w), __builtin_bit_cast(float, kb[c].w), x);
          }
        }
        s[r] = quad_sum(x) * scale_log2;
      }
      const int pos = lblk * kBlockTokens + tk;
      bool raise = false;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s[r] = (ok && pos < vis[r]) ? s[r] : kNegInf;
        raise |= s[r] > mref[r] + kRescaleSlack;
      }
      if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float mnew = fmaxf(mref[r], wave_max(s[r]));
          if (mnew > mref[r]) {
            const float alpha = fast_exp2(mref[r] - mnew);
            lsum[r] *= alpha;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[r][e] *= alpha;
            mref[r] = mnew;
          }
        }
      }
      float p[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        p[r] = fast_exp2(s[r] - (mref[r] == kNegInf ? 0.0f : mref[r]));
        lsum[r] += p[r];
      }
      if (kq == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) s_p[w][tk][r] = p[r];
      }
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int tok = tv + TPV * i;
        float pr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) pr[r] = s_p[w][tok][r];
        float vf[EPC];
        if constexpr (kBF16) {
          vf[0] = bf16_lo(vb[i].x); vf[1] = bf16_hi(vb[i].x);
          vf[2] = bf16_lo(vb[i].y); vf[3] = bf16_hi(vb[i].y);
          vf[4] = bf16_lo(vb[i].z); vf[5] = bf16_hi(vb[i].z);
          vf[6] = bf16_lo(vb[i].w); vf[7] = bf16_hi(vb[i].w);
        } else {
          vf[0] = __builtin_bit_cast(float, vb[i].x); vf[1] = __builtin_bit_cast(float, vb[i].y);
          vf[2] = __builtin_bit_cast(float, vb[i].z); vf[3] = __builtin_bit_cast(float, vb[i].w);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[r][e] = fmaf(pr[r], vf[e], acc[r][e]);
      }
      wave_lds_sync();
    };

    // two register sets in flight: block kk computes while kk + 1 loads
    uint4 kA[NCK], vA[NV], kB[NCK], vB[NV];
    int lA = 0, lB = 0;
    bool okA = false, okB = false;
    issue(0, kA, vA, lA, okA);
    issue(1, kB, vB, lB, okB);
    for (int kk = 0; kk < cnt; kk += 2) {
      compute(kA, vA, lA, okA);
      issue(kk + 2, kA, vA, lA, okA);
      if (kk + 1 < cnt) compute(kB, vB, lB, okB);
      issue(kk + 3, kB, vB, lB, okB);
    }
  }

  // ---- wave totals: l over the 16 tokens (each held by 4 lanes), acc over the value token phases
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float lw = wave_sum(lsum[r]) * 0.25f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      float x = acc[r][e];
#pragma unroll
      for (int off = NC; off < 64; off <<= 1) x += shfl_xor(x, off);
      acc[r][e] = x;
    }
    if (lane == 0) {
      s_m[w][r] = mref[r];
      s_l[w][r] = lw;
    }
    if (lane < NC) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) s_acc[w][r][lane * EPC + e] = acc[r][e];
    }
  }
  __syncthreads();

  // ---- merge the 4 waves, then normalize (single pass) or store the partial (split)
  for (int idx = threadIdx.x; idx < rows * D; idx += kWaves * 64) {
    const int r = idx / D, c = idx % D;
    float M = s_m[0][r];
#pragma unroll
    for (int u = 1; u < kWaves; ++u) M = fmaxf(M, s_m[u][r]);
    float o = 0.0f, l = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int u = 0; u < kWaves; ++u) {
        const float f = fast_exp2(s_m[u][r] - M);
        l += f * s_l[u][r];
        o += f * s_acc[u][r][c];
      }
    }
    const float res = l > 0.0f ? o / l : 0.0f;
    const int j = r / a.group, hh = r % a.group;
    const size_t orow = ((size_t)b * a.q_len + j) * a.n_h + (size_t)g * a.group + hh;
    if (split) {
      const size_t pi = orow * a.num_parts + part;
      a.ws_o[pi * D + c] = res;
      if (c == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = l;
      }
    } else {
      store_out<T>(op + orow * D + c, res);
    }
  }
}

template <typename T, int D, int R>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
  dim3 grid(p.part_blocks > 0 ? p.num_parts : 1, p.n_kv, p.num_seqs);
  hipLaunchKernelGGL((decode_valu_kernel<T, D, R>), grid, dim3(kWaves * 64), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rows(const DecodeParams& p, int rows, hipStream_t s) {
  if (rows <= 1) return launch_one<T, D, 1>(p, s);
  if (rows <= 2) return launch_one<T, D, 2>(p, s);
  if (rows <= 4) return launch_one<T, D, 4>(p, s);
  return launch_one<T, D, 8>(p, s);
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, ElemType t, int head_dim, int rows_per_kv, hipStream_t s) {
  if (t == kF32) {
    return head_dim == 64 ? launch_rows<float, 64>(p, rows_per_kv, s) : launch_rows<float, 128>(p, rows_per_kv, s);
  }
  return head_dim == 64 ? launch_rows<uint16_t, 64>(p, rows_per_kv, s) : launch_rows<uint16_t, 128>(p, rows_per_kv, s);
}

}  // namespace pa
