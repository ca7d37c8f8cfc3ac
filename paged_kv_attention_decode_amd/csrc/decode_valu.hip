// Paged decode attention on the vector ALUs, for up to 8 query rows per KV head.
//
// What is computed (contract in include/pa.h): for every sequence b, KV head g
// and query row r = j * group + hh (query token j, head h = g * group + hh),
//   out = sum_t softmax_t(scale * q . k_t) v_t   over the positions t row r sees,
// reading K and V through the block table one 16-token block at a time
// ("LLM serving: KV cache, batching, paged attention and quantization",
// section 3.5), with one load of each K/V row serving every query row of the
// GQA group (section 3.3: the intensity of decode attention is n_h / n_kv).
//
// A workgroup of NW waves attends a range of blocks of one (sequence, KV
// head); the ranges come from pa_schedule.h (single pass, partitions, or the
// balanced split).  The range's blocks are dealt to the waves round-robin.
//
// Lane layouts inside a wave (bf16, head_dim 128; other shapes scale alike):
//   scores  4 lanes per token, 16 tokens = one block per load; each lane owns
//           4 of the 16 sixteen-byte chunks of the token's row and dots them
//           with the same chunks of every query row (v_dot2_f32_bf16); a quad
//           DPP sum leaves the full score in all 4 lanes.
//   values  16 lanes per token, 4 tokens per load, 4 loads per block; each lane
//           owns one chunk (8 columns) and accumulates p * v for every query
//           row.  Load i of lane row q (lanes 16q .. 16q+15) takes token
//           4q + i, whose weights the score layout holds in lanes 16q + 4i ..
//           16q + 4i + 3 of the same row, so one DPP row_newbcast per row and
//           load moves them (other head shapes use a cross-lane permute).
//           bf16: the weights are rounded to bf16 and the tokens of loads
//           2m and 2m + 1 go through one v_dot2_f32_bf16 per column and row,
//           their column pairs formed by v_perm_b32 (the row sums add the
//           same rounded weights); fp32 multiplies one token at a time.
//
// Memory-level parallelism: K/V are read with buffer loads whose descriptor
// (wave-uniform) points at one physical block, so the per-lane offsets never
// change, and NBUF blocks are in flight per wave.  A descriptor's record count
// ends at the last context token, so rows past it (never written, possibly
// NaN) and invalid or past-the-end blocks load as zeros without touching
// memory; the next loads are therefore issued unconditionally, which keeps
// the compiler's wait counts exact.
//
// Softmax.  The pages' online softmax keeps a running max m, a running sum l
// and a rescaled accumulator, normalized once at the end ("07 - Inference",
// lourdhu02.github.io, sections 5.1 and 5.2).  Any reference value gives the
// same result as long as the weights stay in range, because numerator and
// denominator carry the same factor.  Each wave takes the exact maximum of its
// first block (log2 units, scale * log2 e folded in, v_exp_f32) as the
// reference and never moves it in the hot loop: later weights may grow up to
// 2^kOverflowSlack, which fp32 holds with full relative precision.  A score
// beyond that sets a wave-uniform flag, and after the loop the wave redoes its
// share exactly in two passes (maximum first, then the weighted sums).  The
// hot loop therefore has no rescale branch and the accumulators are only ever
// touched by FMAs.  The waves' (m, l, acc) are merged with the rescaling rule.
#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_schedule.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr float kOverflowSlack = 64.0f;  // log2 units

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
__device__ __forceinline__ void store_elem(T* dst, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float* dst, float x) { *dst = x; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* dst, float x) { *dst = (uint16_t)f32_to_bf16_bits(x); }

// pr[r] = p[r] of lane 4 * i of this lane's DPP row (row_newbcast); i is the
// value-layout load index, a compile-time constant after unrolling
template <int R>
__device__ __forceinline__ void bcast_in_row(float (&pr)[R], const float (&p)[R], int i) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    switch (i) {
      case 0: pr[r] = dpp_mov<0x150>(p[r]); break;
      case 1: pr[r] = dpp_mov<0x154>(p[r]); break;
      case 2: pr[r] = dpp_mov<0x158>(p[r]); break;
      default: pr[r] = dpp_mov<0x15C>(p[r]); break;
    }
  }
}

// x as held by lane src (any lane of the wave)
__device__ __forceinline__ float lane_from(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

template <typename T, int D, int R, int NW>
struct WaveTotals {
  float m[NW][R];
  float l[NW][R];
  alignas(16) float acc[NW][R][D];
};

template <typename T, int D, int R, int NW, int NBUF>
struct ValuAttender {
  static constexpr int kThreads = NW * 64;
  // V loads are non-temporal (cache policy nt), K loads ordinary.  Two
  // alternating runs, us: 8B layer 91.7 / 91.7 warm and 97.8 / 97.4 cold
  // against 100.4 / 100.5 and 103.0 / 103.7 with both non-temporal, and
  // 107.5-108.4 / 106.2-107.7 with neither; long contexts in 512-token
  // partitions 450.8 / 451.6 against 482.3 / 482.2 (both) and 482.5 (neither).
  static constexpr int kVPolicy = 2;
  static constexpr int kD = D;
  static constexpr bool kBF16 = sizeof(T) == 2;
  static constexpr int EPC = Elem<T>::kPer16B;     // elements per 16-byte chunk
  static constexpr int NC = D / EPC;               // chunks per head row
  static constexpr int NCK = NC / 4;               // score layout: chunks per lane
  static constexpr int TPV = 64 / NC;              // value layout: tokens per load
  static constexpr int NV = kBlockTokens / TPV;    // value layout: loads per block
  static constexpr bool kRowTokens = NC == 16;     // value load i of lane row q holds token 4q + i
  static_assert(NC % 4 == 0 && 64 % NC == 0 && kBlockTokens % TPV == 0, "unsupported head layout");

  const DecodeParams& a;
  WaveTotals<T, D, R, NW>& sm;
  const int lane, w, tk, kq, vch, tv;

  __device__ ValuAttender(const DecodeParams& a_, WaveTotals<T, D, R, NW>& sm_)
      : a(a_),
        sm(sm_),
        lane(threadIdx.x & 63),
        w(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),  // wave index, uniform
        tk((threadIdx.x & 63) >> 2),
        kq(threadIdx.x & 3),
        vch((threadIdx.x & 63) % NC),
        tv((threadIdx.x & 63) / NC) {}

  __device__ void store(size_t idx, float x) { store_elem<T>(static_cast<T*>(a.out) + idx, x); }
  // out[idx .. idx + 7] = x in the output type (idx a multiple of 8): 16 or 32 bytes
  __device__ void store8(size_t idx, const float (&x)[8]) {
    if constexpr (kBF16) {
      uint4 v;
      v.x = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
      v.y = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
      v.z = f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16);
      v.w = f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + idx) = v;
    } else {
      float* o = static_cast<float*>(a.out) + idx;
      *reinterpret_cast<float4*>(o) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
  }

  // pa_decode_append: when the new tokens' rows of one head fit one 16-byte
  // chunk per lane, this kernel stores them itself (see run); otherwise the
  // schedule stores them before run
  __device__ static bool defers_append(const DecodeParams& a) {
    return a.q_len * 2 * (a.append_row_bytes / 16) <= 64;
  }

  // merged output of row r, column c over the waves
  __device__ float result(int r, int c, float& M, float& l) const {
    M = sm.m[0][r];
#pragma unroll
    for (int u = 1; u < NW; ++u) M = fmaxf(M, sm.m[u][r]);
    float o = 0.0f;
    l = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        const float f = fast_exp2(sm.m[u][r] - M);
        l += f * sm.l[u][r];
        o += f * sm.acc[u][r][c];
      }
    }
    return l > 0.0f ? o / l : 0.0f;
  }

  // result() of columns c0 .. c0 + 7 of row r (c0 a multiple of 8): the row's
  // maximum and rescaling factors once, each wave's 8 columns in two 16-byte
  // reads, the same sums in the same order
  __device__ void result8(int r, int c0, float (&x)[8]) const {
    float M = sm.m[0][r];
#pragma unroll
    for (int u = 1; u < NW; ++u) M = fmaxf(M, sm.m[u][r]);
    float l = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        const float f = fast_exp2(sm.m[u][r] - M);
        l += f * sm.l[u][r];
        const float4 a0 = *reinterpret_cast<const float4*>(&sm.acc[u][r][c0]);
        const float4 a1 = *reinterpret_cast<const float4*>(&sm.acc[u][r][c0 + 4]);
        x[0] += f * a0.x; x[1] += f * a0.y; x[2] += f * a0.z; x[3] += f * a0.w;
        x[4] += f * a1.x; x[5] += f * a1.y; x[6] += f * a1.z; x[7] += f * a1.w;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = l > 0.0f ? x[k] / l : 0.0f;
  }

  __device__ void run(int b, int g, int L, int lo, int hi) {
    const int rows = a.group * a.q_len;

    // query rows in registers (score layout)
    const T* __restrict__ qp = static_cast<const T*>(a.q);
    uint4 qv[R][NCK];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = r / a.group, hh = r % a.group;
#pragma unroll
      for (int c = 0; c < NCK; ++c) qv[r][c] = make_uint4(0, 0, 0, 0);
      if (r < rows) {
        const T* qrow = qp + (((size_t)b * a.q_len + j) * a.n_h + (size_t)g * a.group + hh) * D;
#pragma unroll
        for (int c = 0; c < NCK; ++c) qv[r][c] = *reinterpret_cast<const uint4*>(qrow + (kq + 4 * c) * EPC);
      }
    }

    int vis[R];  // positions row r may see
#pragma unroll
    for (int r = 0; r < R; ++r) vis[r] = r < rows ? L - a.q_len + r / a.group + 1 : 0;

    float m_ref[R], m_use[R], lsum[R], acc[R][EPC];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m_ref[r] = kNegInf;
      m_use[r] = 0.0f;
      lsum[r] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[r][e] = 0.0f;
    }

    const uint32_t tok_bytes = (uint32_t)a.n_kv * D * sizeof(T);
    const uint32_t blk_bytes = tok_bytes * kBlockTokens;
    const uint32_t head_off = (uint32_t)g * D * sizeof(T);
    const uint32_t k_off = (uint32_t)tk * tok_bytes + head_off + (uint32_t)kq * 16;
    const uint32_t v_off = (uint32_t)(kRowTokens ? TPV * tv : tv) * tok_bytes + head_off + (uint32_t)vch * 16;
    const uint32_t v_step = (kRowTokens ? 1u : (uint32_t)TPV) * tok_bytes;  // bytes between value loads i, i + 1
    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    const int32_t* __restrict__ table = a.tables + (size_t)b * a.max_blocks;
    const float scale_log2 = a.scale_log2;

    // this wave's blocks: lo + w + NW * k
    const int n_mine = hi - lo > w ? (hi - lo - w + NW - 1) / NW : 0;

    // pa_decode_append (one chunk per lane): lane i takes item i of the new
    // tokens' rows of head g (token i / (2 C), K or V, 16-byte chunk i % C);
    // the items of this wave's blocks are loaded now and each is stored just
    // before its block's loads are issued (issue below), in this wave's
    // program order, so the block's loads see it.  The load's latency is
    // spent on the wave's earlier blocks instead of before the first one.
    int app_blk = -1;  // logical block this lane's item goes to (-1: none)
    uint4 app_data = make_uint4(0u, 0u, 0u, 0u);
    char* app_dst = nullptr;
    if (a.new_k && defers_append(a)) {
      const int chunks = a.append_row_bytes / 16;
      if (lane < a.q_len * 2 * chunks) {
        const int j = lane / (2 * chunks), kv = (lane / chunks) & 1, c = lane % chunks;
        const int pos = L - a.q_len + j;
        const int blk = pos >= 0 ? pos / kBlockTokens : -1;
        if (blk >= lo && blk < hi && (blk - lo) % NW == w) {
          const int phys = table[blk];
          if ((unsigned)phys < (unsigned)a.num_blocks) {
            app_blk = blk;
            app_data = *reinterpret_cast<const uint4*>(static_cast<const char*>(kv ? a.new_v : a.new_k) +
                                                       ((size_t)(b * a.q_len + j) * a.n_kv + g) * a.append_row_bytes +
                                                       16 * c);
            app_dst = static_cast<char*>(const_cast<void*>(kv ? a.v_cache : a.k_cache)) +
                      ((size_t)phys * kBlockTokens + pos % kBlockTokens) * a.n_kv * a.append_row_bytes +
                      (size_t)g * a.append_row_bytes + 16 * c;
          }
        }
      }
    }
    const bool app_any = __builtin_amdgcn_ballot_w64(app_blk >= 0) != 0;  // wave-uniform

    // ids of this wave's blocks k0 .. k0 + 63, one per lane
    auto block_ids = [&](int k0, int cnt) { return lane < cnt ? table[lo + w + NW * (k0 + lane)] : 0; };

    auto issue = [&](int ids, int cnt, int k0, int kk, uint4(&kb)[NCK], uint4(&vb)[NV], int& lblk, bool& ok) {
      const int phys = __builtin_amdgcn_readlane(ids, kk < cnt ? kk : 0);
      ok = kk < cnt && (unsigned)phys < (unsigned)a.num_blocks;
      lblk = lo + w + NW * (k0 + kk);
      if (app_any) {  // a new token of this block: stored before the block is loaded
        if (app_blk == lblk) {
          *reinterpret_cast<uint4*>(app_dst) = app_data;
          app_blk = -1;
        }
      }
      const int valid = min(kBlockTokens, L - lblk * kBlockTokens);
      const size_t boff = ok ? (size_t)phys * blk_bytes : 0;
      const uint32_t nrec = ok ? (uint32_t)valid * tok_bytes : 0u;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + boff), (short)0, (int)nrec, kBufferWord3);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + boff), (short)0, (int)nrec, kBufferWord3);
#pragma unroll
      for (int c = 0; c < NCK; ++c)
        kb[c] = __builtin_bit_cast(uint4,
                                   __builtin_amdgcn_raw_buffer_load_b128(kr, k_off + 64 * c, 0, 0));
#pragma unroll
      for (int i = 0; i < NV; ++i)
        vb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, v_off, i * v_step, kVPolicy));
    };

    // scores of this lane's token for every row, log2 units, -inf where masked
    auto scores = [&](const uint4(&kb)[NCK], int lblk, bool ok, float(&s)[R]) {
      const int pos = lblk * kBlockTokens + tk;
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
        const float sr = quad_sum(x) * scale_log2;  // every lane, so the DPP sources are live
        s[r] = (ok && pos < vis[r]) ? sr : kNegInf;
      }
    };

    // weights against the wave's reference, l, and P * V
    auto accumulate = [&](const float(&s)[R], const uint4(&vb)[NV]) {
      float p[R];
#pragma unroll
      for (int r = 0; r < R; ++r) p[r] = fast_exp2(s[r] - m_use[r]);
      if constexpr (kBF16) {
        // bf16 caches: the weights are rounded to bf16 and P V takes two
        // tokens per instruction, v_dot2_f32_bf16 of (p_t, p_t') with
        // (v_t[c], v_t'[c]) for the tokens of value loads 2m and 2m + 1; the
        // row sum adds the same rounded weights
        uint32_t pw[R];  // this lane's token's weight, twice, as a bf16 pair
#pragma unroll
        for (int r = 0; r < R; ++r) {
          pw[r] = pack_bf16(p[r], p[r]);
          lsum[r] += bf16_lo(pw[r]);
        }
#pragma unroll
        for (int m = 0; m < NV / 2; ++m) {
          uint32_t wp[R];  // (weight of load 2m's token, weight of load 2m + 1's token)
          if constexpr (kRowTokens) {
            float w0[R], w1[R];
            float pf[R];
#pragma unroll
            for (int r = 0; r < R; ++r) pf[r] = __builtin_bit_cast(float, pw[r]);
            bcast_in_row<R>(w0, pf, 2 * m);
            bcast_in_row<R>(w1, pf, 2 * m + 1);
#pragma unroll
            for (int r = 0; r < R; ++r)
              wp[r] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, w1[r]), __builtin_bit_cast(uint32_t, w0[r]),
                                            0x05040100u);
          } else {
            const int src0 = 4 * (tv + TPV * (2 * m)), src1 = 4 * (tv + TPV * (2 * m + 1));
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const float pf = __builtin_bit_cast(float, pw[r]);
              wp[r] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, lane_from(pf, src1)),
                                            __builtin_bit_cast(uint32_t, lane_from(pf, src0)), 0x05040100u);
            }
          }
          // column pairs: (v_t[c], v_t'[c]) for the lane's 8 columns
          const uint4 v0 = vb[2 * m], v1 = vb[2 * m + 1];
          const uint32_t d0[4] = {v0.x, v0.y, v0.z, v0.w}, d1[4] = {v1.x, v1.y, v1.z, v1.w};
          uint32_t cp[EPC];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            cp[2 * d] = __builtin_amdgcn_perm(d1[d], d0[d], 0x05040100u);
            cp[2 * d + 1] = __builtin_amdgcn_perm(d1[d], d0[d], 0x07060302u);
          }
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[r][e] = dot2_bf16(wp[r], cp[e], acc[r][e]);
        }
        return;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) lsum[r] += p[r];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        // weights of the token this lane's value load i holds
        float pr[R];
        if constexpr (kRowTokens) {
          bcast_in_row<R>(pr, p, i);
        } else {
          const int src = 4 * (tv + TPV * i);
#pragma unroll
          for (int r = 0; r < R; ++r) pr[r] = lane_from(p[r], src);
        }
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
    };

    auto set_reference = [&](const float(&mx)[R]) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        m_ref[r] = wave_max(mx[r]);
        m_use[r] = m_ref[r] == kNegInf ? 0.0f : m_ref[r];
      }
    };

    bool overflow = false;  // wave-uniform
    for (int k0 = 0; k0 < n_mine; k0 += 64) {
      const int cnt = min(64, n_mine - k0);
      const int ids = block_ids(k0, cnt);

      // NBUF register sets in flight: block kk + u computes while the next NBUF - 1 load
      uint4 kb[NBUF][NCK], vb[NBUF][NV];
      int lb[NBUF];
      bool okb[NBUF];
#pragma unroll
      for (int u = 0; u < NBUF; ++u) issue(ids, cnt, k0, u, kb[u], vb[u], lb[u], okb[u]);
      if (k0 == 0) {
        float s0[R];
        scores(kb[0], lb[0], okb[0], s0);
        set_reference(s0);
      }
      for (int kk = 0; kk < cnt; kk += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          if (kk + u < cnt) {
            float s[R];
            scores(kb[u], lb[u], okb[u], s);
            bool big = false;
#pragma unroll
            for (int r = 0; r < R; ++r) big |= s[r] > m_ref[r] + kOverflowSlack;
            overflow |= __builtin_amdgcn_ballot_w64(big) != 0;
            accumulate(s, vb[u]);
          }
          issue(ids, cnt, k0, kk + u + NBUF, kb[u], vb[u], lb[u], okb[u]);
        }
      }
    }

    if (overflow) {
      // some weight would have left the safe range: redo this wave's share
      // exactly, the maximum first and then the weighted sums
      float mx[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        mx[r] = kNegInf;
        lsum[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[r][e] = 0.0f;
      }
      for (int k0 = 0; k0 < n_mine; k0 += 64) {
        const int cnt = min(64, n_mine - k0);
        const int ids = block_ids(k0, cnt);
        for (int kk = 0; kk < cnt; ++kk) {
          uint4 kb1[NCK], vb1[NV];
          int lb1;
          bool ok1;
          issue(ids, cnt, k0, kk, kb1, vb1, lb1, ok1);
          float s[R];
          scores(kb1, lb1, ok1, s);
#pragma unroll
          for (int r = 0; r < R; ++r) mx[r] = fmaxf(mx[r], s[r]);
        }
      }
      set_reference(mx);
      for (int k0 = 0; k0 < n_mine; k0 += 64) {
        const int cnt = min(64, n_mine - k0);
        const int ids = block_ids(k0, cnt);
        for (int kk = 0; kk < cnt; ++kk) {
          uint4 kb1[NCK], vb1[NV];
          int lb1;
          bool ok1;
          issue(ids, cnt, k0, kk, kb1, vb1, lb1, ok1);
          float s[R];
          scores(kb1, lb1, ok1, s);
          accumulate(s, vb1);
        }
      }
    }

    // wave totals: l over the 16 tokens (each held by 4 lanes), acc over the value token phases
    __syncthreads();  // the previous range's totals have been read
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
        sm.m[w][r] = m_ref[r];
        sm.l[w][r] = lw;
      }
      if (lane < NC) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm.acc[w][r][lane * EPC + e] = acc[r][e];
      }
    }
    __syncthreads();
  }
};

template <typename T, int D, int R, int NW, int NBUF, bool BALANCED>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(DecodeParams a) {
  __shared__ WaveTotals<T, D, R, NW> sm;
  ValuAttender<T, D, R, NW, NBUF> at(a, sm);
  if constexpr (BALANCED) drive_balanced(a, at);
  else drive_fixed(a, at);
}

// Blocks in flight per wave in the fixed schedules: as many as fit next to the
// query chunks and the accumulators in about 200 VGPRs (two waves per SIMD),
// at least 2.
template <typename T, int D, int R>
constexpr int blocks_in_flight() {
  constexpr int chunks = D * (int)sizeof(T) / 16;     // 16-byte chunks per head row
  constexpr int per_block = 4 * (chunks / 4 + kBlockTokens / (64 / chunks));  // VGPRs of one block (K + V)
  constexpr int qregs = 4 * R * (chunks / 4);
  constexpr int budget = 200 - qregs - R * (16 / (int)sizeof(T));  // minus the accumulators
  constexpr int n = budget / per_block;
  return n < 2 ? 2 : (n > 4 ? 4 : n);
}

// blocks in flight per wave in the balanced schedule
constexpr int kBalancedBlocksInFlight = 1;

template <typename T, int D, int R>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
  constexpr int NB = blocks_in_flight<T, D, R>();
  if (p.mode == kBalanced) {
    // One block in flight per wave: a balanced range restarts its pipeline at
    // every sequence it crosses, and the shallower queue of requests in the
    // memory system (lower loaded latency) makes each restart cheaper; the
    // steady state stays at the same bandwidth (measured on the 8B layer:
    // 122 us against 126 us with three blocks).
    static const int resident =
        resident_per_cu(decode_valu_kernel<T, D, R, kWaves, kBalancedBlocksInFlight, true>, kWaves * 64);
    DecodeParams q = p;
    q.num_wgs = balanced_workgroups(resident, p.n_kv);
    hipLaunchKernelGGL((decode_valu_kernel<T, D, R, kWaves, kBalancedBlocksInFlight, true>), dim3(q.num_wgs),
                       dim3(kWaves * 64), 0, s, q);
  } else {
    DecodeParams q = p;
    if (p.mode == kSinglePass) {
      static const int resident = resident_per_cu(decode_valu_kernel<T, D, R, kWaves, NB, false>, kWaves * 64);
      q.pair_stride = one_pass_pairing(resident, p.num_seqs, p.n_kv);
    }
    dim3 grid(p.mode == kPartitions ? p.num_parts : 1, p.n_kv, p.num_seqs);
    hipLaunchKernelGGL((decode_valu_kernel<T, D, R, kWaves, NB, false>), grid, dim3(kWaves * 64), 0, s, q);
  }
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
