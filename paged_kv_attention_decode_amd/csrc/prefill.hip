// Chunked-prefill attention over the paged KV cache (bf16, matrix cores).
//
// A long prompt is processed in chunks, one per engine step, each chunk's
// tokens attending to the whole cached prefix and to the chunk's own earlier
// tokens ("Chapter 18: Speculative Decoding and Serving Optimizations",
// arunshar.com, section 18.2.1; "LLM serving: KV cache, batching, paged
// attention and quantization", learn.mohebi.ai, section 3.6; "07 -
// Inference", lourdhu02.github.io, section 2.4).  One call takes sequences
// with different numbers of new tokens (query_start), so a step's prefill
// chunks and single decode tokens can share it.
//
// With hundreds of query rows per KV head the products are dense, so the
// layout is the reverse of the decode kernels': a workgroup owns 128 query
// rows (new token x head of the GQA group, token-major) of one sequence and
// KV head, 32 rows per wave, and all four waves walk the same KV blocks.
// Each block (16 tokens of K and of V for the head) is staged once per
// workgroup in LDS, double-buffered (the next block's global loads are in
// flight while the current one is multiplied), and every wave reads it from
// there:
//
//   scores  S^T = K_blk Q^T per 16-row tile, v_mfma_f32_16x16x32_bf16 with
//           A = K from LDS (lane l: token l % 16, 8 dims) and B = the wave's
//           query rows, which stay in registers for the whole sweep; lane l
//           ends with tokens 4 (l / 16) .. + 3 of row l % 16;
//   values  O += P V, v_mfma_f32_16x16x16_bf16 with A = P in that same
//           layout and B = V: a lane reads 4 columns of each of its 4 tokens
//           from LDS and a v_perm_b32 4 x 4 transpose forms the operands.
//
// The softmax takes each row's maximum over block 0 (every row sees position
// 0) as a fixed reference; a score more than 2^64 above it raises a flag, and
// a workgroup whose flag is up redoes its rows exactly in two more sweeps
// (true row maxima, then the weighted sums).  Weights are rounded to bf16 for
// the P V product and the row sums add the same rounded weights.
#include "pa_device.h"
#include "pa_prefill.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kPrefillRowsPerWG / kWaves;  // two 16-row tiles
static_assert(kRowsPerWave == 32, "two MFMA row tiles per wave");
constexpr float kOverflowSlack = 64.0f;  // log2 units

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_p __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_p));
}

// one block of one KV head in LDS; rows padded by 16 bytes so that the 16
// token rows one K read touches fall in different banks
template <int D>
struct Stage {
  uint16_t k[kBlockTokens][D + 8];
  uint16_t v[kBlockTokens][D + 8];
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams a) {
  constexpr int KS = D / 32;                          // score k-steps
  constexpr int VH = D / 64;                          // value column halves
  constexpr int CH = D / 8;                           // 16-byte chunks per token row of the head
  constexpr int NCHUNK = 2 * kBlockTokens * CH;       // K and V chunks of one block
  constexpr int LOADS = (NCHUNK + kThreads - 1) / kThreads;
  static_assert(NCHUNK % kThreads == 0, "every thread stages the same number of chunks");

  __shared__ Stage<D> st[2];
  __shared__ int s_overflow;

  const int b = blockIdx.z, g = blockIdx.y;
  const int chunk = (int)gridDim.x - 1 - (int)blockIdx.x;  // the latest rows (most blocks) start first
  const int q0 = a.qstart[b];
  const int n = a.qstart[b + 1] - q0;
  if (q0 < 0 || n <= 0 || n > a.max_q_len || q0 > a.num_q_tokens - n) return;
  const int rows = n * a.group;
  const int r0 = chunk * kPrefillRowsPerWG;
  if (r0 >= rows) return;
  const int r_end = min(r0 + kPrefillRowsPerWG, rows);
  const int Lmax = a.max_blocks * kBlockTokens;
  const int L = min(max(a.lens[b], 0), Lmax);
  const int base = L - n;  // position of new token 0
  const int pos_end = min(L, max(0, base + (r_end - 1) / a.group + 1));  // no row here sees past it
  const int nblk = (pos_end + kBlockTokens - 1) / kBlockTokens;
  const int32_t* __restrict__ table = a.tables + (size_t)b * a.max_blocks;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, grp = lane >> 4;
  const int wr0 = r0 + kRowsPerWave * w;  // the wave's first row
  const bool wave_rows = wr0 < r_end;
  const int wave_end = wave_rows ? min(L, max(0, base + (min(wr0 + kRowsPerWave, r_end) - 1) / a.group + 1)) : 0;

  // the wave's query rows as score B operands: tile tt, row wr0 + 16 tt + j, dims 32 ks + 8 grp .. + 7
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  uint4 qreg[2][KS];
  int vis[2];  // row 16 tt + j of the wave sees positions below vis[tt]
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int row = wr0 + 16 * tt + j;
    const bool ok = row < r_end;
    const int tok = row / a.group, hh = row % a.group;
    vis[tt] = ok ? min(L, max(0, base + tok + 1)) : 0;
    const uint16_t* src = qp + (((size_t)q0 + tok) * a.n_h + (size_t)g * a.group + hh) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[tt][ks] = ok ? *reinterpret_cast<const uint4*>(src + 32 * ks) : make_uint4(0, 0, 0, 0);
  }

  float m_ref[2] = {kNegInf, kNegInf}, m_use[2] = {0.0f, 0.0f}, lsum[2] = {0.0f, 0.0f};
  floatx4_t acc[2][VH][4];
  floatx4_t mx[2];
  auto clear = [&]() {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      lsum[tt] = 0.0f;
      mx[tt] = (floatx4_t){kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tt][h][e] = (floatx4_t){0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  clear();

  // staging: chunk c of a block is K (c < 16 CH) or V, token (c % 16 CH) / CH, 16 bytes (c % CH)
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const size_t tok_stride = (size_t)a.n_kv * D * 2;
  const size_t head_off = (size_t)g * D * 2;
  auto fetch = [&](int k, uint4(&r)[LOADS]) {
    const int phys = table[k];
    const bool blk_ok = (unsigned)phys < (unsigned)a.num_blocks;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = threadIdx.x + u * kThreads;
      const int rem = c % (kBlockTokens * CH);
      const int tok = rem / CH, part = rem % CH;
      const bool ok = blk_ok && k * kBlockTokens + tok < L;
      const char* src = (c < kBlockTokens * CH ? kbase : vbase) +
                        ((size_t)(ok ? phys : 0) * kBlockTokens + tok) * tok_stride + head_off + 16 * part;
      r[u] = ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
    }
  };
  auto put = [&](int buf, const uint4(&r)[LOADS]) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = threadIdx.x + u * kThreads;
      const int rem = c % (kBlockTokens * CH);
      const int tok = rem / CH, part = rem % CH;
      uint16_t* dst = c < kBlockTokens * CH ? &st[buf].k[tok][8 * part] : &st[buf].v[tok][8 * part];
      *reinterpret_cast<uint4*>(dst) = r[u];
    }
  };

  // per-row reference: the row's maximum over the block (lanes j, j+16, j+32, j+48 share a row)
  auto set_reference = [&](const floatx4_t(&s)[2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float x = fmaxf(fmaxf(s[tt][0], s[tt][1]), fmaxf(s[tt][2], s[tt][3]));
      x = fmaxf(x, shfl_xor(x, 16));
      x = fmaxf(x, shfl_xor(x, 32));
      m_ref[tt] = x;
      m_use[tt] = x == kNegInf ? 0.0f : x;
    }
  };

  bool overflow = false;  // wave-uniform
  // mode 0: reference from block 0, weighted sums, overflow check; 1: row maxima only; 2: weighted sums
  auto compute = [&](int k, int buf, int mode) {
    if (!wave_rows || k * kBlockTokens >= wave_end) return;  // wave-uniform
    const bool blk_ok = (unsigned)table[k] < (unsigned)a.num_blocks;
    const int pos0 = k * kBlockTokens + 4 * grp;
    floatx4_t s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      floatx4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kb = *reinterpret_cast<const uint4*>(&st[buf].k[j][32 * ks + 8 * grp]);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb),
                                                    __builtin_bit_cast(bf16x8_t, qreg[tt][ks]), x, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) s[tt][v] = (blk_ok && pos0 + v < vis[tt]) ? x[v] * a.scale_log2 : kNegInf;
    }
    if (mode == 1) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx[tt][v] = fmaxf(mx[tt][v], s[tt][v]);
      return;
    }
    if (mode == 0) {
      if (k == 0) set_reference(s);
      bool big = false;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) big |= s[tt][v] > m_ref[tt] + kOverflowSlack;
      overflow |= __builtin_amdgcn_ballot_w64(big) != 0;
    }
    // B operands of P V: column 4 j + 64 h + e of the lane's 4 tokens, bf16 pairs (tokens 0,1), (2,3)
    uint2 vb[4][VH];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int h = 0; h < VH; ++h) vb[v][h] = *reinterpret_cast<const uint2*>(&st[buf].v[4 * grp + v][4 * j + 64 * h]);
    uint2 vt[VH][4];
#pragma unroll
    for (int h = 0; h < VH; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const bool hi = e >= 2;
        vt[h][e].x = __builtin_amdgcn_perm(hi ? vb[1][h].y : vb[1][h].x, hi ? vb[0][h].y : vb[0][h].x, sel);
        vt[h][e].y = __builtin_amdgcn_perm(hi ? vb[3][h].y : vb[3][h].x, hi ? vb[2][h].y : vb[2][h].x, sel);
      }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] = fast_exp2(s[tt][v] - m_use[tt]);
      uint2 pa2;
      pa2.x = pack_bf16(p[0], p[1]);
      pa2.y = pack_bf16(p[2], p[3]);
      lsum[tt] += (bf16_lo(pa2.x) + bf16_hi(pa2.x)) + (bf16_lo(pa2.y) + bf16_hi(pa2.y));
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[tt][h][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(short4_t, pa2), __builtin_bit_cast(short4_t, vt[h][e]), acc[tt][h][e], 0, 0, 0);
    }
  };

  // one pass over the blocks: block k + 1's loads are in flight while block k is multiplied
  auto sweep = [&](int mode) {
    uint4 r[LOADS];
    fetch(0, r);
    put(0, r);
    __syncthreads();
    for (int k = 0; k < nblk; ++k) {
      const int cur = k & 1;
      if (k + 1 < nblk) fetch(k + 1, r);
      compute(k, cur, mode);
      if (k + 1 < nblk) put(cur ^ 1, r);
      __syncthreads();  // block k + 1 staged; everyone is done with block k
    }
  };

  if (threadIdx.x == 0) s_overflow = 0;
  if (nblk > 0) {
    sweep(0);  // its first barrier also publishes s_overflow = 0
    if (overflow && lane == 0) s_overflow = 1;
    __syncthreads();
    if (s_overflow) {  // exact redo: true row maxima, then the weighted sums
      clear();
      sweep(1);
      if (wave_rows) set_reference(mx);
      clear();
      sweep(2);
    }
  }
  if (!wave_rows) return;

  // row sums over the 4 token groups: lanes j, j+16, j+32, j+48 then hold row j of each tile
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    float x = lsum[tt];
    x += shfl_xor(x, 16);
    x += shfl_xor(x, 32);
    lsum[tt] = x;
  }
  // output: lane l holds rows 4 (l / 16) + i of each tile, columns 4 (l % 16) + 64 h + e
  uint16_t* __restrict__ op = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * grp + i;  // row within the tile
      const float l = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(rr << 2, __builtin_bit_cast(int, lsum[tt])));
      const int row = wr0 + 16 * tt + rr;
      if (row >= r_end) continue;
      const int tok = row / a.group, hh = row % a.group;
      uint16_t* dst = op + (((size_t)q0 + tok) * a.n_h + (size_t)g * a.group + hh) * D + 4 * j;
#pragma unroll
      for (int h = 0; h < VH; ++h) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = l > 0.0f ? acc[tt][h][e][i] / l : 0.0f;
        uint2 packed;
        packed.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
        packed.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
        *reinterpret_cast<uint2*>(dst + 64 * h) = packed;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t s) {
  const long long rows = (long long)p.max_q_len * p.group;
  const unsigned chunks = (unsigned)((rows + kPrefillRowsPerWG - 1) / kPrefillRowsPerWG);
  const dim3 grid(chunks, (unsigned)p.n_kv, (unsigned)p.num_seqs);
  if (head_dim == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
