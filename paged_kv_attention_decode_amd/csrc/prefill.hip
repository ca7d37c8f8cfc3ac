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
// layout is the reverse of the decode kernels': a workgroup owns 256 query
// rows (new token x head of the GQA group, token-major) of one sequence and
// KV head, 32 rows per wave, and all eight waves (two per SIMD, one
// workgroup per CU) walk the same KV blocks.
// Each block (16 tokens of K and of V for the head) is staged once per
// workgroup in LDS, 8 blocks per step, double-buffered: the next step goes
// from memory straight into LDS (gfx950's 16-byte buffer-to-LDS loads, wave
// w loading block w) while the current one is multiplied, and every wave
// reads it from there:
//
//   scores  S^T = K_blk Q^T per 16-row tile, v_mfma_f32_16x16x32_bf16 with
//           A = K from LDS (lane l: token l % 16, 8 dims) and B = the wave's
//           query rows, which stay in registers for the whole sweep; lane l
//           ends with tokens 4 (l / 16) .. + 3 of row l % 16;
//   values  O += P V over two blocks at a time, v_mfma_f32_16x16x32_bf16
//           with A = P in that same layout (k-slots: the lane's 4 tokens of
//           each block) and B = V read with the transposing LDS load
//           ds_read_b64_tr_b16, which hands lane l the 4 tokens of one value
//           column directly; call t covers columns 16 t + l % 16.
//
// The softmax takes each row's maximum over the first pair of blocks (blocks
// 0 and 1; every row sees position 0) as a fixed reference; a score more than
// 2^64 above it raises a flag, and
// a workgroup whose flag is up redoes its rows exactly in two more sweeps
// (true row maxima, then the weighted sums).  Weights are rounded to bf16 for
// the P V product and the row sums add the same rounded weights.
#include "pa_device.h"
#include "pa_prefill.h"

namespace pa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kPrefillRowsPerWG / kWaves;
constexpr int TW = kRowsPerWave / 16;  // 16-row MFMA tiles per wave
static_assert(kRowsPerWave % 16 == 0, "whole MFMA row tiles per wave");
constexpr float kOverflowSlack = 64.0f;  // log2 units
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X
constexpr int kStepBlocks = 8;           // blocks staged per step (per barrier), multiplied two at a time

// one block of one KV head in LDS (64 banks of 4 bytes).  Rows are not padded:
// a buffer-to-LDS load fills 1 KiB contiguous per instruction.  Instead the
// 16-byte chunk c of token row r sits at chunk c ^ kswz(r) of its K row and
// c ^ vswz(r) of its V row.  A K read (16 lanes, 16 bytes each: 16 rows, one
// logical chunk) then touches every bank once, and so does a transposing V
// read (32 lanes, 8 bytes each: 8 token rows x 32 contiguous bytes; the XOR
// is even there, so a row's two chunks stay side by side).
template <int D>
struct Stage {
  uint16_t k[kBlockTokens][D];
  uint16_t v[kBlockTokens][D];
};
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// one 16-byte buffer-to-LDS load per lane (gfx950): LDS lds + 16 lane <- the
// descriptor's bytes at voff, zero past its record count.  Written in asm so
// that the compiler does not track it: it would put a vmcnt(0) before the
// reads of the other buffer, since it cannot tell the two apart.  The caller
// waits for it (vmcnt) before the barrier that publishes it.  m0, which the
// load takes its LDS address from, is restored afterwards (the load reads it
// at issue; the compiler assumes m0 keeps its value across the asm).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, u32x4_t rs) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(void*)p;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams a) {
  constexpr int KS = D / 32;                          // score k-steps
  constexpr int VH = D / 64;                          // value column halves
  constexpr int CH = D / 8;                           // 16-byte chunks per token row of the head

  __shared__ Stage<D> st[2][kStepBlocks];  // [buffer][block of the step]
  __shared__ int s_overflow;

  // Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
  // Renumber them so that the row chunks of one (sequence, KV head), which
  // read the same blocks, run on one XCD: the k-th workgroup an XCD receives
  // takes the k-th item of that XCD's contiguous share of the work.
  const int n_items = (int)(gridDim.x * gridDim.y * gridDim.z);
  const int lin = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int xcd = lin % kXcds, slot = lin / kXcds;
  const int per = n_items / kXcds, extra = n_items % kXcds;
  const int item = xcd * per + min(xcd, extra) + slot;
  const int b = item / (int)(gridDim.x * gridDim.y), g = (item / (int)gridDim.x) % (int)gridDim.y;
  const int chunk = (int)gridDim.x - 1 - item % (int)gridDim.x;  // the latest rows (most blocks) first
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
  // positions below this are seen by every row of the wave (0 when the wave has padding rows)
  const int wave_min_vis = wr0 + kRowsPerWave <= r_end ? min(L, max(0, base + wr0 / a.group + 1)) : 0;

  // the wave's query rows as score B operands: tile tt, row wr0 + 16 tt + j, dims 32 ks + 8 grp .. + 7
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  uint4 qreg[TW][KS];
  int vis[TW];  // row 16 tt + j of the wave sees positions below vis[tt]
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    const int row = wr0 + 16 * tt + j;
    const bool ok = row < r_end;
    const int tok = row / a.group, hh = row % a.group;
    vis[tt] = ok ? min(L, max(0, base + tok + 1)) : 0;
    const uint16_t* src = qp + (((size_t)q0 + tok) * a.n_h + (size_t)g * a.group + hh) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[tt][ks] = ok ? *reinterpret_cast<const uint4*>(src + 32 * ks) : make_uint4(0, 0, 0, 0);
  }

  float m_ref[TW], m_use[TW], lsum[TW];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    m_ref[tt] = kNegInf;
    m_use[tt] = 0.0f;
  }
  floatx4_t acc[TW][VH][4];
  floatx4_t mx[TW];
  auto clear = [&]() {
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      lsum[tt] = 0.0f;
      mx[tt] = (floatx4_t){kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tt][h][e] = (floatx4_t){0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  clear();

  // staging: wave w loads block w of each step, K then V, RPI token rows per
  // instruction; lane l brings 16-byte chunk l % CH of row RPI i + l / CH of
  // the LDS layout, so it reads that row's logical chunk (l % CH) ^ swizzle.
  // A block is read through buffer descriptors whose record count ends at its
  // last context token (the rest reads as zero); a lane's byte offsets inside
  // the block are fixed.
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const uint32_t tok_stride = (uint32_t)a.n_kv * D * 2;
  const size_t blk_bytes = (size_t)tok_stride * kBlockTokens;
  constexpr int RPI = 1024 / (2 * D);     // token rows per 1 KiB load instruction
  constexpr int NI = kBlockTokens / RPI;  // load instructions per block, for K and for V
  static_assert(kStepBlocks == kWaves, "wave w stages block w of every step");
  uint32_t voffk[NI], voffv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * i + lane / CH, pc = lane % CH;
    const uint32_t rb = (uint32_t)row * tok_stride + (uint32_t)g * D * 2;
    voffk[i] = rb + 16u * (uint32_t)(pc ^ kswz<D>(row));
    voffv[i] = rb + 16u * (uint32_t)(pc ^ vswz<D>(row));
  }
  // The block-table entries of step it, one per lane (lane l % 8: block 8 it +
  // l % 8, clamped into the range, nblk >= 1): a vector load issued a whole
  // step before the entries are used, instead of a scalar load per block
  // waited for on the spot, which would stall every wave at every step.
  auto table_vec = [&](int it) -> int {
    const int blk = kStepBlocks * it + (lane & (kStepBlocks - 1));
    return table[min(blk, nblk - 1)];
  };
  // step it into LDS buffer buf: wave w loads block w, its table entries in tv (from
  // table_vec(it)).  Returns bit bb set where block bb of the step is valid (in
  // the range and inside the pool), so that the multiply needs no table reads.
  auto issue = [&](int it, int tv, int buf) -> uint32_t {
    const int bl = kStepBlocks * it + (lane & (kStepBlocks - 1));
    const bool okl = lane < kStepBlocks && bl < nblk && (unsigned)tv < (unsigned)a.num_blocks;
    const uint32_t okm = (uint32_t)__builtin_amdgcn_ballot_w64(okl);
    const int blk = kStepBlocks * it + w;
    const bool ok = (okm >> w) & 1u;
    const int raw = __builtin_amdgcn_readlane(tv, w);
    const uint32_t nrec = ok ? (uint32_t)min(kBlockTokens, L - blk * kBlockTokens) * tok_stride : 0u;
    const size_t boff = ok ? (size_t)raw * blk_bytes : 0;
    const size_t ka = (size_t)(kbase + boff), va = (size_t)(vbase + boff);
    const u32x4_t kr = {(uint32_t)ka, (uint32_t)(ka >> 32) & 0xffffu, nrec, (uint32_t)kBufferWord3};
    const u32x4_t vr = {(uint32_t)va, (uint32_t)(va >> 32) & 0xffffu, nrec, (uint32_t)kBufferWord3};
    const uint32_t kl = lds_u32(&st[buf][w].k[0][0]), vl = lds_u32(&st[buf][w].v[0][0]);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(kl + 1024u * i, voffk[i], kr);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(vl + 1024u * i, voffv[i], vr);
    return okm;
  };

  // per-row reference: the row's maximum (lanes j, j+16, j+32, j+48 share a row)
  auto set_reference = [&](const floatx4_t(&s)[TW]) {
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      float x = fmaxf(fmaxf(s[tt][0], s[tt][1]), fmaxf(s[tt][2], s[tt][3]));
      x = fmaxf(x, shfl_xor(x, 16));
      x = fmaxf(x, shfl_xor(x, 32));
      m_ref[tt] = x;
      m_use[tt] = x == kNegInf ? 0.0f : x;
    }
  };

  // per lane and tile, the largest exponent of the first sweep, checked against
  // the overflow threshold once the sweep is done (the reference is fixed by then)
  float tmax[TW];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) tmax[tt] = kNegInf;
  const float c = a.scale_log2;
  // a pair of blocks: blk0 and blk0 + 1, staged in slots sl and sl + 1 of the buffer, valid
  // where bits 0 and 1 of okb are set.
  // mode 0: reference from the first pair, weighted sums, largest exponents; 1: row maxima only;
  // 2: weighted sums
  auto pair = [&](int blk0, int buf, int sl, int mode, uint32_t okb) {
    // the compiler's interleaving of LDS reads with matrix instructions:
    // 143.5-143.9 against 144.9-145.9 us on four 512-token chunks (three
    // alternating runs; variant 1 143.8-144.1)
    __builtin_amdgcn_iglp_opt(0);
    floatx4_t x[2][TW];  // raw q.k: [block][tile], lane: tokens 4 grp + v of row j
    bool ok[2], whole[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int blk = blk0 + bb;
      ok[bb] = (okb >> bb) & 1u;
      whole[bb] = ok[bb] && (blk + 1) * kBlockTokens <= wave_min_vis;  // every row sees all 16 tokens
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) {
        floatx4_t acc_s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 kb = *reinterpret_cast<const uint4*>(&st[buf][sl + bb].k[j][8 * ((4 * ks + grp) ^ kswz<D>(j))]);
          acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb),
                                                          __builtin_bit_cast(bf16x8_t, qreg[tt][ks]), acc_s, 0, 0, 0);
        }
        x[bb][tt] = acc_s;
      }
    }
    // whether row j of tile tt sees token 4 grp + v of block bb
    auto sees = [&](int bb, int tt, int v) -> bool {
      const int pos = (blk0 + bb) * kBlockTokens + 4 * grp + v;
      return whole[bb] || (ok[bb] && pos < vis[tt]);
    };
    // scores in log2 units, -inf where masked
    auto score = [&](int bb, int tt, int v) -> float { return sees(bb, tt, v) ? x[bb][tt][v] * c : kNegInf; };
    if (mode == 1 || (mode == 0 && blk0 == 0)) {
      floatx4_t sm[TW];
#pragma unroll
      for (int tt = 0; tt < TW; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm[tt][v] = fmaxf(score(0, tt, v), score(1, tt, v));
      if (mode == 1) {
#pragma unroll
        for (int tt = 0; tt < TW; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) mx[tt][v] = fmaxf(mx[tt][v], sm[tt][v]);
        return;
      }
      set_reference(sm);
    }
    // exponent t = scale q.k - m (one fma; -inf where masked, selected without a branch), weights 2^t
    float t[2][TW][4];
    if (whole[0] && whole[1]) {  // wave-uniform: every row sees both blocks whole
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int tt = 0; tt < TW; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) t[bb][tt][v] = __builtin_fmaf(x[bb][tt][v], c, -m_use[tt]);
    } else {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int tt = 0; tt < TW; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            t[bb][tt][v] = sees(bb, tt, v) ? __builtin_fmaf(x[bb][tt][v], c, -m_use[tt]) : kNegInf;
    }
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      const float hi = fmaxf(fmaxf(fmaxf(t[0][tt][0], t[0][tt][1]), fmaxf(t[0][tt][2], t[0][tt][3])),
                             fmaxf(fmaxf(t[1][tt][0], t[1][tt][1]), fmaxf(t[1][tt][2], t[1][tt][3])));
      tmax[tt] = fmaxf(tmax[tt], hi);
    }
    // B operands of P V (16x16x32): k-slots 0-3 are tokens 4 grp + 0..3 of block 0, slots 4-7
    // the same tokens of block 1; call (h, e) covers value columns 16 (4 h + e) + n.  Read with
    // the transposing LDS load (ds_read_b64_tr_b16): within each 16-lane group, output lane
    // 4 q + k takes element k of the 8 bytes addressed by lane 4 e' + q as its element e'.
    // Lane s of the group (s = j) addresses token 4 grp + s / 4, columns 16 t + 4 (s % 4) .. + 3,
    // so lane (j, grp) receives tokens 4 grp + 0..3 of column 16 t + j: its operand half,
    // with no permutes.
    short4_t vt4[2][VH][4];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int vr = 4 * grp + (j >> 2), vc = 2 * (4 * h + e) + ((j & 3) >> 1);  // row, logical chunk
          const uint16_t* src = &st[buf][sl + bb].v[vr][8 * (vc ^ vswz<D>(vr)) + 4 * (j & 1)];
          vt4[bb][h][e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)src);
        }
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      uint4 pa;
      pa.x = pack_bf16(fast_exp2(t[0][tt][0]), fast_exp2(t[0][tt][1]));
      pa.y = pack_bf16(fast_exp2(t[0][tt][2]), fast_exp2(t[0][tt][3]));
      pa.z = pack_bf16(fast_exp2(t[1][tt][0]), fast_exp2(t[1][tt][1]));
      pa.w = pack_bf16(fast_exp2(t[1][tt][2]), fast_exp2(t[1][tt][3]));
      // the row sum adds the same rounded weights the product uses
      constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
      lsum[tt] = dot2_bf16(pa.x, kOnes, dot2_bf16(pa.y, kOnes, dot2_bf16(pa.z, kOnes, dot2_bf16(pa.w, kOnes,
                                                                                                  lsum[tt]))));
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint2 v0 = __builtin_bit_cast(uint2, vt4[0][h][e]), v1 = __builtin_bit_cast(uint2, vt4[1][h][e]);
          const uint4 vt = make_uint4(v0.x, v0.y, v1.x, v1.y);
          acc[tt][h][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pa),
                                                                  __builtin_bit_cast(bf16x8_t, vt), acc[tt][h][e], 0,
                                                                  0, 0);
        }
    }
  };

  // one step: its pairs of blocks, those some row of the wave sees; bit bb of okm is set
  // where block bb of the step is valid.  mid() runs after the first half of
  // the pairs, in every wave, whether or not its rows see them
  auto compute = [&](int it, int buf, int mode, uint32_t okm, auto&& mid) {
#pragma unroll
    for (int pp = 0; pp < kStepBlocks / 2; ++pp) {
      if (pp == kStepBlocks / 4) mid();
      const int blk0 = kStepBlocks * it + 2 * pp;
      if (wave_rows && blk0 * kBlockTokens < wave_end) pair(blk0, buf, 2 * pp, mode, okm >> (2 * pp));  // wave-uniform
    }
  };

  // one pass over the steps.  LDS holds two steps: the one being multiplied
  // and the next one, whose loads are issued halfway through the step's pairs
  // (its buffer was last read in the previous step, which ended at a
  // barrier); each wave waits for its own loads before the barrier that ends
  // the step.  On four 512-token chunks (three alternating runs): 139.3-139.4
  // us; issued at the start of the step 146.2-147.2, after the first pair
  // 141.0-141.3, after the third 141.6-142.2; global loads into registers that
  // the waves then wrote to LDS, 165.0-165.1 us with 32 VGPRs more.
  const int nit = (nblk + kStepBlocks - 1) / kStepBlocks;
  auto sweep = [&](int mode) {
    // table loads are unconditional (clamped to the last step): a register
    // set to 0 on the other path would need a wait for the load in flight into it
    int tvn = table_vec(min(1, nit - 1));
    uint32_t okm = issue(0, table_vec(0), 0);
    wait_dma();
    __syncthreads();
    for (int it = 0; it < nit; ++it) {
      uint32_t okn = 0u;
      compute(it, it & 1, mode, okm, [&] {
        okn = it + 1 < nit ? issue(it + 1, tvn, (it + 1) & 1) : 0u;
        tvn = table_vec(min(it + 2, nit - 1));
      });
      okm = okn;
      wait_dma();
      __syncthreads();  // step it + 1 staged; everyone is done with step it
    }
  };

  if (threadIdx.x == 0) s_overflow = 0;
  if (nblk > 0) {
    sweep(0);  // its first barrier also publishes s_overflow = 0
    // a row without a reference (nothing seen in step 0) redoes on any weight
    bool big = false;
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) big |= tmax[tt] > (m_ref[tt] == kNegInf ? kNegInf : kOverflowSlack);
    if (__builtin_amdgcn_ballot_w64(big) != 0 && lane == 0) s_overflow = 1;
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
  for (int tt = 0; tt < TW; ++tt) {
    float x = lsum[tt];
    x += shfl_xor(x, 16);
    x += shfl_xor(x, 32);
    lsum[tt] = x;
  }
  // output: lane l holds rows 4 (l / 16) + i of each tile, columns 64 h + 16 e + l % 16
  // (the 16 lanes of a group write 32 contiguous bytes per column group)
  uint16_t* __restrict__ op = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * grp + i;  // row within the tile
      const float l = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(rr << 2, __builtin_bit_cast(int, lsum[tt])));
      const int row = wr0 + 16 * tt + rr;
      if (row >= r_end) continue;
      const int tok = row / a.group, hh = row % a.group;
      uint16_t* dst = op + (((size_t)q0 + tok) * a.n_h + (size_t)g * a.group + hh) * D + j;
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[64 * h + 16 * e] = (uint16_t)f32_to_bf16_bits(l > 0.0f ? acc[tt][h][e][i] / l : 0.0f);
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
