// Paged decode attention on the matrix cores (bf16 products), for 8 to 64
// query rows per KV head over bf16 caches, e.g. the K + 1 tokens of a
// speculative verify step times the GQA group, and for every row count from 1
// to 64 over fp8 caches (KV8) and for tree verify (TREE).  Same computation and contract as the vector-ALU kernel (include/pa.h):
// for each sequence b, KV head g and query row r = j * group + hh,
//   out = sum_t softmax_t(scale * q . k_t) v_t   over the positions row r sees,
// with the causal mask among the q_len new tokens ("07 - Inference",
// lourdhu02.github.io, section 3: the target scores all K + 1 positions in one
// pass), reading K and V through the block table one 16-token block at a time
// ("LLM serving: KV cache, batching, paged attention and quantization",
// section 3.5).  With rows = group * q_len query rows per KV head, Q K^T and
// P V are real dense tiles, so they run on MFMA:
//
//   scores  S^T = K_blk Q^T per 16-row tile: v_mfma_f32_16x16x32_bf16 with
//           A = 16 tokens x 32 dims of K (lane l: token l % 16, dims
//           8 (l / 16) .. + 7 of the current 32), B = the same dims of 16 query
//           rows; head_dim / 32 steps.  Lane l ends with tokens 4 (l / 16) .. + 3
//           of row l % 16.
//   values  O += P V: v_mfma_f32_16x16x16_bf16 with A = P (16 rows x 16 tokens),
//           whose layout is exactly the score layout above, so the weights
//           never leave their lanes; B = 16 tokens x 16 value columns.  A lane
//           loads 8 bytes (4 columns) of each of its 4 tokens and a 4 x 4
//           v_perm_b32 transpose gives the B operands; MFMA column j of call
//           (h, e) is value column 4 j + 64 h + e.
//
// Memory traffic and the softmax reference follow the vector-ALU kernel: buffer
// loads through a per-block descriptor whose record count ends at the last
// context token, NBUF blocks in flight per wave, a per-row reference taken
// from the wave's first block, a wave-uniform flag for weights beyond
// 2^kOverflowSlack and an exact two-pass redo when it is raised.  Weights are
// rounded to bf16 (v_cvt_pk_bf16_f32) for the P V product and the row sums
// add the same rounded weights, so numerator and denominator agree.  The waves
// of a workgroup merge one after the other into a single LDS tile.
//
// VLDS (bf16, four row tiles): V goes from memory straight into LDS
// with 16-byte buffer-to-LDS loads, one ring of NBUF slots per wave, so that
// the blocks in flight cost LDS rather than registers (four tiles' accumulators
// leave room for one block of K and V in registers, but three of K).  Slot
// layout: token t's D columns are 2 D contiguous bytes, their 16-byte chunks
// XOR-swizzled by a function X(t) of the token (position chunk ^ 2 X(t)), and
// P V's B operands come out of it through the transposing LDS read
// ds_read_b64_tr_b16: within each 16-lane group, output lane 4 b + k takes
// element k of the 8 bytes that lane 4 a + b addresses, as its element a.
// Lane (a, b) of group grp addresses token 4 grp + a, columns 16 ct + 4 b .. + 3,
// so output lane j holds tokens 4 grp .. + 3 of column 16 ct + j: MFMA column j
// of call (h, e) is value column 64 h + 16 e + j, with no permutes.  The ring
// shares LDS with the merge tile's accumulators, which are written only after
// the block loop.
//
// TREE: the q_len new tokens are the nodes of a draft tree checked in one pass
// ("Chapter 18: Speculative Decoding and Serving Optimizations", arunshar.com,
// section 18.1.2, tree-based verification for Medusa; "07 - Inference",
// section 3.4, the tree attention mask).  Node j sits at position
// L - q_len + j and sees every position before the tree and the nodes on its
// own path to the root, given by a parent array (parent < node, -1 at a
// root).  Each row builds that path as a 64-bit node mask once per range; a
// score then survives when its position is before the tree or its node's bit
// is set.
#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_schedule.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr float kOverflowSlack = 64.0f;  // log2 units
template <int R, int D, int RING = 0>
struct alignas(1024) MergeTile {
  // VLDS: the per-wave rings of staged V blocks (RING bytes), in the same
  // bytes as the accumulators below, which are written only after the block
  // loop; 1 KiB aligned, so each slot's swizzle sees whole 256-byte bank rows
  union {
    uint8_t vring[RING > 0 ? RING : 16];
    // merged P V accumulators in the MFMA output layout, lane-major: entry
    // ((t * (D / 64) + h) * 4 + e) * 64 + lane holds the 4 rows 16 t + 4 (lane / 16)
    // .. + 3 of value column col_of(lane % 16, h, e), so a wave merges its own
    // accumulators with one conflict-free 16-byte LDS read and write each
    floatx4_t acc[R * D / 4];
  };
  float m[R];      // merged row max (log2 units)
  float l[R];      // merged row sum
  float wm[R];     // the merging wave's row max
  float wl[R];     // the merging wave's row sum
  // the query rows of the current range (bf16), read as score B operands; each
  // row is padded by 32 bytes: at 288 bytes (72 dwords, 8 banks past a multiple
  // of 64) the rows one read touches fall in different banks (16-byte padding
  // left 0.85 bank-conflict cycles per active LDS cycle on three tiles, this
  // 0.05)
  uint16_t q[R][D + 16];
  // tree verify: bit i of path[r] is set when node i is on row r's path to the root
  uint64_t path[R];
  // tree verify: the sequence's parent array, staged so the path walks read LDS
  int32_t par[64];
};

typedef __attribute__((address_space(3))) void* lds_void_t;

// VLDS: N transposing LDS reads (8 bytes each) at the given LDS byte
// addresses.  In asm, so that the compiler, which cannot tell which LDS bytes
// the buffer-to-LDS loads in flight will write, does not first wait for all of
// them: the caller waits for the loads of the slot it reads, and the reads
// complete inside the block (lgkmcnt(0)) before that slot is loaded again.
template <int N>
__device__ __forceinline__ void read_v_tr(uint2 (&vt)[N], const uint32_t (&ad)[N]);
template <>
__device__ __forceinline__ void read_v_tr<8>(uint2 (&vt)[8], const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %9\n"
      "ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %12\n"
      "ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n"
      "ds_read_b64_tr_b16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(vt[0]), "=v"(vt[1]), "=v"(vt[2]), "=v"(vt[3]), "=v"(vt[4]), "=v"(vt[5]), "=v"(vt[6]), "=v"(vt[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
      : "memory");
}
template <>
__device__ __forceinline__ void read_v_tr<4>(uint2 (&vt)[4], const uint32_t (&ad)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n"
      "ds_read_b64_tr_b16 %1, %5\n"
      "ds_read_b64_tr_b16 %2, %6\n"
      "ds_read_b64_tr_b16 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(vt[0]), "=v"(vt[1]), "=v"(vt[2]), "=v"(vt[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
}

// VLDS: the other LDS reads of the block loop, in asm for the same reason:
// the query operands of one tile (N 16-byte reads 64 bytes apart) and a row's
// tree path mask
template <int N>
__device__ __forceinline__ void read_q(uint4 (&q)[N], uint32_t ad);
template <>
__device__ __forceinline__ void read_q<4>(uint4 (&q)[4], uint32_t ad) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %4 offset:64\n"
      "ds_read_b128 %2, %4 offset:128\n"
      "ds_read_b128 %3, %4 offset:192\n"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(q[0]), "=v"(q[1]), "=v"(q[2]), "=v"(q[3])
      : "v"(ad)
      : "memory");
}
template <>
__device__ __forceinline__ void read_q<2>(uint4 (&q)[2], uint32_t ad) {
  asm volatile(
      "ds_read_b128 %0, %2\n"
      "ds_read_b128 %1, %2 offset:64\n"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(q[0]), "=v"(q[1])
      : "v"(ad)
      : "memory");
}
__device__ __forceinline__ uint64_t read_u64(uint32_t ad) {
  uint64_t x;
  asm volatile(
      "ds_read_b64 %0, %1\n"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(x)
      : "v"(ad)
      : "memory");
  return x;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(size_t)(lds_void_t)(void*)p; }

// s_waitcnt vmcnt(n), other counters left alone (n < 64)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// fp8 (E4M3) code pair (bytes 0-1, or 2-3 when HIGH) -> bf16 pair, exact:
// every E4M3 value is a bf16 value
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, HIGH));
}

// KV8: the caches hold fp8 codes with per-head scales (pa_decode_fp8).  The
// data path differs only in the loads and their conversion to bf16 operands:
//   K   one 16-byte load per pair of k-steps: lane (j, grp) holds dims
//       64 kp + 16 grp .. + 15 of token j, so k-step 2 kp + par uses dims
//       64 kp + 16 grp + 8 par .. + 7 (the query B operand is read from LDS
//       with the same dims; a dot product does not care about the order);
//   V   D / 16 bytes per token: lane j holds columns (D / 16) j .. + D/16 - 1 of
//       tokens 4 grp .. + 3; a byte-level v_perm_b32 gathers column
//       (D / 16) j + 4 h + e of tokens (0, 1) and (2, 3), converted to the bf16
//       pairs of the P V B operand.
// The K scale of the head multiplies the score scale and the V scale the
// normalized output, exact refactorings of scale * q . (s_k k) and sum p (s_v v).
template <int D, int NT, int NW, int NBUF, bool KV8, bool TREE, bool VLDS>
struct MfmaAttender {
  static constexpr int kThreads = NW * 64;
  // the new tokens of pa_decode_append are stored by the schedule before run
  __device__ static bool defers_append(const DecodeParams&) { return false; }
  static constexpr int kD = D;
  static constexpr int R = 16 * NT;  // rows, padded to whole tiles
  static constexpr int KS = D / 32;  // score k-steps
  static constexpr int VH = D / 64;  // value column halves
  static constexpr int KL = KV8 ? KS / 2 : KS;  // K loads (16 bytes) per block
  // the query rows go through LDS unless one tile's fit in registers (tree
  // verify stages them anyway: its path masks need the same barrier)
  static constexpr bool kStageQ = NT > 1 || TREE;
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(!VLDS || (!KV8 && NT > 1), "staged V: bf16, two or more tiles (used with four)");
  // VLDS: bytes of one staged V block, its 16-byte buffer-to-LDS loads (1 KiB
  // per wave each), and the vector memory instructions one block issues
  static constexpr int kVBytes = 16 * D * 2;
  static constexpr int kVLoads = kVBytes / 1024;
  static constexpr int kRing = VLDS ? NW * NBUF * kVBytes : 0;
  static constexpr int kBlockVmem = KL + (VLDS ? kVLoads : 4 * VH);
  // swizzle of token t's chunks: with 32 lanes reading 8 tokens at one
  // column tile, every chunk pair lands in its own banks
  __device__ static constexpr int swz(int t) { return D == 128 ? (t & 7) : ((t >> 1) & 3); }

  const DecodeParams& a;
  MergeTile<R, D, kRing>& sm;
  const int lane, w, j, grp;
  float out_scale = 1.0f;  // V scale of the current head (fp8 caches)

  // value column of MFMA column j of the P V call (h, e)
  __device__ static constexpr int col_of(int jj, int h, int e) {
    return KV8 ? (D / 16) * jj + 4 * h + e : (VLDS ? 64 * h + 16 * e + jj : 4 * jj + 64 * h + e);
  }
  // slot of the merged accumulators (MergeTile::acc) of tile t, call (h, e), lane
  __device__ static constexpr int acc_slot(int t, int h, int e, int ln) { return ((t * VH + h) * 4 + e) * 64 + ln; }

  __device__ MfmaAttender(const DecodeParams& a_, MergeTile<R, D, kRing>& sm_)
      : a(a_),
        sm(sm_),
        lane(threadIdx.x & 63),
        w(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),
        j(threadIdx.x & 15),
        grp((threadIdx.x & 63) >> 4) {}

  __device__ void store(size_t idx, float x) {
    static_cast<uint16_t*>(a.out)[idx] = (uint16_t)f32_to_bf16_bits(x);
  }
  // result() of columns c0 .. c0 + 7 of row r
  __device__ void result8(int r, int c0, float (&x)[8]) const {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float M, l;
      x[k] = result(r, c0 + k, M, l);
    }
  }
  // out[idx .. idx + 7] = x, one 16-byte store (idx a multiple of 8)
  __device__ void store8(size_t idx, const float (&x)[8]) {
    uint4 v;
    v.x = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
    v.y = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
    v.z = f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16);
    v.w = f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + idx) = v;
  }

  __device__ float result(int r, int c, float& M, float& l) const {
    M = sm.m[r];
    l = sm.l[r];
    // the MFMA column (jj, h, e) holding value column c: the inverse of col_of
    const int jj = KV8 ? c / (D / 16) : (VLDS ? c & 15 : (c & 63) >> 2);
    const int h = KV8 ? (c % (D / 16)) >> 2 : c >> 6;
    const int e = VLDS ? (c >> 4) & 3 : c & 3;
    const float x = sm.acc[acc_slot(r >> 4, h, e, 16 * ((r >> 2) & 3) + jj)][r & 3];
    return l > 0.0f ? x * out_scale / l : 0.0f;
  }

  __device__ void run(int b, int g, int L, int lo, int hi) {
    const int rows = a.group * a.q_len;

    // With more than one tile the query rows go to LDS, not registers (three
    // tiles would hold 48 VGPRs for the whole range): the score MFMA of tile t,
    // step ks reads its B operand, row 16 t + j, dims 32 ks + 8 grp .. + 7, from
    // there.  One tile's rows are loaded straight into registers below.
    const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
    if constexpr (kStageQ)
    for (int idx = threadIdx.x; idx < R * (D / 8); idx += kThreads) {
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < rows)
        v = *reinterpret_cast<const uint4*>(
            qp + (((size_t)b * a.q_len + r / a.group) * a.n_h + (size_t)g * a.group + r % a.group) * D + 8 * c8);
      *reinterpret_cast<uint4*>(&sm.q[r][8 * c8]) = v;
    }
    if constexpr (TREE) {
      // the parent array goes to LDS in one load, so that the walks below are a
      // chain of LDS reads rather than of dependent global loads
      for (int i = threadIdx.x; i < a.q_len; i += kThreads) sm.par[i] = a.parents[(size_t)b * a.q_len + i];
      __syncthreads();
      // row r's path to the root: walk the parents while they point to an
      // earlier node (at most q_len - 1 steps)
      for (int r = threadIdx.x; r < R; r += kThreads) {
        uint64_t m = 0;
        if (r < rows) {
          int cur = r / a.group;
          m = 1ull << cur;
          for (int it = 0; it < 64; ++it) {
            const int pp = sm.par[cur];
            if (pp < 0 || pp >= cur) break;
            m |= 1ull << pp;
            cur = pp;
          }
        }
        sm.path[r] = m;
      }
    }
    if constexpr (kStageQ) __syncthreads();
    // causal: row 16 t + j sees positions below vis[t]; tree: the context
    // positions below vis[t] (the tree's start, 0 for padding rows) and the
    // nodes of its path (sm.path)
    int vis[NT];
    bool real[NT];  // row 16 t + j is a query row, not padding of the tile
    const int tree_base = L - a.q_len;  // tree: position of node 0
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = 16 * t + j;
      real[t] = r < rows;
      vis[t] = r < rows ? (TREE ? tree_base : L - a.q_len + r / a.group + 1) : 0;
    }
    // every query row sees all positions below this (tree: the context before node 0)
    const int vis_all = TREE ? tree_base : L - a.q_len + 1;

    float m_ref[NT], m_use[NT], lsum[NT];
    floatx4_t acc[NT][VH][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m_ref[t] = kNegInf;
      m_use[t] = 0.0f;
      lsum[t] = 0.0f;
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][h][e] = (floatx4_t){0.0f, 0.0f, 0.0f, 0.0f};
    }

    constexpr int esz = KV8 ? 1 : 2;
    const uint32_t tok_bytes = (uint32_t)a.n_kv * D * esz;
    const uint32_t blk_bytes = tok_bytes * kBlockTokens;
    const uint32_t head_off = (uint32_t)g * D * esz;
    const uint32_t k_off = (uint32_t)j * tok_bytes + head_off + (uint32_t)grp * 16;
    const uint32_t v_off = (uint32_t)(4 * grp) * tok_bytes + head_off + (uint32_t)j * (KV8 ? D / 16 : 8);
    // VLDS: the LDS byte address lane (a, b) of group grp reads for column tile
    // 0 of slot 0 of this wave's ring (token 4 grp + a, columns 4 b .. + 3; tile
    // ct flips the swizzle bits by 32 ct), and the source offsets of the wave's
    // loads into a slot (instruction i fills slot bytes 1024 i + 16 lane)
    uint32_t vrd = 0;
    uint32_t vld[VLDS ? kVLoads : 1];
    if constexpr (VLDS) {
      const int ta = 4 * grp + ((lane >> 2) & 3), b4 = lane & 3;
      const uint32_t ring = (uint32_t)(size_t)(lds_void_t)(void*)(sm.vring + w * NBUF * kVBytes);
      vrd = ring + (uint32_t)(ta * (2 * D) + 16 * (b4 >> 1) + 8 * (b4 & 1) + 32 * swz(ta));
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {
        const int pos = 1024 * i + 16 * lane;
        const int t = pos / (2 * D), c = ((pos % (2 * D)) >> 4) ^ (2 * swz(t));
        vld[i] = (uint32_t)t * tok_bytes + head_off + 16u * (uint32_t)c;
      }
    }
    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    const int32_t* __restrict__ table = a.tables + (size_t)b * a.max_blocks;
    const float scale_log2 = KV8 ? a.scale_log2 * a.k_scale[g] : a.scale_log2;
    if constexpr (KV8) out_scale = a.v_scale[g];
    const int n_mine = hi - lo > w ? (hi - lo - w + NW - 1) / NW : 0;

    auto block_ids = [&](int k0, int cnt) { return lane < cnt ? table[lo + w + NW * (k0 + lane)] : 0; };

    // K: KL loads of 16 bytes; V: 4 tokens x VH halves of 8 bytes (bf16), or
    // 4 tokens x D/16 bytes (fp8, in vb[v][0])
    // V loads are non-temporal (cache policy nt), K loads ordinary.  Two
    // alternating runs, us: 70B 193.8 / 194.3 against 208.8 / 208.1, fp8 8B
    // (cold) 57.2 / 56.9 against 60.9 / 61.5, speculative verify 227.3 / 227.0
    // against 237.3 / 235.9, tree verify 217.6 / 217.6 against 226.1 / 226.9.
    // Non-temporal K loads made every one of them slower (224.9, 65.1, 252.0,
    // 234.2 us), and so did both together.
    constexpr int kVPolicy = 2;
    auto issue = [&](int ids, int cnt, int k0, int kk, uint4(&kb)[KL], uint2(&vb)[4][VH], int& lblk, bool& ok,
                     int su) {
      const int phys = __builtin_amdgcn_readlane(ids, kk < cnt ? kk : 0);
      ok = kk < cnt && (unsigned)phys < (unsigned)a.num_blocks;
      lblk = lo + w + NW * (k0 + kk);
      const int valid = min(kBlockTokens, L - lblk * kBlockTokens);
      const size_t boff = ok ? (size_t)phys * blk_bytes : 0;
      const uint32_t nrec = ok ? (uint32_t)valid * tok_bytes : 0u;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + boff), (short)0, (int)nrec, kBufferWord3);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + boff), (short)0, (int)nrec, kBufferWord3);
#pragma unroll
      for (int kl = 0; kl < KL; ++kl)
        kb[kl] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off + 64 * kl, 0, 0));
      if constexpr (VLDS) {
        // V into slot su of this wave's ring
        char* slot = reinterpret_cast<char*>(sm.vring) + (w * NBUF + su) * kVBytes;
#pragma unroll
        for (int i = 0; i < kVLoads; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t)(slot + 1024 * i), 16, (int)vld[i], 0, 0, kVPolicy);
      } else if constexpr (KV8) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if constexpr (D == 128)
            vb[v][0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, v_off, v * tok_bytes, kVPolicy));
          else
            vb[v][0] = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(vr, v_off, v * tok_bytes, kVPolicy), 0u);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int h = 0; h < VH; ++h)
            vb[v][h] = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, v_off + 128 * h, v * tok_bytes, kVPolicy));
      }
    };

    // A operand of score k-step ks: 8 dims of K as bf16
    auto k_operand = [&](const uint4(&kb)[KL], int ks) -> uint4 {
      if constexpr (KV8) {
        const uint4 c = kb[ks / 2];
        const uint32_t lo = (ks & 1) ? c.z : c.x, hi = (ks & 1) ? c.w : c.y;
        return make_uint4(fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo), fp8x2_to_bf16x2<false>(hi),
                          fp8x2_to_bf16x2<true>(hi));
      } else {
        return kb[ks];
      }
    };

    // one tile: its query operands fit in registers for the whole range (16
    // VGPRs at head_dim 128); more tiles read them from LDS at every block
    auto q_dim = [&](int ks) { return KV8 ? 64 * (ks / 2) + 16 * grp + 8 * (ks & 1) : 32 * ks + 8 * grp; };
    uint4 qreg[NT == 1 ? KS : 1];
    if constexpr (NT == 1) {
      if constexpr (kStageQ) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = *reinterpret_cast<const uint4*>(&sm.q[j][q_dim(ks)]);
      } else {
        // row j of the tile, straight from memory (zero for padding rows); the
        // block-table load that follows shares these loads' round trip
        const uint16_t* qrow = qp + (((size_t)b * a.q_len + j / a.group) * a.n_h + (size_t)g * a.group + j % a.group) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qreg[ks] = j < rows ? *reinterpret_cast<const uint4*>(qrow + q_dim(ks)) : make_uint4(0, 0, 0, 0);
      }
    }

    // scores: s[t][v] = row 16 t + j against token 4 grp + v, log2 units, -inf where masked
    auto scores = [&](const uint4(&kb)[KL], int lblk, bool ok, floatx4_t(&s)[NT]) {
      const int pos0 = lblk * kBlockTokens + 4 * grp;
      // keep the compiler from hoisting the query reads out of the block loop
      // into registers, which is what the LDS copy avoids
      if constexpr (NT > 1) asm volatile("" ::: "memory");
      // raw q.k of tile t
      auto tile = [&](int t) -> floatx4_t {
        floatx4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
        uint4 qv[VLDS ? KS : 1];
        if constexpr (VLDS) read_q<KS>(qv, lds_addr(&sm.q[16 * t + j][q_dim(0)]));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint4 qb;
          if constexpr (NT == 1) qb = qreg[ks];
          else if constexpr (VLDS) qb = qv[ks];
          else qb = *reinterpret_cast<const uint4*>(&sm.q[16 * t + j][q_dim(ks)]);
          x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k_operand(kb, ks)),
                                                      __builtin_bit_cast(bf16x8_t, qb), x, 0, 0, 0);
        }
        return x;
      };
      if constexpr (TREE) {
        floatx4_t x[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) x[t] = tile(t);
        // One wave-uniform branch per block: where every query row sees the
        // whole block only the padding rows are masked; otherwise each score
        // is checked against its row's context bound and tree path.
        if (ok && lblk * kBlockTokens + kBlockTokens <= vis_all) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) s[t][v] = real[t] ? x[t][v] * scale_log2 : kNegInf;
        } else {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint64_t path = VLDS ? read_u64(lds_addr(&sm.path[16 * t + j])) : sm.path[16 * t + j];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int rel = pos0 + v - tree_base;  // node index of the position, negative before the tree
              const bool see = pos0 + v < vis[t] || (rel >= 0 && rel < 64 && ((path >> rel) & 1ull));
              s[t][v] = (ok && see) ? x[t][v] * scale_log2 : kNegInf;
            }
          }
        }
      } else {
        // causal: one select per score (measured no slower than a branch here)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const floatx4_t x = tile(t);
#pragma unroll
          for (int v = 0; v < 4; ++v) s[t][v] = (ok && pos0 + v < vis[t]) ? x[v] * scale_log2 : kNegInf;
        }
      }
    };

    // (VLDS: the caller has waited for the loads of slot su)
    auto accumulate = [&](const floatx4_t(&s)[NT], const uint2(&vb)[4][VH], int su) {
      // B operands of P V: column col_of(j, h, e) of the 4 tokens, bf16 pairs (tokens 0,1), (2,3)
      uint2 vt[VH][4];
      if constexpr (VLDS) {
        uint32_t ad[4 * VH];
        uint2 vr[4 * VH];
#pragma unroll
        for (int ct = 0; ct < 4 * VH; ++ct) ad[ct] = (vrd ^ (32u * ct)) + (uint32_t)(su * kVBytes);
        read_v_tr<4 * VH>(vr, ad);
#pragma unroll
        for (int ct = 0; ct < 4 * VH; ++ct) vt[ct >> 2][ct & 3] = vr[ct];
      } else
#pragma unroll
      for (int h = 0; h < VH; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (KV8) {
            // byte e of dword h of tokens (0, 1) and (2, 3), then fp8 -> bf16
            const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + e) << 8) | (uint32_t)e;
            const uint32_t d0 = h ? vb[0][0].y : vb[0][0].x, d1 = h ? vb[1][0].y : vb[1][0].x;
            const uint32_t d2 = h ? vb[2][0].y : vb[2][0].x, d3 = h ? vb[3][0].y : vb[3][0].x;
            vt[h][e].x = fp8x2_to_bf16x2<false>(__builtin_amdgcn_perm(d1, d0, sel));
            vt[h][e].y = fp8x2_to_bf16x2<false>(__builtin_amdgcn_perm(d3, d2, sel));
          } else {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t w01 = (e < 2) ? 0 : 1;
            vt[h][e].x = __builtin_amdgcn_perm(w01 ? vb[1][h].y : vb[1][h].x, w01 ? vb[0][h].y : vb[0][h].x, sel);
            vt[h][e].y = __builtin_amdgcn_perm(w01 ? vb[3][h].y : vb[3][h].x, w01 ? vb[2][h].y : vb[2][h].x, sel);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float p[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) p[v] = fast_exp2(s[t][v] - m_use[t]);
        uint2 pa2;
        pa2.x = pack_bf16(p[0], p[1]);
        pa2.y = pack_bf16(p[2], p[3]);
        // the row sum adds the same rounded weights the product uses
        lsum[t] += (bf16_lo(pa2.x) + bf16_hi(pa2.x)) + (bf16_lo(pa2.y) + bf16_hi(pa2.y));
#pragma unroll
        for (int h = 0; h < VH; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[t][h][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(short4_t, pa2), __builtin_bit_cast(short4_t, vt[h][e]), acc[t][h][e], 0, 0, 0);
      }
    };

    // per-row reference: the row's maximum over the block (lanes j, j+16, j+32, j+48 share a row)
    auto set_reference = [&](const floatx4_t(&mx)[NT]) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float x = fmaxf(fmaxf(mx[t][0], mx[t][1]), fmaxf(mx[t][2], mx[t][3]));
        x = fmaxf(x, shfl_xor(x, 16));
        x = fmaxf(x, shfl_xor(x, 32));
        m_ref[t] = x;
        m_use[t] = x == kNegInf ? 0.0f : x;
      }
    };

    bool overflow = false;  // wave-uniform
    for (int k0 = 0; k0 < n_mine; k0 += 64) {
      const int cnt = min(64, n_mine - k0);
      const int ids = block_ids(k0, cnt);
      uint4 kb[NBUF][KL];
      uint2 vb[NBUF][4][VH];
      int lb[NBUF];
      bool okb[NBUF];
#pragma unroll
      for (int u = 0; u < NBUF; ++u) issue(ids, cnt, k0, u, kb[u], vb[u], lb[u], okb[u], u);
      if (k0 == 0) {
        floatx4_t s0[NT];
        scores(kb[0], lb[0], okb[0], s0);
        set_reference(s0);
      }
      for (int kk = 0; kk < cnt; kk += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          if (kk + u < cnt) {
            floatx4_t s[NT];
            scores(kb[u], lb[u], okb[u], s);
            bool big = false;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
              for (int v = 0; v < 4; ++v) big |= s[t][v] > m_ref[t] + kOverflowSlack;
            overflow |= __builtin_amdgcn_ballot_w64(big) != 0;
            // the loads of the NBUF - 1 blocks after this one may still be in flight
            if constexpr (VLDS) wait_vmcnt<(NBUF - 1) * kBlockVmem>();
            accumulate(s, vb[u], u);
          }
          issue(ids, cnt, k0, kk + u + NBUF, kb[u], vb[u], lb[u], okb[u], u);
        }
      }
    }

    if (overflow) {
      // exact redo of this wave's share: row maxima first, then the weighted sums
      floatx4_t mx[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        mx[t] = (floatx4_t){kNegInf, kNegInf, kNegInf, kNegInf};
        lsum[t] = 0.0f;
#pragma unroll
        for (int h = 0; h < VH; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][h][e] = (floatx4_t){0.0f, 0.0f, 0.0f, 0.0f};
      }
      for (int k0 = 0; k0 < n_mine; k0 += 64) {
        const int cnt = min(64, n_mine - k0);
        const int ids = block_ids(k0, cnt);
        for (int kk = 0; kk < cnt; ++kk) {
          uint4 kb1[KL];
          uint2 vb1[4][VH];
          int lb1;
          bool ok1;
          issue(ids, cnt, k0, kk, kb1, vb1, lb1, ok1, 0);
          floatx4_t s[NT];
          scores(kb1, lb1, ok1, s);
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) mx[t][v] = fmaxf(mx[t][v], s[t][v]);
        }
      }
      set_reference(mx);
      for (int k0 = 0; k0 < n_mine; k0 += 64) {
        const int cnt = min(64, n_mine - k0);
        const int ids = block_ids(k0, cnt);
        for (int kk = 0; kk < cnt; ++kk) {
          uint4 kb1[KL];
          uint2 vb1[4][VH];
          int lb1;
          bool ok1;
          issue(ids, cnt, k0, kk, kb1, vb1, lb1, ok1, 0);
          floatx4_t s[NT];
          scores(kb1, lb1, ok1, s);
          if constexpr (VLDS) wait_vmcnt<0>();
          accumulate(s, vb1, 0);
        }
      }
    }

    // row sums over the 4 token groups; lanes j, j+16, j+32, j+48 then hold row 16 t + j
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float x = lsum[t];
      x += shfl_xor(x, 16);
      x += shfl_xor(x, 32);
      lsum[t] = x;
    }

    // merge the waves one after the other into the LDS tile (VLDS: no load into
    // this wave's ring, which holds the tile's bytes, is still in flight)
    if constexpr (VLDS) wait_vmcnt<0>();
    __syncthreads();  // the previous range's tile has been read
    for (int u = 0; u < NW; ++u) {
      if (w == u) {
        if (grp == 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            sm.wm[16 * t + j] = m_ref[t];
            sm.wl[16 * t + j] = lsum[t];
          }
        }
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // rescaling factors of this lane's 4 rows 16 t + 4 grp + v
          floatx4_t f_old = {0.0f, 0.0f, 0.0f, 0.0f}, f_new = {1.0f, 1.0f, 1.0f, 1.0f};
          if (u > 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int r = 16 * t + 4 * grp + v;
              const float mo = sm.m[r], mw = sm.wm[r];
              const float M = fmaxf(mo, mw);
              f_old[v] = M == kNegInf ? 0.0f : fast_exp2(mo - M);
              f_new[v] = M == kNegInf ? 0.0f : fast_exp2(mw - M);
            }
          }
#pragma unroll
          for (int h = 0; h < VH; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              floatx4_t& dst = sm.acc[acc_slot(t, h, e, lane)];
              dst = (u > 0 ? dst * f_old : (floatx4_t){0.0f, 0.0f, 0.0f, 0.0f}) + acc[t][h][e] * f_new;
            }
        }
        wave_lds_sync();
        if (grp == 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int r = 16 * t + j;
            if (u == 0) {
              sm.m[r] = m_ref[t];
              sm.l[r] = lsum[t];
            } else {
              const float mo = sm.m[r];
              const float M = fmaxf(mo, m_ref[t]);
              const float f_old = M == kNegInf ? 0.0f : fast_exp2(mo - M);
              const float f_new = M == kNegInf ? 0.0f : fast_exp2(m_ref[t] - M);
              sm.l[r] = sm.l[r] * f_old + lsum[t] * f_new;
              sm.m[r] = M;
            }
          }
        }
      }
      __syncthreads();
    }
  }
};

template <int D, int NT, int NW, int NBUF, bool BALANCED, bool KV8, bool TREE, bool VLDS>
// Up to three row tiles the kernel is asked for two waves per SIMD: without
// the bound the allocator keeps values hoisted out of a balanced range's loop
// over sequences and lands at one wave per SIMD, while with it everything fits
// without spilling.  Four tiles fit two waves too in the fixed schedules (two
// blocks in flight, V staged in LDS); the balanced one would spill, so it keeps
// one wave.
__global__ __launch_bounds__(NW * 64, (NT <= 3 || !BALANCED) ? 2 : 1) void decode_mfma_kernel(DecodeParams a) {
  using Attn = MfmaAttender<D, NT, NW, NBUF, KV8, TREE, VLDS>;
  __shared__ MergeTile<16 * NT, D, Attn::kRing> sm;
  Attn at(a, sm);
  if constexpr (BALANCED) drive_balanced(a, at);
  else drive_fixed(a, at);
}

template <int D, int NT, bool KV8, bool TREE>
hipError_t launch_tiles(const DecodeParams& p, hipStream_t s) {
  // Fixed schedules.  Four bf16 tiles stage V in LDS, which leaves registers
  // for two blocks of K in flight per wave where V in registers left one (15-node
  // tree verify on the 8B shape: 226.9 against 232.2 us).  Fewer tiles keep V
  // in registers: staging measured the same there (speculative verify, three
  // tiles: 235.7-236.6 us either way).
  constexpr bool VL = !KV8 && NT >= 4;
  constexpr int NB = VL ? 2 : (NT >= 4 ? 1 : (NT >= 3 ? 2 : 3));  // blocks in flight per wave
  if (p.mode == kBalanced) {
    // one block in flight per wave, as in the vector-ALU kernel: cheaper
    // pipeline restarts at the sequences a range crosses (70B layer: 221 us
    // against 239 us with three)
    static const int resident =
        resident_per_cu(decode_mfma_kernel<D, NT, kWaves, 1, true, KV8, TREE, false>, kWaves * 64);
    DecodeParams q = p;
    q.num_wgs = balanced_workgroups(resident, p.n_kv);
    hipLaunchKernelGGL((decode_mfma_kernel<D, NT, kWaves, 1, true, KV8, TREE, false>), dim3(q.num_wgs), dim3(kWaves * 64),
                       0, s, q);
  } else {
    DecodeParams q = p;
    if (p.mode == kSinglePass) {
      static const int resident =
          resident_per_cu(decode_mfma_kernel<D, NT, kWaves, NB, false, KV8, TREE, VL>, kWaves * 64);
      q.pair_stride = one_pass_pairing(resident, p.num_seqs, p.n_kv);
    }
    dim3 grid(p.mode == kPartitions ? p.num_parts : 1, p.n_kv, p.num_seqs);
    hipLaunchKernelGGL((decode_mfma_kernel<D, NT, kWaves, NB, false, KV8, TREE, VL>), grid, dim3(kWaves * 64), 0, s, q);
  }
  return hipGetLastError();
}

template <int D, bool KV8, bool TREE = false>
hipError_t launch_rows(const DecodeParams& p, int rows, hipStream_t s) {
  if (rows <= 16) return launch_tiles<D, 1, KV8, TREE>(p, s);
  if (rows <= 32) return launch_tiles<D, 2, KV8, TREE>(p, s);
  if (rows <= 48) return launch_tiles<D, 3, KV8, TREE>(p, s);
  return launch_tiles<D, 4, KV8, TREE>(p, s);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, int rows_per_kv, hipStream_t s) {
  return head_dim == 64 ? launch_rows<64, false>(p, rows_per_kv, s) : launch_rows<128, false>(p, rows_per_kv, s);
}

hipError_t launch_decode_mfma_fp8(const DecodeParams& p, int head_dim, int rows_per_kv, hipStream_t s) {
  return head_dim == 64 ? launch_rows<64, true>(p, rows_per_kv, s) : launch_rows<128, true>(p, rows_per_kv, s);
}

hipError_t launch_decode_mfma_tree(const DecodeParams& p, int head_dim, int rows_per_kv, hipStream_t s) {
  return head_dim == 64 ? launch_rows<64, false, true>(p, rows_per_kv, s)
                        : launch_rows<128, false, true>(p, rows_per_kv, s);
}

}  // namespace pa
