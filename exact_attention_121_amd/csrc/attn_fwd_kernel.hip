// Fused exact-attention forward for gfx950 (AMD Instinct MI355X, CDNA4).
//
// One workgroup computes 128 query rows of one (batch, query head): it keeps
// the rows' Q in registers, streams the key/value sequence through LDS in
// tiles, and for each tile computes the scores on the matrix cores, updates
// the online softmax state and accumulates P.V on the matrix cores, so the
// N x N score matrix never leaves the chip.  This is the flow of [CANN-FA]
// sections "Tiling on the Ascend NPU" and "Concrete flow" (one block per Q
// row-block, an inner loop over K/V blocks, running max m and running sum l,
// rescaling of the partial output) and of [FA-Dict] section "Fused kernel",
// with the normalisation deferred to the end ([CANN-FA], the paragraph on the
// online softmax being the key; [FA-Dict] section "Online softmax").
//
// Pages cited:
//   [CANN-FA]  www.mooersco.com/news/1200175 - "FlashAttention operator of the
//              CANN ops-transformer repository: attention acceleration on the
//              Ascend NPU"
//   [FA-Dict]  hwcomputing.csdn.net/6a0dbd08662f9a54cb75eb74.html
//   [FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html
//
// gfx950 mapping
//   * 256 threads = 4 waves of 64; wave w owns query rows q0+32w .. q0+32w+31.
//     Two workgroups share a CU (<= 256 registers per lane, 64 KB of LDS
//     each), so every SIMD interleaves the matrix-core work of one wave with
//     the softmax arithmetic of the other.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_f16: A = 32 keys x 16 dims from LDS, B = 16 dims x
//     32 queries from registers.  In the 32x32 fp32 result, lane L holds query
//     L%32 and the 16 keys 8*(r/4) + 4*(L/32) + r%4 (r = 0..15), so each
//     query's row max is an in-lane reduction plus one v_permlane32_swap with
//     lane L^32, and its row sum stays a per-lane partial until the end.
//   * The probabilities stay in registers and are the B operand of
//     O^T += V^T P^T (same instruction).  The reduction index of that product
//     may be permuted freely, so the eight B slots of lane L simply take the
//     lane's own probability registers; the A operand must then pair slot j of
//     lane group L/32 with key 8*(j/4) + 4*(L/32) + j%4 (+16 per half).  Two
//     ds_read_b64_tr_b16 transpose-reads fetch exactly those keys (4 each)
//     from V kept in its natural [key][dim] layout.
//   * K and V tiles move from device memory straight into LDS with
//     buffer_load_dwordx4 ... lds (no register staging; reads past the end of
//     the sequence return zeros), double-buffered per operand: K_{j+1} and
//     V_j are resident while V_{j+1} and K_{j+2} are in flight ([CANN-FA]
//     section "Ascend C implementation": load block j+1 while block j is
//     computed so that data movement hides behind the matrix unit).  16-byte
//     chunks are XOR-swizzled by row so that the matrix-operand reads hit
//     distinct LDS banks.
//   * Software pipeline per wave: iteration j computes S_{j+1} = K_{j+1} Q^T
//     on the matrix cores interleaved with the softmax of tile j on the
//     vector ALUs, then O += P_j V_j interleaved with the row max of S_{j+1}.
//   * exp is exp2 with scale*log2(e) folded into one fused multiply-add.  The
//     running max is raised lazily (only when a row's new logits exceed it by
//     more than 8 in log2 units), so the O rescale is rare and probabilities
//     stay <= 256; row sums add the fp16 probabilities with v_dot2.
//   * Causal: key tiles entirely above a wave's diagonal are skipped; only
//     tiles crossing the diagonal or the end of the sequence are masked.
//   * Workgroup ids are remapped so that each of the 8 XCDs (each with its
//     own L2) receives a contiguous range of (head, query tile) work, i.e. the
//     query tiles of the same heads share their K/V in one L2; causal query
//     tiles run heaviest first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int kThreads = 256;  // 4 waves of 64 lanes
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.69314718055994531f;
// Buffer resource word 3 for raw (unformatted, stride 0) buffer access on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

// Query blocks of 32 rows per wave, per head_dim.  Two blocks per wave let
// every K/V operand read from LDS feed two matrix instructions and halve the
// K/V traffic per query row (the workgroup covers 256 rows); that needs more
// than 256 registers per lane, so those kernels run one wave per SIMD.
#ifndef ATTN_QB64
#define ATTN_QB64 1
#endif
#ifndef ATTN_QB128
#define ATTN_QB128 1
#endif
#ifndef ATTN_QB256
#define ATTN_QB256 1
#endif
template <int D>
constexpr int query_blocks() {
  return D == 64 ? ATTN_QB64 : (D == 128 ? ATTN_QB128 : ATTN_QB256);
}

template <int D>
struct Cfg {
  static constexpr int QB = query_blocks<D>();     // 32-row query blocks per wave
  static constexpr int WAVE_ROWS = 32 * QB;        // query rows per wave
  static constexpr int BM = kWaves * WAVE_ROWS;    // query rows per workgroup
  static constexpr int BN = (D == 256) ? 32 : 64;  // keys per K/V tile
  static constexpr int NT = BN / 32;               // 32-key sub-tiles of S^T
  static constexpr int DC = D / 16;                // 16-dim k-steps of Q.K
  static constexpr int DT = D / 32;                // 32-dim row tiles of O^T
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D * 2;    // one K (or V) tile
  static constexpr int LOADS = BN * CPR / kThreads;  // 16-byte loads per thread per tile
  // Workgroups per CU the register budget allows.
  static constexpr int WG_PER_CU = (QB == 1 && D != 256) ? 2 : 1;
  // Matrix operands read from LDS ahead of their MFMA (K reads; twice as
  // many V transpose reads, two per MFMA); measured on gfx950.
  static constexpr int K_AHEAD = D == 256 ? 6 : 4;
  static_assert(BN * CPR % kThreads == 0, "tile must split evenly over the workgroup");
};

struct Params {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* lse;
  int N, Hq, Hkv, group, q_tiles;
  float c;          // |scale| * log2(e), or 1 when scale = 0 (Q is then zeroed): always > 0
  uint32_t q_sign;  // 0x80008000 when scale < 0 (Q is negated on load), else 0
  uint32_t q_keep;  // 0 when scale = 0 (every logit is then exactly 0), else all ones
};

// Byte offset of 16-byte chunk `c` of row `r` inside a swizzled tile: the
// chunk index is XORed with a function of the row's low four bits, chosen
// (by exhaustive search over XOR-linear maps) so that both operand reads are
// free of bank conflicts whether the LDS serves 128 or 256 bytes per clock:
//   * K reads (ds_read_b128): 8 or 16 consecutive rows at one chunk;
//   * V transpose reads (ds_read_b64_tr_b16): 4 consecutive keys x 4 chunks.
// Rows of 256+ bytes use a 4-bit map; 128-byte rows (d = 64), where row
// parity already selects the bank half, use a 3-bit map.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr uint64_t kMap16 = 0x73d962c8fb51ea40ull;  // f(r) for r = 0..15, 4 bits each
  constexpr uint64_t kMap8 = 0x4703652156127430ull;   // 3-bit variant for 128-byte rows
  constexpr uint64_t map = Cfg<D>::CPR >= 16 ? kMap16 : kMap8;
  const int f = static_cast<int>((map >> (4 * (r & 15))) & 15);
  return (r * Cfg<D>::CPR + (c ^ f)) * 16;
}

// Byte offsets, relative to a tile's first row, of the 16-byte chunks that
// thread `tid` copies into a swizzled tile (the chunk that belongs at
// position p % CPR of row p / CPR of the tile).
template <int D>
struct LoadOffsets {
  uint32_t src[Cfg<D>::LOADS];
  __device__ __forceinline__ void init(int tid) {
    using C = Cfg<D>;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int p = i * kThreads + tid;  // destination chunk; lanes of a wave are consecutive
      const int row = p / C::CPR;
      const int chunk = (swz<D>(row, p % C::CPR) >> 4) - row * C::CPR;
      src[i] = static_cast<uint32_t>((row * D + chunk * 8) * 2);
    }
  }
};

// A tile base at or above 2^31 bytes lies outside every K/V head (a head is
// at most 2^31 bytes), so each read of the tile fails the buffer range check:
// no memory is touched and the stage receives zeros.  Used for tiles past
// the end of the loop, so that the load instructions need no branch.
constexpr uint32_t kSkipTile = 0x80000000u;

// Queue the copy of the tile whose first row starts at byte `base` of one K
// or V head into a swizzled LDS tile.  Rows at or past N read as zeros
// (buffer range check).
template <int D>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rsrc, char* tile, uint32_t base,
                                          const LoadOffsets<D>& lo, int tid) {
  using C = Cfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    char* dst = tile + (i * kThreads + (tid & ~63)) * 16;  // wave-uniform base
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, static_cast<int>(base + lo.src[i]),
                                             0, 0, 0);
  }
}

// Byte offset of the first row of key tile j inside a head, or kSkipTile.
template <int D>
__device__ __forceinline__ uint32_t tile_base(int j, int nt) {
  return j < nt ? static_cast<uint32_t>(j) * (Cfg<D>::BN * D * 2) : kSkipTile;
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ short4v tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
}

__device__ __forceinline__ float xlane_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float xlane_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Per-lane LDS byte offsets of the matrix operands inside a (swizzled) tile.
// Tile rows 32*t + 16*h (K) or key groups (V) only add a constant, so every
// operand read is one of these registers plus an immediate offset.
template <int D>
struct Offsets {
  int k[Cfg<D>::DC];       // K rows lane%32 (+32 t), chunk 2 dc + lane/32
  int v[2][Cfg<D>::DT];    // V keys 4 g + (lane%16)/4 (+8 for [1]), dims of row tile dt
  __device__ __forceinline__ void init(int lane) {
    using C = Cfg<D>;
    const int lr = lane & 31, g = lane >> 5, m16 = lane & 15;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) k[dc] = swz<D>(lr, 2 * dc + g);
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (m16 & 3);  // dim offset inside a 32-dim tile
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const int dim = 32 * dt + dsub;
        v[hi][dt] = swz<D>(4 * g + (m16 >> 2) + 8 * hi, dim >> 3) + (dim & 7) * 2;
      }
  }
};

template <int D>
using STile = f32x16[Cfg<D>::QB][Cfg<D>::NT];  // logits of one key tile, per query block
template <int D>
using PTile = half8[Cfg<D>::QB][Cfg<D>::NT][2];  // fp16 probabilities of one key tile
template <int D>
using OAcc = f32x16[Cfg<D>::QB][Cfg<D>::DT];  // output accumulators O^T
template <int D>
using QFrag = half8[Cfg<D>::QB][Cfg<D>::DC];  // Q rows as B operands

// S^T = K Q^T for one key tile: s[qb][t] holds keys 32 t .. 32 t + 31 (rows
// of the 32x32 result) against query block qb (columns).  Each K operand
// read from LDS serves every query block of the wave.
template <int D>
__device__ __forceinline__ void qk_tile(const char* ks, const QFrag<D>& qf, const Offsets<D>& off,
                                        STile<D>& s) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int t = 0; t < C::NT; ++t) s[qb][t] = f32x16{};
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const half8 a = *reinterpret_cast<const half8*>(ks + off.k[dc] + 32 * t * C::CPR * 16);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
        s[qb][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[qb][dc], s[qb][t], 0, 0, 0);
    }
}

// Keys past the end of the sequence, or after the query when causal, get
// logit -inf (then exp2 gives exactly 0).  Lane L holds keys
// 32 t + 8 (r/4) + 4 (L/32) + r%4 of query row `qrow` (+32 per block).
template <int D, bool CAUSAL>
__device__ __forceinline__ void mask_tile(STile<D>& s, int kv0, int N, int qrow, int g) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = key < N && (!CAUSAL || key <= qrow + 32 * qb);
        s[qb][t][r] = ok ? s[qb][t][r] : -INFINITY;
      }
}

// Row maxima of a tile's raw logits, in log2 units (c > 0).
template <int D>
__device__ __forceinline__ void tile_max(const STile<D>& s, float c, float (&m)[Cfg<D>::QB]) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    float mx = s[qb][0][0];
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = (t == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[qb][t][r]);
    m[qb] = xlane_max(mx) * c;
  }
}

// The running maximum m is only raised when some row of the wave saw a logit
// more than kLazy (log2 units) above it.  Probabilities are taken relative
// to m, so they stay <= 2^kLazy (exact in fp16, no overflow in fp32) and the
// result is the same function: every term of the numerator and of l shares
// the same reference m, which cancels in O = sum(p v) / sum(p) and is added
// back in LSE = m + log2 l.
constexpr float kLazy = 8.0f;

template <int D>
__device__ __forceinline__ void raise_max(const float (&m_tile)[Cfg<D>::QB], float (&m_run)[Cfg<D>::QB],
                                          float (&l_run)[Cfg<D>::QB], OAcc<D>& oacc) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    if (__any(m_tile[qb] > m_run[qb] + kLazy)) {
      const float m_new = fmaxf(m_run[qb], m_tile[qb]);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);  // 0 while m_run = -inf
      m_run[qb] = m_new;
      l_run[qb] *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) oacc[qb][dt] *= alpha;
    }
  }
}

// P = exp2(c S - m) rounded to fp16: the B operand of the P.V product, in
// the lane's own key order.
template <int D>
__device__ __forceinline__ void softmax_tile(const STile<D>& s, float c, const float (&m_run)[Cfg<D>::QB],
                                             PTile<D>& pf) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pf[qb][t][r >> 3][r & 7] =
            static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][t][r], c, -m_run[qb])));
}

// Adds the sum of the fp16 probabilities (exactly the values multiplied
// into V) to the lane's partial row sums l.
template <int D>
__device__ __forceinline__ void add_row_sums(const PTile<D>& pf, float (&l_run)[Cfg<D>::QB]) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
      {
        const half8 x = pf[qb][t][h];
        l0 = __builtin_amdgcn_fdot2(half2v{x[0], x[1]}, half2v{1.0f16, 1.0f16}, l0, false);
        l1 = __builtin_amdgcn_fdot2(half2v{x[2], x[3]}, half2v{1.0f16, 1.0f16}, l1, false);
        l0 = __builtin_amdgcn_fdot2(half2v{x[4], x[5]}, half2v{1.0f16, 1.0f16}, l0, false);
        l1 = __builtin_amdgcn_fdot2(half2v{x[6], x[7]}, half2v{1.0f16, 1.0f16}, l1, false);
      }
    l_run[qb] += l0 + l1;
  }
}

// O^T += V^T P^T for one key tile.  The A operand pairs B slot j of lane
// group g with key 8 (j/4) + 4 g + j%4 (+16 h, +32 t): two transpose reads of
// four keys each from V in its natural [key][dim] layout, shared by every
// query block of the wave.
template <int D>
__device__ __forceinline__ void pv_tile(const char* vs, const PTile<D>& pf, const Offsets<D>& off,
                                        OAcc<D>& oacc) {
  using C = Cfg<D>;
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = (32 * t + 16 * h) * C::CPR * 16;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const short4v lo = tr_read(vs + off.v[0][dt] + kb);
        const short4v hi = tr_read(vs + off.v[1][dt] + kb);
        const half8 a = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
          oacc[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[qb][t][h], oacc[qb][dt], 0, 0, 0);
      }
    }
}

// Per-wave state of the software pipeline.
template <int D>
struct WaveState {
  QFrag<D> qf;
  OAcc<D> oacc;
  Offsets<D> off;
  float m_run[Cfg<D>::QB], l_run[Cfg<D>::QB];
  float c;
  int N, qw0, qrow, g, nt_w;  // qrow: row of this lane in block 0; nt_w: key tiles this wave computes
};

// LDS layout: K tiles in stages 0/1, then V tiles in stages 0/1.
template <int D>
__device__ __forceinline__ char* k_stage(char* smem, int st) { return smem + st * Cfg<D>::TILE_BYTES; }
template <int D>
__device__ __forceinline__ char* v_stage(char* smem, int st) { return smem + (2 + st) * Cfg<D>::TILE_BYTES; }

// Instruction groups for the compiler's scheduler (masks of
// __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedVMEMRead = 0x020, kSchedDSRead = 0x100;

// Iteration j of the pipeline ([CANN-FA] section "Concrete flow": scores,
// online-softmax update and P.V for key block j).  On entry K_{j+1} sits in
// K stage (j+1)&1, V_j in V stage j&1, and s_cur holds the masked logits of
// tile j with the running max already raised for them.  The matrix cores
// compute S_{j+1} = K_{j+1} Q^T while the vector ALUs turn s_cur into P_j;
// then O += P_j V_j runs while the vector ALUs reduce S_{j+1}.  Meanwhile
// V_{j+1} and K_{j+2} stream into the stages freed by the previous iteration
// ([CANN-FA] section "Ascend C implementation": load the next block while the
// current one is computed).
template <int D, bool CAUSAL, int PAR>
__device__ __forceinline__ void pipeline_step(int j, int nt, char* smem,
                                              __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                              const LoadOffsets<D>& lo, int tid, WaveState<D>& w,
                                              STile<D>& s_cur, STile<D>& s_nxt) {
  using C = Cfg<D>;
  const uint32_t v_base = tile_base<D>(j + 1, nt);
  const uint32_t k_base = tile_base<D>(j + 2, nt);
  if (j < w.nt_w) {
    load_tile<D>(vrs, v_stage<D>(smem, PAR ^ 1), v_base, lo, tid);
    load_tile<D>(krs, k_stage<D>(smem, PAR), k_base, lo, tid);
    // S_{j+1} is computed even past this wave's last tile (reading a stale
    // but in-bounds stage) so that the matrix and vector work stay in one
    // block the scheduler can interleave; it is discarded then.
    qk_tile<D>(k_stage<D>(smem, PAR ^ 1), w.qf, w.off, s_nxt);
    PTile<D> pf;
    softmax_tile<D>(s_cur, w.c, w.m_run, pf);
    // Materialise P_j here, so that the compiler keeps the softmax next to
    // the S_{j+1} product instead of sinking it past the mask branch.
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) asm volatile("" ::"v"(pf[qb][t][h]));
    if constexpr (C::DC >= 8) {
      // One MFMA of S_{j+1}, then a share of the softmax of tile j; a K
      // operand read per group of query blocks; the V/K copies ride along.
      // (With d = 64 the compiler's own order measured faster.)
      constexpr int kMfma = C::DC * C::NT * C::QB;
      constexpr int kValu = (3 * 16 * C::NT * C::QB + kMfma - 1) / kMfma;
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, C::K_AHEAD, 0);
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, kValu, 0);
        if (i % C::QB == C::QB - 1) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        if (i < 2 * C::LOADS) __builtin_amdgcn_sched_group_barrier(kSchedVMEMRead, 1, 0);
      }
    }
    const int kv1 = (j + 1) * C::BN;
    if (kv1 + C::BN > w.N || (CAUSAL && kv1 + C::BN - 1 > w.qw0))
      mask_tile<D, CAUSAL>(s_nxt, kv1, w.N, w.qrow, w.g);
    // Raised issue priority while this wave feeds the matrix cores with
    // P_j V_j, so that the other wave of the SIMD fills the gaps with its
    // vector work rather than the reverse.
    __builtin_amdgcn_s_setprio(1);
    pv_tile<D>(v_stage<D>(smem, PAR), pf, w.off, w.oacc);
    add_row_sums<D>(pf, w.l_run);
    float m_tile[C::QB];
    tile_max<D>(s_nxt, w.c, m_tile);
    if constexpr (C::DC >= 8) {
      // One MFMA of P_j V_j, then V operand reads and a share of the
      // row-max reduction of S_{j+1}.
      constexpr int kMfma = C::NT * 2 * C::DT * C::QB;
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2 * C::K_AHEAD, 0);
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        if (i % C::QB == C::QB - 1) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, 2, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (j + 1 < w.nt_w) raise_max<D>(m_tile, w.m_run, w.l_run, w.oacc);
  } else {
    load_tile<D>(vrs, v_stage<D>(smem, PAR ^ 1), v_base, lo, tid);
    load_tile<D>(krs, k_stage<D>(smem, PAR), k_base, lo, tid);
  }
  wait_vm_all();
  __syncthreads();
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, Cfg<D>::WG_PER_CU) void attn_fwd_kernel(Params p) {
  using C = Cfg<D>;
  // K stages 0/1 then V stages 0/1.
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES];

  // Workgroup id -> (batch*head, query tile), contiguous per XCD.
  const int nb = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3, q8 = nb >> 3, r8 = nb & 7;
  const int u = xcd * q8 + (xcd < r8 ? xcd : r8) + slot;
  const int bh = u / p.q_tiles;
  int qt = u - bh * p.q_tiles;
  if (CAUSAL) qt = p.q_tiles - 1 - qt;
  const int b = bh / p.Hq, hq = bh - b * p.Hq, kvh = hq / p.group;
  const int N = p.N;
  const int q0 = qt * C::BM;

  const size_t qoff = ((size_t)b * p.Hq + hq) * (size_t)N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + kvh) * (size_t)N * D;
  const _Float16* __restrict__ qb_ptr = p.q + qoff;
  // Bytes of one K/V head: <= 2^31 by the library's size limit; the range
  // field holds it as an unsigned 32-bit count.
  const int head_bytes = static_cast<int>(static_cast<uint32_t>(N) * (D * 2));
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kvoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kvoff), (short)0, head_bytes, kBufferWord3);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  WaveState<D> w;
  w.N = N;
  w.c = p.c;
  w.g = lane >> 5;
  w.qw0 = q0 + C::WAVE_ROWS * wv;  // first query row of this wave
  w.qrow = w.qw0 + (lane & 31);    // query row of this lane in block 0
  w.off.init(lane);

  const int kv_tiles = (N + C::BN - 1) / C::BN;
  int nt = kv_tiles;
  if (CAUSAL) {
    const int last_q = (q0 + C::BM < N ? q0 + C::BM : N) - 1;
    const int t_end = last_q / C::BN + 1;
    nt = t_end < kv_tiles ? t_end : kv_tiles;
  }
  if (w.qw0 >= N) {
    w.nt_w = 0;  // every row of this wave is padding
  } else if (CAUSAL) {
    const int last_w = (w.qw0 + C::WAVE_ROWS < N ? w.qw0 + C::WAVE_ROWS : N) - 1;
    w.nt_w = last_w / C::BN + 1;
  } else {
    w.nt_w = nt;
  }

  LoadOffsets<D> lo;
  lo.init(tid);
  load_tile<D>(krs, k_stage<D>(smem, 0), 0, lo, tid);
  load_tile<D>(vrs, v_stage<D>(smem, 0), 0, lo, tid);
  load_tile<D>(krs, k_stage<D>(smem, 1), tile_base<D>(1, nt), lo, tid);

  // Q fragments (B operand of S^T): dims 16*dc + 8*g .. +7 of each row.
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int row = w.qrow + 32 * qb;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      u32x4 x = row < N ? *reinterpret_cast<const u32x4*>(qb_ptr + (size_t)row * D + 16 * dc + 8 * w.g)
                        : u32x4{0u, 0u, 0u, 0u};
      x = (x ^ p.q_sign) & p.q_keep;
      w.qf[qb][dc] = __builtin_bit_cast(half8, x);
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) w.oacc[qb][dt] = f32x16{};
    w.m_run[qb] = -INFINITY;
    w.l_run[qb] = 0.f;
  }

  wait_vm_all();
  __syncthreads();

  // Prologue: logits of tile 0 and the first running max.
  STile<D> sa, sb;
  if (w.nt_w > 0) {
    qk_tile<D>(k_stage<D>(smem, 0), w.qf, w.off, sa);
    if (C::BN > N || (CAUSAL && C::BN - 1 > w.qw0)) mask_tile<D, CAUSAL>(sa, 0, N, w.qrow, w.g);
    // Key 0 is visible to every row, so these maxima are finite.
    tile_max<D>(sa, w.c, w.m_run);
  }
  // Iteration 0 refills K stage 0: every wave must be done reading K_0.
  __syncthreads();

  for (int j = 0; j < nt; j += 2) {
    pipeline_step<D, CAUSAL, 0>(j, nt, smem, krs, vrs, lo, tid, w, sa, sb);
    if (j + 1 < nt) pipeline_step<D, CAUSAL, 1>(j + 1, nt, smem, krs, vrs, lo, tid, w, sb, sa);
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m + log2 l).
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int row = w.qrow + 32 * qb;
    const float l_tot = xlane_sum(w.l_run[qb]);
    if (row < N) {
      const float inv = 1.0f / l_tot;
      _Float16* __restrict__ orow = p.o + qoff + (size_t)row * D;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          half4 h;
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(w.oacc[qb][dt][4 * rq + i] * inv);
          *reinterpret_cast<half4*>(orow + 32 * dt + 8 * rq + 4 * w.g) = h;
        }
      if (p.lse != nullptr && w.g == 0)
        p.lse[((size_t)b * p.Hq + hq) * N + row] = (w.m_run[qb] + __builtin_log2f(l_tot)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_t(const LaunchArgs& a, Params p, hipStream_t s) {
  p.q_tiles = (a.N + Cfg<D>::BM - 1) / Cfg<D>::BM;
  const unsigned grid = static_cast<unsigned>(a.B) * a.Hq * p.q_tiles;
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode (KV cache): Nq new queries against Nk cached keys.
//
// The G query heads that read one key/value head are packed into the rows of
// one workgroup (row r = g * Nq + i), so each K/V byte is read from memory
// once for all of them ([FA-Infer] section 6: GQA and MQA exist to shrink
// the KV cache that inference reads).  Query i is the i-th of the last Nq
// positions of the sequence, so when causal it sees keys 0 .. Nk - Nq + i.
// The keys are split into chunks, one workgroup each, running the same
// pipeline as the forward kernel and writing a partial O (divided by its
// own l) and a partial log2-sum-exp; the merge kernel combines them:
// LSE = log2 sum_s 2^LSE_s, O = sum_s 2^(LSE_s - LSE) O_s.
// ---------------------------------------------------------------------------

struct DecParams {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;      // final output, written here when there is one split
  float* lse;       // final LSE (may be null), likewise
  float* part_o;    // [groups][splits][kDecodeRows][d]
  float* part_lse;  // [groups][splits][kDecodeRows], log2 units
  int Hq, Hkv, group, Nq, Nk, rows, row_blocks, splits, chunk_tiles;
  float c;
  uint32_t q_sign, q_keep;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, Cfg<D>::WG_PER_CU) void attn_decode_split_kernel(DecParams p) {
  using C = Cfg<D>;
  static_assert(C::QB == 1 && C::BM == kDecodeRows, "decode packs 128 rows per workgroup, 32 per wave");
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES];

  const int split = blockIdx.x % p.splits;
  const int grp = blockIdx.x / p.splits;  // (b * Hkv + kvh) * row_blocks + rb
  const int rb = grp % p.row_blocks;
  const int bk = grp / p.row_blocks;      // b * Hkv + kvh
  const int b = bk / p.Hkv, kvh = bk - b * p.Hkv;
  const int Nk = p.Nk, Nq = p.Nq;
  const int off = Nk - Nq;  // absolute position of query 0

  const size_t kvoff = (size_t)bk * (size_t)Nk * D;
  const int head_bytes = static_cast<int>(static_cast<uint32_t>(Nk) * (D * 2));
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kvoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kvoff), (short)0, head_bytes, kBufferWord3);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = rb * C::BM + 32 * wv;     // first packed row of this wave
  const int r = row0 + (lane & 31);          // packed row of this lane
  const bool valid = r < p.rows;
  const int gq = valid ? r / Nq : 0;
  const int iq = valid ? r - gq * Nq : 0;
  const int hq = kvh * p.group + gq;

  WaveState<D> w;
  w.N = Nk;
  w.c = p.c;
  w.g = lane >> 5;
  w.qw0 = CAUSAL ? off : Nk;          // every row sees at least keys 0 .. off
  w.qrow = CAUSAL ? off + iq : Nk;    // last key this lane's row may see
  w.off.init(lane);

  const int t0 = split * p.chunk_tiles;
  const int kv_tiles = (Nk + C::BN - 1) / C::BN;
  const int t1 = t0 + p.chunk_tiles < kv_tiles ? t0 + p.chunk_tiles : kv_tiles;
  w.nt_w = row0 < p.rows ? t1 : t0;    // waves without rows only help with the copies

  LoadOffsets<D> lo;
  lo.init(tid);
  load_tile<D>(krs, k_stage<D>(smem, 0), tile_base<D>(t0, t1), lo, tid);
  load_tile<D>(vrs, v_stage<D>(smem, 0), tile_base<D>(t0, t1), lo, tid);
  load_tile<D>(krs, k_stage<D>(smem, 1), tile_base<D>(t0 + 1, t1), lo, tid);

  const _Float16* __restrict__ qrow_ptr = p.q + (((size_t)b * p.Hq + hq) * Nq + iq) * D;
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    u32x4 x = valid ? *reinterpret_cast<const u32x4*>(qrow_ptr + 16 * dc + 8 * w.g) : u32x4{0u, 0u, 0u, 0u};
    x = (x ^ p.q_sign) & p.q_keep;
    w.qf[0][dc] = __builtin_bit_cast(half8, x);
  }
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) w.oacc[0][dt] = f32x16{};
  w.m_run[0] = -INFINITY;
  w.l_run[0] = 0.f;

  wait_vm_all();
  __syncthreads();

  STile<D> sa, sb;
  if (w.nt_w > t0) {
    const int kv0 = t0 * C::BN;
    qk_tile<D>(k_stage<D>(smem, 0), w.qf, w.off, sa);
    if (kv0 + C::BN > Nk || (CAUSAL && kv0 + C::BN - 1 > w.qw0)) mask_tile<D, CAUSAL>(sa, kv0, Nk, w.qrow, w.g);
    tile_max<D>(sa, w.c, w.m_run);
    // A row that sees no key of this chunk (causal: the chunk starts after
    // its last key; then it sees none of the later tiles either) keeps a
    // finite reference so that its probabilities are exp2(-inf) = 0.
    if (w.m_run[0] == -INFINITY) w.m_run[0] = 0.f;
  }
  __syncthreads();

  for (int j = t0; j < t1; j += 2) {
    pipeline_step<D, CAUSAL, 0>(j, t1, smem, krs, vrs, lo, tid, w, sa, sb);
    if (j + 1 < t1) pipeline_step<D, CAUSAL, 1>(j + 1, t1, smem, krs, vrs, lo, tid, w, sb, sa);
  }

  // Partial result of this chunk for the rows that exist: O_s = O^T / l_s
  // (0 when the row saw no key) and LSE_s = m + log2 l_s (-inf when it saw
  // none).
  const float l_tot = xlane_sum(w.l_run[0]);
  if (!valid) return;
  if (p.splits == 1) {
    // One chunk holds every key (key 0 among them, so l_tot > 0): finish the
    // rows here, as the forward epilogue does, and skip the merge.
    const float inv1 = 1.0f / l_tot;
    _Float16* __restrict__ out = p.o + (((size_t)b * p.Hq + hq) * Nq + iq) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        half4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(w.oacc[0][dt][4 * rq + i] * inv1);
        *reinterpret_cast<half4*>(out + 32 * dt + 8 * rq + 4 * w.g) = h;
      }
    if (p.lse != nullptr && w.g == 0)
      p.lse[((size_t)b * p.Hq + hq) * Nq + iq] = (w.m_run[0] + __builtin_log2f(l_tot)) * kLn2;
    return;
  }
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const size_t slot = ((size_t)grp * p.splits + split) * C::BM + 32 * wv + (lane & 31);
  float* __restrict__ orow = p.part_o + slot * D;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float4 f;
      f.x = w.oacc[0][dt][4 * rq + 0] * inv;
      f.y = w.oacc[0][dt][4 * rq + 1] * inv;
      f.z = w.oacc[0][dt][4 * rq + 2] * inv;
      f.w = w.oacc[0][dt][4 * rq + 3] * inv;
      *reinterpret_cast<float4*>(orow + 32 * dt + 8 * rq + 4 * w.g) = f;
    }
  if (w.g == 0) p.part_lse[slot] = l_tot > 0.f ? w.m_run[0] + __builtin_log2f(l_tot) : -INFINITY;
}

struct MergeParams {
  const float* part_o;
  const float* part_lse;
  _Float16* o;
  float* lse;  // may be null
  int Hq, Hkv, group, Nq, row_blocks, splits;
};

constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;  // splits per thread whose loads are in flight together
// Output dims per merge workgroup: a whole row when there are few splits
// (fewer, fuller workgroups), 32-dim slices of it when there are many.
constexpr int kMergeSliceDims = 32;
constexpr int kMergeFewSplits = 64;

// One workgroup per (query row (b, hq, i), DS output dims).  Each thread
// folds a subset of the splits into its own (m, l, acc) with the online
// rule (m = max LSE_s, l = sum 2^(LSE_s - m), acc = sum 2^(LSE_s - m) O_s),
// reading each split's LSE and O slice in the same pass; the threads then
// combine theirs: LSE = m + log2 l, O = acc / l, rounded once to fp16.
template <int D, int DS>
__global__ __launch_bounds__(kMergeThreads) void attn_decode_merge_kernel(MergeParams p) {
  constexpr int CH = DS / 4;                 // float4 chunks of a slice
  constexpr int PAR = kMergeThreads / CH;    // splits read at once
  constexpr int SLICES = D / DS;
  __shared__ float sm_m[PAR][CH], sm_l[PAR][CH];
  __shared__ float4 sm_acc[PAR][CH];

  const int rowid = blockIdx.x / SLICES;     // (b * Hq + hq) * Nq + i
  const int slice = blockIdx.x - rowid * SLICES;
  const int i = rowid % p.Nq;
  const int bh = rowid / p.Nq;
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int kvh = hq / p.group, gq = hq - kvh * p.group;
  const int r = gq * p.Nq + i;
  const int grp = (b * p.Hkv + kvh) * p.row_blocks + r / (int)kDecodeRows;
  const int rr = r % (int)kDecodeRows;
  const int tid = threadIdx.x, chunk = tid % CH, sp = tid / CH;
  const int S = p.splits;
  const float* __restrict__ lse_s = p.part_lse + (size_t)grp * S * kDecodeRows + rr;  // split s at s * kDecodeRows
  const float* __restrict__ o_s =
      p.part_o + ((size_t)grp * S * kDecodeRows + rr) * D + slice * DS + 4 * chunk;  // at s * kDecodeRows * D

  float m = -INFINITY, l = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = sp; s0 < S; s0 += PAR * kMergeBatch) {
    // Issue the loads of kMergeBatch splits before using any (a split past
    // the end reads split 0 and is then ignored).
    float ls[kMergeBatch];
    float4 x[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int sk = s0 + k * PAR < S ? s0 + k * PAR : 0;
      ls[k] = lse_s[(size_t)sk * kDecodeRows];
      x[k] = *reinterpret_cast<const float4*>(o_s + (size_t)sk * kDecodeRows * D);
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (s0 + k * PAR < S && ls[k] > -INFINITY) {  // a split the row saw no key of adds nothing
        const float mn = fmaxf(m, ls[k]);
        const float a = __builtin_amdgcn_exp2f(m - mn);  // 0 while m = -inf
        const float w = __builtin_amdgcn_exp2f(ls[k] - mn);
        l = l * a + w;
        acc.x = acc.x * a + w * x[k].x;
        acc.y = acc.y * a + w * x[k].y;
        acc.z = acc.z * a + w * x[k].z;
        acc.w = acc.w * a + w * x[k].w;
        m = mn;
      }
    }
  }
  sm_m[sp][chunk] = m;
  sm_l[sp][chunk] = l;
  sm_acc[sp][chunk] = acc;
  __syncthreads();
  if (tid < CH) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < PAR; ++k) M = fmaxf(M, sm_m[k][tid]);  // finite: split 0 holds key 0
    float L = 0.f;
    float4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < PAR; ++k) {
      const float a = __builtin_amdgcn_exp2f(sm_m[k][tid] - M);  // 0 for threads that saw no split
      const float4 x = sm_acc[k][tid];
      L += a * sm_l[k][tid];
      o.x += a * x.x;
      o.y += a * x.y;
      o.z += a * x.z;
      o.w += a * x.w;
    }
    const float inv = 1.0f / L;
    half4 h;
    h[0] = static_cast<_Float16>(o.x * inv);
    h[1] = static_cast<_Float16>(o.y * inv);
    h[2] = static_cast<_Float16>(o.z * inv);
    h[3] = static_cast<_Float16>(o.w * inv);
    *reinterpret_cast<half4*>(p.o + (size_t)rowid * D + slice * DS + 4 * tid) = h;
    if (p.lse != nullptr && slice == 0 && tid == 0) p.lse[rowid] = (M + __builtin_log2f(L)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_decode_t(const DecodeArgs& a, const DecParams& dp, const MergeParams& mp, hipStream_t s) {
  const unsigned groups = static_cast<unsigned>(a.B) * a.Hkv * static_cast<unsigned>(a.plan.row_blocks);
  hipLaunchKernelGGL((attn_decode_split_kernel<D, CAUSAL>), dim3(groups * static_cast<unsigned>(a.plan.splits)),
                     dim3(kThreads), 0, s, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.plan.splits == 1) return e;
  const unsigned rows = static_cast<unsigned>(a.B) * a.Hq * a.Nq;
  if (a.plan.splits <= kMergeFewSplits)
    hipLaunchKernelGGL((attn_decode_merge_kernel<D, D>), dim3(rows), dim3(kMergeThreads), 0, s, mp);
  else
    hipLaunchKernelGGL((attn_decode_merge_kernel<D, kMergeSliceDims>), dim3(rows * (D / kMergeSliceDims)),
                       dim3(kMergeThreads), 0, s, mp);
  return hipGetLastError();
}

}  // namespace

int launch_forward(const LaunchArgs& a, void* stream) {
  Params p;
  p.q = static_cast<const _Float16*>(a.q);
  p.k = static_cast<const _Float16*>(a.k);
  p.v = static_cast<const _Float16*>(a.v);
  p.o = static_cast<_Float16*>(a.o);
  p.lse = a.lse;
  p.N = a.N;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  const double c = static_cast<double>(a.scale) * 1.4426950408889634;
  // The kernel needs c > 0 (a masked logit of -inf must give exp2(-inf) = 0).
  // scale < 0 negates Q (exact in fp16); scale = 0 zeroes Q and uses c = 1,
  // which gives every visible logit exactly 0, as scale = 0 does.
  p.c = a.scale == 0.f ? 1.0f : static_cast<float>(c < 0 ? -c : c);
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  p.q_keep = a.scale == 0.f ? 0u : 0xffffffffu;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (a.d) {
    case 64:
      e = a.causal ? launch_t<64, true>(a, p, s) : launch_t<64, false>(a, p, s);
      break;
    case 128:
      e = a.causal ? launch_t<128, true>(a, p, s) : launch_t<128, false>(a, p, s);
      break;
    case 256:
      e = a.causal ? launch_t<256, true>(a, p, s) : launch_t<256, false>(a, p, s);
      break;
    default:
      e = hipErrorInvalidValue;
  }
  return static_cast<int>(e);
}

int launch_decode(const DecodeArgs& a, void* stream) {
  DecParams dp;
  dp.q = static_cast<const _Float16*>(a.q);
  dp.k = static_cast<const _Float16*>(a.k);
  dp.v = static_cast<const _Float16*>(a.v);
  dp.o = static_cast<_Float16*>(a.o);
  dp.lse = a.lse;
  const int64_t groups = static_cast<int64_t>(a.B) * a.Hkv * a.plan.row_blocks;
  dp.part_o = static_cast<float*>(a.workspace);
  dp.part_lse = dp.part_o + groups * a.plan.splits * kDecodeRows * a.d;
  dp.Hq = a.Hq;
  dp.Hkv = a.Hkv;
  dp.group = a.Hq / a.Hkv;
  dp.Nq = a.Nq;
  dp.Nk = a.Nk;
  dp.rows = dp.group * a.Nq;
  dp.row_blocks = static_cast<int>(a.plan.row_blocks);
  dp.splits = static_cast<int>(a.plan.splits);
  dp.chunk_tiles = static_cast<int>(a.plan.chunk_tiles);
  const double c = static_cast<double>(a.scale) * 1.4426950408889634;
  dp.c = a.scale == 0.f ? 1.0f : static_cast<float>(c < 0 ? -c : c);
  dp.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  dp.q_keep = a.scale == 0.f ? 0u : 0xffffffffu;
  MergeParams mp;
  mp.part_o = dp.part_o;
  mp.part_lse = dp.part_lse;
  mp.o = static_cast<_Float16*>(a.o);
  mp.lse = a.lse;
  mp.Hq = a.Hq;
  mp.Hkv = a.Hkv;
  mp.group = dp.group;
  mp.Nq = a.Nq;
  mp.row_blocks = dp.row_blocks;
  mp.splits = dp.splits;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (a.d) {
    case 64:
      e = a.causal ? launch_decode_t<64, true>(a, dp, mp, s) : launch_decode_t<64, false>(a, dp, mp, s);
      break;
    case 128:
      e = a.causal ? launch_decode_t<128, true>(a, dp, mp, s) : launch_decode_t<128, false>(a, dp, mp, s);
      break;
    case 256:
      e = a.causal ? launch_decode_t<256, true>(a, dp, mp, s) : launch_decode_t<256, false>(a, dp, mp, s);
      break;
    default:
      e = hipErrorInvalidValue;
  }
  return static_cast<int>(e);
}

}  // namespace attn
