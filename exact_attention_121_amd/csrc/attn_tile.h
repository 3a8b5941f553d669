// Device building blocks shared by the fused attention kernels for gfx950
// (the prefill/forward kernel and the decode kernels): fragment types, the
// LDS tile layout and its loads, the score / mask / online-softmax / P.V
// steps of one key tile, and the software-pipelined iteration over key
// tiles.  Included by the kernel sources only; everything lives in an
// unnamed namespace.
//
// Pages cited:
//   [CANN-FA]  www.mooersco.com/news/1200175 - "FlashAttention operator of the
//              CANN ops-transformer repository: attention acceleration on the
//              Ascend NPU"
//   [FA-Dict]  hwcomputing.csdn.net/6a0dbd08662f9a54cb75eb74.html
//   [FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html
#ifndef ATTN_TILE_H_
#define ATTN_TILE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_launch.h"

namespace attn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
  return D == 64 ? ATTN_QB64 : (D == 128 ? ATTN_QB128 : (D == 256 ? ATTN_QB256 : 1));
}

// Keys per K/V tile, matrix operands read ahead of their MFMA and
// workgroups per CU, per head_dim.  The defaults (default_key_tile and
// default_wg_per_cu in attn_launch.h, k_ahead below) are the measured best on
// gfx950; the offline tile sweep (exact_attention_121_amd/tile_sweep.py)
// rebuilds the forward kernel with other values through these hooks (0 = the
// default).
#ifndef ATTN_BN32
#define ATTN_BN32 0
#endif
#ifndef ATTN_BN64
#define ATTN_BN64 0
#endif
#ifndef ATTN_BN96
#define ATTN_BN96 0
#endif
#ifndef ATTN_BN128
#define ATTN_BN128 0
#endif
#ifndef ATTN_BN160
#define ATTN_BN160 0
#endif
#ifndef ATTN_BN192
#define ATTN_BN192 0
#endif
#ifndef ATTN_BN224
#define ATTN_BN224 0
#endif
#ifndef ATTN_BN256
#define ATTN_BN256 0
#endif
#ifndef ATTN_KAHEAD32
#define ATTN_KAHEAD32 0
#endif
#ifndef ATTN_KAHEAD64
#define ATTN_KAHEAD64 0
#endif
#ifndef ATTN_KAHEAD96
#define ATTN_KAHEAD96 0
#endif
#ifndef ATTN_KAHEAD128
#define ATTN_KAHEAD128 0
#endif
#ifndef ATTN_KAHEAD160
#define ATTN_KAHEAD160 0
#endif
#ifndef ATTN_KAHEAD192
#define ATTN_KAHEAD192 0
#endif
#ifndef ATTN_KAHEAD224
#define ATTN_KAHEAD224 0
#endif
#ifndef ATTN_KAHEAD256
#define ATTN_KAHEAD256 0
#endif
#ifndef ATTN_WG32
#define ATTN_WG32 0
#endif
#ifndef ATTN_WG64
#define ATTN_WG64 0
#endif
#ifndef ATTN_WG96
#define ATTN_WG96 0
#endif
#ifndef ATTN_WG128
#define ATTN_WG128 0
#endif
#ifndef ATTN_WG160
#define ATTN_WG160 0
#endif
#ifndef ATTN_WG192
#define ATTN_WG192 0
#endif
#ifndef ATTN_WG224
#define ATTN_WG224 0
#endif
#ifndef ATTN_WG256
#define ATTN_WG256 0
#endif
template <int D>
constexpr int key_tile() {
  constexpr int hook = D == 32 ? ATTN_BN32 : D == 64 ? ATTN_BN64 : D == 96 ? ATTN_BN96 : D == 128 ? ATTN_BN128
                     : D == 160 ? ATTN_BN160 : D == 192 ? ATTN_BN192 : D == 224 ? ATTN_BN224 : ATTN_BN256;
  return hook ? hook : static_cast<int>(default_key_tile(D));
}
// Workgroups per CU the kernel is compiled for (its register budget).
template <int D>
constexpr int wg_per_cu() {
  constexpr int hook = D == 32 ? ATTN_WG32 : D == 64 ? ATTN_WG64 : D == 96 ? ATTN_WG96 : D == 128 ? ATTN_WG128
                     : D == 160 ? ATTN_WG160 : D == 192 ? ATTN_WG192 : D == 224 ? ATTN_WG224 : ATTN_WG256;
  return hook ? hook : static_cast<int>(default_wg_per_cu(D));
}
// Workgroups per CU of the forward kernel: as above, except that without a
// hook d = 256 takes two (a 76-byte spill per lane, but the second wave per
// SIMD hides more latency: +3-5 % measured with the mask; without it the
// offline tile sweep measured +0.5 % at N = 2048 and +4.9 % at N = 8192).
// The decode kernel keeps one: its split plan follows default_wg_per_cu.
template <int D, bool CAUSAL>
constexpr int fwd_wg_per_cu() {
  constexpr int hook = D == 32 ? ATTN_WG32 : D == 64 ? ATTN_WG64 : D == 96 ? ATTN_WG96 : D == 128 ? ATTN_WG128
                     : D == 160 ? ATTN_WG160 : D == 192 ? ATTN_WG192 : D == 224 ? ATTN_WG224 : ATTN_WG256;
  if (query_blocks<D>() != 1) return hook ? hook : 1;
  return hook ? hook : (D == 256 ? 2 : static_cast<int>(default_wg_per_cu(D)));
}
// Operands read ahead: a longer run of them pays only with the register
// budget of one workgroup per CU.
template <int D>
constexpr int k_ahead() {
  constexpr int hook = D == 32 ? ATTN_KAHEAD32 : D == 64 ? ATTN_KAHEAD64 : D == 96 ? ATTN_KAHEAD96
                     : D == 128 ? ATTN_KAHEAD128 : D == 160 ? ATTN_KAHEAD160 : D == 192 ? ATTN_KAHEAD192
                     : D == 224 ? ATTN_KAHEAD224 : ATTN_KAHEAD256;
  return hook ? hook : (wg_per_cu<D>() == 2 ? 4 : 6);
}

// 16-byte chunks per row of an LDS tile: the row's D / 8 chunks, padded to
// 8, 16 or 32 so that the XOR swizzle below permutes whole rows (head_dims
// other than 64, 128 and 256 leave the padding slots unused).
template <int D>
constexpr int lds_row_chunks() {
  return D <= 64 ? 8 : (D <= 128 ? 16 : 32);
}

template <int D>
struct Cfg {
  static constexpr int QB = query_blocks<D>();     // 32-row query blocks per wave
  static constexpr int WAVE_ROWS = 32 * QB;        // query rows per wave
  static constexpr int BM = kWaves * WAVE_ROWS;    // query rows per workgroup
  static constexpr int BN = key_tile<D>();         // keys per K/V tile
  static constexpr int NT = BN / 32;               // 32-key sub-tiles of S^T
  static constexpr int DC = D / 16;                // 16-dim k-steps of Q.K
  static constexpr int DT = D / 32;                // 32-dim row tiles of O^T
  static constexpr int CPR = lds_row_chunks<D>();  // 16-byte chunks per LDS tile row
  static constexpr int SRC_CPR = D / 8;            // 16-byte chunks per row in memory
  static constexpr int TILE_BYTES = BN * CPR * 16;   // one K (or V) tile in LDS
  static constexpr int LOADS = BN * CPR / kThreads;  // 16-byte loads per thread per tile
  // Workgroups per CU the register budget allows.
  static constexpr int WG_PER_CU = QB == 1 ? wg_per_cu<D>() : fwd_wg_per_cu<D, false>();
  // Matrix operands read from LDS ahead of their MFMA (K reads; twice as
  // many V transpose reads, two per MFMA).
  static constexpr int K_AHEAD = k_ahead<D>();
  static_assert(BN * CPR % kThreads == 0, "tile must split evenly over the workgroup");
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

// Source offset of an LDS padding slot: 2^31 past the tile base.  For a
// real tile (base below 2^31) that lies outside the head, which is at most
// 2^31 bytes, so the range check turns the copy into zeros; for a skipped
// tile (below) the sum wraps to offset 0, an in-bounds read.  Either way the
// slot is never read by a matrix operand.
constexpr uint32_t kPadChunk = 0x80000000u;

// Byte offsets, relative to a tile's first row, of the 16-byte chunks that
// thread `tid` copies into a swizzled tile (the chunk that belongs at
// position p % CPR of row p / CPR of the tile, or kPadChunk for a padding
// slot).
// Load i of a thread covers tile row p / CPR with p = i * 256 + tid, so the
// row advances by 256 / CPR per load; the swizzle depends only on a row's
// low four bits, so the offsets repeat, a whole number of rows further on,
// every kPeriod loads and only kPeriod of them are kept (at(i) adds the rows).
template <int D>
struct LoadOffsets {
  using C = Cfg<D>;
  static constexpr int kRowsPerLoad = kThreads / C::CPR;
  static constexpr int kPeriod = kRowsPerLoad >= 16 ? 1 : 16 / kRowsPerLoad;
  static constexpr int kKept = kPeriod < C::LOADS ? kPeriod : C::LOADS;
  uint32_t src[kKept];
  __device__ __forceinline__ void init(int tid) {
#pragma unroll
    for (int i = 0; i < kKept; ++i) {
      const int p = i * kThreads + tid;  // destination chunk; lanes of a wave are consecutive
      const int row = p / C::CPR;
      const int chunk = (swz<D>(row, p % C::CPR) >> 4) - row * C::CPR;
      if constexpr (C::CPR == C::SRC_CPR)
        src[i] = static_cast<uint32_t>((row * D + chunk * 8) * 2);
      else
        src[i] = chunk < C::SRC_CPR ? static_cast<uint32_t>((row * D + chunk * 8) * 2) : kPadChunk;
    }
  }
  // i compile-time in the unrolled loads: a register plus a constant.  A
  // padding slot stays at or above 2^31 (kPadChunk plus rows of the tile).
  __device__ __forceinline__ uint32_t at(int i) const {
    return src[i % kPeriod] + static_cast<uint32_t>((i / kPeriod) * kPeriod * kRowsPerLoad * D * 2);
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
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, static_cast<int>(base + lo.at(i)),
                                             0, 0, 0);
  }
}

// Byte offset of the first row of key tile j inside a head, or kSkipTile.
template <int D>
__device__ __forceinline__ uint32_t tile_base(int j, int nt) {
  return j < nt ? static_cast<uint32_t>(j) * (Cfg<D>::BN * D * 2) : kSkipTile;
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Race-check build (-DATTN_PARANOID_SYNC): at every phase boundary of the
// pipelined loops all outstanding copies and LDS accesses complete and every
// wave of the workgroup arrives.  The arithmetic and its order do not change,
// so that build must give bit-for-bit the same outputs as the default one; a
// difference would mean a stage was read before its copy landed or
// overwritten while another wave still read it.  Called the same number of
// times by every wave of a workgroup.
#ifdef ATTN_PARANOID_SYNC
constexpr bool kParanoidSync = true;
#else
constexpr bool kParanoidSync = false;
#endif
__device__ __forceinline__ void paranoid_sync() {
  if constexpr (kParanoidSync) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

__device__ __forceinline__ short4v tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
}

__device__ __forceinline__ float xlane_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float xlane_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Per-lane LDS byte offsets of the matrix operands inside a (swizzled) tile.
// Tile rows 32*t + 16*h (K) or key groups (V) only add a constant, so every
// operand read is one of these registers plus an immediate offset.  Two
// identities of the swizzle save registers:
//  * in rows of 32 chunks it changes only the low four bits of the chunk
//    index, so chunk c + 16 lies 256 bytes after chunk c: the upper half of
//    the dims reuses the lower half's registers;
//  * with the 16-entry map, row r + 8 XORs with f(r) ^ 8, so key group 1
//    (rows + 8) of row tile dt reads where group 0 of row tile dt ^ 2 does,
//    8 rows further on (when the row tiles come in fours).
template <int D>
struct Offsets {
  using C = Cfg<D>;
  static constexpr bool kHalves = C::CPR == 32;
  static constexpr int KR = kHalves && C::DC > 8 ? 8 : C::DC;  // registers for K chunks
  static constexpr int VR = kHalves && C::DT > 4 ? 4 : C::DT;  // registers for V row tiles
  static constexpr bool kGroup1FromGroup0 = C::CPR >= 16 && VR % 4 == 0;
  static constexpr int VG = kGroup1FromGroup0 ? 1 : 2;         // key groups with registers
  int k[KR];       // K rows lane%32 (+32 t), chunk 2 dc + lane/32
  int v[VG][VR];   // V keys 4 g + (lane%16)/4 (+8 for [1]), dims of row tile dt
  __device__ __forceinline__ void init(int lane) {
    const int lr = lane & 31, g = lane >> 5, m16 = lane & 15;
#pragma unroll
    for (int dc = 0; dc < KR; ++dc) k[dc] = swz<D>(lr, 2 * dc + g);
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (m16 & 3);  // dim offset inside a 32-dim tile
#pragma unroll
    for (int hi = 0; hi < VG; ++hi)
#pragma unroll
      for (int dt = 0; dt < VR; ++dt) {
        const int dim = 32 * dt + dsub;
        v[hi][dt] = swz<D>(4 * g + (m16 >> 2) + 8 * hi, dim >> 3) + (dim & 7) * 2;
      }
  }
  // Offset of K chunk pair dc and of V row tile dt (dc, dt compile-time in
  // the unrolled loops, so the choice and the +256 fold away).
  __device__ __forceinline__ int kofs(int dc) const { return dc < KR ? k[dc] : k[dc - 8] + 256; }
  __device__ __forceinline__ int vofs(int hi, int dt) const {
    if (dt >= VR) return vofs(hi, dt - 4) + 256;
    if (kGroup1FromGroup0 && hi == 1) return v[0][dt ^ 2] + 8 * C::CPR * 16;
    return v[kGroup1FromGroup0 ? 0 : hi][dt];
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

// Element type T of Q, K, V, O and of P in the P.V product: _Float16 or
// __bf16.  Fragments are held as 8 x 16-bit vectors (half8) for either type
// and reinterpreted for the matrix instruction; to_elem rounds an fp32 value
// to T (to nearest even) and returns its 16 bits.
template <typename T>
__device__ __forceinline__ f32x16 mfma16(half8 a, half8 b, f32x16 c) {
  if constexpr (std::is_same_v<T, __bf16>)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ _Float16 to_elem(float x) {
  if constexpr (std::is_same_v<T, __bf16>)
    return __builtin_bit_cast(_Float16, static_cast<__bf16>(x));
  else
    return static_cast<_Float16>(x);
}

// S^T = K Q^T for one key tile: s[qb][t] holds keys 32 t .. 32 t + 31 (rows
// of the 32x32 result) against query block qb (columns).  Each K operand
// read from LDS serves every query block of the wave.
template <int D, typename T = _Float16>
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
      const half8 a = *reinterpret_cast<const half8*>(ks + off.kofs(dc) + 32 * t * C::CPR * 16);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
        s[qb][t] = mfma16<T>(a, qf[qb][dc], s[qb][t]);
    }
}

// Keys past the end of the sequence, or after the query when causal, get
// logit -inf (then exp2 gives exactly 0).  Lane L holds keys
// 32 t + 8 (r/4) + 4 (L/32) + r%4 of query row `qrow` (+32 per block): the
// last visible key gives the lane one limit, and each entry's key offset
// 32 t + 8 (r/4) + r%4 is a compile-time constant compared with it.
template <int D, bool CAUSAL>
__device__ __forceinline__ void mask_tile(STile<D>& s, int kv0, int N, int qrow, int g) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int last = CAUSAL ? min(N - 1, qrow + 32 * qb) : N - 1;   // last visible key of the row
    const int lim = last - kv0 - 4 * g;
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[qb][t][r] = 32 * t + 8 * (r >> 2) + (r & 3) <= lim ? s[qb][t][r] : -INFINITY;
  }
}

// Row maxima of a tile's raw logits, in log2 units (c > 0).  The maxima
// are NaN-propagating (v_maximum3_f32): the logits are finite or -inf, where
// they equal fmaxf, but fmaxf's quieting of signalling NaNs made the compiler
// canonicalise matrix results and permuted values first (8 fewer vector
// instructions per tile at d = 64, +1.2 to +1.6 % there, bit-identical).
template <int D>
__device__ __forceinline__ void tile_max(const STile<D>& s, float c, float (&m)[Cfg<D>::QB]) {
  using C = Cfg<D>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    float mx = s[qb][0][0];
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = (t == 0 ? 1 : 0); r < 16; ++r) mx = __builtin_elementwise_maximum(mx, s[qb][t][r]);
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
template <int D, typename T = _Float16>
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
            to_elem<T>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][t][r], c, -m_run[qb])));
}

// Adds the sum of the fp16 probabilities (exactly the values multiplied
// into V) to the lane's partial row sums l.
//
// v_dot2 does not overlap the matrix instructions on gfx950 (about 4 cycles
// each of the matrix pipe's time, measured), while packed fp16 additions
// mostly do.  At d = 256 the lane's adjacent probabilities are therefore
// first added in pairs in fp16 (one rounding of a sum of two values, a
// relative 2^-11 at most), halving the v_dot2 count: +3 to +6 % on MI355X,
// and at most 4e-4 of LSE error against the fp64 oracle in the tests'
// problems (1.9e-4 before).  At d = 64 and 128 it gained under 1 %, and two
// or more fp16 levels cost more accuracy (1.3e-3 of LSE error with the whole
// tree at d = 64 with spiky logits), so the other head_dims keep v_dot2.
#ifndef ATTN_ROWSUM_PK
#define ATTN_ROWSUM_PK -1  // fp16 pair levels; -1: one at d = 256, none elsewhere
#endif
template <int D>
constexpr int row_sum_fp16_levels() { return ATTN_ROWSUM_PK >= 0 ? ATTN_ROWSUM_PK : (D == 256 ? 1 : 0); }

template <int D, typename T = _Float16>
__device__ __forceinline__ void add_row_sums(const PTile<D>& pf, float (&l_run)[Cfg<D>::QB]) {
  using C = Cfg<D>;
  constexpr int kLevels = row_sum_fp16_levels<D>();
  if constexpr (kLevels > 0 && !std::is_same_v<T, __bf16>) {
    // kLevels levels of a pairwise tree of packed fp16 additions over the
    // tile's 8 NT pairs, then v_dot2 into fp32.
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      constexpr int n = 8 * C::NT;
      half2v v[n];
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[8 * t + 4 * h + i] = half2v{pf[qb][t][h][2 * i], pf[qb][t][h][2 * i + 1]};
      int w = n;
#pragma unroll
      for (int lvl = 0; lvl < kLevels && w > 1; ++lvl) {
        w /= 2;
#pragma unroll
        for (int i = 0; i < w; ++i) v[i] = v[i] + v[i + w];
      }
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int i = 0; i < w; ++i) {
        if (i & 1) l1 = __builtin_amdgcn_fdot2(v[i], half2v{1.0f16, 1.0f16}, l1, false);
        else l0 = __builtin_amdgcn_fdot2(v[i], half2v{1.0f16, 1.0f16}, l0, false);
      }
      l_run[qb] += l0 + l1;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
      {
        const half8 x = pf[qb][t][h];
        if constexpr (std::is_same_v<T, __bf16>) {
          const bf16x8 y = __builtin_bit_cast(bf16x8, x);
          const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
          l0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[0], y[1]}, one, l0, false);
          l1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[2], y[3]}, one, l1, false);
          l0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[4], y[5]}, one, l0, false);
          l1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[6], y[7]}, one, l1, false);
        } else {
          l0 = __builtin_amdgcn_fdot2(half2v{x[0], x[1]}, half2v{1.0f16, 1.0f16}, l0, false);
          l1 = __builtin_amdgcn_fdot2(half2v{x[2], x[3]}, half2v{1.0f16, 1.0f16}, l1, false);
          l0 = __builtin_amdgcn_fdot2(half2v{x[4], x[5]}, half2v{1.0f16, 1.0f16}, l0, false);
          l1 = __builtin_amdgcn_fdot2(half2v{x[6], x[7]}, half2v{1.0f16, 1.0f16}, l1, false);
        }
      }
    l_run[qb] += l0 + l1;
  }
}

// Sum of the 16 probabilities of one lane's 32-key block (two half8 B
// operands), in fp32 with v_dot2 (two partial sums for a shorter chain).
template <typename T>
__device__ __forceinline__ float row_sum16(const half8 (&pf)[2]) {
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const half8 x = pf[h];
    if constexpr (std::is_same_v<T, __bf16>) {
      const bf16x8 y = __builtin_bit_cast(bf16x8, x);
      const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
      l0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[0], y[1]}, one, l0, false);
      l1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[2], y[3]}, one, l1, false);
      l0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[4], y[5]}, one, l0, false);
      l1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{y[6], y[7]}, one, l1, false);
    } else {
      l0 = __builtin_amdgcn_fdot2(half2v{x[0], x[1]}, half2v{1.0f16, 1.0f16}, l0, false);
      l1 = __builtin_amdgcn_fdot2(half2v{x[2], x[3]}, half2v{1.0f16, 1.0f16}, l1, false);
      l0 = __builtin_amdgcn_fdot2(half2v{x[4], x[5]}, half2v{1.0f16, 1.0f16}, l0, false);
      l1 = __builtin_amdgcn_fdot2(half2v{x[6], x[7]}, half2v{1.0f16, 1.0f16}, l1, false);
    }
  }
  return l0 + l1;
}

// O^T += V^T P^T for one key tile.  The A operand pairs B slot j of lane
// group g with key 8 (j/4) + 4 g + j%4 (+16 h, +32 t): two transpose reads of
// four keys each from V in its natural [key][dim] layout, shared by every
// query block of the wave.
template <int D, typename T = _Float16>
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
        const short4v lo = tr_read(vs + off.vofs(0, dt) + kb);
        const short4v hi = tr_read(vs + off.vofs(1, dt) + kb);
        const half8 a = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
          oacc[qb][dt] = mfma16<T>(a, pf[qb][t][h], oacc[qb][dt]);
      }
    }
}

// Stores one wave's 32 finished rows of an output, acc * mult rounded to T:
// NDT 32-dim tiles of each row (the dims from `out` on; rows D elements
// apart in memory).  In the accumulator layout a lane holds 8-byte pieces of
// its own row (lane % 32) at 4 NDT places, so a direct store writes 32 rows x
// 16 bytes per instruction.  The rows are instead written to the wave's own
// LDS region (16-byte chunks XOR-swizzled by row: at most 2-way bank
// conflicts, 4-way for 128-byte rows, once per workgroup) and read back so
// that each lane stores 16 consecutive bytes of a row: fully coalesced
// stores, 2 NDT of them.
// `region` (32 * CPR * 16 bytes) must no longer be in use by copies or
// reads; rows at or past `rows_valid` are not stored.
template <int D, typename T, int NDT = Cfg<D>::DT>
__device__ __forceinline__ void store_rows(char* region, const f32x16 (&acc)[NDT], float mult, _Float16* out,
                                           int rows_valid, int lane) {
  using C = Cfg<D>;
  constexpr int CH = 4 * NDT;  // 16-byte chunks of a row to store
  constexpr int MASK = C::CPR - 1;
  static_assert(CH <= C::CPR, "a row must fit the LDS row pitch");
  const int r = lane & 31, g = lane >> 5;
  // The region may still be read by this wave's previous call.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      half4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = to_elem<T>(acc[dt][4 * rq + i] * mult);
      const int c = 4 * dt + rq;  // chunk of dims 32 dt + 8 rq .. +7; this lane's half is 4 g .. 4 g + 3
      *reinterpret_cast<half4*>(region + (r * C::CPR + (c ^ (r & MASK))) * 16 + 8 * g) = h;
    }
  // Every lane's writes land before any lane reads (LDS work of one wave).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int it = 0; it < 2 * NDT; ++it) {  // 32 rows x CH chunks over 64 lanes
    const int p = it * 64 + lane;
    const int row = p / CH, c = p - row * CH;
    const u32x4 x = *reinterpret_cast<const u32x4*>(region + (row * C::CPR + (c ^ (row & MASK))) * 16);
    if (row < rows_valid) *reinterpret_cast<u32x4*>(out + (size_t)row * D + 8 * c) = x;
  }
}

// LDS region of wave wv for store_rows, inside the K/V stages.
template <int D>
__device__ __forceinline__ char* row_region(char* smem, int wv) {
  static_assert(kWaves * 32 * Cfg<D>::CPR * 16 <= 4 * Cfg<D>::TILE_BYTES, "output staging must fit the K/V stages");
  return smem + wv * (32 * Cfg<D>::CPR * 16);
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
  __device__ __forceinline__ void clear_sums(int qb) { l_run[qb] = 0.f; }
  // The row's sum l over every visible key (both lane halves).
  __device__ __forceinline__ float total_sum(int qb) const { return xlane_sum(l_run[qb]); }
};

// Workgroup id -> position in the list of work, so that each of the 8 XCDs
// (one L2 each) receives a contiguous range of it (consecutive ids go
// round-robin over the XCDs).
__device__ __forceinline__ int xcd_work_index() {
  const int nb = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3, q8 = nb >> 3, r8 = nb & 7;
  return xcd * q8 + (xcd < r8 ? xcd : r8) + slot;
}

// Causal work order: position u of the list -> (head, rank), rank 0 the
// heaviest of the head's `units` tiles.  Heads go in groups of `group`
// (causal_head_group in attn_launch.h); inside a group the tiles of all its
// heads run heaviest first (rank 0 of every head, then rank 1, ...), so that
// the light tiles of the last heads fill the tail.  A bijection for any
// group size (the last group may be smaller).
__device__ __forceinline__ void grouped_order(int u, int units, int heads, int group, int& head, int& rank) {
  const int per_group = group * units;
  const int hg = u / per_group;
  const int rem = u - hg * per_group;
  const int in_group = min(group, heads - hg * group);
  rank = rem / in_group;
  head = hg * group + (rem - rank * in_group);
}

// LDS layout: K tiles in stages 0/1, then V tiles in stages 0/1.
template <int D>
__device__ __forceinline__ char* k_stage(char* smem, int st) { return smem + st * Cfg<D>::TILE_BYTES; }
template <int D>
__device__ __forceinline__ char* v_stage(char* smem, int st) { return smem + (2 + st) * Cfg<D>::TILE_BYTES; }

// The four K/V stages as separate LDS objects (K stages 0/1, V stages 0/1;
// the kernel declares them).  With every stage its own object and the stage
// index a compile-time constant, the compiler can tell that a read of one
// stage does not alias a buffer-to-LDS copy in flight into another, and does
// not wait for those copies before the read; with the stages as parts of
// one array it waits for every copy in flight.
template <int D>
struct KVStages {
  char* k[2];
  char* v[2];
  // LDS region of wave wv for store_rows: the stages in the order K0, K1,
  // V0, V1, each holding TILE_BYTES / (32 CPR 16) waves' regions.
  __device__ __forceinline__ char* region(int wv) const {
    constexpr int kRegion = 32 * Cfg<D>::CPR * 16;
    constexpr int kPer = Cfg<D>::TILE_BYTES / kRegion;
    static_assert(kPer >= 1 && 4 * kPer >= kWaves, "output staging must fit the K/V stages");
    const int obj = wv / kPer;
    char* base = obj == 0 ? k[0] : obj == 1 ? k[1] : obj == 2 ? v[0] : v[1];
    return base + (wv - obj * kPer) * kRegion;
  }
};

// Calls f(std::integral_constant<int, D>{}) for a supported head_dim d
// (a multiple of 32 from 32 to 256) and returns its status.
// ATTN_ONLY_D: instantiate that head_dim alone (the second forward
// translation unit, and the offline tile sweep's variants, which then
// compile in seconds); any other d is refused.
template <typename F>
__host__ hipError_t with_head_dim(int d, F&& f) {
#ifdef ATTN_ONLY_D
  if (d != ATTN_ONLY_D) return hipErrorInvalidValue;
  return f(std::integral_constant<int, ATTN_ONLY_D>{});
#else
  switch (d) {
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    case 96: return f(std::integral_constant<int, 96>{});
    case 128: return f(std::integral_constant<int, 128>{});
    case 160: return f(std::integral_constant<int, 160>{});
    case 192: return f(std::integral_constant<int, 192>{});
    case 224: return f(std::integral_constant<int, 224>{});
    case 256: return f(std::integral_constant<int, 256>{});
    default: return hipErrorInvalidValue;
  }
#endif
}

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
template <int D, bool CAUSAL, int PAR, typename T = _Float16, bool UNIFORM = false>
__device__ __forceinline__ void pipeline_step(int j, int nt, const KVStages<D>& st,
                                              __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                              const LoadOffsets<D>& lo, int tid, WaveState<D>& w,
                                              STile<D>& s_cur, STile<D>& s_nxt) {
  using C = Cfg<D>;
  const uint32_t v_base = tile_base<D>(j + 1, nt);
  const uint32_t k_base = tile_base<D>(j + 2, nt);
  // UNIFORM: the caller's waves all compute every tile (rows past the end
  // only produce values that are never stored).  Telling the compiler so
  // keeps the copies inside the block it schedules with the matrix work
  // instead of ahead of it: +4-5 % for the forward at d = 64 without the
  // mask, -1 to -6 % at the other head_dims, which keep the runtime test.
  if (UNIFORM || j < w.nt_w) {
    load_tile<D>(vrs, st.v[PAR ^ 1], v_base, lo, tid);
    load_tile<D>(krs, st.k[PAR], k_base, lo, tid);
    paranoid_sync();
    // S_{j+1} is computed even past this wave's last tile (reading a stale
    // but in-bounds stage) so that the matrix and vector work stay in one
    // block the scheduler can interleave; it is discarded then.
    qk_tile<D, T>(st.k[PAR ^ 1], w.qf, w.off, s_nxt);
    PTile<D> pf;
    softmax_tile<D, T>(s_cur, w.c, w.m_run, pf);
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
    pv_tile<D, T>(st.v[PAR], pf, w.off, w.oacc);
    add_row_sums<D, T>(pf, w.l_run);
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
    paranoid_sync();
  } else {
    load_tile<D>(vrs, st.v[PAR ^ 1], v_base, lo, tid);
    load_tile<D>(krs, st.k[PAR], k_base, lo, tid);
    paranoid_sync();
    paranoid_sync();
  }
  wait_vm_all();
  __syncthreads();
}

}  // namespace
}  // namespace attn

#endif  // ATTN_TILE_H_
