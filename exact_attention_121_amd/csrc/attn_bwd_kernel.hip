// Fused attention backward for gfx950: dQ, dK, dV from Q, K, V, the
// forward's O and LSE, and the upstream gradient dO, in fp16 or bf16 (P and
// dS take the same type for the products that use them; sums are fp32).
//
// The pages name training as a use of the operator ([CANN-FA], opening
// paragraph) and note that backpropagation must keep gradients ([FA-Dict]
// section "Standard attention"); the gradients follow from the forward
// definition ([CANN-FA] section "Where is the bottleneck of standard
// attention") by the chain rule:
//   P  = exp(scale Q K^T - LSE)          (recomputed tile by tile from the
//                                         stored LSE: no N x N matrix)
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - Delta),  Delta_i = dO_i . O_i
//   dQ = scale dS K,  dK = scale dS^T Q
// As in the forward, S and P never leave the chip.
//
// Two kernels, dQ first:
//   * attn_bwd_dq_kernel: one workgroup per 128 query rows, shaped like the
//     forward kernel: S^T = K Q^T and dP^T = V dO^T, then dQ^T += K^T dS^T.
//     Its prologue also computes each row's Delta_i = dO_i . O_i and
//     LSE_i * log2(e) and stores them in a workspace padded to whole 128-row
//     tiles (padding rows: Delta = 0 and LSE = +inf, so that their
//     probabilities are exactly 0 with no bounds check).
//   * attn_bwd_dkdv_kernel: one workgroup per 128 keys of one key/value head
//     (32 per wave, the lanes' columns; with head_dim 256 on small grids, per
//     half of the output dims as well); K and V stay in registers as matrix
//     operands; the Q and dO tiles of every query head of the group stream
//     through LDS with their Delta / LSE rows.  Per query tile: S = Q K^T and
//     dP = dO V^T on the matrix cores, P and dS on the vector ALUs, then
//     dV^T += dO^T P and dK^T += Q^T dS with P and dS used straight from
//     registers and the transposed tiles read with ds_read_b64_tr_b16 (the
//     forward's P.V step).  Two forms of that step, chosen at launch: the
//     whole tile at once, or one 32-query half at a time, which keeps fewer
//     registers live and runs two workgroups per CU (non-causal grids of two
//     workgroups per CU).
// The two main kernels recompute S and dP each; there are no atomics, and
// every output element is written once.
//
// Pages cited:
//   [CANN-FA]  www.mooersco.com/news/1200175
//   [FA-Dict]  hwcomputing.csdn.net/6a0dbd08662f9a54cb75eb74.html

#include <mutex>
#include <type_traits>

#include "attn_tile.h"

// Fixed scratch of the allocation-free backward (attn_bwd_noalloc): the
// per-row LSE and Delta terms, 2 * 4 bytes per padded query row, for at most
// 2^21 rows.  Each GPU the library runs on holds its own copy until the
// process ends.
static __device__ __align__(256) char scratch[attn::kBwdNoallocScratchBytes];

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// The 16 bits of an element of type T (fp16 or bf16) as fp32 (exact).
template <typename T>
__device__ __forceinline__ float from_elem(_Float16 bits) {
  if constexpr (std::is_same_v<T, __bf16>)
    return static_cast<float>(__builtin_bit_cast(__bf16, bits));
  else
    return static_cast<float>(bits);
}

struct BwdParams {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  const _Float16* o;
  const _Float16* dout;
  const float* lse;   // forward LSE, natural log, [B][Hq][N]
  _Float16* dq;
  _Float16* dk;
  _Float16* dv;
  float* lse2;        // workspace [B][Hq][Npad]: LSE * log2(e); +inf past N
  float* delta;       // workspace [B][Hq][Npad]: dO . O; 0 past N
  int N, Npad, Hq, Hkv, group, rows_total;
  float c;            // scale * log2(e), any sign
  float scale;
  int group_dkdv, group_dq;   // causal: heads whose tiles run interleaved, heaviest first
};

// Probabilities and dS of one tile from the scores s and dP, with per-entry
// LSE (log2) and Delta: P = exp2(c s - lse2), masked entries (arg = -inf)
// give exactly 0; dS = P (dP - delta).  Both rounded to fp16 as the B
// operands of the following products (the forward's P layout).
template <int D, typename T>
__device__ __forceinline__ void p_and_ds(const STile<D>& arg, const STile<D>& dp, const float (&delta)[Cfg<D>::NT][16],
                                         PTile<D>& pf, PTile<D>& dsf) {
  using C = Cfg<D>;
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(arg[0][t][r]);
      pf[0][t][r >> 3][r & 7] = to_elem<T>(pv);
      dsf[0][t][r >> 3][r & 7] = to_elem<T>(pv * (dp[0][t][r] - delta[t][r]));
    }
}

// Workgroups per key block of dK/dV (each takes 1/parts of the output dims
// and recomputes S and dP), chosen at launch.  One everywhere except d = 256
// on a grid of fewer than kDkdvOnePartMinGrid key blocks: there the dims are
// split in two, which doubles the workgroups (and the S / dP work).  With
// one part, d = 256 keeps K, V and both accumulators in 504 registers (the
// sub-tile form, no spill; the whole-tile form spills 68 bytes) at one
// workgroup per CU: +23 % on the LLaMA-7B layer shape and +8.5 % on the
// causal GQA workload (512 key blocks) on MI355X, but -24 % on a 256-block
// grid, where the split's second workgroup per block is what fills the CUs.
constexpr unsigned kDkdvOnePartMinGrid = 512;
template <int D>
inline int bwd_dim_parts(unsigned key_blocks) { return D == 256 && key_blocks < kDkdvOnePartMinGrid ? 2 : 1; }

// Order of the dK/dV work inside a step: one 32-query sub-tile at a time
// (SUB: fewer live registers, two workgroups per CU up to d = 128) or the
// whole tile at once (more independent matrix work in flight per wave).
// Measured on gfx950: sub-tiles are faster without the causal mask once the
// grid gives every CU two workgroups (at d = 256 with one dim part: one
// workgroup per CU either way, and the whole tile would spill); with the
// mask, or on smaller grids, the whole tile is.
template <int D, bool CAUSAL>
constexpr bool bwd_dkdv_subtile_form() { return !CAUSAL; }
constexpr unsigned kDkdvSubtileMinGrid = 512;   // two workgroups for each of the 256 CUs

// dK/dV workgroups per CU the register budget allows (K, V and the two
// accumulators stay in registers).
template <int D, bool SUB>
constexpr int bwd_dkdv_wg_per_cu() { return D <= (SUB ? 128 : 64) ? 2 : 1; }

// dQ workgroups per CU (Q, dO and the dQ accumulators stay in registers):
// two fit without spilling up to d = 160 (at d = 192 the spill cost the
// causal and small grids 7-9 %).
template <int D>
constexpr int bwd_dq_wg_per_cu() { return D <= 160 ? 2 : 1; }

// P and dS of one 32-query sub-tile from its scores s and dP (no mask):
// entry r is query 8 (r / 4) + r % 4 past the lane's first, whose LSE (log2)
// and Delta lse and delta point at in LDS; P = exp2(c s - lse) and dS =
// P (dP - delta), rounded to T.
template <typename T>
__device__ __forceinline__ void p_ds_subtile(const f32x16& s, const f32x16& dp, const float* lse, const float* delta,
                                             float c, half8 (&pf)[2], half8 (&dsf)[2]) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float4 l4 = *reinterpret_cast<const float4*>(lse + 8 * rr);
    const float4 d4 = *reinterpret_cast<const float4*>(delta + 8 * rr);
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
    const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * rr + i;
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lv[i]));
      pf[r >> 3][r & 7] = to_elem<T>(pv);
      dsf[r >> 3][r & 7] = to_elem<T>(pv * (dp[r] - dv[i]));
    }
  }
}

// Sub-tile t of a stage (its 32 rows 32 t .. 32 t + 31, from LDS) times the
// wave's fragments (B operands, 32 columns): S_t = Q_t K^T or dP_t = dO_t V^T.
template <int D, typename T, typename KO>
__device__ __forceinline__ f32x16 rows_times_frags(const char* stage, const QFrag<D>& frags, const KO& kofs, int t) {
  using C = Cfg<D>;
  f32x16 acc = {};
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    const half8 a = *reinterpret_cast<const half8*>(stage + kofs(dc) + 32 * t * C::CPR * 16);
    acc = mfma16<T>(a, frags[0][dc], acc);
  }
  return acc;
}

// acc[i] += (sub-tile t of a stage)^T p over NDT 32-dim output tiles: the
// transposed rows 32 t .. 32 t + 31 as A operands (transpose reads at the
// lane offsets voff(key group, i)), p (the sub-tile's P or dS) as B operands.
template <int D, int NDT, typename T, typename VO>
__device__ __forceinline__ void tr_times_p(const char* stage, const half8 (&p)[2], const VO& voff, int t,
                                           f32x16 (&acc)[NDT]) {
  using C = Cfg<D>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kb = (32 * t + 16 * h) * C::CPR * 16;
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const short4v lo = tr_read(stage + voff(0, i) + kb);
      const short4v hi = tr_read(stage + voff(1, i) + kb);
      const half8 a = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[i] = mfma16<T>(a, p[h], acc[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Query tiles of BN rows stream through LDS (Q in the "K" stages,
// dO in the "V" stages); the wave's 32 keys are the columns of S and dP.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SUB, int NP, typename T>
__global__ __launch_bounds__(kThreads, (bwd_dkdv_wg_per_cu<D, SUB>())) void attn_bwd_dkdv_kernel(BwdParams p, int k_tiles) {
  using C = Cfg<D>;
  static_assert(C::QB == 1, "one 32-key block per wave");
  // The step loop is unrolled by two, so that the stage is a compile-time
  // constant, above d = 64.  Up to d = 64 it is not: there the unrolled
  // whole-tile form spills at two workgroups per CU (72 bytes per lane with
  // the mask), and the unrolled sub-tile form measured 2 % slower.
  constexpr bool kUnrolled = D > 64;
  // Q stages 0/1, dO stages 0/1 and per stage the tile's LSE (log2) and
  // Delta rows (64 floats each; a 32-row tile uses the first half), all
  // filled by buffer-to-LDS copies.  Unrolled, each stage is an LDS object of
  // its own: a read of an object that a copy in flight may write makes the
  // compiler wait for every copy in flight, the next tile's included.  With a
  // run-time stage index they are one object (selecting between objects at
  // run time costs about 50 instructions a step).
  constexpr int kRowTerms = 2 * 64 * 4;
  constexpr int kFirst = kUnrolled ? C::TILE_BYTES : 4 * C::TILE_BYTES + 2 * kRowTerms;
  constexpr int kOther = kUnrolled ? C::TILE_BYTES : 16;
  __shared__ __attribute__((aligned(1024))) char qs0[kFirst];
  __shared__ __attribute__((aligned(1024))) char qs1[kOther];
  __shared__ __attribute__((aligned(1024))) char ds0[kOther];
  __shared__ __attribute__((aligned(1024))) char ds1[kOther];
  __shared__ __attribute__((aligned(16))) char rt0[kUnrolled ? kRowTerms : 16];
  __shared__ __attribute__((aligned(16))) char rt1[kUnrolled ? kRowTerms : 16];
  auto qst = [&](int i) -> char* { return kUnrolled ? (i == 0 ? qs0 : qs1) : qs0 + i * C::TILE_BYTES; };
  auto dost = [&](int i) -> char* { return kUnrolled ? (i == 0 ? ds0 : ds1) : qs0 + (2 + i) * C::TILE_BYTES; };
  // [lse2 | delta][64] of stage i
  auto rts = [&](int i) -> float* {
    return reinterpret_cast<float*>(kUnrolled ? (i == 0 ? rt0 : rt1) : qs0 + 4 * C::TILE_BYTES + i * kRowTerms);
  };

  constexpr int NDT = C::DT / NP;       // 32-dim output tiles of this workgroup
  // Work list position -> (K/V head, key tile, dim part), contiguous per
  // XCD; causal: the heaviest key tiles (the first) first across a group of
  // heads.
  const int wi = xcd_work_index();
  int part, kt, bk;   // bk = b * Hkv + kvh
  if (CAUSAL) {
    int rank;
    grouped_order(wi, k_tiles * NP, gridDim.x / (k_tiles * NP), p.group_dkdv, bk, rank);
    part = rank % NP;
    kt = rank / NP;
  } else {
    part = wi % NP;
    kt = (wi / NP) % k_tiles;
    bk = wi / NP / k_tiles;
  }
  const int b = bk / p.Hkv, kvh = bk - b * p.Hkv;
  const int N = p.N;
  const int k0 = kt * kBwdKeys;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int kw0 = k0 + 32 * wv;          // first key of this wave
  const int key = kw0 + (lane & 31);     // this lane's key (column)

  // K and V rows of the wave as B operands (dims 16 dc + 8 g .. +7).
  const size_t kvoff = (size_t)bk * N * D;
  QFrag<D> kf, vf;
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    const size_t e = kvoff + (size_t)key * D + 16 * dc + 8 * g;
    kf[0][dc] = key < N ? *reinterpret_cast<const half8*>(p.k + e) : half8{};
    vf[0][dc] = key < N ? *reinterpret_cast<const half8*>(p.v + e) : half8{};
  }
  f32x16 dk_acc[NDT], dv_acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) {
    dk_acc[i] = f32x16{};
    dv_acc[i] = f32x16{};
  }
  Offsets<D> off;
  off.init(lane);
  // Transpose-read offsets of this workgroup's output dims: the Offsets
  // registers when one workgroup covers all dims; with the dims split over
  // NP workgroups, those of this workgroup's part (as Offsets::init).
  int vpart[NP == 1 ? 1 : 2][NP == 1 ? 1 : NDT];
  if constexpr (NP > 1) {
    const int m16 = lane & 15;
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (m16 & 3);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int dim = 32 * (part * NDT + i) + dsub;
        vpart[hi][i] = swz<D>(4 * g + (m16 >> 2) + 8 * hi, dim >> 3) + (dim & 7) * 2;
      }
  }
  auto voff = [&](int hi, int i) { return NP == 1 ? off.vofs(hi, i) : vpart[NP == 1 ? 0 : hi][NP == 1 ? 0 : i]; };
  // Q / dO operand read offsets (chunks 2 dc + g of row lane % 32): with the
  // XOR swizzle, swz(r, 2 dc + g) = kbase + 32 (dc ^ (f(r) >> 1)) (+256 for
  // the upper 16 chunks of 32-chunk rows), kbase = (r CPR + (g ^ (f(r) & 1)))
  // 16.  The step recomputes them from these two registers (two vector ops
  // per read) instead of keeping Offsets' eight: at d = 128 the eight spilled,
  // and every reload in the loop waited (vmcnt) for the next tile's copies.
  const int fr = (swz<D>(lane & 31, 0) >> 4) - (lane & 31) * C::CPR;  // f(r)
  int khalf = fr >> 1;
  int kbase = ((lane & 31) * C::CPR + (g ^ (fr & 1))) * 16;
  auto kofs = [&](int dc) {
    return dc < 8 ? kbase + ((dc ^ khalf) << 5) : kbase + (((dc - 8) ^ khalf) << 5) + 256;
  };
  LoadOffsets<D> lo;
  lo.init(tid);

  // Steps: (query head of the group, query tile), query tiles from the one
  // holding key k0 (causal) to the end.
  const int q_tiles = (N + C::BN - 1) / C::BN;
  const int qt0 = CAUSAL ? k0 / C::BN : 0;
  const int nq = q_tiles - qt0;
  const int steps = p.group * nq;
  const int head_bytes = static_cast<int>(static_cast<uint32_t>(N) * (D * 2));
  auto issue = [&](int u, int st) {
    const int gq = u < steps ? u / nq : 0;
    const int qt = u < steps ? qt0 + (u - gq * nq) : 0;
    const size_t qoff = ((size_t)b * p.Hq + kvh * p.group + gq) * N * D;
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + qoff), (short)0, head_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t drs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.dout + qoff), (short)0, head_bytes, kBufferWord3);
    const uint32_t base = tile_base<D>(u < steps ? qt : 0, u < steps ? q_tiles : 0);
    load_tile<D>(qrs, qst(st), base, lo, tid);
    load_tile<D>(drs, dost(st), base, lo, tid);
    // Waves 0 and 1 copy the tile's 64 LSE / Delta rows (4 bytes a lane);
    // rows past the head's padded rows read as 0 and are never used.
    if (wv < 2) {
      const size_t rb = ((size_t)b * p.Hq + kvh * p.group + gq) * p.Npad;
      const float* src = (wv == 0 ? p.lse2 : p.delta) + rb;
      const __amdgpu_buffer_rsrc_t rrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, p.Npad * 4, kBufferWord3);
      const uint32_t voff = u < steps ? static_cast<uint32_t>(qt * C::BN + lane) * 4 : kSkipTile;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rrs, (lds_void*)(rts(st) + wv * 64), 4, static_cast<int>(voff), 0, 0, 0);
    }
  };

  issue(0, 0);
  wait_vm_all();
  __syncthreads();
  // One step per (query head, query tile); `stc` is the LDS stage, a
  // compile-time constant where the loop is unrolled by two, so that the
  // stage addresses fold into the LDS instructions' offsets.
  auto step = [&](auto stc, int u) {
    const int st = stc;
    // Keep the offset computation inside the loop (not hoisted and spilled).
    if constexpr (SUB) asm volatile("" : "+v"(khalf), "+v"(kbase));
    const int gq = u / nq;
    const int q0 = (qt0 + (u - gq * nq)) * C::BN;
    // Causal: skip tiles whose every query precedes every key of the wave
    // (wave-uniform, as the matrix instructions need).
    const bool active = kw0 < N && !(CAUSAL && q0 + C::BN - 1 < kw0);
    issue(u + 1, st ^ 1);
    paranoid_sync();
    if (active) {
      const float* lrow = rts(st);        // LSE (log2) of the tile's queries
      const float* drow = rts(st) + 64;   // Delta of the tile's queries
      if constexpr (SUB) {
        // One 32-query sub-tile t at a time: S_t and dP_t, then P_t and
        // dS_t, then their products, so that only one sub-tile's scores and
        // LSE / Delta are live.  Entry r of sub-tile t is query
        // q0 + 32 t + 8 (r / 4) + 4 g + r % 4.
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
          // Keep the scheduler from hoisting sub-tile t's operand reads into
          // sub-tile t - 1, which lengthens register lifetimes (at d = 128
          // the spill falls from 52 to 36 bytes per lane; 4 % faster).
          __builtin_amdgcn_sched_barrier(0);
          const f32x16 s = rows_times_frags<D, T>(qst(st), kf, kofs, t);   // S_t = Q_t K^T
          const f32x16 dp = rows_times_frags<D, T>(dost(st), vf, kofs, t);  // dP_t = dO_t V^T
          half8 pf[2], dsf[2];
          p_ds_subtile<T>(s, dp, lrow + 32 * t + 4 * g, drow + 32 * t + 4 * g, p.c, pf, dsf);
          tr_times_p<D, NDT, T>(dost(st), pf, voff, t, dv_acc);    // dV^T += dO_t^T P_t
          tr_times_p<D, NDT, T>(qst(st), dsf, voff, t, dk_acc);   // dK^T += Q_t^T dS_t
        }
      } else {
        // The whole tile at once: S and dP of every sub-tile, the causal
        // mask on tiles that cross the wave's diagonal, then P and dS and
        // their products.
        float lse2[C::NT][16], delta[C::NT][16];
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float4 l4 = *reinterpret_cast<const float4*>(lrow + 32 * t + 8 * rr + 4 * g);
            const float4 d4 = *reinterpret_cast<const float4*>(drow + 32 * t + 8 * rr + 4 * g);
            lse2[t][4 * rr + 0] = l4.x;
            lse2[t][4 * rr + 1] = l4.y;
            lse2[t][4 * rr + 2] = l4.z;
            lse2[t][4 * rr + 3] = l4.w;
            delta[t][4 * rr + 0] = d4.x;
            delta[t][4 * rr + 1] = d4.y;
            delta[t][4 * rr + 2] = d4.z;
            delta[t][4 * rr + 3] = d4.w;
          }
        STile<D> s, dp;
        qk_tile<D, T>(qst(st), kf, off, s);    // S = Q K^T: rows queries, columns keys
        qk_tile<D, T>(dost(st), vf, off, dp);   // dP = dO V^T
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[0][t][r] = __builtin_fmaf(s[0][t][r], p.c, -lse2[t][r]);
        if (CAUSAL && q0 < kw0 + 31) {
          // Entry r of sub-tile t is query q0 + 4 g + (32 t + 8 (r / 4) +
          // r % 4): visible iff that constant offset reaches key - q0 - 4 g.
          const int first = key - q0 - 4 * g;
#pragma unroll
          for (int t = 0; t < C::NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              s[0][t][r] = 32 * t + 8 * (r >> 2) + (r & 3) >= first ? s[0][t][r] : -INFINITY;
        }
        PTile<D> pf, dsf;
        p_and_ds<D, T>(s, dp, delta, pf, dsf);
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
          tr_times_p<D, NDT, T>(dost(st), pf[0][t], voff, t, dv_acc);    // dV^T += dO^T P
        }
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
          tr_times_p<D, NDT, T>(qst(st), dsf[0][t], voff, t, dk_acc);   // dK^T += Q^T dS
        }
      }
    }
    paranoid_sync();
    wait_vm_all();
    __syncthreads();
    };
  if constexpr (!kUnrolled) {
    for (int u = 0; u < steps; ++u) step(u & 1, u);
  } else {
    for (int u = 0; u < steps; u += 2) {
      step(std::integral_constant<int, 0>{}, u);
      if (u + 1 < steps) step(std::integral_constant<int, 1>{}, u + 1);
    }
  }

  // The loop's last barrier freed the stages: each wave stages its rows of
  // dK and then dV there for coalesced stores.
  constexpr int kRegion = 32 * C::CPR * 16;  // one wave's rows
  constexpr int kPerStage = C::TILE_BYTES / kRegion;
  static_assert(kPerStage >= 1 && 4 * kPerStage >= kWaves, "the output rows must fit the four stages");
  const int obj = wv / kPerStage;
  char* region = (obj < 2 ? qst(obj) : dost(obj - 2)) + (wv % kPerStage) * kRegion;
  store_rows<D, T, NDT>(region, dk_acc, p.scale, p.dk + kvoff + (size_t)kw0 * D + 32 * part * NDT, N - kw0, lane);
  store_rows<D, T, NDT>(region, dv_acc, 1.0f, p.dv + kvoff + (size_t)kw0 * D + 32 * part * NDT, N - kw0, lane);
}

// ---------------------------------------------------------------------------
// dQ.  Like the forward kernel: 128 query rows per workgroup (32 per wave,
// the lanes' columns), K and V tiles stream through LDS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, typename T>
__global__ __launch_bounds__(kThreads, bwd_dq_wg_per_cu<D>()) void attn_bwd_dq_kernel(BwdParams p, int q_tiles) {
  using C = Cfg<D>;
  static_assert(C::QB == 1, "one 32-row block per wave");
  // K stages 0/1 then V stages 0/1 in one array.  (As separate objects,
  // which drops the compiler's waits for copies in flight before reads of
  // the other stages, the backward steps measured -3 % at d = 64 and within
  // 0.5 % elsewhere.)
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES];
  const KVStages<D> kv{{smem, smem + C::TILE_BYTES}, {smem + 2 * C::TILE_BYTES, smem + 3 * C::TILE_BYTES}};

  // As in the forward: causal query tiles heaviest first across a group of
  // heads.
  const int wi = xcd_work_index();
  int qt, bh;   // bh = b * Hq + hq
  if (CAUSAL) {
    grouped_order(wi, q_tiles, gridDim.x / q_tiles, p.group_dq, bh, qt);
    qt = q_tiles - 1 - qt;
  } else {
    qt = wi % q_tiles;
    bh = wi / q_tiles;
  }
  const int b = bh / p.Hq, hq = bh - b * p.Hq, kvh = hq / p.group;
  const int N = p.N;
  const int q0 = qt * C::BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int qw0 = q0 + 32 * wv;
  const int row = qw0 + (lane & 31);

  const size_t qoff = (size_t)bh * N * D;
  QFrag<D> qf, df;
  float dpart = 0.f;   // this lane's half of Delta = dO . O for its row
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    const size_t e = qoff + (size_t)row * D + 16 * dc + 8 * g;
    qf[0][dc] = row < N ? *reinterpret_cast<const half8*>(p.q + e) : half8{};
    df[0][dc] = row < N ? *reinterpret_cast<const half8*>(p.dout + e) : half8{};
    const half8 of = row < N ? *reinterpret_cast<const half8*>(p.o + e) : half8{};
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart += from_elem<T>(df[0][dc][i]) * from_elem<T>(of[i]);
  }
  // The row terms: Delta (the other half from lane L ^ 32) and LSE in log2
  // units, +inf and 0 past N (probabilities exactly 0).  Stored for the
  // dK/dV kernel, which runs after this one.
  const float delta = xlane_sum(dpart);
  const float lse2 = row < N ? p.lse[(size_t)bh * N + row] * kLog2e : INFINITY;
  if (g == 0) {
    p.delta[(size_t)bh * p.Npad + row] = delta;
    p.lse2[(size_t)bh * p.Npad + row] = lse2;
  }
  OAcc<D> dq_acc;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dq_acc[0][dt] = f32x16{};
  Offsets<D> off;
  off.init(lane);
  LoadOffsets<D> lo;
  lo.init(tid);

  const size_t kvoff = ((size_t)b * p.Hkv + kvh) * N * D;
  const int head_bytes = static_cast<int>(static_cast<uint32_t>(N) * (D * 2));
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kvoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kvoff), (short)0, head_bytes, kBufferWord3);

  const int kv_tiles = (N + C::BN - 1) / C::BN;
  int nt = kv_tiles;
  if (CAUSAL) {
    const int last_q = (q0 + C::BM < N ? q0 + C::BM : N) - 1;
    nt = last_q / C::BN + 1 < kv_tiles ? last_q / C::BN + 1 : kv_tiles;
  }
  int nt_w = nt;  // key tiles this wave needs
  if (qw0 >= N) {
    nt_w = 0;
  } else if (CAUSAL) {
    const int last_w = (qw0 + 32 < N ? qw0 + 32 : N) - 1;
    nt_w = last_w / C::BN + 1;
  }

  load_tile<D>(krs, kv.k[0], 0, lo, tid);
  load_tile<D>(vrs, kv.v[0], 0, lo, tid);
  wait_vm_all();
  __syncthreads();
  // One key tile per step; the stage is a compile-time constant in the
  // loop unrolled by two (see the dK/dV kernel).
  auto step = [&](auto stc, int j) {
    const int st = stc;
    const uint32_t nb = tile_base<D>(j + 1, nt);
    load_tile<D>(krs, kv.k[st ^ 1], nb, lo, tid);
    load_tile<D>(vrs, kv.v[st ^ 1], nb, lo, tid);
    paranoid_sync();
    if (j < nt_w) {
      STile<D> s, dp;
      qk_tile<D, T>(kv.k[st], qf, off, s);    // S^T = K Q^T
      qk_tile<D, T>(kv.v[st], df, off, dp);   // dP^T = V dO^T
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[0][t][r] = __builtin_fmaf(s[0][t][r], p.c, -lse2);
      const int kv0 = j * C::BN;
      if (kv0 + C::BN > N || (CAUSAL && kv0 + C::BN - 1 > qw0)) mask_tile<D, CAUSAL>(s, kv0, N, row, g);
      float dl[C::NT][16];
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dl[t][r] = delta;
      PTile<D> pf, dsf;
      p_and_ds<D, T>(s, dp, dl, pf, dsf);
      pv_tile<D, T>(kv.k[st], dsf, off, dq_acc);   // dQ^T += K^T dS^T
    }
    paranoid_sync();
    wait_vm_all();
    __syncthreads();
    };
  // Unrolled by two (at d = 128 the causal kernel then spills 28 bytes per
  // lane and is still faster than with the rolled loop: +6.5 % on a whole
  // backward step, +2-3 % causal).
  for (int j = 0; j < nt; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < nt) step(std::integral_constant<int, 1>{}, j + 1);
  }

  // As in the forward: rows staged in the freed stages, coalesced stores.
  store_rows<D, T>(kv.region(wv), dq_acc[0], p.scale, p.dq + qoff + (size_t)qw0 * D, N - qw0, lane);
}

template <int D, bool CAUSAL, typename T>
hipError_t launch_bwd_t(const BwdArgs& a, BwdParams p, hipStream_t s) {
  using C = Cfg<D>;
  // Work order groups (causal): a dK/dV head streams the Q and dO of its
  // query heads, a dQ head its K/V head (16-bit elements).
  const int k_tiles = (a.N + kBwdKeys - 1) / kBwdKeys;
  const unsigned key_blocks = static_cast<unsigned>(a.B) * a.Hkv * k_tiles;
  const int parts = bwd_dim_parts<D>(key_blocks);
  {
    const int64_t units = static_cast<int64_t>(k_tiles) * parts;
    p.group_dkdv = CAUSAL ? causal_head_group(static_cast<int64_t>(a.B) * a.Hkv * units, units,
                                              static_cast<int64_t>(p.group) * a.N * D * 4, 1) : 1;
    const int64_t q_tiles = (a.N + C::BM - 1) / C::BM;
    p.group_dq = CAUSAL ? causal_head_group(static_cast<int64_t>(a.B) * a.Hq * q_tiles, q_tiles,
                                            static_cast<int64_t>(a.N) * D * 4, p.group) : 1;
  }
  // dQ first: it also writes the per-row Delta and LSE terms the dK/dV
  // kernel reads.
  const int q_tiles = (a.N + C::BM - 1) / C::BM;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, T>), dim3(static_cast<unsigned>(a.B) * a.Hq * q_tiles),
                     dim3(kThreads), 0, s, p, q_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned dkdv_grid = key_blocks * static_cast<unsigned>(parts);
  [&] {
    if constexpr (D == 256) {
      if (parts == 2) {
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, false, 2, T>), dim3(dkdv_grid), dim3(kThreads), 0, s, p,
                           k_tiles);
        return;
      }
    }
    if (bwd_dkdv_subtile_form<D, CAUSAL>() && dkdv_grid >= kDkdvSubtileMinGrid)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, bwd_dkdv_subtile_form<D, CAUSAL>(), 1, T>),
                         dim3(dkdv_grid), dim3(kThreads), 0, s, p, k_tiles);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, false, 1, T>), dim3(dkdv_grid), dim3(kThreads), 0, s, p,
                         k_tiles);
  }();
  return hipGetLastError();
}

}  // namespace

int launch_backward(const BwdArgs& a, void* stream) {
  BwdParams p;
  p.q = static_cast<const _Float16*>(a.q);
  p.k = static_cast<const _Float16*>(a.k);
  p.v = static_cast<const _Float16*>(a.v);
  p.o = static_cast<const _Float16*>(a.o);
  p.dout = static_cast<const _Float16*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<_Float16*>(a.dq);
  p.dk = static_cast<_Float16*>(a.dk);
  p.dv = static_cast<_Float16*>(a.dv);
  p.N = a.N;
  p.Npad = static_cast<int>(bwd_padded_rows(a.N));
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.rows_total = a.B * a.Hq * p.Npad;
  p.lse2 = static_cast<float*>(a.workspace);
  p.delta = p.lse2 + static_cast<size_t>(p.rows_total);
  p.c = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
  p.scale = a.scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = with_head_dim(a.d, [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    if (a.bf16)
      return a.causal ? launch_bwd_t<D, true, __bf16>(a, p, s) : launch_bwd_t<D, false, __bf16>(a, p, s);
    return a.causal ? launch_bwd_t<D, true, _Float16>(a, p, s) : launch_bwd_t<D, false, _Float16>(a, p, s);
  });
  return static_cast<int>(e);
}


// attn_bwd_noalloc: the per-row terms go to this fixed array instead of a
// caller workspace.  In host code `scratch` names a host-side stand-in, not
// the device memory: its device address is looked up once per device (with
// that device current) and only that address is passed to the kernels.
int launch_backward_noalloc(const BwdArgs& a, void* stream) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
      e = hipGetSymbolAddress(&ptrs[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        ptrs[dev] = nullptr;
        return static_cast<int>(e);
      }
      if (ptrs[dev] == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
    }
    ptr = ptrs[dev];
  }
  BwdArgs b = a;
  b.workspace = ptr;
  return launch_backward(b, stream);
}

}  // namespace attn
