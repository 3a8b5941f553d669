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
// The element type of Q, K, V and O is fp16 (the pages' precision) or bf16;
// P takes the same type for the P.V product, all accumulation is fp32.
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
//   * Epilogue: each wave writes its 32 normalised rows to an LDS region of
//     its own and reads them back row-contiguous, so that O leaves in fully
//     coalesced 16-byte-per-lane stores instead of 8-byte pieces of 32 rows.
//   * Workgroup ids are remapped so that each of the 8 XCDs (each with its
//     own L2) receives a contiguous range of (head, query tile) work, i.e. the
//     query tiles of the same heads share their K/V in one L2; causal query
//     tiles run heaviest first, interleaved across a group of heads so that
//     the light tiles of the XCD's last heads fill the tail.

// Tile configuration of this kernel at head_dim 64 (the offline tile sweep
// overrides it with -D): two 32-row query blocks per wave, so that every K/V
// operand read from LDS feeds two matrix instructions, with 32-key tiles so
// that the registers still fit two workgroups per CU (222 per lane).
// Measured on gfx950 against one block and 64-key tiles: +5.5 % on the
// LLaMA-7B layer shape at d = 64, +1.3 % at N = 8192, +0.6 % on the spiky
// causal prefill.  The decode and backward kernels keep the shared defaults.
#ifndef ATTN_QB64
#define ATTN_QB64 2
#endif
#ifndef ATTN_BN64
#define ATTN_BN64 32
#endif
#ifndef ATTN_WG64
#define ATTN_WG64 2
#endif

#include "attn_tile.h"

namespace attn {
namespace {

struct Params {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* lse;
  int N, Hq, Hkv, group, q_tiles;
  int head_group;   // causal: heads whose query tiles run interleaved, heaviest first
  float c;          // |scale| * log2(e), or 1 when scale = 0 (Q is then zeroed): always > 0
  uint32_t q_sign;  // 0x80008000 when scale < 0 (Q is negated on load), else 0
  uint32_t q_keep;  // 0 when scale = 0 (every logit is then exactly 0), else all ones
};

template <int D, bool CAUSAL, typename T>
__global__ __launch_bounds__(kThreads, (fwd_wg_per_cu<D, CAUSAL>())) void attn_fwd_kernel(Params p) {
  using C = Cfg<D>;
  // K stages 0/1 and V stages 0/1, each an LDS object of its own.
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE_BYTES];
  const KVStages<D> st{{k0s, k1s}, {v0s, v1s}};

  // Work list position -> (batch*head, query tile), contiguous per XCD;
  // causal: heaviest tiles first across a group of heads.
  const int u = xcd_work_index();
  int bh, qt;
  if (CAUSAL) {
    grouped_order(u, p.q_tiles, gridDim.x / p.q_tiles, p.head_group, bh, qt);
    qt = p.q_tiles - 1 - qt;
  } else {
    bh = u / p.q_tiles;
    qt = u - bh * p.q_tiles;
  }
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
  load_tile<D>(krs, st.k[0], 0, lo, tid);
  load_tile<D>(vrs, st.v[0], 0, lo, tid);
  load_tile<D>(krs, st.k[1], tile_base<D>(1, nt), lo, tid);

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
    w.clear_sums(qb);
  }

  wait_vm_all();
  __syncthreads();

  // Prologue: logits of tile 0 and the first running max.
  STile<D> sa, sb;
  if (w.nt_w > 0) {
    qk_tile<D, T>(st.k[0], w.qf, w.off, sa);
    if (C::BN > N || (CAUSAL && C::BN - 1 > w.qw0)) mask_tile<D, CAUSAL>(sa, 0, N, w.qrow, w.g);
    // Key 0 is visible to every row, so these maxima are finite.
    tile_max<D>(sa, w.c, w.m_run);
  }
  // Iteration 0 refills K stage 0: every wave must be done reading K_0.
  __syncthreads();

  // Without the mask every wave could compute every tile (a wave entirely
  // past the end only computes rows that are never stored); at d = 64 the
  // pipeline is scheduled better when it is told so.
  constexpr bool kUniform = !CAUSAL && D == 64;
  for (int j = 0; j < nt; j += 2) {
    pipeline_step<D, CAUSAL, 0, T, kUniform>(j, nt, st, krs, vrs, lo, tid, w, sa, sb);
    if (j + 1 < nt) pipeline_step<D, CAUSAL, 1, T, kUniform>(j + 1, nt, st, krs, vrs, lo, tid, w, sb, sa);
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m + log2 l).  After the loop's last
  // barrier no copy or read uses the K/V stages any more, so each wave
  // stages its rows for a coalesced store in an LDS region of its own.
  char* region = st.region(wv);
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int row = w.qrow + 32 * qb;
    const int row0 = w.qw0 + 32 * qb;
    const float l_tot = w.total_sum(qb);
    store_rows<D, T>(region, w.oacc[qb], 1.0f / l_tot, p.o + qoff + (size_t)row0 * D, N - row0, lane);
    if (p.lse != nullptr && w.g == 0 && row < N)
      p.lse[((size_t)b * p.Hq + hq) * N + row] = (w.m_run[qb] + __builtin_log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong form: 512 threads = 8 waves, 256 query rows per workgroup (32 per
// wave), 32-key K/V tiles.  Waves w and w + 4 share a SIMD.  The two wave
// groups (waves 0-3 and 4-7) run the same program one phase apart, and every
// phase ends at a workgroup barrier, so that on each SIMD one wave feeds the
// matrix cores while the other only moves operands.  Per key tile j a wave
// runs two phases:
//   matrix phase j: S_{j+1} = K_{j+1} Q^T interleaved with O += P_{j-1} V_{j-1}
//       (the dependent chain of the score product alternates with the four
//       independent chains of the output product, so that no matrix
//       instruction waits for its predecessor's result), while the vector
//       ALUs take the row max of S_j (lazy raise of m) and P_j = exp2(c S_j - m)
//       and add the row sums of P_{j-1};
//   copy phase j: wait for this wave's share of the copies queued two tiles
//       ago, queue K_{j+5} and V_{j+3}, and read the K_{j+2} and V_j operands
//       from LDS into registers for the next matrix phase,
// so every matrix instruction finds both operands in registers and the
// softmax of one tile runs under the matrix work of its neighbours ([CANN-FA]
// "Ascend C implementation" and "key design points": data movement
// overlapped with the matrix unit).  Each group copies half of every tile
// (rows 16 g .. 16 g + 15) with one 16-byte buffer-to-LDS load per thread;
// K and V have four LDS stages each, separate objects so that the compiler
// can tell a read of one stage from a copy in flight into another.
template <int D>
struct PPCfg {
  static constexpr int BM = 256;                   // query rows per workgroup
  static constexpr int BN = 32;                    // keys per K/V tile
  static constexpr int DC = D / 16;                // 16-dim k-steps of Q.K
  static constexpr int DT = D / 32;                // 32-dim row tiles of O^T
  static constexpr int CPR = lds_row_chunks<D>();  // 16-byte chunks per LDS row
  static constexpr int TILE = BN * CPR * 16;       // bytes of one K or V tile
  static constexpr int KAHEAD = 5;                 // K_{j+5} is queued in copy phase j
  static constexpr int VAHEAD = 3;                 // V_{j+3}
  static_assert(CPR == 16 && D == 128, "the ping-pong form is built for head_dim 128");
  static_assert(32 * CPR * 16 == TILE, "one wave's output rows fill one stage");
};

constexpr int kPPThreads = 512;
constexpr int kSchedTrans = 0x400;

__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Waits until at most two of this wave's buffer-to-LDS copies are in flight
// (the two queued in the previous copy phase).
__device__ __forceinline__ void wait_vm_two() { asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); }

template <int D, typename T>
__global__ __launch_bounds__(kPPThreads, 1) void attn_fwd_pp_kernel(Params p) {
  using C = PPCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char k2s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char k3s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v2s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v3s[C::TILE];
  // i is a compile-time constant at every use.
  auto kst = [&](int i) -> char* { return i == 0 ? k0s : i == 1 ? k1s : i == 2 ? k2s : k3s; };
  auto vst = [&](int i) -> char* { return i == 0 ? v0s : i == 1 ? v1s : i == 2 ? v2s : v3s; };

  const int u = xcd_work_index();
  const int bh = u / p.q_tiles, qt = u - bh * p.q_tiles;
  const int b = bh / p.Hq, hq = bh - b * p.Hq, kvh = hq / p.group;
  const int N = p.N;
  const size_t qoff = ((size_t)b * p.Hq + hq) * (size_t)N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + kvh) * (size_t)N * D;
  const int head_bytes = static_cast<int>(static_cast<uint32_t>(N) * (D * 2));
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kvoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kvoff), (short)0, head_bytes, kBufferWord3);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv >> 2;
  const int g = lane >> 5;
  const int qw0 = qt * C::BM + 32 * wv;
  const int qrow = qw0 + (lane & 31);
  const int nt = (N + C::BN - 1) / C::BN;
  const float c = p.c;

  // This thread's share of a tile copy: row 16 grp + t / 16 of the tile,
  // LDS slot t % 16 of that row, which holds source chunk (t % 16) ^ f(row).
  const int t = tid & 255;
  const int crow = 16 * grp + (t >> 4);
  const int cchunk = (swz<D>(crow, t & 15) >> 4) - crow * C::CPR;
  const uint32_t csrc = static_cast<uint32_t>((crow * D + cchunk * 8) * 2);
  const int cdst = (16 * grp * C::CPR + (t & ~63)) * 16;  // wave-uniform
  auto copy = [&](__amdgpu_buffer_rsrc_t rs, char* stage, int tile) {
    const uint32_t base = tile < nt ? static_cast<uint32_t>(tile) * (C::BN * D * 2) : kSkipTile;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + cdst), 16, static_cast<int>(base + csrc), 0,
                                             0, 0);
  };

  Offsets<D> off;
  off.init(lane);
  half8 kr[C::DC];      // K_{j+1} operands (A of S^T = K Q^T)
  half8 vr[2][C::DT];   // V_{j-1}^T operands, per 16-key half
  auto load_k = [&](const char* ks) {
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) kr[dc] = *reinterpret_cast<const half8*>(ks + off.kofs(dc));
  };
  auto load_v = [&](const char* vs) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const int kb = 16 * h * C::CPR * 16;
        const short4v lo = tr_read(vs + off.vofs(0, dt) + kb);
        const short4v hi = tr_read(vs + off.vofs(1, dt) + kb);
        vr[h][dt] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  // Keys past the end of the sequence get logit -inf.
  auto mask_tail = [&](f32x16& s, int kv0) {
    const int lim = N - 1 - kv0 - 4 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 8 * (r >> 2) + (r & 3) <= lim ? s[r] : -INFINITY;
  };
  auto row_max = [&](const f32x16& s) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    return xlane_max(mx) * c;
  };

  copy(krs, kst(0), 0);
  copy(krs, kst(1), 1);
  copy(krs, kst(2), 2);
  copy(vrs, vst(0), 0);

  QFrag<D> qf;
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    u32x4 x = qrow < N ? *reinterpret_cast<const u32x4*>(p.q + qoff + (size_t)qrow * D + 16 * dc + 8 * g)
                       : u32x4{0u, 0u, 0u, 0u};
    x = (x ^ p.q_sign) & p.q_keep;
    qf[0][dc] = __builtin_bit_cast(half8, x);
  }
  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float l_run = 0.f;

  wait_vm_all();
  __syncthreads();
  f32x16 s_cur;  // S_j
  load_k(kst(0));
  s_cur = f32x16{};
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) s_cur = mfma16<T>(kr[dc], qf[0][dc], s_cur);
  float m_run = -INFINITY;  // raised to S_0's row max in matrix phase 0
  load_k(kst(1));
  load_v(vst(0));   // stands in for V_{-1}: multiplied by P_{-1} = 0
  half8 pf[2] = {half8{}, half8{}};  // P_{j-1}
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  phase_barrier();  // every wave is done with K_0's stage
  copy(krs, kst(3), 3);   // the copies of copy phases -2 and -1
  copy(vrs, vst(1), 1);
  copy(krs, kst(0), 4);
  copy(vrs, vst(2), 2);
  if (grp == 1) phase_barrier();  // the second group runs one phase behind

  // Matrix phase and copy phase of tile j; ST = j % 4 (compile-time).
  auto iteration = [&](auto stc, int j) {
    constexpr int ST = decltype(stc)::value;
    // Row max of S_j: raise m lazily (the rescale of O waits for this
    // phase's P_{j-1} V_{j-1} products below).
    float alpha = 1.0f;
    bool raise = false;
    if (j < nt) {
      if ((j + 1) * C::BN > N) mask_tail(s_cur, j * C::BN);
      const float m_tile = row_max(s_cur);
      if (__any(m_tile > m_run + kLazy)) {
        const float m_new = fmaxf(m_run, m_tile);
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run = -inf
        m_run = m_new;
        raise = true;
      }
    }
    l_run += row_sum16<T>(pf);  // P_{j-1}, before the rescale
    f32x16 s_nxt = f32x16{};
    half8 pn[2];
#pragma unroll
    for (int i = 0; i < C::DC; ++i) {
      s_nxt = mfma16<T>(kr[i], qf[0][i], s_nxt);
      oacc[i % C::DT] = mfma16<T>(vr[i / C::DT][i % C::DT], pf[i / C::DT], oacc[i % C::DT]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pn[r >> 3][r & 7] = to_elem<T>(__builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], c, -m_run)));
#pragma unroll
    for (int i = 0; i < C::DC; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVALU, 4, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedTrans, 2, 0);
    }
    if (raise) {
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
    }
    pf[0] = pn[0];
    pf[1] = pn[1];
    s_cur = s_nxt;
    phase_barrier();
    // Copy phase: the copies queued two tiles ago have landed; queue
    // K_{j+5} and V_{j+3}; K_{j+2} and V_j operands into registers.
    wait_vm_two();
    copy(krs, kst((ST + 1) & 3), j + C::KAHEAD);
    copy(vrs, vst((ST + 3) & 3), j + C::VAHEAD);
    load_k(kst((ST + 2) & 3));
    load_v(vst(ST));
    phase_barrier();
  };
  // Tiles 0 .. nt: the last matrix phase only adds P_{nt-1} V_{nt-1}.
  int j = 0;
  for (; j + 3 <= nt; j += 4) {
    iteration(std::integral_constant<int, 0>{}, j);
    iteration(std::integral_constant<int, 1>{}, j + 1);
    iteration(std::integral_constant<int, 2>{}, j + 2);
    iteration(std::integral_constant<int, 3>{}, j + 3);
  }
  if (j <= nt) iteration(std::integral_constant<int, 0>{}, j);
  if (j + 1 <= nt) iteration(std::integral_constant<int, 1>{}, j + 1);
  if (j + 2 <= nt) iteration(std::integral_constant<int, 2>{}, j + 2);
  if (grp == 0) phase_barrier();
  // Every copy (including the skipped ones past the end) and every LDS read
  // is complete before the stages are reused for the output rows.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  phase_barrier();

  char* region = wv == 0 ? k0s : wv == 1 ? k1s : wv == 2 ? k2s : wv == 3 ? k3s
               : wv == 4 ? v0s : wv == 5 ? v1s : wv == 6 ? v2s : v3s;
  const float l_tot = xlane_sum(l_run);
  store_rows<D, T>(region, oacc, 1.0f / l_tot, p.o + qoff + (size_t)qw0 * D, N - qw0, lane);
  if (p.lse != nullptr && g == 0 && qrow < N)
    p.lse[((size_t)b * p.Hq + hq) * N + qrow] = (m_run + __builtin_log2f(l_tot)) * kLn2;
}

// Compile-time switch of the head_dim 128, non-causal forward: 1 = the
// ping-pong kernel above, 0 = the 4-wave pipelined kernel.
#ifndef ATTN_FWD_PP
#define ATTN_FWD_PP 0
#endif

template <int D, bool CAUSAL>
hipError_t launch_t(const LaunchArgs& a, Params p, hipStream_t s) {
#ifdef ATTN_FP16_ONLY
  if (a.bf16) return hipErrorInvalidValue;  // offline tile sweep builds: fp16 only
#endif
  p.q_tiles = (a.N + Cfg<D>::BM - 1) / Cfg<D>::BM;
  const unsigned grid = static_cast<unsigned>(a.B) * a.Hq * p.q_tiles;
  // Each head streams its K/V head (K and V, 16-bit elements) through L2.
  p.head_group = CAUSAL ? causal_head_group(grid, p.q_tiles, static_cast<int64_t>(a.N) * D * 4, a.Hq / a.Hkv) : 1;
  if constexpr (D == 128 && !CAUSAL && ATTN_FWD_PP) {
    p.q_tiles = (a.N + PPCfg<D>::BM - 1) / PPCfg<D>::BM;
    const unsigned pgrid = static_cast<unsigned>(a.B) * a.Hq * p.q_tiles;
#ifndef ATTN_FP16_ONLY
    if (a.bf16)
      hipLaunchKernelGGL((attn_fwd_pp_kernel<D, __bf16>), dim3(pgrid), dim3(kPPThreads), 0, s, p);
    else
#endif
      hipLaunchKernelGGL((attn_fwd_pp_kernel<D, _Float16>), dim3(pgrid), dim3(kPPThreads), 0, s, p);
    return hipGetLastError();
  }
#ifndef ATTN_FP16_ONLY
  if (a.bf16)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, __bf16>), dim3(grid), dim3(kThreads), 0, s, p);
  else
#endif
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, _Float16>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// The entry point's name: launch_forward, or another name when this file is
// compiled again with other tiles (attn_fwd_kernel_d64_one_block.hip).
#ifndef ATTN_FWD_ENTRY
#define ATTN_FWD_ENTRY launch_forward
#endif
int ATTN_FWD_ENTRY(const LaunchArgs& a, void* stream) {
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
  const hipError_t e = with_head_dim(a.d, [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    return a.causal ? launch_t<D, true>(a, p, s) : launch_t<D, false>(a, p, s);
  });
  return static_cast<int>(e);
}

}  // namespace attn
