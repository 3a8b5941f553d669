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
//     the sequence return zeros), double-buffered: tile j+1 is in flight while
//     tile j is computed ([CANN-FA] section "Ascend C implementation": load
//     block j+1 while block j is computed so that data movement hides behind
//     the matrix unit).  16-byte chunks are XOR-swizzled by row so that the
//     matrix-operand reads hit distinct LDS banks.
//   * exp is exp2 with scale*log2(e) folded into one fused multiply-add; the
//     O rescale is skipped when no row of the wave raised its maximum.
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
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int kThreads = 256;  // 4 waves of 64 lanes
constexpr int kWaveRows = 32;  // query rows per wave
constexpr int kBM = 128;       // query rows per workgroup
constexpr float kLn2 = 0.69314718055994531f;
// Buffer resource word 3 for raw (unformatted, stride 0) buffer access on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

template <int D>
struct Cfg {
  static constexpr int BN = (D == 256) ? 32 : 64;  // keys per K/V tile
  static constexpr int NT = BN / 32;               // 32-key sub-tiles of S^T
  static constexpr int DC = D / 16;                // 16-dim k-steps of Q.K
  static constexpr int DT = D / 32;                // 32-dim row tiles of O^T
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D * 2;    // one K (or V) tile
  static constexpr int LOADS = BN * CPR / kThreads;  // 16-byte loads per thread per tile
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

// Queue the copy of rows kv0 .. kv0+BN-1 of one K or V head into a swizzled
// LDS tile.  Rows at or past N read as zeros (buffer range check).
template <int D>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rsrc, char* tile, int kv0,
                                          int tid) {
  using C = Cfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int p = i * kThreads + tid;  // destination chunk; lanes of a wave are consecutive
    const int row = p / C::CPR;
    // The chunk that belongs at position p % CPR of the swizzled row.
    const int chunk = (swz<D>(row, p % C::CPR) >> 4) - row * C::CPR;
    const int src = ((kv0 + row) * D + chunk * 8) * 2;
    char* dst = tile + (i * kThreads + (tid & ~63)) * 16;  // wave-uniform base
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, src, 0, 0, 0);
  }
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

// One K/V tile for one wave: S^T = K Q^T, online softmax update, O^T += V^T P^T.
template <int D, bool CAUSAL>
__device__ __forceinline__ void tile_step(const char* __restrict__ ks, const char* __restrict__ vs,
                                          const half8 (&qf)[Cfg<D>::DC],
                                          f32x16 (&oacc)[Cfg<D>::DT], float& m_run,
                                          float& l_run, float c, int kv0, int N, int qrow,
                                          int lane, bool mask) {
  using C = Cfg<D>;
  const int lr = lane & 31, g = lane >> 5;
  f32x16 s[C::NT];
#pragma unroll
  for (int t = 0; t < C::NT; ++t) s[t] = f32x16{};
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int r = 32 * t + lr;
      const half8 a = *reinterpret_cast<const half8*>(ks + swz<D>(r, 2 * dc + g));
      s[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[dc], s[t], 0, 0, 0);
    }
  }

  // Masked keys (past the end of the sequence, or after the query when
  // causal) get logit -inf; only tiles crossing the diagonal or the end need it.
  if (mask) {
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = key < N && (!CAUSAL || key <= qrow);
        s[t][r] = ok ? s[t][r] : -INFINITY;
      }
  }

  float mx = s[0][0];
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
  mx = xlane_max(mx);
  // Raw row max -> log2 units (c > 0); a row with every key of this tile
  // masked has mx = -inf and keeps its m.
  const float m_new = fmaxf(m_run, mx * c);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // exp2(-inf) = 0 on the first tile
  m_run = m_new;

  float lsum = 0.f;
  half8 pf[C::NT][2];
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // Masked keys: fma(-inf, c > 0, -m) = -inf and exp2(-inf) = 0.
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -m_new));
      lsum += p;
      pf[t][r >> 3][r & 7] = static_cast<_Float16>(p);
    }
  l_run = l_run * alpha + lsum;
  if (!__all(alpha == 1.0f)) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
  }

  // A operand of O^T += V^T P^T: dims 32*dt + lane%32, keys of slot group g.
  const int m16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * (m16 & 3);  // dim offset inside a 32-dim tile
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key0 = 32 * t + 16 * h + 4 * g + (m16 >> 2);
      const int key1 = key0 + 8;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const int dim = 32 * dt + dsub;
        const short4v lo = tr_read(vs + swz<D>(key0, dim >> 3) + (dim & 7) * 2);
        const short4v hi = tr_read(vs + swz<D>(key1, dim >> 3) + (dim & 7) * 2);
        const half8 a = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[t][h], oacc[dt], 0, 0, 0);
      }
    }
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void compute_tile(const char* ks, const char* vs, const half8 (&qf)[Cfg<D>::DC],
                                             f32x16 (&oacc)[Cfg<D>::DT], float& m_run, float& l_run,
                                             float c, int kv0, int N, int qw0, int qrow, int lane) {
  using C = Cfg<D>;
  if (qw0 >= N) return;                                   // every row of this wave is padding
  if (CAUSAL && kv0 > qw0 + kWaveRows - 1) return;        // tile above the wave's diagonal
  const bool need_mask = (kv0 + C::BN > N) || (CAUSAL && kv0 + C::BN - 1 > qw0);
  tile_step<D, CAUSAL>(ks, vs, qf, oacc, m_run, l_run, c, kv0, N, qrow, lane, need_mask);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void attn_fwd_kernel(Params p) {
  using C = Cfg<D>;
  // Two stages of (K tile, V tile).
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
  const int q0 = qt * kBM;

  const size_t qoff = ((size_t)b * p.Hq + hq) * (size_t)N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + kvh) * (size_t)N * D;
  const _Float16* __restrict__ qb = p.q + qoff;
  const int head_bytes = N * D * 2;  // < 2^32 by the library's size limit
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kvoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kvoff), (short)0, head_bytes, kBufferWord3);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;
  const int qw0 = q0 + kWaveRows * w;  // first query row of this wave
  const int qrow = qw0 + lr;           // query row of this lane

  const int kv_tiles = (N + C::BN - 1) / C::BN;
  int nt = kv_tiles;
  if (CAUSAL) {
    const int last_q = (q0 + kBM < N ? q0 + kBM : N) - 1;
    const int t_end = last_q / C::BN + 1;
    nt = t_end < kv_tiles ? t_end : kv_tiles;
  }

  load_tile<D>(krs, smem, 0, tid);
  load_tile<D>(vrs, smem + C::TILE_BYTES, 0, tid);

  // Q fragments (B operand of S^T): dims 16*dc + 8*g .. +7 of row qrow.
  half8 qf[C::DC];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    u32x4 x = qrow < N ? *reinterpret_cast<const u32x4*>(qb + (size_t)qrow * D + 16 * dc + 8 * g)
                       : u32x4{0u, 0u, 0u, 0u};
    x = (x ^ p.q_sign) & p.q_keep;
    qf[dc] = __builtin_bit_cast(half8, x);
  }

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  wait_vm_all();
  __syncthreads();

  // Stage j&1 holds tile j; tile j+1 is in flight while tile j is computed.
  for (int j = 0; j < nt; ++j) {
    char* cur = smem + (j & 1) * 2 * C::TILE_BYTES;
    char* nxt = smem + ((j + 1) & 1) * 2 * C::TILE_BYTES;
    if (j + 1 < nt) {
      load_tile<D>(krs, nxt, (j + 1) * C::BN, tid);
      load_tile<D>(vrs, nxt + C::TILE_BYTES, (j + 1) * C::BN, tid);
    }
    compute_tile<D, CAUSAL>(cur, cur + C::TILE_BYTES, qf, oacc, m_run, l_run, p.c, j * C::BN, N,
                            qw0, qrow, lane);
    wait_vm_all();
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m + log2 l).
  const float l_tot = xlane_sum(l_run);
  if (qrow < N) {
    const float inv = 1.0f / l_tot;
    _Float16* __restrict__ orow = p.o + qoff + (size_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        half4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(oacc[dt][4 * rq + i] * inv);
        *reinterpret_cast<half4*>(orow + 32 * dt + 8 * rq + 4 * g) = h;
      }
    if (p.lse != nullptr && g == 0)
      p.lse[((size_t)b * p.Hq + hq) * N + qrow] = (m_run + __builtin_log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_t(const LaunchArgs& a, const Params& p, int q_tiles, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(a.B) * a.Hq * q_tiles;
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int launch_forward(const LaunchArgs& a, void* stream) {
  const int q_tiles = (a.N + kBM - 1) / kBM;
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
  p.q_tiles = q_tiles;
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
      e = a.causal ? launch_t<64, true>(a, p, q_tiles, s) : launch_t<64, false>(a, p, q_tiles, s);
      break;
    case 128:
      e = a.causal ? launch_t<128, true>(a, p, q_tiles, s) : launch_t<128, false>(a, p, q_tiles, s);
      break;
    case 256:
      e = a.causal ? launch_t<256, true>(a, p, q_tiles, s) : launch_t<256, false>(a, p, q_tiles, s);
      break;
    default:
      e = hipErrorInvalidValue;
  }
  return static_cast<int>(e);
}

}  // namespace attn
