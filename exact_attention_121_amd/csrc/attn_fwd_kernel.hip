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
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_f16: A = 32 keys x 16 dims from LDS, B = 16 dims x
//     32 queries from registers.  In the 32x32 fp32 result, lane L holds query
//     L%32 and the 16 keys 8*(r/4) + 4*(L/32) + r%4 (r = 0..15), so each
//     query's row max and row sum are in-lane reductions plus one exchange
//     with lane L^32.
//   * The probabilities stay in registers and are the B operand of
//     O^T += V^T P^T (same instruction).  The reduction index of that product
//     may be permuted freely, so the B operand's eight slots of lane L simply
//     take the lane's own score registers; the A operand must then pair slot
//     j of lane group L/32 with key 8*(j/4) + 4*(L/32) + j%4 (+16 per half).
//     V is stored transposed in LDS with key positions bits 2 and 3 swapped,
//     which turns exactly that key set into 8 consecutive halfs: one 16-byte
//     LDS read per operand.
//   * K/V tiles are double-buffered in LDS: the global loads of tile j+1 are
//     issued before tile j is computed and written to the other buffer after
//     it ([CANN-FA] section "Ascend C implementation", double buffering so
//     that data movement hides behind the matrix unit).
//   * exp is exp2 with scale*log2(e) folded into one fused multiply-add.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 waves of 64 lanes
constexpr int kWaveRows = 32;  // query rows per wave
constexpr int kBM = 128;       // query rows per workgroup
constexpr float kLn2 = 0.69314718055994531f;

template <int D>
struct Cfg {
  static constexpr int BN = (D == 256) ? 32 : 64;  // keys per K/V tile
  static constexpr int NT = BN / 32;               // 32-key sub-tiles of S^T
  static constexpr int DC = D / 16;                // 16-dim k-steps of Q.K
  static constexpr int DT = D / 32;                // 32-dim row tiles of O^T
  static constexpr int KS = D + 8;                 // K row stride in LDS (halfs)
  static constexpr int VS = BN + 8;                // V^T row stride in LDS (halfs)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = BN * D / 8;  // 16-byte chunks per K tile
  static constexpr int K_PER_THREAD = K_CHUNKS / kThreads;
  static constexpr int V_UNITS = BN * D / 32;  // (4 keys x 8 dims) units per V tile
  static_assert(K_CHUNKS % kThreads == 0, "K tile must split evenly");
  static_assert(V_UNITS <= kThreads, "one V unit per thread at most");
};

struct Params {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* lse;
  int N, Hq, Hkv, group, q_tiles;
  float c;          // |scale| * log2(e)
  uint32_t q_sign;  // 0x80008000 when scale < 0 (Q is negated on load), else 0
};

// Key position inside a V^T tile row: bits 2 and 3 of the key index swapped.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D>
__device__ __forceinline__ void load_kv(const _Float16* __restrict__ kb,
                                        const _Float16* __restrict__ vb, int kv0, int N,
                                        int tid, u32x4 (&kr)[Cfg<D>::K_PER_THREAD],
                                        u32x4 (&vr)[4]) {
  using C = Cfg<D>;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < C::K_PER_THREAD; ++i) {
    const int id = tid + i * kThreads;
    const int row = id / CPR, ch = id % CPR;
    const int key = kv0 + row;
    kr[i] = key < N ? *reinterpret_cast<const u32x4*>(kb + (size_t)key * D + ch * 8)
                    : u32x4{0u, 0u, 0u, 0u};
  }
  if (tid < C::V_UNITS) {
    const int k0 = (tid / CPR) * 4, d0 = (tid % CPR) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kv0 + k0 + i;
      vr[i] = key < N ? *reinterpret_cast<const u32x4*>(vb + (size_t)key * D + d0)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_kv(_Float16* __restrict__ ks, _Float16* __restrict__ vts,
                                         int tid, const u32x4 (&kr)[Cfg<D>::K_PER_THREAD],
                                         const u32x4 (&vr)[4]) {
  using C = Cfg<D>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < C::K_PER_THREAD; ++i) {
    const int id = tid + i * kThreads;
    const int row = id / CPR, ch = id % CPR;
    *reinterpret_cast<u32x4*>(ks + row * C::KS + ch * 8) = kr[i];
  }
  if (tid < C::V_UNITS) {
    const int k0 = (tid / CPR) * 4, d0 = (tid % CPR) * 8;
    const int pos = vt_pos(k0);
    // Transpose 4 keys x 8 dims into 8 dims x 4 keys.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(vr[1][j >> 1], vr[0][j >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(vr[3][j >> 1], vr[2][j >> 1], sel);
      *reinterpret_cast<u32x2*>(vts + (d0 + j) * C::VS + pos) = u32x2{lo, hi};
    }
  }
}

// One K/V tile for one wave: S^T = K Q^T, online softmax update, O^T += V^T P^T.
template <int D, bool MASK, bool CAUSAL>
__device__ __forceinline__ void tile_step(const _Float16* __restrict__ ks,
                                          const _Float16* __restrict__ vts,
                                          const half8 (&qf)[Cfg<D>::DC],
                                          f32x16 (&oacc)[Cfg<D>::DT], float& m_run,
                                          float& l_run, float c, int kv0, int N, int qrow,
                                          int lr, int g) {
  using C = Cfg<D>;
  f32x16 s[C::NT];
#pragma unroll
  for (int t = 0; t < C::NT; ++t) s[t] = f32x16{};
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const half8 a = *reinterpret_cast<const half8*>(ks + (32 * t + lr) * C::KS + 16 * dc + 8 * g);
      s[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[dc], s[t], 0, 0, 0);
    }
  }

  if (MASK) {
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = key < N && (!CAUSAL || key <= qrow);
        if (!ok) s[t][r] = -INFINITY;
      }
  }

  float mx = s[0][0];
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // Raw row max -> log2 units; a row with every key of this tile masked keeps m.
  const float m_tile = (MASK && mx == -INFINITY) ? -INFINITY : mx * c;
  const float m_new = fmaxf(m_run, m_tile);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // exp2(-inf) = 0 on the first tile
  m_run = m_new;

  float lsum = 0.f;
  half8 pf[C::NT][2];
#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -m_new));
      if (MASK) p = (s[t][r] == -INFINITY) ? 0.f : p;
      lsum += p;
      pf[t][r >> 3][r & 7] = static_cast<_Float16>(p);
    }
  l_run = l_run * alpha + lsum;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;

#pragma unroll
  for (int t = 0; t < C::NT; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const half8 a =
            *reinterpret_cast<const half8*>(vts + (32 * dt + lr) * C::VS + 32 * t + 16 * h + 8 * g);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[t][h], oacc[dt], 0, 0, 0);
      }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * C::BUF_ELEMS];

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
  const _Float16* __restrict__ kb = p.k + kvoff;
  const _Float16* __restrict__ vb = p.v + kvoff;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;
  const int qw0 = q0 + kWaveRows * w;  // first query row of this wave
  const int qrow = qw0 + lr;           // query row of this lane

  // Q fragments (B operand of S^T): dims 16*dc + 8*g .. +7 of row qrow.
  half8 qf[C::DC];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    u32x4 x = qrow < N ? *reinterpret_cast<const u32x4*>(qb + (size_t)qrow * D + 16 * dc + 8 * g)
                       : u32x4{0u, 0u, 0u, 0u};
    x ^= p.q_sign;
    qf[dc] = __builtin_bit_cast(half8, x);
  }

  const int kv_tiles = (N + C::BN - 1) / C::BN;
  int nt = kv_tiles;
  if (CAUSAL) {
    const int last_q = (q0 + kBM < N ? q0 + kBM : N) - 1;
    const int t_end = last_q / C::BN + 1;
    nt = t_end < kv_tiles ? t_end : kv_tiles;
  }

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  u32x4 kr[C::K_PER_THREAD];
  u32x4 vr[4];
  load_kv<D>(kb, vb, 0, N, tid, kr, vr);
  store_kv<D>(smem, smem + C::K_ELEMS, tid, kr, vr);
  __syncthreads();

  const bool wave_live = qw0 < N;
  for (int j = 0; j < nt; ++j) {
    const int cur = j & 1;
    const int kv0 = j * C::BN;
    if (j + 1 < nt) load_kv<D>(kb, vb, kv0 + C::BN, N, tid, kr, vr);

    const _Float16* ks = smem + cur * C::BUF_ELEMS;
    const _Float16* vts = ks + C::K_ELEMS;
    const bool skip = !wave_live || (CAUSAL && kv0 > qw0 + kWaveRows - 1);
    if (!skip) {
      const bool need_mask = (kv0 + C::BN > N) || (CAUSAL && kv0 + C::BN - 1 > qw0);
      if (need_mask)
        tile_step<D, true, CAUSAL>(ks, vts, qf, oacc, m_run, l_run, p.c, kv0, N, qrow, lr, g);
      else
        tile_step<D, false, CAUSAL>(ks, vts, qf, oacc, m_run, l_run, p.c, kv0, N, qrow, lr, g);
    }

    if (j + 1 < nt) {
      _Float16* nks = smem + (cur ^ 1) * C::BUF_ELEMS;
      store_kv<D>(nks, nks + C::K_ELEMS, tid, kr, vr);
    }
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m + log2 l).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (wave_live && qrow < N) {
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
  p.c = static_cast<float>(c < 0 ? -c : c);
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
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
