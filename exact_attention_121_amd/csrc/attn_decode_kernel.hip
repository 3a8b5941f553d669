// Decode (KV cache) kernels for gfx950: Nq new queries against Nk cached
// keys, the key sequence split into chunks whose partial results a second
// kernel merges.  The per-chunk kernel runs the forward kernel's software
// pipeline (attn_tile.h) over its chunk.
//
// Pages cited:
//   [CANN-FA]  www.mooersco.com/news/1200175
//   [FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html

#include "attn_tile.h"

namespace attn {
namespace {

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

template <int D, bool CAUSAL, typename T, int WGS>
__global__ __launch_bounds__(kThreads, WGS) void attn_decode_split_kernel(DecParams p) {
  using C = Cfg<D>;
  static_assert(C::QB == 1 && C::BM == kDecodeRows, "decode packs 128 rows per workgroup, 32 per wave");
  // K stages 0/1 then V stages 0/1 in one array.  (As separate objects,
  // which spares the forward its waits for copies in flight before the V
  // operand reads, the decode steps measured 0.4 % faster to 1.4 % slower.)
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES];
  const KVStages<D> st{{smem, smem + C::TILE_BYTES}, {smem + 2 * C::TILE_BYTES, smem + 3 * C::TILE_BYTES}};

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
  load_tile<D>(krs, st.k[0], tile_base<D>(t0, t1), lo, tid);
  load_tile<D>(vrs, st.v[0], tile_base<D>(t0, t1), lo, tid);
  load_tile<D>(krs, st.k[1], tile_base<D>(t0 + 1, t1), lo, tid);

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
  w.clear_sums(0);

  wait_vm_all();
  __syncthreads();

  STile<D> sa, sb;
  if (w.nt_w > t0) {
    const int kv0 = t0 * C::BN;
    qk_tile<D, T>(st.k[0], w.qf, w.off, sa);
    if (kv0 + C::BN > Nk || (CAUSAL && kv0 + C::BN - 1 > w.qw0)) mask_tile<D, CAUSAL>(sa, kv0, Nk, w.qrow, w.g);
    tile_max<D>(sa, w.c, w.m_run);
    // A row that sees no key of this chunk (causal: the chunk starts after
    // its last key; then it sees none of the later tiles either) keeps a
    // finite reference so that its probabilities are exp2(-inf) = 0.
    if (w.m_run[0] == -INFINITY) w.m_run[0] = 0.f;
  }
  __syncthreads();

  for (int j = t0; j < t1; j += 2) {
    pipeline_step<D, CAUSAL, 0, T>(j, t1, st, krs, vrs, lo, tid, w, sa, sb);
    if (j + 1 < t1) pipeline_step<D, CAUSAL, 1, T>(j + 1, t1, st, krs, vrs, lo, tid, w, sb, sa);
  }

  // Partial result of this chunk for the rows that exist: O_s = O^T / l_s
  // (0 when the row saw no key) and LSE_s = m + log2 l_s (-inf when it saw
  // none).
  const float l_tot = w.total_sum(0);
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
        for (int i = 0; i < 4; ++i) h[i] = to_elem<T>(w.oacc[0][dt][4 * rq + i] * inv1);
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
template <int D, int DS, typename T>
__global__ __launch_bounds__(kMergeThreads) void attn_decode_merge_kernel(MergeParams p) {
  constexpr int CH = DS / 4;                 // float4 chunks of a slice
  constexpr int PAR = kMergeThreads / CH;    // splits read at once
  constexpr int SLICES = D / DS;
  static_assert(kMergeThreads % CH == 0 && D % DS == 0, "the splits must cover the workgroup evenly");
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
    h[0] = to_elem<T>(o.x * inv);
    h[1] = to_elem<T>(o.y * inv);
    h[2] = to_elem<T>(o.z * inv);
    h[3] = to_elem<T>(o.w * inv);
    *reinterpret_cast<half4*>(p.o + (size_t)rowid * D + slice * DS + 4 * tid) = h;
    if (p.lse != nullptr && slice == 0 && tid == 0) p.lse[rowid] = (M + __builtin_log2f(L)) * kLn2;
  }
}

template <int D, bool CAUSAL, typename T>
hipError_t launch_decode_t(const DecodeArgs& a, const DecParams& dp, const MergeParams& mp, hipStream_t s) {
  static_assert(Cfg<D>::BN == decode_key_tile(D), "the decode plan and the kernel must use the same key tile");
  const unsigned groups = static_cast<unsigned>(a.B) * a.Hkv * static_cast<unsigned>(a.plan.row_blocks);
  const unsigned grid = groups * static_cast<unsigned>(a.plan.splits);
  constexpr int kWide = D == 256 ? 2 : static_cast<int>(default_wg_per_cu(D));
  if (decode_wg_per_cu(D, grid) == kWide)
    hipLaunchKernelGGL((attn_decode_split_kernel<D, CAUSAL, T, kWide>), dim3(grid), dim3(kThreads), 0, s, dp);
  else
    hipLaunchKernelGGL((attn_decode_split_kernel<D, CAUSAL, T, static_cast<int>(default_wg_per_cu(D))>), dim3(grid),
                       dim3(kThreads), 0, s, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.plan.splits == 1) return e;
  const unsigned rows = static_cast<unsigned>(a.B) * a.Hq * a.Nq;
  // Whole rows need kMergeThreads to split evenly into D / 4 lanes per split
  // (head_dims 32, 64, 128, 256); other head_dims always take 32-dim slices.
  constexpr bool kWholeRows = kMergeThreads % (D / 4) == 0;
  if (kWholeRows && a.plan.splits <= kMergeFewSplits)
    hipLaunchKernelGGL((attn_decode_merge_kernel<D, kWholeRows ? D : kMergeSliceDims, T>), dim3(rows),
                       dim3(kMergeThreads), 0, s, mp);
  else
    hipLaunchKernelGGL((attn_decode_merge_kernel<D, kMergeSliceDims, T>), dim3(rows * (D / kMergeSliceDims)),
                       dim3(kMergeThreads), 0, s, mp);
  return hipGetLastError();
}

}  // namespace

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
  const hipError_t e = with_head_dim(a.d, [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    if (a.bf16)
      return a.causal ? launch_decode_t<D, true, __bf16>(a, dp, mp, s) : launch_decode_t<D, false, __bf16>(a, dp, mp, s);
    return a.causal ? launch_decode_t<D, true, _Float16>(a, dp, mp, s)
                    : launch_decode_t<D, false, _Float16>(a, dp, mp, s);
  });
  return static_cast<int>(e);
}

}  // namespace attn
