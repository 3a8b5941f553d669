// C-ABI front end of the fused attention forward: argument validation,
// status strings and the hand-off to the HIP launcher.  Plain C++ with no HIP
// headers, so that the validation runs (and is tested) on machines without a
// GPU.  The declarations and their contract are in include/attn_fwd.h.

#include "../../include/attn_fwd.h"

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "attn_launch.h"

namespace {

constexpr int64_t kLimit31 = int64_t{1} << 31;
// A dispatch holds fewer than 2^32 work-items: with 256 threads per
// workgroup, fewer than 2^24 workgroups.
constexpr int64_t kLimitGroups = int64_t{1} << 24;
constexpr int64_t kLimitHead = int64_t{1} << 30;  // elements per head
constexpr int64_t kRowsPerBlock = 128;  // query rows per workgroup

// [a, a + na) and [b, b + nb) share a byte (empty ranges never overlap).
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const auto pa = reinterpret_cast<uintptr_t>(a);
  const auto pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

// The kernels move Q, K, V, O and the decode workspace in 16-byte vectors
// and the LSE as 4-byte words.
bool misaligned(const void* p, uintptr_t align) { return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0; }

// Head dims the kernels are built for: the multiples of 32 from 32 to 256
// (32-dim output tiles of the matrix instructions).
bool head_dim_supported(int64_t d) { return d >= 32 && d <= 256 && d % 32 == 0; }

bool misaligned_tensors(const void* q, const void* k, const void* v, const void* o, const float* lse) {
  return misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4);
}

}  // namespace

extern "C" int attn_check_args(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t N, int64_t d, float scale) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (!head_dim_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) return ATTN_OK;  // empty problem: nothing to touch
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return ATTN_ERR_INVALID_ARG;
  if (misaligned_tensors(q, k, v, o, lse)) return ATTN_ERR_INVALID_ARG;

  // 32-bit index limits of the kernel: one K/V head spans at most 2^31 bytes
  // (N * d <= 2^30), so a byte offset at or above 2^31 is always outside it.
  if (N > kLimitHead / d) return ATTN_ERR_INVALID_ARG;
  const int64_t q_tiles = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  if (Hq >= kLimit31 || B >= kLimit31 / Hq) return ATTN_ERR_INVALID_ARG;
  if (B * Hq >= kLimitGroups / q_tiles) return ATTN_ERR_INVALID_ARG;  // workgroups < 2^24

  // B * Hq < 2^31 and N * d <= 2^30, so these byte counts fit in int64.
  const int64_t q_bytes = B * Hq * N * d * 2;
  const int64_t kv_bytes = B * Hkv * N * d * 2;
  const int64_t lse_bytes = B * Hq * N * 4;
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, kv_bytes) ||
      overlaps(o, q_bytes, v, kv_bytes))
    return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr &&
      (overlaps(lse, lse_bytes, o, q_bytes) || overlaps(lse, lse_bytes, q, q_bytes) ||
       overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes)))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

namespace {

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
               int64_t Hkv, int64_t N, int64_t d, float scale, int causal, int bf16, struct ihipStream_t* stream) {
  const int st = attn_check_args(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (B == 0 || N == 0) return ATTN_OK;
  attn::LaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = static_cast<int>(B);
  a.Hq = static_cast<int>(Hq);
  a.Hkv = static_cast<int>(Hkv);
  a.N = static_cast<int>(N);
  a.d = static_cast<int>(d);
  a.scale = scale;
  a.causal = causal != 0;
  a.bf16 = bf16;
  const bool one_block = d == 64 && attn::forward_d64_one_block(B, Hq, N, a.causal);
  const int e = one_block ? attn::launch_forward_d64_one_block(a, stream) : attn::launch_forward(a, stream);
  return e == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float scale,
                        int causal, struct ihipStream_t* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 0, stream);
}

extern "C" int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float scale,
                             int causal, struct ihipStream_t* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 1, stream);
}

namespace {

// Shape rules of the decode entry points (no pointer is looked at).
int check_decode_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale) {
  if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (!head_dim_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (Nq > Nk) return ATTN_ERR_INVALID_ARG;  // the queries are the last Nq of Nk positions
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (Nk > kLimitHead / d) return ATTN_ERR_INVALID_ARG;
  // The merge runs d / 32 workgroups per query row.
  if (Hq >= kLimit31 || B >= kLimit31 / Hq || B * Hq >= kLimitGroups / (Nq * (d / 32)))
    return ATTN_ERR_INVALID_ARG;
  const attn::DecodePlan plan = attn::decode_plan(B, Hq, Hkv, Nq, Nk, d);
  if (B * Hkv * plan.row_blocks >= kLimitGroups / plan.splits) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                          int64_t d, int64_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  const int st = check_decode_shape(B, Hq, Hkv, Nq, Nk, d, 1.0f);
  if (st != ATTN_OK) return st;
  *bytes = (B == 0 || Nq == 0) ? 0 : attn::decode_plan(B, Hq, Hkv, Nq, Nk, d).workspace_bytes;
  return ATTN_OK;
}

extern "C" int attn_check_decode_args(const void* q, const void* k, const void* v, const void* o,
                                      const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                                      int64_t Nk, int64_t d, float scale, const void* workspace,
                                      int64_t workspace_bytes) {
  const int st = check_decode_shape(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != ATTN_OK) return st;
  if (B == 0 || Nq == 0) return ATTN_OK;  // empty problem: nothing to touch
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || workspace == nullptr)
    return ATTN_ERR_INVALID_ARG;
  if (misaligned_tensors(q, k, v, o, lse) || misaligned(workspace, 16)) return ATTN_ERR_INVALID_ARG;
  const int64_t need = attn::decode_plan(B, Hq, Hkv, Nq, Nk, d).workspace_bytes;
  if (workspace_bytes < need) return ATTN_ERR_INVALID_ARG;
  const int64_t q_bytes = B * Hq * Nq * d * 2;
  const int64_t kv_bytes = B * Hkv * Nk * d * 2;
  const int64_t lse_bytes = B * Hq * Nq * 4;
  const void* ins[3] = {q, k, v};
  const int64_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(o, q_bytes, ins[i], in_bytes[i])) return ATTN_ERR_INVALID_ARG;
    if (overlaps(workspace, need, ins[i], in_bytes[i])) return ATTN_ERR_INVALID_ARG;
    if (lse != nullptr && overlaps(lse, lse_bytes, ins[i], in_bytes[i])) return ATTN_ERR_INVALID_ARG;
  }
  if (overlaps(workspace, need, o, q_bytes)) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && (overlaps(lse, lse_bytes, o, q_bytes) || overlaps(lse, lse_bytes, workspace, need)))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

namespace {

int decode_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                  int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, void* workspace,
                  int64_t workspace_bytes, int bf16, struct ihipStream_t* stream) {
  const int st = attn_check_decode_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, workspace,
                                        workspace_bytes);
  if (st != ATTN_OK) return st;
  if (B == 0 || Nq == 0) return ATTN_OK;
  attn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.workspace = workspace;
  a.B = static_cast<int>(B);
  a.Hq = static_cast<int>(Hq);
  a.Hkv = static_cast<int>(Hkv);
  a.Nq = static_cast<int>(Nq);
  a.Nk = static_cast<int>(Nk);
  a.d = static_cast<int>(d);
  a.scale = scale;
  a.causal = causal != 0;
  a.bf16 = bf16;
  a.plan = attn::decode_plan(B, Hq, Hkv, Nq, Nk, d);
  return attn::launch_decode(a, stream) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

}  // namespace

extern "C" int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                           int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                           void* workspace, int64_t workspace_bytes, struct ihipStream_t* stream) {
  return decode_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes, 0, stream);
}

extern "C" int attn_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                                void* workspace, int64_t workspace_bytes, struct ihipStream_t* stream) {
  return decode_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes, 1, stream);
}

extern "C" int attn_bwd_workspace_size(int64_t B, int64_t Hq, int64_t N, int64_t d, int64_t* bytes) {
  if (bytes == nullptr || B < 0 || N < 0 || Hq < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (!head_dim_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) {
    *bytes = 0;
    return ATTN_OK;
  }
  if (N > kLimitHead / d || Hq >= kLimit31 || B >= kLimit31 / Hq) return ATTN_ERR_INVALID_ARG;
  *bytes = attn::bwd_workspace_bytes(B, Hq, N);
  return ATTN_OK;
}

namespace {

// The validation of attn_bwd; with own_workspace false (attn_bwd_noalloc) the
// workspace arguments are not looked at: the scratch is the library's own.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              const void* dq, const void* dk, const void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
              float scale, const void* workspace, int64_t workspace_bytes, bool own_workspace) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (!head_dim_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) return ATTN_OK;  // empty problem: nothing to touch
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr || (own_workspace && workspace == nullptr))
    return ATTN_ERR_INVALID_ARG;
  if (misaligned_tensors(q, k, v, o, lse) || misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) ||
      misaligned(dv, 16) || (own_workspace && misaligned(workspace, 16)))
    return ATTN_ERR_INVALID_ARG;
  if (N > kLimitHead / d) return ATTN_ERR_INVALID_ARG;
  if (Hq >= kLimit31 || B >= kLimit31 / Hq) return ATTN_ERR_INVALID_ARG;
  const int64_t q_tiles = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  // Workgroups of the dQ kernel (one per query tile) below 2^24; the dK/dV
  // kernel has at most as many (one per 128 keys of a K/V head, twice that
  // only on grids of fewer than 512).  The workspace rows (padded to whole
  // query tiles) are indexed with 32-bit integers.
  if (B * Hq >= kLimitGroups / q_tiles) return ATTN_ERR_INVALID_ARG;
  const int64_t rows = B * Hq * attn::bwd_padded_rows(N);
  if (rows >= kLimit31) return ATTN_ERR_INVALID_ARG;
  if (own_workspace && workspace_bytes < attn::bwd_workspace_bytes(B, Hq, N)) return ATTN_ERR_INVALID_ARG;
  const int64_t q_bytes = B * Hq * N * d * 2;
  const int64_t kv_bytes = B * Hkv * N * d * 2;
  const int64_t lse_bytes = B * Hq * N * 4;
  const int64_t ws_bytes = own_workspace ? attn::bwd_workspace_bytes(B, Hq, N) : 0;
  const void* ins[6] = {q, k, v, o, lse, dout};
  const int64_t in_bytes[6] = {q_bytes, kv_bytes, kv_bytes, q_bytes, lse_bytes, q_bytes};
  const void* outs[4] = {dq, dk, dv, own_workspace ? workspace : nullptr};
  const int64_t out_bytes[4] = {q_bytes, kv_bytes, kv_bytes, ws_bytes};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return ATTN_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_check_bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                   const void* dout, const void* dq, const void* dk, const void* dv, int64_t B,
                                   int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float scale,
                                   const void* workspace, int64_t workspace_bytes) {
  return check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, workspace, workspace_bytes, true);
}

namespace {

// own_workspace false: attn_bwd_noalloc (the library's fixed scratch).
int bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float scale,
               int causal, void* workspace, int64_t workspace_bytes, int bf16, struct ihipStream_t* stream,
               bool own_workspace = true) {
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, workspace, workspace_bytes,
                           own_workspace);
  if (st != ATTN_OK) return st;
  if (B == 0 || N == 0) return ATTN_OK;
  if (!own_workspace && attn::bwd_workspace_bytes(B, Hq, N) > attn::kBwdNoallocScratchBytes) return ATTN_ERR_SCRATCH;
  attn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.workspace = workspace;
  a.B = static_cast<int>(B);
  a.Hq = static_cast<int>(Hq);
  a.Hkv = static_cast<int>(Hkv);
  a.N = static_cast<int>(N);
  a.d = static_cast<int>(d);
  a.scale = scale;
  a.causal = causal != 0;
  a.bf16 = bf16;
  const int e = own_workspace ? attn::launch_backward(a, stream) : attn::launch_backward_noalloc(a, stream);
  return e == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                        int64_t N, int64_t d, float scale, int causal, void* workspace, int64_t workspace_bytes,
                        struct ihipStream_t* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, workspace, workspace_bytes,
                    0, stream);
}

extern "C" int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                             int64_t N, int64_t d, float scale, int causal, void* workspace,
                             int64_t workspace_bytes, struct ihipStream_t* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, workspace, workspace_bytes,
                    1, stream);
}

static_assert(attn::kBwdNoallocScratchBytes == ATTN_BWD_NOALLOC_SCRATCH_BYTES, "scratch size mismatch");

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                                int64_t N, int64_t d, float scale, int causal, struct ihipStream_t* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, nullptr, 0, 0, stream,
                    false);
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK:
      return "ok";
    case ATTN_ERR_INVALID_ARG:
      return "invalid argument (null pointer, size, head grouping, scale, overlap or limit)";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported head_dim (must be a multiple of 32 from 32 to 256)";
    case ATTN_ERR_DEVICE:
      return "the HIP runtime refused the kernel launch";
    case ATTN_ERR_SCRATCH:
      return "problem too large for the fixed scratch of attn_bwd_noalloc (B * Hq * round_up(N, 128) > 2^21)";
    default:
      return "unknown status";
  }
}

extern "C" const char* attn_version(void) { return "attn_fwd 0.4.0 gfx950"; }
