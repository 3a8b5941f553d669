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
constexpr int64_t kLimitHead = int64_t{1} << 30;  // elements per head
constexpr int64_t kRowsPerBlock = 128;  // query rows per workgroup

// [a, a + na) and [b, b + nb) share a byte (empty ranges never overlap).
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const auto pa = reinterpret_cast<uintptr_t>(a);
  const auto pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

}  // namespace

extern "C" int attn_check_args(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t N, int64_t d, float scale) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) return ATTN_OK;  // empty problem: nothing to touch
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return ATTN_ERR_INVALID_ARG;

  // 32-bit index limits of the kernel: one K/V head spans at most 2^31 bytes
  // (N * d <= 2^30), so a byte offset at or above 2^31 is always outside it.
  if (N > kLimitHead / d) return ATTN_ERR_INVALID_ARG;
  const int64_t q_tiles = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  if (Hq >= kLimit31 || B >= kLimit31 / Hq) return ATTN_ERR_INVALID_ARG;
  if (B * Hq >= kLimit31 / q_tiles) return ATTN_ERR_INVALID_ARG;  // grid < 2^31

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

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float scale,
                        int causal, struct ihipStream_t* stream) {
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
  return attn::launch_forward(a, stream) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK:
      return "ok";
    case ATTN_ERR_INVALID_ARG:
      return "invalid argument (null pointer, size, head grouping, scale, overlap or limit)";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported head_dim (must be 64, 128 or 256)";
    case ATTN_ERR_DEVICE:
      return "the HIP runtime refused the kernel launch";
    default:
      return "unknown status";
  }
}

extern "C" const char* attn_version(void) { return "attn_fwd 0.1.0 gfx950"; }
