// Internal interface between the C-ABI front end (attn_api.cpp, plain C++)
// and the HIP kernels (attn_fwd_kernel.hip).  Not installed, not public.
#ifndef ATTN_LAUNCH_H_
#define ATTN_LAUNCH_H_

#include <stdint.h>

namespace attn {

// Arguments after validation: every size fits the kernel's 32-bit index math
// (N * d <= 2^30, B * Hq * ceil(N / 128) < 2^31) and d is 64, 128 or 256.
struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, N, d;
  float scale;
  int causal;
};

// Queues the fused forward kernel on `stream` (a hipStream_t).  Returns the
// HIP runtime's status of the launch (0 = hipSuccess).
int launch_forward(const LaunchArgs& a, void* stream);

}  // namespace attn

#endif  // ATTN_LAUNCH_H_
