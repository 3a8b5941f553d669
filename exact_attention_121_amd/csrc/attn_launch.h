// Internal interface between the C-ABI front end (attn_api.cpp, plain C++)
// and the HIP kernels (attn_fwd_kernel.hip).  Not installed, not public.
#ifndef ATTN_LAUNCH_H_
#define ATTN_LAUNCH_H_

#include <stdint.h>

namespace attn {

// Arguments after validation: every size fits the kernel's 32-bit index math
// (N * d <= 2^30, B * Hq * ceil(N / 128) < 2^31) and d is a multiple of 32
// from 32 to 256.
struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, N, d;
  float scale;
  int causal;
  int bf16;    // element type of q, k, v, o: 0 = fp16, 1 = bf16
};

// Queues the fused forward kernel on `stream` (a hipStream_t).  Returns the
// HIP runtime's status of the launch (0 = hipSuccess).
int launch_forward(const LaunchArgs& a, void* stream);

// The same forward, head_dim 64 only, built with one 32-row query block per
// wave and 64-key tiles (launch_forward's head_dim 64 kernel takes two
// blocks per wave and 32-key tiles).
int launch_forward_d64_one_block(const LaunchArgs& a, void* stream);

// Tile choice at head_dim 64, from the offline tile sweep on MI355X: the
// one-block kernel for causal problems whose grid of two-block (256-row)
// workgroups is below 2048 (fewer than four rounds of 512 co-resident
// workgroups: the heaviest-first causal order then leaves the CUs unevenly
// loaded at the end; one-block workgroups are twice as many), the two-block
// kernel otherwise (it reads each K/V operand once for 64 query rows).
constexpr int64_t kD64TwoBlockMinGrid = 2048;
inline bool forward_d64_one_block(int64_t B, int64_t Hq, int64_t N, int causal) {
  return causal && B * Hq * ((N + 255) / 256) < kD64TwoBlockMinGrid;
}

// Decode (KV cache) work plan: Nq new queries per query head against Nk
// cached keys.  The G = Hq / Hkv query heads of a key/value head are packed
// into rows r = g * Nq + i (row blocks of kDecodeRows); the keys are split
// into `splits` chunks of `chunk_tiles` key tiles, each chunk handled by one
// workgroup that writes a partial O and LSE to the workspace; a second
// kernel merges the partials.  With one split the workgroups write O and LSE
// themselves and the merge is not launched.  Shared by the validation (workspace size) and
// the launcher so both see the same plan.
constexpr int64_t kDecodeRows = 128;  // packed rows per workgroup

// Causal work order of the forward and backward kernels: how many heads
// interleave their tiles heaviest first (grouped_order in attn_tile.h).
// `grid` workgroups, `units` of them per head, each head streaming `bytes`
// of operands through L2, `share` consecutive heads streaming the same
// bytes (query heads of one K/V head).  A group never straddles two XCDs'
// ranges of work (the ranges must hold whole heads, else 1), and the
// distinct bytes it streams fit kHeadGroupBytes of L2 (at least one head's,
// however large).  Measured on gfx950 for the forward: 8 heads of the spiky
// causal prefill (1 MB of K/V each) run 8 % faster than one at a time, 4
// query heads of one 8 MB GQA K/V head 3 %, while groups that straddle XCDs
// or stream 16 MB lose 20-30 %.
constexpr int64_t kHeadGroupBytes = 8 << 20;

inline int causal_head_group(int64_t grid, int64_t units, int64_t bytes, int64_t share) {
  if (units <= 0 || grid % 8 != 0 || (grid / 8) % units != 0) return 1;
  const int64_t per_xcd = grid / 8 / units;  // whole heads per XCD
  int64_t fit = bytes > 0 ? kHeadGroupBytes / bytes : per_xcd;
  if (fit < 1) fit = 1;
  const int64_t cap = fit * share;
  int64_t g = 1;
  for (int64_t c = 1; c <= per_xcd && c <= cap; ++c)
    if (per_xcd % c == 0) g = c;
  return static_cast<int>(g);
}

// Workgroups per CU of the forward and decode kernels' default build: two
// (each SIMD interleaves two waves) wherever the registers of a 32-row query
// block hold Q, the output accumulators and two score tiles without
// spilling, i.e. up to d = 224; one at d = 256.
constexpr int64_t default_wg_per_cu(int64_t d) { return d <= 224 ? 2 : 1; }

// Workgroups the chip holds at once (256 CUs times the workgroups per CU):
// the split count aims at one full round of them.
constexpr int64_t decode_target_groups(int64_t d) { return 256 * default_wg_per_cu(d); }

// Workgroups per CU of the decode kernel, chosen at launch: the default
// build's count, except that at d = 256 a grid of at least two workgroups
// per CU runs a second instance compiled for two (it spills 72 bytes per
// lane and still streams a batch of long caches 7 % faster; on a grid of one
// workgroup per CU the spilling instance is 18 % slower).
constexpr int64_t decode_wg_per_cu(int64_t d, int64_t grid) {
  return d == 256 && grid >= 512 ? 2 : default_wg_per_cu(d);
}

struct DecodePlan {
  int64_t row_blocks, kv_tiles, splits, chunk_tiles;
  int64_t workspace_bytes;  // partial O (fp32) and LSE (fp32) of every split
};

// Keys per K/V tile of the kernels' default build, per head_dim: 64 up to
// d = 128 (two workgroups per CU), 32 above (one workgroup per CU; the
// output accumulators take the other half of the register file).
constexpr int64_t default_key_tile(int64_t d) { return d > 128 ? 32 : 64; }

constexpr int64_t decode_key_tile(int64_t d) { return default_key_tile(d); }

inline DecodePlan decode_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d) {
  DecodePlan p;
  const int64_t rows = (Hq / Hkv) * Nq;
  p.row_blocks = (rows + kDecodeRows - 1) / kDecodeRows;
  const int64_t bn = decode_key_tile(d);
  p.kv_tiles = (Nk + bn - 1) / bn;
  const int64_t groups = B * Hkv * p.row_blocks;
  const int64_t target = decode_target_groups(d);
  int64_t s = (target + groups - 1) / groups;
  if (s > p.kv_tiles) s = p.kv_tiles;
  if (s < 1) s = 1;
  p.chunk_tiles = (p.kv_tiles + s - 1) / s;
  p.splits = (p.kv_tiles + p.chunk_tiles - 1) / p.chunk_tiles;  // no empty chunk
  p.workspace_bytes = groups * p.splits * kDecodeRows * (d + 1) * 4;
  return p;
}

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  void* workspace;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int bf16;    // element type of q, k, v, o: 0 = fp16, 1 = bf16
  DecodePlan plan;
};

// Queues the split kernel and the merge kernel on `stream`.
int launch_decode(const DecodeArgs& a, void* stream);

// Backward: keys per dK/dV workgroup (32 per wave) and the workspace rows
// per (batch, query head): N rounded up to whole 128-row query tiles.
constexpr int64_t kBwdKeys = 128;
inline int64_t bwd_padded_rows(int64_t N) { return (N + 127) / 128 * 128; }
// Workspace: LSE in log2 units and Delta = dO . O, fp32, per padded row.
inline int64_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t N) {
  return 2 * B * Hq * bwd_padded_rows(N) * 4;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;
  int B, Hq, Hkv, N, d;
  float scale;
  int causal;
  int bf16;    // element type of q, k, v, o, dout and the gradients: 0 = fp16, 1 = bf16
};

// Queues the two backward kernels on `stream`: dQ (which also writes the
// per-row LSE and Delta terms to the workspace), then dK/dV.
int launch_backward(const BwdArgs& a, void* stream);

// The allocation-free backward: a.workspace is ignored and replaced by the
// library's fixed scratch array on the current device (kBwdNoallocScratchBytes;
// the caller has checked bwd_workspace_bytes against it).  Returns the HIP
// status of the address lookup or of the launches.
constexpr int64_t kBwdNoallocScratchBytes = int64_t{16} << 20;
int launch_backward_noalloc(const BwdArgs& a, void* stream);

}  // namespace attn

#endif  // ATTN_LAUNCH_H_
