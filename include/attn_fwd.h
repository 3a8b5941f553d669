/*
 * attn_fwd.h - C ABI of the fused exact-attention forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation ([CANN-FA] section "Where is the bottleneck of standard
 * attention"; [FA-Infer] section 2) is, per batch b and query head h,
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 *     LSE_i = ln sum_{j visible to i} exp(scale * q_i . k_j),
 *
 * computed as one fused kernel in the tiled, online-softmax form the pages
 * describe ([CANN-FA] sections "Tiling on the Ascend NPU" and "Concrete
 * flow"; [FA-Dict] sections "FlashAttention page by page", "Online softmax"
 * and "Fused kernel"): the N x N score matrix never reaches device memory.
 *
 * Pages cited:
 *   [CANN-FA]  www.mooersco.com/news/1200175 - "FlashAttention operator of
 *              the CANN ops-transformer repository: attention acceleration
 *              on the Ascend NPU"
 *   [FA-Dict]  hwcomputing.csdn.net/6a0dbd08662f9a54cb75eb74.html - the
 *              "dictionary, page by page" FlashAttention tutorial
 *   [FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html - why
 *              Transformer inference is slow; FlashAttention on Ascend/CANN
 *
 * Conventions shared by every entry point
 *   - Layout ([CANN-FA] section "Calling FlashAttention from PyTorch" and
 *     [FA-Dict] section "Calling" show (batch, heads, seq, head_dim) fp16
 *     tensors): q and o are [B][Hq][N][d], k and v are [B][Hkv][N][d], all
 *     IEEE binary16, densely packed in that order (row-major, no strides).
 *     lse is [B][Hq][N] IEEE binary32.
 *   - GQA / MQA ([FA-Infer] section 6): Hq must be a multiple of Hkv; query
 *     head h reads key/value head h / (Hq / Hkv) (contiguous groups).
 *   - head_dim ([CANN-FA], the closing note on head_dim): the pages' fused
 *     operator takes d = 64, 128 or 256 and falls back to unfused attention
 *     for other values.  This library runs the same fused kernels for every
 *     multiple of 32 from 32 to 256 (32, 64, 96, 128, 160, 192, 224, 256);
 *     for any other d it returns ATTN_ERR_UNSUPPORTED and launches nothing.
 *   - causal != 0: key j is visible to query i iff j <= i ([CANN-FA] section
 *     "Calling FlashAttention from PyTorch", is_causal).  Queries and keys
 *     have the same length N.
 *   - Memory: every pointer is device memory on the current HIP device,
 *     owned by the caller, which keeps it alive until the work queued on
 *     `stream` has completed.  The library allocates nothing and keeps no
 *     state between calls; calls from several host threads are safe.
 *   - Graphs: the entry points queue kernel launches only (no allocation,
 *     no memset, no copy), so a call can be captured in a HIP graph on
 *     `stream` and replayed; a replay reads the captured buffers' current
 *     contents.
 *   - Asynchrony: attn_fwd only queues work on `stream` (NULL = the default
 *     stream) and returns; it never synchronises.  A device fault surfaces at
 *     the caller's next synchronisation.
 *   - Errors: on any status other than ATTN_OK nothing has been launched and
 *     the outputs are untouched.
 */
#ifndef ATTN_FWD_H_
#define ATTN_FWD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream handle type (hipStream_t is `struct ihipStream_t*`),
 * declared here so that this header does not need the HIP headers. */
struct ihipStream_t;

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* NULL or misaligned pointer, bad size, bad grouping,
                               non-finite scale, overlapping output, size over
                               limits, workspace too small */
  ATTN_ERR_UNSUPPORTED = 2, /* head_dim not a multiple of 32 in [32, 256] */
  ATTN_ERR_DEVICE = 3,      /* the HIP runtime refused the launch */
  ATTN_ERR_SCRATCH = 4      /* attn_bwd_noalloc: the problem needs more than
                               ATTN_BWD_NOALLOC_SCRATCH_BYTES of scratch */
};

/*
 * attn_fwd - fused attention forward.
 *
 *   q      [B][Hq][N][d]  fp16, read only
 *   k, v   [B][Hkv][N][d] fp16, read only
 *   o      [B][Hq][N][d]  fp16, written: every element exactly once
 *   lse    [B][Hq][N]     fp32, written (natural log), or NULL to skip it
 *   B, N   >= 0; B == 0 or N == 0 is an empty problem: ATTN_OK, nothing is
 *          launched and no pointer is touched (they may then be NULL)
 *   Hq, Hkv >= 1 with Hq % Hkv == 0
 *   d      a multiple of 32 from 32 to 256
 *   scale  finite multiplier on q.k (1/sqrt(d) in the pages' usage,
 *          [FA-Dict] sections "Fused kernel" and "Calling"); any finite
 *          value, including 0 and negative values, is accepted
 *   causal 0 or non-zero
 *   stream HIP stream to queue the kernel on (NULL = default stream)
 *
 * Limits: N * d <= 2^30 and B * Hq * ceil(N / 128) < 2^24 (one dispatch of
 * 256-thread workgroups holds fewer than 2^32 work-items).  The output o (and
 * lse) must not overlap q, k, v or each other.  q, k, v and o must be 16-byte
 * aligned and lse 4-byte aligned (ATTN_ERR_INVALID_ARG otherwise).
 * Returns an attn_status value.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
             float scale, int causal, struct ihipStream_t* stream);

/*
 * attn_fwd_bf16 - attn_fwd for bfloat16 q, k, v and o (same arguments,
 * layout, limits and status codes; lse stays fp32).  The pages use fp16
 * ([CANN-FA] section "Performance vs standard attention"); bf16 is the
 * other 16-bit type models are trained in.  P is rounded to bf16 for the
 * P.V product, every sum is fp32, O is rounded to bf16 (to nearest even).
 */
int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                  float scale, int causal, struct ihipStream_t* stream);

/*
 * attn_check_args - the argument validation of attn_fwd, on the host only.
 * Pointers are compared with NULL and with each other's address ranges but
 * never dereferenced; no HIP call is made, so it runs without a GPU.
 * Returns the status attn_fwd would return before launching.
 */
int attn_check_args(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t N, int64_t d, float scale);

/*
 * Decode (KV cache): Nq new queries per query head against Nk cached keys.
 *
 * The computation is the same definition as attn_fwd ([CANN-FA] section
 * "Where is the bottleneck of standard attention"), for queries that are the
 * last Nq positions of an Nk-long sequence: query i sits at position
 * Nk - Nq + i, so with causal != 0 it sees keys 0 .. Nk - Nq + i (with
 * Nq == Nk this is attn_fwd's causal mask).  GQA/MQA ([FA-Infer] section 6)
 * is what makes this path cheap: the G = Hq / Hkv query heads of a key/value
 * head are computed together, so each cached K/V byte is read once.
 *
 *   q      [B][Hq][Nq][d]  fp16, read only
 *   k, v   [B][Hkv][Nk][d] fp16, read only (the cache)
 *   o      [B][Hq][Nq][d]  fp16, written: every element exactly once
 *   lse    [B][Hq][Nq]     fp32 natural log, or NULL
 *   B, Nq  >= 0 (0 is an empty problem: ATTN_OK, nothing touched);
 *          1 <= Nq <= Nk otherwise
 *   Hq, Hkv, d, scale, causal, stream: as for attn_fwd
 *   workspace, workspace_bytes: caller-owned device memory of at least
 *          attn_decode_workspace_size(...) bytes, used for the per-chunk
 *          partial results; its contents on entry do not matter and on
 *          return are unspecified.  It must be 16-byte aligned, must not
 *          overlap any other buffer, and two calls in flight must not share
 *          it.  Pointer alignment as for attn_fwd.
 *
 * One or two kernels are queued on `stream` (the per-chunk pass, then the
 * merge when the keys were split into more than one chunk); the call never
 * synchronises.  Limits: Nk * d <= 2^30 and B * Hq * Nq * d / 32 < 2^24.
 * Returns an attn_status value; on any status other than ATTN_OK nothing
 * has been launched.
 */
int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                int64_t d, float scale, int causal, void* workspace,
                int64_t workspace_bytes, struct ihipStream_t* stream);

/*
 * attn_decode_bf16 - attn_decode for bfloat16 q, k, v and o (same arguments,
 * workspace, limits and status codes; lse and the workspace stay fp32).
 */
int attn_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                     int64_t d, float scale, int causal, void* workspace,
                     int64_t workspace_bytes, struct ihipStream_t* stream);

/*
 * attn_decode_workspace_size - bytes of workspace attn_decode needs for this
 * shape (0 for an empty problem), written to *bytes.  Host only.  Returns
 * ATTN_ERR_INVALID_ARG / ATTN_ERR_UNSUPPORTED for shapes attn_decode would
 * reject, and ATTN_ERR_INVALID_ARG when bytes is NULL.
 */
int attn_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                               int64_t Nk, int64_t d, int64_t* bytes);

/*
 * attn_check_decode_args - the argument validation of attn_decode on the
 * host only (pointers compared, never dereferenced; no HIP call).
 */
int attn_check_decode_args(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, int64_t B,
                           int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                           int64_t d, float scale, const void* workspace,
                           int64_t workspace_bytes);

/*
 * attn_bwd - fused attention backward: the gradients of attn_fwd's O with
 * respect to q, k and v, given the upstream gradient dout of O.
 *
 * The pages name training as a use of the operator ([CANN-FA], opening
 * paragraph) and backpropagation's need to keep gradients ([FA-Dict] section
 * "Standard attention"); the gradients are the chain rule applied to
 * attn_fwd's definition: with P = exp(scale q k^T - lse) (masked entries 0),
 * dv = P^T dout, dP = dout v^T, dS = P o (dP - rowsum(dout o o)),
 * dq = scale dS k, dk = scale dS^T q (summed over the query heads that share
 * a key/value head).  P is recomputed from q, k and lse; nothing N x N is
 * stored.
 *
 *   q, o, dout   [B][Hq][N][d]  fp16, read only (o as attn_fwd wrote it)
 *   k, v         [B][Hkv][N][d] fp16, read only
 *   lse          [B][Hq][N]     fp32, read only: attn_fwd's lse (required)
 *   dq           [B][Hq][N][d]  fp16, written: every element once
 *   dk, dv       [B][Hkv][N][d] fp16, written: every element once
 *   B, Hq, Hkv, N, d, scale, causal, stream: as for attn_fwd (the same
 *          values the forward ran with)
 *   workspace, workspace_bytes: caller-owned device memory of at least
 *          attn_bwd_workspace_size(...) bytes (per-row fp32 terms); contents
 *          on entry do not matter, on return unspecified; must not overlap
 *          any other buffer; two calls in flight must not share it.
 *
 * Two kernels are queued on `stream`; the call never synchronises.  The
 * outputs must not overlap the inputs, each other or the workspace.  Every
 * pointer is 16-byte aligned (lse 4-byte).  Limits as for attn_fwd, and
 * B * Hq * round_up(N, 128) < 2^31.  Returns an attn_status value; on any
 * status other than ATTN_OK nothing has been launched.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
             float scale, int causal, void* workspace, int64_t workspace_bytes,
             struct ihipStream_t* stream);

/*
 * attn_bwd_bf16 - attn_bwd for bfloat16 q, k, v, o, dout and gradients (the
 * output of attn_fwd_bf16); same arguments, workspace, limits and status
 * codes.  P and dS are rounded to bf16 for the products that use them.
 */
int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq, void* dk,
                  void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                  int64_t d, float scale, int causal, void* workspace,
                  int64_t workspace_bytes, struct ihipStream_t* stream);

/*
 * attn_bwd_workspace_size - bytes of workspace attn_bwd needs (0 for an
 * empty problem), written to *bytes.  Host only.  ATTN_ERR_INVALID_ARG for
 * a NULL bytes or invalid sizes, ATTN_ERR_UNSUPPORTED for other head_dims.
 */
int attn_bwd_workspace_size(int64_t B, int64_t Hq, int64_t N, int64_t d,
                            int64_t* bytes);

/*
 * attn_check_bwd_args - the argument validation of attn_bwd on the host
 * only (pointers compared, never dereferenced; no HIP call).
 */
int attn_check_bwd_args(const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        const void* dq, const void* dk, const void* dv,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                        int64_t d, float scale, const void* workspace,
                        int64_t workspace_bytes);

/* Bytes of the fixed scratch of attn_bwd_noalloc (per GPU). */
#define ATTN_BWD_NOALLOC_SCRATCH_BYTES ((int64_t)16 << 20)

/*
 * attn_bwd_noalloc - attn_bwd (fp16) for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight training
 * loops, harnesses that forbid allocation.  The same kernels, with the
 * per-row terms kept in a fixed scratch array inside the library (one per
 * GPU, ATTN_BWD_NOALLOC_SCRATCH_BYTES = 16 MiB, held until the process
 * ends) instead of a caller workspace; the call allocates nothing.
 *
 *   Arguments as for attn_bwd without workspace and workspace_bytes.
 *   Limit: attn_bwd_workspace_size(B, Hq, N, d) <= 16 MiB, i.e.
 *          B * Hq * round_up(N, 128) <= 2^21 rows; larger problems return
 *          ATTN_ERR_SCRATCH and launch nothing.
 *   Every call on one GPU uses that GPU's scratch: two calls in flight at
 *   once on the same GPU (e.g. on two streams) race and give wrong
 *   gradients; calls on one stream, or on different GPUs, do not.  The
 *   scratch needs no clearing (every row term is written before it is
 *   read).  The first call on a device (the current one) looks up the
 *   scratch's device address; ATTN_ERR_DEVICE if that fails.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk,
                     void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                     int64_t d, float scale, int causal,
                     struct ihipStream_t* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(int status);

/* Static version string of the library, e.g. "attn_fwd 0.4.0 gfx950". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H_ */
