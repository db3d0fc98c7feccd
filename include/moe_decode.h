/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) single-token routed-expert MoE
 * decode layer.
 *
 * The layer, for each of M tokens x[m, :] (hidden size H):
 *   1. router GEMV     logits[m, e] = sum_h Wr[e, h] x[m, h]                  (E experts)
 *   2. top-K + softmax expert_ids[m, :] = the K largest logits, largest first,
 *                      equal logits -> lower expert id first;
 *                      weights = softmax over all E taken at those ids, divided
 *                      by their sum when renormalize != 0
 *   3. W13 GEMV + SiLU activated[m, k, j] = silu(g) * u with
 *                      g = sum_h W13[e, j, h] x[m, h], u = sum_h W13[e, I + j, h] x[m, h],
 *                      e = expert_ids[m, k], silu(g) = g / (1 + exp(-g))
 *   4. W2 GEMV + combine r[m, h] = sum_k weights[m, k] sum_j W2[e, h, j] activated[m, k, j]
 *   5. shared expert   s[m, h] = the same gate/up -> SiLU*mul -> down chain with
 *                      the shared expert's weights, added with weight 1:
 *                      y[m, h] = fp16(r[m, h] + s[m, h])   (one rounding)
 *
 * Where the pages define it:
 *   "如何在天垓 BI-V100 上优化大模型推理：一份工作日志" (BI-V100 inference
 *   worklog): part 3 -- the MoE fallback gathers the selected experts' weights
 *   with index_select and re-reads them; the direct_routed method indexes the
 *   expert tensor by expert id inside the GEMV instead (steps 3 and 4);
 *   part 10 -- the W13 kernel maps input(1, H) x W13[expert_ids[k], row, :] to
 *   gate_up(K, 2I); the W2 kernel maps activated(K, I) x W2[expert_ids[k], h, :]
 *   to expert_out(H) with the weighted sum; part 8 -- the routing step is a
 *   top-k and a softmax; part 2 -- the shared expert is gate_up, SiluAndMul and
 *   down.  "decode analysis report 2026-07-14", profiling section: the MoE
 *   block is gate, routing top-k, routed experts and shared expert.
 *
 * Conventions for every entry point:
 *   - fp16 tensors are IEEE binary16, row-major, contiguous, passed as void*.
 *   - All tensor pointers are DEVICE pointers of the current HIP device; the
 *     caller owns every buffer (including the workspace) and keeps it alive
 *     until the work queued on `stream` has finished.  The library keeps no
 *     pointer after a call returns and holds no mutable global state.
 *   - Every call only enqueues kernels on `stream`: it never allocates, never
 *     synchronises and never reads device memory on the host, so it may be
 *     recorded into a hipGraph by stream capture.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and a negative moe_status is returned.
 *   - Device-data preconditions are NOT checked (no device reads on the host):
 *     expert ids must lie in [0, E) and be distinct within a token; all values
 *     must be finite.  Violating them is undefined behaviour.
 *   - M = 0 is a valid empty call: nothing is enqueued, MOE_OK is returned.
 *
 * Supported sizes (MOE_ERR_SHAPE otherwise):
 *   0 <= M <= 8;  H a multiple of 512, 512 <= H <= 4096 (H > 2048 needs M <= 4);
 *   1 <= E <= 1024;  1 <= K <= min(E, 16);
 *   I and Is multiples of 64, 64 <= I, Is <= 2048.
 * The kernels reduce a down-projection row of width n (I, or Is) in a lane
 * mapping chosen by n alone: LPR lanes per row, CPL 16-byte chunks per lane,
 * n = 8*LPR*CPL exactly where n/8 = LPR*CPL for some LPR in {8, 16, 32, 64}
 * and CPL <= 4 (for example I = 768: 32 lanes x 3 chunks); any other width
 * takes 64 lanes with the chunks past the row's end weighted zero.
 * Alignment (MOE_ERR_ALIGN otherwise): fp16 tensors 16 bytes, fp32/int32
 * arrays 4 bytes, workspace 256 bytes.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5
#define MOE_MAX_TOKENS 8
#define MOE_MAX_TOPK 16
#define MOE_MAX_EXPERTS 1024

typedef int moe_status;
#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)       /* a size is outside the supported set */
#define MOE_ERR_ALIGN (-3)       /* a pointer is not aligned as required */
#define MOE_ERR_WORKSPACE (-4)   /* ws_bytes < moe_workspace_bytes(...) */
#define MOE_ERR_HIP (-5)         /* a kernel launch failed (hipGetLastError) */
#define MOE_ERR_SCRATCH (-6)     /* sizes beyond moe_layer_decode_noalloc's static buffer */

/* ABI version of the loaded library (MOE_ABI_VERSION it was built with). */
int moe_abi_version(void);

/* Identity of the sources the library was built from: the hex SHA-256 over
 * the names and contents of its source and header files (static string,
 * never NULL; "unversioned" for a build that did not set it).  Loaders compare
 * it with the sources at hand to refuse an out-of-date binary. */
const char *moe_build_id(void);

/* Static English description of a status code; never NULL. */
const char *moe_status_str(moe_status status);

/* Bytes of device workspace `ws` that shared_expert, moe_decode_fused and
 * moe_layer_decode need for these sizes (one buffer of this size serves every
 * call issued on the same stream).  Returns 0 for unsupported sizes.
 *
 * The first 8192 bytes of a workspace are a state block that the
 * single-launch layer (moe_dbg_layer_stage stage 5) keeps between calls: one call counter
 * per workgroup and its hand-off flags (no atomics are used; a flag is current
 * when it holds the call count of this call).  It must be zero before the
 * first call with a workspace -- allocate it zero-filled or call
 * moe_workspace_init once -- and is then left to the library.  Word 1024 of the
 * block counts the waits that ran out and computed the awaited data
 * themselves (0 in normal operation; the results are the same either way).
 * The other entry points use the workspace past the state block as scratch. */
size_t moe_workspace_bytes(int M, int H, int E, int I, int K, int Is);

/* Zeroes the state block of `ws` (ws_bytes >= 8192, 256-byte aligned) with a
 * kernel on `stream`.  MOE_ERR_NULL / MOE_ERR_ALIGN / MOE_ERR_WORKSPACE. */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Steps 1-2: router GEMV, top-K selection and routing weights.
 *   x           [M, H]  fp16   token activations
 *   w_router    [E, H]  fp16   router weight
 *   renormalize 0: weights are the full softmax at the selected ids;
 *               else: divided by their sum (the weights then sum to 1)
 *   topk_ids    [M, K]  int32  out: selected expert ids, largest logit first,
 *                              equal logits -> lower id first
 *   topk_w      [M, K]  fp32   out: routing weights in the same order
 *   logits      [M, E]  fp32   out: router logits (needed by the selection;
 *                              also returned for diagnostics)
 * Arithmetic: fp16 products accumulated in fp32; softmax in fp32. */
moe_status moe_route(const void *x, const void *w_router, int M, int H, int E, int K,
                     int renormalize, int32_t *topk_ids, float *topk_w, float *logits,
                     hipStream_t stream);

/* Step 5 on its own: the shared expert (no routing, weight 1).
 *   x          [M, H]    fp16
 *   w_gate_up  [2Is, H]  fp16  rows [0, Is) gate, rows [Is, 2Is) up
 *   w_down     [H, Is]   fp16
 *   s_out      [M, H]    fp32  out: shared-expert output, not rounded to fp16
 *   ws         device workspace of at least moe_workspace_bytes(M, H, 1, 64, 1, Is)
 *              bytes (any of the call's sizes work; only Is matters here)
 * Arithmetic: fp32 accumulation; the SiLU*mul activation is kept in fp32. */
moe_status shared_expert(const void *x, const void *w_gate_up, const void *w_down, int M, int H,
                         int Is, float *s_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Steps 3-5 fused: expert-indexed W13 GEMV with SiLU*mul in its epilogue, then
 * the W2 GEMV with the weighted combine, the optional shared-expert add and
 * the single fp16 rounding.  The expert tensors are read in place at
 * W13 + expert_id * (2I*H) and W2 + expert_id * (H*I): no gathered copy.
 * With M > 1 every distinct selected expert's rows are read once for all the
 * tokens that route to it.
 *   x          [M, H]      fp16
 *   w13        [E, 2I, H]  fp16  per expert: rows [0, I) gate, rows [I, 2I) up
 *   w2         [E, H, I]   fp16
 *   topk_ids   [M, K]      int32 (from moe_route or the caller)
 *   topk_w     [M, K]      fp32
 *   shared_in  [M, H]      fp32 or NULL: added to the routed sum before rounding
 *   y          [M, H]      fp16  out
 *   ws         device workspace, >= moe_workspace_bytes(M, H, E, I, K, 0) bytes
 * Summation order is fixed (no atomics): per token, experts in routing order
 * (for M > 1: in order of first appearance scanning topk_ids row by row), the
 * shared term last; results are bitwise reproducible run to run. */
moe_status moe_decode_fused(const void *x, const void *w13, const void *w2,
                            const int32_t *topk_ids, const float *topk_w, const float *shared_in,
                            int M, int H, int E, int I, int K, void *y, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* Steps 1-5, the whole layer, in as few launches as the sizes allow.
 * Results equal the three-call sequence shared_expert, moe_route,
 * moe_decode_fused bit for bit (routing outputs and y), whichever way it runs.
 *
 * For M = 1 (K*I <= 16384) it is three launches: the router rows; the
 * routed gate/up rows (each workgroup selecting the experts from the logits
 * itself); the routed down rows with the weighted combine.  A shared expert as
 * wide as a routed one (Is == I) has its gate/up rows in the second launch
 * and its down rows in the third; any other width has its gate/up rows in the
 * first launch and its down rows in the second.  For
 * M = 2..8: the router and shared gate/up rows; the distinct experts' gate/up
 * rows with the shared down rows; the down rows with the combine -- three
 * launches for M <= 4, where the workgroups of the second launch select
 * themselves (those of token 0's experts with only as many top-k rounds as
 * they need, the others every token's selection and the grouping of the
 * distinct experts; token 0's workgroups also compute the shared down rows,
 * unless those outnumber what they take, which then get a launch of their
 * own first), four for M = 5..8, where one workgroup selects and groups in a
 * launch of its own.
 * Other sizes run the three calls' kernels in sequence.  See
 * moe_layer_launches.
 *   x, w_router, w13, w2  as for moe_route / moe_decode_fused
 *   w_gate_up, w_down     shared expert [2Is, H] / [H, Is], or both NULL (Is ignored)
 *   topk_ids, topk_w, logits  outputs as for moe_route
 *   y          [M, H] fp16 out
 *   ws         >= moe_workspace_bytes(M, H, E, I, K, Is) bytes of device memory,
 *              256-byte aligned; its state block must be zero before the first
 *              call (see moe_workspace_bytes).  Calls that share a ws must not
 *              overlap in time. */
moe_status moe_layer_decode(const void *x, const void *w_router, const void *w13, const void *w2,
                            const void *w_gate_up, const void *w_down, int M, int H, int E, int I,
                            int K, int Is, int renormalize, int32_t *topk_ids, float *topk_w,
                            float *logits, void *y, void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_decode for callers that cannot allocate device memory (code under
 * hipGraph capture, serving loops, harnesses that forbid hipMalloc): the same
 * arguments, results and launches, without `ws`.  Its workspace is a static
 * device buffer of 512 KiB inside the library, one per GPU, held from the
 * first call on that GPU until the process ends; the call itself allocates
 * nothing and frees nothing.  Sizes whose moe_workspace_bytes exceeds 512 KiB
 * (for example M = 8, K = 16, I = 2048) return MOE_ERR_SCRATCH before anything
 * is enqueued.  The buffer is shared by every call on that GPU and keeps the
 * last call's contents (the call needs none of it to start at any value):
 * calls that overlap in time on one GPU, from any stream or thread, race and
 * must be avoided.  The first call on a device looks the buffer's address up
 * (thread-safe; not a stream operation).  Other errors as for moe_layer_decode. */
moe_status moe_layer_decode_noalloc(const void *x, const void *w_router, const void *w13,
                                    const void *w2, const void *w_gate_up, const void *w_down,
                                    int M, int H, int E, int I, int K, int Is, int renormalize,
                                    int32_t *topk_ids, float *topk_w, float *logits, void *y,
                                    hipStream_t stream);

/* Number of kernels moe_layer_decode enqueues for these sizes: 3 at
 * M = 1..4 (4 at M = 2..4 when the shared expert's down rows outnumber what
 * token 0's gate/up workgroups take, for example K = 1 with narrow experts
 * and a wide shared expert, and they get a launch of their own), 4 at
 * M = 5..8; more where it runs the three calls' kernels; 0 for unsupported
 * sizes or M = 0. */
int moe_layer_launches(int M, int H, int E, int I, int K, int Is);

/* ---- test-only probes (not part of the decode path) --------------------- */

/* moe_layer_decode by a chosen path, for tests and timing.
 * Stages 1..3 run one step of moe_layer_decode's launches alone.  At M = 1:
 * 1 = router (writes logits; with Is != I also the shared activations, to
 * ws), 2 = expand (reads them; writes topk_ids, topk_w, the routed
 * activations, and the shared activations (Is == I) or the shared output
 * (Is != I)), 3 = reduce (reads those; writes y).  At M = 2..8: 1 = router and
 * shared gate/up rows (logits, shared activations), 2 = the selection and the
 * distinct experts' gate/up rows with the shared down rows (one launch at
 * M <= 4 (two where the shared down rows get a launch of their own), two at
 * M = 5..8; topk_ids, topk_w, the group table, the routed
 * activations, the shared output), 3 = the down rows and the combine (y).  A
 * stage reads what the previous stage left in the same buffers, so only a
 * full call (or stages 1, 2, 3 in order) on them makes its inputs valid.
 * Stage 4 runs the launches whole (moe_layer_decode).  Sizes that
 * moe_layer_decode runs as the separate calls' kernels (see
 * moe_layer_launches) take no stage 1..4.
 *
 * Stage 5 runs the layer as ONE launch, on a GPU with 256 CUs in 8 XCDs
 * (MI355X), for H in {1024, 2048}, E <= 256, K <= 8, I in {64, ..., 1024},
 * Is in {0, I} and K*I <= 4096: 256 workgroups of 16 waves, one per CU.  Each
 * XCD computes every router logit itself and hands them over through its own
 * L2; every workgroup selects the experts, streams one gate/up row pair per
 * wave and requests the down rows of its output rows before the activations
 * are known; the activations are exchanged once across the XCDs through
 * device-coherent stores and flags, one workgroup per XCD watching the 256
 * device-wide flags and relaying through a flag in its XCD's L2.  The
 * workgroups wait on each other without atomics, through the workspace's
 * state block (see moe_workspace_bytes); every wait is bounded, and a
 * workgroup whose wait runs out computes the data itself, so a call always
 * completes with the same results -- the three-launch path's bits.  On an
 * MI355X it is slower than the three launches (the hand-offs cost more than
 * the launches they remove), so moe_layer_decode does not use it.
 * Stage 6 is stage 5 with every wait giving up at once (each workgroup
 * computes the logits and every activation itself; slow, for testing that
 * path).
 * Arguments as for moe_layer_decode; MOE_ERR_SHAPE for a stage outside 1..6
 * or sizes that do not take the chosen path. */
moe_status moe_dbg_layer_stage(int stage, const void *x, const void *w_router, const void *w13,
                               const void *w2, const void *w_gate_up, const void *w_down, int M,
                               int H, int E, int I, int K, int Is, int renormalize,
                               int32_t *topk_ids, float *topk_w, float *logits, void *y, void *ws,
                               size_t ws_bytes, hipStream_t stream);

/* An empty kernel: launch latency and the gap between hipGraph kernel nodes. */
moe_status moe_probe_empty(hipStream_t stream);

/* Streams `bytes` (a multiple of 16) of device memory at `src` with
 * non-temporal 16-byte loads (8 in flight per thread; 1 per thread below
 * 4 MiB, so that short reads still spread over many workgroups): the
 * achievable read bandwidth, and the floor of a launch structure timed with
 * several reads in a graph.  out: one device float, written only in a case
 * that zero-filled input never produces. */
moe_status moe_probe_read(const void *src, size_t bytes, float *out, hipStream_t stream);

/* Copies `bytes` (a multiple of 16) from src to dst (device, not overlapping)
 * with a plain 16-byte load/store kernel: a known read and write byte count,
 * the calibration for the memory-traffic counters. */
moe_status moe_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* The lane mapping the kernels use for down-projection rows n fp16 wide (a
 * host query; nothing is enqueued): *lanes_per_row (LPR), *chunks_per_lane
 * (CPL, 16-byte chunks per lane) and *padded (1 if LPR*CPL*8 > n, the steps
 * past the row's end carrying zero weights).  Returns MOE_ERR_SHAPE unless n
 * is a multiple of 64 in [64, 2048], MOE_ERR_NULL for a null output. */
moe_status moe_dbg_lane_map(int n, int *lanes_per_row, int *chunks_per_lane, int *padded);

/* Sums 64 fp32 values with one wavefront's cross-lane (DPP) reduction, the
 * same routine the GEMV kernels use; out[0] = the sum.  in: [64] device. */
moe_status moe_dbg_wave_sum(const float *in, float *out, hipStream_t stream);

/* Step 3 alone: activated [M, K, I] fp32 written to `activated` (device, may be
 * the caller's buffer); same arguments as moe_decode_fused otherwise. */
moe_status moe_dbg_w13_silu(const void *x, const void *w13, const int32_t *topk_ids, int M, int H,
                            int E, int I, int K, float *activated, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* Step 4 alone, with injected activations: the W2 GEMV + weighted combine (+
 * shared_in) of moe_decode_fused reading `activated` [M, K, I] fp32 (device)
 * instead of the W13 stage's output; same arguments as moe_decode_fused
 * otherwise. */
moe_status moe_dbg_w2_combine(const float *activated, const void *w2, const int32_t *topk_ids,
                              const float *topk_w, const float *shared_in, int M, int H, int E,
                              int I, int K, void *y, void *ws, size_t ws_bytes,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
