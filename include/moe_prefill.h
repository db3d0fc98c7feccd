/*
 * moe_prefill.h -- C ABI of the many-token (prefill) MoE layer on MI355X
 * (gfx950): the layer of moe_decode.h (router, top-K + softmax, routed
 * gate/up + SiLU*mul, down + weighted combine, shared expert), for T tokens
 * at once, with each expert's weights read once per tile of up to 128 of the
 * tokens routed to it and the products on the matrix cores.
 *
 * Where the pages define it: "如何在天垓 BI-V100 上优化大模型推理：一份工作
 * 日志" (BI-V100 inference worklog), part 8 -- for T > 1 the MoE products are
 * matrix products whose arithmetic intensity grows with the tokens per expert,
 * where tiling applies; "decode analysis report 2026-07-14", next steps -- the
 * prefill path loops over the distinct experts one by one and is to become a
 * grouped (batched) GEMM.  The layer itself is the one of moe_decode.h.
 *
 * Conventions are those of moe_decode.h (device pointers, caller-owned
 * buffers, enqueue-only, host-side validation, no device-data checks), with:
 *   - sizes (MOE_ERR_SHAPE otherwise): 0 <= T <= 65536; H a multiple of 64 in
 *     [64, 16384]; 1 <= E <= 1024; 1 <= K <= min(E, 16); I a multiple of 64 in
 *     [64, 4096]; Is = 0 (no shared expert) or a multiple of 64 in [64, 4096];
 *   - T = 0 is a valid empty call;
 *   - alignment (MOE_ERR_ALIGN otherwise): as moe_decode.h, except that y must
 *     be 8-byte aligned (it is written four halves at a time).
 */
#ifndef MOE_PREFILL_H
#define MOE_PREFILL_H

#include "moe_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes moe_layer_prefill needs for these sizes (0 if unsupported).
 * It holds the per-call plan (per-expert row lists, tile lists), the routed
 * activations [T*K, I] fp16, the shared activations [T, Is] fp16 and the
 * per-(token, slot) down products [T*K, H] fp32. */
size_t moe_prefill_workspace_bytes(int T, int H, int E, int I, int K, int Is);

/* The whole layer for T tokens; every output of moe_layer_decode, with the
 * same meaning and layout:
 *   x          [T, H] fp16
 *   w_router   [E, H] fp16;  w13 [E, 2I, H] fp16 (rows [0, I) gate, [I, 2I) up);
 *   w2         [E, H, I] fp16
 *   w_gate_up, w_down  shared expert [2Is, H] / [H, Is] fp16, or both NULL
 *   topk_ids   [T, K] int32 out, each token's experts, largest logit first
 *              (equal logits: lower id first)
 *   topk_w     [T, K] fp32 out, routing weights (renormalised when
 *              renormalize != 0)
 *   logits     [T, E] fp32 out (router products)
 *   y          [T, H] fp16 out: fp16(sum_k topk_w[t,k] down_k[t, h] + s[t, h]),
 *              k in routing order in fp32, one rounding
 *   ws         >= moe_prefill_workspace_bytes(...) bytes; scratch only.  Calls
 *              sharing a ws must not overlap in time.
 * Seven launches: the router GEMM (in slices of H) and the ordered sum of its
 * slices, top-K, the plan (one workgroup: per-expert pair lists and tile
 * lists), the gate/up grouped GEMM with SiLU*mul (routed experts plus the
 * shared expert as one more group), the down grouped GEMM (same groups; fp32
 * products per (token, slot) and per token for the shared expert), and the
 * combine: weighted sum in routing order plus the shared output, one fp16
 * rounding.
 * The routed activations are rounded to fp16 before the down products. */
moe_status moe_layer_prefill(const void *x, const void *w_router, const void *w13,
                             const void *w2, const void *w_gate_up, const void *w_down, int T,
                             int H, int E, int I, int K, int Is, int renormalize,
                             int32_t *topk_ids, float *topk_w, float *logits, void *y, void *ws,
                             size_t ws_bytes, hipStream_t stream);

/* Test-only: one stage of moe_layer_prefill alone, for timing each kernel:
 * 1 router (the partial logits), 2 top-K (their sum into logits, then the
 * selection), 3 plan, 4 gate/up, 5 down, 6 combine.
 * A stage reads what the previous ones left in the same buffers; arguments as
 * for moe_layer_prefill; MOE_ERR_SHAPE for a stage outside 1..6. */
moe_status moe_dbg_prefill_stage(int stage, const void *x, const void *w_router, const void *w13,
                                 const void *w2, const void *w_gate_up, const void *w_down,
                                 int T, int H, int E, int I, int K, int Is, int renormalize,
                                 int32_t *topk_ids, float *topk_w, float *logits, void *y,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PREFILL_H */
