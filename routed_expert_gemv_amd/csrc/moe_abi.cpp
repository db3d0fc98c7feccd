// moe_abi.cpp -- C ABI entry points of libmoe_decode (declared in
// include/moe_decode.h): host-side argument validation, workspace carving and
// kernel launches on the caller's stream.  Every check runs before anything is
// enqueued; nothing here allocates, synchronises or reads device memory.
#include "moe_decode.h"
#include "moe_prefill.h"

#include "moe_internal.h"

using namespace moe;

namespace {

// hidden width: a multiple of 512 up to 4096 (each lane of a wave holds H/512
// 16-byte chunks of a row); expert widths I, Is: multiples of 64 up to 2048
// (any such width has a lane mapping of its down-projection rows)
bool h_ok(int H) { return H >= 512 && H <= 4096 && H % 512 == 0; }
bool i_ok(int I) { return I >= 64 && I <= kMaxInter && I % 64 == 0; }
// above H = 2048, x of more than 4 tokens no longer fits the multi-token
// kernels' registers
bool m_ok(int M, int H) { return M >= 0 && M <= kMaxTokens && (H <= 2048 || M <= 4); }
bool ek_ok(int E, int K) { return E >= 1 && E <= kMaxExperts && K >= 1 && K <= kMaxTopk && K <= E; }

bool al(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t routed_ws_bytes(int M, int I, int K)
{
    return kRoutedActOffset + align256((size_t)M * K * I * sizeof(float));
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool pf_dim_ok(int n, int hi) { return n >= 64 && n <= hi && n % 64 == 0; }
// The grouped GEMMs address token rows with 32-bit byte offsets: the routed
// activations [T*K, I] fp16 must stay below 4 GiB (x and the shared
// activations always do at these bounds).
bool pf_shape_ok(int T, int H, int E, int I, int K, int Is)
{
    return T >= 0 && T <= 65536 && pf_dim_ok(H, 16384) && ek_ok(E, K) && pf_dim_ok(I, 4096) &&
           (Is == 0 || pf_dim_ok(Is, 4096)) &&
           (uint64_t)T * K * I * 2 + (uint64_t)I * 2 < (1ull << 32);
}

} // namespace

static moe_status layer_prefill(const void *x, const void *w_router, const void *w13,
                                const void *w2, const void *w_gate_up, const void *w_down, int T,
                                int H, int E, int I, int K, int Is, int renormalize,
                                int32_t *topk_ids, float *topk_w, float *logits, void *y,
                                void *ws, size_t ws_bytes, int stage, hipStream_t stream)
{
    const bool shared = w_gate_up != nullptr || w_down != nullptr;
    if (!shared) Is = 0;
    if (!pf_shape_ok(T, H, E, I, K, Is) || (shared && Is == 0)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !w13 || !w2 || !topk_ids || !topk_w || !logits || !y || !ws ||
        (shared && (!w_gate_up || !w_down)))
        return MOE_ERR_NULL;
    // y is written four halves (8 bytes) at a time
    if (!al(x, 16) || !al(w_router, 16) || !al(w13, 16) || !al(w2, 16) || !al(topk_ids, 4) ||
        !al(topk_w, 4) || !al(logits, 4) || !al(y, 8) || !al(ws, 256) ||
        (shared && (!al(w_gate_up, 16) || !al(w_down, 16))))
        return MOE_ERR_ALIGN;
    if (ws_bytes < prefill_layout(T, H, E, I, K, Is).bytes) return MOE_ERR_WORKSPACE;
    return hip_status(launch_prefill(x, w_router, w13, w2, w_gate_up, w_down, T, H, E, I, K, Is,
                                     renormalize, topk_ids, topk_w, logits, y, ws, stage, stream));
}

// moe_layer_decode; stage > 0 (three-launch path only) runs that launch alone.
static moe_status layer_decode(const void *x, const void *w_router, const void *w13,
                               const void *w2, const void *w_gate_up, const void *w_down, int M,
                               int H, int E, int I, int K, int Is, int renormalize,
                               int32_t *topk_ids, float *topk_w, float *logits, void *y, void *ws,
                               size_t ws_bytes, int stage, hipStream_t stream)
{
    const bool shared = w_gate_up != nullptr || w_down != nullptr;
    if (!shared) Is = 0;
    if (!m_ok(M, H) || !h_ok(H) || !ek_ok(E, K) || !i_ok(I) || (shared && !i_ok(Is)))
        return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!x || !w_router || !w13 || !w2 || !topk_ids || !topk_w || !logits || !y || !ws ||
        (shared && (!w_gate_up || !w_down)))
        return MOE_ERR_NULL;
    if (!al(x, 16) || !al(w_router, 16) || !al(w13, 16) || !al(w2, 16) || !al(topk_ids, 4) ||
        !al(topk_w, 4) || !al(logits, 4) || !al(y, 2) || !al(ws, 256) ||
        (shared && (!al(w_gate_up, 16) || !al(w_down, 16))))
        return MOE_ERR_ALIGN;
    if (ws_bytes < routed_ws_bytes(M, I, K)) return MOE_ERR_WORKSPACE;
    // stage 1..3: one step of the layer launches (M = 1: one launch each; M > 1:
    // router, selection with gate/up, W2); stage 4: the layer launches whole;
    // 5: the single launch; 6: the single launch with every wait giving up at
    // once
    if (stage < 0 || stage > 6) return MOE_ERR_SHAPE;
    if (stage >= 1 && stage <= 4 && !lean_ok(M, H, E, I, K, Is) && !lean_m_ok(M, H, E, I, K, Is))
        return MOE_ERR_SHAPE;
    if (stage >= 5 && !layer1_ok(M, H, E, I, K, Is)) return MOE_ERR_SHAPE;
    char *base = static_cast<char *>(ws);
    float *act_s = reinterpret_cast<float *>(base + kScratch);
    float *act = reinterpret_cast<float *>(base + kRoutedActOffset);
    if (stage >= 5)
        return hip_status(launch_layer1(x, w_router, w13, w2, w_gate_up, w_down, H, E, I, K, Is,
                                        renormalize, topk_ids, topk_w, logits, y, ws,
                                        stage == 6 ? 0u : kLayer1Spin, stream));
    if (stage == 4) stage = 0;
    if (lean_ok(M, H, E, I, K, Is))
        return hip_status(launch_lean(x, w_router, w13, w2, w_gate_up, w_down, H, E, I, K, Is,
                                      renormalize, topk_ids, topk_w, logits, y, act, act_s,
                                      reinterpret_cast<float *>(base + kSharedOutOffset), stage,
                                      stream));
    float *s_out = shared ? reinterpret_cast<float *>(base + kSharedOutOffset) : nullptr;
    GroupTable *table = reinterpret_cast<GroupTable *>(base + kGroupOffset);
    if (lean_m_ok(M, H, E, I, K, Is))
        return hip_status(launch_lean_m(x, w_router, w13, w2, w_gate_up, w_down, M, H, E, I, K,
                                        Is, renormalize, topk_ids, topk_w, logits, y, act, act_s,
                                        reinterpret_cast<float *>(base + kSharedOutOffset),
                                        table, stage, stream));
    hipError_t err = hipSuccess;
    if (shared) err = launch_shared(x, w_gate_up, w_down, M, H, Is, s_out, act_s, stream);
    if (err == hipSuccess)
        err = launch_route(x, w_router, M, H, E, K, renormalize, topk_ids, topk_w, logits, stream);
    if (err == hipSuccess)
        err = launch_fused(x, w13, w2, topk_ids, topk_w, s_out, M, H, E, I, K, y, act, table,
                           stream);
    return hip_status(err);
}

#ifndef MOE_BUILD_ID
#define MOE_BUILD_ID "unversioned"
#endif

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_build_id(void) { return MOE_BUILD_ID; }

const char *moe_status_str(moe_status s)
{
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is outside the supported set";
    case MOE_ERR_ALIGN: return "a pointer is not aligned as required";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "a kernel launch failed";
    case MOE_ERR_SCRATCH: return "the sizes need more scratch than the library's static buffer";
    default: return "unknown status";
    }
}

size_t moe_workspace_bytes(int M, int H, int E, int I, int K, int Is)
{
    if (!m_ok(M, H) || !h_ok(H) || !ek_ok(E, K) || !i_ok(I) || (Is != 0 && !i_ok(Is))) return 0;
    return routed_ws_bytes(M < 1 ? 1 : M, I, K);
}

moe_status moe_route(const void *x, const void *w_router, int M, int H, int E, int K,
                     int renormalize, int32_t *topk_ids, float *topk_w, float *logits,
                     hipStream_t stream)
{
    if (!m_ok(M, H) || !h_ok(H) || !ek_ok(E, K)) return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w || !logits) return MOE_ERR_NULL;
    if (!al(x, 16) || !al(w_router, 16) || !al(topk_ids, 4) || !al(topk_w, 4) || !al(logits, 4))
        return MOE_ERR_ALIGN;
    return hip_status(launch_route(x, w_router, M, H, E, K, renormalize, topk_ids, topk_w, logits,
                                   stream));
}

moe_status shared_expert(const void *x, const void *w_gate_up, const void *w_down, int M, int H,
                         int Is, float *s_out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!m_ok(M, H) || !h_ok(H) || !i_ok(Is)) return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!x || !w_gate_up || !w_down || !s_out || !ws) return MOE_ERR_NULL;
    if (!al(x, 16) || !al(w_gate_up, 16) || !al(w_down, 16) || !al(s_out, 4) || !al(ws, 256))
        return MOE_ERR_ALIGN;
    if (ws_bytes < kScratch + (size_t)M * Is * sizeof(float)) return MOE_ERR_WORKSPACE;
    return hip_status(launch_shared(x, w_gate_up, w_down, M, H, Is, s_out,
                                    reinterpret_cast<float *>(static_cast<char *>(ws) + kScratch),
                                    stream));
}

moe_status moe_decode_fused(const void *x, const void *w13, const void *w2,
                            const int32_t *topk_ids, const float *topk_w, const float *shared_in,
                            int M, int H, int E, int I, int K, void *y, void *ws, size_t ws_bytes,
                            hipStream_t stream)
{
    if (!m_ok(M, H) || !h_ok(H) || !ek_ok(E, K) || !i_ok(I)) return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!x || !w13 || !w2 || !topk_ids || !topk_w || !y || !ws) return MOE_ERR_NULL;
    if (!al(x, 16) || !al(w13, 16) || !al(w2, 16) || !al(topk_ids, 4) || !al(topk_w, 4) ||
        !al(y, 2) || !al(ws, 256) || (shared_in && !al(shared_in, 4)))
        return MOE_ERR_ALIGN;
    if (ws_bytes < routed_ws_bytes(M, I, K)) return MOE_ERR_WORKSPACE;
    char *base = static_cast<char *>(ws);
    return hip_status(launch_fused(x, w13, w2, topk_ids, topk_w, shared_in, M, H, E, I, K, y,
                                   reinterpret_cast<float *>(base + kRoutedActOffset),
                                   reinterpret_cast<GroupTable *>(base + kGroupOffset), stream));
}

moe_status moe_layer_decode(const void *x, const void *w_router, const void *w13, const void *w2,
                            const void *w_gate_up, const void *w_down, int M, int H, int E, int I,
                            int K, int Is, int renormalize, int32_t *topk_ids, float *topk_w,
                            float *logits, void *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return layer_decode(x, w_router, w13, w2, w_gate_up, w_down, M, H, E, I, K, Is, renormalize,
                        topk_ids, topk_w, logits, y, ws, ws_bytes, 0, stream);
}

moe_status moe_layer_decode_noalloc(const void *x, const void *w_router, const void *w13,
                                    const void *w2, const void *w_gate_up, const void *w_down,
                                    int M, int H, int E, int I, int K, int Is, int renormalize,
                                    int32_t *topk_ids, float *topk_w, float *logits, void *y,
                                    hipStream_t stream)
{
    const bool shared = w_gate_up != nullptr || w_down != nullptr;
    const size_t need = moe_workspace_bytes(M, H, E, I, K, shared ? Is : 0);
    if (need == 0 || (shared && !i_ok(Is))) return MOE_ERR_SHAPE;
    if (need > kNoAllocScratchBytes) return MOE_ERR_SCRATCH;
    if (M == 0) return MOE_OK;
    void *ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
    return layer_decode(x, w_router, w13, w2, w_gate_up, w_down, M, H, E, I, K, Is, renormalize,
                        topk_ids, topk_w, logits, y, ws, kNoAllocScratchBytes, 0, stream);
}

moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!ws) return MOE_ERR_NULL;
    if (!al(ws, 256)) return MOE_ERR_ALIGN;
    if (ws_bytes < kStateBytes) return MOE_ERR_WORKSPACE;
    return hip_status(launch_state_clear(ws, stream));
}

moe_status moe_dbg_layer_stage(int stage, const void *x, const void *w_router, const void *w13,
                               const void *w2, const void *w_gate_up, const void *w_down, int M,
                               int H, int E, int I, int K, int Is, int renormalize,
                               int32_t *topk_ids, float *topk_w, float *logits, void *y, void *ws,
                               size_t ws_bytes, hipStream_t stream)
{
    if (stage < 1 || stage > 6) return MOE_ERR_SHAPE;
    return layer_decode(x, w_router, w13, w2, w_gate_up, w_down, M, H, E, I, K, Is, renormalize,
                        topk_ids, topk_w, logits, y, ws, ws_bytes, stage, stream);
}

int moe_layer_launches(int M, int H, int E, int I, int K, int Is)
{
    if (!m_ok(M, H) || !h_ok(H) || !ek_ok(E, K) || !i_ok(I) || (Is != 0 && !i_ok(Is))) return 0;
    if (M == 0) return 0;
    if (lean_ok(M, H, E, I, K, Is)) return 3;
    // M <= 4: router, expand with the selection folded in, W2; else a
    // separate selection launch before the expand
    if (lean_m_ok(M, H, E, I, K, Is)) return lean_m_launches(M, H, I, K, Is);
    // shared_expert (2) + moe_route (2) + moe_decode_fused (2)
    return (Is ? 2 : 0) + 2 + 2;
}

size_t moe_prefill_workspace_bytes(int T, int H, int E, int I, int K, int Is)
{
    if (!pf_shape_ok(T, H, E, I, K, Is)) return 0;
    return prefill_layout(T < 1 ? 1 : T, H, E, I, K, Is).bytes;
}

moe_status moe_layer_prefill(const void *x, const void *w_router, const void *w13,
                             const void *w2, const void *w_gate_up, const void *w_down, int T,
                             int H, int E, int I, int K, int Is, int renormalize,
                             int32_t *topk_ids, float *topk_w, float *logits, void *y, void *ws,
                             size_t ws_bytes, hipStream_t stream)
{
    return layer_prefill(x, w_router, w13, w2, w_gate_up, w_down, T, H, E, I, K, Is, renormalize,
                         topk_ids, topk_w, logits, y, ws, ws_bytes, 0, stream);
}

moe_status moe_dbg_prefill_stage(int stage, const void *x, const void *w_router, const void *w13,
                                 const void *w2, const void *w_gate_up, const void *w_down,
                                 int T, int H, int E, int I, int K, int Is, int renormalize,
                                 int32_t *topk_ids, float *topk_w, float *logits, void *y,
                                 void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (stage < 1 || stage > 6) return MOE_ERR_SHAPE;
    return layer_prefill(x, w_router, w13, w2, w_gate_up, w_down, T, H, E, I, K, Is, renormalize,
                         topk_ids, topk_w, logits, y, ws, ws_bytes, stage, stream);
}

moe_status moe_probe_empty(hipStream_t stream) { return hip_status(launch_probe_empty(stream)); }

moe_status moe_probe_read(const void *src, size_t bytes, float *out, hipStream_t stream)
{
    if (!src || !out) return MOE_ERR_NULL;
    if (!al(src, 16) || !al(out, 4) || bytes % 16) return MOE_ERR_ALIGN;
    return hip_status(launch_probe_read(src, bytes, out, stream));
}

moe_status moe_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t stream)
{
    if (!src || !dst) return MOE_ERR_NULL;
    if (!al(src, 16) || !al(dst, 16) || bytes % 16) return MOE_ERR_ALIGN;
    return hip_status(launch_probe_copy(src, dst, bytes, stream));
}

moe_status moe_dbg_lane_map(int n, int *lanes_per_row, int *chunks_per_lane, int *padded)
{
    if (!i_ok(n)) return MOE_ERR_SHAPE;
    if (!lanes_per_row || !chunks_per_lane || !padded) return MOE_ERR_NULL;
    lane_map_of(n, lanes_per_row, chunks_per_lane, padded);
    return MOE_OK;
}

moe_status moe_dbg_wave_sum(const float *in, float *out, hipStream_t stream)
{
    if (!in || !out) return MOE_ERR_NULL;
    if (!al(in, 4) || !al(out, 4)) return MOE_ERR_ALIGN;
    return hip_status(launch_dbg_wave_sum(in, out, stream));
}

moe_status moe_dbg_w13_silu(const void *x, const void *w13, const int32_t *topk_ids, int M, int H,
                            int E, int I, int K, float *activated, void *ws, size_t ws_bytes,
                            hipStream_t stream)
{
    if (!m_ok(M, H) || !h_ok(H) || !ek_ok(E, K) || !i_ok(I)) return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!x || !w13 || !topk_ids || !activated || !ws) return MOE_ERR_NULL;
    if (!al(x, 16) || !al(w13, 16) || !al(topk_ids, 4) || !al(activated, 16) || !al(ws, 256))
        return MOE_ERR_ALIGN;
    if (ws_bytes < routed_ws_bytes(M, I, K)) return MOE_ERR_WORKSPACE;
    char *base = static_cast<char *>(ws);
    return hip_status(launch_w13_routed(x, w13, topk_ids, M, H, E, I, K, activated,
                                        reinterpret_cast<GroupTable *>(base + kGroupOffset),
                                        stream));
}

moe_status moe_dbg_w2_combine(const float *activated, const void *w2, const int32_t *topk_ids,
                              const float *topk_w, const float *shared_in, int M, int H, int E,
                              int I, int K, void *y, void *ws, size_t ws_bytes,
                              hipStream_t stream)
{
    if (!m_ok(M, H) || !h_ok(H) || !ek_ok(E, K) || !i_ok(I)) return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!activated || !w2 || !topk_ids || !topk_w || !y || !ws) return MOE_ERR_NULL;
    if (!al(activated, 16) || !al(w2, 16) || !al(topk_ids, 4) || !al(topk_w, 4) || !al(y, 2) ||
        !al(ws, 256) || (shared_in && !al(shared_in, 4)))
        return MOE_ERR_ALIGN;
    if (ws_bytes < routed_ws_bytes(M, I, K)) return MOE_ERR_WORKSPACE;
    char *base = static_cast<char *>(ws);
    return hip_status(launch_w2_routed(activated, w2, topk_ids, topk_w, shared_in, M, H, E, I, K,
                                       y, reinterpret_cast<GroupTable *>(base + kGroupOffset),
                                       stream));
}

} // extern "C"
