// moe_internal.h -- shared between the kernels (moe_kernels.hip) and the host
// entry points (moe_abi.cpp); not part of the public ABI.
#ifndef MOE_INTERNAL_H
#define MOE_INTERNAL_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxTokens = 8;
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxSlots = kMaxTokens * kMaxTopk; // M*K entries of topk_ids
constexpr int kMaxInter = 2048;                  // largest I / Is

// Distinct selected experts of an M > 1 call (written by the group-table kernel,
// read by the W13 and W2 kernels of the same call).
struct GroupTable {
    int n_u;
    int pad_[63];
    int u_expert[kMaxSlots];
    unsigned u_mask[kMaxSlots];
    signed char u_slot[kMaxSlots][kMaxTokens];
};

// State the single-launch layer keeps in the workspace between calls (zero
// before the first call): one call counter per workgroup and the hand-off
// flags, which hold the call count of the call that last set them.
constexpr int kLayer1Grid = 256; // workgroups of the single-launch layer (one per CU)
constexpr int kPerXcd = 32;      // of them on each of the 8 XCDs
struct Layer1State {
    unsigned epoch[kLayer1Grid];     // calls each workgroup has completed
    unsigned flag_route[8][kPerXcd]; // router rows stored, per XCD and workgroup
    unsigned flag_act[kLayer1Grid];  // activations published, per workgroup
    unsigned flag_xact[8][kPerXcd];  // [x][0]: every activation published (seen by XCD x)
    unsigned gave_up;                // waits that ran out and computed the data themselves
    unsigned pad_[2047 - 4 * kLayer1Grid];
};
static_assert(sizeof(Layer1State) == 8192, "state block");

// Workspace layout (bytes from the start of ws, 256-byte aligned regions):
//   [0, kStateBytes)                      Layer1State (kept between calls)
//   [kScratch, +kSharedActBytes)          shared-expert activations [M, Is] fp32
//   [kGroupOffset, +sizeof(GroupTable))   GroupTable
//   [kSharedOutOffset, +M*H*4)            shared-expert output [M, H] fp32
//   [kRoutedActOffset, +M*K*I*4)          routed activations [M, K, I] fp32
// The single-launch layer uses [kLayer1LogitsOffset, +8*E*4) for each XCD's
// logits and [kLayer1ActOffset, +(K*I + Is)*4) for the published activations
// (inside the scratch regions above, which it does not otherwise use).
constexpr size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
constexpr size_t kStateBytes = sizeof(Layer1State);
constexpr size_t kScratch = kStateBytes;
constexpr size_t kSharedActBytes = (size_t)kMaxTokens * kMaxInter * sizeof(float);
constexpr size_t kLayer1LogitsOffset = kScratch;
constexpr size_t kLayer1ActOffset = kLayer1LogitsOffset + 8 * kMaxExperts * sizeof(float);
constexpr size_t kGroupOffset = kScratch + align256(kSharedActBytes);
constexpr size_t kSharedOutOffset = kGroupOffset + align256(sizeof(GroupTable));
constexpr size_t kSharedOutBytes = (size_t)kMaxTokens * 4096 * sizeof(float);
constexpr size_t kRoutedActOffset = kSharedOutOffset + align256(kSharedOutBytes);

// Many-token (prefill) layer: per-call plan in the workspace.
constexpr int kPrefillRows = 128; // token rows per grouped-GEMM tile
struct PrefillPlan {
    int total13; // W13 tiles (routed + shared)
    int total2;  // W2 tiles
    int pairs;   // (token, slot) pairs with a valid expert id
    int pad_[61];
    int count[kMaxExperts]; // pairs per expert
    int start[kMaxExperts]; // first entry of each expert in the pair list
};
// Byte offsets of the prefill workspace regions (256-byte aligned) and the
// W13 / W2 grid sizes (multiples of 8, at least the largest tile count).
struct PrefillLayout {
    size_t plan, part, desc13, desc2, perm, act, act_s, down, bytes;
    int grid13, grid2, router_split;
};
PrefillLayout prefill_layout(int T, int H, int E, int I, int K, int Is);
// stage 0: all launches; 1..6: router (partial GEMMs), top-k (the partials
// summed into logits, then the selection), plan, W13, W2, combine alone.
hipError_t launch_prefill(const void *x, const void *wr, const void *w13, const void *w2,
                          const void *wsgu, const void *wsd, int T, int H, int E, int I, int K,
                          int Is, int renorm, int32_t *ids, float *w, float *logits, void *y,
                          void *ws, int stage, hipStream_t s);
hipError_t launch_topk(const float *logits, int M, int E, int K, int renorm, int32_t *ids,
                       float *w, hipStream_t s);
hipError_t launch_topk_sum(const float *part, int P, int M, int E, int K, int renorm,
                           float *logits, int32_t *ids, float *w, hipStream_t s);

inline int mt_of(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

hipError_t launch_route(const void *x, const void *wr, int M, int H, int E, int K, int renorm,
                        int32_t *ids, float *w, float *logits, hipStream_t s);
hipError_t launch_shared(const void *x, const void *wgu, const void *wd, int M, int H, int Is,
                         float *s_out, float *act_shared, hipStream_t s);
hipError_t launch_w13_routed(const void *x, const void *w13, const int32_t *ids, int M, int H,
                             int E, int I, int K, float *act, GroupTable *table, hipStream_t s);
hipError_t launch_fused(const void *x, const void *w13, const void *w2, const int32_t *ids,
                        const float *tw, const float *shared_in, int M, int H, int E, int I, int K,
                        void *y, float *act, GroupTable *table, hipStream_t s);
hipError_t launch_w2_routed(const float *act, const void *w2, const int32_t *ids, const float *tw,
                            const float *shared_in, int M, int H, int E, int I, int K, void *y,
                            GroupTable *table, hipStream_t s);
hipError_t launch_probe_empty(hipStream_t s);
hipError_t launch_probe_read(const void *src, size_t bytes, float *out, hipStream_t s);
hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t s);
hipError_t launch_dbg_wave_sum(const float *in, float *out, hipStream_t s);
// the down-projection lane mapping of rows n fp16 wide (n % 64 == 0, 64..2048)
void lane_map_of(int n, int *lpr, int *cpl, int *pad);
// The layer at M = 1 in three launches (router + shared gate/up, expand, reduce);
// stage 0 runs all three, stage 1..3 that launch alone.
// The layer for 2..8 tokens: router + shared gate/up; the selection with the
// gate/up rows (one launch at M <= 4; a selection launch and the expand
// launch at M = 5..8); the staged W2 kernel.  stage 0 runs every launch,
// stage 1..3 one of those three steps alone.
bool lean_m_ok(int M, int H, int E, int I, int K, int Is);
// kernels launch_lean_m enqueues for these sizes (3, or 4 with a selection
// launch at M = 5..8 or a shared down launch of its own at M <= 4)
int lean_m_launches(int M, int H, int I, int K, int Is);
hipError_t launch_lean_m(const void *x, const void *wr, const void *w13, const void *w2,
                         const void *wsgu, const void *wsd, int M, int H, int E, int I, int K,
                         int Is, int renorm, int32_t *ids, float *w, float *logits, void *y,
                         float *act, float *act_s, float *s_out, GroupTable *table, int stage,
                         hipStream_t s);
bool lean_ok(int M, int H, int E, int I, int K, int Is);
// The layer at M = 1 in one launch (moe_layer1.hip); spin bounds each wait
// (0: every wait gives up at once and computes the data itself).
bool layer1_ok(int M, int H, int E, int I, int K, int Is);
hipError_t launch_layer1(const void *x, const void *wr, const void *w13, const void *w2,
                         const void *wsgu, const void *wsd, int H, int E, int I, int K, int Is,
                         int renorm, int32_t *ids, float *w, float *logits, void *y, void *ws,
                         unsigned spin, hipStream_t s);
constexpr unsigned kLayer1Spin = 1u << 16;
hipError_t launch_state_clear(void *ws, hipStream_t s);
// The static device buffer of moe_layer_decode_noalloc (moe_noalloc.hip): its
// size, and its address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = 512 * 1024;
hipError_t noalloc_scratch(void **out);
hipError_t launch_lean(const void *x, const void *wr, const void *w13, const void *w2,
                       const void *wsgu, const void *wsd, int H, int E, int I, int K, int Is,
                       int renorm, int32_t *ids, float *w, float *logits, void *y, float *act,
                       float *act_s, float *s_out, int stage, hipStream_t s);

} // namespace moe

#endif
