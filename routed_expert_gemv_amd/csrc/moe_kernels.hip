// moe_kernels.hip -- gfx950 (CDNA4) kernels of the single-token routed-expert
// MoE decode layer.  Host entry points and argument checks are in moe_abi.cpp.
//
// Method (BI-V100 inference worklog, "如何在天垓 BI-V100 上优化大模型推理：
// 一份工作日志"): part 3 -- read the selected experts' rows in place by
// expert id instead of gathering copies; part 10 -- W13 GEMV input(1,H) x
// W13[expert_ids[k], row, :] and W2 GEMV activated(K,I) x W2[expert_ids[k], h, :]
// with the weighted sum; part 8 -- routing is a top-k plus a softmax.  The
// pages' own kernels (one 64-wide warp per row, shared-memory or shfl_down
// reductions, SiLU as a separate op) were built for another GPU; here:
//   * every weight row is streamed with coalesced 16-byte loads (one wave
//     instruction moves 1 KiB of contiguous row data) marked non-temporal,
//     since each weight is used exactly once per token;
//   * products use v_dot2 (two fp16 products into an fp32 accumulator);
//   * cross-lane sums use DPP in registers (no LDS, no barriers, no atomics),
//     in one fixed tree, so results are bitwise reproducible;
//   * SiLU*mul is applied in the W13 epilogue (computed once per row pair);
//   * the top-k weights are folded into each lane's partial before the single
//     cross-lane reduction of the W2 kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ f16x8 stream_load(const f16x8 *p)
{
    return __builtin_nontemporal_load(p);
}

// acc + sum_i a[i] * b[i] over 8 fp16 pairs, as four v_dot2 (fp32 accumulate)
__device__ __forceinline__ float dot8(f16x8 a, f16x8 b, float acc)
{
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1),
                                 __builtin_shufflevector(b, b, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3),
                                 __builtin_shufflevector(b, b, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5),
                                 __builtin_shufflevector(b, b, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7),
                                 __builtin_shufflevector(b, b, 6, 7), acc, false);
    return acc;
}

// value of lane (src per DPP_CTRL) for lanes whose row is enabled in ROW_MASK, 0 elsewhere
template <int DPP_CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 DPP_CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8, 16, 32 or 64), fixed tree:
//   quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
//   row_half_mirror (8-lane halves), row_mirror (16-lane rows),
//   row_bcast:15 (row r-1's last lane into rows 1 and 3),
//   row_bcast:31 (lane 31 into rows 2 and 3).
// The group sum is valid in group_holder<G>(g) (and, for G <= 16, in every
// lane of the group).
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group size");
    v += dpp<0xB1, 0xF>(v);
    v += dpp<0x4E, 0xF>(v);
    v += dpp<0x141, 0xF>(v);
    if (G >= 16) v += dpp<0x140, 0xF>(v);
    if (G >= 32) v += dpp<0x142, 0xA>(v);
    if (G >= 64) v += dpp<0x143, 0xC>(v);
    return v;
}

template <int G>
__device__ __forceinline__ int group_holder(int g)
{
    return G <= 16 ? g * G : (G == 32 ? g * 32 + 31 : 63);
}

// Whole-wave sum, returned as a wave-uniform value.
__device__ __forceinline__ float wave_sum(float v)
{
    v = group_sum<64>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// ---------------------------------------------------------------- grouping
// For M > 1 tokens: the distinct selected experts U, in order of first
// appearance scanning topk_ids row by row, with the tokens that use each one
// and the slot k at which each of those tokens selected it.  One wave scans
// the M*K <= 128 entries: lane i (and i + 64) owns entry i = m*K + k.
template <int MT>
struct GroupScan {
    int v[2];          // expert id of the lane's entries (-1: none)
    bool first[2];     // first appearance of that id
    unsigned mask[2];  // tokens that selected that id
    int slot[2][MT];   // slot k per token (valid where mask is set)
    int rank[2];       // index of that id in U (valid where first)
    int n_u;           // |U|
};

template <int MT>
__device__ __forceinline__ GroupScan<MT> group_scan(const int32_t *ids, int M, int K)
{
    const int lane = lane_id();
    const int n = M * K;
    GroupScan<MT> g;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = lane + q * kWave;
        g.v[q] = i < n ? ids[i] : -1;
        g.first[q] = i < n;
        g.mask[q] = 0u;
#pragma unroll
        for (int m = 0; m < MT; ++m) g.slot[q][m] = 0;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m >= M) break;
        for (int k = 0; k < K; ++k) {
            const int j = m * K + k;
            const int vj = j < kWave ? __builtin_amdgcn_readlane(g.v[0], j)
                                     : __builtin_amdgcn_readlane(g.v[1], j - kWave);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                if (vj == g.v[q]) {
                    if (j < lane + q * kWave) g.first[q] = false;
                    g.mask[q] |= 1u << m;
                    g.slot[q][m] = k;
                }
        }
    }
    const uint64_t b0 = __ballot(g.first[0]);
    const uint64_t b1 = __ballot(g.first[1]);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    g.rank[0] = __popcll(b0 & below);
    g.rank[1] = __popcll(b0) + __popcll(b1 & below);
    g.n_u = __popcll(b0) + __popcll(b1);
    return g;
}

// The entry of U at index u, read from the lane that holds it (wave-uniform).
template <int MT>
__device__ __forceinline__ void group_pick(const GroupScan<MT> &g, int u, int &expert,
                                           unsigned &mask, int (&slot)[MT])
{
    const uint64_t h0 = __ballot(g.first[0] && g.rank[0] == u);
    const uint64_t h1 = __ballot(g.first[1] && g.rank[1] == u);
    const int q = h0 ? 0 : 1;
    const int src = h0 ? __builtin_ctzll(h0) : __builtin_ctzll(h1);
    expert = __builtin_amdgcn_readlane(q == 0 ? g.v[0] : g.v[1], src);
    mask = (unsigned)__builtin_amdgcn_readlane(q == 0 ? (int)g.mask[0] : (int)g.mask[1], src);
#pragma unroll
    for (int m = 0; m < MT; ++m)
        slot[m] = __builtin_amdgcn_readlane(q == 0 ? g.slot[0][m] : g.slot[1][m], src);
}

// Store U (ids, token masks, slots) for the W2 kernel.
template <int MT>
__device__ __forceinline__ void group_store(const GroupScan<MT> &g, GroupTable *table)
{
#pragma unroll
    for (int q = 0; q < 2; ++q)
        if (g.first[q]) {
            const int r = g.rank[q];
            table->u_expert[r] = g.v[q];
            table->u_mask[r] = g.mask[q];
#pragma unroll
            for (int m = 0; m < kMaxTokens; ++m)
                table->u_slot[r][m] = (signed char)(m < MT ? g.slot[q][m < MT ? m : 0] : 0);
        }
    if (lane_id() == 0) table->n_u = g.n_u;
}

// ---------------------------------------------------------------- router GEMV
// One wave per expert row e: logits[m, e] = sum_h Wr[e, h] x[m, h].
// Lane l holds 16-byte chunks c*64 + l of the row (c < HC, H = 512*HC).
template <int HC>
__global__ __launch_bounds__(kWave) void k_router(const f16 *__restrict__ x,
                                                  const f16 *__restrict__ wr, int M, int E,
                                                  float *__restrict__ logits)
{
    constexpr int H = 512 * HC;
    const int e = blockIdx.x;
    const int lane = lane_id();
    const f16x8 *row = reinterpret_cast<const f16x8 *>(wr + (size_t)e * H);
    f16x8 w[HC];
#pragma unroll
    for (int c = 0; c < HC; ++c) w[c] = stream_load(row + c * kWave + lane);
    for (int m = 0; m < M; ++m) {
        const f16x8 *xr = reinterpret_cast<const f16x8 *>(x + (size_t)m * H);
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < HC; ++c) acc = dot8(w[c], xr[c * kWave + lane], acc);
        const float t = wave_sum(acc);
        if (lane == 0) logits[(size_t)m * E + e] = t;
    }
}

// ---------------------------------------------------------------- top-k + softmax
// One wave per token.  Key = order-preserving map of the fp32 logit in the
// high word, ~expert_id in the low word: the largest key is the largest logit,
// and among equal logits the lower id.  K rounds of a wave arg-max.
__device__ __forceinline__ uint64_t topk_key(float v, int e)
{
    v = v + 0.0f; // -0 -> +0, so the two zeros tie
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__global__ __launch_bounds__(kWave) void k_topk(const float *__restrict__ logits, int E, int K,
                                                int renormalize, int32_t *__restrict__ ids,
                                                float *__restrict__ weights)
{
    constexpr int NPL = kMaxExperts / kWave;
    const int m = blockIdx.x;
    const int lane = lane_id();
    const float *L = logits + (size_t)m * E;
    uint64_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = i * kWave + lane;
        key[i] = e < E ? topk_key(L[e], e) : 0ull;
    }
    int my_id = 0;
    float my_l = 0.0f, lmax = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint64_t o = __shfl_xor(best, off);
            best = o > best ? o : best;
        }
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (key[i] == best) key[i] = 0ull;
        const int id = (int)(0xFFFFFFFFu - (uint32_t)best);
        const float lv = L[id];
        if (k == 0) lmax = lv;
        if (lane == k) {
            my_id = id;
            my_l = lv;
        }
    }
    const float ex = lane < K ? expf(my_l - lmax) : 0.0f;
    float z;
    if (renormalize) {
        z = wave_sum(ex);
    } else {
        float part = 0.0f;
        for (int e = lane; e < E; e += kWave) part += expf(L[e] - lmax);
        z = wave_sum(part);
    }
    if (lane < K) {
        ids[(size_t)m * K + lane] = my_id;
        weights[(size_t)m * K + lane] = ex / z;
    }
}

// ---------------------------------------------------------------- W13 + SiLU
// One wave per (expert, row pair j): gate row j and up row I + j of that
// expert, read in place at W13 + expert*(2I*H).  Both rows are loaded before
// any arithmetic (2*HC 16-byte loads in flight per lane); for every token that
// routes to the expert, gate and up dot products are reduced across the wave
// and activated = silu(gate) * up is stored (fp32) at act[m, slot, j].
//
// SHARED: the shared expert (one "expert" at `w13`, every token, slot 0).
template <int HC, int MT, bool SHARED>
__global__ __launch_bounds__(kBlock) void k_w13_silu(const f16 *__restrict__ x,
                                                     const f16 *__restrict__ w13,
                                                     const int32_t *__restrict__ ids, int M,
                                                     int I, int K, float *__restrict__ act,
                                                     GroupTable *__restrict__ table)
{
    constexpr int H = 512 * HC;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int blocks_per_expert = I / kWavesPerBlock;
    const int u = blockIdx.x / blocks_per_expert;
    const int j = (blockIdx.x % blocks_per_expert) * kWavesPerBlock + wave;

    int expert;
    unsigned mask;
    int slot[MT];
    if (SHARED) {
        expert = 0;
        mask = (1u << M) - 1u;
#pragma unroll
        for (int m = 0; m < MT; ++m) slot[m] = 0;
    } else if (MT == 1) {
        expert = ids[u];
        mask = 1u;
        slot[0] = u;
    } else {
        const GroupScan<MT> g = group_scan<MT>(ids, M, K);
        if (blockIdx.x == 0 && wave == 0) group_store<MT>(g, table);
        if (u >= g.n_u) return; // fewer distinct experts than slots: nothing to do
        group_pick<MT>(g, u, expert, mask, slot);
    }

    // x first (L2-resident, shared by every wave), then the two weight rows
    f16x8 xv[MT][HC];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        if (mask & (1u << m)) {
            const f16x8 *xr = reinterpret_cast<const f16x8 *>(x + (size_t)m * H);
#pragma unroll
            for (int c = 0; c < HC; ++c) xv[m][c] = xr[c * kWave + lane];
        }
    const f16 *base = w13 + (size_t)expert * 2 * I * H;
    const f16x8 *grow = reinterpret_cast<const f16x8 *>(base + (size_t)j * H);
    const f16x8 *urow = reinterpret_cast<const f16x8 *>(base + (size_t)(I + j) * H);
    f16x8 wg[HC], wu[HC];
#pragma unroll
    for (int c = 0; c < HC; ++c) {
        wg[c] = stream_load(grow + c * kWave + lane);
        wu[c] = stream_load(urow + c * kWave + lane);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
        if (mask & (1u << m)) {
            float ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int c = 0; c < HC; ++c) {
                ag = dot8(wg[c], xv[m][c], ag);
                au = dot8(wu[c], xv[m][c], au);
            }
            const float g = wave_sum(ag);
            const float up = wave_sum(au);
            if (lane == 0) act[((size_t)m * K + slot[m]) * I + j] = silu_mul(g, up);
        }
}

// ---------------------------------------------------------------- W2 + combine
// A wave owns RPL = 64/LPR consecutive output rows h; LPR lanes share one
// row, each holding CPL 16-byte chunks of it (I = 8*LPR*CPL).  For every
// selected expert (routing order; for M > 1 the distinct experts in order of
// first appearance) the wave loads its rows of W2[expert] in place, batches of
// up to 8 experts in flight, and each lane accumulates
//     acc[m] += w[m, k] * sum_{its elements j} W2[expert, h, j] * act[m, k, j]
// so the routing weights are applied before the one cross-lane reduction per
// (token, row).  The shared-expert term is added last, then y is rounded to
// fp16 once.
//
// SHARED: the shared expert's down projection (one expert at `w2`, weight 1,
// every token, fp32 output without rounding, nothing added).
template <int LPR, int CPL, int MT, bool SHARED>
__global__ __launch_bounds__(kBlock) void k_w2_combine(
    const float *__restrict__ act, const f16 *__restrict__ w2, const int32_t *__restrict__ ids,
    const float *__restrict__ topk_w, const float *__restrict__ shared_in, int M, int H, int I,
    int K, const GroupTable *__restrict__ table, void *__restrict__ out)
{
    constexpr int RPL = kWave / LPR;
    constexpr int BATCH = 8;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int r = lane / LPR;
    const int cl = lane % LPR;
    const int h = (blockIdx.x * kWavesPerBlock + wave) * RPL + r;

    const int n_u = SHARED ? 1 : (MT == 1 ? K : table->n_u);
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    for (int u0 = 0; u0 < n_u; u0 += BATCH) {
        const int cnt = n_u - u0 < BATCH ? n_u - u0 : BATCH;
        f16x8 wv[BATCH][CPL];
#pragma unroll
        for (int t = 0; t < BATCH; ++t)
            if (t < cnt) {
                int e;
                if (SHARED) e = 0;
                else if (MT == 1) e = ids[u0 + t];
                else e = table->u_expert[u0 + t];
                const f16x8 *row =
                    reinterpret_cast<const f16x8 *>(w2 + ((size_t)e * H + h) * I);
#pragma unroll
                for (int c = 0; c < CPL; ++c) wv[t][c] = stream_load(row + c * LPR + cl);
            }
#pragma unroll
        for (int t = 0; t < BATCH; ++t)
            if (t < cnt) {
                unsigned mask;
                if (SHARED) mask = (1u << M) - 1u;
                else if (MT == 1) mask = 1u;
                else mask = table->u_mask[u0 + t];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (mask & (1u << m)) {
                        int k;
                        if (SHARED) k = 0;
                        else if (MT == 1) k = u0 + t;
                        else k = table->u_slot[u0 + t][m];
                        const float wt = SHARED ? 1.0f : topk_w[(size_t)m * K + k];
                        const float *a = act + ((size_t)m * (SHARED ? 1 : K) + k) * I;
                        float d = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c) {
                            const f32x4 *ap = reinterpret_cast<const f32x4 *>(a + (c * LPR + cl) * 8);
                            const f32x4 a0 = ap[0], a1 = ap[1];
                            const f16x8 wc = wv[t][c];
                            d = fmaf((float)wc[0], a0[0], d);
                            d = fmaf((float)wc[1], a0[1], d);
                            d = fmaf((float)wc[2], a0[2], d);
                            d = fmaf((float)wc[3], a0[3], d);
                            d = fmaf((float)wc[4], a1[0], d);
                            d = fmaf((float)wc[5], a1[1], d);
                            d = fmaf((float)wc[6], a1[2], d);
                            d = fmaf((float)wc[7], a1[3], d);
                        }
                        acc[m] = fmaf(wt, d, acc[m]);
                    }
            }
    }

    const bool holder = lane == group_holder<LPR>(r);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const float t = group_sum<LPR>(acc[m]);
        if (m < M && holder) {
            const size_t o = (size_t)m * H + h;
            if (SHARED) {
                static_cast<float *>(out)[o] = t;
            } else {
                const float v = shared_in ? t + shared_in[o] : t;
                static_cast<f16 *>(out)[o] = (f16)v;
            }
        }
    }
}

// ---------------------------------------------------------------- group table only
// One wave: store U for a W2 stage that runs without the W13 kernel before it.
template <int MT>
__global__ __launch_bounds__(kWave) void k_group_table(const int32_t *__restrict__ ids, int M,
                                                       int K, GroupTable *__restrict__ table)
{
    const GroupScan<MT> g = group_scan<MT>(ids, M, K);
    group_store<MT>(g, table);
}

// ---------------------------------------------------------------- probes
__global__ __launch_bounds__(kWave) void k_dbg_wave_sum(const float *__restrict__ in,
                                                         float *__restrict__ out)
{
    const float t = wave_sum(in[lane_id()]);
    if (lane_id() == 0) out[0] = t;
}

// ---------------------------------------------------------------- launchers
static inline hipError_t last() { return hipGetLastError(); }

template <int HC>
static hipError_t launch_router_hc(const void *x, const void *wr, int M, int E, float *logits,
                                   hipStream_t s)
{
    hipLaunchKernelGGL(k_router<HC>, dim3(E), dim3(kWave), 0, s, (const f16 *)x,
                       (const f16 *)wr, M, E, logits);
    return last();
}

hipError_t launch_route(const void *x, const void *wr, int M, int H, int E, int K, int renorm,
                        int32_t *ids, float *w, float *logits, hipStream_t s)
{
    hipError_t err;
    switch (H / 512) {
    case 1: err = launch_router_hc<1>(x, wr, M, E, logits, s); break;
    case 2: err = launch_router_hc<2>(x, wr, M, E, logits, s); break;
    case 4: err = launch_router_hc<4>(x, wr, M, E, logits, s); break;
    case 8: err = launch_router_hc<8>(x, wr, M, E, logits, s); break;
    default: return hipErrorInvalidValue;
    }
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_topk, dim3(M), dim3(kWave), 0, s, logits, E, K, renorm, ids, w);
    return last();
}

template <int HC, int MT, bool SHARED>
static hipError_t launch_w13_t(const void *x, const void *w13, const int32_t *ids, int M, int I,
                               int K, int n_slots, float *act, GroupTable *table, hipStream_t s)
{
    const int blocks = n_slots * (I / kWavesPerBlock);
    hipLaunchKernelGGL((k_w13_silu<HC, MT, SHARED>), dim3(blocks), dim3(kBlock), 0, s,
                       (const f16 *)x, (const f16 *)w13, ids, M, I, K, act, table);
    return last();
}

template <int HC, bool SHARED>
static hipError_t launch_w13_hc(const void *x, const void *w13, const int32_t *ids, int M, int I,
                                int K, int n_slots, float *act, GroupTable *table, hipStream_t s)
{
    switch (mt_of(M)) {
    case 1: return launch_w13_t<HC, 1, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
    case 2: return launch_w13_t<HC, 2, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
    case 4: return launch_w13_t<HC, 4, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
    case 8:
        if constexpr (HC <= 4)
            return launch_w13_t<HC, 8, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
        return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

template <bool SHARED>
static hipError_t launch_w13(const void *x, const void *w13, const int32_t *ids, int M, int H,
                             int I, int K, int n_slots, float *act, GroupTable *table,
                             hipStream_t s)
{
    switch (H / 512) {
    case 1: return launch_w13_hc<1, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
    case 2: return launch_w13_hc<2, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
    case 4: return launch_w13_hc<4, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
    case 8: return launch_w13_hc<8, SHARED>(x, w13, ids, M, I, K, n_slots, act, table, s);
    }
    return hipErrorInvalidValue;
}

template <int LPR, int CPL, int MT, bool SHARED>
static hipError_t launch_w2_t(const float *act, const void *w2, const int32_t *ids,
                              const float *tw, const float *shared_in, int M, int H, int I, int K,
                              const GroupTable *table, void *out, hipStream_t s)
{
    constexpr int rows_per_block = (kWave / LPR) * kWavesPerBlock;
    const int blocks = H / rows_per_block;
    hipLaunchKernelGGL((k_w2_combine<LPR, CPL, MT, SHARED>), dim3(blocks), dim3(kBlock), 0, s,
                       act, (const f16 *)w2, ids, tw, shared_in, M, H, I, K, table, out);
    return last();
}

template <int LPR, int CPL, bool SHARED>
static hipError_t launch_w2_i(const float *act, const void *w2, const int32_t *ids,
                              const float *tw, const float *shared_in, int M, int H, int I, int K,
                              const GroupTable *table, void *out, hipStream_t s)
{
    switch (mt_of(M)) {
    case 1: return launch_w2_t<LPR, CPL, 1, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 2: return launch_w2_t<LPR, CPL, 2, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 4: return launch_w2_t<LPR, CPL, 4, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 8: return launch_w2_t<LPR, CPL, 8, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    }
    return hipErrorInvalidValue;
}

template <bool SHARED>
static hipError_t launch_w2(const float *act, const void *w2, const int32_t *ids, const float *tw,
                            const float *shared_in, int M, int H, int I, int K,
                            const GroupTable *table, void *out, hipStream_t s)
{
    switch (I) {
    case 64: return launch_w2_i<8, 1, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 128: return launch_w2_i<16, 1, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 256: return launch_w2_i<32, 1, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 512: return launch_w2_i<64, 1, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 1024: return launch_w2_i<64, 2, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 2048: return launch_w2_i<64, 4, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_shared(const void *x, const void *wgu, const void *wd, int M, int H, int Is,
                         float *s_out, float *act_shared, hipStream_t s)
{
    hipError_t err = launch_w13<true>(x, wgu, nullptr, M, H, Is, 1, 1, act_shared, nullptr, s);
    if (err != hipSuccess) return err;
    return launch_w2<true>(act_shared, wd, nullptr, nullptr, nullptr, M, H, Is, 1, nullptr, s_out,
                           s);
}

hipError_t launch_w13_routed(const void *x, const void *w13, const int32_t *ids, int M, int H,
                             int E, int I, int K, float *act, GroupTable *table, hipStream_t s)
{
    const int n_slots = M * K < E ? M * K : E;
    return launch_w13<false>(x, w13, ids, M, H, I, K, n_slots, act, table, s);
}

hipError_t launch_fused(const void *x, const void *w13, const void *w2, const int32_t *ids,
                        const float *tw, const float *shared_in, int M, int H, int E, int I, int K,
                        void *y, float *act, GroupTable *table, hipStream_t s)
{
    hipError_t err = launch_w13_routed(x, w13, ids, M, H, E, I, K, act, table, s);
    if (err != hipSuccess) return err;
    return launch_w2<false>(act, w2, ids, tw, shared_in, M, H, I, K, table, y, s);
}

hipError_t launch_w2_routed(const float *act, const void *w2, const int32_t *ids, const float *tw,
                            const float *shared_in, int M, int H, int E, int I, int K, void *y,
                            GroupTable *table, hipStream_t s)
{
    (void)E;
    if (M > 1) {
        switch (mt_of(M)) {
        case 2: hipLaunchKernelGGL(k_group_table<2>, dim3(1), dim3(kWave), 0, s, ids, M, K, table); break;
        case 4: hipLaunchKernelGGL(k_group_table<4>, dim3(1), dim3(kWave), 0, s, ids, M, K, table); break;
        default: hipLaunchKernelGGL(k_group_table<8>, dim3(1), dim3(kWave), 0, s, ids, M, K, table); break;
        }
        const hipError_t err = last();
        if (err != hipSuccess) return err;
    }
    return launch_w2<false>(act, w2, ids, tw, shared_in, M, H, I, K, table, y, s);
}

hipError_t launch_dbg_wave_sum(const float *in, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(k_dbg_wave_sum, dim3(1), dim3(kWave), 0, s, in, out);
    return last();
}

} // namespace moe
