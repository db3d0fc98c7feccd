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

#include <atomic>
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;

// ---------------------------------------------------------------- lane mappings
// How a wave covers rows of a down projection (W2 rows, I wide; shared down
// rows, Is wide; n = 16-byte chunks per row): LPR lanes per row (8, 16, 32 or
// 64, so a wave holds RPL = 64/LPR rows), each lane loading CPL chunks, chunk
// q = c*LPR + cl in its c-th step.  A lane's partial sum runs over its chunks
// in step order, then the group tree of LPR lanes adds the partials.
// When n = LPR*CPL for some LPR with CPL <= 4 the mapping is exact (the largest
// such LPR); otherwise PAD: LPR = 64, CPL = ceil(n/64), and a step past the end
// of the row re-reads the row's last chunk with zero weights, which appends
// exact zeros to the end of that lane's chain.  The mapping depends on the row
// width alone, so every kernel that reduces rows of one width adds in one order.
template <int LPR_, int CPL_, bool PAD_>
struct LaneMap {
    static constexpr int LPR = LPR_;
    static constexpr int CPL = CPL_;
    static constexpr bool PAD = PAD_;
    static_assert(LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "lanes per row");
    static_assert(CPL >= 1 && CPL <= 4, "chunks per lane");
    static_assert(!PAD || LPR == 64, "a padded row takes a whole wave");
};
// the mapping used where a kernel instance has no down-projection rows
using NoLaneMap = LaneMap<64, 1, false>;

template <class LM>
__device__ __forceinline__ int lm_chunk(int c, int cl, int n)
{
    const int q = c * LM::LPR + cl;
    if constexpr (LM::PAD) return q < n ? q : n - 1;
    return q;
}

template <class LM>
__device__ __forceinline__ f16x8 lm_weights(f16x8 w, int c, int cl, int n)
{
    if constexpr (LM::PAD) {
        const f16x8 zero = {};
        return c * LM::LPR + cl < n ? w : zero;
    }
    return w;
}

// ---------------------------------------------------------------- router GEMV
// One wave, expert row e: logits[m, e] = sum_h Wr[e, h] x[m, h] for m < M.
template <int HC>
__device__ __forceinline__ void router_row(const f16 *__restrict__ x,
                                           const f16 *__restrict__ wr, int M, int E, int e,
                                           float *__restrict__ logits)
{
    constexpr int H = 512 * HC;
    f16x8 w[HC];
    load_row<HC>(wr + (size_t)e * H, w);
    for (int m = 0; m < M; ++m) {
        f16x8 xv[HC];
        load_x<HC>(x + (size_t)m * H, xv);
        const float t = row_dot<HC>(w, xv);
        if (lane_id() == 0) logits[(size_t)m * E + e] = t;
    }
}

template <int HC>
__global__ __launch_bounds__(kWave) void k_router(const f16 *__restrict__ x,
                                                  const f16 *__restrict__ wr, int M, int E,
                                                  float *__restrict__ logits)
{
    router_row<HC>(x, wr, M, E, blockIdx.x, logits);
}

// ---------------------------------------------------------------- top-k kernels
template <int NPL>
__global__ __launch_bounds__(kWave) void k_topk(const float *__restrict__ logits, int E, int K,
                                                int renormalize, int32_t *__restrict__ ids,
                                                float *__restrict__ weights)
{
    const int m = blockIdx.x;
    const int lane = lane_id();
    const float *L = logits + (size_t)m * E;
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) v[i] = i * kWave + lane < E ? L[i * kWave + lane] : 0.0f;
    int my_id;
    float my_l;
    const float lmax = wave_topk_vals<NPL>(v, E, K, my_id, my_l);
    const float w = topk_weight_vals<NPL>(v, E, K, renormalize, my_l, lmax);
    if (lane < K) {
        ids[(size_t)m * K + lane] = my_id;
        weights[(size_t)m * K + lane] = w;
    }
}

// The top-k kernel's work on logits that arrive as P partial sums over slices
// of H (part[p][M*E], the many-token router's output): each logit is summed
// p = 0, 1, ..., P-1 in that order and written to logits, then token m's
// experts are selected and weighted exactly as k_topk does.
template <int NPL>
__global__ __launch_bounds__(kWave) void k_topk_sum(const float *__restrict__ part, int P, int M,
                                                    int E, int K, int renormalize,
                                                    float *__restrict__ logits,
                                                    int32_t *__restrict__ ids,
                                                    float *__restrict__ weights)
{
    const int m = blockIdx.x;
    const int lane = lane_id();
    const size_t n = (size_t)M * E;
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = i * kWave + lane;
        v[i] = 0.0f;
        if (e < E) {
            const size_t o = (size_t)m * E + e;
            float t = part[o];
            for (int p = 1; p < P; ++p) t += part[(size_t)p * n + o];
            v[i] = t;
            logits[o] = t;
        }
    }
    int my_id;
    float my_l;
    const float lmax = wave_topk_vals<NPL>(v, E, K, my_id, my_l);
    const float w = topk_weight_vals<NPL>(v, E, K, renormalize, my_l, lmax);
    if (lane < K) {
        ids[(size_t)m * K + lane] = my_id;
        weights[(size_t)m * K + lane] = w;
    }
}

// Slot (top-k index) of token m in distinct-expert entry u: the entry's 8
// slot bytes are read with one 8-byte load at a uniform address, which the
// compiler issues as a scalar load.  (Reading the byte alone becomes a vector
// byte load, and waiting for it also waits for every weight load in flight.)
__device__ __forceinline__ int table_slot(const GroupTable *__restrict__ table, int u, int m)
{
    const uint64_t row = *reinterpret_cast<const uint64_t *>(table->u_slot[u]);
    return (int)(signed char)(uint8_t)(row >> (8 * m));
}

// ---------------------------------------------------------------- W13 + SiLU
// One wave per (expert, row pair j): gate row j and up row I + j of that
// expert, read in place at W13 + expert*(2I*H).  Both rows are loaded before
// any arithmetic (2*HC 16-byte loads in flight per lane); for every token that
// routes to the expert, gate and up dot products are reduced across the wave
// and activated = silu(gate) * up is stored (fp32) at act[m, slot, j].
//
// SHARED: the shared expert (one "expert" at `w13`, every token, slot 0).
template <int HC, bool SHARED>
__global__ __launch_bounds__(kBlock) void k_w13_silu(const f16 *__restrict__ x,
                                                     const f16 *__restrict__ w13,
                                                     const int32_t *__restrict__ ids, int I,
                                                     float *__restrict__ act)
{
    constexpr int H = 512 * HC;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int blocks_per_expert = I / kWavesPerBlock;
    const int u = blockIdx.x / blocks_per_expert;
    const int j = (blockIdx.x % blocks_per_expert) * kWavesPerBlock + wave;
    const int expert = SHARED ? 0 : ids[u];

    // x first (L2-resident, shared by every wave), then the two weight rows
    const f16 *base = w13 + (size_t)expert * 2 * I * H;
    const f16x8 *grow = reinterpret_cast<const f16x8 *>(base + (size_t)j * H);
    const f16x8 *urow = reinterpret_cast<const f16x8 *>(base + (size_t)(I + j) * H);
    f16x8 xv[HC], wg[HC], wu[HC];
    load_x<HC>(x, xv);
#pragma unroll
    for (int c = 0; c < HC; ++c) {
        wg[c] = stream_load(grow + c * kWave + lane);
        wu[c] = stream_load(urow + c * kWave + lane);
    }
    const float g = row_dot<HC>(wg, xv);
    const float up = row_dot<HC>(wu, xv);
    if (lane == 0) act[(size_t)(SHARED ? 0 : u) * I + j] = silu_mul(g, up);
}

// The same for M > 1 tokens.  The distinct selected experts U (with each
// one's token mask and slots) come from the group table; a workgroup takes
// expert u and R row pairs per wave (rows j0 + i*4, the next pair's loads
// issued before the current pair's arithmetic).  x [M, H] is staged in LDS
// once per workgroup; for every token that routes to the expert:
// act[m, slot, j] = silu(gate . x_m) * (up . x_m), the single-token arithmetic.
// SHARED: the shared expert (every token, slot 0, one "expert" at w13).
// Row pairs per wave R: the shared expert one (its single expert still spreads
// over the chip); routed experts 4 at 3..4 tokens and 2 otherwise (measured in
// one process with the replays interleaved: 4 pairs against 2 give M = 2
// 27.74 / 27.50, M = 4 43.92 / 45.77, M = 8 76.96 / 75.56 µs per layer).
template <bool SHARED, int MT>
constexpr int rows_per_wave_m() { return SHARED ? 1 : MT == 4 ? 4 : 2; }

// Workgroup b's row pairs of `expert` (xs: LDS for x, MT*HC*64 chunks).  The
// row pairs and x are requested first; then mid(mask, slot) gives the tokens
// routed to the expert and their slots (it may hold barriers: every thread of
// the workgroup calls it), so that they can still be worked out while the
// rows are in flight; then x is staged and the products computed.
template <int HC, int MT, bool SHARED, class Mid>
__device__ __forceinline__ void w13_multi_rows(const f16 *__restrict__ x,
                                               const f16 *__restrict__ w13, int M, int I, int K,
                                               float *__restrict__ act, int expert, int b,
                                               f16x8 *xs, Mid &&mid)
{
    constexpr int H = 512 * HC;
    constexpr int kRowsPerWaveM = rows_per_wave_m<SHARED, MT>();
    constexpr int kRowsPerBlockM = kRowsPerWaveM * kWavesPerBlock;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int bpe = I / kRowsPerBlockM;
    const int j0 = (b % bpe) * kRowsPerBlockM + wave;
    const f16 *base = w13 + (size_t)expert * 2 * I * H;
    constexpr int D = kRowsPerWaveM < 2 ? kRowsPerWaveM : 2; // row pairs in flight
    f16x8 wg[D][HC], wu[D][HC];
    auto load_pair = [&](int i, int buf) {
        const int j = j0 + i * kWavesPerBlock;
        const f16x8 *grow = reinterpret_cast<const f16x8 *>(base + (size_t)j * H);
        const f16x8 *urow = reinterpret_cast<const f16x8 *>(base + (size_t)(I + j) * H);
#pragma unroll
        for (int c = 0; c < HC; ++c) {
            wg[buf][c] = stream_load(grow + c * kWave + lane);
            wu[buf][c] = stream_load(urow + c * kWave + lane);
        }
    };
    // x is requested before the first row pair and stored to LDS
    // unconditionally (past the end, the last chunk's own value again): a
    // wave's vector loads complete in issue order, so staging requested after
    // the pair, or stored under a branch, would wait for the whole pair.
    constexpr int kPer = (MT * HC * kWave + kBlock - 1) / kBlock; // 16-byte chunks per thread
    const int n16 = M * HC * kWave;
    const f16x8 *x16 = reinterpret_cast<const f16x8 *>(x);
    f16x8 st[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int q = threadIdx.x + i * kBlock;
        st[i] = x16[q < n16 ? q : n16 - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int PRE = D > 1 ? D - 1 : 1; // row pairs requested before the staging stores
#pragma unroll
    for (int p = 0; p < PRE; ++p) load_pair(p, p % D);
    __builtin_amdgcn_sched_barrier(0);
    unsigned mask;
    int slot[MT];
    mid(mask, slot);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int q = threadIdx.x + i * kBlock;
        xs[q < n16 ? q : n16 - 1] = st[i];
    }
    __syncthreads();

    // Results stay in registers until every row pair is consumed: a store
    // under the token-mask branch would leave the compiler unsure how many
    // memory operations are outstanding, and it would then wait for all of
    // them (the prefetched row pair included) before the next product.
    float res[kRowsPerWaveM][MT];
#pragma unroll
    for (int i = 0; i < kRowsPerWaveM; ++i) {
        const int buf = i % D;
        if (i + D - 1 >= PRE && i + D - 1 < kRowsPerWaveM) load_pair(i + D - 1, (i + D - 1) % D);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            res[i][m] = 0.0f;
            if (mask & (1u << m)) {
                f16x8 xv[HC];
#pragma unroll
                for (int c = 0; c < HC; ++c) xv[c] = xs[(m * HC + c) * kWave + lane];
                const float g = row_dot<HC>(wg[buf], xv);
                const float up = row_dot<HC>(wu[buf], xv);
                res[i][m] = silu_mul(g, up);
            }
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kRowsPerWaveM; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (mask & (1u << m))
                    act[((size_t)m * K + slot[m]) * I + j0 + i * kWavesPerBlock] = res[i][m];
    }
}

// Workgroup b of the multi-token W13 work: distinct expert u = b / (blocks
// per expert) of the group table (SHARED: the shared expert, every token).
template <int HC, int MT, bool SHARED>
__device__ __forceinline__ void w13_multi_block(const f16 *__restrict__ x,
                                                const f16 *__restrict__ w13, int M, int I, int K,
                                                float *__restrict__ act,
                                                const GroupTable *__restrict__ table, int b,
                                                f16x8 *xs)
{
    constexpr int kRowsPerBlockM = rows_per_wave_m<SHARED, MT>() * kWavesPerBlock;
    const int u = b / (I / kRowsPerBlockM);
    int expert;
    unsigned mask;
    int slot[MT];
    if (SHARED) {
        expert = 0;
        mask = (1u << M) - 1u;
#pragma unroll
        for (int m = 0; m < MT; ++m) slot[m] = 0;
    } else {
        if (u >= table->n_u) return; // fewer distinct experts than slots: nothing to do
        expert = table->u_expert[u];
        mask = table->u_mask[u];
#pragma unroll
        for (int m = 0; m < MT; ++m) slot[m] = table_slot(table, u, m);
    }
    w13_multi_rows<HC, MT, SHARED>(x, w13, M, I, K, act, expert, b, xs,
                                   [&](unsigned &mk, int (&sl)[MT]) {
                                       mk = mask;
#pragma unroll
                                       for (int m = 0; m < MT; ++m) sl[m] = slot[m];
                                   });
}

template <int HC, int MT, bool SHARED>
__global__ __launch_bounds__(kBlock) void k_w13_multi(const f16 *__restrict__ x,
                                                      const f16 *__restrict__ w13, int M, int I,
                                                      int K, float *__restrict__ act,
                                                      const GroupTable *__restrict__ table)
{
    __shared__ f16x8 xs[MT * HC * kWave];
    w13_multi_block<HC, MT, SHARED>(x, w13, M, I, K, act, table, blockIdx.x, xs);
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
template <class LM, int MT, bool SHARED>
__global__ __launch_bounds__(kBlock) void k_w2_combine(
    const float *__restrict__ act, const f16 *__restrict__ w2, const int32_t *__restrict__ ids,
    const float *__restrict__ topk_w, const float *__restrict__ shared_in, int M, int H, int I,
    int K, const GroupTable *__restrict__ table, void *__restrict__ out)
{
    constexpr int LPR = LM::LPR;
    constexpr int CPL = LM::CPL;
    constexpr int RPL = kWave / LPR;
    const int nch = I / 8;
    constexpr int BATCH = 8;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int r = lane / LPR;
    const int cl = lane % LPR;
    const int h = (blockIdx.x * kWavesPerBlock + wave) * RPL + r;
    float s_row[MT];
    load_column<MT>(SHARED ? nullptr : shared_in, M, H, h, s_row);

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
                for (int c = 0; c < CPL; ++c)
                    wv[t][c] = lm_weights<LM>(stream_load(row + lm_chunk<LM>(c, cl, nch)), c, cl, nch);
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
                        else k = table_slot(table, u0 + t, m);
                        const float wt = SHARED ? 1.0f : topk_w[(size_t)m * K + k];
                        const float *a = act + ((size_t)m * (SHARED ? 1 : K) + k) * I;
                        float d = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c) {
                            const f32x4 *ap = reinterpret_cast<const f32x4 *>(a + lm_chunk<LM>(c, cl, nch) * 8);
                            d = dot8_f32(wv[t][c], ap[0], ap[1], d);
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
                const float v = shared_in ? t + s_row[m] : t;
                static_cast<f16 *>(out)[o] = (f16)v;
            }
        }
    }
}


// ---------------------------------------------------------------- W2 + combine, several tokens
// The W2 kernel's work and arithmetic for M > 1, with the activations [M, K,
// I] (or the shared expert's [M, Is]) staged in LDS once per workgroup of
// kSWaves waves instead of every lane fetching its chunks of every (token,
// slot) pair from L2 inside the combine loop.  The first batch of W2 rows is
// requested right after the staging loads, and every later batch before the
// previous one is combined (experts still in order of first appearance).
constexpr int kSWaves = 8;
// shared down blocks that each of token 0's workgroups takes in the M <= 4
// expand launch at most (the benched sizes: 1 at M = 2, 2 at M = 4)
constexpr int kSharedPerTok0 = 4;
constexpr int kSBlock = kSWaves * kWave;

template <class LM, int MT, bool SHARED>
__global__ __launch_bounds__(kSBlock) void k_w2_staged(
    const float *__restrict__ act, const f16 *__restrict__ w2, const float *__restrict__ topk_w,
    const float *__restrict__ shared_in, int M, int H, int I, int K,
    const GroupTable *__restrict__ table, void *__restrict__ out)
{
    extern __shared__ float lds[];
    constexpr int LPR = LM::LPR;
    constexpr int CPL = LM::CPL;
    constexpr int RPL = kWave / LPR;
    const int nch = I / 8;
    // experts per buffer: 2 at CPL = 1, else 1 (2 or more 16-byte chunks per
    // lane).  Two buffers keep at most 4 experts' rows in flight per wave: in
    // one process with the replays interleaved, batches of 2 / 4 / 8 experts
    // give M = 8 70.3 / 72.1 / 73.5, M = 4 39.8 / 40.1 / 41.7 us per layer
    // (1 expert: 74.2 and 41.5), so fewer experts read at once stream faster.
    constexpr int BATCH = CPL == 1 ? 2 : 1;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int r = lane / LPR;
    const int cl = lane % LPR;
    const int h = (blockIdx.x * kSWaves + wave) * RPL + r;
    const int slots = SHARED ? 1 : K;
    float s_row[MT];
    load_column<MT>(SHARED ? nullptr : shared_in, M, H, h, s_row);
    const int n_u = SHARED ? 1 : table->n_u;

    // two batches of W2 rows: the next batch is requested before the current
    // one is combined.  Every load is issued (none under a branch, so the
    // compiler waits for exactly the batch it combines): a slot past the last
    // distinct expert reads through a zero-sized buffer range, which returns
    // zeros and touches no memory.  Each batch's expert ids are read with it
    // (scalar loads at uniform addresses); the token masks and slot bytes the
    // combine needs are staged in LDS with the activations, so the combine
    // waits on nothing but its batch.
    f16x8 wv[2][BATCH][CPL];
    auto load_batch = [&](int buf, int u0) {
        const int ub = u0 < kMaxSlots - BATCH ? u0 : kMaxSlots - BATCH; // entries stay in the table
        int ids[BATCH];
#pragma unroll
        for (int t = 0; t < BATCH; ++t) ids[t] = SHARED ? 0 : table->u_expert[ub + t];
#pragma unroll
        for (int t = 0; t < BATCH; ++t) {
            const bool ok = u0 + t < n_u;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<f16 *>(w2) + (size_t)(ok ? ids[t] : 0) * H * I, (short)0,
                ok ? H * I * 2 : 0, kBufferWord3);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                wv[buf][t][c] = lm_weights<LM>(
                    __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs, (uint32_t)(h * I + lm_chunk<LM>(c, cl, nch) * 8) * 2,
                                                  0, kLoadNT)),
                    c, cl, nch);
        }
    };
    // A wave's vector loads complete in issue order, so what is staged in LDS
    // is requested before the first W2 batch: the routing weights [M, K], the
    // distinct experts' token masks and slot bytes (read per expert and token
    // by the combine; entry indices past the end re-read the last entry), and
    // the first kSReg 16-byte chunks per thread of the activations.  The LDS
    // stores are unconditional (past the end, the last element's own value
    // again): a store under a branch would pull its load behind the batch.
    static_assert(kSBlock >= kMaxSlots, "one table entry per thread");
    constexpr int kSReg = 2 * MT; // covers K*I <= 4096 in one pass
    const int ti = (int)threadIdx.x < kMaxSlots ? (int)threadIdx.x : kMaxSlots - 1;
    float tw_r = 0.0f;
    unsigned mask_r = 0u;
    uint64_t slot_r = 0u;
    if constexpr (!SHARED) {
        tw_r = topk_w[ti < M * K ? ti : M * K - 1];
        mask_r = table->u_mask[ti];
        slot_r = *reinterpret_cast<const uint64_t *>(table->u_slot[ti]);
    }
    const int n4 = M * slots * I / 4;
    // every workgroup copies the same M*K*I activations; in the rotated
    // order, M = 8 69.43 -> 69.13 and M = 4 39.44 -> 39.36 us per layer (one
    // process, replays interleaved; the M = 1 reduce kernel's 16 KB copy
    // measured 0.03 us slower that way and keeps the plain order)
    const int rot = stage_rotation(n4);
    const f32x4 *a4 = reinterpret_cast<const f32x4 *>(act);
    f32x4 *l4 = reinterpret_cast<f32x4 *>(lds);
    f32x4 st0[kSReg];
#pragma unroll
    for (int i = 0; i < kSReg; ++i)
        st0[i] = a4[staged_chunk(threadIdx.x + i * kSBlock, n4, rot)];
    // the rest of act (K*I > 4096): 16-byte chunks, 4 in flight per thread
    // per step, staged before the first batch is requested (so that no load
    // of this loop is still outstanding once the batches are)
    for (int q0 = kSReg * kSBlock; q0 < n4; q0 += 4 * kSBlock) {
        f32x4 st[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st[i] = a4[staged_chunk(q0 + threadIdx.x + i * kSBlock, n4, rot)];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = q0 + threadIdx.x + i * kSBlock;
            if (q < n4) l4[staged_chunk(q, n4, rot)] = st[i];
        }
    }
    // keep the batch's loads together, after the staging loads and ahead of
    // the LDS stores (which wait)
    __builtin_amdgcn_sched_barrier(0);
    load_batch(0, 0);
    __builtin_amdgcn_sched_barrier(0);

    __shared__ float s_tw[kMaxSlots];
    __shared__ unsigned s_mask[kMaxSlots];
    __shared__ uint64_t s_slot[kMaxSlots];
    if constexpr (!SHARED) {
        s_tw[ti] = tw_r;
        s_mask[ti] = mask_r;
        s_slot[ti] = slot_r;
    }
#pragma unroll
    for (int i = 0; i < kSReg; ++i)
        l4[staged_chunk(threadIdx.x + i * kSBlock, n4, rot)] = st0[i];
    __syncthreads();

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    auto combine = [&](int buf, int u0) {
        const int cnt = n_u - u0 < BATCH ? n_u - u0 : BATCH;
#pragma unroll
        for (int t = 0; t < BATCH; ++t)
            if (t < cnt) {
                const unsigned mask = SHARED ? (1u << M) - 1u : s_mask[u0 + t];
                const uint64_t slot8 = SHARED ? 0 : s_slot[u0 + t];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (mask & (1u << m)) {
                        const int k = (int)(signed char)(uint8_t)(slot8 >> (8 * m));
                        const float wt = SHARED ? 1.0f : s_tw[m * K + k];
                        const float *a = lds + ((size_t)m * slots + k) * I;
                        float d = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c) {
                            const f32x4 *ap = reinterpret_cast<const f32x4 *>(a + lm_chunk<LM>(c, cl, nch) * 8);
                            d = dot8_f32(wv[buf][t][c], ap[0], ap[1], d);
                        }
                        acc[m] = fmaf(wt, d, acc[m]);
                    }
            }
    };
    for (int u0 = 0; u0 < n_u; u0 += 2 * BATCH) {
        load_batch(1, u0 + BATCH);
        combine(0, u0);
        load_batch(0, u0 + 2 * BATCH);
        combine(1, u0 + BATCH);
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
                const float v = shared_in ? t + s_row[m] : t;
                static_cast<f16 *>(out)[o] = (f16)v;
            }
        }
    }
}

// ---------------------------------------------------------------- layer path (M = 1)
// Three launches for a whole layer at M = 1, plain grids of independent
// workgroups (the kernel boundaries are the only hand-offs):
//   k_router1        router rows -> logits, one single-wave workgroup per row
//   k_expand         each routed workgroup selects the experts from the logits
//                    itself, then its gate/up rows of the selected expert ->
//                    activations; the shared gate/up rows -> SiLU*mul
//                    activations (routing-independent bytes that stream while
//                    the routed workgroups select)
//   k_reduce         routed down rows with the weighted combine, the shared
//                    down rows, the one fp16 rounding
// That placement needs the shared down projection to use the routed one's
// lane mapping (Is == I).  For any other shared width the shared gate/up rows
// stream beside the router (k_router_shared) and the shared down rows in
// k_expand (-> s, fp32), which k_reduce adds.
// The per-element arithmetic is the separate kernels' (the same device
// functions, lane mappings and reduction trees, in the same order), so the
// results equal shared_expert + moe_route + moe_decode_fused bit for bit.

// One single-wave workgroup per router row (the router kernel's arithmetic):
// a layer's router is latency-bound, and 256 small workgroups spread its rows
// over every CU.
template <int HC>
__global__ __launch_bounds__(kWave) void k_router1(const f16 *__restrict__ x,
                                                   const f16 *__restrict__ wr,
                                                   float *__restrict__ logits)
{
    constexpr int H = 512 * HC;
    const int e = blockIdx.x;
    f16x8 w[HC], xv[HC];
    load_row<HC>(wr + (size_t)e * H, w);
    load_x<HC>(x, xv);
    const float t = row_dot<HC>(w, xv);
    if (lane_id() == 0) logits[e] = t;
}

// Workgroups [0, ceil(E/4)): one wave per router row (the router kernel's
// arithmetic); the rest: one wave per shared gate/up row pair.
template <int HC>
__global__ __launch_bounds__(kBlock) void k_router_shared(const f16 *__restrict__ x,
                                                          const f16 *__restrict__ wr,
                                                          const f16 *__restrict__ wsgu, int E,
                                                          int Is, float *__restrict__ logits,
                                                          float *__restrict__ act_s)
{
    constexpr int H = 512 * HC;
    const int wave = threadIdx.x / kWave;
    const int router_blocks = (E + kWavesPerBlock - 1) / kWavesPerBlock;
    if ((int)blockIdx.x < router_blocks) {
        const int e = blockIdx.x * kWavesPerBlock + wave;
        if (e >= E) return;
        f16x8 w[HC], xv[HC];
        load_row<HC>(wr + (size_t)e * H, w);
        load_x<HC>(x, xv);
        const float t = row_dot<HC>(w, xv);
        if (lane_id() == 0) logits[e] = t;
    } else {
        const int j = (blockIdx.x - router_blocks) * kWavesPerBlock + wave;
        const float a = w13_pair<HC>(x, wsgu, Is, j);
        if (lane_id() == 0) act_s[j] = a;
    }
}

// Wave wi of the shared down projection: rows h = wi*RPL + r (RPL = 64/LPR)
// for every token, the W2 kernel's arithmetic with weight 1: s[m, h] in fp32.
template <class LM, int MT>
__device__ __forceinline__ void shared_down_rows(const f16 *__restrict__ wsd,
                                                 const float *__restrict__ act_s, int M, int H,
                                                 int Is, int wi, float *__restrict__ s_out)
{
    constexpr int LPR = LM::LPR;
    constexpr int CPL = LM::CPL;
    constexpr int RPL = kWave / LPR;
    const int lane = lane_id();
    const int r = lane / LPR;
    const int cl = lane % LPR;
    const int nch = Is / 8;
    const int h = wi * RPL + r;
    const f16x8 *row = reinterpret_cast<const f16x8 *>(wsd + (size_t)h * Is);
    f16x8 wv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        wv[c] = lm_weights<LM>(stream_load(row + lm_chunk<LM>(c, cl, nch)), c, cl, nch);
    const bool holder = lane == group_holder<LPR>(r);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float d = 0.0f;
        if (m < M) {
            const float *am = act_s + (size_t)m * Is;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const f32x4 *ap = reinterpret_cast<const f32x4 *>(am + lm_chunk<LM>(c, cl, nch) * 8);
                d = dot8_f32(wv[c], ap[0], ap[1], d);
            }
        }
        const float t = group_sum<LPR>(fmaf(1.0f, d, 0.0f));
        if (m < M && holder) s_out[(size_t)m * H + h] = t;
    }
}

// shared_down_rows for a whole workgroup of shared-down waves (wave wi0 + w),
// with the shared activations [M, Is] staged once in the workgroup's LDS
// (`stage`, NS 16-byte chunks) instead of every wave reading all of them from
// L2; the same arithmetic on the same values.  With M*Is/4 > NS chunks it
// falls back to per-wave loads.  Every thread of the workgroup must call it.
// (At M = 8, I = Is = 512 the per-wave reads were 32 MB of L2 traffic per
// layer for 2 MB of shared down rows; staged, M = 2 / 4 / 8 measured 23.89 /
// 38.66 / 67.66 -> 23.84 / 38.48 / 67.52 us per layer, replays interleaved.)
template <class LM, int MT, int NS>
__device__ __forceinline__ void shared_down_block(const f16 *__restrict__ wsd,
                                                  const float *__restrict__ act_s, int M, int H,
                                                  int Is, int wi0, float *__restrict__ s_out,
                                                  f32x4 *stage)
{
    const int n4 = M * Is / 4;
    if (n4 > NS) {
        shared_down_rows<LM, MT>(wsd, act_s, M, H, Is, wi0 + threadIdx.x / kWave, s_out);
        return;
    }
    constexpr int LPR = LM::LPR;
    constexpr int CPL = LM::CPL;
    constexpr int RPL = kWave / LPR;
    const int lane = lane_id();
    const int r = lane / LPR;
    const int cl = lane % LPR;
    const int nch = Is / 8;
    const int h = (wi0 + (int)(threadIdx.x / kWave)) * RPL + r;
    const f16x8 *row = reinterpret_cast<const f16x8 *>(wsd + (size_t)h * Is);
    f16x8 wv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        wv[c] = lm_weights<LM>(stream_load(row + lm_chunk<LM>(c, cl, nch)), c, cl, nch);
    // the row first, then the staging loads (stores unconditional: past the
    // end, the last chunk's own value again)
    constexpr int kPer = (NS + kBlock - 1) / kBlock;
    const f32x4 *a4 = reinterpret_cast<const f32x4 *>(act_s);
    f32x4 st[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int q = threadIdx.x + i * kBlock;
        st[i] = a4[q < n4 ? q : n4 - 1];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int q = threadIdx.x + i * kBlock;
        stage[q < n4 ? q : n4 - 1] = st[i];
    }
    __syncthreads();
    const float *ls = reinterpret_cast<const float *>(stage);
    const bool holder = lane == group_holder<LPR>(r);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float d = 0.0f;
        if (m < M) {
            const float *am = ls + (size_t)m * Is;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const f32x4 *ap = reinterpret_cast<const f32x4 *>(am + lm_chunk<LM>(c, cl, nch) * 8);
                d = dot8_f32(wv[c], ap[0], ap[1], d);
            }
        }
        const float t = group_sum<LPR>(fmaf(1.0f, d, 0.0f));
        if (m < M && holder) s_out[(size_t)m * H + h] = t;
    }
}

// Shared-expert work placed in the expand launch.
enum : int { kExpandNoShared = 0, kExpandSharedDown = 1, kExpandSharedGateUp = 2 };

// Routed workgroups [0, K*I/4) take (slot u, row pair j).  Wave 0 selects
// from the logits only as far as it needs: u + 1 rounds of the top-k give slot
// u's expert (the rounds are the top-k kernel's), so the workgroups of early
// slots start streaming sooner.  The first workgroup of the last slot runs all
// K rounds and also writes ids and weights (the top-k kernel's arithmetic).
// The workgroups after them (SM):
//   kExpandSharedGateUp  one wave per shared gate/up row pair (wsh = the
//                        shared gate/up weights) -> act_s;
//   kExpandSharedDown    one wave per RPL = 64/LPR rows of the shared down
//                        projection (wsh = the shared down weights; the W2
//                        kernel's arithmetic with weight 1) -> s (fp32).
template <int HC, int NPL, class LM, int SM>
__global__ __launch_bounds__(kBlock) void k_expand(
    const f16 *__restrict__ x, const f16 *__restrict__ w13, const f16 *__restrict__ wsh,
    const float *__restrict__ logits, float *__restrict__ act_s, int E, int I, int K, int Is,
    int renormalize, int32_t *__restrict__ ids, float *__restrict__ weights,
    float *__restrict__ act, float *__restrict__ s_out)
{
    constexpr int H = 512 * HC;
    __shared__ int sh_id;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int routed_blocks = K * (I / kWavesPerBlock);
    const int b = blockIdx.x;
    if (b < routed_blocks) {
        const int per_expert = I / kWavesPerBlock;
        const int u = b / per_expert;
        if (wave == 0) {
            float v[NPL];
#pragma unroll
            for (int i = 0; i < NPL; ++i) v[i] = i * kWave + lane < E ? logits[i * kWave + lane] : 0.0f;
            const bool writer = u == K - 1 && b % per_expert == 0;
            int my_id;
            float my_l;
            const float lmax = wave_topk_vals<NPL>(v, E, writer ? K : u + 1, my_id, my_l);
            if (lane == u) sh_id = my_id;
            if (writer) {
                const float w = topk_weight_vals<NPL>(v, E, K, renormalize, my_l, lmax);
                if (lane < K) {
                    ids[lane] = my_id;
                    weights[lane] = w;
                }
            }
        }
        __syncthreads();
        const int j = (b % per_expert) * kWavesPerBlock + wave;
        const float a = w13_pair<HC>(x, w13 + (size_t)sh_id * 2 * I * H, I, j);
        if (lane == 0) act[(size_t)u * I + j] = a;
    } else if constexpr (SM == kExpandSharedGateUp) {
        const int j = (b - routed_blocks) * kWavesPerBlock + wave;
        const float a = w13_pair<HC>(x, wsh, Is, j);
        if (lane == 0) act_s[j] = a;
    } else if constexpr (SM == kExpandSharedDown) {
        shared_down_rows<LM, 1>(wsh, act_s, 1, 512 * HC, Is,
                                (b - routed_blocks) * kWavesPerBlock + wave, s_out);
    }
}

// Routed down projections and the combine, RW = LPR/8 waves per workgroup, so
// that a workgroup always covers 8 rows of H (H/8 workgroups: one per CU at
// H = 2048, whatever the row width).  Each wave owns RPL = 64/LPR rows h, LPR lanes per row with CPL 16-byte chunks each (I = 8*LPR*CPL).  The wave
// requests the ids and weights and its share of the activations [K*I], then
// its W2 rows for up to 8/CPL experts; the workgroup stages the activations in
// LDS while the rows arrive, then every lane accumulates as the W2 kernel
// does: acc += w[k] * (its part of row h of W2[e_k] . act_k), experts in
// routing order; one group reduction; y = fp16(acc + s[h]).
// SH: the shared down projection is computed here too (Is == I, so its rows
// use the same lane mapping): s[h] = the W2 kernel's arithmetic with weight 1
// over row h of the shared down weights and act_s, added as s_in would be.
constexpr int kRRows = 8; // rows of H per workgroup
template <class LM>
constexpr int reduce_waves() { return LM::LPR / 8; }
[[maybe_unused]] constexpr int kMaxStaged = 16384; // K*I fp32 values staged in LDS (64 KB)

// STAGE: 16-byte activation loads per thread, ceil(K*I / (4 * 64 * RW)).
template <class LM, int STAGE, bool SH>
__global__ __launch_bounds__(reduce_waves<LM>() * kWave) void k_reduce(const float *__restrict__ act,
                                                    const f16 *__restrict__ w2,
                                                    const int32_t *__restrict__ ids,
                                                    const float *__restrict__ tw,
                                                    const float *__restrict__ s_in,
                                                    const f16 *__restrict__ wsd,
                                                    const float *__restrict__ act_s, int H,
                                                    int I, int K, f16 *__restrict__ y)
{
    extern __shared__ float lds[]; // [K*I] routed activations
    // K >= 1 (checked on the host); stated so that the compiler keeps the
    // first batch of loads ahead of the staging barrier
    __builtin_assume(K > 0);
    constexpr int LPR = LM::LPR;
    constexpr int CPL = LM::CPL;
    constexpr int RPL = kWave / LPR;
    constexpr int BATCH = 8 / CPL;
    constexpr int kRWaves = reduce_waves<LM>();
    constexpr int kRBlock = kRWaves * kWave;
    const int nch = I / 8;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int r = lane / LPR;
    const int cl = lane % LPR;
    const int h = (blockIdx.x * kRWaves + wave) * RPL + r;

    // Everything this wave reads is requested up front, in the order it is
    // needed: a wave's vector loads complete in issue order, so a wait for one
    // load also waits for every load issued before it.  First ids and weights
    // (lane k holds slot k) and s[h]; then the activations to stage (indices
    // past the end re-read the last chunk); then, with SH, the shared down row
    // and act_s; and after the ids are in, the W2 rows of a whole batch.
    // Batch slots past K reload the last expert's row (a cache hit, unused),
    // so the loads need no branches.
    const int my_id = lane < K ? ids[lane] : 0;
    const float my_tw = lane < K ? tw[lane] : 0.0f;
    const float s_h = !SH && s_in ? s_in[h] : 0.0f;
    const int n4 = K * I / 4;
    f32x4 st[STAGE];
    {
        const f32x4 *a4 = reinterpret_cast<const f32x4 *>(act);
#pragma unroll
        for (int i = 0; i < STAGE; ++i) {
            const int q = threadIdx.x + i * kRBlock;
            st[i] = a4[q < n4 ? q : n4 - 1];
        }
    }
    f16x8 sv[CPL];
    f32x4 sa[2 * CPL];
    if constexpr (SH) {
        const f16x8 *srow = reinterpret_cast<const f16x8 *>(wsd + (size_t)h * I);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            sv[c] = lm_weights<LM>(stream_load(srow + lm_chunk<LM>(c, cl, nch)), c, cl, nch);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const f32x4 *ap = reinterpret_cast<const f32x4 *>(act_s + lm_chunk<LM>(c, cl, nch) * 8);
            sa[2 * c] = ap[0];
            sa[2 * c + 1] = ap[1];
        }
        // the shared row goes out before the wait for the ids
        __builtin_amdgcn_sched_barrier(0);
    }
    f16x8 wv[BATCH][CPL];
    auto load_batch = [&](int u0) {
#pragma unroll
        for (int t = 0; t < BATCH; ++t) {
            const int k = u0 + t < K ? u0 + t : K - 1;
            const int e = __builtin_amdgcn_readlane(my_id, k);
            const f16x8 *row = reinterpret_cast<const f16x8 *>(w2 + ((size_t)e * H + h) * I);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                wv[t][c] = lm_weights<LM>(stream_load(row + lm_chunk<LM>(c, cl, nch)), c, cl, nch);
        }
    };
    load_batch(0);
    // Stage act.  The store is unconditional (past the end, the last chunk
    // stores its own value again): a store under a branch would pull its
    // load into the branch, behind the W2 batch.
    f32x4 *l4 = reinterpret_cast<f32x4 *>(lds);
#pragma unroll
    for (int i = 0; i < STAGE; ++i) {
        const int q = threadIdx.x + i * kRBlock;
        l4[q < n4 ? q : n4 - 1] = st[i];
    }
    __syncthreads();

    // Per slot: d = this lane's part of row h of W2[e_k] . act_k; then
    // acc += w_k * d in routing order.  A full batch computes its BATCH
    // independent d first (no branches, so their chains interleave).
    auto slot_dot = [&](int t, int k) {
        const float *ak = lds + (size_t)k * I;
        float d = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const f32x4 *ap = reinterpret_cast<const f32x4 *>(ak + lm_chunk<LM>(c, cl, nch) * 8);
            d = dot8_f32(wv[t][c], ap[0], ap[1], d);
        }
        return d;
    };
    auto weight = [&](int k) {
        return __builtin_bit_cast(float,
                                  __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_tw), k));
    };
    float acc = 0.0f;
    for (int u0 = 0; u0 < K; u0 += BATCH) {
        if (u0 > 0) load_batch(u0);
        if (K - u0 >= BATCH) {
            float d[BATCH];
#pragma unroll
            for (int t = 0; t < BATCH; ++t) d[t] = slot_dot(t, u0 + t);
#pragma unroll
            for (int t = 0; t < BATCH; ++t) acc = fmaf(weight(u0 + t), d[t], acc);
        } else {
#pragma unroll
            for (int t = 0; t < BATCH; ++t)
                if (t < K - u0) acc = fmaf(weight(u0 + t), slot_dot(t, u0 + t), acc);
        }
    }
    float s_add = s_h;
    if constexpr (SH) {
        float d = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) d = dot8_f32(sv[c], sa[2 * c], sa[2 * c + 1], d);
        s_add = group_sum<LPR>(fmaf(1.0f, d, 0.0f));
    }
    const float t = group_sum<LPR>(acc);
    if (lane == group_holder<LPR>(r)) y[h] = (f16)(SH || s_in ? t + s_add : t);
}

// ---------------------------------------------------------------- grouping
// For M > 1 tokens: the distinct selected experts U, in order of first
// appearance scanning topk_ids row by row, with the tokens that use each one
// and the slot k at which each of those tokens selected it.  Threads
// [0, kGroupThreads) of a workgroup, thread i owning entry i = m*K + k (M*K <=
// 128): per expert, the smallest entry index selecting it (LDS atomic min),
// the token mask (atomic or) and the slot per token; an entry is a first
// appearance when it holds that minimum, and its rank in U is the number of
// first appearances before it.  Every thread of the workgroup must call it.
constexpr int kGroupThreads = 2 * kWave;

struct GroupScratch {
    int first_of[kMaxExperts];
    unsigned tokens_of[kMaxExperts];
    signed char slot_of[kMaxExperts][kMaxTokens];
    int n_first0;
};

__device__ __forceinline__ void build_group_table(const int32_t *ids, int M, int K, int E,
                                                  GroupTable *__restrict__ table,
                                                  GroupScratch &g)
{
    const int i = threadIdx.x;
    const int n = M * K;
    for (int e = i; e < E; e += blockDim.x) {
        g.first_of[e] = 0x7FFFFFFF;
        g.tokens_of[e] = 0u;
#pragma unroll
        for (int m = 0; m < kMaxTokens; ++m) g.slot_of[e][m] = 0;
    }
    __syncthreads();
    const bool mine = i < kGroupThreads && i < n;
    const int e = mine ? ids[i] : 0;
    if (mine) {
        const int m = i / K;
        atomicMin(&g.first_of[e], i);
        atomicOr(&g.tokens_of[e], 1u << m);
        g.slot_of[e][m] = (signed char)(i % K);
    }
    __syncthreads();
    const bool first = mine && g.first_of[e] == i;
    const uint64_t b = __ballot(first);
    const int lane = lane_id();
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    if (i == 0) g.n_first0 = __popcll(b);
    __syncthreads();
    const int rank = __popcll(b & below) + (i >= kWave ? g.n_first0 : 0);
    if (first) {
        table->u_expert[rank] = e;
        table->u_mask[rank] = g.tokens_of[e];
#pragma unroll
        for (int m = 0; m < kMaxTokens; ++m) table->u_slot[rank][m] = g.slot_of[e][m];
    }
    if (i == kWave) table->n_u = g.n_first0 + __popcll(b);
}

#if MOE_PART == 0 // kernels that are not templates live in the part that launches them
__global__ __launch_bounds__(kGroupThreads) void k_group_table(const int32_t *__restrict__ ids,
                                                               int M, int K, int E,
                                                               GroupTable *__restrict__ table)
{
    __shared__ GroupScratch g;
    build_group_table(ids, M, K, E, table, g);
}
#endif

// ---------------------------------------------------------------- layer path (M > 1)
// Four launches for a whole layer with 2..8 tokens, the multi-token kernels'
// arithmetic throughout (so the results equal the three calls bit for bit):
//   k_route_shared_m  router rows for every token; shared gate/up row pairs
//   k_select_m        one workgroup: every token's top-k, then the group table
//   k_expand_m        routed gate/up rows of the distinct experts; shared down
//   (the staged W2 kernel with the shared output added)

template <int HC, int MT>
__global__ __launch_bounds__(kBlock) void k_route_shared_m(const f16 *__restrict__ x,
                                                           const f16 *__restrict__ wr,
                                                           const f16 *__restrict__ wsgu, int M,
                                                           int E, int Is,
                                                           float *__restrict__ logits,
                                                           float *__restrict__ act_s)
{
    __shared__ f16x8 xs[MT * HC * kWave];
    const int router_blocks = (E + kWavesPerBlock - 1) / kWavesPerBlock;
    if ((int)blockIdx.x < router_blocks) {
        const int e = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
        if (e < E) router_row<HC>(x, wr, M, E, e, logits);
        return;
    }
    w13_multi_block<HC, MT, true>(x, wsgu, M, Is, 1, act_s, nullptr, blockIdx.x - router_blocks,
                                  xs);
}

constexpr int kSelBlock = kMaxTokens * kWave; // one wave per token

template <int NPL>
__global__ __launch_bounds__(kSelBlock) void k_select_m(const float *__restrict__ logits, int M,
                                                     int E, int K, int renormalize,
                                                     int32_t *__restrict__ ids,
                                                     float *__restrict__ weights,
                                                     GroupTable *__restrict__ table)
{
    __shared__ GroupScratch g;
    __shared__ int32_t sids[kMaxSlots];
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    for (int m = wave; m < M; m += kMaxTokens) { // the top-k kernel's work, token m
        const float *L = logits + (size_t)m * E;
        float v[NPL];
#pragma unroll
        for (int i = 0; i < NPL; ++i) v[i] = i * kWave + lane < E ? L[i * kWave + lane] : 0.0f;
        int my_id;
        float my_l;
        const float lmax = wave_topk_vals<NPL>(v, E, K, my_id, my_l);
        const float w = topk_weight_vals<NPL>(v, E, K, renormalize, my_l, lmax);
        if (lane < K) {
            ids[(size_t)m * K + lane] = my_id;
            weights[(size_t)m * K + lane] = w;
            sids[m * K + lane] = my_id;
        }
    }
    __syncthreads();
    build_group_table(sids, M, K, E, table, g);
}

// Routed workgroups: the multi-token W13 work.  Shared workgroups: RPL = 64/LPR
// rows of the shared down projection per wave for every token (the W2
// kernel's arithmetic with weight 1), s[m, h] in fp32.
template <int HC, int MT, class LM>
__global__ __launch_bounds__(kBlock) void k_expand_m(const f16 *__restrict__ x,
                                                     const f16 *__restrict__ w13,
                                                     const f16 *__restrict__ wsd,
                                                     const float *__restrict__ act_s, int M, int H,
                                                     int I, int K, int Is, int routed_blocks,
                                                     float *__restrict__ act,
                                                     float *__restrict__ s_out,
                                                     const GroupTable *__restrict__ table)
{
    __shared__ f16x8 xs[MT * HC * kWave];
    // the shared down workgroups come first in the grid, so that they start
    // with the routed stream instead of after it (dispatched last, each one's
    // row latency lengthened the launch's tail): M = 8 67.55 -> 66.55 us per
    // layer, replays interleaved
    const int b = ((int)blockIdx.x + routed_blocks) % (int)gridDim.x;
    if (b < routed_blocks) {
        w13_multi_block<HC, MT, false>(x, w13, M, I, K, act, table, b, xs);
        return;
    }
    shared_down_block<LM, MT, MT * HC * kWave>(wsd, act_s, M, H, Is,
                                               (b - routed_blocks) * kWavesPerBlock, s_out,
                                               reinterpret_cast<f32x4 *>(xs));
}

// k_expand_m with the selection folded in (M <= 4, one wave per token): every
// routed workgroup selects its expert itself, so the separate selection
// launch and its hand-off are gone.  The group table lists token 0's experts
// first, in routing order, so distinct expert u < K is token 0's u-th choice:
// its workgroups run u + 1 top-k rounds on token 0 (the top-k kernel's
// rounds), request their row pairs at once, and while the rows are in flight
// find every other token's place of that expert in its own top-k order
// (topk_rank), which gives the token mask and slots of the group table's
// entry u.  The workgroups of a later entry run every token's selection and
// build the group table in LDS (the same device functions as k_select_m)
// before they request their rows.  Workgroup 0 (entry 0) also runs the full
// selection while its rows are in flight and, after its products, writes
// ids, weights and the table that the W2 kernel reads.  After their rows, token
// 0's workgroups (which start first) also compute the shared down rows, the
// work of k_expand_m's shared workgroups with the same arithmetic, up to
// kSharedPerTok0 blocks each (beyond that, those workgroups run on their own
// in a launch of k_expand_m before this one).  As
// separate workgroups at the end of the grid they ran in a later round of
// resident workgroups and lengthened the launch: M = 2 23.89 -> 23.74 and
// M = 4 38.59 -> 38.37 us per layer with them folded in (replays
// interleaved).  First in the grid they delayed token 0's experts (M = 4
// 38.60 -> 38.77 us), and between those and the later entries too (M = 2
// 23.94 -> 24.34 us).  (At M = 8 each wave would select for two tokens in
// turn, and the selection launch is kept.)
template <int HC, int MT, class LM, int NPL>
__global__ __launch_bounds__(kBlock) void k_expand_sel_m(
    const f16 *__restrict__ x, const f16 *__restrict__ w13, const f16 *__restrict__ wsd,
    const float *__restrict__ act_s, const float *__restrict__ logits, int M, int H, int E, int I,
    int K, int Is, int renormalize, int routed_blocks, int32_t *__restrict__ ids,
    float *__restrict__ weights, float *__restrict__ act, float *__restrict__ s_out,
    GroupTable *__restrict__ table)
{
    static_assert(MT <= kWavesPerBlock, "one wave per token");
    __shared__ f16x8 xs[MT * HC * kWave];
    __shared__ GroupScratch g;
    __shared__ GroupTable tl;
    __shared__ int32_t sids[kMaxSlots];
    __shared__ int s_e;
    __shared__ int s_rank[MT];
    const int b = blockIdx.x;
    const int lane = lane_id();
    (void)routed_blocks; // every workgroup is a routed one
    const int wave = threadIdx.x / kWave;
    constexpr int kRowsPerBlockM = rows_per_wave_m<false, MT>() * kWavesPerBlock;
    const int u = b / (I / kRowsPerBlockM);
    // wave m < M: token m's logits and (key, id) pairs
    const bool tok = wave < M;
    float v[NPL];
    uint32_t key[NPL];
    int id[NPL];
    {
        const float *L = logits + (size_t)(tok ? wave : 0) * E;
#pragma unroll
        for (int i = 0; i < NPL; ++i) v[i] = i * kWave + lane < E ? L[i * kWave + lane] : 0.0f;
        topk_pairs<NPL>(v, E, key, id);
    }
    if (u >= K) {
        // a later entry: every token's selection, then the group table
        if (tok) {
            uint32_t my_key;
            int my_id;
            wave_topk_keys<NPL>(key, id, K, my_key, my_id);
            if (lane < K) sids[wave * K + lane] = my_id;
        }
        __syncthreads();
        build_group_table(sids, M, K, E, &tl, g);
        __syncthreads();
        w13_multi_block<HC, MT, false>(x, w13, M, I, K, act, &tl, b, xs);
        return;
    }
    // token 0's u-th choice
    const bool writer = b == 0;
    uint32_t my_key = 0u;
    int my_id = 0;
    if (wave == 0) {
        topk_sort_lane<NPL>(key, id);
        topk_rounds<NPL>(key, id, 0, u + 1, my_key, my_id);
        if (lane == u) s_e = my_id;
    }
    __syncthreads();
    const int e = s_e;
    float w = 0.0f;
    w13_multi_rows<HC, MT, false>(x, w13, M, I, K, act, e, b, xs, [&](unsigned &mask, int (&slot)[MT]) {
        if (wave > 0 && tok) {
            const int r = topk_rank<NPL>(key, id, e);
            if (lane == 0) s_rank[wave] = r;
        }
        if (writer) {
            // the full selection (token 0 continues from round u + 1) and the
            // group table, kept in LDS and registers until the products are done
            if (tok) {
                if (wave > 0) topk_sort_lane<NPL>(key, id);
                topk_rounds<NPL>(key, id, wave > 0 ? 0 : u + 1, K, my_key, my_id);
                const float my_l = my_key ? key_value(my_key) : 0.0f;
                const float lmax = key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
                w = topk_weight_vals<NPL>(v, E, K, renormalize, my_l, lmax);
                if (lane < K) sids[wave * K + lane] = my_id;
            }
            __syncthreads();
            build_group_table(sids, M, K, E, &tl, g);
        }
        __syncthreads();
        mask = 1u;
        slot[0] = u;
#pragma unroll
        for (int m = 1; m < MT; ++m) {
            const int r = m < M ? s_rank[m] : K;
            if (r < K) mask |= 1u << m;
            slot[m] = r < K ? r : 0;
        }
    });
    if (writer) {
        if (tok && lane < K) {
            ids[(size_t)wave * K + lane] = my_id;
            weights[(size_t)wave * K + lane] = w;
        }
        const int *src = reinterpret_cast<const int *>(&tl);
        int *dst = reinterpret_cast<int *>(table);
        for (int i = threadIdx.x; i < (int)(sizeof(GroupTable) / sizeof(int)); i += kBlock)
            dst[i] = src[i];
    }
    // then the shared down rows: token 0's workgroups take the shared down
    // blocks sb = b, b + (their count), ... -- at most kSharedPerTok0 each;
    // with more, the blocks run on their own in a launch before this one
    if (Is > 0) {
        const int r0 = K * (I / kRowsPerBlockM);
        const int shared_blocks = H / (kWavesPerBlock * (kWave / LM::LPR));
        if (shared_blocks <= kSharedPerTok0 * r0) {
            for (int sb = b; sb < shared_blocks; sb += r0) {
                __syncthreads(); // xs is free again
                shared_down_block<LM, MT, MT * HC * kWave>(wsd, act_s, M, H, Is,
                                                           sb * kWavesPerBlock, s_out,
                                                           reinterpret_cast<f32x4 *>(xs));
            }
        }
    }
}

// ---------------------------------------------------------------- probes
#if MOE_PART == 0
// empty kernel (launch latency and graph node gap)
__global__ void k_probe_empty() {}

// stream `n16` 16-byte chunks with non-temporal loads, L per thread in flight
template <int L>
__global__ __launch_bounds__(256) void k_probe_read(const f16x8 *__restrict__ src, size_t n16,
                                                    float *__restrict__ out)
{
    const size_t base = (size_t)blockIdx.x * blockDim.x * L + threadIdx.x;
    f16x8 v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const size_t idx = base + (size_t)i * blockDim.x;
        v[i] = idx < n16 ? stream_load(src + idx) : f16x8{};
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < L; ++i) acc += (float)v[i][0];
    if (acc == 1.25e-3f) out[0] = acc; // keeps the loads; never true for zero-filled input
}

// Plain device copy of n16 16-byte chunks (8 per thread): reads and writes a
// known byte count, the calibration for the memory-traffic counters.
__global__ __launch_bounds__(256) void k_probe_copy(const f16x8 *__restrict__ src,
                                                    f16x8 *__restrict__ dst, size_t n16)
{
    constexpr int L = 8;
    const size_t base = (size_t)blockIdx.x * blockDim.x * L + threadIdx.x;
    f16x8 v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const size_t idx = base + (size_t)i * blockDim.x;
        if (idx < n16) v[i] = stream_load(src + idx);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const size_t idx = base + (size_t)i * blockDim.x;
        if (idx < n16) dst[idx] = v[i];
    }
}

__global__ __launch_bounds__(kWave) void k_dbg_wave_sum(const float *__restrict__ in,
                                                         float *__restrict__ out)
{
    const float t = wave_sum(in[lane_id()]);
    if (lane_id() == 0) out[0] = t;
}
#endif

// ---------------------------------------------------------------- launchers
// The host side is compiled as several translation units of this one file
// (MOE_PART, set by the build), so that the kernel instances compile in
// parallel; every kernel instance belongs to exactly one part:
//   part 0       the entry points of moe_internal.h, top-k, grouping, probes,
//                and the dispatch on the hidden width H and on the row widths
//   parts 1..8   the kernels of hidden width H = 512 * part (router, gate/up,
//                the expand launches of the layer paths)
//   parts 9..21  the down-projection kernels (W2 + combine, reduce) of one
//                lane mapping each, in LaneMaps order
#ifndef MOE_PART
#error "moe_kernels.hip is compiled once per part: -DMOE_PART=0..21"
#endif

static inline hipError_t last() { return hipGetLastError(); }

template <class... T>
struct TypeList {};
template <int N, class L>
struct TypeAt;
template <int N, class T0, class... T>
struct TypeAt<N, TypeList<T0, T...>> : TypeAt<N - 1, TypeList<T...>> {};
template <class T0, class... T>
struct TypeAt<0, TypeList<T0, T...>> {
    using type = T0;
};
using LaneMaps = TypeList<LaneMap<8, 1, false>, LaneMap<16, 1, false>, LaneMap<8, 3, false>,
                          LaneMap<32, 1, false>, LaneMap<16, 3, false>, LaneMap<64, 1, false>,
                          LaneMap<32, 3, false>, LaneMap<64, 2, false>, LaneMap<64, 4, false>,
                          LaneMap<64, 1, true>, LaneMap<64, 2, true>, LaneMap<64, 3, true>,
                          LaneMap<64, 4, true>>;
#define MOE_FIRST_LANE_PART 9 // parts MOE_FIRST_LANE_PART .. +12: LaneMaps[part - 9]
#define MOE_LAST_PART 21

// f(LaneMap) with the lane mapping of rows n fp16 wide (n % 64 == 0, 64 <= n
// <= 2048, as the entry points require): exact where n/8 = LPR*CPL, LPR in
// {8, 16, 32, 64}, CPL <= 4 (largest LPR), padded 64-lane rows otherwise.
// n = 1536 (64 lanes x 3 chunks) runs on the padded 64 x 3 instance, whose
// steps then all lie inside the row: the same arithmetic as an exact one.
template <class F>
static auto with_lane_map(int n, F &&f) -> decltype(f(NoLaneMap{}))
{
    switch (n / 8) {
    case 8: return f(LaneMap<8, 1, false>{});
    case 16: return f(LaneMap<16, 1, false>{});
    case 24: return f(LaneMap<8, 3, false>{});
    case 32: return f(LaneMap<32, 1, false>{});
    case 48: return f(LaneMap<16, 3, false>{});
    case 64: return f(LaneMap<64, 1, false>{});
    case 96: return f(LaneMap<32, 3, false>{});
    case 128: return f(LaneMap<64, 2, false>{});
    case 256: return f(LaneMap<64, 4, false>{});
    }
    switch ((n / 8 + kWave - 1) / kWave) {
    case 1: return f(LaneMap<64, 1, true>{});
    case 2: return f(LaneMap<64, 2, true>{});
    case 3: return f(LaneMap<64, 3, true>{});
    default: return f(LaneMap<64, 4, true>{});
    }
}

// lanes per row of the mapping of rows n fp16 wide
static inline int lpr_of(int n)
{
    return with_lane_map(n, [](auto lm) { return decltype(lm)::LPR; });
}

template <int N>
using IntC = std::integral_constant<int, N>;

// f(IntC<HC>) for H = 512 * HC, HC = 1..8
template <class F>
static hipError_t with_hc(int H, F &&f)
{
    switch (H / 512) {
    case 1: return f(IntC<1>{});
    case 2: return f(IntC<2>{});
    case 3: return f(IntC<3>{});
    case 4: return f(IntC<4>{});
    case 5: return f(IntC<5>{});
    case 6: return f(IntC<6>{});
    case 7: return f(IntC<7>{});
    case 8: return f(IntC<8>{});
    }
    return hipErrorInvalidValue;
}

// Where a layer's shared-expert work goes (the three-launch path): with
// Is == I the shared down projection shares the routed one's lane mapping,
// so its gate/up rows stream in k_expand and its down rows in k_reduce;
// otherwise gate/up beside the router and down in k_expand.
static inline bool shared_folded(int I, int Is) { return Is == I; }

// ---- per-H entry points (defined in part H/512)
template <int HC>
hipError_t hc_router(const void *x, const void *wr, int M, int E, float *logits, hipStream_t s);
template <int HC>
hipError_t hc_w13(bool shared, const void *x, const void *w13, const int32_t *ids, int M, int I,
                  int K, int n_slots, float *act, GroupTable *table, hipStream_t s);
template <int HC>
hipError_t hc_lean(const void *x, const void *wr, const void *w13, const void *wsgu,
                   const void *wsd, int E, int I, int K, int Is, int renorm, int32_t *ids,
                   float *w, float *logits, float *act, float *act_s, float *s_out, int stage,
                   hipStream_t s);
template <int HC>
hipError_t hc_lean_m(const void *x, const void *wr, const void *w13, const void *wsgu,
                     const void *wsd, int M, int E, int I, int K, int Is, int renorm,
                     int32_t *ids, float *w, float *logits, float *act, float *act_s,
                     float *s_out, GroupTable *table, int stage, hipStream_t s);
// ---- per-lane-mapping entry points (defined in the part of that mapping)
template <class LM>
hipError_t lm_w2(bool shared, const float *act, const void *w2, const int32_t *ids,
                 const float *tw, const float *shared_in, int M, int H, int I, int K,
                 const GroupTable *table, void *out, hipStream_t s);
template <class LM>
hipError_t lm_reduce(const float *act, const void *w2, const int32_t *ids, const float *w,
                     const float *s_in, const void *wsd, const float *act_s, bool shared, int H,
                     int I, int K, void *y, hipStream_t s);
// ---- part 0
hipError_t launch_select_m(const float *logits, int M, int E, int K, int renorm, int32_t *ids,
                           float *w, GroupTable *table, hipStream_t s);

#if MOE_PART == 0
// ================================================================ part 0
hipError_t launch_route(const void *x, const void *wr, int M, int H, int E, int K, int renorm,
                        int32_t *ids, float *w, float *logits, hipStream_t s)
{
    hipError_t err = with_hc(H, [&](auto hc) {
        return hc_router<decltype(hc)::value>(x, wr, M, E, logits, s);
    });
    if (err != hipSuccess) return err;
    return launch_topk(logits, M, E, K, renorm, ids, w, s);
}

hipError_t launch_topk(const float *logits, int M, int E, int K, int renorm, int32_t *ids,
                       float *w, hipStream_t s)
{
    if (E <= kWave)
        hipLaunchKernelGGL(k_topk<1>, dim3(M), dim3(kWave), 0, s, logits, E, K, renorm, ids, w);
    else if (E <= 4 * kWave)
        hipLaunchKernelGGL(k_topk<4>, dim3(M), dim3(kWave), 0, s, logits, E, K, renorm, ids, w);
    else
        hipLaunchKernelGGL(k_topk<kMaxExperts / kWave>, dim3(M), dim3(kWave), 0, s, logits, E, K,
                           renorm, ids, w);
    return last();
}

hipError_t launch_topk_sum(const float *part, int P, int M, int E, int K, int renorm,
                           float *logits, int32_t *ids, float *w, hipStream_t s)
{
    if (E <= kWave)
        hipLaunchKernelGGL(k_topk_sum<1>, dim3(M), dim3(kWave), 0, s, part, P, M, E, K, renorm,
                           logits, ids, w);
    else if (E <= 4 * kWave)
        hipLaunchKernelGGL(k_topk_sum<4>, dim3(M), dim3(kWave), 0, s, part, P, M, E, K, renorm,
                           logits, ids, w);
    else
        hipLaunchKernelGGL(k_topk_sum<kMaxExperts / kWave>, dim3(M), dim3(kWave), 0, s, part, P,
                           M, E, K, renorm, logits, ids, w);
    return last();
}

hipError_t launch_select_m(const float *logits, int M, int E, int K, int renorm, int32_t *ids,
                           float *w, GroupTable *table, hipStream_t s)
{
    if (E <= kWave)
        hipLaunchKernelGGL(k_select_m<1>, dim3(1), dim3(kSelBlock), 0, s, logits, M, E, K, renorm,
                           ids, w, table);
    else if (E <= 4 * kWave)
        hipLaunchKernelGGL(k_select_m<4>, dim3(1), dim3(kSelBlock), 0, s, logits, M, E, K, renorm,
                           ids, w, table);
    else
        hipLaunchKernelGGL(k_select_m<kMaxExperts / kWave>, dim3(1), dim3(kSelBlock), 0, s, logits,
                           M, E, K, renorm, ids, w, table);
    return last();
}

static hipError_t launch_w13(bool shared, const void *x, const void *w13, const int32_t *ids,
                             int M, int H, int I, int K, int n_slots, float *act,
                             GroupTable *table, hipStream_t s)
{
    return with_hc(H, [&](auto hc) {
        return hc_w13<decltype(hc)::value>(shared, x, w13, ids, M, I, K, n_slots, act, table, s);
    });
}

static hipError_t launch_w2(bool shared, const float *act, const void *w2, const int32_t *ids,
                            const float *tw, const float *shared_in, int M, int H, int I, int K,
                            const GroupTable *table, void *out, hipStream_t s)
{
    return with_lane_map(I, [&](auto lm) {
        return lm_w2<decltype(lm)>(shared, act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    });
}

hipError_t launch_shared(const void *x, const void *wgu, const void *wd, int M, int H, int Is,
                         float *s_out, float *act_shared, hipStream_t s)
{
    hipError_t err = launch_w13(true, x, wgu, nullptr, M, H, Is, 1, 1, act_shared, nullptr, s);
    if (err != hipSuccess) return err;
    return launch_w2(true, act_shared, wd, nullptr, nullptr, nullptr, M, H, Is, 1, nullptr, s_out,
                     s);
}

// For M > 1: the distinct selected experts, read by the W13 and W2 kernels.
static hipError_t launch_group_table(const int32_t *ids, int M, int K, int E, GroupTable *table,
                                     hipStream_t s)
{
    hipLaunchKernelGGL(k_group_table, dim3(1), dim3(kGroupThreads), 0, s, ids, M, K, E, table);
    return last();
}

hipError_t launch_w13_routed(const void *x, const void *w13, const int32_t *ids, int M, int H,
                             int E, int I, int K, float *act, GroupTable *table, hipStream_t s)
{
    if (M > 1) {
        const hipError_t err = launch_group_table(ids, M, K, E, table, s);
        if (err != hipSuccess) return err;
    }
    const int n_slots = M * K < E ? M * K : E;
    return launch_w13(false, x, w13, ids, M, H, I, K, n_slots, act, table, s);
}

hipError_t launch_fused(const void *x, const void *w13, const void *w2, const int32_t *ids,
                        const float *tw, const float *shared_in, int M, int H, int E, int I, int K,
                        void *y, float *act, GroupTable *table, hipStream_t s)
{
    hipError_t err = launch_w13_routed(x, w13, ids, M, H, E, I, K, act, table, s);
    if (err != hipSuccess) return err;
    return launch_w2(false, act, w2, ids, tw, shared_in, M, H, I, K, table, y, s);
}

hipError_t launch_w2_routed(const float *act, const void *w2, const int32_t *ids, const float *tw,
                            const float *shared_in, int M, int H, int E, int I, int K, void *y,
                            GroupTable *table, hipStream_t s)
{
    if (M > 1) {
        const hipError_t err = launch_group_table(ids, M, K, E, table, s);
        if (err != hipSuccess) return err;
    }
    return launch_w2(false, act, w2, ids, tw, shared_in, M, H, I, K, table, y, s);
}

hipError_t launch_probe_empty(hipStream_t s)
{
    hipLaunchKernelGGL(k_probe_empty, dim3(1), dim3(kWave), 0, s);
    return last();
}

hipError_t launch_probe_read(const void *src, size_t bytes, float *out, hipStream_t s)
{
    // below 4 MB one load per thread, so that a short read still spreads over
    // hundreds of workgroups (a layer's router-sized read: 257 of them)
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    if (bytes < (4u << 20)) {
        const unsigned blocks = (unsigned)((n16 + 255) / 256);
        hipLaunchKernelGGL(k_probe_read<1>, dim3(blocks), dim3(256), 0, s, (const f16x8 *)src,
                           n16, out);
    } else {
        const size_t per_block = 256 * 8;
        const unsigned blocks = (unsigned)((n16 + per_block - 1) / per_block);
        hipLaunchKernelGGL(k_probe_read<8>, dim3(blocks), dim3(256), 0, s, (const f16x8 *)src,
                           n16, out);
    }
    return last();
}

hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t s)
{
    const size_t n16 = bytes / 16;
    const size_t per_block = 256 * 8;
    const unsigned blocks = (unsigned)((n16 + per_block - 1) / per_block);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_probe_copy, dim3(blocks), dim3(256), 0, s, (const f16x8 *)src,
                       (f16x8 *)dst, n16);
    return last();
}

void lane_map_of(int n, int *lpr, int *cpl, int *pad)
{
    with_lane_map(n, [&](auto lm) {
        using LM = decltype(lm);
        *lpr = LM::LPR;
        *cpl = LM::CPL;
        // padded when a step lies past the row's end (n = 1536 runs the
        // padded instance, whose steps all lie inside the row)
        *pad = LM::LPR * LM::CPL * 8 > n ? 1 : 0;
        return 0;
    });
}

hipError_t launch_dbg_wave_sum(const float *in, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(k_dbg_wave_sum, dim3(1), dim3(kWave), 0, s, in, out);
    return last();
}

bool lean_ok(int M, int H, int E, int I, int K, int Is)
{
    // k_reduce stages [K*I] fp32 in LDS; its workgroups and k_expand's shared
    // workgroups cover whole row groups of H
    return M == 1 && E <= kMaxExperts && K * I <= kMaxStaged &&
           H % kRRows == 0 &&
           (Is == 0 || H % (kWavesPerBlock * (kWave / lpr_of(Is))) == 0);
}

bool lean_m_ok(int M, int H, int E, int I, int K, int Is)
{
    (void)E;
    (void)I;
    (void)K;
    return M >= 2 && M <= kMaxTokens && (Is == 0 || H % (kWavesPerBlock * (kWave / lpr_of(Is))) == 0);
}

int lean_m_launches(int M, int H, int I, int K, int Is)
{
    if (mt_of(M) > kWavesPerBlock) return 4; // a selection launch
    const int rows = (mt_of(M) == 4 ? rows_per_wave_m<false, 4>() : rows_per_wave_m<false, 2>()) *
                     kWavesPerBlock;
    const int r0 = K * (I / rows);
    const int shared = Is ? H / (kWavesPerBlock * (kWave / lpr_of(Is))) : 0;
    return shared > kSharedPerTok0 * r0 ? 4 : 3;
}

hipError_t launch_lean_m(const void *x, const void *wr, const void *w13, const void *w2,
                         const void *wsgu, const void *wsd, int M, int H, int E, int I, int K,
                         int Is, int renorm, int32_t *ids, float *w, float *logits, void *y,
                         float *act, float *act_s, float *s_out, GroupTable *table, int stage,
                         hipStream_t s)
{
    // stage 0: every launch; 1: router (+ shared gate/up); 2: the selection and
    // the gate/up rows (one launch at M <= 4, two at M = 5..8); 3: the W2 launch
    if (stage < 0 || stage > 3) return hipErrorInvalidValue;
    if (stage <= 2) {
        const hipError_t err = with_hc(H, [&](auto hc) {
            return hc_lean_m<decltype(hc)::value>(x, wr, w13, wsgu, wsd, M, E, I, K, Is, renorm,
                                                  ids, w, logits, act, act_s, s_out, table, stage,
                                                  s);
        });
        if (err != hipSuccess || stage != 0) return err;
    }
    return launch_w2(false, act, w2, ids, w, Is ? s_out : nullptr, M, H, I, K, table, y, s);
}

hipError_t launch_lean(const void *x, const void *wr, const void *w13, const void *w2,
                       const void *wsgu, const void *wsd, int H, int E, int I, int K, int Is,
                       int renorm, int32_t *ids, float *w, float *logits, void *y, float *act,
                       float *act_s, float *s_out, int stage, hipStream_t s)
{
    // stage 0: the three launches; 1, 2, 3: that launch alone
    if (stage < 0 || stage > 3) return hipErrorInvalidValue;
    if (stage <= 2) {
        const hipError_t err = with_hc(H, [&](auto hc) {
            return hc_lean<decltype(hc)::value>(x, wr, w13, wsgu, wsd, E, I, K, Is, renorm, ids,
                                                w, logits, act, act_s, s_out, stage, s);
        });
        if (err != hipSuccess || stage != 0) return err;
    }
    const bool folded = Is != 0 && shared_folded(I, Is);
    const float *s_in = Is && !folded ? s_out : nullptr;
    return with_lane_map(I, [&](auto lm) {
        return lm_reduce<decltype(lm)>(act, w2, ids, w, s_in, wsd, act_s, folded, H, I, K, y, s);
    });
}

#elif MOE_PART >= 1 && MOE_PART <= 8
// ================================================================ parts 1..8: H = 512 * MOE_PART
template <int HC>
hipError_t hc_router(const void *x, const void *wr, int M, int E, float *logits, hipStream_t s)
{
    hipLaunchKernelGGL(k_router<HC>, dim3(E), dim3(kWave), 0, s, (const f16 *)x,
                       (const f16 *)wr, M, E, logits);
    return last();
}

template <int HC, int MT, bool SHARED>
static hipError_t launch_w13_t(const void *x, const void *w13, const int32_t *ids, int M, int I,
                               int K, int n_slots, float *act, GroupTable *table, hipStream_t s)
{
    if constexpr (MT == 1) {
        const int blocks = n_slots * (I / kWavesPerBlock);
        hipLaunchKernelGGL((k_w13_silu<HC, SHARED>), dim3(blocks), dim3(kBlock), 0, s,
                           (const f16 *)x, (const f16 *)w13, ids, I, act);
    } else {
        const int blocks = n_slots * (I / (rows_per_wave_m<SHARED, MT>() * kWavesPerBlock));
        hipLaunchKernelGGL((k_w13_multi<HC, MT, SHARED>), dim3(blocks), dim3(kBlock), 0, s,
                           (const f16 *)x, (const f16 *)w13, M, I, K, act, table);
    }
    return last();
}

template <int HC, bool SHARED>
static hipError_t launch_w13_mt(const void *x, const void *w13, const int32_t *ids, int M, int I,
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

template <int HC>
hipError_t hc_w13(bool shared, const void *x, const void *w13, const int32_t *ids, int M, int I,
                  int K, int n_slots, float *act, GroupTable *table, hipStream_t s)
{
    return shared ? launch_w13_mt<HC, true>(x, w13, ids, M, I, K, n_slots, act, table, s)
                  : launch_w13_mt<HC, false>(x, w13, ids, M, I, K, n_slots, act, table, s);
}

template <int HC, int NPL, class LM, int SM>
static void launch_expand_t(dim3 grid, const void *x, const void *w13, const void *wsh,
                            const float *logits, float *act_s, int E, int I, int K, int Is,
                            int renorm, int32_t *ids, float *w, float *act, float *s_out,
                            hipStream_t s)
{
    hipLaunchKernelGGL((k_expand<HC, NPL, LM, SM>), grid, dim3(kBlock), 0, s, (const f16 *)x,
                       (const f16 *)w13, (const f16 *)wsh, logits, act_s, E, I, K, Is, renorm,
                       ids, w, act, s_out);
}

template <int HC, int NPL>
static void launch_expand_n(dim3 grid, const void *x, const void *w13, const void *wsgu,
                            const void *wsd, const float *logits, float *act_s, int E, int I,
                            int K, int Is, int renorm, int32_t *ids, float *w, float *act,
                            float *s_out, hipStream_t s)
{
    if (Is == 0) {
        launch_expand_t<HC, NPL, NoLaneMap, kExpandNoShared>(grid, x, w13, nullptr, logits, act_s, E, I, K, Is, renorm, ids, w, act, s_out, s);
        return;
    }
    if (shared_folded(I, Is)) {
        launch_expand_t<HC, NPL, NoLaneMap, kExpandSharedGateUp>(grid, x, w13, wsgu, logits, act_s, E, I, K, Is, renorm, ids, w, act, s_out, s);
        return;
    }
    // the shared down projection with the lane mapping of rows Is wide
    with_lane_map(Is, [&](auto lm) {
        launch_expand_t<HC, NPL, decltype(lm), kExpandSharedDown>(grid, x, w13, wsd, logits, act_s, E, I, K, Is, renorm, ids, w, act, s_out, s);
        return 0;
    });
}

template <int HC>
hipError_t hc_lean(const void *x, const void *wr, const void *w13, const void *wsgu,
                   const void *wsd, int E, int I, int K, int Is, int renorm, int32_t *ids,
                   float *w, float *logits, float *act, float *act_s, float *s_out, int stage,
                   hipStream_t s)
{
    constexpr int H = 512 * HC;
    const bool router_only = Is == 0 || shared_folded(I, Is);
    if (stage == 0 || stage == 1) {
        if (router_only) {
            hipLaunchKernelGGL((k_router1<HC>), dim3(E), dim3(kWave), 0, s, (const f16 *)x,
                               (const f16 *)wr, logits);
        } else {
            const int rb = (E + kWavesPerBlock - 1) / kWavesPerBlock;
            hipLaunchKernelGGL((k_router_shared<HC>), dim3(rb + Is / kWavesPerBlock),
                               dim3(kBlock), 0, s, (const f16 *)x, (const f16 *)wr,
                               (const f16 *)wsgu, E, Is, logits, act_s);
        }
        const hipError_t err = last();
        if (err != hipSuccess || stage == 1) return err;
    }
    if (stage != 0 && stage != 2) return hipSuccess;
    const int shared_blocks = Is == 0 ? 0
                              : shared_folded(I, Is) ? Is / kWavesPerBlock
                                                     : H / (kWavesPerBlock * (kWave / lpr_of(Is)));
    const dim3 grid(K * (I / kWavesPerBlock) + shared_blocks);
    if (E <= kWave)
        launch_expand_n<HC, 1>(grid, x, w13, wsgu, wsd, logits, act_s, E, I, K, Is, renorm, ids, w, act, s_out, s);
    else if (E <= 4 * kWave)
        launch_expand_n<HC, 4>(grid, x, w13, wsgu, wsd, logits, act_s, E, I, K, Is, renorm, ids, w, act, s_out, s);
    else
        launch_expand_n<HC, kMaxExperts / kWave>(grid, x, w13, wsgu, wsd, logits, act_s, E, I, K, Is, renorm, ids, w, act, s_out, s);
    return last();
}

template <int HC, int MT, class LM>
static hipError_t launch_expand_m_t(const void *x, const void *w13, const void *wsd,
                                    const float *act_s, int M, int I, int K, int Is, int n_slots,
                                    float *act, float *s_out, const GroupTable *table, hipStream_t s)
{
    constexpr int H = 512 * HC;
    const int routed = n_slots * (I / (rows_per_wave_m<false, MT>() * kWavesPerBlock));
    const int shared = Is ? H / (kWavesPerBlock * (kWave / LM::LPR)) : 0;
    hipLaunchKernelGGL((k_expand_m<HC, MT, LM>), dim3(routed + shared), dim3(kBlock), 0, s,
                       (const f16 *)x, (const f16 *)w13, (const f16 *)wsd, act_s, M, H, I, K, Is,
                       routed, act, s_out, table);
    return last();
}

template <int HC, int MT>
static hipError_t launch_lean_m_t(const void *x, const void *wr, const void *w13,
                                  const void *wsgu, const void *wsd, int M, int E, int I, int K,
                                  int Is, int renorm, int32_t *ids, float *w, float *logits,
                                  float *act, float *act_s, float *s_out, GroupTable *table,
                                  int stage, hipStream_t s)
{
    hipError_t err = hipSuccess;
    if (stage != 2) {
        const int rb = (E + kWavesPerBlock - 1) / kWavesPerBlock;
        hipLaunchKernelGGL((k_route_shared_m<HC, MT>), dim3(rb + Is / kWavesPerBlock),
                           dim3(kBlock), 0, s, (const f16 *)x, (const f16 *)wr,
                           (const f16 *)wsgu, M, E, Is, logits, act_s);
        err = last();
        if (err != hipSuccess || stage == 1) return err;
    }
    const int n_slots = M * K < E ? M * K : E;
    // without a shared expert the mapping is unused (no shared workgroups)
    const int lm_width = Is ? Is : 512;
    if constexpr (MT <= kWavesPerBlock) {
        // the selection folded into the expand launch (one wave per token)
        constexpr int H = 512 * HC;
        const int routed = n_slots * (I / (rows_per_wave_m<false, MT>() * kWavesPerBlock));
        return with_lane_map(lm_width, [&](auto lm) {
            using LM = decltype(lm);
            // the shared down blocks go with token 0's K*I/rows workgroups,
            // up to kSharedPerTok0 each; beyond that they run first, on their
            // own, as k_expand_m's shared workgroups (one more launch, for
            // sizes such as K = 1 with narrow experts and a wide shared one)
            const int shared = Is ? H / (kWavesPerBlock * (kWave / LM::LPR)) : 0;
            const int r0 = K * (I / (rows_per_wave_m<false, MT>() * kWavesPerBlock));
            if (shared > kSharedPerTok0 * r0) {
                hipLaunchKernelGGL((k_expand_m<HC, MT, LM>), dim3(shared), dim3(kBlock), 0, s,
                                   (const f16 *)x, (const f16 *)w13, (const f16 *)wsd, act_s, M,
                                   H, I, K, Is, 0, act, s_out, table);
                const hipError_t e = last();
                if (e != hipSuccess) return e;
            }
            const dim3 grid(routed);
#define SEL_LAUNCH(NPL_)                                                                          \
    hipLaunchKernelGGL((k_expand_sel_m<HC, MT, LM, NPL_>), grid, dim3(kBlock), 0, s,              \
                       (const f16 *)x, (const f16 *)w13, (const f16 *)wsd, act_s, logits, M, H, E, \
                       I, K, Is, renorm, routed, ids, w, act, s_out, table)
            if (E <= kWave) SEL_LAUNCH(1);
            else if (E <= 4 * kWave) SEL_LAUNCH(4);
            else SEL_LAUNCH(kMaxExperts / kWave);
#undef SEL_LAUNCH
            return last();
        });
    }
    if ((err = launch_select_m(logits, M, E, K, renorm, ids, w, table, s)) != hipSuccess) return err;
    return with_lane_map(lm_width, [&](auto lm) {
        return launch_expand_m_t<HC, MT, decltype(lm)>(x, w13, wsd, act_s, M, I, K, Is, n_slots,
                                                       act, s_out, table, s);
    });
}

template <int HC>
hipError_t hc_lean_m(const void *x, const void *wr, const void *w13, const void *wsgu,
                     const void *wsd, int M, int E, int I, int K, int Is, int renorm,
                     int32_t *ids, float *w, float *logits, float *act, float *act_s,
                     float *s_out, GroupTable *table, int stage, hipStream_t s)
{
    switch (mt_of(M)) {
    case 2: return launch_lean_m_t<HC, 2>(x, wr, w13, wsgu, wsd, M, E, I, K, Is, renorm, ids, w, logits, act, act_s, s_out, table, stage, s);
    case 4: return launch_lean_m_t<HC, 4>(x, wr, w13, wsgu, wsd, M, E, I, K, Is, renorm, ids, w, logits, act, act_s, s_out, table, stage, s);
    case 8:
        if constexpr (HC <= 4)
            return launch_lean_m_t<HC, 8>(x, wr, w13, wsgu, wsd, M, E, I, K, Is, renorm, ids, w, logits, act, act_s, s_out, table, stage, s);
        return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

template hipError_t hc_router<MOE_PART>(const void *, const void *, int, int, float *, hipStream_t);
template hipError_t hc_w13<MOE_PART>(bool, const void *, const void *, const int32_t *, int, int,
                                     int, int, float *, GroupTable *, hipStream_t);
template hipError_t hc_lean<MOE_PART>(const void *, const void *, const void *, const void *,
                                      const void *, int, int, int, int, int, int32_t *, float *,
                                      float *, float *, float *, float *, int, hipStream_t);
template hipError_t hc_lean_m<MOE_PART>(const void *, const void *, const void *, const void *,
                                        const void *, int, int, int, int, int, int, int32_t *,
                                        float *, float *, float *, float *, float *, GroupTable *,
                                        int, hipStream_t);

#elif MOE_PART >= MOE_FIRST_LANE_PART && MOE_PART <= MOE_LAST_PART
// ================================================================ parts 9..21: one lane mapping
constexpr int kMaxDevices = 64;

// Largest dynamic LDS a workgroup may opt into on the current device (looked
// up once per device; 64 KiB if the query fails).
static size_t lds_optin_bytes()
{
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
    if (dev >= 0 && dev < kMaxDevices && (v = cached[dev].load(std::memory_order_relaxed)) > 0)
        return (size_t)v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeSharedMemPerBlockOptin, dev) != hipSuccess ||
        v <= 0)
        return 64 * 1024;
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(v, std::memory_order_relaxed);
    return (size_t)v;
}

template <class LM, int MT, bool SHARED>
static hipError_t launch_w2_t(const float *act, const void *w2, const int32_t *ids,
                              const float *tw, const float *shared_in, int M, int H, int I, int K,
                              const GroupTable *table, void *out, hipStream_t s)
{
    if constexpr (MT > 1) {
        // several tokens: stage the activations in LDS when they fit
        const size_t lds = (size_t)M * (SHARED ? 1 : K) * I * sizeof(float);
        constexpr int rows = (kWave / LM::LPR) * kSWaves;
        // the kernel's static LDS (routing weights, table masks and slots)
        // comes on top of `lds`
        if (H % rows == 0 && lds + kMaxSlots * 16 <= lds_optin_bytes()) {
            auto kern = k_w2_staged<LM, MT, SHARED>;
            // Opt this instance into the device's full LDS once per device,
            // whatever this call's size: the launch's LDS is the dynamic bytes
            // plus the kernel's static arrays, and the default 64 KiB limit
            // applies to that sum.
            static std::atomic<bool> opted[kMaxDevices] = {};
            int dev = 0;
            hipError_t e = hipGetDevice(&dev);
            if (e != hipSuccess) return e;
            if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
            if (!opted[dev].load(std::memory_order_acquire)) {
                hipFuncAttributes fa;
                e = hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(kern));
                if (e != hipSuccess) return e;
                e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)(lds_optin_bytes() - fa.sharedSizeBytes));
                if (e != hipSuccess) return e;
                opted[dev].store(true, std::memory_order_release);
            }
            hipLaunchKernelGGL(kern, dim3(H / rows), dim3(kSBlock), lds, s, act,
                               (const f16 *)w2, tw, shared_in, M, H, I, K, table, out);
            return last();
        }
    }
    constexpr int rows_per_block = (kWave / LM::LPR) * kWavesPerBlock;
    const int blocks = H / rows_per_block;
    hipLaunchKernelGGL((k_w2_combine<LM, MT, SHARED>), dim3(blocks), dim3(kBlock), 0, s, act,
                       (const f16 *)w2, ids, tw, shared_in, M, H, I, K, table, out);
    return last();
}

template <class LM, bool SHARED>
static hipError_t launch_w2_mt(const float *act, const void *w2, const int32_t *ids,
                               const float *tw, const float *shared_in, int M, int H, int I, int K,
                               const GroupTable *table, void *out, hipStream_t s)
{
    switch (mt_of(M)) {
    case 1: return launch_w2_t<LM, 1, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 2: return launch_w2_t<LM, 2, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 4: return launch_w2_t<LM, 4, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    case 8: return launch_w2_t<LM, 8, SHARED>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
    }
    return hipErrorInvalidValue;
}

template <class LM>
hipError_t lm_w2(bool shared, const float *act, const void *w2, const int32_t *ids,
                 const float *tw, const float *shared_in, int M, int H, int I, int K,
                 const GroupTable *table, void *out, hipStream_t s)
{
    return shared ? launch_w2_mt<LM, true>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s)
                  : launch_w2_mt<LM, false>(act, w2, ids, tw, shared_in, M, H, I, K, table, out, s);
}

template <class LM, bool SH>
static void launch_reduce_s(dim3 grid, size_t lds, int stage, const float *act, const f16 *w2,
                            const int32_t *ids, const float *w, const float *s_in, const f16 *wsd,
                            const float *act_s, int H, int I, int K, f16 *y, hipStream_t s)
{
    const dim3 block(reduce_waves<LM>() * kWave);
    if (stage <= 1)
        hipLaunchKernelGGL((k_reduce<LM, 1, SH>), grid, block, lds, s, act, w2, ids, w, s_in, wsd, act_s, H, I, K, y);
    else if (stage <= 2)
        hipLaunchKernelGGL((k_reduce<LM, 2, SH>), grid, block, lds, s, act, w2, ids, w, s_in, wsd, act_s, H, I, K, y);
    else if (stage <= 4)
        hipLaunchKernelGGL((k_reduce<LM, 4, SH>), grid, block, lds, s, act, w2, ids, w, s_in, wsd, act_s, H, I, K, y);
    else if (stage <= 8)
        hipLaunchKernelGGL((k_reduce<LM, 8, SH>), grid, block, lds, s, act, w2, ids, w, s_in, wsd, act_s, H, I, K, y);
    else // K*I <= 16384 with 64 lanes per 8 rows' worth of width: at most 12 loads
        hipLaunchKernelGGL((k_reduce<LM, 16, SH>), grid, block, lds, s, act, w2, ids, w, s_in, wsd, act_s, H, I, K, y);
}

// shared: the shared down projection runs here (wsd, act_s), else s_in (or
// nullptr without a shared expert) is added
template <class LM>
hipError_t lm_reduce(const float *act, const void *w2, const int32_t *ids, const float *w,
                     const float *s_in, const void *wsd, const float *act_s, bool shared, int H,
                     int I, int K, void *y, hipStream_t s)
{
    constexpr int block = reduce_waves<LM>() * kWave;
    constexpr int rows = reduce_waves<LM>() * (kWave / LM::LPR);
    static_assert(rows == kRRows, "a reduce workgroup covers 8 rows");
    const size_t lds = (size_t)K * I * sizeof(float);
    const int stage = (K * I / 4 + block - 1) / block;
    if (stage > 16) return hipErrorInvalidValue;
    const dim3 grid(H / rows);
    if (shared)
        launch_reduce_s<LM, true>(grid, lds, stage, act, (const f16 *)w2, ids, w, nullptr,
                                  (const f16 *)wsd, act_s, H, I, K, (f16 *)y, s);
    else
        launch_reduce_s<LM, false>(grid, lds, stage, act, (const f16 *)w2, ids, w, s_in, nullptr,
                                   nullptr, H, I, K, (f16 *)y, s);
    return last();
}

using PartLM = TypeAt<MOE_PART - MOE_FIRST_LANE_PART, LaneMaps>::type;
template hipError_t lm_w2<PartLM>(bool, const float *, const void *, const int32_t *,
                                  const float *, const float *, int, int, int, int,
                                  const GroupTable *, void *, hipStream_t);
template hipError_t lm_reduce<PartLM>(const float *, const void *, const int32_t *, const float *,
                                      const float *, const void *, const float *, bool, int, int,
                                      int, void *, hipStream_t);
#else
#error "MOE_PART out of range"
#endif

} // namespace moe
