// moe_prefill.hip -- gfx950 (CDNA4) kernels of the MoE layer over many tokens
// at once (prefill): the same layer the decode kernels compute, for T tokens.
//
// Method (BI-V100 inference worklog, "如何在天垓 BI-V100 上优化大模型推理：
// 一份工作日志", part 8: once T > 1 the expert products are matrix products
// whose arithmetic intensity grows with the tokens per expert, so tiling pays;
// the decode report of 2026-07-14, next steps: replace the prefill path's
// per-expert loop by one grouped GEMM).  Design for CDNA4:
//   * one workgroup groups the (token, slot) pairs by expert and writes a list
//     of tiles; every expert's weight rows are then streamed from HBM once per
//     tile of up to 128 of its tokens (tiles of one expert are placed on one
//     XCD so a second tile's re-read can be served by that XCD's L2);
//   * the products run on the matrix cores, v_mfma_f32_16x16x32_f16 (fp16
//     inputs, fp32 accumulators).  The weight operand goes from HBM straight
//     into registers in the instruction's operand layout: one load instruction
//     reads 64 contiguous bytes from each of 16 weight rows (16 whole 64-byte
//     sectors per 1 KiB), two k steps ahead of its products.  The token
//     operand is read through buffer loads (padding rows of a partly filled
//     tile read nothing) and staged in LDS once per workgroup with a 144-byte
//     row stride, which keeps the 16-byte fragment reads free of bank
//     conflicts;
//   * gate row j and up row I + j sit in accumulator tiles of the same wave at
//     the same lane positions, so SiLU(gate) * up is formed in registers and
//     stored once (fp16);
//   * the router is a GEMM over slices of H (enough workgroups for its small
//     weight), summed in a fixed order;
//   * the shared expert is one more group of both grouped GEMMs (every token);
//     the down products are written per (token, slot) in fp32 and a last pass
//     sums them with the routing weights in routing order, adds the shared
//     expert's output and rounds y to fp16 once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRouterWaves = 4;            // waves per router workgroup
constexpr int kRouterBlock = 64 * kRouterWaves;
constexpr int kBM = kPrefillRows;       // token rows per grouped-GEMM tile: eight 16-row MFMA tiles
constexpr int kBK = 64;                 // k per main-loop step (two 32-wide MFMA steps)
constexpr int kLdsRow = kBK + 8;        // halves per staged row (144 bytes)
constexpr int kRouterRows = 64;         // token rows per router tile
constexpr int kGemmWaves = 4;           // waves per grouped-GEMM workgroup
constexpr int kDepth = 2;               // k steps in flight in the GEMM main loops
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kPlanThreads = 1024;
constexpr int kPlanIds = 16;            // expert ids per plan thread per pass

__device__ __forceinline__ f16x8 ld16_stream(const f16 *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f16x8 *>(p));
}

__device__ __forceinline__ float silu_times(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Row of the 16x16 accumulator tile held in element r by lane `lane`
// (v_mfma_f32_16x16x32_f16: lane l holds column l % 16, rows 4 (l / 16) + r).
__device__ __forceinline__ int acc_row(int lane, int r) { return (lane >> 4) * 4 + r; }

// One 64-wide k step of this lane's weight rows: for MFMA step s (k offset
// 32 s) lane l reads k = 32 s + 8 (l / 16) + [0, 8) of row brow[ct] -- the
// 16-byte chunk that the instruction's operand layout puts in that lane.
template <int NCT>
__device__ __forceinline__ void load_b(const f16 *const (&brow)[NCT], int k, int quarter,
                                       f16x8 (&b)[NCT][2])
{
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            b[ct][s] = ld16_stream(brow[ct] + k * kBK + 32 * s + 8 * quarter);
}

// Token rows of one tile, read through a buffer resource: row i of the tile
// starts at byte off[i] of the source; a padding row (past the tile's valid
// rows) gets off = the source's size, so every load of it is out of range and
// returns zeros without touching memory.
template <int SL>
struct TokRows {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t off[SL];
};

template <int SL>
__device__ __forceinline__ TokRows<SL> tok_rows(const f16 *src, uint32_t src_bytes)
{
    TokRows<SL> a;
    a.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<f16 *>(src), (short)0, (int)src_bytes,
                                               kBufferWord3);
    return a;
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, class F>
__device__ __forceinline__ void unroll(F &&f)
{
    if constexpr (N > 0) {
        unroll<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// acc[mt][ct] += A(rows 16 mt .. 16 mt + 15) * B(ct)^T over kdim for one wave
// (MT row tiles of 16 tokens, NCT column tiles of 16 weight rows), in a
// workgroup of WAVES waves, with D k steps in flight.
//   a.off[i]: byte offset of this thread's token row for staging chunk i
//             (tile row t/8 + 8 WAVES i), whose 16-byte chunk t % 8 of each k
//             step it copies into LDS;
//   brow[ct]: this lane's weight row (row lane % 16 of column tile ct); a
//             wave without valid columns passes clamped valid rows, computes
//             products anyway and does not store them;
//   bb[0]:    the first k step of the weight rows, already loaded by the
//             caller; bb[1..D] are this function's other weight buffers.
// Every thread of the block must call this (it contains barriers).  The
// token tile is double-buffered in LDS; token rows and weights are loaded
// into registers D steps ahead of their products.
template <int WAVES, int MT>
constexpr int stage_loads() { return MT * 16 * kBK / 8 / (64 * WAVES); } // 16-byte loads per thread

template <int WAVES, int MT, int NCT, int D>
__device__ __forceinline__ void mfma_rows(const TokRows<stage_loads<WAVES, MT>()> &arows,
                                          const f16 *const (&brow)[NCT], int kdim, f16 *lds,
                                          f16x8 (&bb)[D + 1][NCT][2], f32x4 (&acc)[MT][NCT])
{
    constexpr int kStageLoads = stage_loads<WAVES, MT>();
    static_assert(kStageLoads >= 1, "tile too small for the workgroup");
    constexpr int kLdsStage = MT * 16 * kLdsRow;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int quarter = lane >> 4;
    const int kc = t & 7;
    const int nk = kdim / kBK;
    int wofs[kStageLoads];
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) wofs[i] = (t / 8 + 8 * WAVES * i) * kLdsRow + kc * 8;
    const int rofs = (lane & 15) * kLdsRow + 8 * quarter;
    f16x8 aa[D + 1][kStageLoads];

    auto load_a = [&](int k, f16x8 (&a)[kStageLoads]) {
#pragma unroll
        for (int i = 0; i < kStageLoads; ++i)
            a[i] = __builtin_bit_cast(
                f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                           arows.rsrc, arows.off[i] + (uint32_t)(k * kBK + kc * 8) * 2, 0, 0));
    };
    auto store_a = [&](const f16x8 (&a)[kStageLoads], int st) {
#pragma unroll
        for (int i = 0; i < kStageLoads; ++i)
            *reinterpret_cast<f16x8 *>(lds + st * kLdsStage + wofs[i]) = a[i];
    };
    auto mma = [&](int st, const f16x8 (&b)[NCT][2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f16x8 av = *reinterpret_cast<const f16x8 *>(
                    lds + st * kLdsStage + rofs + 16 * mt * kLdsRow + 32 * s);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    acc[mt][ct] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[ct][s], acc[mt][ct], 0, 0, 0);
            }
    };

    // prologue: steps 0 .. D-1 in flight, step 0's token rows into LDS stage 0
    unroll<D>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if constexpr (j > 0) load_b<NCT>(brow, min(j, nk - 1), quarter, bb[j]);
        load_a(min(j, nk - 1), aa[j]);
    });
    store_a(aa[0], 0);
    __syncthreads();
    // Step k: products from LDS stage k & 1 and bb[k % (D+1)] while step
    // k + D loads into the buffers step k - 1 freed; step k + 1's token rows
    // go to the other LDS stage.  Load indices are clamped to the last step,
    // so no load sits under a branch: the compiler then waits for exactly the
    // loads each use needs (the clamped repeats near the end re-read rows just
    // read, from L2).
    int k = 0;
    for (; k + D + 1 <= nk; k += D + 1) {
        unroll<D + 1>([&](auto J) {
            constexpr int j = decltype(J)::value;
            const int kk = k + j;
            load_a(min(kk + D, nk - 1), aa[(j + D) % (D + 1)]);
            load_b<NCT>(brow, min(kk + D, nk - 1), quarter, bb[(j + D) % (D + 1)]);
            mma(kk & 1, bb[j]);
            store_a(aa[(j + 1) % (D + 1)], (kk + 1) & 1);
            __syncthreads();
        });
    }
    // the last nk - k (< D + 1) steps: everything is loaded already
    const int r = nk - k;
    unroll<D + 1>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if (j < r) {
            mma((k + j) & 1, bb[j]);
            if (j + 1 < r) {
                store_a(aa[(j + 1) % (D + 1)], (k + j + 1) & 1);
                __syncthreads();
            }
        }
    });
}

// Tile descriptor written by the plan: x = group | n_tile << 11 | rows << 22
// (x < 0: no tile for this workgroup), y = first entry of the tile's rows
// (in the pair list for a routed expert, the first token for the shared one).
struct TileDesc {
    int g, n, rows, first;
};

__device__ __forceinline__ bool read_desc(const int2 *desc, TileDesc &d)
{
    const int2 v = desc[blockIdx.x];
    if (v.x < 0) return false;
    d.g = v.x & 2047;
    d.n = (v.x >> 11) & 2047;
    d.rows = v.x >> 22;
    d.first = v.y;
    return true;
}

// ---------------------------------------------------------------- router GEMM
// part[p][T, E] = x[T, Hp] Wr[E, Hp]^T over the p-th of P slices of H (kper
// columns each).  Workgroup: 4 waves, 64 tokens x 128 experts (two 16-expert
// column tiles per wave); grid = P x ceil(T/64) x ceil(E/128).  Splitting H
// gives the small router enough workgroups and a short k loop each; the
// slices are summed in a fixed order by the top-k launch (k_topk_sum).
__global__ __launch_bounds__(kRouterBlock) __attribute__((amdgpu_waves_per_eu(2, 2))) void
k_pf_router(const f16 *__restrict__ x, const f16 *__restrict__ wr, int T, int H, int E, int kper,
            float *__restrict__ part)
{
    constexpr int MT = kRouterRows / 16;
    constexpr int SL = stage_loads<kRouterWaves, MT>();
    __shared__ f16 lds[2 * kRouterRows * kLdsRow];
    const int mtiles = (T + kRouterRows - 1) / kRouterRows;
    const int ntiles = (E + 127) / 128;
    const int b = blockIdx.x;
    const int m0 = (b % mtiles) * kRouterRows;
    const int c0 = ((b / mtiles) % ntiles) * 128 + 32 * (threadIdx.x >> 6);
    const int split = b / (mtiles * ntiles);
    const int h0 = split * kper;
    const int t = threadIdx.x, lane = t & 63;
    const int rows = min(kRouterRows, T - m0);
    const bool active = c0 < E;
    const f16 *brow[2] = {wr + (size_t)min(c0 + (lane & 15), E - 1) * H + h0,
                          wr + (size_t)min(c0 + 16 + (lane & 15), E - 1) * H + h0};
    f16x8 bb[kDepth + 1][2][2];
    load_b<2>(brow, 0, lane >> 4, bb[0]);
    const uint32_t x_bytes = (uint32_t)T * H * 2;
    TokRows<SL> arows = tok_rows<SL>(x, x_bytes);
#pragma unroll
    for (int i = 0; i < SL; ++i) {
        const int r = t / 8 + 8 * kRouterWaves * i;
        arows.off[i] = r < rows ? (uint32_t)((m0 + r) * H + h0) * 2 : x_bytes;
    }
    f32x4 acc[MT][2] = {};
    mfma_rows<kRouterWaves, MT, 2, kDepth>(arows, brow, kper, lds, bb, acc);
    if (!active) return;
    float *out = part + (size_t)split * T * E;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int col = c0 + 16 * ct + (lane & 15);
        if (col >= E) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + acc_row(lane, r);
                if (i < rows) out[(size_t)(m0 + i) * E + col] = acc[mt][ct][r];
            }
    }
}

// ---------------------------------------------------------------- plan
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}

// Exclusive prefix sum over the workgroup's threads in thread order; `total`
// receives the sum of all.  buf: kPlanThreads / 64 ints of LDS.
__device__ int block_exclusive_scan(int v, int *buf, int &total)
{
    constexpr int kWaves = kPlanThreads / 64;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) buf[w] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int wt = buf[i];
        if (i < w) before += wt;
        total += wt;
    }
    __syncthreads();
    return before + incl - v;
}

// Descriptors of tiles tau in [0, total) for workgroups f in [0, grid): tau =
// (f % 8) * ceil(total / 8) + f / 8, so workgroup f (which the dispatcher
// places on XCD f % 8) takes a run of consecutive tiles of that XCD's share;
// the tiles of one (group, column tile) are consecutive.  The group of tile
// tau (the largest g with ts[g] <= tau) comes from a table gof in LDS filled
// group by group when total <= kGofCap (the shared expert's long run, group
// `wide`, by every thread), else from a binary search over ts.  Every thread
// of the workgroup must call this.
constexpr int kGofCap = 8192;
__device__ void write_descs(const int *ts, int ngroups, int wide, const int *rows_of,
                            const int *first_of, int total, int grid, int2 *desc, short *gof)
{
    const bool table = total <= kGofCap;
    if (table) {
        for (int g = threadIdx.x; g < ngroups; g += kPlanThreads)
            if (g != wide)
                for (int tau = ts[g]; tau < ts[g + 1]; ++tau) gof[tau] = (short)g;
        if (wide >= 0 && wide < ngroups)
            for (int tau = ts[wide] + threadIdx.x; tau < ts[wide + 1]; tau += kPlanThreads)
                gof[tau] = (short)wide;
    }
    __syncthreads();
    const int per_xcd = (total + 7) / 8;
    for (int f = threadIdx.x; f < grid; f += kPlanThreads) {
        const int slot = f / 8;
        const int tau = (f % 8) * per_xcd + slot;
        int2 v = make_int2(-1, 0);
        if (slot < per_xcd && tau < total) {
            int lo = 0, hi = ngroups - 1; // largest g with ts[g] <= tau
            if (table) {
                lo = gof[tau];
            } else {
                while (lo < hi) {
                    const int mid = (lo + hi + 1) / 2;
                    if (ts[mid] <= tau) lo = mid;
                    else hi = mid - 1;
                }
            }
            const int g = lo;
            const int n_rows = rows_of[g];
            const int mtiles = (n_rows + kBM - 1) / kBM;
            const int local = tau - ts[g];
            const int m = local % mtiles;
            const int n = local / mtiles;
            const int rows = min(kBM, n_rows - m * kBM);
            v.x = g | (n << 11) | (rows << 22);
            v.y = first_of[g] + m * kBM;
        }
        desc[f] = v;
    }
    __syncthreads(); // gof is reused by the next call
}

// One workgroup: counts the (token, slot) pairs of each expert, lists them
// expert by expert (perm), and writes the W13 and W2 tile descriptors; the
// shared expert (when present) is group E of both, with every token.
// Entries with an expert id outside [0, E) are dropped (ids are a
// precondition; this only keeps a bad id from indexing out of bounds).
__global__ __launch_bounds__(kPlanThreads) void k_pf_plan(const int32_t *__restrict__ ids, int T,
                                                          int K, int E, int nt13, int nt13_shared,
                                                          int nt2, int shared, int grid13,
                                                          int grid2,
                                                          int32_t *__restrict__ perm,
                                                          PrefillPlan *__restrict__ plan,
                                                          int2 *__restrict__ desc13,
                                                          int2 *__restrict__ desc2)
{
    __shared__ int cnt[kMaxExperts + 1];
    __shared__ int first[kMaxExperts + 1];
    __shared__ int cursor[kMaxExperts];
    __shared__ int ts13[kMaxExperts + 2];
    __shared__ int ts2[kMaxExperts + 2];
    __shared__ int buf[kPlanThreads / 64];
    // the pair list, when one pass covers every pair: scattered here and
    // written out in order (scattered 4-byte global stores from one workgroup
    // cost several times more)
    __shared__ int sperm[kPlanThreads * kPlanIds];
    const int t = threadIdx.x;
    const int pairs = T * K;
    const bool one_pass = pairs <= kPlanThreads * kPlanIds;
    for (int e = t; e < E; e += kPlanThreads) cnt[e] = 0;
    __syncthreads();
    // ids are read kPlanIds per thread at a time, all loads issued before the
    // LDS atomics that use them; with one pass they stay in registers for the
    // listing below
    int e0[kPlanIds];
#pragma unroll
    for (int i = 0; i < kPlanIds; ++i) e0[i] = -1;
    for (int base = 0; base < pairs; base += kPlanThreads * kPlanIds) {
        int e[kPlanIds];
#pragma unroll
        for (int i = 0; i < kPlanIds; ++i) {
            const int p = base + i * kPlanThreads + t;
            e[i] = p < pairs ? ids[p] : -1;
        }
#pragma unroll
        for (int i = 0; i < kPlanIds; ++i) {
            e0[i] = e[i];
            if ((unsigned)e[i] < (unsigned)E) atomicAdd(&cnt[e[i]], 1);
        }
    }
    __syncthreads();
    const int c = t < E ? cnt[t] : 0;
    const int mt = (c + kBM - 1) / kBM;
    int n_pairs, tot13, tot2;
    const int st = block_exclusive_scan(c, buf, n_pairs);
    const int s13 = block_exclusive_scan(mt * nt13, buf, tot13);
    const int s2 = block_exclusive_scan(mt * nt2, buf, tot2);
    if (t < E) {
        first[t] = st;
        cursor[t] = st;
        ts13[t] = s13;
        ts2[t] = s2;
        plan->count[t] = c;
        plan->start[t] = st;
    }
    const int shared_mt = shared ? (T + kBM - 1) / kBM : 0;
    const int groups = E + (shared ? 1 : 0);
    if (t == 0) {
        cnt[E] = T; // the shared expert: every token, in order
        first[E] = 0;
        ts13[E] = tot13;
        ts13[groups] = tot13 + shared_mt * nt13_shared;
        ts2[E] = tot2;
        ts2[groups] = tot2 + shared_mt * nt2;
        plan->total13 = tot13 + shared_mt * nt13_shared;
        plan->total2 = tot2 + shared_mt * nt2;
        plan->pairs = n_pairs;
    }
    __syncthreads();
    if (one_pass) {
#pragma unroll
        for (int i = 0; i < kPlanIds; ++i)
            if ((unsigned)e0[i] < (unsigned)E) sperm[atomicAdd(&cursor[e0[i]], 1)] = i * kPlanThreads + t;
        __syncthreads();
        for (int q = t; q < n_pairs; q += kPlanThreads) perm[q] = sperm[q];
    } else {
        for (int base = 0; base < pairs; base += kPlanThreads * kPlanIds) {
            int e[kPlanIds];
#pragma unroll
            for (int i = 0; i < kPlanIds; ++i) {
                const int p = base + i * kPlanThreads + t;
                e[i] = p < pairs ? ids[p] : -1;
            }
#pragma unroll
            for (int i = 0; i < kPlanIds; ++i)
                if ((unsigned)e[i] < (unsigned)E)
                    perm[atomicAdd(&cursor[e[i]], 1)] = base + i * kPlanThreads + t;
        }
    }
    __shared__ short gof[kGofCap];
    const int wide = shared ? E : -1;
    write_descs(ts13, groups, wide, cnt, first, ts13[groups], grid13, desc13, gof);
    write_descs(ts2, groups, wide, cnt, first, ts2[groups], grid2, desc2, gof);
}

// ---------------------------------------------------------------- W13 + SiLU
// Tile: 128 rows of one group x 16 kGemmWaves activation columns; wave w owns
// columns j = 16 (kGemmWaves n + w) + [0, 16): gate rows j (column tile 0) and up rows
// Ig + j (column tile 1), so silu(gate) * up pairs accumulator elements lane
// by lane.  Routed expert g < E: rows are pairs p from perm, token p / K,
// output act[p, j] (fp16, [T*K, I]).  Group E is the shared expert: rows are
// tokens, weights w_gate_up [2 Is, H], output act_s[t, j] (fp16, [T, Is]).
__global__ __launch_bounds__(64 * kGemmWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void
k_pf_w13(const f16 *__restrict__ x, const f16 *__restrict__ w13, const f16 *__restrict__ wsgu,
         int T, int H, int E, int I, int K, int Is, const int32_t *__restrict__ perm,
         const int2 *__restrict__ desc, f16 *__restrict__ act, f16 *__restrict__ act_s)
{
    constexpr int MT = kBM / 16;
    constexpr int SL = stage_loads<kGemmWaves, MT>();
    __shared__ f16 lds[2 * kBM * kLdsRow];
    __shared__ int rid[64 * kGemmWaves > kBM ? 64 * kGemmWaves : kBM]; // rows kBM.. unread
    TileDesc d;
    if (!read_desc(desc, d)) return;
    const int t = threadIdx.x, lane = t & 63;
    const bool shared = d.g == E;
    const int Ig = shared ? Is : I;
    const f16 *wbase = shared ? wsgu : w13 + (size_t)d.g * 2 * I * H;
    const int j0 = d.n * (16 * kGemmWaves) + 16 * (t >> 6);
    const bool active = j0 < Ig;
    const int j = min(j0 + (lane & 15), Ig - 1);
    const f16 *brow[2] = {wbase + (size_t)j * H, wbase + (size_t)(Ig + j) * H};
    // The tile's pair-list entry is requested before the first weight step
    // and stored unconditionally (threads past the tile's rows store into the
    // unread tail of rid): a wave's vector loads complete in issue order, so
    // an entry requested after the weights, or stored under a branch, would
    // wait for them, and the token rows could not be requested until then.
    const int pv = perm[d.first + min(t, max(d.rows - 1, 0))];
    f16x8 bb[kDepth + 1][2][2];
    load_b<2>(brow, 0, lane >> 4, bb[0]);
    rid[t] = t < d.rows ? (shared ? d.first + t : pv) : -1;
    __syncthreads();
    const uint32_t x_bytes = (uint32_t)T * H * 2;
    TokRows<SL> arows = tok_rows<SL>(x, x_bytes);
#pragma unroll
    for (int i = 0; i < SL; ++i) {
        const int r = t / 8 + 8 * kGemmWaves * i;
        const int q = rid[r];
        arows.off[i] = q >= 0 ? (uint32_t)(shared ? q : q / K) * H * 2 : x_bytes;
    }
    f32x4 acc[MT][2] = {};
    mfma_rows<kGemmWaves, MT, 2, kDepth>(arows, brow, H, lds, bb, acc);
    if (!active) return;
    f16 *out = shared ? act_s : act;
    const int col = j0 + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * mt + acc_row(lane, r);
            if (i < d.rows)
                out[(size_t)rid[i] * Ig + col] = (f16)silu_times(acc[mt][0][r], acc[mt][1][r]);
        }
}

// ---------------------------------------------------------------- W2
// Tile: 128 rows of one group x 32 kGemmWaves output columns h; wave w owns
// h = 32 (kGemmWaves n + w) + 16 ct + [0, 16).  Routed expert g < E:
// down[p, h] = sum_j W2[g, h, j] act[p, j] (fp32, row p of [T*K + T, H]).
// Group E, the shared expert: down[T*K + t, h] = sum_j Wsd[h, j] act_s[t, j].
__global__ __launch_bounds__(64 * kGemmWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void
k_pf_w2(const f16 *__restrict__ act, const f16 *__restrict__ act_s, const f16 *__restrict__ w2,
        const f16 *__restrict__ wsd, int T, int H, int E, int I, int K, int Is,
        const int32_t *__restrict__ perm, const int2 *__restrict__ desc,
        float *__restrict__ down)
{
    constexpr int MT = kBM / 16;
    constexpr int SL = stage_loads<kGemmWaves, MT>();
    __shared__ f16 lds[2 * kBM * kLdsRow];
    __shared__ int rid[64 * kGemmWaves > kBM ? 64 * kGemmWaves : kBM]; // rows kBM.. unread
    TileDesc d;
    if (!read_desc(desc, d)) return;
    const int t = threadIdx.x, lane = t & 63;
    const bool shared = d.g == E;
    const int kdim = shared ? Is : I;
    const f16 *wbase = shared ? wsd : w2 + (size_t)d.g * H * I;
    const int c0 = d.n * (32 * kGemmWaves) + 32 * (t >> 6);
    const bool active = c0 < H;
    const f16 *brow[2] = {wbase + (size_t)min(c0 + (lane & 15), H - 1) * kdim,
                          wbase + (size_t)min(c0 + 16 + (lane & 15), H - 1) * kdim};
    // the pair-list entry before the first weight step, as in k_pf_w13
    const int pv = perm[d.first + min(t, max(d.rows - 1, 0))];
    f16x8 bb[kDepth + 1][2][2];
    load_b<2>(brow, 0, lane >> 4, bb[0]);
    rid[t] = t < d.rows ? (shared ? d.first + t : pv) : -1;
    __syncthreads();
    const uint32_t a_bytes = shared ? (uint32_t)T * Is * 2 : (uint32_t)T * K * I * 2;
    TokRows<SL> arows = tok_rows<SL>(shared ? act_s : act, a_bytes);
#pragma unroll
    for (int i = 0; i < SL; ++i) {
        const int q = rid[t / 8 + 8 * kGemmWaves * i];
        arows.off[i] = q >= 0 ? (uint32_t)q * kdim * 2 : a_bytes;
    }
    f32x4 acc[MT][2] = {};
    mfma_rows<kGemmWaves, MT, 2, kDepth>(arows, brow, kdim, lds, bb, acc);
    if (!active) return;
    const size_t row_base = shared ? (size_t)T * K : 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * mt + acc_row(lane, r);
            if (i >= d.rows) continue;
            float *orow = down + (row_base + rid[i]) * H + c0 + (lane & 15);
            orow[0] = acc[mt][0][r];
            orow[16] = acc[mt][1][r];
        }
}

// ---------------------------------------------------------------- combine
// y[t, h] = fp16( sum_k w[t, k] down[t K + k, h] (k in routing order, fp32)
//                 + down[T K + t, h] (the shared expert, when present) ),
// four consecutive h per thread.
__global__ __launch_bounds__(256) void k_pf_combine(const float *__restrict__ down,
                                                    const float *__restrict__ tw, int T, int H,
                                                    int K, int shared, f16 *__restrict__ y)
{
    const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int hq = H / 4;
    if (i4 >= (size_t)T * hq) return;
    const int tok = (int)(i4 / hq);
    const int h = (int)(i4 % hq) * 4;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < K; ++k) {
        const float wk = tw[(size_t)tok * K + k];
        const f32x4 dk = *reinterpret_cast<const f32x4 *>(down + ((size_t)tok * K + k) * H + h);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = fmaf(wk, dk[c], v[c]);
    }
    if (shared) {
        const f32x4 s = *reinterpret_cast<const f32x4 *>(down + ((size_t)T * K + tok) * H + h);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] += s[c];
    }
    typedef f16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = (f16)v[c];
    *reinterpret_cast<f16x4 *>(y + (size_t)tok * H + h) = o;
}

inline hipError_t last() { return hipGetLastError(); }

constexpr int round8(long long n) { return (int)((n + 7) / 8 * 8); }
// H slices of the router GEMM: a whole number of k steps each, at least 8,
// at most 4 slices
constexpr int router_split(int H)
{
    return (H / kBK) % 4 == 0 && H / kBK >= 32 ? 4 : (H / kBK) % 2 == 0 && H / kBK >= 16 ? 2 : 1;
}
constexpr int w13_col_tiles(int I) { return (I + 16 * kGemmWaves - 1) / (16 * kGemmWaves); }
constexpr int w2_col_tiles(int H) { return (H + 32 * kGemmWaves - 1) / (32 * kGemmWaves); }

} // namespace

PrefillLayout prefill_layout(int T, int H, int E, int I, int K, int Is)
{
    PrefillLayout L{};
    const long long pairs = (long long)T * K;
    // sum over experts of ceil(n_e / kBM) is at most this
    const long long max_row_tiles = (pairs + kBM - 1) / kBM + E;
    const long long shared_row_tiles = Is > 0 ? (T + kBM - 1) / kBM : 0;
    L.grid13 = round8(max_row_tiles * w13_col_tiles(I) + shared_row_tiles * w13_col_tiles(Is));
    L.grid2 = round8((max_row_tiles + shared_row_tiles) * w2_col_tiles(H));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    L.router_split = router_split(H);
    L.plan = take(sizeof(PrefillPlan));
    L.part = take((size_t)L.router_split * T * E * 4);
    L.desc13 = take((size_t)L.grid13 * 8);
    L.desc2 = take((size_t)L.grid2 * 8);
    L.perm = take((size_t)pairs * 4);
    L.act = take((size_t)pairs * I * 2);
    L.act_s = take((size_t)T * Is * 2);
    L.down = take((size_t)(pairs + (Is > 0 ? T : 0)) * H * 4);
    L.bytes = off;
    return L;
}

hipError_t launch_prefill(const void *x, const void *wr, const void *w13, const void *w2,
                          const void *wsgu, const void *wsd, int T, int H, int E, int I, int K,
                          int Is, int renorm, int32_t *ids, float *w, float *logits, void *y,
                          void *ws, int stage, hipStream_t s)
{
    const PrefillLayout L = prefill_layout(T, H, E, I, K, Is);
    char *base = static_cast<char *>(ws);
    PrefillPlan *plan = reinterpret_cast<PrefillPlan *>(base + L.plan);
    int2 *desc13 = reinterpret_cast<int2 *>(base + L.desc13);
    int2 *desc2 = reinterpret_cast<int2 *>(base + L.desc2);
    int32_t *perm = reinterpret_cast<int32_t *>(base + L.perm);
    f16 *act = reinterpret_cast<f16 *>(base + L.act);
    f16 *act_s = reinterpret_cast<f16 *>(base + L.act_s);
    float *down = reinterpret_cast<float *>(base + L.down);
    const int P = L.router_split;
    const int router_tiles = P * ((T + kRouterRows - 1) / kRouterRows) * ((E + 127) / 128);
    float *part = reinterpret_cast<float *>(base + L.part);
    hipError_t err = hipSuccess;
    if (stage == 0 || stage == 1) {
        hipLaunchKernelGGL(k_pf_router, dim3(router_tiles), dim3(kRouterBlock), 0, s,
                           (const f16 *)x, (const f16 *)wr, T, H, E, H / P, part);
        if ((err = last()) != hipSuccess) return err;
    }
    if (stage == 0 || stage == 2) {
        // the slices summed in a fixed order into logits, then the selection
        if ((err = launch_topk_sum(part, P, T, E, K, renorm, logits, ids, w, s)) != hipSuccess)
            return err;
    }
    if (stage == 0 || stage == 3) {
        hipLaunchKernelGGL(k_pf_plan, dim3(1), dim3(kPlanThreads), 0, s, ids, T, K, E,
                           w13_col_tiles(I), w13_col_tiles(Is), w2_col_tiles(H), Is > 0 ? 1 : 0,
                           L.grid13, L.grid2, perm, plan, desc13, desc2);
        if ((err = last()) != hipSuccess) return err;
    }
    if (stage == 0 || stage == 4) {
        hipLaunchKernelGGL(k_pf_w13, dim3(L.grid13), dim3(64 * kGemmWaves), 0, s, (const f16 *)x,
                           (const f16 *)w13, (const f16 *)wsgu, T, H, E, I, K, Is, perm, desc13,
                           act, act_s);
        if ((err = last()) != hipSuccess) return err;
    }
    if (stage == 0 || stage == 5) {
        hipLaunchKernelGGL(k_pf_w2, dim3(L.grid2), dim3(64 * kGemmWaves), 0, s, act, act_s,
                           (const f16 *)w2, (const f16 *)wsd, T, H, E, I, K, Is, perm, desc2,
                           down);
        if ((err = last()) != hipSuccess) return err;
    }
    if (stage == 0 || stage == 6) {
        hipLaunchKernelGGL(k_pf_combine, dim3((unsigned)(((size_t)T * (H / 4) + 255) / 256)),
                           dim3(256), 0, s, down, w, T, H, K, Is > 0 ? 1 : 0, (f16 *)y);
        if ((err = last()) != hipSuccess) return err;
    }
    return hipSuccess;
}

} // namespace moe
