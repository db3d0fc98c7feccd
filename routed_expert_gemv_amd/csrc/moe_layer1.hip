// moe_layer1.hip -- the whole single-token MoE layer in ONE launch on gfx950.
//
// What it computes is the decode layer of the BI-V100 inference worklog
// ("如何在天垓 BI-V100 上优化大模型推理：一份工作日志"): part 8, routing is a
// top-k and a softmax; part 10, W13 GEMV over W13[expert_ids[k]] -> gate/up ->
// SiLU*mul, W2 GEMV over W2[expert_ids[k]] with the weighted sum; part 2, the
// shared expert.  Part 9's launch-reduction route ends at one kernel per
// layer; this is that kernel, designed for the MI355X's 8 XCDs:
//
//   * 256 workgroups of 16 waves, one per CU.  The dispatcher deals a
//     launch's workgroups to the 8 XCDs round-robin from where the previous
//     launch stopped, so each XCD gets 32 of them with distinct b / 8; each
//     workgroup reads its XCD from the XCC_ID hardware register.  If the
//     placement is ever different, some hand-off flags never arrive and those
//     waits give up (below), which changes the speed and not the results;
//   * router: each XCD computes all E logits itself (its 32 workgroups, one
//     row per wave) and hands them over through its own L2: plain stores, a
//     per-workgroup flag, sc1 (device-coherent) polls.  No atomics in the
//     hand-offs (only a wait that gives up counts itself with one): every
//     workgroup keeps its own call counter (epoch) in the workspace, all
//     counters advance in lockstep, and a flag is current when it holds this
//     call's epoch;
//   * each workgroup then selects the experts itself (only as many top-k
//     rounds as its own gate/up rows need before it requests them);
//   * gate/up: one row pair per wave (K*I pairs over 4096 waves), SiLU*mul in
//     registers; the shared expert's gate/up and down rows are requested
//     before any routing is known, and the routed down rows as soon as the
//     workgroup has all K expert ids, before the activation hand-off;
//   * the activations cross the XCDs once: write-through (sc1) stores, one
//     flag per workgroup, sc1 polls; the W2 rows are already in flight, so the
//     hand-off overlaps the W2 stream;
//   * down rows and combine: the arithmetic of the three-launch path (a wave
//     per output row, the routing weights folded in before the one reduction,
//     the shared row added last, one fp16 rounding), so the results are the
//     same bits.
// Every wait is bounded.  A wait that gives up computes what it waited for
// itself, with the same device functions (so the results do not change), and
// counts the event in the workspace; every workgroup always runs to its end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kL1Waves = 16;
constexpr int kL1Block = kL1Waves * kWave;
constexpr int kL1Slots = kLayer1Grid * kL1Waves; // waves in the launch
constexpr int kDownWaves = 8;                    // waves 0..7 routed rows, 8..15 shared rows
constexpr int kSc1 = 16;                         // buffer cache policy: device scope (sc1)
constexpr int kMaxPairsPerWave = 2;
constexpr int kMaxSharedPerWg = kL1Waves / 2;    // shared gate/up pairs per workgroup (waves 15..8)
// activations [K*I + Is] <= 2*4096 + 2048 fp32, 16-byte chunks per thread of waves 8..15
constexpr int kActChunks = (kMaxPairsPerWave * kL1Slots + kLayer1Grid * kMaxSharedPerWg + 4 * kDownWaves * kWave - 1) / (4 * kDownWaves * kWave);

__device__ __forceinline__ unsigned xcc_id()
{
    return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u; // HW_REG_XCC_ID, bits [3:0]
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             kBufferWord3);
}

// 16-byte chunk `chunk` of a weight row through a buffer resource, non-temporal.
// A resource of zero bytes (a row this wave does not own) returns zeros and
// reads nothing: every wave issues the same loads, so the compiler's counts of
// loads in flight stay exact and no wait covers a later load than it needs.
constexpr int kNt = 2; // buffer cache policy: non-temporal
__device__ __forceinline__ f16x8 ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kNt));
}

__device__ __forceinline__ f16x8 row_chunk(__amdgpu_buffer_rsrc_t r, int chunk)
{
    return ld16_nt(r, (uint32_t)chunk * 16);
}

template <int HC>
__device__ __forceinline__ void load_row_if(const f16 *row, bool valid, f16x8 (&w)[HC])
{
    const __amdgpu_buffer_rsrc_t r = rsrc(row, valid ? HC * 1024 : 0);
#pragma unroll
    for (int c = 0; c < HC; ++c) w[c] = row_chunk(r, c * kWave + lane_id());
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st_u32(unsigned *p, unsigned v, bool sc1)
{
    if (sc1) __builtin_amdgcn_raw_buffer_store_b32(v, rsrc(p, 4), 0, 0, kSc1);
    else *p = v;
}

__device__ __forceinline__ void st_f32(float *p, float v, bool sc1)
{
    if (sc1) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rsrc(p, 4), 0, 0, kSc1);
    else *p = v;
}

// Barrier for LDS hand-offs between the waves of a workgroup; loads in flight
// (the prefetched weight rows) are not waited for.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The vmcnt(0) wait: every vector memory operation of this wave has completed
// (stores acknowledged).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0); }

// Row j of the gate/up pairs a wave owns: pair p of K*I routed pairs is
// (slot p / I, row p % I).  contig: p = 16*b + wave + 4096*i (one slot per
// workgroup and i when 16 | I); spread: p = b + 256*(wave + 16*i).
__device__ __forceinline__ int pair_index(bool contig, int b, int wave, int i)
{
    return contig ? kL1Waves * b + wave + kL1Slots * i : b + kLayer1Grid * (wave + kL1Waves * i);
}

// Per-call arguments.
struct L1Args {
    const f16 *x, *wr, *w13, *w2, *wsgu, *wsd;
    int E, I, K, Is, renorm, contig;
    int32_t *ids_out;
    float *w_out, *logits_out;
    f16 *y;
    Layer1State *st;
    float *logits_x; // [8][E] per-XCD logits
    float *act_pub;  // [K*I + Is] activations published across XCDs
    unsigned spin;   // poll limit per wait
};

template <int HC, int NPL, int LPR, int CPL, int KMAX, bool SH, int PPW>
__global__ __launch_bounds__(kL1Block) void k_layer1(const L1Args a)
{
    constexpr int H = 512 * HC;
    constexpr int RPL = kWave / LPR;
    constexpr bool kTwoRouterRows = NPL > 2 * kL1Waves * kPerXcd / (2 * kWave); // E > 512
    extern __shared__ float s_act[]; // [K*I + Is] every activation of the layer
    __shared__ int s_ids[KMAX];
    __shared__ float s_w[KMAX];
    __shared__ float s_mine[kL1Waves * kMaxPairsPerWave + kMaxSharedPerWg];
    __shared__ float s_sadd[kDownWaves * kWave];
    __shared__ int s_gave_up;

    // The dispatcher deals the workgroups of a launch to the XCDs round-robin,
    // continuing where the previous launch stopped: workgroup b runs on XCD
    // (b + c) % 8 for one c per launch, so b / 8 numbers the 32 workgroups of
    // each XCD 0..31 whatever c is.  The XCD itself comes from the hardware.
    const int b = blockIdx.x;
    const unsigned xhw = xcc_id();
    const bool placed = xhw < 8u; // else: every wait below gives up at once
    const int xc = (int)(xhw & 7u), r = b >> 3;
    // wave-uniform values (readfirstlane) keep the buffer descriptors in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = lane_id();
    const int E = a.E, I = a.I, K = a.K, Is = a.Is;
    const int pr = K * I; // routed row pairs
    const unsigned e = a.st->epoch[b] + 1u; // this call's epoch
    const int rpw = H / kLayer1Grid;         // output rows per workgroup
    const int groups = rpw / RPL;            // row groups (one per down wave)

    // ---- phase 0: every request that needs no routing ---------------------
    f16x8 xv[HC];
    load_x<HC>(a.x, xv);
    // router rows of this XCD's copy: row (wave + 16*i)*32 + r
    const int rrow0 = wave * kPerXcd + r;
    const int rrow1 = (wave + kL1Waves) * kPerXcd + r;
    const bool has_r0 = rrow0 < E, has_r1 = kTwoRouterRows && rrow1 < E;
    f16x8 rw0[HC], rw1[HC];
    load_row_if<HC>(a.wr + (size_t)(has_r0 ? rrow0 : 0) * H, has_r0, rw0);
    if constexpr (kTwoRouterRows) load_row_if<HC>(a.wr + (size_t)(has_r1 ? rrow1 : 0) * H, has_r1, rw1);
    __builtin_amdgcn_sched_barrier(0); // the router rows go out first (the critical path)
    // shared gate/up pair t = 15 - wave: row j = b + 256*t
    const int sh_t = kL1Waves - 1 - wave;
    const int sh_j = b + kLayer1Grid * sh_t;
    const bool has_sp = SH && sh_t < kMaxSharedPerWg && sh_j < Is;
    f16x8 sg[HC], su[HC];
    if constexpr (SH) {
        load_row_if<HC>(a.wsgu + (size_t)(has_sp ? sh_j : 0) * H, has_sp, sg);
        load_row_if<HC>(a.wsgu + (size_t)(has_sp ? Is + sh_j : 0) * H, has_sp, su);
    }
    // shared down rows: group wave - 8 (RPL rows, LPR lanes per row)
    const int dgroup = wave & (kDownWaves - 1);
    const bool down_wave = dgroup < groups;
    const int h0 = b * rpw + dgroup * RPL; // the group's first row
    const int h = h0 + lane / LPR;
    const int cl = lane % LPR;
    f16x8 sv[CPL];
    if constexpr (SH) {
        const bool mine = wave >= kDownWaves && down_wave;
        const __amdgpu_buffer_rsrc_t sr =
            rsrc(a.wsd + (size_t)(mine ? h0 : 0) * Is, mine ? RPL * Is * 2 : 0);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            sv[c] = ld16_nt(sr, (uint32_t)((lane / LPR) * Is * 2 + (c * LPR + cl) * 16));
    }

    // ---- phase 1: router rows -> this XCD's logits --------------------------
    if (has_r0 || has_r1) {
        if (has_r0) {
            const float t = row_dot<HC>(rw0, xv);
            if (lane == 0) {
                st_f32(a.logits_x + (size_t)xc * E + rrow0, t, !placed);
                if (xc == 0) a.logits_out[rrow0] = t;
            }
        }
        if (has_r1) {
            const float t = row_dot<HC>(rw1, xv);
            if (lane == 0) {
                st_f32(a.logits_x + (size_t)xc * E + rrow1, t, !placed);
                if (xc == 0) a.logits_out[rrow1] = t;
            }
        }
        wait_vm_all(); // the logits are in this XCD's L2 before the flag goes out
    }
    lds_barrier(); // B1: every router row of this workgroup is stored

    // the shared gate/up pair (rows requested first thing), while wave 0 waits
    // for the logits: its data is in by now, and computing it after the gate/up
    // rows are requested would wait behind them
    if (has_sp) {
        const float a_sh = silu_mul(row_dot<HC>(sg, xv), row_dot<HC>(su, xv));
        if (lane == 0) s_mine[kL1Waves * kMaxPairsPerWave + sh_t] = a_sh;
    }

    // ---- phase 2: wave 0 waits for the XCD's logits and selects ------------
    constexpr int ppw = PPW; // routed pairs per wave
    uint32_t key[NPL];
    int kid[NPL];
    uint32_t my_key = 0u;
    int my_id = 0;
    float v[NPL];
    if (wave == 0) {
        if (lane == 0) st_u32(&a.st->flag_route[xc][r], e, !placed);
        bool ok = false;
        if (placed) {
            const __amdgpu_buffer_rsrc_t fr = rsrc(&a.st->flag_route[xc][0], kPerXcd * 4);
            for (unsigned it = 0; it < a.spin; ++it) {
                // lanes past the XCD's 32 flags read zero through the descriptor's bound
                const unsigned f0 = __builtin_amdgcn_raw_buffer_load_b32(fr, (uint32_t)lane * 4, 0, kSc1);
                const unsigned f = lane < kPerXcd ? f0 : e;
                if (__all((int)(f - e) >= 0)) {
                    ok = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (ok) {
            const __amdgpu_buffer_rsrc_t lr = rsrc(a.logits_x + (size_t)xc * E, (uint32_t)E * 4);
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                     lr, (uint32_t)(i * kWave + lane) * 4, 0, kSc1));
        } else {
            // gave up (or placed elsewhere): every router row here, the same arithmetic
            if (lane == 0) atomicAdd(&a.st->gave_up, 1u);
#pragma unroll
            for (int i = 0; i < NPL; ++i) v[i] = 0.0f;
            for (int row = 0; row < E; ++row) {
                f16x8 w[HC];
                load_row<HC>(a.wr + (size_t)row * H, w);
                const float t = row_dot<HC>(w, xv);
#pragma unroll
                for (int i = 0; i < NPL; ++i)
                    if (row == i * kWave + lane) v[i] = t;
            }
            wait_vm_all();
        }
        // rounds needed before this workgroup's gate/up rows can be requested
        int need = K;
        if (a.contig) need = (pair_index(true, b, 0, ppw - 1) / I) + 1;
        topk_pairs<NPL>(v, E, key, kid);
        topk_sort_lane<NPL>(key, kid);
        topk_rounds<NPL>(key, kid, 0, need, my_key, my_id);
        if (lane < need) s_ids[lane] = my_id;
    }
    lds_barrier(); // B2: the first `need` expert ids

    // ---- phase 3: gate/up rows of this wave's pairs -------------------------
    f16x8 wg[PPW][HC], wu[PPW][HC];
    int pidx[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        pidx[i] = pair_index(a.contig, b, wave, i);
        const bool mine = pidx[i] < pr;
        const int u = mine ? pidx[i] / I : 0, j = mine ? pidx[i] % I : 0;
        const int eid = __builtin_amdgcn_readfirstlane(s_ids[u]);
        const f16 *base = a.w13 + (size_t)eid * 2 * I * H;
        load_row_if<HC>(base + (size_t)j * H, mine, wg[i]);
        load_row_if<HC>(base + (size_t)(I + j) * H, mine, wu[i]);
    }
    if (wave == 0) {
        int need = K;
        if (a.contig) need = (pair_index(true, b, 0, ppw - 1) / I) + 1;
        topk_rounds<NPL>(key, kid, need, K, my_key, my_id);
        if (lane < K) s_ids[lane] = my_id;
    }
    lds_barrier(); // B3: every expert id
    // the routing weights (needed only by the combine; read after B4)
    if (wave == 0) {
        const float my_l = my_key ? key_value(my_key) : 0.0f;
        const float lmax = key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
        const float wt = topk_weight_vals<NPL>(v, E, K, a.renorm, my_l, lmax);
        if (lane < K) {
            s_w[lane] = wt;
            if (b == 0) {
                a.ids_out[lane] = my_id;
                a.w_out[lane] = wt;
            }
        }
    }

    // ---- phase 4: routed down rows requested (waves 0..7) -------------------
    f16x8 dv[KMAX][CPL];
    {
        const bool rows = wave < kDownWaves && down_wave;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const bool mine = rows && k < K; // slots past K read nothing
            const int eid = __builtin_amdgcn_readfirstlane(s_ids[k < K ? k : 0]);
            const __amdgpu_buffer_rsrc_t dr =
                rsrc(a.w2 + ((size_t)eid * H + (mine ? h0 : 0)) * I, mine ? RPL * I * 2 : 0);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                dv[k][c] = ld16_nt(dr, (uint32_t)((lane / LPR) * I * 2 + (c * LPR + cl) * 16));
        }
    }
    // this wave's routed pairs -> SiLU*mul, into LDS for the publishing wave
#pragma unroll
    for (int i = 0; i < PPW; ++i)
        if (pidx[i] < pr) {
            const float g = row_dot<HC>(wg[i], xv);
            const float up = row_dot<HC>(wu[i], xv);
            if (lane == 0) s_mine[i * kL1Waves + wave] = silu_mul(g, up);
        }
    lds_barrier(); // B4: this workgroup's activations

    // ---- phase 5: publish them, wait for everyone's (wave 15) --------------
    if (wave == kL1Waves - 1) {
        // lane l < 16*ppw: pair (l / 16) of wave l % 16; then the shared pairs
        const __amdgpu_buffer_rsrc_t ar = rsrc(a.act_pub, (uint32_t)(pr + Is) * 4);
        const int i = lane / kL1Waves, wv = lane % kL1Waves;
        if (i < ppw) {
            const int p = pair_index(a.contig, b, wv, i);
            if (p < pr)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(unsigned, s_mine[i * kL1Waves + wv]), ar, (uint32_t)p * 4, 0, kSc1);
        }
        if (SH && lane >= kL1Waves * kMaxPairsPerWave) {
            const int t = lane - kL1Waves * kMaxPairsPerWave;
            const int j = b + kLayer1Grid * t;
            if (t < kMaxSharedPerWg && j < Is)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(unsigned, s_mine[kL1Waves * kMaxPairsPerWave + t]), ar,
                    (uint32_t)(pr + j) * 4, 0, kSc1);
        }
        wait_vm_all();
        if (lane == 0) st_u32(&a.st->flag_act[b], e, true);
        // One workgroup per XCD (b / 8 == 0) polls the 256 device-wide flags and
        // then raises its XCD's flag in that XCD's L2; the others poll only
        // that local flag (device-coherent polls of all 256 flags by every
        // workgroup take memory bandwidth from the W2 rows still streaming).
        bool ok = placed;
        if (ok && r == 0) {
            ok = false;
            const __amdgpu_buffer_rsrc_t fr = rsrc(a.st->flag_act, kLayer1Grid * 4);
            for (unsigned it = 0; it < a.spin; ++it) {
                // four flags per lane
                const u32x4 f = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(fr, (uint32_t)lane * 16, 0, kSc1));
                const bool mine = (int)(f[0] - e) >= 0 && (int)(f[1] - e) >= 0 &&
                                  (int)(f[2] - e) >= 0 && (int)(f[3] - e) >= 0;
                if (__all(mine)) {
                    ok = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            if (ok && lane == 0) st_u32(&a.st->flag_xact[xc][0], e, false);
        }
        if (ok) {
            ok = false;
            for (unsigned it = 0; it < a.spin; ++it) {
                const unsigned f = __builtin_amdgcn_raw_buffer_load_b32(
                    rsrc(&a.st->flag_xact[xc][0], 4), 0, 0, kSc1);
                if ((int)(f - e) >= 0) {
                    ok = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0) {
            s_gave_up = ok ? 0 : 1;
            if (!ok) atomicAdd(&a.st->gave_up, 1u);
        }
    }
    lds_barrier(); // B5
    const int n_act = pr + Is;
    if (!s_gave_up) {
        // every activation, from the other workgroups' write-through stores
        if (wave >= kDownWaves) {
            // all requests first (offsets past the end read zeros), then the LDS stores
            const int t = threadIdx.x - kDownWaves * kWave;
            const __amdgpu_buffer_rsrc_t ar = rsrc(a.act_pub, (uint32_t)n_act * 4);
            f32x4 *l4 = reinterpret_cast<f32x4 *>(s_act);
            f32x4 st[kActChunks];
#pragma unroll
            for (int i = 0; i < kActChunks; ++i)
                st[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      ar, (uint32_t)(t + i * kDownWaves * kWave) * 16, 0, kSc1));
#pragma unroll
            for (int i = 0; i < kActChunks; ++i) {
                const int q = t + i * kDownWaves * kWave;
                if (q < n_act / 4) l4[q] = st[i];
            }
        }
    } else {
        // gave up: every activation here, the same arithmetic
        for (int p = wave; p < n_act; p += kL1Waves) {
            float t;
            if (p < pr) t = w13_pair<HC>(a.x, a.w13 + (size_t)s_ids[p / I] * 2 * I * H, I, p % I);
            else t = w13_pair<HC>(a.x, a.wsgu, Is, p - pr);
            if (lane == 0) s_act[p] = t;
        }
    }
    lds_barrier(); // B6: s_act holds every activation

    // ---- phase 6: down rows, combine, one rounding --------------------------
    float tsum = 0.0f;
    if (down_wave) {
        if (wave < kDownWaves) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (k < K) {
                    const float *ak = s_act + (size_t)k * I;
                    float d = 0.0f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const f32x4 *ap = reinterpret_cast<const f32x4 *>(ak + (c * LPR + cl) * 8);
                        d = dot8_f32(dv[k][c], ap[0], ap[1], d);
                    }
                    acc = fmaf(s_w[k], d, acc);
                }
            tsum = group_sum<LPR>(acc);
        } else if (SH) {
            float d = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const f32x4 *ap = reinterpret_cast<const f32x4 *>(s_act + pr + (c * LPR + cl) * 8);
                d = dot8_f32(sv[c], ap[0], ap[1], d);
            }
            const float sadd = group_sum<LPR>(fmaf(1.0f, d, 0.0f));
            if (lane == group_holder<LPR>(lane / LPR)) s_sadd[dgroup * kWave + lane] = sadd;
        }
    }
    if (SH) lds_barrier(); // B7: the shared rows' outputs
    if (wave < kDownWaves && down_wave && lane == group_holder<LPR>(lane / LPR)) {
        const float t = SH ? tsum + s_sadd[dgroup * kWave + lane] : tsum;
        a.y[h] = (f16)t;
    }
    if (threadIdx.x == 0) a.st->epoch[b] = e;
}

constexpr size_t kLayer1Lds = 96 * 1024; // > half a CU's LDS: one workgroup per CU

struct DevInfo {
    int checked, ok;
};
DevInfo g_dev[64];

bool device_fits()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    DevInfo &d = g_dev[dev];
    if (!d.checked) {
        int cus = 0, xccs = 0, lds = 0;
        d.ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) ==
                   hipSuccess &&
               hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess &&
               hipDeviceGetAttribute(&lds, hipDeviceAttributeSharedMemPerBlockOptin, dev) ==
                   hipSuccess &&
               cus == kLayer1Grid && xccs == 8 && (size_t)lds >= kLayer1Lds;
        d.checked = 1;
    }
    return d.ok;
}

template <int HC, int NPL, int LPR, int CPL, int KMAX, bool SH, int PPW>
hipError_t launch_t(const L1Args &a, hipStream_t s)
{
    auto kern = k_layer1<HC, NPL, LPR, CPL, KMAX, SH, PPW>;
    static std::atomic<bool> opted[64] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!opted[dev].load(std::memory_order_acquire)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLayer1Lds);
        if (err != hipSuccess) return err;
        opted[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(kLayer1Grid), dim3(kL1Block), kLayer1Lds, s, a);
    return hipGetLastError();
}

// One routed row pair per wave (K*I <= 4096): with two, the register
// budget of a 1024-thread workgroup (128 per lane) spills.
template <int HC, int NPL, int LPR, int CPL, int KMAX>
hipError_t launch_p(const L1Args &a, hipStream_t s)
{
    return a.Is > 0 ? launch_t<HC, NPL, LPR, CPL, KMAX, true, 1>(a, s)
                    : launch_t<HC, NPL, LPR, CPL, KMAX, false, 1>(a, s);
}

template <int HC, int NPL, int LPR, int CPL>
hipError_t launch_k(const L1Args &a, hipStream_t s)
{
    if (a.K <= 4) return launch_p<HC, NPL, LPR, CPL, 4>(a, s);
    if constexpr (CPL == 1) return launch_p<HC, NPL, LPR, CPL, 8>(a, s);
    return hipErrorInvalidValue; // I = 1024 with K > 4 has K*I > 4096 (not this path)
}

template <int HC, int NPL>
hipError_t launch_i(const L1Args &a, hipStream_t s)
{
    switch (a.I) {
    case 64: return launch_k<HC, NPL, 8, 1>(a, s);
    case 128: return launch_k<HC, NPL, 16, 1>(a, s);
    case 256: return launch_k<HC, NPL, 32, 1>(a, s);
    case 512: return launch_k<HC, NPL, 64, 1>(a, s);
    case 1024: return launch_k<HC, NPL, 64, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int HC>
hipError_t launch_e(const L1Args &a, hipStream_t s)
{
    if (a.E <= kWave) return launch_i<HC, 1>(a, s);
    return launch_i<HC, 4>(a, s);
}

} // namespace

bool layer1_ok(int M, int H, int E, int I, int K, int Is)
{
    if (M != 1 || !device_fits()) return false;
    if (H != 1024 && H != 2048) return false;
    // E <= 256 and one routed row pair per wave keep every instance within
    // the register budget (no scratch)
    if (E < 1 || E > 4 * kWave) return false;
    if (K < 1 || K > 8 || K > E) return false;
    if (I != 64 && I != 128 && I != 256 && I != 512 && I != 1024) return false;
    if (Is != 0 && Is != I) return false;
    const int lpr = I >= 512 ? 64 : I / 8;
    const int rpl = kWave / lpr;
    const int rpw = H / kLayer1Grid;
    if (rpw % rpl != 0 || rpw / rpl > kDownWaves) return false;
    const int pr = K * I;
    if (pr > kL1Slots) return false;
    if (Is > kLayer1Grid * kMaxSharedPerWg) return false;
    if ((size_t)(pr + Is) * 4 > kLayer1Lds) return false;
    return true;
}

hipError_t launch_layer1(const void *x, const void *wr, const void *w13, const void *w2,
                         const void *wsgu, const void *wsd, int H, int E, int I, int K, int Is,
                         int renorm, int32_t *ids, float *w, float *logits, void *y, void *ws,
                         unsigned spin, hipStream_t s)
{
    char *base = static_cast<char *>(ws);
    L1Args a;
    a.x = (const f16 *)x;
    a.wr = (const f16 *)wr;
    a.w13 = (const f16 *)w13;
    a.w2 = (const f16 *)w2;
    a.wsgu = (const f16 *)wsgu;
    a.wsd = (const f16 *)wsd;
    a.E = E;
    a.I = I;
    a.K = K;
    a.Is = Is;
    a.renorm = renorm;
    a.contig = (K * I) % kL1Slots == 0;
    a.ids_out = ids;
    a.w_out = w;
    a.logits_out = logits;
    a.y = (f16 *)y;
    a.st = reinterpret_cast<Layer1State *>(base);
    a.logits_x = reinterpret_cast<float *>(base + kLayer1LogitsOffset);
    a.act_pub = reinterpret_cast<float *>(base + kLayer1ActOffset);
    a.spin = spin;
    switch (H) {
    case 1024: return launch_e<2>(a, s);
    case 2048: return launch_e<4>(a, s);
    }
    return hipErrorInvalidValue;
}

} // namespace moe

namespace moe {
namespace {
__global__ __launch_bounds__(256) void k_state_clear(unsigned *st)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) st[threadIdx.x + 256 * i] = 0u;
}
} // namespace

hipError_t launch_state_clear(void *ws, hipStream_t s)
{
    static_assert(sizeof(Layer1State) == 8 * 256 * sizeof(unsigned), "one word per thread x8");
    hipLaunchKernelGGL(k_state_clear, dim3(1), dim3(256), 0, s, static_cast<unsigned *>(ws));
    return hipGetLastError();
}
} // namespace moe
