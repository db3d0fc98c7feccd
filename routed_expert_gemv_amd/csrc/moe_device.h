// moe_device.h -- device helpers shared by the decode kernels (moe_kernels.hip)
// and the single-launch layer kernel (moe_layer1.hip): the row dot products,
// the DPP reduction trees, the top-k selection and the SiLU*mul epilogue.
// Every kernel that must agree bit for bit with another one uses these same
// functions, lane mappings and reduction orders.
#ifndef MOE_DEVICE_H
#define MOE_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of the buffer-load builtins: nontemporal (the weight
// streams are read once, as the global loads' __builtin_nontemporal_load).
constexpr int kLoadNT = 2;

// ---------------------------------------------------------------- helpers
// Staging order of a buffer of n4 16-byte chunks that every workgroup copies
// into its LDS (the activations): chunk q of the loop is chunk
// staged_chunk(q, n4, rot), the order rotated by a start that depends on the
// workgroup's place among those of its XCD (workgroups are dealt to the 8
// XCDs in turn), so that the 32 workgroups of an XCD, which copy the same
// bytes at the same time, do not request the same L2 lines at once.  Indices
// past the end map to the last chunk of the unrotated order, whose copy
// stores its own value again.
__device__ __forceinline__ int stage_rotation(int n4)
{
    return (int)(((blockIdx.x >> 3) & 31u) * (unsigned)(n4 >> 5));
}
__device__ __forceinline__ int staged_chunk(int q, int n4, int rot)
{
    const int x = (q < n4 ? q : n4 - 1) + rot;
    return x >= n4 ? x - n4 : x;
}

// Element h of rows 0..MT-1 of an [M, H] fp32 tensor (the shared-expert
// output that the W2 kernels add after their combine), 0 for rows past M or
// for a null tensor.  The W2 kernels request it before their weight stream:
// a load after the combine would cost every wave a full memory latency per
// token at its end.  The loads go through a buffer range that is empty for a
// null tensor and ends at row M, so every load is issued unconditionally and
// none touches memory outside the tensor.
template <int MT>
__device__ __forceinline__ void load_column(const float *t, int M, int H, int h, float (&v)[MT])
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(t), (short)0, t ? M * H * (int)sizeof(float) : 0, kBufferWord3);
#pragma unroll
    for (int m = 0; m < MT; ++m)
        v[m] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(m * H + h) * 4u, 0, 0));
}

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

// ---------------------------------------------------------------- router GEMV
// Lane l holds 16-byte chunks c*64 + l of a 2048-wide (H = 512*HC) row.
template <int HC>
__device__ __forceinline__ void load_row(const f16 *row, f16x8 (&w)[HC])
{
    const f16x8 *r = reinterpret_cast<const f16x8 *>(row);
#pragma unroll
    for (int c = 0; c < HC; ++c) w[c] = stream_load(r + c * kWave + lane_id());
}

template <int HC>
__device__ __forceinline__ void load_x(const f16 *xrow, f16x8 (&xv)[HC])
{
    const f16x8 *r = reinterpret_cast<const f16x8 *>(xrow);
#pragma unroll
    for (int c = 0; c < HC; ++c) xv[c] = r[c * kWave + lane_id()];
}

// sum over the row of w * x: per-lane v_dot2 chain over its chunks, then the wave tree
template <int HC>
__device__ __forceinline__ float row_dot(const f16x8 (&w)[HC], const f16x8 (&xv)[HC])
{
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < HC; ++c) acc = dot8(w[c], xv[c], acc);
    return wave_sum(acc);
}

// ---------------------------------------------------------------- top-k + softmax
// One wave selects for one token.  A finite fp32 logit maps to an
// order-preserving non-zero uint32 key (0 marks "no entry"); K rounds of a
// wave-wide DPP max find the largest remaining key, and a ballot over the
// lane's slots (slot i holds expert i*64 + lane) picks the lowest expert id
// holding it, so equal logits order by the lower id.
__device__ __forceinline__ uint32_t order_key(float v)
{
    v = v + 0.0f; // -0 -> +0, so the two zeros tie
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k)
{
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __builtin_bit_cast(float, u);
}

template <int DPP_CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = umax(v, dpp_u32<0xB1, 0xF>(v));
    v = umax(v, dpp_u32<0x4E, 0xF>(v));
    v = umax(v, dpp_u32<0x141, 0xF>(v));
    v = umax(v, dpp_u32<0x140, 0xF>(v));
    v = umax(v, dpp_u32<0x142, 0xA>(v));
    v = umax(v, dpp_u32<0x143, 0xC>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ int wave_min_i32(int v)
{
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x142, 0xA, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// Top-K over the wave of N (key, id) pairs per lane (key 0 = no entry; ids
// distinct): lane k < K receives the k-th largest key and its id, equal keys
// ordered by ascending id.  Each lane first sorts its pairs by descending key,
// ascending id (odd-even transposition, swapping only strictly out-of-order
// neighbours: stable for pairs that arrive in ascending id order, and ties
// between pairs in any order are decided by the id test); then every round
// takes the largest head key over the wave, the lowest id among the heads
// holding it (a second reduction only when several lanes tie), and that lane
// pops its head.
template <int N>
__device__ __forceinline__ void topk_sort_lane(uint32_t (&key)[N], int (&id)[N])
{
#pragma unroll
    for (int r = 0; r < N; ++r)
#pragma unroll
        for (int i = r & 1; i + 1 < N; i += 2)
            if (key[i] < key[i + 1] || (key[i] == key[i + 1] && id[i] > id[i + 1])) {
                const uint32_t tk = key[i];
                key[i] = key[i + 1];
                key[i + 1] = tk;
                const int ti = id[i];
                id[i] = id[i + 1];
                id[i + 1] = ti;
            }
}

// Rounds k0 .. k1-1 of the selection over lane-sorted pairs (the rounds
// before k0 already popped their winners): lane k receives round k's key and
// id.  Running rounds 0..a-1 and then a..K-1 gives what 0..K-1 gives.
template <int N>
__device__ __forceinline__ void topk_rounds(uint32_t (&key)[N], int (&id)[N], int k0, int k1,
                                            uint32_t &my_key, int &my_id)
{
    const int lane = lane_id();
    for (int k = k0; k < k1; ++k) {
        const uint32_t m = wave_max_u32(key[0]);
        const uint64_t b = __ballot(key[0] == m);
        int winner = __builtin_ctzll(b);
        int wid = __builtin_amdgcn_readlane(id[0], winner);
        if (__builtin_popcountll(b) > 1) { // equal keys in several lanes: lowest id first
            wid = wave_min_i32(key[0] == m ? id[0] : 0x7FFFFFFF);
            winner = __builtin_ctzll(__ballot(key[0] == m && id[0] == wid));
        }
        if (lane == winner) {
#pragma unroll
            for (int i = 0; i + 1 < N; ++i) {
                key[i] = key[i + 1];
                id[i] = id[i + 1];
            }
            key[N - 1] = 0u;
        }
        if (lane == k) {
            my_key = m;
            my_id = wid;
        }
    }
}

template <int N>
__device__ __forceinline__ void wave_topk_keys(uint32_t (&key)[N], int (&id)[N], int K,
                                               uint32_t &my_key, int &my_id)
{
    topk_sort_lane<N>(key, id);
    my_key = 0u;
    my_id = 0;
    topk_rounds<N>(key, id, 0, K, my_key, my_id);
}

// Place of expert e in the top-k order of the wave's (key, id) pairs (key 0 =
// no entry; keys of real entries are nonzero): how many pairs have a larger
// key, or an equal key and a lower id.  The selection takes e iff that is
// below K, and e is then its rank-th choice.  e must be one of the pairs
// (the entry of id e, wherever the pairs were moved within their lane); the
// result is wave-uniform.
template <int N>
__device__ __forceinline__ int topk_rank(const uint32_t (&key)[N], const int (&id)[N], int e)
{
    uint32_t ke = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) ke = id[i] == e ? key[i] : ke;
    ke = wave_max_u32(ke); // the one lane holding e supplies its key
    int r = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
        r += __builtin_popcountll(__ballot(key[i] > ke || (key[i] == ke && id[i] < e)));
    return r;
}

// The (key, id) pairs of E <= 64*NPL logits held by the wave (v[i] is the
// logit of expert i*64 + lane; key 0 where that is >= E).
template <int NPL>
__device__ __forceinline__ void topk_pairs(const float (&v)[NPL], int E, uint32_t (&key)[NPL],
                                           int (&id)[NPL])
{
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        id[i] = i * kWave + lane_id();
        key[i] = id[i] < E ? order_key(v[i]) : 0u;
    }
}

// Top-K of E <= 64*NPL logits held by the wave: v[i] is the logit of expert
// i*64 + lane (ignored where that is >= E).  Lane k < K receives the k-th
// selected expert id and its logit; returns the largest logit (wave-uniform).
template <int NPL>
__device__ __forceinline__ float wave_topk_vals(const float (&v)[NPL], int E, int K, int &my_id,
                                                float &my_l)
{
    uint32_t key[NPL];
    int id[NPL];
    topk_pairs<NPL>(v, E, key, id);
    uint32_t my_key;
    wave_topk_keys<NPL>(key, id, K, my_key, my_id);
    my_l = my_key ? key_value(my_key) : 0.0f;
    return key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
}

// Routing weight of the slot held by this lane (valid in lanes < K): softmax
// over the selected logits (renormalize) or over all E logits.
template <int NPL>
__device__ __forceinline__ float topk_weight_vals(const float (&v)[NPL], int E, int K,
                                                  int renormalize, float my_l, float lmax)
{
    const int lane = lane_id();
    const float ex = lane < K ? expf(my_l - lmax) : 0.0f;
    float z;
    if (renormalize) {
        z = wave_sum(ex);
    } else {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (i * kWave + lane < E) part += expf(v[i] - lmax);
        z = wave_sum(part);
    }
    return ex / z;
}

// ---------------------------------------------------------------- W2 + combine
// d + sum_i w[i] * a[i] over one 16-byte chunk of a W2 row (8 fp16 weights)
// and the matching 8 fp32 activations, in element order.
__device__ __forceinline__ float dot8_f32(f16x8 w, f32x4 a0, f32x4 a1, float d)
{
    d = fmaf((float)w[0], a0[0], d);
    d = fmaf((float)w[1], a0[1], d);
    d = fmaf((float)w[2], a0[2], d);
    d = fmaf((float)w[3], a0[3], d);
    d = fmaf((float)w[4], a1[0], d);
    d = fmaf((float)w[5], a1[1], d);
    d = fmaf((float)w[6], a1[2], d);
    d = fmaf((float)w[7], a1[3], d);
    return d;
}

// ---------------------------------------------------------------- W13 + SiLU, one row pair
// gate row j and up row I + j of the expert at `base` -> silu(gate) * up
// (the W13 kernel's arithmetic for one token)
template <int HC>
__device__ __forceinline__ float w13_pair(const f16 *__restrict__ x, const f16 *__restrict__ base,
                                          int I, int j)
{
    constexpr int H = 512 * HC;
    f16x8 xv[HC], wg[HC], wu[HC];
    load_x<HC>(x, xv);
    const f16x8 *grow = reinterpret_cast<const f16x8 *>(base + (size_t)j * H);
    const f16x8 *urow = reinterpret_cast<const f16x8 *>(base + (size_t)(I + j) * H);
#pragma unroll
    for (int c = 0; c < HC; ++c) {
        wg[c] = stream_load(grow + c * kWave + lane_id());
        wu[c] = stream_load(urow + c * kWave + lane_id());
    }
    const float g = row_dot<HC>(wg, xv);
    const float up = row_dot<HC>(wu, xv);
    return silu_mul(g, up);
}

} // namespace moe

#endif
