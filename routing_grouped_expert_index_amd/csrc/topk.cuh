// Top-k of one token's router logits with one wavefront (used by the routing
// kernels and by the route-direct kernels that take logits): order-preserving
// integer keys of the values, k wave-wide maxima, ties to the lower expert id.
#pragma once
#include "common.cuh"

namespace moe {

// Row permutations of DPP (lane i of a row of 16 reads lane ...)
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]: i ^ 1
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]: i ^ 2
constexpr int kDppRowMirror = 0x140;    // 15 - i
constexpr int kDppHalfMirror = 0x141;   // 7 - i within each half row

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane_f32(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Max and sum over the 64 lanes of a fully active wave, the same bits in every
// lane: symmetric exchanges inside each row of 16 (xor 1, xor 2, half-row
// mirror, row mirror), then the four row results read as scalars.
__device__ __forceinline__ float wave_max_full(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum_full(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}


// One token's logits in a wave: lane l holds ids l + 64 i, i < VPL.
template <int VPL>
struct TopkRow {
    float v[VPL];
    uint32_t avail;
};

// the row's logits, lane + 64 i for i < VPL (-0 -> +0; comparisons treat them
// equal anyway).  The loads are unconditional (a clamped index, masked after):
// a guarded load compiles to a branch that waits for every load before it.
template <int VPL>
__device__ __forceinline__ void topk_load(const float* __restrict__ row, int E, TopkRow<VPL>& r) {
    const int lane = lane_id();
    r.avail = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        const float x = row[e < E ? e : E - 1] + 0.0f;
        r.v[i] = e < E ? x : -INFINITY;
        r.avail |= (e < E ? 1u : 0u) << i;
    }
}

// Order-preserving map of a float's bits to an unsigned key: a larger float
// gives a larger key (-inf lowest, +inf highest among non-NaN values).
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key.
__device__ __forceinline__ float key_to_float(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Max over the 64 lanes of a fully active wave (unsigned): the exchanges of
// wave_max_full, on integers (no NaN canonicalisation between the steps, and
// each exchange folds into its max instruction).
__device__ __forceinline__ uint32_t readlane_u32(uint32_t x, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppRowMirror>(v));
    return max(max(readlane_u32(v, 0), readlane_u32(v, 16)), max(readlane_u32(v, 32), readlane_u32(v, 48)));
}

// The k largest logits of one token (row) with one whole wave: slot[i] is the
// pick (0..k-1) held by the lane's entry i, or -1; pick j is the j-th largest
// value, ties to the lower expert id.  Gates (computed by the callers):
// exp(l_j - m) / S, m the largest logit, S the sum over the picks of
// exp(l_i - m) (the full softmax denominator cancels in the renormalisation).
// Logits are taken as finite (with NaN the picks stay in range and distinct
// but their order is unspecified).
//
// Pick j is a wave max over order-preserving integer keys (taken and padding
// entries hold key 0, real ones at least 1), then of the entries holding that
// key the lowest id: a ballot per slot, taken in id order (id = lane + 64 i,
// slot-major).  Some entry always holds the maximum key exactly, so no NaN
// fallback is needed.
template <int VPL>
__device__ __forceinline__ void topk_core(const TopkRow<VPL>& r, int k, int (&slot)[VPL], float& m, float& S) {
    const int lane = lane_id();
    uint32_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        key[i] = ((r.avail >> i) & 1u) ? max(order_key(r.v[i]), 1u) : 0u;
        slot[i] = -1;
    }
    uint32_t top = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t lm = key[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i) lm = max(lm, key[i]);
        const uint32_t M = wave_max_u32(lm);
        if (j == 0) top = M;
        int win = 0;
#pragma unroll
        for (int i = VPL - 1; i >= 0; --i) {   // the lowest slot holding M wins
            const uint64_t b = __ballot(key[i] == M);
            if (b != 0) win = __builtin_ctzll(b) + kWave * i;
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (win == lane + kWave * i) {
                key[i] = 0;
                slot[i] = j;
            }
    }
    m = key_to_float(top);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (slot[i] >= 0) part += expf(r.v[i] - m);
    S = wave_sum_full(part);
}

// topk_core, then the lane that owns a picked logit writes ids[j] and w[j]
// itself (and the LDS copies when given), so no value travels back through
// memory.
template <int VPL>
__device__ __forceinline__ void topk_pick(TopkRow<VPL>& r, int k, int32_t* __restrict__ ids,
                                          float* __restrict__ w, int32_t* __restrict__ ids_lds,
                                          int32_t* __restrict__ cnt_lds) {
    const int lane = lane_id();
    int slot[VPL];
    float m, S;
    topk_core<VPL>(r, k, slot, m, S);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if (slot[i] >= 0) {
            const int e = lane + kWave * i, j = slot[i];
            ids[j] = e;
            w[j] = expf(r.v[i] - m) / S;
            if (ids_lds) ids_lds[j] = e;
            if (cnt_lds) atomicAdd(&cnt_lds[e], 1);
        }
    }
}

// The expert id and gate of pick j (the same bits topk_pick writes), returned
// in every lane of the wave.
template <int VPL>
__device__ __forceinline__ void topk_slot(const TopkRow<VPL>& r, int k, int j, int& id, float& gate) {
    const int lane = lane_id();
    int slot[VPL];
    float m, S;
    topk_core<VPL>(r, k, slot, m, S);
    int my_id = -1;
    float my_w = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if (slot[i] == j) {
            my_id = lane + kWave * i;
            my_w = expf(r.v[i] - m) / S;
        }
    }
    const int src = (int)__builtin_ctzll(__ballot(my_id >= 0));
    id = __builtin_amdgcn_readlane(my_id, src);
    gate = readlane_f32(my_w, src);
}

// topk_slot on a row of E fp32 logits (E <= 512), registers sized to E
__device__ __forceinline__ void topk_slot_row(const float* row, int E, int k, int j, int& id, float& gate) {
    if (E <= 64) {
        TopkRow<1> r;
        topk_load<1>(row, E, r);
        topk_slot<1>(r, k, j, id, gate);
    } else if (E <= 128) {
        TopkRow<2> r;
        topk_load<2>(row, E, r);
        topk_slot<2>(r, k, j, id, gate);
    } else if (E <= 256) {
        TopkRow<4> r;
        topk_load<4>(row, E, r);
        topk_slot<4>(r, k, j, id, gate);
    } else {
        TopkRow<8> r;
        topk_load<8>(row, E, r);
        topk_slot<8>(r, k, j, id, gate);
    }
}

}  // namespace moe
