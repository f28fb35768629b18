// Route-direct MoE forward for small decode batches on gfx950.
//
// "perf: add small-batch route MMA for MoE", Summary and Motivation: when
// B * top_k is far below the expert count, each route (token t, slot j) reads
// its expert's weights directly; the expert sort, the gather, the prefix and
// the task map are skipped and the data stays in route order; Gate/Up, then a
// step that finishes the Gate/Up reduction with SwiGLU and the Down-input
// quantisation, then Down, then a contiguous top-k reduction.
//
// On MI355X this path is bound by HBM: each route streams 3*H*I weight
// elements and does 2 flops per element, so the matrix cores have nothing to
// gain; the kernels keep as many contiguous weight loads in flight as they can.
// Weights are read in the packed layout (layout.cuh) as whole 2 KB blocks of
// 32 rows x 64 K bytes, one contiguous kilobyte per wave-wide load; lane
// l = 32*hh + j accumulates row j over K bytes [32hh, 32hh+32) of every slice
// and the two halves are added at the end.
//  * Gate/Up: a workgroup owns (route, 32 h columns): the gate block and the up
//    block of those columns; its NW waves split K, their partial sums meet in
//    LDS in wave order, then SwiGLU and the h store (bf16, or fp32 ahead of the
//    FP8 requantisation).
//  * Down + combine: a workgroup owns (token, 32 output columns, item), an item
//    being one route slot and one of KP parts of its K range, so that a batch
//    of one token still spreads over about a thousand workgroups.  Each writes
//    its gate-weighted partial sums to the workspace and takes a ticket from a
//    device-scope counter; the last of the output block's workgroups to arrive
//    adds all partials in item order and writes the bf16 output.  The order of
//    the sum never depends on arrival order, so two runs give the same bits.
//  * FP8 per-tensor: the activation scales are whole-tensor maxima.  Each
//    Gate/Up workgroup takes the maximum of x over [T, H] itself (a few
//    kilobytes at decode sizes) and records the maximum of its 32 h values; the
//    Down workgroups reduce those few hundred maxima.  So the path is two
//    launches with nothing in between.
//  * FP8 blockwise: x and h are quantised per token (route row) and 128
//    channels in the workgroups that use them; each 64-byte K slice lies in one
//    scale block.
//  * MX ("[mxfp8 moe training] add per group blocked scale kernels", Summary:
//    mxfp8 scales): x and h are quantised per 32 channels with an E8M0 byte in
//    the workgroups that use them.  The weights are packed in the scaled MFMA's
//    chunk order, so a lane's two 16-byte pieces of a slice belong to its two
//    MX blocks (K [16hh, 16hh+16) of block 2s, [32+16hh, 48+16hh) of block
//    2s+1); each piece's dot product takes its block's weight and activation
//    scales.  The weight scale bytes come from the dwords moe_pack_mx_scales
//    lays out for the grouped GEMM: dword (32-row block, slice group g, lane
//    32hh' + j) holds row j's scales of blocks 8g + 2u + hh' in byte u.
#include <hip/hip_ext.h>

#include "common.cuh"
#include "launch.h"
#include "layout.cuh"
#include "topk.cuh"

#include <algorithm>
#include <atomic>
#include <initializer_list>

namespace moe {

enum RdQuant { RD_BF16 = 0, RD_TENSOR = 1, RD_BLOCK = 2, RD_MX = 3 };

struct RdArgs {
    const uint8_t* act;      // x bf16 [T,H]
    const int32_t* ids;      // [T*k]
    const float* tw;         // [T*k]
    const uint8_t* wgu;      // packed Gate/Up
    const uint8_t* wd;       // packed Down
    const float* s_gu;       // weight scales (MX: the packed E8M0 dwords)
    const float* s_d;
    const uint8_t* h;        // Down input: bf16 [R][I] | fp32 [R][I] (FP8, quantised by the Down kernel)
    void* hout;              // Gate/Up output: bf16 [R][I] | fp32 [R][I]
    float* hmax;             // per-tensor: max |h| per Gate/Up workgroup [R][I/32]
    float* part;             // Down partial sums [T*H/32][items][32]
    int32_t* cnt;            // Down arrival counters [T*H/32], zeroed by the Gate/Up kernel
    uint16_t* out;           // [T][H]
    int T, H, I, E, k;
    int kp;                  // per-block Down: K parts per route slot
    int rs;                  // Gate/Up row split (workgroups per 32-row block pair)
    int e0, nloc;            // expert slice held by the weights (expert e at index e - e0)
    // routing folded into the Gate/Up kernel: with logits set, each Gate/Up
    // workgroup takes its route's expert from the top-k of its token's logits,
    // and the first workgroup of a route writes the route's id and gate to
    // ids_w / tw_w (which the Down kernel then reads as ids / tw)
    const float* logits;     // fp32 [T][E] or null
    int32_t* ids_w;
    float* tw_w;
    int acc;                 // out += the layer sum (else out = it)
    // FP8 inspection copies in the workspace (null for bf16): each token's x
    // codes [T][H] and block scales [T][H/128] (MX: E8M0 bytes [T][H/32] in
    // the MX GEMM's byte order); per-tensor x and h scales (scal_out[0],
    // scal_out[1]); blockwise h scales [R][I/128] (MX: bytes [R][I/32]) in
    // route order
    uint8_t* xq_out;
    float* sx_out;
    float* scal_out;
    float* sh_out;
};

// 8 values from 16 bytes of bf16
__device__ __forceinline__ void bf16x8_to_f32(const u32x4& w, float v[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// 16 values from 16 bytes of e4m3
__device__ __forceinline__ void e4m3x16_to_f32(const u32x4& w, float v[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[4 * i] = e4m3_to_f32<0>(w[i]);
        v[4 * i + 1] = e4m3_to_f32<1>(w[i]);
        v[4 * i + 2] = e4m3_to_f32<2>(w[i]);
        v[4 * i + 3] = e4m3_to_f32<3>(w[i]);
    }
}


// workgroup-wide max |v| over n values of T (bf16 bits or fp32), n % 8 == 0
template <typename T, int NW>
__device__ __forceinline__ float block_amax(const T* p, long n, float* sred) {
    float m = 0.0f;
    for (long i = (long)threadIdx.x * 8; i < n; i += 64L * NW * 8) {
        float v[8];
        if constexpr (sizeof(T) == 2) {
            bf16x8_to_f32(*reinterpret_cast<const u32x4*>(p + i), v);
        } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(p + i);
            const f32x4 b = *reinterpret_cast<const f32x4*>(p + i + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) { v[q] = a[q]; v[4 + q] = b[q]; }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
    }
    m = wave_max(m);
    if (lane_id() == 0) sred[threadIdx.x >> 6] = m;
    __syncthreads();
    m = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, sred[w]);
    return m;
}

// workgroup-wide max of one value per thread (sred: NW floats of LDS)
template <int NW>
__device__ __forceinline__ float block_max(float m, float* sred) {
    m = wave_max(m);
    if (lane_id() == 0) sred[threadIdx.x >> 6] = m;
    __syncthreads();
    m = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, sred[w]);
    return m;
}

// wave-uniform 32-bit load through the constant address space (a scalar load:
// it counts on lgkmcnt, so waiting for it never waits for vector loads)
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int i) {
    return ((const __attribute__((address_space(4))) int32_t*)(p))[__builtin_amdgcn_readfirstlane(i)];
}
__device__ __forceinline__ float ld_uniform_f(const float* p, int i) {
    return ((const __attribute__((address_space(4))) float*)(p))[__builtin_amdgcn_readfirstlane(i)];
}

// Activation rows are staged in LDS once per workgroup (every lane of a
// 32-row weight block needs the same activation values): bf16 values, or e4m3
// codes (quantised here for per-tensor FP8, copied for blockwise).
constexpr int kRdActBytes = 8192;          // one activation row: H * elem <= 8192

// The lane's 32 activation bytes of slice s from an LDS row, as fp32 values
// (bf16: 16 values; e4m3: 32 values).
template <bool FP8>
__device__ __forceinline__ void lds_act_slice(const uint8_t* row, int s, int hh, float v[32]) {
    const uint8_t* p = row + s * 64 + hh * 32;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(p);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(p + 16);
    if constexpr (!FP8) {
        bf16x8_to_f32(w0, v);
        bf16x8_to_f32(w1, v + 8);
    } else {
        e4m3x16_to_f32(w0, v);
        e4m3x16_to_f32(w1, v + 16);
    }
}

// copy n bytes (n % 16 == 0) of a global row into LDS, whole workgroup
template <int NW>
__device__ __forceinline__ void stage_row(uint8_t* dst, const uint8_t* src, int n) {
    for (int i = threadIdx.x * 16; i < n; i += 64 * NW * 16)
        *reinterpret_cast<u32x4*>(dst + i) = *reinterpret_cast<const u32x4*>(src + i);
}

// quantise n values (n % 8 == 0) of a bf16 (or fp32) row with scale s into e4m3
// codes in LDS, whole workgroup
template <typename T, int NW>
__device__ __forceinline__ void quant_row(uint8_t* dst, const T* src, int n, float s) {
    for (int i = threadIdx.x * 8; i < n; i += 64 * NW * 8) {
        float v[8];
        if constexpr (sizeof(T) == 2) {
            bf16x8_to_f32(*reinterpret_cast<const u32x4*>(src + i), v);
        } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(src + i);
            const f32x4 b = *reinterpret_cast<const f32x4*>(src + i + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) { v[q] = a[q]; v[4 + q] = b[q]; }
        }
        uint2 c;
        c.x = f32x4_to_e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
        c.y = f32x4_to_e4m3x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
        *reinterpret_cast<uint2*>(dst + i) = c;
    }
}

// quantise n values (n % 128 == 0) of a bf16 (or fp32) row per 128-value group
// into e4m3 codes in LDS, s = amax/448 of the group into sdst[group]; whole
// workgroup, 16 lanes per group (8 values each)
template <typename T, int NW>
__device__ __forceinline__ void quant_row_block128(uint8_t* dst, float* sdst, const T* src, int n) {
    for (int i = threadIdx.x * 8; i < n; i += 64 * NW * 8) {
        float v[8];
        if constexpr (sizeof(T) == 2) {
            bf16x8_to_f32(*reinterpret_cast<const u32x4*>(src + i), v);
        } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(src + i);
            const f32x4 b = *reinterpret_cast<const f32x4*>(src + i + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) { v[q] = a[q]; v[4 + q] = b[q]; }
        }
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));   // the group's 16 lanes
        const float sc = scale_from_amax(m);
        uint2 c;
        c.x = f32x4_to_e4m3x4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
        c.y = f32x4_to_e4m3x4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
        *reinterpret_cast<uint2*>(dst + i) = c;
        if ((threadIdx.x & 15) == 0) sdst[i / 128] = sc;
    }
}

// quantise n values (n % 32 == 0) of a bf16 (or fp32) row per 32-value MX
// group: the group's E8M0 byte (mx_byte of its amax) into sdst[group] and
// codes e4m3(v * 2^(127 - b)) into dst in LDS; whole workgroup, 4 lanes per
// group (8 values each)
template <typename T, int NW>
__device__ __forceinline__ void quant_row_mx32(uint8_t* dst, uint8_t* sdst, const T* src, int n) {
    for (int i = threadIdx.x * 8; i < n; i += 64 * NW * 8) {
        float v[8];
        if constexpr (sizeof(T) == 2) {
            bf16x8_to_f32(*reinterpret_cast<const u32x4*>(src + i), v);
        } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(src + i);
            const f32x4 b = *reinterpret_cast<const f32x4*>(src + i + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) { v[q] = a[q]; v[4 + q] = b[q]; }
        }
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
        m = fmaxf(m, __shfl_xor(m, 1));   // the group's 4 lanes
        m = fmaxf(m, __shfl_xor(m, 2));
        const uint32_t b = mx_byte(m);
        const float inv = mx_inv(b);
        uint2 c;
        c.x = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        c.y = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
        *reinterpret_cast<uint2*>(dst + i) = c;
        if ((threadIdx.x & 3) == 0) sdst[i / 32] = (uint8_t)b;
    }
}

// MX: the dot of one 16-byte piece of e4m3 weights with 16 e4m3 activations
__device__ __forceinline__ float dot16_e4m3(const u32x4& w, const u32x4& x) {
    float wf[16], xf[16];
    e4m3x16_to_f32(w, wf);
    e4m3x16_to_f32(x, xf);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = fmaf(wf[i], xf[i], acc);
    return acc;
}

// MX: the lane's two weight pieces of a slice (blocks 2s and 2s+1) times the
// activation codes of the same K positions, each scaled by its blocks'
// weight scale (byte `sh` of dword ws[q]) and activation scale byte sa[q]
__device__ __forceinline__ float dot_slice_mx(const u32x4 w[2], const uint8_t* act, int s, int hh,
                                              const uint32_t ws[2], const uint8_t* sa, int sh) {
    const uint8_t* p = act + s * 64 + hh * 16;
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(p + 32 * q);
        const float sc = e8m0_to_f32((ws[q] >> sh) & 255u) * e8m0_to_f32(sa[2 * s + q]);
        acc = fmaf(dot16_e4m3(w[q], x), sc, acc);
    }
    return acc;
}

// dot of the lane's two weight halves of one slice with its activation values
template <bool FP8>
__device__ __forceinline__ float dot_slice(const u32x4 w[2], const float v[32]) {
    float acc = 0.0f;
    if constexpr (!FP8) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float wf[8];
            bf16x8_to_f32(w[q], wf);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = fmaf(wf[i], v[8 * q + i], acc);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float wf[16];
            e4m3x16_to_f32(w[q], wf);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc = fmaf(wf[i], v[16 * q + i], acc);
        }
    }
    return acc;
}

// bf16: the lane's 16 weights times the 16 activations of the same K positions,
// two products per instruction (v_dot2c_f32_bf16) straight from the packed words
__device__ __forceinline__ float dot_slice_bf16(const u32x4 w[2], const u32x4 x[2], float acc) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        // the words go through scalars: a bit cast taken straight from a vector
        // element was compiled as a cast of element 0 for every i
        const uint32_t wv[4] = {w[q][0], w[q][1], w[q][2], w[q][3]};
        const uint32_t xv[4] = {x[q][0], x[q][1], x[q][2], x[q][3]};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv[i]),
                                                  __builtin_bit_cast(bf16x2_t, xv[i]), acc, false);
    }
    return acc;
}

// the lane's 32 activation bytes of slice s from an LDS row, as packed words
__device__ __forceinline__ void lds_act_raw(const uint8_t* row, int s, int hh, u32x4 x[2]) {
    const uint8_t* p = row + s * 64 + hh * 32;
    x[0] = *reinterpret_cast<const u32x4*>(p);
    x[1] = *reinterpret_cast<const u32x4*>(p + 16);
}

// ---------------------------------------------------------------- Gate/Up --
template <int Q, int NW, int U>
__global__ void __launch_bounds__(64 * NW)
rd_gate_up_kernel(const RdArgs a) {
    constexpr bool FP8 = Q != RD_BF16;
    __shared__ __attribute__((aligned(16))) uint8_t xrow[kRdActBytes];
    __shared__ float sxs[Q == RD_BLOCK ? kRdActBytes / 128 : 1];   // blockwise: the row's x scales
    __shared__ uint8_t sxb[Q == RD_MX ? kRdActBytes / 32 : 4];     // MX: the row's x scale bytes
    __shared__ float red[NW][2][32];
    __shared__ float sred[NW];
    __shared__ int s_eg;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int j = lane & 31, hh = lane >> 5;
    const int r = blockIdx.x, G = blockIdx.y;   // route; 64-row group (gate block 2G, up block 2G+1)
    // Row split RS = gridDim.z (1, 2, 4, 8): this workgroup owns rows
    // [RW rs, RW rs + RW) of both blocks, RW = 32 / RS.  Lane j reads row
    // RW rs + j % RW of slice RS S + j / RW of each super-slice S (RS
    // consecutive slices), so one wave-wide load still fetches RS x RW rows x
    // 32 distinct bytes, and the RS lanes of a row are added at the end.
    const int lrs = __builtin_ctz(gridDim.z), RS = 1 << lrs, RW = 32 >> lrs, rs = blockIdx.z;
    const int ls = j >> (5 - lrs), jr = rs * RW + (j & (RW - 1));
    const int t = r / a.k;
    // With logits, wave 0 takes the route's expert from the token's top-k
    // while the workgroup stages x, and the weight stream starts after the
    // barrier that publishes it; otherwise the expert comes from the routes and
    // the weight stream starts first.
    const bool from_logits = a.logits != nullptr;
    // The activation values go out before anything else (vector loads complete
    // in issue order, so waiting for them later never waits for the weight
    // stream behind them): this thread's 16-byte chunks c = threadIdx.x + p NT
    // of the token's bf16 row and, for the per-tensor scale, of all of x
    // (clamped indices, masked when used).  Workgroups of fewer than 4 waves
    // would need too many registers for the row and read it after the weights.
    constexpr int NT = 64 * NW;
    constexpr bool PRE = NW >= 4;
    constexpr int RP = PRE ? (kRdActBytes * 2 / 16 + NT - 1) / NT : 1;   // bf16 row: H <= 8192 values
    constexpr int AP = Q == RD_TENSOR && PRE ? 16384 / 8 / NT : 1;      // all of x while T H <= 16384
    const uint16_t* x = reinterpret_cast<const uint16_t*>(a.act);
    const int rch = a.H / 8;                     // 16-byte chunks in the row
    const long ach = (long)a.T * a.H / 8;        // ... in all of x
    u32x4 xr[RP], xa[AP];
    if constexpr (PRE) {
        const u32x4* xt = reinterpret_cast<const u32x4*>(x + (long)t * a.H);
#pragma unroll
        for (int p = 0; p < RP; ++p) xr[p] = xt[min((int)threadIdx.x + p * NT, rch - 1)];
        if constexpr (Q == RD_TENSOR) {
#pragma unroll
            for (int p = 0; p < AP; ++p)
                xa[p] = reinterpret_cast<const u32x4*>(x)[min((long)threadIdx.x + p * NT, ach - 1)];
        }
    }
    if (from_logits && wave == 0) {
        int eg0;
        float gate;
        topk_slot_row(a.logits + (size_t)t * a.E, a.E, a.k, r - t * a.k, eg0, gate);
        if (lane == 0) {
            s_eg = eg0;
            if (G == 0 && rs == 0) {   // one writer per route
                a.ids_w[r] = eg0;
                a.tw_w[r] = gate;
            }
        }
    }
    constexpr int elem = FP8 ? 1 : 2;
    // wave w takes the U-super-slice chunks w, w + NW, w + 2 NW, ...: at each
    // step the waves of the workgroup read one contiguous window
    const int Kb = a.H * elem, NSL = Kb / kSliceBytes, NSS = NSL >> lrs, per = NSS / NW, s0 = wave * U;
    constexpr int SB = NW * U;   // super-slice step between a wave's batches
    const long gstride = 32L * Kb;
    if (r == 0 && G == 0 && rs == 0)   // the Down kernel that follows counts arrivals from zero
        for (int i = threadIdx.x; i < a.T * (a.H / 32); i += 64 * NW) a.cnt[i] = 0;
    int e = 0;
    const uint8_t *wg = nullptr, *wu = nullptr;
    // MX: this lane's row in the scale dwords of the gate and up blocks
    // (dwords [slice group][64 lanes]; piece q of a slice reads lane jr + 32q)
    const uint32_t *swg = nullptr, *swu = nullptr;
    const int NG = a.H / 256;
    // the expert's index in this call's slice and its weight rows; false for
    // another slice's expert (no h, a zero share of the h amax)
    float sgu = 1.0f;
    auto resolve = [&](int eg) __attribute__((always_inline)) {
        e = eg - a.e0;
        if ((unsigned)e >= (unsigned)a.nloc) {
            if constexpr (Q == RD_TENSOR) {
                if (threadIdx.x == 0) a.hmax[((long)r * (a.I / 32) + G) * RS + rs] = 0.0f;
            }
            return false;
        }
        wg = a.wgu + (long)e * 2 * a.I * Kb + (long)(2 * G) * gstride + (32 * hh + jr) * 16 + ls * 2048;
        wu = wg + gstride;
        // (the per-tensor weight scale is requested now: read only at the end, a
        // load there would add a whole memory latency after the products)
        if constexpr (Q == RD_TENSOR) sgu = ld_uniform_f(a.s_gu, e);
        if constexpr (Q == RD_MX) {
            swg = reinterpret_cast<const uint32_t*>(a.s_gu) + ((long)e * (2 * a.I / 32) + 2 * G) * NG * 64 + jr;
            swu = swg + NG * 64;
        }
        return true;
    };
    // FP8: one workgroup of each token (h block 0, split 0, and the token's
    // first slot whose expert lies in this call's slice; with the routing
    // folded in, slot 0, before it learns its expert) also leaves the token's
    // codes and scales in the workspace
    const bool mine = from_logits || resolve(ld_uniform(a.ids, r));
    if (!mine) return;
    bool writer = FP8 && a.xq_out != nullptr && G == 0 && rs == 0;
    if (writer && !from_logits)
        for (int jj = 0; jj < r - t * a.k; ++jj)
            writer = writer && (unsigned)(ld_uniform(a.ids, t * a.k + jj) - a.e0) >= (unsigned)a.nloc;
    else if (writer)
        writer = r == t * a.k;

    // two load buffers: batch b+1 is requested before batch b is computed
    // (MX: with each slice's scale dwords of its two pieces)
    u32x4 vg[2][U][2], vu[2][U][2];
    uint32_t mg[Q == RD_MX ? 2 : 1][U][2], mu[Q == RD_MX ? 2 : 1][U][2];
    auto load_batch = [&](auto Bc, int S) __attribute__((always_inline)) {
        constexpr int B = decltype(Bc)::value;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const long off = ((long)(S + u) << lrs) * 2048 + q * 1024;
                vg[B][u][q] = *reinterpret_cast<const u32x4*>(wg + off);
                vu[B][u][q] = *reinterpret_cast<const u32x4*>(wu + off);
                if constexpr (Q == RD_MX) {
                    const int g = ((((S + u) << lrs) + ls) >> 2) * 64 + 32 * q;
                    mg[B][u][q] = swg[g];
                    mu[B][u][q] = swu[g];
                }
            }
        __builtin_amdgcn_sched_barrier(0);   // the whole batch stays in flight
    };
    std::integral_constant<int, 0> B0;
    std::integral_constant<int, 1> B1;
    float xs = 1.0f;
    // the activation row staged in LDS (x quantised for FP8): written out twice
    // below, once per mode, so that no branch joins between the weight loads
    // and the first use of the preloaded activations (a join would make the
    // compiler wait for every load issued on either side)
    auto stage_x = [&]() __attribute__((always_inline)) {
    if constexpr (!PRE) {
        if constexpr (Q == RD_TENSOR) {
            xs = scale_from_amax(block_amax<uint16_t, NW>(x, (long)a.T * a.H, sred));
            quant_row<uint16_t, NW>(xrow, x + (long)t * a.H, a.H, xs);
        } else if constexpr (Q == RD_BLOCK) {   // the token's codes and per-128 scales, here
            quant_row_block128<uint16_t, NW>(xrow, sxs, x + (long)t * a.H, a.H);
        } else if constexpr (Q == RD_MX) {      // ... per-32 E8M0 bytes
            quant_row_mx32<uint16_t, NW>(xrow, sxb, x + (long)t * a.H, a.H);
        } else {
            stage_row<NW>(xrow, a.act + (long)t * Kb, Kb);
        }
    } else if constexpr (Q == RD_TENSOR) {
        // the x amax from the preloaded chunks (and any beyond them), then the
        // row's codes from its preloaded chunks
        float m = 0.0f;
#pragma unroll
        for (int p = 0; p < AP; ++p) {
            float v[8];
            bf16x8_to_f32(xa[p], v);
            float mp = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) mp = fmaxf(mp, fabsf(v[q]));
            m = (long)threadIdx.x + p * NT < ach ? fmaxf(m, mp) : m;
        }
        for (long c = (long)threadIdx.x + AP * NT; c < ach; c += NT) {
            float v[8];
            bf16x8_to_f32(reinterpret_cast<const u32x4*>(x)[c], v);
#pragma unroll
            for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
        }
        xs = scale_from_amax(block_max<NW>(m, sred));
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int c = threadIdx.x + p * NT;
            float v[8];
            bf16x8_to_f32(xr[p], v);
            uint2 q8;
            q8.x = f32x4_to_e4m3x4(v[0] / xs, v[1] / xs, v[2] / xs, v[3] / xs);
            q8.y = f32x4_to_e4m3x4(v[4] / xs, v[5] / xs, v[6] / xs, v[7] / xs);
            if (c < rch) *reinterpret_cast<uint2*>(xrow + 8 * c) = q8;
        }
    } else if constexpr (Q == RD_BLOCK) {
        // per 128 values (16 lanes of 8): amax over the group, s = amax/448, codes
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int c = threadIdx.x + p * NT;
            float v[8];
            bf16x8_to_f32(xr[p], v);
            float m = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));   // the group's 16 lanes
            const float sc = scale_from_amax(m);
            uint2 q8;
            q8.x = f32x4_to_e4m3x4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
            q8.y = f32x4_to_e4m3x4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
            if (c < rch) {
                *reinterpret_cast<uint2*>(xrow + 8 * c) = q8;
                if ((threadIdx.x & 15) == 0) sxs[c / 16] = sc;
            }
        }
    } else if constexpr (Q == RD_MX) {
        // per 32 values (4 lanes of 8): the E8M0 byte of the group's amax, codes
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int c = threadIdx.x + p * NT;
            float v[8];
            bf16x8_to_f32(xr[p], v);
            float m = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
            m = fmaxf(m, __shfl_xor(m, 1));   // the group's 4 lanes
            m = fmaxf(m, __shfl_xor(m, 2));
            const uint32_t bx = mx_byte(m);
            const float inv = mx_inv(bx);
            uint2 q8;
            q8.x = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
            q8.y = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
            if (c < rch) {
                *reinterpret_cast<uint2*>(xrow + 8 * c) = q8;
                if ((threadIdx.x & 3) == 0) sxb[c / 4] = (uint8_t)bx;
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int c = threadIdx.x + p * NT;
            if (c < rch) reinterpret_cast<u32x4*>(xrow)[c] = xr[p];
        }
    }
    __syncthreads();
    };
    if (!from_logits) {
        load_batch(B0, s0);   // the weight stream goes out right behind the activations
        stage_x();
    } else {
        stage_x();
    }
    if (writer) {
        uint8_t* xq = a.xq_out + (long)t * a.H;
        for (int i = threadIdx.x * 16; i < a.H; i += 64 * NW * 16)
            *reinterpret_cast<u32x4*>(xq + i) = *reinterpret_cast<const u32x4*>(xrow + i);
        if constexpr (Q == RD_BLOCK) {
            for (int i = threadIdx.x; i < a.H / 128; i += 64 * NW) a.sx_out[(long)t * (a.H / 128) + i] = sxs[i];
        } else if constexpr (Q == RD_MX) {
            uint8_t* so = reinterpret_cast<uint8_t*>(a.sx_out) + (long)t * (a.H / 32);
            for (int i = threadIdx.x; i < a.H / 32; i += 64 * NW) so[mx_scale_pos(i)] = sxb[i];
        } else {
            if (t == 0 && threadIdx.x == 0) a.scal_out[0] = xs;
        }
    }
    if (from_logits) {   // the expert wave 0 published; then the weight stream
        if (!resolve(__builtin_amdgcn_readfirstlane(s_eg))) return;
        load_batch(B0, s0);
    }
    int cg = 0, cu = 0;           // blockwise: scale columns of the gate and up blocks
    if constexpr (Q == RD_BLOCK) {
        cg = (32 * G) / 128;
        cu = (a.I + 32 * G) / 128;
    }

    float accg = 0.0f, accu = 0.0f;
    auto compute = [&](auto Bc, int S) __attribute__((always_inline)) {
        constexpr int B = decltype(Bc)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sl = ((S + u) << lrs) + ls;   // this lane's slice
            float dg = 0.0f, du = 0.0f;
            if constexpr (Q == RD_MX) {   // the scales are inside the products
                const int sh = 8 * (sl & 3);
                dg = dot_slice_mx(vg[B][u], xrow, sl, hh, mg[B][u], sxb, sh);
                du = dot_slice_mx(vu[B][u], xrow, sl, hh, mu[B][u], sxb, sh);
            } else if constexpr (!FP8) {
                u32x4 xw[2];
                lds_act_raw(xrow, sl, hh, xw);
                dg = dot_slice_bf16(vg[B][u], xw, 0.0f);
                du = dot_slice_bf16(vu[B][u], xw, 0.0f);
            } else {
                float v[32];
                lds_act_slice<FP8>(xrow, sl, hh, v);
                dg = dot_slice<FP8>(vg[B][u], v);
                du = dot_slice<FP8>(vu[B][u], v);
            }
            if constexpr (Q == RD_BLOCK) {
                const int kb = sl / 2;   // 128-deep scale block
                const float sa = sxs[kb];
                const float* swr = a.s_gu + ((long)e * (a.H / 128) + kb) * (2 * a.I / 128);
                accg = fmaf(dg, sa * swr[cg], accg);
                accu = fmaf(du, sa * swr[cu], accu);
            } else {
                accg += dg;
                accu += du;
            }
        }
    };
    // nb batches of U super-slices: pairs while more than two remain (batch b+2
    // goes into the freed buffer), then the last one or two
    const int nb = per / U;
    int S = s0, b = 0;
    for (; b + 2 < nb; b += 2, S += 2 * SB) {
        load_batch(B1, S + SB);
        compute(B0, S);
        load_batch(B0, S + 2 * SB);
        compute(B1, S + SB);
    }
    if (nb - b == 2) {
        load_batch(B1, S + SB);
        compute(B0, S);
        compute(B1, S + SB);
    } else {
        compute(B0, S);
    }
    // the two K halves of a lane pair, then the RS slices of a row
    accg += __shfl_xor(accg, 32);
    accu += __shfl_xor(accu, 32);
    for (int off = 16; off >= RW; off >>= 1) {
        accg += __shfl_xor(accg, off);
        accu += __shfl_xor(accu, off);
    }
    if (hh == 0 && j < RW) {
        red[wave][0][j] = accg;
        red[wave][1][j] = accu;
    }
    __syncthreads();
    if (wave == 0 && hh == 0) {
        float gv = 0.0f, uv = 0.0f;
        if (j < RW) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                gv += red[w][0][j];
                uv += red[w][1][j];
            }
        }
        if constexpr (Q == RD_TENSOR) {
            const float fsc = xs * sgu;
            gv *= fsc;
            uv *= fsc;
        }
        const float hv = silu(gv) * uv;
        if constexpr (Q == RD_TENSOR) {   // this workgroup's share of the h amax
            float m = j < RW ? fabsf(hv) : 0.0f;
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            if (j == 0) a.hmax[((long)r * (a.I / 32) + G) * RS + rs] = m;
        }
        // row jr of the pair's blocks is h column 32G + 16hh' + 4a + b, jr = 8a + 4hh' + b
        const int c = 32 * G + 16 * ((jr >> 2) & 1) + 4 * (jr >> 3) + (jr & 3);
        if (j < RW) {
            if constexpr (Q == RD_BF16)
                static_cast<uint16_t*>(a.hout)[(long)r * a.I + c] = f32_to_bf16(hv);
            else
                static_cast<float*>(a.hout)[(long)r * a.I + c] = hv;
        }
    }
}

// ------------------------------------------------------------ Down+combine --
// The end of a Down piece: wave 0 publishes the piece's partial v (lanes 0..31)
// and takes the output block's arrival ticket; the last arrival sums the k*KP
// partials in a fixed order and writes the block's 32 outputs.  Partials and
// the ticket use device-scope atomic stores, loads and adds, which are
// performed at the device-coherent level without the whole-L2 write-back a
// device-scope fence costs on this multi-XCD GPU; the wave's partial stores
// have completed (vmcnt 0) before it takes its ticket.  Every thread of the
// workgroup calls this (it holds a barrier).
__device__ __forceinline__ void rd_part_publish(const RdArgs& a, int tb, int t, int g32, int it,
                                                int items, float v, int& last_s) {
    const int lane = lane_id(), wave = threadIdx.x >> 6, hh = lane >> 5;
    float* part = a.part + (long)tb * items * 32;
    if (wave == 0) {
        if (hh == 0) __hip_atomic_store(part + it * 32 + lane, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Order: partial stores, then vmcnt(0) (the stores are acknowledged by
        // the device-coherent level: agent-scope atomic stores bypass the
        // non-coherent caches), then the ticket.  The signal fences keep the
        // compiler from moving either memory operation across the wait; the
        // hardware completes the stores before the wait returns, so any
        // workgroup that draws the last ticket finds every partial in memory
        // (its loads are agent-scope atomics too, read at that same level).
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));   // vmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0)
            last_s = __hip_atomic_fetch_add(a.cnt + tb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == items - 1;
    }
    __syncthreads();
    if (!last_s) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the partial loads stay after the ticket
    if (wave == 0 && hh == 0) {
        float o = 0.0f;
        for (int i = 0; i < items; ++i)   // fixed order
            o += __hip_atomic_load(part + i * 32 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint16_t* op = a.out + (long)t * a.H + down_col_of_packed(32 * g32 + lane);
        if (a.acc) o += __uint_as_float((uint32_t)*op << 16);   // shared output: one rounding of out + sum
        *op = f32_to_bf16(o);
        if (lane == 0) __hip_atomic_store(a.cnt + tb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int Q, int NW, int KP, int U>
__global__ void __launch_bounds__(64 * NW)
rd_down_part_kernel(const RdArgs a) {
    constexpr bool FP8 = Q != RD_BF16;
    // FP8: the route's h row as e4m3 codes (quantised here), blockwise with its
    // per-128 scales, MX with its per-32 E8M0 bytes
    __shared__ __attribute__((aligned(16))) uint8_t hrow_s[FP8 ? 2048 : 16];
    __shared__ float shs[Q == RD_BLOCK ? 2048 / 128 : 1];
    __shared__ uint8_t shb[Q == RD_MX ? 2048 / 32 : 4];
    __shared__ float red[NW][32];
    __shared__ int last_s;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int hh = lane >> 5;
    const int nb = a.H / 32;
    const int tb = blockIdx.x, t = tb / nb, g32 = tb - t * nb;
    const int items = a.k * KP, it = blockIdx.y;
    const int jj = it / KP, kp = it - jj * KP;
    const int r = t * a.k + jj, e = a.ids[r] - a.e0;   // index in this call's expert slice
    if ((unsigned)e >= (unsigned)a.nloc) {   // another slice's expert: a zero partial, no weights
        rd_part_publish(a, tb, t, g32, it, items, 0.0f, last_s);
        return;
    }
    constexpr int elem = FP8 ? 1 : 2;
    const int Kb = a.I * elem, NSL = Kb / kSliceBytes, spw = NSL / KP / NW;
    const int s0 = kp * (NSL / KP) + wave * spw;
    const int n0 = down_col_of_packed(32 * g32);   // all 32 rows lie in one 128-column block
    const uint8_t* wb = a.wd + (long)e * a.H * Kb + (long)g32 * 32 * Kb + lane * 16;
    // MX: row j's scale dwords of this 32-row block (piece q of a slice: lane j + 32q)
    const uint32_t* swd = Q == RD_MX ? reinterpret_cast<const uint32_t*>(a.s_d) +
                                           ((long)e * nb + g32) * (a.I / 256) * 64 + (lane & 31)
                                     : nullptr;

    // the route's gate (and per-tensor weight scale), used only at the end:
    // requested before the weight stream so their latency is hidden under it
    const float gate = ld_uniform_f(a.tw, r);
    const float sdw = Q == RD_TENSOR ? ld_uniform_f(a.s_d, e) : 1.0f;
    u32x4 vw[U][2];
    uint32_t mw[Q == RD_MX ? U : 1][2];
    u32x4 va[U][2];   // bf16: activation slices of the batch (the row is not staged in LDS)
    const uint8_t* hg = a.h + (long)r * Kb + hh * 32;
    auto load_batch = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                vw[u][q] = *reinterpret_cast<const u32x4*>(wb + (long)(s + u) * 2048 + q * 1024);
                if constexpr (Q == RD_MX) mw[u][q] = swd[((s + u) >> 2) * 64 + 32 * q];
            }
        if constexpr (!FP8) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    va[u][q] = *reinterpret_cast<const u32x4*>(hg + (s + u) * 64 + q * 16);
        }
    };
    load_batch(s0);   // the weight stream starts before the h row is prepared
    __builtin_amdgcn_sched_barrier(0);   // keep the whole batch in flight (no sinking below the activations)

    float hs = 1.0f;
    const uint8_t* hrow = hrow_s;
    if constexpr (Q == RD_TENSOR) {
        // whole-tensor h amax from the Gate/Up workgroups' maxima, then this
        // route's h row quantised into LDS
        float m = 0.0f;
        const int nmax = a.T * a.k * (a.I / 32) * a.rs;
        for (int i = threadIdx.x; i < nmax; i += 64 * NW) m = fmaxf(m, a.hmax[i]);
        m = wave_max(m);
        if (lane == 0) red[wave][0] = m;
        __syncthreads();
        m = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, red[w][0]);
        hs = scale_from_amax(m);
        if (tb == 0 && threadIdx.x == 0) a.scal_out[1] = hs;   // (inspection copy; every writer stores the same value)
        quant_row<float, NW>(hrow_s, reinterpret_cast<const float*>(a.h) + (long)r * a.I, a.I, hs);
        __syncthreads();
    } else if constexpr (Q == RD_BLOCK) {   // the route's h row per 128 channels, here
        quant_row_block128<float, NW>(hrow_s, shs, reinterpret_cast<const float*>(a.h) + (long)r * a.I, a.I);
        __syncthreads();
        if (g32 == 0 && kp == 0)   // inspection copy of the route's h scales
            for (int i = threadIdx.x; i < a.I / 128; i += 64 * NW) a.sh_out[(long)r * (a.I / 128) + i] = shs[i];
    } else if constexpr (Q == RD_MX) {     // ... per 32 channels
        quant_row_mx32<float, NW>(hrow_s, shb, reinterpret_cast<const float*>(a.h) + (long)r * a.I, a.I);
        __syncthreads();
        if (g32 == 0 && kp == 0) {
            uint8_t* so = reinterpret_cast<uint8_t*>(a.sh_out) + (long)r * (a.I / 32);
            for (int i = threadIdx.x; i < a.I / 32; i += 64 * NW) so[mx_scale_pos(i)] = shb[i];
        }
    }

    float y = 0.0f;
    for (int s = s0; s < s0 + spw; s += U) {
        if (s != s0) {
            load_batch(s);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float d;
            if constexpr (Q == RD_MX) {
                d = dot_slice_mx(vw[u], hrow, s + u, hh, mw[u], shb, 8 * ((s + u) & 3));
            } else if constexpr (!FP8) {
                d = dot_slice_bf16(vw[u], va[u], 0.0f);
            } else {
                float v[32];
                lds_act_slice<true>(hrow, s + u, hh, v);
                d = dot_slice<FP8>(vw[u], v);
            }
            if constexpr (Q == RD_BLOCK) {
                const int kb = (s + u) / 2;
                const float sc = shs[kb] *
                                 a.s_d[((long)e * (a.I / 128) + kb) * (a.H / 128) + n0 / 128];
                y = fmaf(d, sc, y);
            } else {
                y += d;
            }
        }
    }
    y += __shfl_xor(y, 32);
    if (hh == 0) red[wave][lane] = y;
    __syncthreads();
    float v = 0.0f;
    if (wave == 0 && hh == 0) {
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[w][lane];
        float gw = gate;
        if constexpr (Q == RD_TENSOR) gw *= hs * sdw;
        v *= gw;
    }
    rd_part_publish(a, tb, t, g32, it, items, v, last_s);
}

// ------------------------------------------------------- Down, per block --
// When one output block's Down weights are small (k slots x 32 rows x I
// elements, at most 64 KB), a workgroup owns (token, 32 output columns) with
// all k route slots: its waves take (slot, K part) pieces, request each piece's
// weight slices at once, and the pieces meet in LDS in a fixed order -- no
// partial sums in memory and no arrival counter.  Larger blocks take the split
// form above, which spreads them over more CUs (one CU streams about 20 GB/s).
constexpr int kRdBlockWaves = 16;
constexpr int kRdBlockMaxSlices = 12;         // per piece, held in registers (bf16)
constexpr int kRdBlockMaxSlicesFp8 = 4;       // e4m3 (decoding needs more registers)
constexpr int kRdBlockMaxItems = 64;
constexpr int kRdBlockStage = kRdBlockMaxSlices * kSliceBytes;   // staged activations per wave
constexpr long kRdBlockMaxBytes = 64 * 1024;  // one block's Down weights

template <int Q>
__global__ void __launch_bounds__(64 * kRdBlockWaves) rd_down_block_kernel(const RdArgs a) {
    constexpr bool FP8 = Q != RD_BF16;
    constexpr int elem = FP8 ? 1 : 2;
    constexpr int MS = FP8 ? kRdBlockMaxSlicesFp8 : kRdBlockMaxSlices;
    constexpr int GPL = (MS * 16 + 63) / 64;   // fp32 h (per-tensor): groups of 4 values per lane
    constexpr int QPL = (MS * 4 + 63) / 64;    // bf16 h: 16-byte pieces per lane
    __shared__ __attribute__((aligned(16))) uint8_t hst_all[kRdBlockWaves * kRdBlockStage];
    __shared__ float red[kRdBlockMaxItems * 32];
    const int nw = blockDim.x >> 6;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int j = lane & 31, hh = lane >> 5;
    const int nb = a.H / 32, t = blockIdx.x / nb, g32 = blockIdx.x - t * nb;
    const int Kb = a.I * elem, NSL = Kb / kSliceBytes;
    const int KP = a.kp, spw = NSL / KP, items = a.k * KP;
    uint8_t* hst = hst_all + wave * kRdBlockStage;

    // One piece (route slot, K part): its weight slices and its activations are
    // requested together (clamped indices, masked after: a guarded load waits
    // for all before it); the slot's expert comes by a scalar load, so the
    // weight addresses wait only for that.
    u32x4 vw[MS][2];
    f32x4 hf[GPL];
    u32x4 hb[QPL];
    int r = 0, e = 0, s0 = 0;
    bool live = false;
    float gate = 0.0f, sdw = 1.0f;
    auto issue = [&](int it) __attribute__((always_inline)) {
        const int jj = it / KP, kp = it - jj * KP;
        r = t * a.k + jj;
        s0 = kp * spw;
        if constexpr (Q == RD_TENSOR) {
            const float* hp = reinterpret_cast<const float*>(a.h) + (long)r * a.I + s0 * 64;
            const int ng = spw * 16;
#pragma unroll
            for (int q = 0; q < GPL; ++q) hf[q] = *reinterpret_cast<const f32x4*>(hp + 4 * min(lane + 64 * q, ng - 1));
        } else {
            const u32x4* hp = reinterpret_cast<const u32x4*>(a.h + (long)r * Kb + s0 * 64);
            const int nq = spw * 4;
#pragma unroll
            for (int q = 0; q < QPL; ++q) hb[q] = hp[min(lane + 64 * q, nq - 1)];
        }
        e = ld_uniform(a.ids, r) - a.e0;   // index in this call's expert slice
        live = (unsigned)e < (unsigned)a.nloc;
        // the slot's gate and weight scale with its weights (used after the dot)
        gate = ld_uniform_f(a.tw, r);
        if constexpr (Q == RD_TENSOR) sdw = ld_uniform_f(a.s_d, live ? e : 0);
        if (live) {
            const uint8_t* wb = a.wd + (long)e * a.H * Kb + (long)g32 * 32 * Kb + (long)s0 * 2048 + lane * 16;
#pragma unroll
            for (int u = 0; u < MS; ++u)
                if (u < spw)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        vw[u][q] = *reinterpret_cast<const u32x4*>(wb + u * 2048 + q * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // the wave's first piece goes out before the h scale's inputs
    if (wave < items) issue(wave);

    float hs = 1.0f;
    if constexpr (Q == RD_TENSOR) {
        // the whole-tensor h scale from the Gate/Up workgroups' maxima (loads of
        // clamped indices, masked after)
        const int nmax = a.T * a.k * (a.I / 32) * a.rs;
        float m = 0.0f;
        for (int base = 0; base < nmax; base += 512) {
            float mv[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) mv[q] = a.hmax[min(base + lane + 64 * q, nmax - 1)];
#pragma unroll
            for (int q = 0; q < 8; ++q) m = base + lane + 64 * q < nmax ? fmaxf(m, mv[q]) : m;
        }
        hs = scale_from_amax(wave_max(m));
        if (blockIdx.x == 0 && threadIdx.x == 0) a.scal_out[1] = hs;   // inspection copy
    }
    for (int it = wave; it < items; it += nw) {
        if (it != wave) issue(it);
        if (!live) {   // another slice's expert: a zero piece
            if (hh == 0) red[it * 32 + j] = 0.0f;
            continue;
        }
        // the piece's activations into this wave's LDS area: bf16 h copied,
        // per-tensor fp32 h quantised into e4m3 codes
        if constexpr (Q == RD_TENSOR) {
            const int ng = spw * 16;
#pragma unroll
            for (int q = 0; q < GPL; ++q) {
                const int gi = lane + 64 * q;
                if (gi < ng)
                    reinterpret_cast<uint32_t*>(hst)[gi] =
                        f32x4_to_e4m3x4(hf[q][0] / hs, hf[q][1] / hs, hf[q][2] / hs, hf[q][3] / hs);
            }
        } else {
            const int nq = spw * 4;
#pragma unroll
            for (int q = 0; q < QPL; ++q)
                if (lane + 64 * q < nq) reinterpret_cast<u32x4*>(hst)[lane + 64 * q] = hb[q];
        }
        // one wave's LDS accesses execute in order; this keeps the compiler from
        // moving the reads above the writes
        __asm__ volatile("" ::: "memory");
        float y = 0.0f;
#pragma unroll
        for (int u = 0; u < MS; ++u) {
            if (u < spw) {
                if constexpr (!FP8) {
                    u32x4 xw[2];
                    lds_act_raw(hst, u, hh, xw);
                    y = dot_slice_bf16(vw[u], xw, y);
                } else {
                    float v[32];
                    lds_act_slice<true>(hst, u, hh, v);
                    y += dot_slice<true>(vw[u], v);
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // one slice's activations at a time
        }
        y += __shfl_xor(y, 32);
        float gw = gate;
        if constexpr (Q == RD_TENSOR) gw *= hs * sdw;
        if (hh == 0) red[it * 32 + j] = gw * y;
        __asm__ volatile("" ::: "memory");
    }
    __syncthreads();
    if (wave == 0 && hh == 0) {
        float o = 0.0f;
        for (int it = 0; it < items; ++it) o += red[it * 32 + lane];   // fixed order
        uint16_t* op = a.out + (long)t * a.H + down_col_of_packed(32 * g32 + lane);
        if (a.acc) o += __uint_as_float((uint32_t)*op << 16);   // shared output: one rounding of out + sum
        *op = f32_to_bf16(o);
    }
}

// ----------------------------------------------------------------------------

static RdArgs rd_args(const FwdPlan& p) {
    RdArgs a{};
    a.act = reinterpret_cast<const uint8_t*>(p.x);
    a.ids = p.ids;
    a.tw = p.tw;
    a.wgu = static_cast<const uint8_t*>(p.wgu);
    a.wd = static_cast<const uint8_t*>(p.wd);
    a.s_gu = p.s_gu;
    a.s_d = p.s_d;
    a.h = static_cast<const uint8_t*>(p.h);
    a.hout = p.h;
    a.hmax = p.rd_hmax;
    a.part = p.rd_part;
    a.cnt = p.rd_cnt;
    a.out = p.out;
    a.T = p.T; a.H = p.H; a.I = p.I; a.E = p.E; a.k = p.k;
    a.kp = 1;
    a.rs = rd_gate_up_split(p.T, p.H, p.I, p.k, p.quant);
    a.e0 = p.e0;
    a.nloc = p.nloc;
    a.acc = p.acc;
    a.logits = p.logits;
    a.ids_w = p.ids_w;
    a.tw_w = p.tw_w;
    a.xq_out = p.xq;
    a.sx_out = p.sx;
    a.scal_out = p.scal;
    a.sh_out = p.sh;
    return a;
}

// Slices per load batch: the largest of 8, 6, 4, 3, 2, 1 that divides the
// wave's slice count n and is at most cap (the loops walk n in steps of U and
// must never step past the last slice).
static int largest_unroll(int n, int cap) {
    for (int u : {8, 6, 4, 3, 2})
        if (u <= cap && n % u == 0) return u;
    return 1;
}

// ---- Gate/Up launch shape
//
// Three choices per call: the row split RS (1, 2 or 4 workgroups share a
// 32-row block pair, each taking RW = 32/RS rows of every slice: at RS = 4
// one 128-byte line per slice half), the waves per workgroup nw (K split
// evenly between them) and the slices per load batch U.  One workgroup
// streams at only a fraction of HBM bandwidth and a decode step is short, so
// the rule maximises the number of waves in flight (up to about 4096) among
// the shapes whose whole grid is resident at once: a second round of
// workgroups would double the kernel's time.  Residency comes from the
// runtime's occupancy figure for the exact kernel.  Ties keep the smaller
// split (measured: a split that only repacks the same waves into more,
// smaller workgroups loses a little).  The blockwise format splits too: each
// lane reads the scales of its own slice's 128-deep block.
struct RdGuCfg {
    int rs, nw, U;
};

// two load batches live in registers: 16-wave groups (128 VGPRs) take at most
// 2 bf16 slices (1 e4m3) per batch, smaller groups 4 (2 e4m3), which keeps
// every launched variant clear of spills
static int rd_gu_unroll(int quant, int nw, int per) {
    return largest_unroll(per, nw == 16 ? (quant != Q_BF16 ? 1 : 2) : (quant != Q_BF16 ? 2 : 4));
}

template <int Q, int NW>
static const void* rd_gu_fn_nw(int U) {
    if constexpr (NW < 16) {
        if (U == 4) return reinterpret_cast<const void*>(&rd_gate_up_kernel<Q, NW, 4>);
        if (U == 3) return reinterpret_cast<const void*>(&rd_gate_up_kernel<Q, NW, 3>);
    }
    if (U == 2) {
        if constexpr (NW < 16 || Q == RD_BF16) return reinterpret_cast<const void*>(&rd_gate_up_kernel<Q, NW, 2>);
        return nullptr;   // (e4m3 16-wave groups take one slice per batch)
    }
    if (U == 1) return reinterpret_cast<const void*>(&rd_gate_up_kernel<Q, NW, 1>);
    return nullptr;
}

template <int Q>
static const void* rd_gu_fn_q(int nw, int U) {
    switch (nw) {
        case 1: return rd_gu_fn_nw<Q, 1>(U);
        case 2: return rd_gu_fn_nw<Q, 2>(U);
        case 4: return rd_gu_fn_nw<Q, 4>(U);
        case 8: return rd_gu_fn_nw<Q, 8>(U);
        case 16: return rd_gu_fn_nw<Q, 16>(U);
        default: return nullptr;
    }
}

// the instantiated kernel for (quant, nw, U), null for a combination that is
// not built
static const void* rd_gu_fn(int quant, int nw, int U) {
    if (quant == Q_BF16) return rd_gu_fn_q<RD_BF16>(nw, U);
    if (quant == Q_FP8_TENSOR) return rd_gu_fn_q<RD_TENSOR>(nw, U);
    if (quant == Q_FP8_MX) return rd_gu_fn_q<RD_MX>(nw, U);
    return rd_gu_fn_q<RD_BLOCK>(nw, U);
}

// Workgroups of one kernel resident on the whole device at once, cached per
// (device, quant, nw, U).  0 when the runtime cannot tell (the shape is then
// never taken as resident).
constexpr int kRdMaxDevices = 64;
static long rd_gu_resident(int quant, int nw, int U) {
    static std::atomic<int> cus[kRdMaxDevices];
    static std::atomic<int> occ[kRdMaxDevices][4][5][9];   // 1 + occupancy, 0 = not asked yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kRdMaxDevices) return 0;
    int lg = 0;
    while ((1 << lg) < nw) ++lg;
    if (quant < 0 || quant > 3 || lg > 4 || U < 1 || U > 8) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 0;
        n = c + 1;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    int o = occ[dev][quant][lg][U].load(std::memory_order_relaxed);
    if (o == 0) {
        const void* fn = rd_gu_fn(quant, nw, U);
        int blocks = 0;
        if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, 64 * nw, 0) != hipSuccess) blocks = 0;
        o = blocks + 1;
        occ[dev][quant][lg][U].store(o, std::memory_order_relaxed);
    }
    return (long)(n - 1) * (o - 1);
}

static RdGuCfg rd_gu_cfg(int T, int H, int I, int k, int quant) {
    const int NSL = H * (quant == Q_BF16 ? 2 : 1) / kSliceBytes;
    const long groups = (long)T * k * (I / 32);
    RdGuCfg best{0, 0, 0};
    long best_waves = -1;
    for (int rs = 1; rs <= 4; rs *= 2) {
        if (NSL % rs != 0) break;
        const int NSS = NSL / rs;
        const long wgs = groups * rs;
        RdGuCfg c{rs, 1, rd_gu_unroll(quant, 1, NSS)};
        long waves = 0;   // one-wave groups when no larger shape is resident
        for (int nw = 16; nw >= 1; nw /= 2) {
            if (NSS % nw != 0 || wgs * nw > 4096) continue;
            const int U = rd_gu_unroll(quant, nw, NSS / nw);
            if (wgs <= rd_gu_resident(quant, nw, U)) {
                c = RdGuCfg{rs, nw, U};
                waves = wgs * nw;
                break;
            }
        }
        if (waves > best_waves) {
            best = c;
            best_waves = waves;
        }
    }
    return best;
}

int rd_gate_up_split(int T, int H, int I, int k, int quant) { return rd_gu_cfg(T, H, I, k, quant).rs; }

hipError_t launch_route_direct_gate_up(const FwdPlan& p, hipStream_t st) {
    RdArgs a = rd_args(p);
    const RdGuCfg c = rd_gu_cfg(p.T, p.H, p.I, p.k, p.quant);
    const int NSL = p.H * (p.quant == Q_BF16 ? 2 : 1) / kSliceBytes;
    // the kernel walks NSL / rs super-slices in nw x U steps and never past the end
    if (c.rs < 1 || c.rs > 4 || NSL % c.rs != 0 || (NSL / c.rs) % (c.nw * c.U) != 0) return hipErrorInvalidValue;
    const void* fn = rd_gu_fn(p.quant, c.nw, c.U);
    if (!fn) return hipErrorInvalidValue;
    void* args[] = {&a};
    return hipExtLaunchKernel(fn, dim3(p.T * p.k, p.I / 32, c.rs), dim3(64 * c.nw), args, 0, st, p.ev_first_start,
                              p.ev_stage_end, 0);
}

// Down split: K parts per route (1, 2 or 4, dividing NSL) only while the grid
// stays small (every item of an output block takes a ticket from the same
// counter, and those atomics serialise), then waves per workgroup (1, 2 or 4)
// until each wave streams at most 4 slices (blockwise E=128 decode: 0.8-2.2 us
// faster than at most 8, bf16 unchanged), then the batch size.
struct RdDownCfg {
    int kp, nw, U;
};
static RdDownCfg rd_down_cfg(int T, int H, int I, int k, int quant) {
    const int elem = quant == Q_BF16 ? 2 : 1;
    const int NSL = I * elem / kSliceBytes;
    const long tb = (long)T * (H / 32);
    RdDownCfg c{1, 1, 1};
    while (c.kp < 4 && NSL % (c.kp * 2) == 0 && tb * k * c.kp * 2 <= 256) c.kp *= 2;
    const int per = NSL / c.kp;
    while (c.nw < 4 && per % (c.nw * 2) == 0 && per / c.nw > 4) c.nw *= 2;
    c.U = largest_unroll(per / c.nw, 8);
    return c;
}

int rd_down_items(int T, int H, int I, int k, int quant) { return k * rd_down_cfg(T, H, I, k, quant).kp; }

template <int Q, int NW, int KP>
static hipError_t rd_dn_kp(const RdArgs& a, int U, hipStream_t st, hipEvent_t ev) {
    dim3 grid(a.T * (a.H / 32), a.k * KP);
    switch (U) {
        case 8: hipExtLaunchKernelGGL((rd_down_part_kernel<Q, NW, KP, 8>), grid, dim3(64 * NW), 0, st, nullptr, ev, 0, a); break;
        case 6: hipExtLaunchKernelGGL((rd_down_part_kernel<Q, NW, KP, 6>), grid, dim3(64 * NW), 0, st, nullptr, ev, 0, a); break;
        case 4: hipExtLaunchKernelGGL((rd_down_part_kernel<Q, NW, KP, 4>), grid, dim3(64 * NW), 0, st, nullptr, ev, 0, a); break;
        case 3: hipExtLaunchKernelGGL((rd_down_part_kernel<Q, NW, KP, 3>), grid, dim3(64 * NW), 0, st, nullptr, ev, 0, a); break;
        case 2: hipExtLaunchKernelGGL((rd_down_part_kernel<Q, NW, KP, 2>), grid, dim3(64 * NW), 0, st, nullptr, ev, 0, a); break;
        default: hipExtLaunchKernelGGL((rd_down_part_kernel<Q, NW, KP, 1>), grid, dim3(64 * NW), 0, st, nullptr, ev, 0, a); break;
    }
    return hipGetLastError();
}

template <int Q, int NW>
static hipError_t rd_dn_nw(const RdArgs& a, const RdDownCfg& c, hipStream_t st, hipEvent_t ev) {
    switch (c.kp) {
        case 1: return rd_dn_kp<Q, NW, 1>(a, c.U, st, ev);
        case 2: return rd_dn_kp<Q, NW, 2>(a, c.U, st, ev);
        default: return rd_dn_kp<Q, NW, 4>(a, c.U, st, ev);
    }
}

template <int Q>
static hipError_t rd_dn(const RdArgs& a, int quant, hipStream_t st, hipEvent_t ev) {
    const int elem = Q == RD_BF16 ? 2 : 1;
    const int NSL = a.I * elem / kSliceBytes;
    const RdDownCfg c = rd_down_cfg(a.T, a.H, a.I, a.k, quant);
    if (NSL % (c.kp * c.nw) != 0 || (NSL / c.kp / c.nw) % c.U != 0) return hipErrorInvalidValue;
    switch (c.nw) {
        case 1: return rd_dn_nw<Q, 1>(a, c, st, ev);
        case 2: return rd_dn_nw<Q, 2>(a, c, st, ev);
        default: return rd_dn_nw<Q, 4>(a, c, st, ev);
    }
}

// Per-block Down (bf16, FP8 per-tensor) when a block's weights are small:
// K parts per slot (1, 2, 4) while k * kp fits 16 waves or a piece would exceed
// the register budget; waves = min(16, k * kp), looping over pieces.
struct RdBlockCfg {
    bool ok;
    int kp, nw;
};
static RdBlockCfg rd_block_cfg(int H, int I, int k, int quant) {
    RdBlockCfg c{false, 1, 1};
    if (quant == Q_FP8_BLOCK || quant == Q_FP8_MX) return c;
    const int elem = quant == Q_BF16 ? 2 : 1;
    const int NSL = I * elem / kSliceBytes, ms = quant == Q_BF16 ? kRdBlockMaxSlices : kRdBlockMaxSlicesFp8;
    if ((long)k * 32 * I * elem > kRdBlockMaxBytes || NSL < 1) return c;
    while (c.kp < 4 && NSL % (c.kp * 2) == 0 && (k * c.kp * 2 <= kRdBlockWaves || NSL / c.kp > ms)) c.kp *= 2;
    if (NSL % c.kp != 0 || NSL / c.kp > ms || k * c.kp > kRdBlockMaxItems) return c;
    c.nw = k * c.kp < kRdBlockWaves ? k * c.kp : kRdBlockWaves;
    c.ok = true;
    (void)H;
    return c;
}

RdLaunchInfo rd_launch_info(int T, int H, int I, int k, int quant) {
    RdLaunchInfo li{};
    const RdGuCfg c = rd_gu_cfg(T, H, I, k, quant);
    li.gu_split = c.rs;
    li.gu_waves = c.nw;
    const RdBlockCfg bc = rd_block_cfg(H, I, k, quant);
    if (bc.ok) {
        li.down_form = 1;
        li.down_parts = bc.kp;
    } else {
        li.down_form = 0;
        li.down_parts = rd_down_cfg(T, H, I, k, quant).kp;
    }
    return li;
}

hipError_t launch_route_direct_down(const FwdPlan& p, hipStream_t st) {
    RdArgs a = rd_args(p);
    const RdBlockCfg bc = rd_block_cfg(p.H, p.I, p.k, p.quant);
    if (bc.ok) {
        a.kp = bc.kp;
        const dim3 grid((unsigned)((long)p.T * (p.H / 32))), block(64 * bc.nw);
        if (p.quant == Q_BF16)
            hipExtLaunchKernelGGL((rd_down_block_kernel<RD_BF16>), grid, block, 0, st, nullptr, p.ev_stage_end, 0, a);
        else
            hipExtLaunchKernelGGL((rd_down_block_kernel<RD_TENSOR>), grid, block, 0, st, nullptr, p.ev_stage_end, 0, a);
        return hipGetLastError();
    }
    if (p.quant == Q_BF16) return rd_dn<RD_BF16>(a, p.quant, st, p.ev_stage_end);
    if (p.quant == Q_FP8_TENSOR) return rd_dn<RD_TENSOR>(a, p.quant, st, p.ev_stage_end);
    if (p.quant == Q_FP8_MX) return rd_dn<RD_MX>(a, p.quant, st, p.ev_stage_end);
    return rd_dn<RD_BLOCK>(a, p.quant, st, p.ev_stage_end);
}

}  // namespace moe
