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
// elements and does 2 flops per element, so there is nothing for the matrix
// cores to gain.  The kernels are built to keep as many 16-byte weight loads
// in flight as possible:
//  * Gate/Up: one wave per (route, JW h columns) streams 2*JW packed weight
//    rows (K-contiguous) with 16-byte lane loads, dots them with x (or its e4m3
//    codes) in fp32, reduces across the wave, applies SwiGLU and stores h
//    (bf16, or fp32 for the FP8 requantisation that follows);
//  * Down + combine: a workgroup of 4 waves owns 4 output columns of one token;
//    wave w handles slots j = w, w+4, ...; 16 lanes share one weight row.  The
//    four per-wave partial sums are added in wave order, so the top-k combine
//    has a fixed summation order and needs no atomics and no y round trip.
#include "common.cuh"
#include "launch.h"

namespace moe {

// dot of 16 bytes of weights with 16 bytes of activations
template <bool FP8>
__device__ __forceinline__ float dot16(const u32x4& w, const u32x4& a) {
    float s = 0.0f;
    if constexpr (!FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = fmaf(__uint_as_float(w[i] << 16), __uint_as_float(a[i] << 16), s);
            s = fmaf(__uint_as_float(w[i] & 0xffff0000u), __uint_as_float(a[i] & 0xffff0000u), s);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = fmaf(e4m3_to_f32<0>(w[i]), e4m3_to_f32<0>(a[i]), s);
            s = fmaf(e4m3_to_f32<1>(w[i]), e4m3_to_f32<1>(a[i]), s);
            s = fmaf(e4m3_to_f32<2>(w[i]), e4m3_to_f32<2>(a[i]), s);
            s = fmaf(e4m3_to_f32<3>(w[i]), e4m3_to_f32<3>(a[i]), s);
        }
    }
    return s;
}

struct RdArgs {
    const uint8_t* act;      // x bf16 [T,H] or xq e4m3 [T,H]
    const float* sx;         // block: [T][H/128]; tensor: &s_x
    const int32_t* ids;      // [T*k]
    const float* tw;         // [T*k]
    const uint8_t* wgu;      // packed [E][2I][H]
    const uint8_t* wd;       // packed [E][H][I]
    const float* s_gu;
    const float* s_d;
    const uint8_t* h;        // bf16 h [R][I] (bf16) or e4m3 hq [R][I] (fp8), Down input
    const float* sh;         // block: [R][I/128]; tensor: &s_h
    void* hout;              // Gate/Up output: bf16 [R][I] or fp32 [R][I]
    uint16_t* out;           // [T][H]
    int T, H, I, E, k;
};

// ---------------------------------------------------------------- Gate/Up --
template <bool FP8, int SC, int NCH, int JW>
__global__ void __launch_bounds__(256)
rd_gate_up_kernel(const RdArgs a) {
    const int lane = lane_id(), wave = threadIdx.x / 64;
    const int r = blockIdx.x;
    const int j0 = (blockIdx.y * 4 + wave) * JW;
    if (j0 >= a.I) return;
    const int t = r / a.k, e = a.ids[r];
    const int elem = FP8 ? 1 : 2;
    const long Kb = (long)a.H * elem;
    const int chunks = (int)(Kb / 16);
    const uint8_t* xa = a.act + (long)t * Kb;

    const uint8_t* wrow[2 * JW];
#pragma unroll
    for (int q = 0; q < JW; ++q) {
        const int j = j0 + q;
        const long gate_row = 32L * (j / 16) + (j % 16);
        wrow[2 * q] = a.wgu + ((long)e * 2 * a.I + gate_row) * Kb;
        wrow[2 * q + 1] = a.wgu + ((long)e * 2 * a.I + gate_row + 16) * Kb;
    }
    u32x4 wv[2 * JW][NCH], xv[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        const bool ok = c < chunks;
#pragma unroll
        for (int q = 0; q < 2 * JW; ++q)
            wv[q][i] = ok ? *reinterpret_cast<const u32x4*>(wrow[q] + c * 16) : u32x4{0, 0, 0, 0};
        xv[i] = ok ? *reinterpret_cast<const u32x4*>(xa + c * 16) : u32x4{0, 0, 0, 0};
    }
    float acc[2 * JW];
#pragma unroll
    for (int q = 0; q < 2 * JW; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if constexpr (SC == 2) {
            if (c < chunks) {
                const int kb = c / 8;   // 16 e4m3 per chunk, 128 per block
                const float s_a = a.sx[(long)t * (a.H / 128) + kb];
#pragma unroll
                for (int q = 0; q < 2 * JW; ++q) {
                    const int j = j0 + q / 2;
                    const int col = (q & 1) ? a.I + j : j;
                    const float s_w = a.s_gu[((long)e * (a.H / 128) + kb) * (2 * a.I / 128) + col / 128];
                    acc[q] = fmaf(dot16<FP8>(wv[q][i], xv[i]), s_a * s_w, acc[q]);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 2 * JW; ++q) acc[q] += dot16<FP8>(wv[q][i], xv[i]);
        }
    }
#pragma unroll
    for (int q = 0; q < 2 * JW; ++q) acc[q] = wave_sum(acc[q]);
    if (SC == 1) {
        const float f = a.sx[0] * a.s_gu[e];
#pragma unroll
        for (int q = 0; q < 2 * JW; ++q) acc[q] *= f;
    }
    if (lane < JW) {
        float hv = 0.0f;
#pragma unroll
        for (int q = 0; q < JW; ++q)
            if (q == lane) hv = silu(acc[2 * q]) * acc[2 * q + 1];
        const int j = j0 + lane;
        if (j < a.I) {
            if constexpr (!FP8) {
                static_cast<uint16_t*>(a.hout)[(long)r * a.I + j] = f32_to_bf16(hv);
            } else {
                static_cast<float*>(a.hout)[(long)r * a.I + j] = hv;   // requantised afterwards
            }
        }
    }
}

// ------------------------------------------------------------ Down+combine --
template <bool FP8, int SC, int NCH>
__global__ void __launch_bounds__(256)
rd_down_combine_kernel(const RdArgs a) {
    __shared__ float part[4][4];
    const int lane = lane_id(), wave = threadIdx.x / 64;
    const int t = blockIdx.x;
    const int grp = lane / 16, sub = lane % 16;
    const int n = blockIdx.y * 4 + grp;          // output column of this 16-lane group
    const int elem = FP8 ? 1 : 2;
    const long Kb = (long)a.I * elem;
    const int chunks = (int)(Kb / 16);
    float o = 0.0f;
    for (int j = wave; j < a.k; j += 4) {
        const int r = t * a.k + j;
        const int e = a.ids[r];
        const uint8_t* wrow = a.wd + ((long)e * a.H + n) * Kb;
        const uint8_t* hrow = a.h + (long)r * Kb;
        u32x4 wv[NCH], hv[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = sub + 16 * i;
            const bool ok = c < chunks;
            wv[i] = ok ? *reinterpret_cast<const u32x4*>(wrow + c * 16) : u32x4{0, 0, 0, 0};
            hv[i] = ok ? *reinterpret_cast<const u32x4*>(hrow + c * 16) : u32x4{0, 0, 0, 0};
        }
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = sub + 16 * i;
            if constexpr (SC == 2) {
                if (c < chunks) {
                    const int kb = c / 8;
                    const float s = a.sh[(long)r * (a.I / 128) + kb] *
                                    a.s_d[((long)e * (a.I / 128) + kb) * (a.H / 128) + n / 128];
                    y = fmaf(dot16<FP8>(wv[i], hv[i]), s, y);
                }
            } else {
                y += dot16<FP8>(wv[i], hv[i]);
            }
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) y += __shfl_xor(y, off);
        if (SC == 1) y *= a.sh[0] * a.s_d[e];
        o = fmaf(a.tw[r], y, o);
    }
    if (sub == 0) part[wave][grp] = o;
    __syncthreads();
    if (threadIdx.x < 4) {
        const int g2 = threadIdx.x;
        const float s = ((part[0][g2] + part[1][g2]) + part[2][g2]) + part[3][g2];
        a.out[(long)t * a.H + blockIdx.y * 4 + g2] = f32_to_bf16(s);
    }
}

// ----------------------------------------------------------------------------

static RdArgs rd_args(const FwdPlan& p) {
    RdArgs a{};
    const bool fp8 = p.quant != Q_BF16;
    a.act = fp8 ? p.xq : reinterpret_cast<const uint8_t*>(p.x);
    a.sx = p.quant == Q_FP8_BLOCK ? p.sx : &p.scal[0];
    a.ids = p.ids;
    a.tw = p.tw;
    a.wgu = static_cast<const uint8_t*>(p.wgu);
    a.wd = static_cast<const uint8_t*>(p.wd);
    a.s_gu = p.s_gu;
    a.s_d = p.s_d;
    a.h = fp8 ? p.hq : static_cast<const uint8_t*>(p.h);
    a.sh = p.quant == Q_FP8_BLOCK ? p.sh : &p.scal[1];
    a.hout = p.h;
    a.out = p.out;
    a.T = p.T; a.H = p.H; a.I = p.I; a.E = p.E; a.k = p.k;
    return a;
}

template <bool FP8, int SC, int JW>
static hipError_t rd_gu(const RdArgs& a, int nch, hipStream_t st) {
    dim3 grid(a.T * a.k, ceil_div(a.I, 4 * JW));
    switch (nch) {
        case 1: hipLaunchKernelGGL((rd_gate_up_kernel<FP8, SC, 1, JW>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((rd_gate_up_kernel<FP8, SC, 2, JW>), grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL((rd_gate_up_kernel<FP8, SC, 4, JW>), grid, dim3(256), 0, st, a); break;
        case 8: hipLaunchKernelGGL((rd_gate_up_kernel<FP8, SC, 8, JW>), grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

static int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

hipError_t launch_route_direct_gate_up(const FwdPlan& p, hipStream_t st) {
    const RdArgs a = rd_args(p);
    const int elem = p.quant == Q_BF16 ? 2 : 1;
    const int nch = pow2_at_least(ceil_div(p.H * elem / 16, 64));
    if (nch > 8) return hipErrorInvalidValue;
    const bool wide = (long)p.T * p.k * p.I >= 8192;   // enough waves: 2 h columns per wave
    if (p.quant == Q_BF16) return wide ? rd_gu<false, 0, 2>(a, nch, st) : rd_gu<false, 0, 1>(a, nch, st);
    if (p.quant == Q_FP8_TENSOR) return wide ? rd_gu<true, 1, 2>(a, nch, st) : rd_gu<true, 1, 1>(a, nch, st);
    return wide ? rd_gu<true, 2, 2>(a, nch, st) : rd_gu<true, 2, 1>(a, nch, st);
}

template <bool FP8, int SC>
static hipError_t rd_dn(const RdArgs& a, int nch, hipStream_t st) {
    dim3 grid(a.T, a.H / 4);
    switch (nch) {
        case 1: hipLaunchKernelGGL((rd_down_combine_kernel<FP8, SC, 1>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((rd_down_combine_kernel<FP8, SC, 2>), grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL((rd_down_combine_kernel<FP8, SC, 4>), grid, dim3(256), 0, st, a); break;
        case 8: hipLaunchKernelGGL((rd_down_combine_kernel<FP8, SC, 8>), grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_route_direct_down(const FwdPlan& p, hipStream_t st) {
    const RdArgs a = rd_args(p);
    const int elem = p.quant == Q_BF16 ? 2 : 1;
    const int nch = pow2_at_least(ceil_div(p.I * elem / 16, 16));
    if (nch > 8) return hipErrorInvalidValue;
    if (p.quant == Q_BF16) return rd_dn<false, 0>(a, nch, st);
    if (p.quant == Q_FP8_TENSOR) return rd_dn<true, 1>(a, nch, st);
    return rd_dn<true, 2>(a, nch, st);
}

}  // namespace moe
