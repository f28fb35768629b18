// Small kernels of the MoE forward on gfx950: per-call initialisation and the
// device-built tile map of the grouped path, FP8 activation quantisation, the
// Down-input requantisation, and the deterministic top-k combine.
//
// Tile map ("perf: add small-batch route MMA for MoE", Motivation: prefix/task
// map; Code changes: task-map bound tightened to the non-empty workload;
// "[mxfp8 moe training] add per group blocked scale kernels", Summary: per-group
// start rows computed on device with no device-to-host sync): expert e owns
// ceil(count_e / 128) row tiles; the tiles of all experts are listed in expert
// order with their first sorted row, and the count of listed tiles is left in
// device memory.  GEMM grids are launched at the bound ceil(R/128) + min(E, R)
// and workgroups past the count exit at once.
//
// Combine ("Port necessary FBGEMM MoE kernels", Summary: scatter_add_dense_tokens;
// "perf: add small-batch route MMA for MoE", Code changes: top-k reduction):
// out[t] = sum_{j=0..k-1} w[t,j] * y[route_pos[t*k + j]], where y holds the Down
// outputs in sorted (expert) order and route_pos is the inverse of the sort,
// summed in fp32 in ascending j and rounded to bf16 once -- no atomics, so two
// runs give the same bits.
#include <hip/hip_ext.h>

#include "common.cuh"
#include "launch.h"

namespace moe {

int grouped_max_tiles(int R, int E) { return ceil_div(R, kGemmBM) + (E < R ? E : R); }

__global__ void __launch_bounds__(kMaxExperts)
forward_init_kernel(int E, const int32_t* __restrict__ offsets, int build_tiles,
                    int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles,
                    uint32_t* __restrict__ amax) {
    __shared__ int32_t wsum[kMaxExperts / kWave];
    const int e = threadIdx.x, lane = lane_id(), wave = e / kWave;
    if (amax && e < 2) amax[e] = 0u;
    if (!build_tiles) return;
    int nt = 0, o0 = 0;
    if (e < E) {
        o0 = offsets[e];
        nt = ceil_div(offsets[e + 1] - o0, kGemmBM);
    }
    int incl = nt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int start = before + incl - nt;
    for (int i = 0; i < nt; ++i) {
        tiles[2 * (start + i)] = e;
        tiles[2 * (start + i) + 1] = o0 + i * kGemmBM;
    }
    if (e == blockDim.x - 1) ntiles[0] = before + incl;
}

hipError_t launch_forward_init(const FwdPlan& p, bool build_tiles, hipStream_t st) {
    // the tile map covers the expert slice: offsets + e0 for nloc experts, so a
    // tile names its expert by its index in the slice (the weights' index)
    hipExtLaunchKernelGGL(forward_init_kernel, dim3(1), dim3(kMaxExperts), 0, st, p.ev_first_start, p.ev_stage_end, 0,
                          p.nloc, p.offsets + p.e0, build_tiles ? 1 : 0, p.tiles, p.ntiles, p.amax);
    return hipGetLastError();
}

// ---------------------------------------------------------------- FP8 quant --

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float v[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

__device__ __forceinline__ void store8_e4m3(uint8_t* q, const float v[8], float s) {
    uint2 w;
    w.x = f32x4_to_e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
    w.y = f32x4_to_e4m3x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
    *reinterpret_cast<uint2*>(q) = w;
}

// Per row, per 128 columns: s = amax/448, q = e4m3(v / s).  16 threads per group.
template <typename TIn>
__global__ void __launch_bounds__(256)
quant_block128_kernel(const TIn* __restrict__ in, int rows, int cols, uint8_t* __restrict__ q,
                      float* __restrict__ scales) {
    const int groups_per_row = cols / 128;
    const long g = (long)blockIdx.x * 16 + threadIdx.x / 16;
    if (g >= (long)rows * groups_per_row) return;
    const int sub = threadIdx.x & 15;
    const long row = g / groups_per_row;
    const int c = (int)(g % groups_per_row);
    const long base = row * cols + (long)c * 128 + sub * 8;
    float v[8];
    load8<TIn>(in + base, v);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    const float s = scale_from_amax(a);
    store8_e4m3(q + base, v, s);
    if (sub == 0) scales[row * groups_per_row + c] = s;
}

// MX: per row, per 32 columns, E8M0 byte b = 2^(floor(log2 amax) - 8) (the
// float exponent field of amax less 8, at least 0) and codes e4m3(v * 2^(127-b))
// (exact power-of-two scaling).  4 threads per group.  The bytes of a row go in
// the order the MX GEMM reads them: group c at 8(c/8) + 4(c%2) + (c%8)/2, so
// dword 2g + hh holds groups 8g + hh, 8g + 2 + hh, 8g + 4 + hh, 8g + 6 + hh.
template <typename TIn>
__global__ void __launch_bounds__(256)
quant_mx32_kernel(const TIn* __restrict__ in, int rows, int cols, uint8_t* __restrict__ q,
                  uint8_t* __restrict__ scales) {
    const int gpr = cols / 32;
    const long g = (long)blockIdx.x * 64 + threadIdx.x / 4;
    if (g >= (long)rows * gpr) return;
    const int sub = threadIdx.x & 3;
    const long row = g / gpr;
    const int c = (int)(g % gpr);
    const long base = row * cols + (long)c * 32 + sub * 8;
    float v[8];
    load8<TIn>(in + base, v);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    const uint32_t b = mx_byte(a);
    const float inv = mx_inv(b);   // 2^(127 - b)
    uint2 w;
    w.x = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    w.y = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<uint2*>(q + base) = w;
    if (sub == 0) scales[row * gpr + mx_scale_pos(c)] = (uint8_t)b;
}

// amax over n values (n % 8 == 0), folded into *amax_bits with atomicMax on
// the bit pattern (non-negative floats order like their bits).
// Element range [lo, hi) of a row-major tensor with `cols` columns: all n
// elements, or (rows != null) the sorted rows [rows[0], rows[nr]) of an expert
// slice (its routes are contiguous in sorted order).
struct ElemRange {
    const int32_t* rows;
    int nr, cols;
};
__device__ __forceinline__ void elem_range(const ElemRange& g, long n, long& lo, long& hi) {
    lo = 0;
    hi = n;
    if (g.rows) {
        lo = (long)g.rows[0] * g.cols;
        hi = (long)g.rows[g.nr] * g.cols;
    }
}

template <typename TIn>
__global__ void __launch_bounds__(256)
amax_kernel(const TIn* __restrict__ in, long n, ElemRange er, uint32_t* __restrict__ amax_bits) {
    float a = 0.0f;
    long lo, hi;
    elem_range(er, n, lo, hi);
    for (long i = lo + ((long)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < hi;
         i += (long)gridDim.x * blockDim.x * 8) {
        float v[8];
        load8<TIn>(in + i, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
    }
    __shared__ float part[256 / kWave];
    a = wave_max(a);
    if (lane_id() == 0) part[threadIdx.x / kWave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x / kWave); ++w) a = fmaxf(a, part[w]);
        atomicMax(amax_bits, __float_as_uint(a));   // one atomic per workgroup
    }
}

template <typename TIn>
__global__ void __launch_bounds__(256)
quant_tensor_kernel(const TIn* __restrict__ in, long n, ElemRange er, const uint32_t* __restrict__ amax_bits,
                    uint8_t* __restrict__ q, float* __restrict__ scale_out) {
    const float s = scale_from_amax(__uint_as_float(*amax_bits));
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    long lo, hi;
    elem_range(er, n, lo, hi);
    for (long i = lo + ((long)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < hi;
         i += (long)gridDim.x * blockDim.x * 8) {
        float v[8];
        load8<TIn>(in + i, v);
        store8_e4m3(q + i, v, s);
    }
}

// One workgroup does amax and quantisation of a small tensor in one launch.
template <typename TIn>
__global__ void __launch_bounds__(1024)
quant_tensor_small_kernel(const TIn* __restrict__ in, long n, ElemRange er, uint8_t* __restrict__ q,
                          float* __restrict__ scale_out) {
    __shared__ float part[1024 / kWave];
    float a = 0.0f;
    long lo, hi;
    elem_range(er, n, lo, hi);
    for (long i = lo + (long)threadIdx.x * 8; i < hi; i += (long)blockDim.x * 8) {
        float v[8];
        load8<TIn>(in + i, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
    }
    a = wave_max(a);
    if (lane_id() == 0) part[threadIdx.x / kWave] = a;
    __syncthreads();
    a = 0.0f;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) a = fmaxf(a, part[w]);
    const float s = scale_from_amax(a);
    if (threadIdx.x == 0) *scale_out = s;
    for (long i = lo + (long)threadIdx.x * 8; i < hi; i += (long)blockDim.x * 8) {
        float v[8];
        load8<TIn>(in + i, v);
        store8_e4m3(q + i, v, s);
    }
}

constexpr long kSmallQuant = 1L << 16;

hipError_t launch_quant_x(const FwdPlan& p, hipStream_t st) {
    if (p.quant == Q_FP8_MX) {
        const long groups = (long)p.T * (p.H / 32);
        hipExtLaunchKernelGGL(quant_mx32_kernel<uint16_t>, dim3((unsigned)((groups + 63) / 64)), dim3(256), 0, st,
                              nullptr, p.ev_stage_end, 0, p.x, p.T, p.H, p.xq, reinterpret_cast<uint8_t*>(p.sx));
        return hipGetLastError();
    }
    const long n = (long)p.T * p.H;
    if (p.quant == Q_FP8_BLOCK) {
        const long groups = (long)p.T * (p.H / 128);
        hipExtLaunchKernelGGL(quant_block128_kernel<uint16_t>, dim3((unsigned)ceil_div((int)groups, 16)),
                              dim3(256), 0, st, nullptr, p.ev_stage_end, 0, p.x, p.T, p.H, p.xq, p.sx);
        return hipGetLastError();
    }
    const ElemRange all{nullptr, 0, 0};
    if (n <= kSmallQuant) {
        hipExtLaunchKernelGGL(quant_tensor_small_kernel<uint16_t>, dim3(1), dim3(1024), 0, st, nullptr,
                              p.ev_stage_end, 0, p.x, n, all, p.xq, &p.scal[0]);
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)std::min<long>(2048, (n / 8 + 255) / 256);
    hipLaunchKernelGGL(amax_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, p.x, n, all, &p.amax[0]);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipExtLaunchKernelGGL(quant_tensor_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, nullptr, p.ev_stage_end, 0,
                          p.x, n, all, &p.amax[0], p.xq, &p.scal[0]);
    return hipGetLastError();
}

// h (fp32 [R, I]) -> e4m3 codes: per-tensor with one scale over all routes,
// blockwise per row per 128 columns.
hipError_t launch_quant_h(const FwdPlan& p, hipStream_t st) {
    const long n = (long)p.R * p.I;
    const float* h = static_cast<const float*>(p.h);
    if (p.quant == Q_FP8_BLOCK) {
        const long groups = (long)p.R * (p.I / 128);
        hipExtLaunchKernelGGL(quant_block128_kernel<float>, dim3((unsigned)ceil_div((int)groups, 16)),
                              dim3(256), 0, st, nullptr, p.ev_stage_end, 0, h, p.R, p.I, p.hq, p.sh);
        return hipGetLastError();
    }
    // per-tensor: the scale covers the expert slice's routes, sorted rows
    // [offsets[e0], offsets[e0 + nloc]) (the only rows of h this call writes)
    const ElemRange local{p.offsets + p.e0, p.nloc, p.I};
    if (n <= kSmallQuant) {
        hipExtLaunchKernelGGL(quant_tensor_small_kernel<float>, dim3(1), dim3(1024), 0, st, nullptr,
                              p.ev_stage_end, 0, h, n, local, p.hq, &p.scal[1]);
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)std::min<long>(2048, (n / 8 + 255) / 256);
    hipLaunchKernelGGL(amax_kernel<float>, dim3(grid), dim3(256), 0, st, h, n, local, &p.amax[1]);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipExtLaunchKernelGGL(quant_tensor_kernel<float>, dim3(grid), dim3(256), 0, st, nullptr, p.ev_stage_end, 0,
                          h, n, local, &p.amax[1], p.hq, &p.scal[1]);
    return hipGetLastError();
}

// ------------------------------------------------------------------ combine --

// Expert slice: only routes whose sorted position lies in the slice's rows
// [rows[0], rows[nr]) were computed (the other rows of y are not written) and
// enter the sum; with accumulate the old output is added before the rounding.
__global__ void __launch_bounds__(256)
combine_kernel(const uint16_t* __restrict__ y, const float* __restrict__ tw, const int32_t* __restrict__ route_pos,
               int H, int k, const int32_t* __restrict__ rows, int nr, int accumulate, uint16_t* __restrict__ out) {
    const int t = blockIdx.x;
    const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (c >= H) return;
    const __attribute__((address_space(4))) int32_t* rw = (const __attribute__((address_space(4))) int32_t*)rows;
    const int lo = rw[0], hi = rw[nr];
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // eight slots at a time: their positions and gates (uniform, scalar loads),
    // then all eight y rows requested before the first one is used; slots past
    // k re-read slot k-1 and are not added.  The sum still runs in ascending j.
    const __attribute__((address_space(4))) int32_t* rp =
        (const __attribute__((address_space(4))) int32_t*)(route_pos + (size_t)t * k);
    const __attribute__((address_space(4))) float* wp =
        (const __attribute__((address_space(4))) float*)(tw + (size_t)t * k);
    for (int j0 = 0; j0 < k; j0 += 8) {
        int pos[8];
        float w[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int j = min(j0 + jj, k - 1);
            pos[jj] = rp[j];
            w[jj] = wp[j];
        }
        u32x4 raw[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) raw[jj] = *reinterpret_cast<const u32x4*>(y + (size_t)pos[jj] * H + c);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            if (j0 + jj < k && pos[jj] >= lo && pos[jj] < hi) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(w[jj], __uint_as_float(raw[jj][i] << 16), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(w[jj], __uint_as_float(raw[jj][i] & 0xffff0000u), acc[2 * i + 1]);
                }
            }
        }
    }
    u32x4* op = reinterpret_cast<u32x4*>(out + (size_t)t * H + c);
    if (accumulate) {
        const u32x4 old = *op;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += __uint_as_float(old[i] << 16);
            acc[2 * i + 1] += __uint_as_float(old[i] & 0xffff0000u);
        }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *op = o;
}

hipError_t launch_combine(const FwdPlan& p, hipStream_t st) {
    dim3 grid(p.T, ceil_div(p.H / 8, 256));
    hipExtLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, nullptr, p.ev_stage_end, 0, p.y, p.tw, p.route_pos,
                          p.H, p.k, p.offsets + p.e0, p.nloc, p.acc, p.out);
    return hipGetLastError();
}

}  // namespace moe
