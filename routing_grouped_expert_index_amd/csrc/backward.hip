// Backward of the MoE FFN layer under the MX training recipe ("[mxfp8 moe
// training] add per group blocked scale kernels": Summary and its stacked pull
// requests -- the "dim1" cast in the backward, per-expert weight scales,
// per-group padded scale rows).  Every backward product runs on MX operands
// (e4m3 codes, one E8M0 scale per 32 values) quantised along that product's
// own reduction dimension:
//   input gradients   dh = dy W_down^T (along H), dx_r = dGU W_gate_up^T
//                     (along 2I): the grouped MX GEMM of the forward, on
//                     weights packed transposed;
//   weight gradients  dW_down[e] = h_e^T dy_e, dW_gate_up[e] = x_e^T dGU_e:
//                     both operands quantised along the expert's routes (the
//                     "dim1" cast), each expert's route segment padded to 64
//                     with zeros at offsets built on device, and multiplied
//                     by wgrad_kernel.
// The quantisers pass gradients through unchanged (straight-through).
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.cuh"
#include "launch.h"
#include "layout.cuh"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));
#define MOE_LDS_B(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ uint8_t e4m3_byte(float v) { return (uint8_t)(f32x2_to_e4m3x2(v, 0.0f) & 0xffu); }

// ------------------------------------------------------------- weights --

// bf16 master weights -> an MX operand set in the packed layout the grouped
// MX GEMM reads (layout.cuh, MX chunk order; plain column order, or with
// GATE_UP the forward's gate/up interleave of N = 2I columns), one scale per
// 32 consecutive k of each output column n, in one pass:
//   along_k = 1: src [E][K][N] (the groups run down the source's rows);
//   along_k = 0: src [E][N][K] (the groups run along the source's rows: the
//                transposed use of a weight).
// One thread per (expert, 32-group, column), columns fastest.  The group's 32
// codes are two 16-byte pieces: K values 32kb + [0, 16) and + [16, 32) are
// lane halves 0 and 1, half q = kb % 2, of slice kb / 2 of the column's packed
// row; its E8M0 byte goes to the packed scale dword of that row and K group.
template <bool ALONG_K, bool GATE_UP>
__global__ void __launch_bounds__(256)
mx_pack_weights_kernel(const uint16_t* __restrict__ src, int E, int K, int N, uint8_t* __restrict__ packed,
                       uint8_t* __restrict__ packed_s, uint8_t* __restrict__ plain, uint8_t* __restrict__ plain_s) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    const int nkb = K / 32;
    if (g >= (long)E * nkb * N) return;
    const int n = (int)(g % N);
    const int kb = (int)((g / N) % nkb);
    const long e = g / N / nkb;
    float v[32];
    if constexpr (ALONG_K) {   // down a column: each load is 64 lanes' adjacent columns
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) v[jj] = bf16_to_f32(src[(e * K + 32 * kb + jj) * N + n]);
    } else {                   // along a row: the group's 64 bytes as four 16-byte loads
        const u32x4* p4 = reinterpret_cast<const u32x4*>(src + (e * N + n) * K + 32 * kb);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4 w4 = p4[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * t + 2 * i] = __uint_as_float(w4[i] << 16);
                v[8 * t + 2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
            }
        }
    }
    float a = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) a = fmaxf(a, fabsf(v[jj]));
    const uint32_t b = mx_byte(a);
    const float inv = mx_inv(b);
    u32x4 lo, hi;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        lo[t] = f32x4_to_e4m3x4(v[4 * t] * inv, v[4 * t + 1] * inv, v[4 * t + 2] * inv, v[4 * t + 3] * inv);
        hi[t] = f32x4_to_e4m3x4(v[16 + 4 * t] * inv, v[16 + 4 * t + 1] * inv, v[16 + 4 * t + 2] * inv,
                                v[16 + 4 * t + 3] * inv);
    }
    // the group's pieces and byte at packed row P of a set
    auto put = [&](uint8_t* dst, uint8_t* dst_s, int P) __attribute__((always_inline)) {
        const int g32 = P >> 5, j = P & 31, nsl = K / 64;
        uint8_t* blk = dst + e * (long)N * K + (((long)g32 * nsl + (kb >> 1)) * 2 + (kb & 1)) * 1024;
        *reinterpret_cast<u32x4*>(blk + j * 16) = lo;
        *reinterpret_cast<u32x4*>(blk + (32 + j) * 16) = hi;
        const long dw = (((e * (N / 32) + g32) * (K / 256) + kb / 8) * 64 + 32 * (kb & 1) + j);
        dst_s[dw * 4 + ((kb & 7) >> 1)] = (uint8_t)b;
    };
    put(packed, packed_s,
        GATE_UP ? (n < N / 2 ? packed_gate_row(n) : packed_up_row(n - N / 2)) : packed_down_row(n));
    // GATE_UP may also write the same codes in plain column order (the second
    // set quantised along the same K)
    if (GATE_UP && plain) put(plain, plain_s, packed_down_row(n));
}

hipError_t launch_mx_pack_weights(const uint16_t* src, int E, int K, int N, bool along_k, bool gate_up,
                                  uint8_t* packed, uint8_t* packed_s, uint8_t* plain, uint8_t* plain_s,
                                  hipStream_t st) {
    const long groups = (long)E * (K / 32) * N;
    const dim3 grid((unsigned)((groups + 255) / 256));
    if ((gate_up && !along_k) || (plain && !gate_up)) return hipErrorInvalidValue;
    if (gate_up)
        hipLaunchKernelGGL((mx_pack_weights_kernel<true, true>), grid, dim3(256), 0, st, src, E, K, N, packed,
                           packed_s, plain, plain_s);
    else if (along_k)
        hipLaunchKernelGGL((mx_pack_weights_kernel<true, false>), grid, dim3(256), 0, st, src, E, K, N, packed,
                           packed_s, plain, plain_s);
    else
        hipLaunchKernelGGL((mx_pack_weights_kernel<false, false>), grid, dim3(256), 0, st, src, E, K, N, packed,
                           packed_s, plain, plain_s);
    return hipGetLastError();
}

// ------------------------------------------------- row-wise MX of routes --

// Four threads quantise one group of 32 values of a row (8 each): returns the
// group's E8M0 byte; codes written as 8 bytes at q.
__device__ __forceinline__ uint32_t mx_quad(const float v[8], uint8_t* q) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    const uint32_t b = mx_byte(a);
    const float inv = mx_inv(b);
    uint2 w;
    w.x = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    w.y = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<uint2*>(q) = w;
    return b;
}

__device__ __forceinline__ void load8_bf16(const uint16_t* p, float v[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ void load8_f32(const float* p, float v[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = a[i];
        v[4 + i] = b[i];
    }
}

__device__ __forceinline__ void store8_f32(float* p, const float v[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Forward recomputation: g|u (fp32 [R][2I], sorted routes) -> h = silu(g) u
// (fp32 [R][I], kept for the weight gradient) and its MX rows (codes [R][I],
// bytes [R][I/32] in the MX GEMM's scale order) for the Down product.
__global__ void __launch_bounds__(256)
swiglu_fwd_kernel(const float* __restrict__ gu, long R, int I, float* __restrict__ h32, uint8_t* __restrict__ hq,
                  uint8_t* __restrict__ sh) {
    const int gpr = I / 32;
    const long grp = (long)blockIdx.x * 64 + threadIdx.x / 4;
    if (grp >= R * gpr) return;   // (whole quads: 64 groups per workgroup)
    const int sub = threadIdx.x & 3;
    const long row = grp / gpr;
    const int c = (int)(grp % gpr) * 32 + sub * 8;
    float g[8], u[8], h[8];
    load8_f32(gu + row * 2 * I + c, g);
    load8_f32(gu + row * 2 * I + I + c, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = silu(g[i]) * u[i];
    store8_f32(h32 + row * I + c, h);
    const uint32_t b = mx_quad(h, hq + row * I + c);
    if (sub == 0) sh[row * gpr + mx_scale_pos((int)(grp % gpr))] = (uint8_t)b;
}

// One workgroup per sorted route i (route r = perm[i] of token t = r / k, gate
// w = tw[r]): dy = w * dout[t] in fp32, its MX rows (codes [R][H], bytes
// [R][H/32]) for dh = dy W_down^T, and the gate's gradient <dout[t], y_i>
// (y: the recomputed Down output, bf16 [R][H] sorted: it enters only this
// dot product, where its rounding averages out) written to dgate[r].
// The sum runs per thread over its columns in order, then over the wave and
// the four waves in a fixed order.
__global__ void __launch_bounds__(256)
dy_kernel(const uint16_t* __restrict__ dout, const float* __restrict__ tw, const int32_t* __restrict__ perm, int k,
          const uint16_t* __restrict__ y, int H, uint8_t* __restrict__ dyq, uint8_t* __restrict__ sdy,
          float* __restrict__ dgate) {
    __shared__ float part[4];
    const long i = blockIdx.x;
    const int r = perm[i];
    const int t = r / k;
    const float w = tw[r];
    const int gpr = H / 32;
    float dsum = 0.0f;
    for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
        float d[8], yy[8], v[8];
        load8_bf16(dout + (long)t * H + c, d);
        load8_bf16(y + i * H + c, yy);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[j] = w * d[j];
            dsum = fmaf(d[j], yy[j], dsum);
        }
        const uint32_t b = mx_quad(v, dyq + i * H + c);
        if ((threadIdx.x & 3) == 0) sdy[i * gpr + mx_scale_pos(c / 32)] = (uint8_t)b;
    }
    dsum = wave_sum(dsum);
    if (lane_id() == 0) part[threadIdx.x / kWave] = dsum;
    __syncthreads();
    if (threadIdx.x == 0) dgate[r] = ((part[0] + part[1]) + part[2]) + part[3];
}

// SwiGLU backward per sorted route (g|u and dh fp32): dgate = dh u s (1 + g (1 - s)), dup = dh
// g s (s = sigmoid(g)), kept as fp32 [R][2I] for the weight gradient, and its
// MX rows (codes [R][2I], bytes [R][2I/32]) for dx_r = dGU W_gate_up^T.
__global__ void __launch_bounds__(256)
swiglu_bwd_kernel(const float* __restrict__ gu, const float* __restrict__ dh, long R, int I,
                  float* __restrict__ dgu, uint8_t* __restrict__ dguq, uint8_t* __restrict__ sdgu) {
    const int gpr = I / 32, gpr2 = 2 * gpr;
    const long grp = (long)blockIdx.x * 64 + threadIdx.x / 4;
    if (grp >= R * gpr) return;
    const int sub = threadIdx.x & 3;
    const long row = grp / gpr;
    const int cg = (int)(grp % gpr);
    const int c = cg * 32 + sub * 8;
    float g[8], u[8], d[8], dg[8], du[8];
    load8_f32(gu + row * 2 * I + c, g);
    load8_f32(gu + row * 2 * I + I + c, u);
    load8_f32(dh + row * I + c, d);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float s = 1.0f / (1.0f + __expf(-g[j]));
        dg[j] = d[j] * u[j] * s * (1.0f + g[j] * (1.0f - s));
        du[j] = d[j] * g[j] * s;
    }
    float* o = dgu + row * 2 * I;
    store8_f32(o + c, dg);
    store8_f32(o + I + c, du);
    const uint32_t bg = mx_quad(dg, dguq + row * 2 * I + c);
    const uint32_t bu = mx_quad(du, dguq + row * 2 * I + I + c);
    if (sub == 0) {
        sdgu[row * gpr2 + mx_scale_pos(cg)] = (uint8_t)bg;
        sdgu[row * gpr2 + mx_scale_pos(gpr + cg)] = (uint8_t)bu;
    }
}

// ------------------------------------------------- per-expert route segments --

// poff[e] = sum over e' < e of the expert's route count rounded up to 64 (the
// weight-gradient product's K step), poff[E] the padded total: the per-group
// padded start offsets, built on the device from the routing's offsets; and
// seg[s] = the expert whose padded segment holds 64-position slice s (for
// every s below nseg; slices past poff[E] get E).
__global__ void __launch_bounds__(256)
pad_offsets_kernel(const int32_t* __restrict__ offsets, int E, int32_t* __restrict__ poff, int32_t* __restrict__ seg,
                   int nseg) {
    __shared__ int sp[kMaxExperts + 1];
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int e = 0; e < E; ++e) {
            sp[e] = acc;
            poff[e] = acc;
            acc += (offsets[e + 1] - offsets[e] + 63) & ~63;
        }
        sp[E] = acc;
        poff[E] = acc;
    }
    __syncthreads();
    for (int s = threadIdx.x; s < nseg; s += 256) {
        const int p = 64 * s;
        int lo = 0, hi = E;                    // sp[lo] <= p < sp[hi]
        if (p >= sp[E]) {
            lo = E;
        } else {
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (sp[mid] <= p) lo = mid;
                else hi = mid;
            }
        }
        seg[s] = lo;
    }
}

// The "dim1" cast: an operand v[i][m] over sorted routes i (M columns),
// quantised along the routes of each expert, 32 per E8M0 scale, and written
// transposed: row m of the output holds the padded route positions p (expert
// e's routes at poff[e] + (i - offsets[e]), zeros up to poff[e+1]) as e4m3
// codes, each 64-position slice in chunk order 0, 2, 1, 3 (the scaled MFMA's
// lane-half order: lane half hh reads bytes [32hh, 32hh + 32) of a slice),
// stored slice-major: slice s of row m at bytes 64 (s M + m), so that the 128
// rows of a product tile hold one slice in 8 KB in a row (read in 128-byte
// lines where row-major rows gave a 64-byte request a row and slice), and
// the scale bytes in groups of 8 route blocks (256 positions): group q of row m
// at bytes 8 (q M + m), route block b's byte at mx_scale_pos(b) % 8 of its
// group, so that the 128 rows of a product tile hold one group's scales in 1 KB
// in a row (the weight-gradient kernel reads them in 64-byte pieces, where with
// each row's bytes together every 8-byte read was a request of its own).
// One workgroup per 128 padded positions (two slices) and 64 columns, a
// transpose through LDS in three steps:
//   1. the tile's 128 route rows of 64 source columns come in by 16-byte
//      loads (eight lanes a 128-byte bf16 row segment, sixteen a 256-byte
//      fp32 one) and go into LDS as loaded (dy's gates beside them), zero
//      for padding positions;
//   2. wave q quantises block q of 32 positions, lane l column l, reading its
//      32 values down the LDS tile (to fp32, times the gate for dy): the
//      amax, the E8M0 byte (stored), and 32
//      e4m3 codes written to an LDS tile of the output's 64 rows x 128 bytes;
//   3. eight lanes write each output row's 128-byte line.
// Against one lane per column reading its 32 routes straight from memory (two
// bytes a lane for bf16) and writing its 32 codes as two 16-byte pieces into
// a different row from every lane, this cuts the write requests to the L2
// about fourfold.
enum Dim1Src { D1_X = 0, D1_DY = 1, D1_F32 = 2 };
constexpr int kD1CodeStride = 144;   // bytes an output row in LDS (128 + 16: writes by 8 lanes hit distinct banks)

template <int SRC>
__global__ void __launch_bounds__(256)
dim1_kernel(const void* __restrict__ src, const uint16_t* __restrict__ dout, const float* __restrict__ tw,
            const int32_t* __restrict__ perm, uint32_t kdiv_m, int kdiv_s, const int32_t* __restrict__ offsets,
            const int32_t* __restrict__ poff, const int32_t* __restrict__ seg, int E, int M, long ldo,
            uint8_t* __restrict__ out, uint8_t* __restrict__ sout) {
    // [route position][column]: fp32 for fp32 sources, the bf16 values as
    // loaded for x and dout (16 KB: eight workgroups a CU instead of five),
    // with dy's gates beside them
    constexpr bool F32 = SRC == D1_F32;
    __shared__ __attribute__((aligned(16))) float tile[F32 ? 128 * 64 : 128 * 32];
    __shared__ float gate[SRC == D1_DY ? 128 : 1];
    // (a route's token r / k as a multiply-shift)
    auto tok = [&](int r) { return (long)(((uint64_t)(uint32_t)r * kdiv_m) >> kdiv_s); };
    const int x = blockIdx.x, m0 = blockIdx.y * 64;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    // the two 64-position slices: expert, sorted row of the slice's first
    // position, real routes in the slice (may be <= 0)
    int first[2], cnt[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = seg[2 * x + h];
        if (e < E) {
            first[h] = offsets[e] + (64 * (2 * x + h) - poff[e]);
            cnt[h] = min(64, offsets[e + 1] - first[h]);
        } else {
            first[h] = 0;
            cnt[h] = 0;
        }
    }
    // 1. source rows into LDS; a padding position loads a real row of the
    // tile (every load unconditional: a load under a per-route condition
    // would become a branch that waits for every load before it) and stores
    // 0 (a select, not a multiply by 0: the re-read row may hold an infinity)
    const bool any = cnt[0] > 0 || cnt[1] > 0;
    const int anyrow = cnt[0] > 0 ? first[0] : first[1];
    auto row_of = [&](int r, bool& ok) __attribute__((always_inline)) {
        const int h = r >> 6, j = r & 63;
        ok = j < cnt[h];
        return ok ? first[h] + j : anyrow;
    };
    if (any) {
        if constexpr (F32) {
            const int c = t & 15;   // 4 columns
            float4 v[8];
            bool ok[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = row_of((t >> 4) + 16 * i, ok[i]);
                v[i] = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + (long)row * M + m0 + 4 * c);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 z = ok[i] ? v[i] : float4{0.0f, 0.0f, 0.0f, 0.0f};
                *reinterpret_cast<float4*>(tile + ((t >> 4) + 16 * i) * 64 + 4 * c) = z;
            }
        } else {
            const int c = t & 7;   // 8 columns
            u32x4 v[4];
            float g[4];
            bool ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row_of((t >> 3) + 32 * i, ok[i]);
                const int r = perm[row];
                const uint16_t* base = SRC == D1_X ? static_cast<const uint16_t*>(src) : dout;
                v[i] = *reinterpret_cast<const u32x4*>(base + tok(r) * M + m0 + 8 * c);
                g[i] = SRC == D1_DY ? tw[r] : 1.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = (t >> 3) + 32 * i;
                *reinterpret_cast<u32x4*>(tile + rr * 32 + 4 * c) = ok[i] ? v[i] : u32x4{0u, 0u, 0u, 0u};
                if constexpr (SRC == D1_DY)
                    if (c == 0) gate[rr] = ok[i] ? g[i] : 0.0f;
            }
        }
    } else {
        for (int i = t; i < (F32 ? 128 * 64 : 128 * 32) / 4; i += 256)
            reinterpret_cast<float4*>(tile)[i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (SRC == D1_DY)
            if (t < 128) gate[t] = 0.0f;
    }
    __syncthreads();
    // 2. block q = wave of 32 positions, column lane
    float v[32];
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const int rr = 32 * wave + j;
        if constexpr (F32) {
            v[j] = tile[rr * 64 + lane];
        } else {
            v[j] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(tile)[rr * 64 + lane] << 16);
            if constexpr (SRC == D1_DY) v[j] = gate[rr] * v[j];
        }
        a = fmaxf(a, fabsf(v[j]));
    }
    const uint32_t b = mx_byte(a);
    const float inv = mx_inv(b);
    u32x4 lo4, hi4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        lo4[u] = f32x4_to_e4m3x4(v[4 * u] * inv, v[4 * u + 1] * inv, v[4 * u + 2] * inv, v[4 * u + 3] * inv);
        hi4[u] = f32x4_to_e4m3x4(v[16 + 4 * u] * inv, v[16 + 4 * u + 1] * inv, v[16 + 4 * u + 2] * inv,
                                 v[16 + 4 * u + 3] * inv);
    }
    const int gi = 4 * x + wave;   // block of 32 padded positions
    sout[((long)(gi >> 3) * M + m0 + lane) * 8 + (mx_scale_pos(gi) & 7)] = (uint8_t)b;
    __syncthreads();   // every wave is done reading the source tile
    // block gi of its 64-position slice: even -> chunks 0, 1 at bytes 0, 32;
    // odd -> chunks 2, 3 at bytes 16, 48
    uint8_t* ct = reinterpret_cast<uint8_t*>(tile);
    uint8_t* cr = ct + lane * kD1CodeStride + 64 * (wave >> 1) + 16 * (wave & 1);
    *reinterpret_cast<u32x4*>(cr) = lo4;
    *reinterpret_cast<u32x4*>(cr + 32) = hi4;
    __syncthreads();
    // 3. slice 2x + h of rows m0 .. m0 + 63: 4 KB in a row, 16 bytes a lane
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rr = t >> 2, c = t & 3;
        const u32x4 w = *reinterpret_cast<const u32x4*>(ct + rr * kD1CodeStride + 64 * h + 16 * c);
        *reinterpret_cast<u32x4*>(out + ((long)(2 * x + h) * M + m0 + rr) * 64 + 16 * c) = w;
    }
}

// ------------------------------------------------------- weight gradients --

// C[e] (bf16 [M][N], the master weights' type) = sum over expert e's padded
// route positions p of
// A[m][p] B[n][p], with A, B the dim1-cast operands (codes slice-major, 64
// bytes of a row per 64-position slice, ldo bytes a row in all;
// scales in groups of 8 route blocks, a group holding 8 bytes for each of the
// M (N) rows, lds_ bytes a row in all).  One workgroup per 128x128 output
// tile.  The tile's 128 rows of A and of B come into LDS by buffer loads with
// the LDS bit, one 64-position slice (16 KB) at a time into two alternating
// buffers, and their E8M0 scale dwords once per group of four slices (2 KB)
// into two alternating scale areas: slice s + 1's loads are issued before the
// wait for slice s, so each wait covers one slice's latency less (the
// expert's K is short, 4-5 slices, and the tile is bound by latency, its
// output stores and the number of requests the L2 serves, not by its
// products: with each row's scale bytes 8 bytes apart from the next row's,
// the 8-byte scale reads were half of the kernel's L2 requests, and storing
// them group-major took dW_gate_up from 452 to 388 us and dW_down from 234
// to 182 us at the MX prefill shape).  What counts beside that is how many workgroups share
// a CU: 36 KB of LDS and 128 registers a lane keep four per SIMD (staging
// two or four slices per round in one buffer measured 5% and 23% slower than
// one; the two buffers against one: dW_gate_up 507 -> 459 us, dW_down 270 ->
// 237 us, same bits).  Row r's 16-byte chunk c sits at physical chunk
// c ^ ((r / 4) % 4).  Wave w then takes rows 64 (w / 2) and columns
// 64 (w % 2) of the tile as 2x2 blocks of the scaled 32x32x64 MFMA, B's rows
// as the first operand so that a lane holds 4 consecutive columns of C per
// result group; a wave's two 32x32 blocks of one row block go through LDS as
// bf16 so that each non-temporal store instruction writes whole 128-byte
// lines of C (C is written once and not read back here; against 16-byte fp32
// stores straight from the result registers: dW_gate_up 750 -> 694 us,
// dW_down 419 -> 353 us, and bf16 instead of fp32 output 700 -> 520 us and
// 357 -> 274 us).  An expert without routes gets zeros.  (C is row-major with
// N a multiple of 128.)
constexpr int kWgBuf = 2 * 128 * 64 + 2 * 128 * 8;   // 18 KB: A and B rows of a slice, then their scale dwords
constexpr int kWgOperandLds = 2 * kWgBuf;             // two buffers
constexpr int kWgStageLds = 4 * 32 * 72 * 2;          // 18 KB: each wave's 32 rows of 72 bf16
constexpr int kWgLds = kWgOperandLds > kWgStageLds ? kWgOperandLds : kWgStageLds;

__global__ void __launch_bounds__(256)
wgrad_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ B,
             const uint8_t* __restrict__ sB, long ldo, long lds_, const int32_t* __restrict__ poff, int E, int M,
             int N, uint16_t* __restrict__ C) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tm = M / 128, tn = N / 128;
    const long total = (long)E * tm * tn;
    long tile = blockIdx.x;
    // consecutive tiles (one expert's, sharing operand rows) on one XCD:
    // workgroup b runs on XCD b % 8
    if (total % 8 == 0) tile = (long)(blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
    const int e = (int)(tile / ((long)tm * tn));
    const int rem = (int)(tile % ((long)tm * tn));
    const int mt = rem / tn, nt = rem % tn;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 31, hh = lane >> 5;
    const int s0 = poff[e] / 64, s1 = poff[e + 1] / 64;
    f32x16 acc[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[f][g][i] = 0.0f;
    // the tile's rows of A and B as buffer resources (128 rows each)
    // (slice-major operands: slice s of row r at bytes 64 (s M + r); the
    // resources start at the tile's first row of slice 0)
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A) + (long)mt * 128 * 64, 0, (int)((long)M * ldo - (long)mt * 128 * 64), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B) + (long)nt * 128 * 64, 0, (int)((long)N * ldo - (long)nt * 128 * 64), 0x00020000);
    // this lane's DMA row (two 16-row groups per wave and slice) and the
    // logical chunk its physical chunk holds
    const int dr0 = 32 * wave + (lane >> 2), dr1 = dr0 + 16;
    const uint32_t dof0 = (uint32_t)(dr0 * 64) + 16u * (uint32_t)((lane & 3) ^ ((dr0 >> 2) & 3));
    const uint32_t dof1 = (uint32_t)(dr1 * 64) + 16u * (uint32_t)((lane & 3) ^ ((dr1 >> 2) & 3));
    // fragment rows of this lane: A rows ra0 + 32f, B rows rb0 + 32g
    const int ra0 = (wave >> 1) * 64 + j, rb0 = (wave & 1) * 64 + j;
    auto frag = [&](const uint8_t* base, int r) __attribute__((always_inline)) {
        const int sw = (r >> 2) & 3;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + r * 64 + 16 * ((2 * hh) ^ sw));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + r * 64 + 16 * ((2 * hh + 1) ^ sw));
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // two LDS buffers of one slice each (A rows, B rows, then their scale
    // dwords): slice s + 1's DMA goes out before the wait for slice s.  The
    // loop's barriers are bare s_barrier between compiler memory fences:
    // __syncthreads' release fence would wait for every load into LDS still
    // in flight, slice s + 1's included; the explicit vmcnt waits order the
    // loads against the reads instead.
    // the scale arrays: groups of 8 route blocks, each group M (N) rows of 8
    // bytes; this lane's 4 bytes of the wave's 32 rows (row 32 wave + lane / 2,
    // lane half lane % 2) in group 0
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sA), 0,
                                                                         (int)(M * lds_), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sB), 0,
                                                                         (int)(N * lds_), 0x00020000);
    const uint32_t sofa = (uint32_t)((mt * 128 + 32 * wave) * 8 + 4 * lane);
    const uint32_t sofb = (uint32_t)((nt * 128 + 32 * wave) * 8 + 4 * lane);
    auto issue = [&](int s, int buf) __attribute__((always_inline)) {
        const uint32_t soa = (uint32_t)s * (uint32_t)M * 64u, sob = (uint32_t)s * (uint32_t)N * 64u;
        uint8_t* lb = smem + buf * kWgBuf;
        uint8_t* la = lb + wave * 2048;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MOE_LDS_B(la), 16, dof0 + soa, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MOE_LDS_B(la + 1024), 16, dof1 + soa, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, MOE_LDS_B(la + 8192), 16, dof0 + sob, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, MOE_LDS_B(la + 8192 + 1024), 16, dof1 + sob, 0, 0, 0);
        if (s == s0 || (s & 3) == 0) {
            // the scales of slice s's group of 4 slices, once per group, into
            // the scale area of buffer (group % 2)
            const uint32_t q = (uint32_t)(s >> 2);
            uint8_t* lq = smem + (q & 1) * kWgBuf;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, MOE_LDS_B(lq + 16384 + wave * 256), 4,
                                                     sofa + q * (uint32_t)M * 8u, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, MOE_LDS_B(lq + 17408 + wave * 256), 4,
                                                     sofb + q * (uint32_t)N * 8u, 0, 0, 0);
        }
    };
    if (s0 < s1) issue(s0, 0);
    for (int s = s0; s < s1; ++s) {
        const int buf = (s - s0) & 1;
        __asm__ volatile("" ::: "memory");
        if (s + 1 < s1) {
            __builtin_amdgcn_s_barrier();          // every wave is done reading the other buffer
            __asm__ volatile("" ::: "memory");
            issue(s + 1, buf ^ 1);
            if (((s + 1) & 3) == 0)
                __builtin_amdgcn_s_waitcnt(0x0F76);    // vmcnt(6): slice s has landed (s + 1's 6 requests may not)
            else
                __builtin_amdgcn_s_waitcnt(0x0F74);    // vmcnt(4): the same, s + 1 without scales
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0)
        }
        __builtin_amdgcn_s_barrier();              // ... for every wave
        __asm__ volatile("" ::: "memory");
        const int sh = 8 * (s & 3);   // byte (slice % 4) of the scale dword: this lane half's block
        const uint8_t* la = smem + buf * kWgBuf;
        const uint32_t* ls = reinterpret_cast<const uint32_t*>(smem + ((s >> 2) & 1) * kWgBuf + 16384);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const i32x8 av = frag(la, ra0 + 32 * f);
            const uint32_t sa = ls[(ra0 + 32 * f) * 2 + hh];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const i32x8 bv = frag(la + 8192, rb0 + 32 * g);
                const uint32_t sb = ls[256 + (rb0 + 32 * g) * 2 + hh];
                acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bv, av, acc[f][g], 0, 0, 0, (int)((sb >> sh) & 0xffu), 0, (int)((sa >> sh) & 0xffu));
            }
        }
    }
    __syncthreads();   // every wave is done reading the operand slices
    uint16_t* ws = reinterpret_cast<uint16_t*>(smem) + wave * (32 * 72);
    uint16_t* ce = C + (long)e * M * N;
    const int n0 = nt * 128 + (wave & 1) * 64;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2*>(ws + j * 72 + 32 * g + 8 * q + 4 * hh) =
                    uint2{pack_bf16x2(acc[f][g][4 * q], acc[f][g][4 * q + 1]),
                          pack_bf16x2(acc[f][g][4 * q + 2], acc[f][g][4 * q + 3])};
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int rr = 8 * p + (lane >> 3), cc = 8 * (lane & 7);
            const u32x4 v = *reinterpret_cast<const u32x4*>(ws + rr * 72 + cc);
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>(ce + (long)(mt * 128 + (wave >> 1) * 64 + 32 * f + rr) * N + n0 + cc));
        }
        __asm__ volatile("" ::: "memory");
    }
}

// The gates' gradient taken to the router logits: the gates are the softmax
// over the k picked logits (the softmax over all E renormalised over the
// picks), and the picks are piecewise constant, so row t of dlogits is zero
// except dl[ids[t][j]] = w_j (g_j - sum_i w_i g_i) (the sum in ascending j).
// One workgroup per token; the picks of a token are distinct experts.
__global__ void __launch_bounds__(256)
route_grad_kernel(const int32_t* __restrict__ ids, const float* __restrict__ tw, const float* __restrict__ dgate,
                  int E, int k, float* __restrict__ dlogits) {
    const long t = blockIdx.x;
    float* row = dlogits + t * E;
    for (int c = threadIdx.x; c < E; c += 256) row[c] = 0.0f;
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s = fmaf(tw[t * k + j], dgate[t * k + j], s);
    __syncthreads();   // (the zeros are written before the picks overwrite theirs)
    for (int j = threadIdx.x; j < k; j += 256) {
        const long r = t * k + j;
        row[ids[r]] = tw[r] * (dgate[r] - s);
    }
}

hipError_t launch_route_grad(const int32_t* ids, const float* tw, const float* dgate, int T, int E, int k,
                             float* dlogits, hipStream_t st) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(route_grad_kernel, dim3((unsigned)T), dim3(256), 0, st, ids, tw, dgate, E, k, dlogits);
    return hipGetLastError();
}

// a fill kernel (no memset node where a caller captures the sequence)
__global__ void __launch_bounds__(256) fill_f32_kernel(float* __restrict__ p, long n, float v) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = v;
}

// ------------------------------------------------------------- launchers --

hipError_t launch_fill_f32(float* p, long n, float v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<long>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(fill_f32_kernel, dim3(grid), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const float* gu, long R, int I, float* h32, uint8_t* hq, uint8_t* sh,
                             hipEvent_t ev_end, hipStream_t st) {
    const long groups = R * (I / 32);
    if (groups == 0) return hipSuccess;
    hipExtLaunchKernelGGL(swiglu_fwd_kernel, dim3((unsigned)((groups + 63) / 64)), dim3(256), 0, st, nullptr, ev_end,
                          0, gu, R, I, h32, hq, sh);
    return hipGetLastError();
}

hipError_t launch_dy(const uint16_t* dout, const float* tw, const int32_t* perm, int k, const uint16_t* y, long R,
                     int H, uint8_t* dyq, uint8_t* sdy, float* dgate, hipEvent_t ev_end, hipStream_t st) {
    if (R == 0) return hipSuccess;
    hipExtLaunchKernelGGL(dy_kernel, dim3((unsigned)R), dim3(256), 0, st, nullptr, ev_end, 0, dout, tw, perm, k, y,
                          H, dyq, sdy, dgate);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* gu, const float* dh, long R, int I, float* dgu, uint8_t* dguq,
                             uint8_t* sdgu, hipEvent_t ev_end, hipStream_t st) {
    const long groups = R * (I / 32);
    if (groups == 0) return hipSuccess;
    hipExtLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((groups + 63) / 64)), dim3(256), 0, st, nullptr, ev_end,
                          0, gu, dh, R, I, dgu, dguq, sdgu);
    return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, int32_t* seg, int nseg, hipStream_t st) {
    hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(256), 0, st, offsets, E, poff, seg, nseg);
    return hipGetLastError();
}

hipError_t launch_dim1(int src_kind, const void* src, const uint16_t* dout, const float* tw, const int32_t* perm,
                       int k, const int32_t* offsets, const int32_t* poff, const int32_t* seg, int E, int M, long Rp,
                       long ldo, long lds_, uint8_t* out, uint8_t* sout, hipEvent_t ev_end, hipStream_t st) {
    if (M % 64 != 0 || Rp % 128 != 0 || ldo != Rp || lds_ * 32 != Rp) return hipErrorInvalidValue;   // whole tiles
    const dim3 grid((unsigned)(Rp / 128), (unsigned)(M / 64));
    if (Rp == 0) return hipSuccess;
    // r / k == (r * m) >> s for every r < 2^31 and 1 <= k <= 2^10, with
    // s = 31 + ceil(log2 k) and m = ceil(2^s / k) < 2^32
    int l = 0;
    while ((1 << l) < k) ++l;
    const int kdiv_s = 31 + l;
    const uint32_t kdiv_m = (uint32_t)(((1ULL << kdiv_s) + (uint64_t)k - 1) / (uint64_t)k);
    if (src_kind == D1_X)
        hipExtLaunchKernelGGL(dim1_kernel<D1_X>, grid, dim3(256), 0, st, nullptr, ev_end, 0, src, dout, tw, perm, kdiv_m, kdiv_s,
                              offsets, poff, seg, E, M, ldo, out, sout);
    else if (src_kind == D1_DY)
        hipExtLaunchKernelGGL(dim1_kernel<D1_DY>, grid, dim3(256), 0, st, nullptr, ev_end, 0, src, dout, tw, perm, kdiv_m, kdiv_s,
                              offsets, poff, seg, E, M, ldo, out, sout);
    else
        hipExtLaunchKernelGGL(dim1_kernel<D1_F32>, grid, dim3(256), 0, st, nullptr, ev_end, 0, src, dout, tw, perm,
                              kdiv_m, kdiv_s, offsets, poff, seg, E, M, ldo, out, sout);
    return hipGetLastError();
}

hipError_t launch_wgrad(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, long ldo, long lds_,
                        const int32_t* poff, int E, int M, int N, uint16_t* C, hipEvent_t ev_end, hipStream_t st) {
    const long total = (long)E * (M / 128) * (N / 128);
    // 32-bit offsets within the operand and scale arrays (codes: ldo bytes a
    // row, slice-major; scales: ldo / 32 bytes a row)
    if ((long)std::max(M, N) * ldo > 0x7fffffffL || lds_ * 32 != ldo || ldo % 64 != 0) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(wgrad_kernel, dim3((unsigned)total), dim3(256), kWgLds, st, nullptr, ev_end, 0, A, sA, B,
                          sB, ldo, lds_, poff, E, M, N, C);
    return hipGetLastError();
}

}  // namespace moe
