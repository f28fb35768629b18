// One-time re-layout of the expert weights into the form the forward kernels
// stream: every matrix is stored with its reduction (K) dimension contiguous,
// so MFMA operands and GEMV lanes read 16-byte runs along K.
//
//  w_gate_up [E][H][2I]  ->  packed [E][2I][H]: packed row n' holds column
//     c(n') of the source, where each group of 32 packed rows interleaves 16
//     gate columns and the 16 up columns of the same h outputs:
//        n' = 32*g + s, s < 16  -> gate column 16*g + s
//                       s >= 16 -> up column   I + 16*g + (s - 16)
//     so a 16-column MFMA block is all gate or all up and the SwiGLU pairs
//     sit in the same lane of neighbouring accumulator tiles.
//  w_down    [E][I][H]   ->  packed [E][H][I] (plain transpose).
//
// The element is moved bit for bit (bf16 or e4m3); scales are not re-laid out.
#include "common.cuh"
#include "launch.h"

namespace moe {

template <typename T, bool GATE_UP>
__global__ void __launch_bounds__(256)
pack_kernel(const T* __restrict__ src, T* __restrict__ dst, int K, int N, int I) {
    // dst[e][n'][k] = src[e][k][col(n')]; one 64x64 (k, n') tile per workgroup
    __shared__ T tile[64][65];
    const int e = blockIdx.z;
    const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
    const T* s = src + (size_t)e * K * N;
    T* d = dst + (size_t)e * K * N;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int np = n0 + tx, k = k0 + i;
        if (np < N && k < K) {
            int col = np;
            if (GATE_UP) {
                const int g = np >> 5, sl = np & 31;
                col = sl < 16 ? 16 * g + sl : I + 16 * g + (sl - 16);
            }
            tile[i][tx] = s[(size_t)k * N + col];
        }
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int np = n0 + i, k = k0 + tx;
        if (np < N && k < K) d[(size_t)np * K + k] = tile[tx][i];
    }
}

template <typename T, bool GATE_UP>
static hipError_t launch_pack(const void* src, void* dst, int E, int K, int N, int I,
                              hipStream_t st) {
    dim3 grid(ceil_div(K, 64), ceil_div(N, 64), E);
    hipLaunchKernelGGL((pack_kernel<T, GATE_UP>), grid, dim3(256), 0, st,
                       static_cast<const T*>(src), static_cast<T*>(dst), K, N, I);
    return hipGetLastError();
}

hipError_t launch_pack_gate_up(const void* src, void* dst, int E, int H, int I, int elem_bytes,
                               hipStream_t st) {
    return elem_bytes == 2 ? launch_pack<uint16_t, true>(src, dst, E, H, 2 * I, I, st)
                           : launch_pack<uint8_t, true>(src, dst, E, H, 2 * I, I, st);
}

hipError_t launch_pack_down(const void* src, void* dst, int E, int H, int I, int elem_bytes,
                            hipStream_t st) {
    return elem_bytes == 2 ? launch_pack<uint16_t, false>(src, dst, E, I, H, I, st)
                           : launch_pack<uint8_t, false>(src, dst, E, I, H, I, st);
}

}  // namespace moe
