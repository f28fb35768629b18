// One-time re-layout of the expert weights into the packed form every forward
// kernel reads (layout.cuh): per expert, K-sliced 2 KB blocks of 32 output
// columns in MFMA operand-lane order, with the output columns permuted inside
// groups of 64 so that each MFMA result lane holds contiguous outputs.
//
//  w_gate_up [E][H][2I] -> packed gate/up matrix (N = 2I, K = H)
//  w_down    [E][I][H]  -> packed down matrix    (N = H,  K = I)
//
// Elements move bit for bit (bf16 or e4m3); scales keep the caller's layout.
#include "common.cuh"
#include "launch.h"
#include "layout.cuh"

namespace moe {

constexpr int kPackSlicesPerWG = 8;

// one workgroup: expert e, one 64-row permutation group, up to 8 K slices.
// MX codes take the chunk order of the scaled MFMA: half q of lane half hh is
// slice chunk hh + 2q (else 2hh + q), so lane half hh holds the slice's MX
// block hh whole.
template <typename T, bool GATE_UP, bool MXO>
__global__ void __launch_bounds__(256)
pack_kernel(const T* __restrict__ src, uint8_t* __restrict__ dst, int K, int N, int I) {
    constexpr int elem = sizeof(T);
    constexpr int KS = kSliceBytes / elem;          // K values per slice
    __shared__ T tile[KS][kGroupRows + 1];
    const int e = blockIdx.x, G = blockIdx.y;
    const int Kb = K * elem, NSL = Kb / kSliceBytes;
    const T* s = src + (size_t)e * K * N;
    uint8_t* d = dst + (size_t)e * N * Kb;
    const int tid = threadIdx.x;
    for (int sl = blockIdx.z * kPackSlicesPerWG; sl < min(NSL, (blockIdx.z + 1) * kPackSlicesPerWG); ++sl) {
        // source tile: KS rows of K, the group's 64 source columns
        for (int i = tid; i < KS * kGroupRows; i += 256) {
            const int kl = i / kGroupRows, cl = i % kGroupRows;
            int col;
            if (GATE_UP) col = cl < 32 ? 32 * G + cl : I + 32 * G + (cl - 32);
            else col = kGroupRows * G + cl;
            tile[kl][cl] = s[(size_t)(sl * KS + kl) * N + col];
        }
        __syncthreads();
        // 2 blocks (32 packed rows each) x 2 halves x 64 lanes of 16 bytes
        for (int pc = tid; pc < 256; pc += 256) {
            const int lane = pc & 63, q = (pc >> 6) & 1, gl = pc >> 7;
            const int hh = lane >> 5, j = lane & 31;
            const int p = 32 * gl + j;                                  // packed row in the group
            const int cl = GATE_UP ? gate_up_col_of_packed(p, 32) : down_col_of_packed(p);
            const int k0 = (MXO ? 16 * hh + 32 * q : 32 * hh + 16 * q) / elem;
            union { T v[16 / elem]; u32x4 u; } piece;
#pragma unroll
            for (int t = 0; t < 16 / elem; ++t) piece.v[t] = tile[k0 + t][cl];
            const int g32 = 2 * G + gl;
            *reinterpret_cast<u32x4*>(d + (((long)g32 * NSL + sl) * 2 + q) * 1024 + lane * 16) = piece.u;
        }
        __syncthreads();
    }
}

template <typename T, bool GATE_UP, bool MXO = false>
static hipError_t launch_pack(const void* src, void* dst, int E, int K, int N, int I, hipStream_t st) {
    const int NSL = K * (int)sizeof(T) / kSliceBytes;
    dim3 grid(E, N / kGroupRows, ceil_div(NSL, kPackSlicesPerWG));
    hipLaunchKernelGGL((pack_kernel<T, GATE_UP, MXO>), grid, dim3(256), 0, st, static_cast<const T*>(src),
                       static_cast<uint8_t*>(dst), K, N, I);
    return hipGetLastError();
}

hipError_t launch_pack_mx(const void* src, void* dst, int E, int K, int N, int I, bool gate_up, hipStream_t st) {
    return gate_up ? launch_pack<uint8_t, true, true>(src, dst, E, K, N, I, st)
                   : launch_pack<uint8_t, false, true>(src, dst, E, K, N, I, st);
}

// MX weight scales: E8M0 bytes [E][K/32][N] (per 32 K rows and output column)
// -> per expert [N/32 packed row blocks][K/256 groups][64 lanes] dwords, lane
// 32hh + j of block rb holding, in byte u, the scale of packed row 32rb + j and
// K block 8g + 2u + hh (slice 4g + u, lane half hh): one dword per lane covers
// the 4 slices of a group and a wave-wide load is 256 contiguous bytes.
template <bool GATE_UP>
__global__ void __launch_bounds__(256)
pack_mx_scales_kernel(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int K, int N, int I,
                      long total) {
    const long o = (long)blockIdx.x * 256 + threadIdx.x;
    if (o >= total) return;
    const int NG = K / 256, NB = N / 32;
    const int lane = (int)(o & 63);
    long r = o >> 6;
    const int grp = (int)(r % NG);
    r /= NG;
    const int rb = (int)(r % NB);
    const long e = r / NB;
    const int P = 32 * rb + (lane & 31), hh = lane >> 5;
    const int col = GATE_UP ? gate_up_col_of_packed(P, I) : down_col_of_packed(P);
    uint32_t v = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int kb = 8 * grp + 2 * u + hh;
        v |= (uint32_t)src[(e * (K / 32) + kb) * N + col] << (8 * u);
    }
    dst[o] = v;
}

hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int E, int K, int N, int I, bool gate_up,
                                 hipStream_t st) {
    const long total = (long)E * (N / 32) * (K / 256) * 64;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (gate_up)
        hipLaunchKernelGGL(pack_mx_scales_kernel<true>, dim3(grid), dim3(256), 0, st, src,
                           reinterpret_cast<uint32_t*>(dst), K, N, I, total);
    else
        hipLaunchKernelGGL(pack_mx_scales_kernel<false>, dim3(grid), dim3(256), 0, st, src,
                           reinterpret_cast<uint32_t*>(dst), K, N, I, total);
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
