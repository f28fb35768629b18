// Pieces of the grouped-GEMM kernel (gemm.hip: bf16, FP8 per-tensor, FP8
// 128x128-blockwise and MX FP8).
#pragma once
#include "common.cuh"
#include "launch.h"

namespace moe {

enum Epi { EPI_SWIGLU_BF16 = 0, EPI_SWIGLU_F32 = 1, EPI_SWIGLU_Q128 = 2, EPI_Y_BF16 = 3, EPI_SWIGLU_MX = 4, EPI_Y_F32 = 5 };
enum Scale { SC_NONE = 0, SC_TENSOR = 1, SC_BLOCK = 2, SC_MX = 3 };

struct GemmArgs {
    const uint8_t* A;       // row-major activations, lda bytes per row
    long lda;
    const int32_t* perm;    // gather: sorted row i -> token perm[i] / k; Down: output row perm[i]
    int k;
    uint32_t kdiv_m;        // perm[i] / k == (perm[i] * kdiv_m) >> kdiv_s (exact: perm[i] < 2^31)
    int kdiv_s;
    const uint8_t* B;       // packed weights (layout.cuh), N packed rows, Kb bytes of K
    int N;
    int Kb;
    const int32_t* tiles;   // [max_tiles][2] (expert, first sorted row)
    const int32_t* ntiles;
    const int32_t* offsets; // [E+1]
    const float* sa;        // tensor: &scalar; block: [rows][sa_ld]; MX: E8M0 bytes [rows][4 sa_ld]
    int sa_ld;
    const float* sw;        // tensor: [E]; block: [E][K/128][nb_orig]
    const uint32_t* swx;    // MX: packed weight scales [E][N/32][K/128][64 lanes] (4 E8M0 bytes each)
    int nb_orig;
    int I;                  // Gate/Up: h width
    void* C;                // output
    long ldc;               // output row stride in elements
    float* cscale;          // Q128: [R][I/128]; MX: E8M0 bytes [R][I/32]
    int max_tiles;
    int order;              // tile order: 0 column tile major, 1 row tile major
    long a_bytes;           // bytes of A addressable by the token loads
    long c_bytes;           // bytes of C addressable by the epilogue stores
    long sa_bytes;          // block: bytes of sa (activation scales)
    long cs_bytes;          // Q128: bytes of cscale
};

#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Read-only tables (tile map, offsets) are read through the constant address
// space: with a uniform index that gives scalar loads, which count on lgkmcnt
// and leave the hand-counted vmcnt waits of the GEMM loop undisturbed.
__device__ __forceinline__ int32_t ld_const(const int32_t* p, long i) {
    return ((const __attribute__((address_space(4))) int32_t*)(p))[i];
}
__device__ __forceinline__ float ld_const(const float* p, long i) {
    return ((const __attribute__((address_space(4))) float*)(p))[i];
}

// s_waitcnt with vmcnt <= N and lgkmcnt == 0 (expcnt untouched)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
}

// s_waitcnt with vmcnt <= N only
template <int N>
__device__ __forceinline__ void wait_vm_only() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// s_waitcnt with lgkmcnt == 0 only
__device__ __forceinline__ void wait_lgkm_only() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// Persistent schedule: workgroup w runs on XCD w % 8 (round-robin dispatch);
// each XCD walks one contiguous range of the tile space, so neighbouring tiles
// share that XCD's L2.  With fewer than 8 workgroups there are fewer ranges, so
// every range has a workgroup walking it.
struct XcdRange {
    int lo, hi, first, stride;
};
__device__ __forceinline__ XcdRange xcd_range(int total) {
    const int nwg = gridDim.x;
    const int nx = nwg < 8 ? nwg : 8;
    const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
    XcdRange r;
    r.stride = nwg / nx + (xcd < nwg % nx ? 1 : 0);
    r.lo = (int)((long)total * xcd / nx);
    r.hi = (int)((long)total * (xcd + 1) / nx);
    r.first = r.lo + slot;
    return r;
}

int gemm_num_cus();


}  // namespace moe
