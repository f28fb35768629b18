// Device helpers shared by the gfx950 kernels of the MoE forward.
// (Internal to the HIP library: the CPU oracle has its own, separate codecs.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Two fp32 -> two OCP e4m3fn codes (hardware round-to-nearest-even) in the low
// 16 bits.  Inputs are clamped to +-448 first so the conversion saturates.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
    return f32x2_to_e4m3x2(a, b) | (f32x2_to_e4m3x2(c, d) << 16);
}

// e4m3 code held in byte `sel` of a 32-bit word -> fp32 (exact).
template <int sel>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), sel);
}

// Scale of a quantisation group: amax / 448 (true fp32 division), 1 if all zero.
__device__ __forceinline__ float scale_from_amax(float amax) {
    return amax > 0.0f ? amax / 448.0f : 1.0f;
}

// MX (E8M0 scale per 32 values): the byte of a group whose largest magnitude
// is amax is floor(log2 amax) - 8 + 127 -- the float exponent field less 8, 8
// being the largest exponent of e4m3 -- at least 0 (also for amax = 0 or
// subnormal); the group's codes are e4m3(v * 2^(127 - b)), an exact scaling.
__device__ __forceinline__ uint32_t mx_byte(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 255);
    return (uint32_t)(ef > 8 ? ef - 8 : 0);
}
__device__ __forceinline__ float mx_inv(uint32_t b) { return __uint_as_float((254u - b) << 23); }
// 2^(b - 127) as fp32 (b = 0: the subnormal 2^-127; b <= 254)
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return __uint_as_float(b ? b << 23 : 0x00400000u);
}
// Position of group c's byte in a row of MX scale bytes as the MX GEMM reads
// them: dword 2g + hh holds groups 8g + hh, 8g + 2 + hh, 8g + 4 + hh, 8g + 6 + hh.
__device__ __forceinline__ int mx_scale_pos(int c) { return 8 * (c >> 3) + 4 * (c & 1) + ((c & 7) >> 1); }

// z * sigmoid(z) with the hardware reciprocal (about 1 ulp in fp32)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (static_cast<uint64_t>(1) << lane_id()) - 1;
}

// Lanes of the (active part of the) wave holding the same key as this lane:
// one ballot per key bit (a wave-wide match_any).
__device__ __forceinline__ uint64_t match_any(int key, int nbits) {
    uint64_t m = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
