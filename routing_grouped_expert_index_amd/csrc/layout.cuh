// Packed expert-weight layout shared by the packing kernel and every kernel that
// reads the packed weights (grouped GEMM, route-direct GEMV).
//
// A weight matrix with reduction length K (Kb = K * element bytes) and N output
// columns is stored, per expert, as
//
//     [N/32 row blocks][Kb/64 slices][2 halves q][64 lanes][16 bytes]
//
// Packed row P = 32*g + j (j < 32) is one output column; slice s covers K bytes
// [64s, 64s+64) of it.  Lane l = 32*hh + j of the 2 KB block (g, s) holds bytes
// [32*hh + 16*q, +16) of row P in half q.  So one wave-wide 16-byte load of half
// q fetches a contiguous kilobyte, and lane l then holds exactly the K values a
// 32x32 MFMA operand lane needs: row l%32, K group l/32 (8 bf16 per half for
// the 32x32x16 bf16 instruction; both halves = 32 e4m3 for 32x32x64).
//
// Packed rows are permuted inside groups of 64 so that a 32x32 MFMA result,
// whose lane l holds rows 8*(i/4) + 4*(l/32) + i%4 (i < 16) of a 32-row block,
// covers contiguous output columns in each lane:
//     packed row p = 32f + 8a + 4hh + b   (f, hh < 2; a, b < 4)
//   Down (N = H):       group G holds output columns [64G, 64G+64):
//                       p -> column 64G + 32hh + 16f + 4a + b
//   Gate/Up (N = 2I):   group G holds h columns [32G, 32G+32):
//                       p -> f == 0: gate of h column 32G + 16hh + 4a + b
//                            f == 1: up of the same h column
//   (gate of h column c is source column c, up is source column I + c).
#pragma once
#include <stdint.h>

namespace moe {

constexpr int kSliceBytes = 64;     // K bytes per slice
constexpr int kGroupRows = 64;      // permutation group

// offset in bytes of (packed row P, K byte kb) inside one expert's matrix
__host__ __device__ inline long packed_offset(int P, int kb, int Kb) {
    const int g = P >> 5, j = P & 31;
    const int s = kb >> 6, w = kb & 63;
    const int hh = w >> 5, q = (w >> 4) & 1, byte = w & 15;
    return (((long)g * (Kb / kSliceBytes) + s) * 2 + q) * 1024 + (hh * 32 + j) * 16 + byte;
}

// output column of Down packed row P
__host__ __device__ inline int down_col_of_packed(int P) {
    const int G = P >> 6, p = P & 63;
    const int f = p >> 5, a = (p >> 3) & 3, hh = (p >> 2) & 1, b = p & 3;
    return 64 * G + 32 * hh + 16 * f + 4 * a + b;
}

// source column of Gate/Up packed row P (gate: h column c; up: I + c)
__host__ __device__ inline int gate_up_col_of_packed(int P, int I) {
    const int G = P >> 6, p = P & 63;
    const int f = p >> 5, a = (p >> 3) & 3, hh = (p >> 2) & 1, b = p & 3;
    const int c = 32 * G + 16 * hh + 4 * a + b;
    return f == 0 ? c : I + c;
}

// packed rows of the gate and up columns of h column c
__host__ __device__ inline int packed_gate_row(int c) {
    const int G = c >> 5, t = c & 31;
    const int hh = t >> 4, a = (t >> 2) & 3, b = t & 3;
    return 64 * G + 8 * a + 4 * hh + b;
}
__host__ __device__ inline int packed_up_row(int c) { return packed_gate_row(c) + 32; }

// packed row of Down output column n
__host__ __device__ inline int packed_down_row(int n) {
    const int G = n >> 6, t = n & 63;
    const int hh = t >> 5, f = (t >> 4) & 1, a = (t >> 2) & 3, b = t & 3;
    return 64 * G + 32 * f + 8 * a + 4 * hh + b;
}

}  // namespace moe
