// Grouped expert GEMMs of the MoE forward on gfx950 (MFMA).
//
// "perf: add small-batch route MMA for MoE", Motivation: after the routes are
// grouped by expert, a Gate/Up grouped GEMM, the activation (SwiGLU) with
// optional FP8 quantisation, and a Down grouped GEMM; Summary: FP8 per-tensor
// and 128x128 blockwise scaling.
//
// One kernel template serves both projections and all three number formats:
//  * tiles: BM=128 sorted rows of one expert (from the device-built tile map)
//    x BN packed output columns; K is walked 128 bytes at a time (64 bf16 or
//    128 e4m3 values), staged through LDS in two stages, rows padded to 144 B
//    so the 16-byte MFMA operand reads are bank-conflict free;
//  * the Gate/Up A operand is gathered on the fly: sorted row i reads token
//    perm[i] / k of x (or of its e4m3 codes), so no gathered copy is written;
//  * MFMA: bf16 v_mfma_f32_16x16x32_bf16, e4m3 v_mfma_f32_16x16x128_f8f6f4;
//    every lane loads A and B with the same K layout, so the instruction's
//    internal K order does not matter;
//  * blockwise FP8: one K step is one 128-deep scale block, so each MFMA
//    partial is rescaled by s_a[row] * s_w[block] in fp32 before accumulation;
//  * persistent, XCD-aware schedule: workgroup w runs on XCD w % 8 (round-robin
//    dispatch); each XCD walks a contiguous range of the (m-tile, n-tile) space,
//    so the 12-16 n-tiles of an m-tile and neighbouring m-tiles of one expert
//    share that XCD's L2;
//  * epilogues: SwiGLU to bf16 h; SwiGLU to fp32 h plus a global amax (the
//    per-tensor Down-input scale); SwiGLU with per-row 128-column e4m3
//    requantisation; Down output written as bf16 to route order perm[i].
#include "common.cuh"
#include "launch.h"

namespace moe {

enum Epi { EPI_SWIGLU_BF16 = 0, EPI_SWIGLU_F32 = 1, EPI_SWIGLU_Q128 = 2, EPI_Y_BF16 = 3 };
enum Scale { SC_NONE = 0, SC_TENSOR = 1, SC_BLOCK = 2 };

struct GemmArgs {
    const uint8_t* A;       // row-major, lda bytes per row
    long lda;
    const int32_t* perm;    // gather: sorted row i -> token perm[i] / k; Down: output row perm[i]
    int k;
    const uint8_t* B;       // packed [E][N][K]
    int N;                  // packed output columns
    int Kb;                 // K in bytes (multiple of 128)
    const int32_t* tiles;   // [max_tiles][2] (expert, first sorted row)
    const int32_t* ntiles;
    const int32_t* offsets; // [E+1]
    const float* sa;        // tensor: &scalar; block: [rows][sa_ld]
    int sa_ld;
    const float* sw;        // tensor: [E]; block: [E][K/128][nb_orig]
    int nb_orig;
    int I;                  // Gate/Up: h width (column un-interleave)
    void* C;                // output
    long ldc;               // output row stride in elements
    float* cscale;          // Q128: [R][I/128]
    uint32_t* amax;         // F32: amax bits
    int max_tiles;
};

constexpr int kLdsRow = 144;   // 128 data bytes + 16 pad

template <bool FP8, bool GATHER, int SC, int EPI, int BM, int BN, int WM, int WN>
struct Gemm {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int MI = TM / 16, NI = TN / 16;
    static constexpr int CA = BM * 8 / NT, CB = BN * 8 / NT;   // 16-byte chunks per thread
    static constexpr int STAGE = (BM + BN) * kLdsRow + (SC == SC_BLOCK ? BM * 4 : 0);
    static constexpr int LDS = 2 * STAGE;
    static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
    static_assert(MI >= 1 && NI >= 2 && NI % 2 == 0, "wave tile");
};

template <bool FP8, bool GATHER, int SC, int EPI, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_kernel(const GemmArgs g) {
    using G = Gemm<FP8, GATHER, SC, EPI, BM, BN, WM, WN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
    const int wm = wave / WN, wn = wave % WN;
    const int NTN = g.N / BN;
    const int total = g.ntiles[0] * NTN;
    const int KT = (g.Kb + 127) / 128;   // a partial last step is zero-filled (per-tensor I % 128 != 0)

    // XCD-aware contiguous ranges of the real tile space
    const int nwg = gridDim.x;
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int per_xcd_wg = nwg / 8 + (xcd < nwg % 8 ? 1 : 0);
    const int lo = (int)((long)total * xcd / 8), hi = (int)((long)total * (xcd + 1) / 8);

    for (int L = lo + slot; L < hi; L += per_xcd_wg) {
        const int mt = L / NTN, nt = L % NTN;
        const int e = g.tiles[2 * mt], row0 = g.tiles[2 * mt + 1];
        const int rows = min(BM, g.offsets[e + 1] - row0);
        const int n0 = nt * BN;

        // per-thread global pointers (fixed over K)
        const uint8_t* ap[G::CA];
        bool av[G::CA];
#pragma unroll
        for (int i = 0; i < G::CA; ++i) {
            const int c = tid + G::NT * i, r = c / 8;
            av[i] = r < rows;
            long src = row0 + (av[i] ? r : 0);
            if (GATHER) src = g.perm[src] / g.k;
            ap[i] = g.A + src * g.lda + (c % 8) * 16;
        }
        const uint8_t* bp[G::CB];
#pragma unroll
        for (int i = 0; i < G::CB; ++i) {
            const int c = tid + G::NT * i;
            bp[i] = g.B + ((long)e * g.N + n0 + c / 8) * g.Kb + (c % 8) * 16;
        }
        const float* sap = nullptr;
        if (SC == SC_BLOCK && tid < BM) {
            long src = row0 + (tid < rows ? tid : 0);
            if (GATHER) src = g.perm[src] / g.k;
            sap = g.sa + src * g.sa_ld;
        }
        // weight-scale block columns of this wave's 16-wide column groups
        int swcol[G::NI];
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni) {
            const int pc = n0 + wn * G::TN + ni * 16;
            int oc = pc;
            if (EPI != EPI_Y_BF16) {
                const int grp = pc / 16;
                oc = (grp & 1) ? g.I + 16 * (grp >> 1) : 16 * (grp >> 1);
            }
            swcol[ni] = oc / 128;
        }

        f32x4 acc[G::MI][G::NI];
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < G::NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

        u32x4 ra[G::CA], rb[G::CB];
        float rsa = 0.0f;
        auto gload = [&](int kt) {
#pragma unroll
            for (int i = 0; i < G::CA; ++i) {
                const bool kin = kt * 128 + ((tid + G::NT * i) % 8) * 16 < g.Kb;
                ra[i] = (av[i] && kin) ? *reinterpret_cast<const u32x4*>(ap[i] + kt * 128) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < G::CB; ++i) {
                const bool kin = kt * 128 + ((tid + G::NT * i) % 8) * 16 < g.Kb;
                rb[i] = kin ? *reinterpret_cast<const u32x4*>(bp[i] + kt * 128) : u32x4{0, 0, 0, 0};
            }
            if (SC == SC_BLOCK && tid < BM) rsa = tid < rows ? sap[kt] : 0.0f;
        };
        auto sstore = [&](int stage) {
            uint8_t* As = smem + stage * G::STAGE;
            uint8_t* Bs = As + BM * kLdsRow;
#pragma unroll
            for (int i = 0; i < G::CA; ++i) {
                const int c = tid + G::NT * i;
                *reinterpret_cast<u32x4*>(As + (c / 8) * kLdsRow + (c % 8) * 16) = ra[i];
            }
#pragma unroll
            for (int i = 0; i < G::CB; ++i) {
                const int c = tid + G::NT * i;
                *reinterpret_cast<u32x4*>(Bs + (c / 8) * kLdsRow + (c % 8) * 16) = rb[i];
            }
            if (SC == SC_BLOCK && tid < BM)
                reinterpret_cast<float*>(Bs + BN * kLdsRow)[tid] = rsa;
        };

        gload(0);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT) gload(kt + 1);
            const uint8_t* As = smem + cur * G::STAGE;
            const uint8_t* Bs = As + BM * kLdsRow;
            if constexpr (!FP8) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int kb = kk * 64 + (lane / 16) * 16;
                    bf16x8 af[G::MI], bfr[G::NI];
#pragma unroll
                    for (int mi = 0; mi < G::MI; ++mi)
                        af[mi] = *reinterpret_cast<const bf16x8*>(
                            As + (wm * G::TM + mi * 16 + lane % 16) * kLdsRow + kb);
#pragma unroll
                    for (int ni = 0; ni < G::NI; ++ni)
                        bfr[ni] = *reinterpret_cast<const bf16x8*>(
                            Bs + (wn * G::TN + ni * 16 + lane % 16) * kLdsRow + kb);
#pragma unroll
                    for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                        for (int ni = 0; ni < G::NI; ++ni)
                            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni],
                                                                                 acc[mi][ni], 0, 0, 0);
                }
            } else {
                const int kb = (lane / 16) * 32;
                i32x8 af[G::MI], bfr[G::NI];
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi) {
                    const uint8_t* p = As + (wm * G::TM + mi * 16 + lane % 16) * kLdsRow + kb;
                    const u32x4 lo4 = *reinterpret_cast<const u32x4*>(p);
                    const u32x4 hi4 = *reinterpret_cast<const u32x4*>(p + 16);
                    af[mi] = i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                                   (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
                }
#pragma unroll
                for (int ni = 0; ni < G::NI; ++ni) {
                    const uint8_t* p = Bs + (wn * G::TN + ni * 16 + lane % 16) * kLdsRow + kb;
                    const u32x4 lo4 = *reinterpret_cast<const u32x4*>(p);
                    const u32x4 hi4 = *reinterpret_cast<const u32x4*>(p + 16);
                    bfr[ni] = i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                                    (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
                }
                if constexpr (SC == SC_BLOCK) {
                    const float* SA = reinterpret_cast<const float*>(Bs + BN * kLdsRow);
                    float swv[G::NI];
#pragma unroll
                    for (int ni = 0; ni < G::NI; ++ni)
                        swv[ni] = g.sw[((long)e * KT + kt) * g.nb_orig + swcol[ni]];
#pragma unroll
                    for (int mi = 0; mi < G::MI; ++mi) {
                        const f32x4 sav = *reinterpret_cast<const f32x4*>(
                            SA + wm * G::TM + mi * 16 + (lane / 16) * 4);
#pragma unroll
                        for (int ni = 0; ni < G::NI; ++ni) {
                            const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                af[mi], bfr[ni], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc[mi][ni][q] = fmaf(p[q], sav[q] * swv[ni], acc[mi][ni][q]);
                        }
                    }
                } else {
#pragma unroll
                    for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                        for (int ni = 0; ni < G::NI; ++ni)
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                af[mi], bfr[ni], acc[mi][ni], 0, 0, 0, 0, 0, 0);
                }
            }
            if (kt + 1 < KT) sstore(cur ^ 1);
            __syncthreads();
        }

        if constexpr (SC == SC_TENSOR) {
            const float f = g.sa[0] * g.sw[e];
#pragma unroll
            for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[mi][ni][q] *= f;
        }

        // ------------------------------------------------------------ epilogue
        // accumulator (mi, ni, q) of this lane: tile row wm*TM + mi*16 + (lane/16)*4 + q,
        // tile column wn*TN + ni*16 + lane%16
        const int rbase = wm * G::TM + (lane / 16) * 4;
        if constexpr (EPI == EPI_Y_BF16) {
            constexpr int ROWB = BN * 2 + 16;
            uint8_t* Ys = smem;
#pragma unroll
            for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint16_t*>(Ys + (rbase + mi * 16 + q) * ROWB +
                                                     (wn * G::TN + ni * 16 + lane % 16) * 2) =
                            f32_to_bf16(acc[mi][ni][q]);
            __syncthreads();
            constexpr int CPR = BN * 2 / 16;   // 16-byte chunks per row
            for (int c = tid; c < BM * CPR; c += G::NT) {
                const int r = c / CPR, cc = c % CPR;
                if (r < rows) {
                    const long dst_row = g.perm[row0 + r];
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.C) + dst_row * g.ldc + n0 + cc * 8) =
                        *reinterpret_cast<const u32x4*>(Ys + r * ROWB + cc * 16);
                }
            }
            __syncthreads();
        } else {
            // SwiGLU: accumulator pairs (2p gate, 2p+1 up) share lane and register slot
            // h overwrites the gate accumulator (keeps register pressure down)
#pragma unroll
            for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                for (int p = 0; p < G::NI / 2; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[mi][2 * p][q] = silu(acc[mi][2 * p][q]) * acc[mi][2 * p + 1][q];
#define H_AT(mi, p, q) acc[mi][2 * (p)][q]
            // h columns of this wave: hc0 + p*16 + lane%16 (global), tile-local hl0 + ...
            const int hc0 = (n0 + wn * G::TN) / 2;
            const int hl0 = wn * G::TN / 2;
            if constexpr (EPI == EPI_SWIGLU_F32) {
                float am = 0.0f;
                float* H = static_cast<float*>(g.C);
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = rbase + mi * 16 + q;
                        if (r < rows) {
#pragma unroll
                            for (int p = 0; p < G::NI / 2; ++p) {
                                H[(long)(row0 + r) * g.ldc + hc0 + p * 16 + lane % 16] = H_AT(mi, p, q);
                                am = fmaxf(am, fabsf(H_AT(mi, p, q)));
                            }
                        }
                    }
                am = wave_max(am);
                if (lane == 0) atomicMax(g.amax, __float_as_uint(am));
            } else if constexpr (EPI == EPI_SWIGLU_BF16) {
                constexpr int HW = BN / 2;               // h columns per tile
                constexpr int ROWB = HW * 2 + 16;
                uint8_t* Hs = smem;
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                    for (int p = 0; p < G::NI / 2; ++p)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<uint16_t*>(Hs + (rbase + mi * 16 + q) * ROWB +
                                                         (hl0 + p * 16 + lane % 16) * 2) =
                                f32_to_bf16(H_AT(mi, p, q));
                __syncthreads();
                constexpr int CPR = HW * 2 / 16;
                for (int c = tid; c < BM * CPR; c += G::NT) {
                    const int r = c / CPR, cc = c % CPR;
                    if (r < rows)
                        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.C) + (long)(row0 + r) * g.ldc +
                                                  n0 / 2 + cc * 8) =
                            *reinterpret_cast<const u32x4*>(Hs + r * ROWB + cc * 16);
                }
                __syncthreads();
            } else {  // EPI_SWIGLU_Q128: the tile holds exactly one 128-column h block
                static_assert(BN == 256, "Q128 epilogue needs 128 h columns per tile");
                constexpr int ROWB = 128 + 16;
                float* RA = reinterpret_cast<float*>(smem);          // [WN][BM]
                uint8_t* Qs = smem + WN * BM * 4;
                float rowmax[G::MI][4];
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float a = 0.0f;
#pragma unroll
                        for (int p = 0; p < G::NI / 2; ++p) a = fmaxf(a, fabsf(H_AT(mi, p, q)));
#pragma unroll
                        for (int off = 8; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
                        rowmax[mi][q] = a;
                    }
                if (lane % 16 == 0) {
#pragma unroll
                    for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                        for (int q = 0; q < 4; ++q) RA[wn * BM + rbase + mi * 16 + q] = rowmax[mi][q];
                }
                __syncthreads();
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = rbase + mi * 16 + q;
                        float a = 0.0f;
#pragma unroll
                        for (int w = 0; w < WN; ++w) a = fmaxf(a, RA[w * BM + r]);
                        const float s = scale_from_amax(a);
#pragma unroll
                        for (int p = 0; p < G::NI / 2; ++p)
                            Qs[r * ROWB + hl0 + p * 16 + lane % 16] =
                                (uint8_t)(f32x2_to_e4m3x2(H_AT(mi, p, q) / s, 0.0f) & 0xffu);
                        if (wn == 0 && lane % 16 == 0 && r < rows)
                            g.cscale[(long)(row0 + r) * (g.I / 128) + n0 / 256] = s;
                    }
                __syncthreads();
                for (int c = tid; c < BM * 8; c += G::NT) {
                    const int r = c / 8, cc = c % 8;
                    if (r < rows)
                        *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(g.C) + (long)(row0 + r) * g.ldc +
                                                  n0 / 2 + cc * 16) =
                            *reinterpret_cast<const u32x4*>(Qs + r * ROWB + cc * 16);
                }
                __syncthreads();
            }
        }
    }
}

#undef H_AT

// ----------------------------------------------------------------------------

static int g_num_cus = 0;

static int num_cus() {
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            g_num_cus = n;
        else
            g_num_cus = 256;
    }
    return g_num_cus;
}

template <bool FP8, bool GATHER, int SC, int EPI, int BM, int BN, int WM, int WN>
static hipError_t run_gemm(const GemmArgs& a, int wg_per_cu, hipStream_t st) {
    using G = Gemm<FP8, GATHER, SC, EPI, BM, BN, WM, WN>;
    auto kern = grouped_gemm_kernel<FP8, GATHER, SC, EPI, BM, BN, WM, WN>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    const long total_bound = (long)a.max_tiles * (a.N / BN);
    long grid = std::min<long>(total_bound, (long)num_cus() * wg_per_cu);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(G::NT), G::LDS, st, a);
    return hipGetLastError();
}

static GemmArgs gate_up_args(const FwdPlan& p, int elem) {
    GemmArgs a{};
    const bool fp8 = p.quant != Q_BF16;
    a.A = fp8 ? p.xq : reinterpret_cast<const uint8_t*>(p.x);
    a.lda = (long)p.H * elem;
    a.perm = p.perm;
    a.k = p.k;
    a.B = static_cast<const uint8_t*>(p.wgu);
    a.N = 2 * p.I;
    a.Kb = p.H * elem;
    a.tiles = p.tiles;
    a.ntiles = p.ntiles;
    a.offsets = p.offsets;
    a.sa = p.quant == Q_FP8_BLOCK ? p.sx : &p.scal[0];
    a.sa_ld = p.H / 128;
    a.sw = p.s_gu;
    a.nb_orig = 2 * p.I / 128;
    a.I = p.I;
    a.max_tiles = p.max_tiles;
    return a;
}

hipError_t launch_grouped_gate_up(const FwdPlan& p, hipStream_t st) {
    if (p.quant == Q_BF16) {
        GemmArgs a = gate_up_args(p, 2);
        a.C = p.h;
        a.ldc = p.I;
        return run_gemm<false, true, SC_NONE, EPI_SWIGLU_BF16, 128, 128, 2, 2>(a, 2, st);
    }
    if (p.quant == Q_FP8_TENSOR) {
        GemmArgs a = gate_up_args(p, 1);
        a.C = p.h;
        a.ldc = p.I;
        a.amax = &p.amax[1];
        return run_gemm<true, true, SC_TENSOR, EPI_SWIGLU_F32, 128, 128, 2, 2>(a, 2, st);
    }
    GemmArgs a = gate_up_args(p, 1);
    a.C = p.hq;
    a.ldc = p.I;
    a.cscale = p.sh;
    return run_gemm<true, true, SC_BLOCK, EPI_SWIGLU_Q128, 128, 256, 2, 2>(a, 1, st);
}

hipError_t launch_grouped_down(const FwdPlan& p, hipStream_t st) {
    GemmArgs a{};
    const bool fp8 = p.quant != Q_BF16;
    const int elem = fp8 ? 1 : 2;
    a.A = fp8 ? p.hq : static_cast<const uint8_t*>(p.h);
    a.lda = (long)p.I * elem;
    a.perm = p.perm;
    a.k = p.k;
    a.B = static_cast<const uint8_t*>(p.wd);
    a.N = p.H;
    a.Kb = p.I * elem;
    a.tiles = p.tiles;
    a.ntiles = p.ntiles;
    a.offsets = p.offsets;
    a.sa = p.quant == Q_FP8_BLOCK ? p.sh : &p.scal[1];
    a.sa_ld = p.I / 128;
    a.sw = p.s_d;
    a.nb_orig = p.H / 128;
    a.I = p.I;
    a.C = p.y;
    a.ldc = p.H;
    a.max_tiles = p.max_tiles;
    if (p.quant == Q_BF16) return run_gemm<false, false, SC_NONE, EPI_Y_BF16, 128, 128, 2, 2>(a, 2, st);
    if (p.quant == Q_FP8_TENSOR) return run_gemm<true, false, SC_TENSOR, EPI_Y_BF16, 128, 128, 2, 2>(a, 2, st);
    return run_gemm<true, false, SC_BLOCK, EPI_Y_BF16, 128, 128, 2, 2>(a, 1, st);
}

}  // namespace moe
