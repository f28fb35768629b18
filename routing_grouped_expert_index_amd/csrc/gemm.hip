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

#include <type_traits>

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
    int max_tiles;
};

// LDS tile layout: a K step of a tile row is 128 bytes = 8 chunks of 16 bytes;
// chunk c of row r lives at r*128 + ((c ^ (r & 7)) * 16).  The XOR spreads the
// 16-byte MFMA operand reads of 8 consecutive rows over all 32 banks.
constexpr int kRowB = 128;
constexpr int kStages = 3;

__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + ((c ^ (r & 7)) << 4); }

// 16 zero bytes: the source of K-tail chunks past the end of a row.
__device__ __attribute__((aligned(16))) const uint32_t kZero16[4] = {0u, 0u, 0u, 0u};

#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with vmcnt <= N and lgkmcnt == 0 (expcnt untouched)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
}

// Scheduling hint for one straight-line region: groups of (1 VMEM load, 1 DS read,
// 2 MFMAs) while they last, so loads and LDS reads issue between matrix ops.
template <int NV, int ND, int NM>
__device__ __forceinline__ void interleave_hint() {
    if constexpr (NV > 0 || ND > 0 || NM > 0) {
        if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if constexpr (ND > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        constexpr int m = NM >= 2 ? 2 : NM;
        if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        interleave_hint<(NV > 0 ? NV - 1 : 0), (ND > 0 ? ND - 1 : 0), NM - m>();
    }
}

template <bool FP8, bool GATHER, int SC, int EPI, int BM, int BN, int WM, int WN>
struct Gemm {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int MI = TM / 16, NI = TN / 16;
    static constexpr int DA = BM / 8 / NW, DB = BN / 8 / NW;   // 1 KB DMA loads per wave per stage
    static constexpr int DS = SC == SC_BLOCK ? 1 : 0;          // + one row-scale load
    static constexpr int DMA = DA + DB + DS;
    static constexpr int STAGE = (BM + BN) * kRowB + DS * NW * 256;
    static constexpr int SWT = SC == SC_BLOCK ? 64 * (BN / 16) * 4 : 0;   // K up to 64 blocks
    static constexpr int LDS = kStages * STAGE + SWT;
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile/wave mismatch");
    static_assert(MI >= 1 && NI >= 2 && NI % 2 == 0, "wave tile");
    static_assert(NW * 64 >= BM, "row scales: one lane per tile row");
};

template <bool FP8, bool GATHER, int SC, int EPI, int BM, int BN, int WM, int WN, bool KTAIL>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_kernel(const GemmArgs g) {
    using G = Gemm<FP8, GATHER, SC, EPI, BM, BN, WM, WN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
    const int wm = wave / WN, wn = wave % WN;
    const int NTN = g.N / BN;
    const int total = g.ntiles[0] * NTN;
    const int KT = (g.Kb + 127) / 128;   // a partial last step reads zeros past the row end

    // XCD-aware contiguous ranges of the real tile space: one range per XCD
    // (fewer ranges when the grid has fewer than 8 workgroups, so that every
    // range has at least one workgroup walking it)
    const int nwg = gridDim.x;
    const int nx = nwg < 8 ? nwg : 8;
    const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
    const int per_xcd_wg = nwg / nx + (xcd < nwg % nx ? 1 : 0);
    const int lo = (int)((long)total * xcd / nx), hi = (int)((long)total * (xcd + 1) / nx);

    // this lane's place in every 1 KB DMA block: row lane/8 of the block, physical
    // chunk lane%8, which holds logical chunk (lane%8) ^ (lane/8)
    const int dma_row = lane / 8, dma_chunk = (lane % 8) ^ (lane / 8);

    for (int L = lo + slot; L < hi; L += per_xcd_wg) {
        const int mt = L / NTN, nt = L % NTN;
        const int e = g.tiles[2 * mt], row0 = g.tiles[2 * mt + 1];
        const int rows = min(BM, g.offsets[e + 1] - row0);
        const int n0 = nt * BN;

        // per-lane DMA source rows (fixed over K); rows past the expert's end
        // re-read the tile's first row (finite data; their outputs are dropped)
        const uint8_t* ap[G::DA];
#pragma unroll
        for (int i = 0; i < G::DA; ++i) {
            const int r = (wave * G::DA + i) * 8 + dma_row;
            long src = row0 + (r < rows ? r : 0);
            if (GATHER) src = g.perm[src] / g.k;
            ap[i] = g.A + src * g.lda + dma_chunk * 16;
        }
        const uint8_t* bp[G::DB];
#pragma unroll
        for (int i = 0; i < G::DB; ++i) {
            const int r = (wave * G::DB + i) * 8 + dma_row;
            bp[i] = g.B + ((long)e * g.N + n0 + r) * g.Kb + dma_chunk * 16;
        }
        const float* sap = nullptr;
        if constexpr (SC == SC_BLOCK) {
            const int r = wave * 64 + lane;          // lanes past BM fetch a valid, unused row
            long src = row0 + (r < rows ? r : 0);
            if (GATHER) src = g.perm[src] / g.k;
            sap = g.sa + src * g.sa_ld;
        }
        // blockwise FP8: the tile's weight-scale table [KT][BN/16] goes to LDS once
        // per tile (read back in the K loop without global loads in flight)
        float* SWT = reinterpret_cast<float*>(smem + kStages * G::STAGE);
        if constexpr (SC == SC_BLOCK) {
            constexpr int GR = BN / 16;
            for (int i = tid; i < KT * GR; i += G::NT) {
                const int kt = i / GR, pc = n0 + (i % GR) * 16;
                int oc = pc;
                if (EPI != EPI_Y_BF16) {
                    const int grp = pc / 16;
                    oc = (grp & 1) ? g.I + 16 * (grp >> 1) : 16 * (grp >> 1);
                }
                SWT[i] = g.sw[((long)e * KT + kt) * g.nb_orig + oc / 128];
            }
        }

        f32x4 acc[G::MI][G::NI];
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < G::NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

        // one stage: G::DMA direct global->LDS loads per wave
        // request the data of K step skt into ring slot `slot`
        auto issue = [&](int skt, int slot) {
            uint8_t* st = smem + slot * G::STAGE;
            const bool kin = !KTAIL || skt * 128 + dma_chunk * 16 < g.Kb;
#pragma unroll
            for (int i = 0; i < G::DA; ++i) {
                const void* src = kin ? static_cast<const void*>(ap[i] + skt * 128)
                                      : static_cast<const void*>(kZero16);
                __builtin_amdgcn_global_load_lds(src, MOE_LDS(st + (wave * G::DA + i) * 1024), 16, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < G::DB; ++i) {
                const void* src = kin ? static_cast<const void*>(bp[i] + skt * 128)
                                      : static_cast<const void*>(kZero16);
                __builtin_amdgcn_global_load_lds(src, MOE_LDS(st + BM * kRowB + (wave * G::DB + i) * 1024),
                                                 16, 0, 0);
            }
            if constexpr (SC == SC_BLOCK)
                __builtin_amdgcn_global_load_lds(sap + skt, MOE_LDS(st + (BM + BN) * kRowB + wave * 256), 4, 0, 0);
        };
        // Fragments of one K step are read from LDS in two halves (bf16: the two
        // 32-deep MFMA K slices; fp8: the two halves of the wave's columns, with
        // the A fragments kept per step parity).  The next half is always read
        // while the current half's MFMAs run, so LDS latency stays hidden.
        bf16x8 fa[2][G::MI], fb[2][G::NI];
        i32x8 qa[2][G::MI], qb[G::NI];
        f32x4 sav[2][G::MI];
        constexpr int NH = G::NI / 2;
        auto load_half = [&](auto Pc, int stage, int h) {
            constexpr int P = decltype(Pc)::value;
            const uint8_t* As = smem + stage * G::STAGE;
            const uint8_t* Bs = As + BM * kRowB;
            if constexpr (!FP8) {
                const int c = h * 4 + lane / 16;
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
                    fa[h][mi] = *reinterpret_cast<const bf16x8*>(As + swz(wm * G::TM + mi * 16 + lane % 16, c));
#pragma unroll
                for (int ni = 0; ni < G::NI; ++ni)
                    fb[h][ni] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * G::TN + ni * 16 + lane % 16, c));
            } else {
                const int c0 = (lane / 16) * 2;
                auto rd32 = [&](const uint8_t* base, int r) {
                    const u32x4 lo4 = *reinterpret_cast<const u32x4*>(base + swz(r, c0));
                    const u32x4 hi4 = *reinterpret_cast<const u32x4*>(base + swz(r, c0 + 1));
                    return i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                                 (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
                };
                if (h == 0) {
#pragma unroll
                    for (int mi = 0; mi < G::MI; ++mi) {
                        qa[P][mi] = rd32(As, wm * G::TM + mi * 16 + lane % 16);
                        if constexpr (SC == SC_BLOCK)
                            sav[P][mi] = *reinterpret_cast<const f32x4*>(
                                reinterpret_cast<const float*>(Bs + BN * kRowB) + wm * G::TM + mi * 16 + (lane / 16) * 4);
                    }
#pragma unroll
                    for (int ni = 0; ni < NH; ++ni) qb[ni] = rd32(Bs, wn * G::TN + ni * 16 + lane % 16);
                } else {
#pragma unroll
                    for (int ni = NH; ni < G::NI; ++ni) qb[ni] = rd32(Bs, wn * G::TN + ni * 16 + lane % 16);
                }
            }
        };
        auto mfma_half = [&](auto Pc, int kt, int h) {
            constexpr int P = decltype(Pc)::value;
            if constexpr (!FP8) {
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < G::NI; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[h][mi], fb[h][ni], acc[mi][ni], 0, 0, 0);
            } else {
                const float* swt = SWT + kt * (BN / 16) + wn * G::TN / 16;
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                    for (int nj = 0; nj < NH; ++nj) {
                        const int ni = h * NH + nj;
                        if constexpr (SC == SC_BLOCK) {
                            const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                qa[P][mi], qb[ni], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                            const float sw = swt[ni];
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                acc[mi][ni][q] = fmaf(p[q], sav[P][mi][q] * sw, acc[mi][ni][q]);
                        } else {
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                qa[P][mi], qb[ni], acc[mi][ni], 0, 0, 0, 0, 0, 0);
                        }
                    }
            }
        };
        // one K step: half 1 of kt is read, half 0 of kt computes, then (barrier)
        // stage kt is released, kt+3 is requested and half 0 of kt+1 is read
        // while half 1 of kt computes
        // DS reads and LDS-DMA issues are spread between the MFMAs so the matrix
        // core keeps working while the memory pipes are fed
        constexpr int kDsHalf = FP8 ? 2 * G::NI / 2 + 2 * G::MI : G::MI + G::NI;   // ds_reads of half 0
        constexpr int kDsHalf1 = FP8 ? 2 * (G::NI - G::NI / 2) : G::MI + G::NI;    // ds_reads of half 1
        constexpr int kMfmaHalf = FP8 ? G::MI * (G::NI / 2) : G::MI * G::NI;
        auto step = [&](auto Pc, int kt) {
            constexpr int P = decltype(Pc)::value;
            std::integral_constant<int, P ^ 1> Qc;
            load_half(Pc, kt % kStages, 1);
            mfma_half(Pc, kt, 0);
            interleave_hint<0, kDsHalf1, kMfmaHalf>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);   // keep this step's LDS reads above
            wait_vm_lgkm<G::DMA>();                    // stage kt+1 landed (this wave)
            __builtin_amdgcn_s_barrier();             // ... for every wave; slot kt is free
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            // always one stage per step: past the end the last step is re-read into
            // the free slot, so the wait above is the same for every step
            issue(min(kt + 3, KT - 1), (kt + 3) % kStages);
            load_half(Qc, (kt + 1) % kStages, 0);
            mfma_half(Pc, kt, 1);
            interleave_hint<G::DMA, kDsHalf, kMfmaHalf>();
        };

        // three-stage ring, three steps requested ahead
        issue(0, 0);
        issue(min(1, KT - 1), 1);
        issue(min(2, KT - 1), 2);
        wait_vm_lgkm<2 * G::DMA>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        load_half(std::integral_constant<int, 0>{}, 0, 0);
        for (int kt = 0; kt < KT; kt += 2) {
            step(std::integral_constant<int, 0>{}, kt);
            if (kt + 1 < KT) step(std::integral_constant<int, 1>{}, kt + 1);
        }
        __syncthreads();   // the epilogue reuses the stage buffers

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
                // fp32 h; its per-tensor scale is taken over all routes afterwards
                float* H = static_cast<float*>(g.C);
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = rbase + mi * 16 + q;
                        if (r < rows) {
#pragma unroll
                            for (int p = 0; p < G::NI / 2; ++p)
                                H[(long)(row0 + r) * g.ldc + hc0 + p * 16 + lane % 16] = H_AT(mi, p, q);
                        }
                    }
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

template <bool FP8, bool GATHER, int SC, int EPI, int BM, int BN, int WM, int WN, bool KTAIL = false>
static hipError_t run_gemm(const GemmArgs& a, int wg_per_cu, hipStream_t st) {
    using G = Gemm<FP8, GATHER, SC, EPI, BM, BN, WM, WN>;
    auto kern = grouped_gemm_kernel<FP8, GATHER, SC, EPI, BM, BN, WM, WN, KTAIL>;
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

// 128 x 256 tiles (8 waves of 64 x 64: two waves per SIMD, so one wave's MFMAs
// run while the other issues its loads) where the output width allows,
// 128 x 128 tiles (4 waves of 64 x 64) otherwise.
template <bool FP8, bool GATHER, int SC, int EPI>
static hipError_t run_any(const GemmArgs& a, hipStream_t st) {
    if (a.N % 256 == 0) {
        if constexpr (SC == SC_BLOCK)   // per-block rescale needs more registers: 4 waves of 64 x 128
            return run_gemm<FP8, GATHER, SC, EPI, 128, 256, 2, 2>(a, 1, st);
        else
            return run_gemm<FP8, GATHER, SC, EPI, 128, 256, 2, 4>(a, 1, st);
    }
    if constexpr (EPI == EPI_SWIGLU_Q128) {
        return hipErrorInvalidValue;
    } else {
        return run_gemm<FP8, GATHER, SC, EPI, 128, 128, 2, 2>(a, 1, st);
    }
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
        return run_any<false, true, SC_NONE, EPI_SWIGLU_BF16>(a, st);
    }
    if (p.quant == Q_FP8_TENSOR) {
        GemmArgs a = gate_up_args(p, 1);
        a.C = p.h;
        a.ldc = p.I;
        return run_any<true, true, SC_TENSOR, EPI_SWIGLU_F32>(a, st);
    }
    GemmArgs a = gate_up_args(p, 1);
    a.C = p.hq;
    a.ldc = p.I;
    a.cscale = p.sh;
    return run_any<true, true, SC_BLOCK, EPI_SWIGLU_Q128>(a, st);
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
    if (p.quant == Q_BF16) return run_any<false, false, SC_NONE, EPI_Y_BF16>(a, st);
    if (p.quant == Q_FP8_TENSOR) {
        if (a.Kb % 128 != 0)   // I % 128 != 0: the last K step reads zeros past the row end
            return a.N % 256 == 0 ? run_gemm<true, false, SC_TENSOR, EPI_Y_BF16, 128, 256, 2, 4, true>(a, 1, st)
                                  : run_gemm<true, false, SC_TENSOR, EPI_Y_BF16, 128, 128, 2, 2, true>(a, 1, st);
        return run_any<true, false, SC_TENSOR, EPI_Y_BF16>(a, st);
    }
    return run_any<true, false, SC_BLOCK, EPI_Y_BF16>(a, st);
}

}  // namespace moe
