// Grouped expert GEMMs of the MoE forward on gfx950: FP8 with 128x128
// blockwise scales.
//
// "perf: add small-batch route MMA for MoE", Motivation and Summary: the Gate/Up
// and Down grouped GEMMs of the grouped pipeline with 128x128 blockwise FP8
// scaling and the Down-input quantisation fused into the Gate/Up epilogue.
//
// Every 128-deep K block carries its own activation (per row) and weight (per
// 128 output columns) scale, so each K step's MFMA partial is rescaled in fp32
// before it is accumulated.  That needs the partials in VGPRs next to the
// accumulators, so this kernel uses 16x16x128 e4m3 MFMAs on 64 x 128 wave
// tiles (the accumulators stay in VGPRs) and stages both operands through a
// three-stage LDS ring filled by direct global->LDS DMA:
//  * tiles: 128 sorted rows of one expert x 256 packed weight rows (two
//    128-row wave columns of two 64-row permutation groups each), K walked 128
//    bytes at a time;
//  * weight rows are read from the packed layout (layout.cuh): the 16-byte
//    chunk c of a 128-byte K step of packed row P sits in slice 2*step + c/4,
//    half c%2, lane 32*((c%4)/2) + P%32 of that slice's 2 KB block;
//  * the Gate/Up A operand is gathered on the fly (sorted row i reads token
//    perm[i] / k of the e4m3 activations);
//  * epilogues: SwiGLU with per-row 128-column e4m3 requantisation (the tile
//    holds exactly one 128-column h block), and the Down output written as
//    bf16 in sorted row order.
#include "gemm_common.cuh"
#include "layout.cuh"

#include <type_traits>

namespace moe {

// LDS tile layout: a K step of a tile row is 128 bytes = 8 chunks of 16 bytes;
// chunk c of row r lives at r*128 + ((c ^ (r & 7)) * 16).  The XOR spreads the
// 16-byte MFMA operand reads of 8 consecutive rows over all 32 banks.
constexpr int kRowB = 128;
constexpr int kStages = 3;

__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + ((c ^ (r & 7)) << 4); }

// 16 zero bytes: the source of K-tail chunks past the end of a row.
__device__ __attribute__((aligned(16))) const uint32_t kZero16[4] = {0u, 0u, 0u, 0u};

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
            // packed row n0 + r, chunk dma_chunk of each 128-byte K step: slice
            // 2*step + chunk/4, half chunk%2, lane 32*((chunk%4)/2) + row%32
            const int P = n0 + r;
            const int c = dma_chunk;
            bp[i] = g.B + (long)e * g.N * g.Kb +
                    (((long)(P >> 5) * (g.Kb / kSliceBytes) + (c >> 2)) * 2 + (c & 1)) * 1024 +
                    (((c & 3) >> 1) * 32 + (P & 31)) * 16;
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
                // the 16 packed rows from pc on lie in one 128-column scale block
                const int oc = EPI == EPI_Y_BF16 ? down_col_of_packed(pc) : gate_up_col_of_packed(pc, g.I);
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
                const void* src = kin ? static_cast<const void*>(bp[i] + skt * 4096)
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
                                                     down_col_of_packed(wn * G::TN + ni * 16 + lane % 16) * 2) =
                            f32_to_bf16(acc[mi][ni][q]);
            __syncthreads();
            constexpr int CPR = BN * 2 / 16;   // 16-byte chunks per row
            for (int c = tid; c < BM * CPR; c += G::NT) {
                const int r = c / CPR, cc = c % CPR;
                if (r < rows) {
                    const long dst_row = row0 + r;
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.C) + dst_row * g.ldc + n0 + cc * 8) =
                        *reinterpret_cast<const u32x4*>(Ys + r * ROWB + cc * 16);
                }
            }
            __syncthreads();
        } else {
            // SwiGLU: each wave holds two 64-row permutation groups of 16-row blocks
            // 0-3 and 4-7; in a group, blocks 0-1 are gate and blocks 2-3 the up rows
            // of the same h columns, in the same lanes and register slots.  h
            // overwrites the gate accumulator.
            static_assert(G::NI == 8 && EPI == EPI_SWIGLU_Q128, "two permutation groups per wave");
            constexpr int gi[4] = {0, 1, 4, 5};
#pragma unroll
            for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[mi][gi[p]][q] = silu(acc[mi][gi[p]][q]) * acc[mi][gi[p] + 2][q];
#define H_AT(mi, p, q) acc[mi][gi[p]][q]
            // h column of gate block gi[p] in this lane, inside the wave's 64 (tile-local: hl0 + ...)
            const int hl0 = wn * G::TN / 2;
            int hcol[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) hcol[p] = gate_up_col_of_packed(gi[p] * 16 + lane % 16, 64);
            {   // Q128: the tile holds exactly one 128-column h block
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
                        for (int p = 0; p < 4; ++p) a = fmaxf(a, fabsf(H_AT(mi, p, q)));
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
                        for (int p = 0; p < 4; ++p)
                            Qs[r * ROWB + hl0 + hcol[p]] =
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

template <int EPI>
static hipError_t run_block(const GemmArgs& a, hipStream_t st) {
    constexpr int BM = 128, BN = 256, WM = 2, WN = 2;
    using G = Gemm<true, EPI != EPI_Y_BF16, SC_BLOCK, EPI, BM, BN, WM, WN>;
    auto kern = grouped_gemm_kernel<true, EPI != EPI_Y_BF16, SC_BLOCK, EPI, BM, BN, WM, WN, false>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    if (a.N % BN != 0) return hipErrorInvalidValue;
    const long total_bound = (long)a.max_tiles * (a.N / BN);
    long grid = std::min<long>(total_bound, (long)gemm_num_cus());
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(G::NT), G::LDS, st, a);
    return hipGetLastError();
}

hipError_t launch_block_gate_up(const GemmArgs& a, hipStream_t st) { return run_block<EPI_SWIGLU_Q128>(a, st); }
hipError_t launch_block_down(const GemmArgs& a, hipStream_t st) { return run_block<EPI_Y_BF16>(a, st); }

}  // namespace moe
