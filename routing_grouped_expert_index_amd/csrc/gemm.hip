// Grouped expert GEMMs of the MoE forward on gfx950: bf16, FP8 per-tensor, FP8
// with 128x128 block scales, and MX FP8 (an E8M0 scale per 32 K values, applied
// by the scaled MFMA).
//
// "perf: add small-batch route MMA for MoE", Motivation: after the routes are
// grouped by expert, a Gate/Up grouped GEMM, the activation (SwiGLU) with
// optional FP8 quantisation, and a Down grouped GEMM; Summary: FP8 per-tensor
// and 128x128 blockwise scaling, the Down-input quantisation fused into the
// Gate/Up epilogue.
//
// Tile: 128 sorted rows of one expert (from the device-built tile map) x 512
// packed weight rows; eight waves, two per SIMD, each owning 64 weight rows and
// all 128 token rows, i.e. a 2 x 4 grid of 32x32 MFMA blocks (128 fp32
// accumulators per lane, which the compiler keeps in AGPRs).  Two waves per
// SIMD matter twice: a SIMD's MFMAs keep running while one wave waits, and the
// vector-memory throughput a CU sustains grows with the number of waves issuing
// loads (about 13 B/clk per CU from L2 with one wave per SIMD, twice that with
// two).
//  * K advances in 64-byte slices (32 bf16 or 64 e4m3 values).
//  * Token rows move by direct global->LDS DMA into a 5-stage ring, four
//    slices ahead; the Gate/Up A operand is gathered on the fly (sorted row i
//    reads token perm[i] / k), so no gathered copy is ever written.
//  * Weight rows are not shared between waves, so they skip LDS: each wave loads
//    its own 32x32 operand blocks straight into registers (a 4-slot ring, three
//    slices ahead) from the packed layout, where each wave-wide 16-byte load is
//    one contiguous kilobyte.
//  * MFMA: bf16 v_mfma_f32_32x32x16_bf16 (two per slice and block), e4m3
//    v_mfma_f32_32x32x64_f8f6f4 (one per slice and block).  Both operands of an
//    MFMA take the same K values in each lane, so the instruction's internal K
//    order does not matter.
//  * Epilogue from the accumulators: the packed column permutation gives each
//    lane 32 contiguous output columns (Down) or the gate and up values of 16
//    contiguous h columns (Gate/Up) of one row; each wave stages its rows in
//    its own LDS area and writes whole 64- or 128-byte row segments in sorted
//    row order (the combine finds a route's Down row through the inverse
//    permutation).
#include <hip/hip_ext.h>

#include <atomic>

#include "gemm_common.cuh"
#include "layout.cuh"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace g32 {
constexpr int BM = 128;                     // token rows per tile
constexpr int WROWS = 64;                   // packed weight rows per wave
constexpr int NWAVE = 8;
constexpr int NT = 64 * NWAVE;
constexpr int BN = WROWS * NWAVE;           // packed weight rows per tile
constexpr int STAGES = 5;                   // token ring: slices s .. s+4
constexpr int STAGE_B = BM * kSliceBytes;   // 8 KB
constexpr int LDS = STAGES * STAGE_B;
constexpr int kEpiStageBytes = 8192;        // per wave: epilogue staging
constexpr int LDS_TOTAL = LDS + NWAVE * kEpiStageBytes;
// VMEM instructions per wave and slice: weight loads, token DMA
constexpr int WLOADS = 4, DMAS = 1;
// At the top of step s (after its weight loads) the token DMA of slice s,
// issued in step s-4 (or the prologue), is followed by at least the weights
// and DMA of steps s-3 .. s-1 and the weights of step s.
constexpr int WAIT_STEP = 4 * WLOADS + 3 * DMAS;
// Before the MFMAs of step s: the weights of slice s, requested in step s-3
// (or the prologue), are followed by at least the prologue's later weights
// (8), the weights and DMA of step s (5): 13 operations.
constexpr int WAIT_W = 2 * WLOADS + WLOADS + DMAS;
}  // namespace g32

template <bool FP8, bool GATHER, int SC, int EPI, bool SHORT>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm32_kernel(const GemmArgs g) {
    using namespace g32;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int j = lane & 31, hh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // The lane index through an opaque copy at each use: addresses built from
    // it (scale tables, epilogue offsets, the weight-row pointer) are then
    // computed where they are used instead of being hoisted out of the loops
    // and held across the K loop (the long-K FP8 instantiations run at the
    // 256-register limit).
    auto lane_o = [&]() __attribute__((always_inline)) {
        int lo = lane;
        __asm__ volatile("" : "+v"(lo));
        return lo;
    };
    const int NTN = (g.N + BN - 1) / BN;
    const int ntm = ld_const(g.ntiles, 0);
    const int NSL = g.Kb / kSliceBytes;
    const long gstride = 32L * g.Kb;               // bytes between 32-row blocks
    const XcdRange xr = xcd_range(ntm * NTN);
    int L = xr.first;
    if (L >= xr.hi) return;

    // tile L -> (expert, first sorted row, valid rows, this wave's first packed row)
    auto decode = [&](int Lx, int& e_, int& row0_, int& rows_, int& wn0_) __attribute__((always_inline)) {
        int nt, mt;
        if (g.order) { mt = Lx / NTN; nt = Lx - mt * NTN; }     // row tile major
        else { nt = Lx / ntm; mt = Lx - nt * ntm; }             // column tile major
        e_ = ld_const(g.tiles, 2 * mt);
        row0_ = ld_const(g.tiles, 2 * mt + 1);
        rows_ = min(BM, ld_const(g.offsets, e_ + 1) - row0_);
        wn0_ = nt * BN + wave_u * WROWS;   // wave-uniform (scalar registers)
    };
    // token DMA: this wave fills tile rows 16*wave + lane/4, physical chunk
    // lane%4, which holds logical chunk (lane%4) ^ (row/4 % 4); padding rows
    // re-read a valid row.  The wave's 16 source rows are read with scalar
    // loads (a vector load here would need a vmcnt wait that drains the
    // prefetch) and each lane picks its own.
    auto src_row = [&](int row0_, int rows_) __attribute__((always_inline)) {
        int sel = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 16 * wave_u + i;
            const int idx = row0_ + (r < rows_ ? r : 0);
            const int v = GATHER ? ld_const(g.perm, idx) : idx;
            sel = (lane >> 2) == i ? v : sel;
        }
        // (the division by k as a multiply-shift from the host: a divide here
        // would hold a reciprocal in a register through the K loop)
        return GATHER ? (int)(((uint64_t)(uint32_t)sel * g.kdiv_m) >> g.kdiv_s) : sel;
    };
    // The token DMA is a buffer load (MUBUF) with the LDS bit, not the FLAT
    // global_load_lds: the compiler treats a pending FLAT access that may touch
    // LDS as completing out of order and would wait for every LDS read with
    // lgkmcnt(0).  Offsets are unsigned 32-bit byte counts from the resource's
    // base: the gathered x as a whole (the host keeps it below 4 GiB), or, for
    // the sorted rows of h, a base at the tile's first row (64-bit address
    // arithmetic in scalar registers), so h may be any size.
    auto make_arsrc = [&](int row0_) __attribute__((always_inline)) {
        long base = 0, left = g.a_bytes;
        if constexpr (!GATHER) {
            base = (long)row0_ * g.lda;
            left -= base;
        }
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.A) + base, 0,
                                                 (int)(uint32_t)(left < 0xffffffffL ? left : 0xffffffffL),
                                                 0x00020000);
    };
    // A padding row (past the tile's valid rows) takes offset 0xfff00000 plus its
    // slice: past the end of the A resource whenever A is smaller than that
    // (every shape the layer runs at), so the range check turns its loads into
    // zeros and no A bytes are fetched for it; otherwise the offset still lies
    // inside the resource's range and reads valid bytes.  Its MFMAs' results
    // are dropped either way.  (Against re-reading a valid row: the bf16
    // Gate/Up 0-1.5% faster over two sets of interleaved runs, FP8 unchanged.)
    // (the lane's DMA row 16 wave + lane/4 from the opaque lane index: see lane_o)
    auto make_ap = [&](int src, int row0_, int rows_) __attribute__((always_inline)) {
        const int lo = lane_o();
        const int dma_r = 16 * wave_u + (lo >> 2);
        const long rel = GATHER ? src : src - row0_;
        return (dma_r >= rows_ ? 0xFFF00000u : (uint32_t)(rel * g.lda)) +
               (uint32_t)(((lo & 3) ^ ((dma_r >> 2) & 3)) * 16);
    };
    // idle waves (past N) load a valid block, so every wave issues the same loads
    // Epilogue stores are buffer stores through a resource covering C: the
    // rows a wave must not write (tile padding, waves past N) get an offset
    // past the end, which the range check drops, so every wave issues the same
    // SX stores per tile and the K loop's waits can count them (below).
    // The resource starts at the tile's first output row (64-bit address
    // arithmetic in scalar registers) and covers at most 2 GiB, so C may be any
    // size and offset 2^31 is always past its end.
    constexpr long EBC = EPI == EPI_SWIGLU_F32 || EPI == EPI_Y_F32 ? 4 : (EPI == EPI_Y_BF16 || EPI == EPI_SWIGLU_BF16) ? 2 : 1;
    auto make_crsrc = [&](int row0_) __attribute__((always_inline)) {
        const long base = (long)row0_ * g.ldc * EBC, left = g.c_bytes - base;
        return __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(g.C) + base, 0,
                                                 (int)(left < 0x7fffffffL ? left : 0x7fffffffL), 0x00020000);
    };
    constexpr uint32_t kDropped = 0x80000000u;                // past the end of every C resource
    constexpr int CPL = EPI == EPI_SWIGLU_BF16 ? 2 : EPI == EPI_Y_F32 ? 8 : 4;   // chunks per lane and row
    constexpr int CB = 2 * CPL;                               // chunks per row segment
    constexpr int RPP = kEpiStageBytes / (CB * 16);           // staged rows per phase
    constexpr int MPP = RPP / 32;                             // m blocks per phase
    // store instructions per wave and tile (Q128: four rows of codes, four of scales)
    constexpr int SX = EPI == EPI_SWIGLU_Q128 || EPI == EPI_SWIGLU_MX ? 8 : (4 / MPP) * (RPP * CB / 64);
    auto make_wp = [&](int e_, int wn0_) __attribute__((always_inline)) {
        return g.B + (long)e_ * g.N * g.Kb + (long)((wn0_ < g.N ? wn0_ : 0) / 32) * gstride + lane_o() * 16;
    };

    // 128x128-blockwise e4m3: every 128-deep K block kb has its own activation
    // scale per token row and weight scale per 128 output columns.  The
    // accumulators are kept in units of the current block's scale: at the first
    // slice of block kb they are multiplied by s(kb-1)/s(kb) (per token row and
    // weight half, all positive), the MFMAs keep accumulating in place, and after
    // the K loop they are multiplied by s(KT-1).  The tile's activation scales
    // come into LDS ([KT/4][BM][4] floats) by a DMA issued before the tile's
    // prologue: older than every request the K loop waits for, so in-order
    // completion lands them before the first step and no wait counts change.
    constexpr bool BLK = SC == SC_BLOCK;
    // MX e4m3: one E8M0 scale per 32 K values of every token row and weight
    // column, applied by the MFMA itself (v_mfma_scale: the scale of K block kb
    // of row r comes from operand lane r + 32 kb, one byte of a dword picked by
    // op_sel).  That instruction's K blocks are bytes 0-15 of lanes r and r+32
    // (block 0) and bytes 16-31 of them (block 1), so for MX the lanes take the
    // 16-byte chunks hh + 2q of a slice (weights packed that way, tokens read
    // that way): lane half hh then holds MX block 2s + hh of slice s.  Token
    // scales of a row are dwords of 4 bytes, dword 2g + hh holding blocks
    // 8g + 2u + hh (u = slice 4g + u), staged per tile in LDS like the
    // blockwise table; a wave's weight scales are one dword per lane and
    // 32-row block per 4 slices, loaded three slices ahead with the weights.
    constexpr bool MX = SC == SC_MX;
    const int KT = NSL / 2;
    float* sat = reinterpret_cast<float*>(smem + LDS_TOTAL);
    const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(g.sa), 0, BLK || MX ? g.sa_bytes : 0, 0x00020000);
    // this lane's row (16 wave + lane/4, source row src) and scale blocks 4t + lane%4
    // (MX: scale dwords 4t + lane%4)
    auto table = [&](int src) __attribute__((always_inline)) {
        if constexpr (BLK || MX) {
            for (int t = 0; t < (KT + 3) / 4; ++t) {
                const int kb = min(4 * t + (lane_o() & 3), KT - 1);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, MOE_LDS(sat + t * 4 * BM + wave_u * 64), 4,
                                                         (uint32_t)(((long)src * g.sa_ld + kb) * 4), 0, 0, 0);
            }
        }
    };
    // the 128-column weight-scale blocks of this wave's two 32-row halves, made
    // visibly wave-uniform (wn0 comes from threadIdx): the weight scales are
    // then scalar loads, not vector loads whose waits would drain the K loop
    auto col_blocks = [&](int wn0_, int& c0, int& c1) __attribute__((always_inline)) {
        const int P = wn0_ < g.N ? wn0_ : 0;
        if constexpr (EPI == EPI_Y_BF16 || EPI == EPI_Y_F32) {
            c0 = c1 = down_col_of_packed(P) / 128;
        } else {
            c0 = gate_up_col_of_packed(P, g.I) / 128;
            c1 = gate_up_col_of_packed(P + 32, g.I) / 128;
        }
        c0 = __builtin_amdgcn_readfirstlane(c0);
        c1 = __builtin_amdgcn_readfirstlane(c1);
    };

    // MX: the wave's two 32-row blocks' scale dwords of scale group grp (slices
    // 4 grp .. 4 grp + 3; K is a multiple of 256), into wsn; wsc holds the
    // current group's
    const int NB32 = g.N / 32, NG = NSL / 4;
    // (the block base is made visibly wave-uniform, so it lives in scalar
    // registers and each load adds only the lane's offset)
    auto make_wsp = [&](int e_, int wn0_) __attribute__((always_inline)) {
        const int rb = __builtin_amdgcn_readfirstlane((wn0_ < g.N ? wn0_ : 0) / 32);
        return g.swx + ((long)e_ * NB32 + rb) * (long)NG * 64;
    };
    uint32_t wsn[2] = {0u, 0u}, wsc[2] = {0u, 0u};
    auto wsload = [&](const uint32_t* wsp_, int grp) __attribute__((always_inline)) {
        if constexpr (MX) {
#pragma unroll
            for (int f = 0; f < 2; ++f) wsn[f] = wsp_[((long)f * NG + min(grp, NG - 1)) * 64 + lane];
        }
    };

    int e, row0, rows, wn0;
    decode(L, e, row0, rows, wn0);
    const int src0 = src_row(row0, rows);
    __amdgpu_buffer_rsrc_t arsrc = make_arsrc(row0);
    uint32_t ap = make_ap(src0, row0, rows);
    const uint8_t* wp = make_wp(e, wn0);
    const uint32_t* wsp = MX ? make_wsp(e, wn0) : nullptr;
    table(src0);

    f32x16 acc[2][4];
    u32x4 w[4][2][2];     // [slot][block f][half q]

    auto wload = [&](const uint8_t* wp_, int s, int slot) __attribute__((always_inline)) {
        const uint8_t* p = wp_ + (long)s * 2048;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                w[slot][f][q] = *reinterpret_cast<const u32x4*>(p + f * gstride + q * 1024);
    };
    auto dma = [&](uint32_t ap_, int s, int stage) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, MOE_LDS(smem + stage * STAGE_B + wave * 1024), 16,
                                                 ap_ + (uint32_t)(s * kSliceBytes), 0, 0, 0);
    };
    // a tile's first requests: token DMA of slices 0..3, (MX: the weight scales
    // of slices 0..3,) weights of slices 0..2
    auto prologue = [&](uint32_t ap_, const uint8_t* wp_, const uint32_t* wsp_) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) dma(ap_, min(u, NSL - 1), u);
        __builtin_amdgcn_sched_barrier(0);
        wsload(wsp_, 0);
        wload(wp_, 0, 0);
        wload(wp_, min(1, NSL - 1), 1);
        wload(wp_, min(2, NSL - 1), 2);
    };
    // token operand of block m, K half q (16 bytes: chunk 2hh + q of row 32m + j;
    // MX: chunk hh + 2q)
    auto tok = [&](const uint8_t* st, int m, int q) __attribute__((always_inline)) {
        const int r = 32 * m + j, c = MX ? hh + 2 * q : 2 * hh + q;
        return *reinterpret_cast<const u32x4*>(st + r * kSliceBytes + ((c ^ ((r >> 2) & 3)) << 4));
    };
    // The LDS reads of the token operands run ahead of the MFMAs that consume
    // them (scheduling groups pin the interleave; left alone, the compiler
    // reuses one register quad and waits for each read right before its MFMAs).
    // (blockwise e4m3, first slice of a K block: each accumulator block is
    // multiplied by fac[f][m] just before its MFMA, so the multiplies of the next
    // block run under the current MFMA)
    uint32_t tsc[4] = {0u, 0u, 0u, 0u};   // MX: the token rows' scale dwords of the current group
    auto mma = [&](auto Rc, auto Uc, int stage, const float (&fac)[2][4]) __attribute__((always_inline)) {
        constexpr bool RS = decltype(Rc)::value;
        constexpr int slot = decltype(Uc)::value;
        const uint8_t* st = smem + stage * STAGE_B;
        if constexpr (!FP8) {
            // operand kk = 4q + m: K half q of token block m; the two MFMAs of one
            // accumulator (q = 0, 1) are eight instructions apart
            u32x4 tb[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) tb[kk] = tok(st, kk & 3, kk >> 2);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, tb[kk]);
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    acc[f][kk & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, w[slot][f][kk >> 2]), b, acc[f][kk & 3], 0, 0, 0);
            }
            // reads three ahead: R R R, (M M R) x 5, M x 6
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
            for (int kk = 0; kk < 5; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        } else {
            u32x4 tb[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                tb[m][0] = tok(st, m, 0);
                tb[m][1] = tok(st, m, 1);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const u32x4 b0 = tb[m][0], b1 = tb[m][1];
                const i32x8 bv{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                               (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const u32x4 a0 = w[slot][f][0], a1 = w[slot][f][1];
                    const i32x8 av{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                    if constexpr (RS) {
                        const float a = fac[0][m] * fac[1][f];
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[f][m][i] *= a;
                    }
                    if constexpr (MX)   // op_sel: the byte of this slice
                        acc[f][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            av, bv, acc[f][m], 0, 0, slot, (int)wsc[f], slot, (int)tsc[m]);
                    else
                        acc[f][m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[f][m], 0, 0, 0, 0,
                                                                                     0, 0);
                }
            }
            if constexpr (!BLK) {
                // reads one token block ahead: R R R R, (M M R R) x 2, M x 4
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            } else {
                // blockwise (the K loop runs at the register limit): the next
                // token block only, R R, (M M R R) x 3, M M, on K-block starts
                // each M preceded by its block's 16 multiplies
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
#pragma unroll
                    for (int f = 0; f < 2; ++f) {
                        if constexpr (RS) __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    }
                    if (m < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
        }
    };
    // Block kb's scales: sa of the lane's token rows from the LDS table, sw of
    // the wave's two halves by scalar loads.  Nothing is kept across steps: the
    // previous block's scales are read again (registers are the K loop's limit).
    int cb0 = 0, cb1 = 0;
    // the lane's row within a 32-row block (opaque: see lane_o)
    auto jrow = [&]() __attribute__((always_inline)) { return lane_o() & 31; };
    auto sa_of = [&](int kb, int m) __attribute__((always_inline)) {
        return sat[(kb >> 2) * 4 * BM + (32 * m + jrow()) * 4 + (kb & 3)];
    };
    auto sw_of = [&](int kb, int c) __attribute__((always_inline)) {
        return ld_const(g.sw, ((long)e * KT + kb) * g.nb_orig + c);
    };
    // factors into block kb's units (the first block of a tile: 1); the ratios
    // use the hardware reciprocal (about 1 ulp): a few 1e-7 relative over a
    // whole K, and an IEEE division's temporaries would spill the K loop
    // fac[0][m]: the token rows' ratio; fac[1][0..1]: the two halves' weight
    // ratios (wave-uniform, held in scalar registers)
    auto block_factors = [&](int kb, float (&fac)[2][4]) __attribute__((always_inline)) {
        const int kp = kb > 0 ? kb - 1 : 0;
        fac[1][0] = __int_as_float(__builtin_amdgcn_readfirstlane(
            __float_as_int(sw_of(kp, cb0) * __builtin_amdgcn_rcpf(sw_of(kb, cb0)))));
        fac[1][1] = __int_as_float(__builtin_amdgcn_readfirstlane(
            __float_as_int(sw_of(kp, cb1) * __builtin_amdgcn_rcpf(sw_of(kb, cb1)))));
#pragma unroll
        for (int m = 0; m < 4; ++m) fac[0][m] = sa_of(kp, m) * __builtin_amdgcn_rcpf(sa_of(kb, m));
    };
    // The hand-counted waits assume this VMEM order in every step: weight
    // loads, then (after the barrier) the token DMA, with no later load hoisted
    // above the DMA -- a load moved above it would leave fewer than WAIT_STEP
    // loads behind the DMA being waited for.  Scheduling barriers pin that
    // order.  (Extra loads issued later, like the next tile's indices or the
    // epilogue's stores, only add operations behind a DMA and keep the waits
    // sufficient.)
    // One K slice s: weights of s+3 requested; (barrier) tokens of s landed
    // everywhere and every wave is done with stage s-1; DMA of s+4 requested
    // into that stage; MFMAs of s, reading tokens from LDS.  Requests past the
    // end repeat the last slice, so every step waits for the same count.
    // (MFMAs of idle waves and of the padding rows run on valid data and are
    // dropped; a branch around them would make the compiler drain every load
    // first.)
    //
    // A tile's SX epilogue stores are issued after the next tile's prologue, so
    // in the next tile's first four steps XS of them sit between the awaited
    // prologue requests and the newer ones.  Loads complete in issue order
    // among themselves, but a store may complete before older loads, so the
    // wait before the barrier (the only guarantee that the other waves' token
    // DMA has landed) does not count the stores: with younger stores still
    // pending it waits longer, never too little (0-2% on the bf16 prefill GEMMs
    // against counting them, none measurable on FP8).  The weight wait counts
    // them (XW, for the weights of slices 0-2): a wave's weights are its own
    // registers, and the compiler adds its own load-only wait before their
    // first use.
    auto step = [&](auto Uc, int s, bool last, auto Xs, auto Xw) __attribute__((always_inline)) {
        constexpr int U = decltype(Uc)::value;
        constexpr int XS = decltype(Xs)::value, XW = decltype(Xw)::value;
        static_assert(XS == 0 || XS == SX, "stores between the awaited requests and the newer ones");
        // MX: the next scale group's weight scales go out with slice s+3's
        // weights (older than them, so the weight wait of slice s+3 covers them)
        if constexpr (MX && U == 1) wsload(wsp, (s + 3) >> 2);
        wload(wp, min(s + 3, NSL - 1), (U + 3) & 3);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm<WAIT_STEP>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        __builtin_amdgcn_sched_barrier(0);
        dma(ap, min(s + 4, NSL - 1), (s + 4) % STAGES);
        __builtin_amdgcn_sched_barrier(0);
        // the weights of s were requested in step s-3 (or the prologue): at
        // least WAIT_W loads follow them
        // blockwise: the first slice of a K block carries the rescale (its scales
        // are read before the weight wait, the table landed before step 0)
        constexpr bool RS = BLK && (U & 1) == 0;
        std::integral_constant<bool, RS> Rc;
        float fac[2][4];
        if constexpr (RS) block_factors(min(s >> 1, KT - 1), fac);
        if constexpr (MX) {
            // the token rows' scale dwords 2g + hh of this slice's group from the
            // LDS table (landed before step 0; read every step, so they hold no
            // registers across steps)
            const uint32_t* st32 = reinterpret_cast<const uint32_t*>(sat);
            const int d = 2 * min(s >> 2, NG - 1) + hh;
#pragma unroll
            for (int m = 0; m < 4; ++m) tsc[m] = st32[(d >> 2) * 4 * BM + (32 * m + jrow()) * 4 + (d & 3)];
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vm_only<WAIT_W + XW>();
        if constexpr (MX && U == 0) {
            wsc[0] = wsn[0];
            wsc[1] = wsn[1];
        }
        if (!last) mma(Rc, Uc, s % STAGES, fac);
        else if (s < NSL) mma(Rc, Uc, s % STAGES, fac);
    };

    prologue(ap, wp, wsp);
    // the first tile has no epilogue before it: SX dropped stores take its place
    // so that every tile's first steps see the same request counts
    __builtin_amdgcn_sched_barrier(0);
    {
        const __amdgpu_buffer_rsrc_t crsrc = make_crsrc(0);
#pragma unroll
        for (int i = 0; i < SX; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, crsrc, kDropped, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    for (;;) {
        // the next tile's indices are loaded now; their latency hides under this
        // tile's K loop
        const int Ln = L + xr.stride;
        const bool more = Ln < xr.hi;
        int ne = 0, nrow0 = 0, nrows = 1, nwn0 = 0;
        int nsrc = 0;
        if (more) {
            decode(Ln, ne, nrow0, nrows, nwn0);
            nsrc = src_row(nrow0, nrows);
        }

#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[f][m][i] = 0.0f;
        if constexpr (BLK) col_blocks(wn0, cb0, cb1);
        std::integral_constant<int, 0> X0;
        std::integral_constant<int, SX> XE;
        if constexpr (!SHORT) {   // NSL >= 4
            // the first four steps: the previous epilogue's stores in flight
            step(std::integral_constant<int, 0>{}, 0, false, XE, XE);
            step(std::integral_constant<int, 1>{}, 1, false, XE, XE);
            step(std::integral_constant<int, 2>{}, 2, false, XE, XE);
            step(std::integral_constant<int, 3>{}, 3, false, XE, X0);   // weights of 3: step 0
            int s = 4;
            for (; s + 4 <= NSL; s += 4) {
                step(std::integral_constant<int, 0>{}, s, false, X0, X0);
                step(std::integral_constant<int, 1>{}, s + 1, false, X0, X0);
                step(std::integral_constant<int, 2>{}, s + 2, false, X0, X0);
                step(std::integral_constant<int, 3>{}, s + 3, false, X0, X0);
            }
            if (s < NSL) {   // 1-3 slices left
                step(std::integral_constant<int, 0>{}, s, true, X0, X0);
                step(std::integral_constant<int, 1>{}, s + 1, true, X0, X0);
                step(std::integral_constant<int, 2>{}, s + 2, true, X0, X0);
            }
        } else {   // 1-3 slices: every step is among the first four
            step(std::integral_constant<int, 0>{}, 0, true, XE, XE);
            step(std::integral_constant<int, 1>{}, 1, true, XE, XE);
            step(std::integral_constant<int, 2>{}, 2, true, XE, XE);
        }
        // out of the last block's units: the epilogue's conversion multiplies by
        // sal[m] * swl[f] (read now: the next tile's scales overwrite the table below)
        float sal[4], swl0 = 1.0f, swl1 = 1.0f;   // (the weight scales stay scalar)
        if constexpr (BLK) {
            swl0 = sw_of(KT - 1, cb0);
            swl1 = sw_of(KT - 1, cb1);
#pragma unroll
            for (int m = 0; m < 4; ++m) sal[m] = sa_of(KT - 1, m);
        }
        // Every wave is done reading this tile's ring, so the next tile's
        // requests may go out before this tile's stores.  DMA left in flight from
        // this tile's last steps lands in issue order, before the new requests.
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm_only();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (more) table(nsrc);   // (every wave is past its last read of this tile's scales)
        __builtin_amdgcn_sched_barrier(0);
        // (after the last tile the requests repeat this tile's valid data: an
        // unconditional prologue keeps the loop's wait counts exact)
        if (!GATHER && more) arsrc = make_arsrc(nrow0);   // (the DMAs of this tile are all issued)
        const uint32_t nap = more ? make_ap(nsrc, nrow0, nrows) : ap;
        const uint8_t* nwp = more ? make_wp(ne, nwn0) : wp;
        const uint32_t* nwsp = MX && more ? make_wsp(ne, nwn0) : wsp;
        prologue(nap, nwp, nwsp);
        __builtin_amdgcn_sched_barrier(0);

        // ------------------------------------------------------------ epilogue
        // (output offsets count from this tile's first row)
        const __amdgpu_buffer_rsrc_t crsrc = make_crsrc(row0);
        const int lane_e = lane_o();
        const int j_e = lane_e & 31;
        // acc[f][m][i]: token row 32m + j, packed row wn0 + 32f + 8(i/4) + 4hh + i%4.
        // Each lane holds CPL 16-byte chunks of one output row segment per m:
        //   Y (bf16):       columns wn0 + 32hh + 16f + 8hv + [0,8)  -> chunk 4hh + 2f + hv
        //   SwiGLU bf16:    h columns wn0/2 + 16hh + 8h2 + [0,8)     -> chunk 2hh + h2
        //   SwiGLU fp32:    h columns wn0/2 + 16hh + 4h4 + [0,4)     -> chunk 4hh + h4
        //   Y (fp32):       columns wn0 + 32hh + 16f + 8hv + 4q + [0,4) -> chunk 8hh + 4f + 2hv + q
        // Written straight out, one store instruction would touch 32 rows with two
        // 16-byte pieces each.  Instead the wave stages its segments in its own
        // LDS area and stores whole segments: each store instruction then covers
        // 64/CB rows of CB contiguous chunks (128 or 64 bytes per row).
        //   SwiGLU Q128:    h columns wn0/2 + 16hh + [0,16), one 16-byte chunk of
        //                   e4m3 codes per row, stored straight out (see below)
        if constexpr (EPI == EPI_SWIGLU_MX) {
            // h = silu(gate) * up (the MFMAs applied every scale).  A wave's 32 h
            // columns are one MX group per token row, held by the lane pair hh =
            // 0, 1: its E8M0 byte is 2^(floor(log2 amax) - 8) (the float exponent
            // field of amax less 8, at least 0), the codes e4m3(h * 2^(127 - b))
            // (exact power-of-two scaling); each lane stores its 16 codes as one
            // chunk and lane hh = 0 the byte, at the group's place in the row's
            // scale layout (byte 8(c/8) + 4(c%2) + (c%8)/2 for group c).
            const bool live = wn0 < g.N;
            const int hc0 = (live ? wn0 : 0) / 2 + 16 * hh;      // this lane's first h column
            const int hg = (live ? wn0 : 0) / 64;                 // the wave's MX group
            const int spos = 8 * (hg >> 3) + 4 * (hg & 1) + ((hg & 7) >> 1);
            const __amdgpu_buffer_rsrc_t qsrc = __builtin_amdgcn_make_buffer_rsrc(g.cscale, 0, g.cs_bytes, 0x00020000);
            const int nbh = g.I / 32;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc[0][m][i] = silu(acc[0][m][i]) * acc[1][m][i];
                    a = fmaxf(a, fabsf(acc[0][m][i]));
                }
                a = fmaxf(a, __shfl_xor(a, 32));
                const uint32_t b = mx_byte(a);
                const float inv = mx_inv(b);   // 2^(127 - b), b <= 246
                u32x4 q;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    q[t] = f32x4_to_e4m3x4(acc[0][m][4 * t] * inv, acc[0][m][4 * t + 1] * inv,
                                           acc[0][m][4 * t + 2] * inv, acc[0][m][4 * t + 3] * inv);
                const int r = 32 * m + j;
                const bool ok = live && r < rows;
                const uint32_t orow = (uint32_t)(row0 + r);
                __builtin_amdgcn_raw_buffer_store_b128(
                    q, crsrc, ok ? (uint32_t)(32 * m + j_e) * (uint32_t)g.ldc + (uint32_t)hc0 : kDropped, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b8(
                    (uint8_t)b, qsrc, ok && hh == 0 ? orow * (uint32_t)nbh + (uint32_t)spos : kDropped, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (EPI == EPI_SWIGLU_Q128) {
            // h = silu(gate) * up in place of the gate accumulators.  A 128-column
            // h block is 256 packed rows: waves 4b..4b+3 of the tile.  Per token
            // row each wave takes the amax of its 32 columns, the four waves of a
            // block meet in LDS, and each lane then quantises its 16 values with
            // the row's block scale (amax/448) and stores them as one 16-byte
            // chunk; the first wave of the block stores the scale.
            const bool live = wn0 < g.N;
            float* RA = reinterpret_cast<float*>(smem + LDS);     // [NWAVE][BM]
            const int hb = (live ? wn0 : 0) / 256;                // h block of this wave
            const int hc0 = (live ? wn0 : 0) / 2 + 16 * hh;       // this lane's first h column
            const __amdgpu_buffer_rsrc_t qsrc = __builtin_amdgcn_make_buffer_rsrc(g.cscale, 0, g.cs_bytes, 0x00020000);
            const int nbh = g.I / 128;
            // one row block at a time (scheduling barriers keep the compiler from
            // widening the SiLU and division work over all 64 values: the next
            // tile's weight loads are in flight and hold 48 registers)
            float amx[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc[0][m][i] = silu(acc[0][m][i] * (sal[m] * swl0)) * (acc[1][m][i] * (sal[m] * swl1));
                    a = fmaxf(a, fabsf(acc[0][m][i]));
                }
                amx[m] = fmaxf(a, __shfl_xor(a, 32));
                __builtin_amdgcn_sched_barrier(0);
            }
            if (hh == 0) {
#pragma unroll
                for (int m = 0; m < 4; ++m) RA[wave * BM + 32 * m + j_e] = amx[m];
            }
            __asm__ volatile("" ::: "memory");
            wait_lgkm_only();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            __asm__ volatile("" ::: "memory");
            const int grp = wave & ~3;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 32 * m + j;
                const int re = 32 * m + j_e;
                const float a = fmaxf(fmaxf(RA[grp * BM + re], RA[(grp + 1) * BM + re]),
                                      fmaxf(RA[(grp + 2) * BM + re], RA[(grp + 3) * BM + re]));
                const float sc = scale_from_amax(a);
                u32x4 q;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    q[t] = f32x4_to_e4m3x4(acc[0][m][4 * t] / sc, acc[0][m][4 * t + 1] / sc,
                                           acc[0][m][4 * t + 2] / sc, acc[0][m][4 * t + 3] / sc);
                const bool ok = live && r < rows;
                const uint32_t orow = (uint32_t)(row0 + r);
                __builtin_amdgcn_raw_buffer_store_b128(
                    q, crsrc, ok ? (uint32_t)(32 * m + j_e) * (uint32_t)g.ldc + (uint32_t)hc0 : kDropped, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(sc), qsrc,
                    ok && hh == 0 && (wave & 3) == 0 ? (orow * (uint32_t)nbh + (uint32_t)hb) * 4u : kDropped, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            // (the next tile's epilogue rewrites RA only after its K loop's barriers)
        } else {
            // this lane's store offset for staged row lane/CB of phase 0, and how
            // many rows past it are valid (none for waves past N): a store of
            // row rr is kept while rr - lane/CB < rlim
            constexpr int EB = EPI == EPI_SWIGLU_F32 || EPI == EPI_Y_F32 ? 4 : 2;   // bytes per element
            constexpr int CE = 16 / EB;                                  // elements per chunk
            const int c0 = EPI == EPI_Y_BF16 || EPI == EPI_Y_F32 ? wn0 : wn0 / 2;
            const uint32_t lane_off =
                ((uint32_t)(lane_e / CB) * (uint32_t)g.ldc + (uint32_t)(c0 + CE * (lane_e % CB))) * EB;
            const int rlim = wn0 < g.N ? rows - lane / CB : 0;
            const uint32_t row_bytes = (uint32_t)g.ldc * EB;
            // XOR swizzle of the chunk position: the 8 lanes an LDS cycle serves
            // land on 8 distinct 16-byte bank groups, for writes and reads
            auto swz = [](int rr) { return CB == 16 ? (rr & 15) : CB == 8 ? (rr & 7) : ((rr >> 1) & 3); };
            uint8_t* ys = smem + LDS + wave * kEpiStageBytes;
            float fs = 1.0f;
            if constexpr (SC == SC_TENSOR) fs = ld_const(g.sa, 0) * ld_const(g.sw, e);
            // per accumulator block: the tensor scale, or the last K block's scales
            auto fsc = [&](int f, int m) __attribute__((always_inline)) {
                if constexpr (BLK) return sal[m] * (f ? swl1 : swl0);
                else return fs;
            };
#pragma unroll
            for (int ph = 0; ph < 4 / MPP; ++ph) {
#pragma unroll
                for (int mm = 0; mm < MPP; ++mm) {
                    const int m = ph * MPP + mm, rr = 32 * mm + j;
                    u32x4 ch[CPL];
                    if constexpr (EPI == EPI_Y_BF16) {
#pragma unroll
                        for (int f = 0; f < 2; ++f)
#pragma unroll
                            for (int hv = 0; hv < 2; ++hv)
#pragma unroll
                                for (int t = 0; t < 4; ++t)
                                    ch[2 * f + hv][t] = pack_bf16x2(acc[f][m][8 * hv + 2 * t] * fsc(f, m),
                                                                    acc[f][m][8 * hv + 2 * t + 1] * fsc(f, m));
                    } else if constexpr (EPI == EPI_Y_F32) {
                        // (each chunk goes to LDS as it is formed: 8 chunks held
                        // at once would not fit beside the next tile's loads)
#pragma unroll
                        for (int u = 0; u < 8; ++u) {   // u = 4f + 2hv + q: columns ... + 8hv + 4q + [0,4)
                            u32x4 v;
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                v[t] = __float_as_uint(acc[u >> 2][m][8 * ((u >> 1) & 1) + 4 * (u & 1) + t] *
                                                       fsc(u >> 2, m));
                            *reinterpret_cast<u32x4*>(ys + rr * (CB * 16) + (((CPL * hh + u) ^ swz(rr)) << 4)) = v;
                        }
                    } else {
                        float hv[16];
#pragma unroll
                        for (int i = 0; i < 16; ++i) hv[i] = silu(acc[0][m][i] * fs) * (acc[1][m][i] * fs);
                        if constexpr (EPI == EPI_SWIGLU_BF16) {
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                                for (int t = 0; t < 4; ++t)
                                    ch[h2][t] = pack_bf16x2(hv[8 * h2 + 2 * t], hv[8 * h2 + 2 * t + 1]);
                        } else {
#pragma unroll
                            for (int h4 = 0; h4 < 4; ++h4)
#pragma unroll
                                for (int t = 0; t < 4; ++t) ch[h4][t] = __float_as_uint(hv[4 * h4 + t]);
                        }
                    }
                    if constexpr (EPI != EPI_Y_F32) {
#pragma unroll
                        for (int u = 0; u < CPL; ++u)
                            *reinterpret_cast<u32x4*>(ys + rr * (CB * 16) + (((CPL * hh + u) ^ swz(rr)) << 4)) = ch[u];
                    }
                }
                // LDS operations of one wave execute in order; this only keeps the
                // compiler from moving the reads above the writes
                __asm__ volatile("" ::: "memory");
#pragma unroll
                for (int t = 0; t < RPP * CB / 64; ++t) {
                    const int rr = t * (64 / CB) + lane / CB, c = lane % CB;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(ys + rr * (CB * 16) + ((c ^ swz(rr)) << 4));
                    const int dr = t * (64 / CB);   // rows past lane/CB (plus the phase's)
                    const int rp = ph * RPP + dr;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v, crsrc, rp < rlim ? lane_off + (uint32_t)rp * row_bytes : kDropped, 0, 0);
                }
                __asm__ volatile("" ::: "memory");
            }
        }
        if (!more) break;
        L = Ln;
        e = ne;
        row0 = nrow0;
        rows = nrows;
        wn0 = nwn0;
        ap = nap;
        wp = nwp;
        wsp = nwsp;
    }
}

// ----------------------------------------------------------------------------

// compute units of the current device, asked once per device (the persistent
// grid's size; 256 if the runtime cannot tell)
int gemm_num_cus() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cus[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <bool FP8, bool GATHER, int SC, int EPI>
static hipError_t run_gemm32(const GemmArgs& a, hipStream_t st, hipEvent_t ev_end) {
    const bool short_k = a.Kb / kSliceBytes < 4;
    size_t lds = g32::LDS_TOTAL;
    if constexpr (SC == SC_BLOCK) {
        // e4m3 K in whole 128-deep scale blocks; the tile's activation scales,
        // [KT/4][128][4] floats, sit behind the epilogue staging (KT <= 64: 32 KB)
        const int KT = a.Kb / 128;
        if (a.Kb % 128 != 0 || KT < 1 || KT > 64 || a.sa_bytes <= 0 || a.sa_bytes > 0x7fffffffL)
            return hipErrorInvalidValue;
        if (EPI == EPI_SWIGLU_Q128 && (a.I % 128 != 0 || a.cs_bytes <= 0 || a.cs_bytes > 0x7fffffffL))
            return hipErrorInvalidValue;
        lds += (size_t)((KT + 3) / 4) * 4 * g32::BM * sizeof(float);
    }
    if constexpr (SC == SC_MX) {
        // K in whole 256-deep scale groups (a dword of 4 E8M0 bytes per lane and
        // 4 slices); the tile's token scale dwords, K/128 per row, sit in LDS
        // behind the epilogue staging like the blockwise table
        const int KT = a.Kb / 128;
        if (a.Kb % 256 != 0 || KT < 2 || KT > 64 || !a.swx || a.sa_bytes <= 0 || a.sa_bytes > 0x7fffffffL)
            return hipErrorInvalidValue;
        if (EPI == EPI_SWIGLU_MX && (a.I % 64 != 0 || a.cs_bytes <= 0 || a.cs_bytes > 0x7fffffffL))
            return hipErrorInvalidValue;
        lds += (size_t)((KT + 3) / 4) * 4 * g32::BM * sizeof(uint32_t);
    }
    // 32-bit offsets into the gathered x (Gate/Up); h and y are addressed from a
    // base per row tile, so only a row's offsets need 32 bits
    if (a.a_bytes <= 0 || (GATHER && a.a_bytes > 0xffffffffL) || a.c_bytes <= 0 ||
        a.lda * g32::BM > 0x7fffffffL || a.ldc * g32::BM * 4 > 0x7fffffffL)
        return hipErrorInvalidValue;
    const long total_bound = (long)a.max_tiles * ((a.N + g32::BN - 1) / g32::BN);
    long grid = std::min<long>(total_bound, (long)gemm_num_cus());
    if (grid < 1) grid = 1;
    if (short_k)
        hipExtLaunchKernelGGL((gemm32_kernel<FP8, GATHER, SC, EPI, true>), dim3((unsigned)grid), dim3(g32::NT), lds,
                              st, nullptr, ev_end, 0, a);
    else
        hipExtLaunchKernelGGL((gemm32_kernel<FP8, GATHER, SC, EPI, false>), dim3((unsigned)grid), dim3(g32::NT), lds,
                              st, nullptr, ev_end, 0, a);
    return hipGetLastError();
}

// n / d == (n * m) >> s for every n < 2^31 and 1 <= d <= 2^10, with
// s = 31 + ceil(log2 d) and m = ceil(2^s / d) < 2^32: the error n (m - 2^s/d) / 2^s
// is below n / 2^s < 1/d, so the floor is exact.
static void div_magic(int d, uint32_t& m, int& s) {
    int l = 0;
    while ((1 << l) < d) ++l;
    s = 31 + l;
    m = (uint32_t)(((1ULL << s) + (uint64_t)d - 1) / (uint64_t)d);
}

static GemmArgs gate_up_args(const FwdPlan& p, int elem) {
    GemmArgs a{};
    const bool fp8 = p.quant != Q_BF16;
    a.A = fp8 ? p.xq : reinterpret_cast<const uint8_t*>(p.x);
    a.lda = (long)p.H * elem;
    a.perm = p.perm;
    a.k = p.k;
    div_magic(p.k, a.kdiv_m, a.kdiv_s);
    a.B = static_cast<const uint8_t*>(p.wgu);
    a.N = 2 * p.I;
    a.Kb = p.H * elem;
    a.tiles = p.tiles;
    a.ntiles = p.ntiles;
    a.offsets = p.offsets + p.e0;   // the expert slice (the tile map indexes it)
    a.sa = p.quant == Q_FP8_BLOCK || p.quant == Q_FP8_MX ? p.sx : &p.scal[0];
    a.sa_ld = p.H / 128;   // floats per row (block), or dwords of 4 E8M0 bytes (MX)
    a.sw = p.s_gu;
    a.nb_orig = 2 * p.I / 128;
    a.I = p.I;
    a.max_tiles = p.max_tiles;
    a.a_bytes = (long)p.T * a.lda;
    return a;
}

hipError_t launch_grouped_gate_up(const FwdPlan& p, hipStream_t st) {
    if (p.quant == Q_BF16) {
        GemmArgs a = gate_up_args(p, 2);
        a.C = p.h;
        a.ldc = p.I;
        a.c_bytes = (long)p.T * p.k * p.I * 2;
        return run_gemm32<false, true, SC_NONE, EPI_SWIGLU_BF16>(a, st, p.ev_stage_end);
    }
    if (p.quant == Q_FP8_TENSOR) {
        GemmArgs a = gate_up_args(p, 1);
        a.C = p.h;
        a.ldc = p.I;
        a.c_bytes = (long)p.T * p.k * p.I * 4;
        return run_gemm32<true, true, SC_TENSOR, EPI_SWIGLU_F32>(a, st, p.ev_stage_end);
    }
    GemmArgs a = gate_up_args(p, 1);
    a.C = p.hq;
    a.ldc = p.I;
    a.c_bytes = (long)p.T * p.k * p.I;
    a.cscale = p.sh;
    if (p.quant == Q_FP8_MX) {   // E8M0 bytes: x [T][H/32] in, h [R][I/32] out
        a.swx = reinterpret_cast<const uint32_t*>(p.s_gu);
        a.cs_bytes = (long)p.T * p.k * (p.I / 32);
        a.sa_bytes = (long)p.T * (p.H / 32);
        return run_gemm32<true, true, SC_MX, EPI_SWIGLU_MX>(a, st, p.ev_stage_end);
    }
    a.cs_bytes = (long)p.T * p.k * (p.I / 128) * 4;
    a.sa_bytes = (long)p.T * (p.H / 128) * 4;
    return run_gemm32<true, true, SC_BLOCK, EPI_SWIGLU_Q128>(a, st, p.ev_stage_end);
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
    a.offsets = p.offsets + p.e0;   // the expert slice (the tile map indexes it)
    a.sa = p.quant == Q_FP8_BLOCK || p.quant == Q_FP8_MX ? p.sh : &p.scal[1];
    a.sa_ld = p.I / 128;
    a.sw = p.s_d;
    a.nb_orig = p.H / 128;
    a.I = p.I;
    a.C = p.y;
    a.ldc = p.H;
    a.c_bytes = (long)p.T * p.k * p.H * 2;
    a.max_tiles = p.max_tiles;
    a.a_bytes = (long)p.T * p.k * a.lda;
    if (p.quant == Q_BF16) return run_gemm32<false, false, SC_NONE, EPI_Y_BF16>(a, st, p.ev_stage_end);
    if (p.quant == Q_FP8_TENSOR) return run_gemm32<true, false, SC_TENSOR, EPI_Y_BF16>(a, st, p.ev_stage_end);
    if (p.quant == Q_FP8_MX) {
        a.swx = reinterpret_cast<const uint32_t*>(p.s_d);
        a.sa_bytes = (long)p.T * p.k * (p.I / 32);
        return run_gemm32<true, false, SC_MX, EPI_Y_BF16>(a, st, p.ev_stage_end);
    }
    a.sa_bytes = (long)p.T * p.k * (p.I / 128) * 4;
    return run_gemm32<true, false, SC_BLOCK, EPI_Y_BF16>(a, st, p.ev_stage_end);
}

hipError_t launch_grouped_mx_y(const MxProduct& q, hipStream_t st) {
    GemmArgs a{};
    a.A = q.A;
    a.lda = q.K;
    a.perm = q.perm;
    a.k = q.k;
    div_magic(q.k, a.kdiv_m, a.kdiv_s);
    a.B = q.B;
    a.N = q.N;
    a.Kb = q.K;
    a.tiles = q.tiles;
    a.ntiles = q.ntiles;
    a.offsets = q.offsets;
    a.sa = reinterpret_cast<const float*>(q.sa);   // E8M0 bytes, K/128 dwords per row
    a.sa_ld = q.K / 128;
    a.swx = reinterpret_cast<const uint32_t*>(q.swx);
    a.I = q.N;
    a.C = q.C;
    a.ldc = q.N;
    a.c_bytes = q.R * q.N * (q.out_f32 ? 4 : 2);
    a.max_tiles = q.max_tiles;
    a.a_bytes = q.a_rows * q.K;
    a.sa_bytes = q.a_rows * (q.K / 32);
    if (q.out_f32)
        return q.gather ? run_gemm32<true, true, SC_MX, EPI_Y_F32>(a, st, q.ev_end)
                        : run_gemm32<true, false, SC_MX, EPI_Y_F32>(a, st, q.ev_end);
    if (q.gather) return hipErrorInvalidValue;
    return run_gemm32<true, false, SC_MX, EPI_Y_BF16>(a, st, q.ev_end);
}

}  // namespace moe
