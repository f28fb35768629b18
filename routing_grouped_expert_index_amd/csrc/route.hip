// Routing for the MoE forward on gfx950: top-k with renormalised softmax gates,
// then the grouped form of the routes -- per-expert counts, their exclusive
// prefix, and a stable permutation of the route ids r = t*k + j by expert
// ("Port necessary FBGEMM MoE kernels", Summary: index_shuffling;
//  "perf: add small-batch route MMA for MoE", Motivation: count/sort, prefix).
//
// Design:
//  * one wavefront per token; each lane keeps ceil(E/64) logits in registers
//    and the k picks are k wave-wide arg-max reductions over order-preserving
//    integer keys of the values, ties to the lower id (-0 is read as +0, so
//    the two compare equal);
//  * counting sort without global atomics: workgroup histograms in LDS, a
//    column scan over workgroups, then a stable scatter in which each wave
//    ranks its routes with a ballot-based match (one ballot per key bit);
//  * a single-workgroup fused kernel serves small T*k (decode) in one launch.
#include <algorithm>

#include "common.cuh"
#include "launch.h"
#include "topk.cuh"

namespace moe {

// Inclusive prefix sum over the 64 lanes of a fully active wave: shifts by 1,
// 2, 4 and 8 inside each row of 16 (lanes shifted in from outside the row read
// 0), then lane 15 of a row added to the next row (rows 1 and 3) and lane 31 to
// rows 2 and 3.
constexpr int kDppRowShr = 0x110;       // + n: lane i reads lane i - n of its row
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 to rows 2 and 3
__device__ __forceinline__ int wave_scan_incl(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 1, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 2, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 4, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 8, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
    return v;
}

// ----------------------------------------------------------------------------
// Small T*k: everything in one workgroup of 16 waves; top-k takes one wave per
// token, counting and scattering one wave per 64 routes (at most 16).
constexpr int kSmallWaves = 16;

__host__ __device__ inline int small_sort_waves(int R) {
    const int n = ceil_div(R, kWave);
    return n < 1 ? 1 : (n > kSmallWaves ? kSmallWaves : n);
}

// The whole routing of T tokens by one workgroup of kSmallWaves waves; `lds`
// holds route_small_lds_bytes(T, E, k).  `logits` may point to global memory
// or to LDS.  Every thread of the workgroup calls it (it holds barriers).
template <int VPL>
__device__ __forceinline__ void route_small_body(const float* __restrict__ logits, int T, int E, int k, int nbits,
                                                 const RouteOut& o, int32_t* lds) {
    int32_t* __restrict__ ids = o.ids;
    float* __restrict__ weights = o.weights;
    int32_t* __restrict__ counts = o.counts;
    int32_t* __restrict__ offsets = o.offsets;
    int32_t* __restrict__ perm = o.perm;
    int32_t* __restrict__ route_pos = o.route_pos;
    const int R = T * k;
    const int nws = small_sort_waves(R);         // waves that count and scatter
    int32_t* sid = lds;                          // [R]
    int32_t* wcnt = sid + R;                     // [nws][E]
    int32_t* base = wcnt + nws * E;              // [E + 1]
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();

    if (T > 0) {
        // the first row of every wave is requested before the LDS set-up (waves
        // past T re-read row T-1 and drop it: an unconditional load is not waited
        // on early)
        TopkRow<VPL> row;
        topk_load<VPL>(logits + (size_t)min(wave, T - 1) * E, E, row);
        for (int i = tid; i < nws * E; i += blockDim.x) wcnt[i] = 0;
        for (int t = wave; t < T; t += kSmallWaves) {
            if (t != wave) topk_load<VPL>(logits + (size_t)t * E, E, row);
            topk_pick<VPL>(row, k, ids + (size_t)t * k, weights + (size_t)t * k, sid + t * k, nullptr);
        }
    } else {   // no routes: zero counts and offsets only (logits may be null)
        for (int i = tid; i < nws * E; i += blockDim.x) wcnt[i] = 0;
    }
    __syncthreads();

    // wave w < nws owns the contiguous route range [lo, hi)
    const int per = ceil_div(R, nws);
    const int lo = wave < nws ? min(R, wave * per) : R, hi = min(R, lo + per);
    for (int r = lo + lane; r < hi; r += kWave) atomicAdd(&wcnt[wave * E + sid[r]], 1);
    __syncthreads();

    // per expert: exclusive prefix over the waves' ranges (route order)
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int w = 0; w < nws; ++w) {
            const int c = wcnt[w * E + e];
            wcnt[w * E + e] = run;
            run += c;
        }
        base[e] = run;                           // count, scanned below
    }
    __syncthreads();
    if (wave == 0) {
        // exclusive scan of the E counts, 8 per lane (E <= 512)
        int c[8], s = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = lane * 8 + i;
            c[i] = e < E ? base[e] : 0;
            s += c[i];
        }
        int run = wave_scan_incl(s) - s;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = lane * 8 + i;
            if (e < E) {
                counts[e] = c[i];
                offsets[e] = run;
                base[e] = run;
            }
            run += c[i];
        }
        if (lane == kWave - 1) { offsets[E] = run; base[E] = run; }
    }
    __syncthreads();

    // stable scatter: each wave walks its own range in order
    for (int s0 = lo; s0 < hi; s0 += kWave) {
        const int r = s0 + lane;
        if (r < hi) {
            const int key = sid[r];
            const uint64_t peers = match_any(key, nbits);
            const int rank = __popcll(peers & lanemask_lt());
            const int p = base[key] + wcnt[wave * E + key] + rank;
            perm[p] = r;
            route_pos[r] = p;
            if (lane == 63 - __clzll(peers)) wcnt[wave * E + key] += __popcll(peers);
        }
    }
}

template <int VPL>
__global__ void __launch_bounds__(kSmallWaves * kWave)
route_small_kernel(const float* __restrict__ logits, int T, int E, int k, int nbits, const RouteOut o) {
    extern __shared__ int32_t lds[];
    route_small_body<VPL>(logits, T, E, k, nbits, o, lds);
}

// ----------------------------------------------------------------------------
// Large T*k: three kernels over blocks of 16 tokens (top-k: one wave per token).
constexpr int kTokPerBlock = 16;
constexpr int kBigWaves = 4;          // scatter kernel
constexpr int kTopkWaves = 16;        // top-k kernel: one token per wave

template <int VPL>
__global__ void __launch_bounds__(kTopkWaves * kWave)
route_topk_hist_kernel(const float* __restrict__ logits, int T, int E, int k,
                       int32_t* __restrict__ ids, float* __restrict__ weights,
                       int32_t* __restrict__ block_hist) {
    __shared__ int32_t cnt[kMaxExperts];
    const int tid = threadIdx.x, wave = tid / kWave;
    const int t0 = blockIdx.x * kTokPerBlock, t1 = min(T, t0 + kTokPerBlock);
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    // the wave's tokens t0 + wave + 16 i: every row is requested before the first pick
    constexpr int TPW = kTokPerBlock / kTopkWaves;
    TopkRow<VPL> rows[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {   // (rows past the block's end re-read its last row, unused)
        const int t = min(t0 + wave + kTopkWaves * i, t1 - 1);
        topk_load<VPL>(logits + (size_t)t * E, E, rows[i]);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = t0 + wave + kTopkWaves * i;
        if (t < t1)
            topk_pick<VPL>(rows[i], k, ids + (size_t)t * k, weights + (size_t)t * k, nullptr, cnt);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) block_hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Column scan over the workgroup histograms: block b's count of expert e
// becomes the number of expert e's routes in blocks before b, and counts[e] the
// column total.  A workgroup owns 8 expert columns; its 32 row groups per
// column each keep their rows in registers between the two passes (a single
// workgroup moving the whole histogram would be bound by one CU's bandwidth).
// The exclusive prefix over experts is taken by the scatter kernel.
constexpr int kScanCols = 8;
constexpr int kScanGroups = 32;
constexpr int kScanRows = 16;   // rows per thread and chunk, loads in flight together

__global__ void __launch_bounds__(kScanCols * kScanGroups)
route_scan_kernel(int nblk, int E, int32_t* __restrict__ block_hist, int32_t* __restrict__ counts) {
    __shared__ int32_t part[kScanGroups][kScanCols];
    const int c = threadIdx.x % kScanCols, p = threadIdx.x / kScanCols;
    const int e = blockIdx.x * kScanCols + c, ec = min(e, E - 1);
    const int per = ceil_div(nblk, kScanGroups);
    const int b0 = min(nblk, p * per), b1 = min(nblk, b0 + per);
    // unconditional loads of clamped rows, masked afterwards (a guarded load
    // compiles to a branch that waits for everything before it)
    int sum = 0;
    for (int b = b0; b < b1; b += kScanRows) {
        int v[kScanRows];
#pragma unroll
        for (int i = 0; i < kScanRows; ++i) v[i] = block_hist[(size_t)min(b + i, nblk - 1) * E + ec];
#pragma unroll
        for (int i = 0; i < kScanRows; ++i) sum += b + i < b1 ? v[i] : 0;
    }
    part[p][c] = sum;
    __syncthreads();
    int before = 0, total = 0;
    for (int q = 0; q < kScanGroups; ++q) {
        const int x = part[q][c];
        if (q < p) before += x;
        total += x;
    }
    __syncthreads();   // every thread has read its rows before any is rewritten
    if (e < E) {
        int run = before;
        for (int b = b0; b < b1; b += kScanRows) {
            int v[kScanRows];
#pragma unroll
            for (int i = 0; i < kScanRows; ++i) v[i] = block_hist[(size_t)min(b + i, nblk - 1) * E + e];
#pragma unroll
            for (int i = 0; i < kScanRows; ++i) {
                if (b + i < b1) {
                    block_hist[(size_t)(b + i) * E + e] = run;
                    run += v[i];
                }
            }
        }
        if (p == 0) counts[e] = total;
    }
}

__global__ void __launch_bounds__(kBigWaves * kWave)
route_scatter_kernel(int T, int E, int k, int nbits, const int32_t* __restrict__ ids,
                     const int32_t* __restrict__ block_hist, const int32_t* __restrict__ counts,
                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                     int32_t* __restrict__ route_pos) {
    __shared__ int32_t wcnt[kBigWaves * kMaxExperts];
    __shared__ int32_t base[kMaxExperts];
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    if (wave == 0) {
        // exclusive prefix of the E counts, 8 per lane (E <= 512); workgroup 0
        // publishes it as the expert offsets
        int cv[8], sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = lane * 8 + i;
            cv[i] = counts[e < E ? e : E - 1];
            cv[i] = e < E ? cv[i] : 0;
            sum += cv[i];
        }
        int run = wave_scan_incl(sum) - sum;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = lane * 8 + i;
            if (e < E) {
                base[e] = run;
                if (blockIdx.x == 0) offsets[e] = run;
            }
            run += cv[i];
        }
        if (blockIdx.x == 0 && lane == kWave - 1) offsets[E] = run;
    }
    const int r0 = blockIdx.x * kTokPerBlock * k;
    const int r1 = min(T, (blockIdx.x + 1) * kTokPerBlock) * k;
    const int per = ceil_div(r1 - r0, kBigWaves);
    const int lo = min(r1, r0 + wave * per), hi = min(r1, lo + per);
    for (int i = tid; i < kBigWaves * E; i += blockDim.x) wcnt[i] = 0;
    __syncthreads();
    for (int r = lo + lane; r < hi; r += kWave) atomicAdd(&wcnt[wave * E + ids[r]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        int run = base[e] + block_hist[(size_t)blockIdx.x * E + e];
        for (int w = 0; w < kBigWaves; ++w) {
            const int c = wcnt[w * E + e];
            wcnt[w * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int s0 = lo; s0 < hi; s0 += kWave) {
        const int r = s0 + lane;
        if (r < hi) {
            const int key = ids[r];
            const uint64_t peers = match_any(key, nbits);
            const int rank = __popcll(peers & lanemask_lt());
            const int p = wcnt[wave * E + key] + rank;
            perm[p] = r;
            route_pos[r] = p;
            if (lane == 63 - __clzll(peers)) wcnt[wave * E + key] += __popcll(peers);
        }
    }
}


// ------------------------------------------------------------------ router --
// Router scores logits = x W_r in fp32 (x bf16 [T, H], W_r fp32 [H, E]
// row-major), optionally followed in the same launch by the routing above.
//
// Workgroup (ks, tb) takes tokens [tb TB, tb TB + TB) over the rows
// [ks hk, ks hk + hk) of W_r, in steps of 64 rows: wave w takes rows 4w..4w+3
// of a step, lane l holds columns l + 64 i (i < VPL) for the TB tokens (TB VPL
// <= 16 accumulators), so one W_r row is one coalesced wave load and the token
// values are wave-uniform (scalar loads).  Each accumulator adds its rows in
// ascending order; the 16 waves' sums meet in a fixed tree (wave w adds wave
// w + 8, then w + 4, w + 2, w + 1) and K-split partials are added in
// ascending ks, so the scores are the same on every run.
//
// Fused form (decode-sized T): the workgroups publish their partials and take
// an arrival ticket (device-scope atomics, stores complete before the ticket,
// as in the route-direct Down kernel); the last one adds the partials into
// LDS and the logits output, returns the ticket to zero and routes from LDS.
constexpr int kRpWaves = kSmallWaves;     // the fused routing runs in the last workgroup
constexpr int kRpRows = 4;                // W_r rows per wave per step
constexpr int kRpStep = kRpWaves * kRpRows;
constexpr int kRpAcc = 16;                // accumulators per lane (tokens x columns)
constexpr size_t kRpTreeBytes = sizeof(float) * (kRpWaves / 2) * kRpAcc * kWave;
constexpr size_t kRpMaxLds = 60 * 1024;
// tokens per workgroup: 16 accumulators, at most 8 tokens (each token's row
// pointer and two in-flight x words live in scalar registers)
__host__ __device__ constexpr int rp_tokens(int vpl) { return kRpAcc / vpl < 8 ? kRpAcc / vpl : 8; }

struct RpArgs {
    const uint16_t* x;   // bf16 [T, H]
    const float* w;      // fp32 [H, E]
    int T, H, E, k, nbits;
    int hk;              // W_r rows per workgroup, a multiple of kRpStep
    float* logits;       // [T, E]
    float* part;         // fused: [gridDim.x][T][E] partial scores
    int32_t* ticket;     // fused: arrival counter, zero between calls
    RouteOut o;
};

template <int VPL, bool FUSED>
__global__ void __launch_bounds__(kRpWaves * kWave)
router_project_kernel(const RpArgs a) {
    constexpr int TB = rp_tokens(VPL);
    extern __shared__ __attribute__((aligned(16))) float rp_lds[];
    __shared__ int last_s;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int T = a.T, H = a.H, E = a.E;
    const int ks = blockIdx.x, t0 = blockIdx.y * TB;
    // token rows (rows past T repeat row T-1; their sums are never written)
    const uint16_t* xr[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) xr[tt] = a.x + (size_t)min(t0 + tt, T - 1) * H;
    int col[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) col[i] = min(lane + kWave * i, E - 1);

    float acc[TB][VPL];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt)
#pragma unroll
        for (int i = 0; i < VPL; ++i) acc[tt][i] = 0.0f;

    const int h_end = (ks + 1) * a.hk;
    float wv[kRpRows][VPL];
    uint2 xv[TB];
    auto load_step = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < kRpRows; ++r)
#pragma unroll
            for (int i = 0; i < VPL; ++i) wv[r][i] = a.w[(size_t)(h0 + r) * E + col[i]];
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) xv[tt] = *reinterpret_cast<const uint2*>(xr[tt] + h0);
    };
    int h0 = ks * a.hk + wave * kRpRows;
    load_step(h0);
    for (; h0 < h_end; h0 += kRpStep) {
        float wc[kRpRows][VPL];
        uint2 xc[TB];
#pragma unroll
        for (int r = 0; r < kRpRows; ++r)
#pragma unroll
            for (int i = 0; i < VPL; ++i) wc[r][i] = wv[r][i];
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) xc[tt] = xv[tt];
        if (h0 + kRpStep < h_end) load_step(h0 + kRpStep);   // the next step's rows in flight
#pragma unroll
        for (int r = 0; r < kRpRows; ++r)
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) {
                const uint32_t pair = (r < 2) ? xc[tt].x : xc[tt].y;
                const float xf = __uint_as_float((r & 1) ? (pair & 0xffff0000u) : (pair << 16));
#pragma unroll
                for (int i = 0; i < VPL; ++i) acc[tt][i] = fmaf(xf, wc[r][i], acc[tt][i]);
            }
    }

    // the waves' sums in a fixed tree through LDS
    for (int half = kRpWaves / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int tt = 0; tt < TB; ++tt)
#pragma unroll
                for (int i = 0; i < VPL; ++i)
                    rp_lds[((wave - half) * kRpAcc + tt * VPL + i) * kWave + lane] = acc[tt][i];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int tt = 0; tt < TB; ++tt)
#pragma unroll
                for (int i = 0; i < VPL; ++i) acc[tt][i] += rp_lds[(wave * kRpAcc + tt * VPL + i) * kWave + lane];
        }
        __syncthreads();
    }

    if constexpr (!FUSED) {
        if (wave == 0) {
#pragma unroll
            for (int tt = 0; tt < TB; ++tt)
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int t = t0 + tt, e = lane + kWave * i;
                    if (t < T && e < E) a.logits[(size_t)t * E + e] = acc[tt][i];
                }
        }
    } else {
        if (wave == 0) {
#pragma unroll
            for (int tt = 0; tt < TB; ++tt)
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int t = t0 + tt, e = lane + kWave * i;
                    if (t < T && e < E)
                        __hip_atomic_store(a.part + ((size_t)ks * T + t) * E + e, acc[tt][i], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            // partial stores, vmcnt(0), then the ticket: agent-scope atomic
            // stores are acknowledged by the device-coherent level, so once the
            // wait returns they are visible to the agent-scope loads of whichever
            // workgroup draws the last ticket; the signal fences keep the
            // compiler from moving either memory operation across the wait
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));   // vmcnt(0)
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (lane == 0)
                last_s = __hip_atomic_fetch_add(a.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                         (int)(gridDim.x * gridDim.y) - 1;
        }
        __syncthreads();
        if (!last_s) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the partial loads stay after the ticket
        // the last workgroup: all partials into LDS at once (8 requests per thread
        // in flight, clamped indices, masked after), the scores added in ks order
        // into LDS and the output, then the routing
        const int n = T * E, KS = gridDim.x, np = KS * n;
        float* stage = rp_lds;                       // [KS][n]
        float* lg = rp_lds + ((np + 3) & ~3);        // [n]
        int32_t* rl = reinterpret_cast<int32_t*>(lg + ((n + 3) & ~3));
        for (int j0 = threadIdx.x; j0 < np; j0 += 8 * (int)blockDim.x) {
            float pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                pv[u] = __hip_atomic_load(a.part + min(j0 + u * (int)blockDim.x, np - 1), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (j0 + u * (int)blockDim.x < np) stage[j0 + u * blockDim.x] = pv[u];
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
            float v = 0.0f;
            for (int q = 0; q < KS; ++q) v += stage[q * n + idx];
            lg[idx] = v;
            a.logits[idx] = v;
        }
        if (threadIdx.x == 0) __hip_atomic_store(a.ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        route_small_body<VPL>(lg, T, E, a.k, a.nbits, a.o, rl);
    }
}

// ----------------------------------------------------------------------------

static int bits_for(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

size_t route_small_lds_bytes(int T, int E, int k) {
    return sizeof(int32_t) * ((size_t)T * k + (size_t)small_sort_waves(T * k) * E + E + 1);
}

bool route_use_small(int T, int E, int k) {
    return (size_t)T * k <= kRouteSmallMaxRoutes && route_small_lds_bytes(T, E, k) <= 64 * 1024;
}

size_t route_workspace_bytes(int T, int E, int k) {
    if (T == 0 || route_use_small(T, E, k)) return 0;
    return sizeof(int32_t) * (size_t)ceil_div(T, kTokPerBlock) * E;
}

#define MOE_VPL_DISPATCH(E, KERNEL, ...)                                   \
    ((E) <= 64 ? (KERNEL<1>)(__VA_ARGS__)                                  \
     : (E) <= 128 ? (KERNEL<2>)(__VA_ARGS__)                               \
     : (E) <= 256 ? (KERNEL<4>)(__VA_ARGS__) : (KERNEL<8>)(__VA_ARGS__))

template <int VPL>
static hipError_t launch_small(const float* logits, int T, int E, int k, const RouteOut& o,
                               hipStream_t st) {
    const size_t lds = route_small_lds_bytes(T, E, k);
    hipLaunchKernelGGL(route_small_kernel<VPL>, dim3(1), dim3(kSmallWaves * kWave), lds, st,
                       logits, T, E, k, bits_for(E), o);
    return hipGetLastError();
}

template <int VPL>
static hipError_t launch_topk_hist(const float* logits, int T, int E, int k, const RouteOut& o,
                                   int32_t* hist, hipStream_t st) {
    hipLaunchKernelGGL(route_topk_hist_kernel<VPL>, dim3(ceil_div(T, kTokPerBlock)),
                       dim3(kTopkWaves * kWave), 0, st, logits, T, E, k, o.ids, o.weights, hist);
    return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, const RouteOut& o,
                        void* ws, hipStream_t st) {
    if (route_use_small(T, E, k)) return MOE_VPL_DISPATCH(E, launch_small, logits, T, E, k, o, st);
    const int nblk = ceil_div(T, kTokPerBlock);
    int32_t* hist = static_cast<int32_t*>(ws);
    hipError_t err = MOE_VPL_DISPATCH(E, launch_topk_hist, logits, T, E, k, o, hist, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_scan_kernel, dim3(ceil_div(E, kScanCols)), dim3(kScanCols * kScanGroups), 0, st,
                       nblk, E, hist, o.counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(nblk), dim3(kBigWaves * kWave), 0, st, T, E, k,
                       bits_for(E), o.ids, hist, o.counts, o.offsets, o.perm, o.route_pos);
    return hipGetLastError();
}

// ---- router scores (+ routing)
static int vpl_for(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : 8; }

RouteProjectPlan route_project_plan(int T, int H, int E, int k) {
    RouteProjectPlan p{};
    const int TB = rp_tokens(vpl_for(E));
    p.ntb = ceil_div(T, TB);
    const size_t lg_bytes = sizeof(float) * (((size_t)T * E + 3) & ~(size_t)3);
    p.lds = kRpTreeBytes;
    // the last workgroup stages every partial in LDS next to the scores and the
    // routing's own arrays: K splits (a divisor of the 64-row steps, at most 64)
    // as many as fit
    const size_t fixed = lg_bytes + route_small_lds_bytes(T, E, k);
    p.fused = T > 0 && route_use_small(T, E, k) && fixed + lg_bytes <= kRpMaxLds;
    p.ks = 1;
    if (p.fused) {
        const int steps = H / kRpStep;
        const int cap = (int)std::min<size_t>(64, (kRpMaxLds - fixed) / lg_bytes);
        for (int d = 1; d <= steps && d <= cap; ++d)
            if (steps % d == 0) p.ks = d;
        p.lds = std::max(p.lds, fixed + (size_t)p.ks * lg_bytes);
    }
    p.hk = H / p.ks;
    p.ws_bytes = kRpTicketBytes + (p.fused ? sizeof(float) * (size_t)p.ks * T * E
                                           : route_workspace_bytes(T, E, k));
    return p;
}

template <int VPL>
static hipError_t launch_project(const RpArgs& a, const RouteProjectPlan& p, hipStream_t st) {
    if (p.fused)
        hipLaunchKernelGGL((router_project_kernel<VPL, true>), dim3(p.ks, p.ntb), dim3(kRpWaves * kWave), p.lds, st, a);
    else
        hipLaunchKernelGGL((router_project_kernel<VPL, false>), dim3(p.ks, p.ntb), dim3(kRpWaves * kWave), p.lds, st, a);
    return hipGetLastError();
}

hipError_t launch_route_project(const uint16_t* x, const float* w_router, int T, int H, int E, int k,
                                float* logits, const RouteOut& o, void* ws, hipStream_t st) {
    if (T == 0) return launch_route(nullptr, 0, E, k, o, nullptr, st);   // counts and offsets only
    const RouteProjectPlan p = route_project_plan(T, H, E, k);
    RpArgs a{};
    a.x = x;
    a.w = w_router;
    a.T = T; a.H = H; a.E = E; a.k = k; a.nbits = bits_for(E);
    a.hk = p.hk;
    a.logits = logits;
    a.ticket = static_cast<int32_t*>(ws);
    a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + kRpTicketBytes);
    a.o = o;
    const int vpl = vpl_for(E);
    hipError_t err = vpl == 1 ? launch_project<1>(a, p, st) : vpl == 2 ? launch_project<2>(a, p, st)
                   : vpl == 4 ? launch_project<4>(a, p, st) : launch_project<8>(a, p, st);
    if (err != hipSuccess || p.fused) return err;
    return launch_route(logits, T, E, k, o, static_cast<char*>(ws) + kRpTicketBytes, st);
}

}  // namespace moe
