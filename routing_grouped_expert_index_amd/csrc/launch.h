// Internal launch interface between the host library (moe_api.cpp) and the
// gfx950 kernels.  Not part of the public C ABI (include/moe.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 512;

// Records a message for moe_last_error() on the calling thread; returns code.
int set_error(int code, const char* fmt, ...);
constexpr int kRouteSmallMaxRoutes = 4096;

struct RouteOut {
    int32_t* ids;
    float* weights;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* route_pos;
};

// ---- routing (route.hip)
size_t route_workspace_bytes(int T, int E, int k);
hipError_t launch_route(const float* logits, int T, int E, int k, const RouteOut& o, void* ws,
                        hipStream_t st);

// ---- router scores x W_r, then the routing (route.hip)
constexpr size_t kRpTicketBytes = 256;   // workspace head: the fused kernel's arrival counter
struct RouteProjectPlan {
    bool fused;        // scores and routing in one launch
    int ks, hk, ntb;   // K splits, W_r rows per split, token blocks
    size_t lds;        // dynamic LDS bytes
    size_t ws_bytes;   // workspace: ticket + partial scores (fused) or the routing's own
};
RouteProjectPlan route_project_plan(int T, int H, int E, int k);
hipError_t launch_route_project(const uint16_t* x, const float* w_router, int T, int H, int E, int k,
                                float* logits, const RouteOut& o, void* ws, hipStream_t st);

// ---- weight packing (pack.hip)
hipError_t launch_pack_gate_up(const void* src, void* dst, int E, int H, int I, int elem_bytes,
                               hipStream_t st);
hipError_t launch_pack_down(const void* src, void* dst, int E, int H, int I, int elem_bytes,
                            hipStream_t st);
// MX: e4m3 codes in the chunk order of the scaled MFMA, and the E8M0 scales
// [E][K/32][N] re-laid as [E][N/32][K/256][64 lanes] dwords
hipError_t launch_pack_mx(const void* src, void* dst, int E, int K, int N, int I, bool gate_up, hipStream_t st);
hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int E, int K, int N, int I, bool gate_up,
                                 hipStream_t st);

// ---- forward pieces
enum Quant { Q_BF16 = 0, Q_FP8_TENSOR = 1, Q_FP8_BLOCK = 2, Q_FP8_MX = 3 };

struct FwdPlan {
    // problem
    int T, H, I, E, k, R;
    int quant;
    // inputs
    const uint16_t* x;          // bf16 [T, H]
    const int32_t* ids;         // [T, k]
    const float* tw;            // [T, k]
    const int32_t* offsets;     // [E + 1]
    const int32_t* perm;        // [R]
    const int32_t* route_pos;   // [R] inverse of perm
    const void* wgu;            // packed [E][2I][H]
    const void* wd;             // packed [E][H][I]
    const float* s_gu;          // per-tensor [E] | block [E][H/128][2I/128] | MX: packed E8M0 dwords
    const float* s_d;           // per-tensor [E] | block [E][I/128][H/128] | MX: packed E8M0 dwords
    uint16_t* out;              // bf16 [T, H]
    // workspace carve-up (null where unused)
    int32_t* tiles;             // [max_tiles] (expert << 16 | tile-in-expert) pairs as int2
    int32_t* ntiles;            // [1]
    uint32_t* amax;             // [2]: x amax bits, h amax bits (per-tensor)
    float* scal;                // [2]: s_x, s_h (per-tensor)
    uint8_t* xq;                // e4m3 [T, H]
    float* sx;                  // block: [T, H/128] | MX: E8M0 bytes [T, H/32] (in scale-dword order)
    void* h;                    // bf16 [R, I] (bf16) | fp32 [R, I] (fp8 paths, before requant)
    uint8_t* hq;                // e4m3 [R, I]
    float* sh;                  // block: [R, I/128] | MX: E8M0 bytes [R, I/32] (in scale-dword order)
    uint16_t* y;                // bf16 [R, H] (grouped path, sorted order)
    float* rd_hmax;             // route-direct per-tensor: max |h| of each Gate/Up workgroup [R * I/32 * split]
    float* rd_part;             // route-direct Down partial sums [T * H/32][items][32]
    int32_t* rd_cnt;            // route-direct Down arrival counters [T * H/32]
    int max_tiles;
    // expert slice [e0, e0 + nloc) held by the weights (index e - e0); acc: out += sum
    int e0, nloc, acc;
    // route-direct with the routing folded in: logits [T][E]; the Gate/Up kernel
    // writes each route's id and gate to ids_w / tw_w (ids / tw point there too)
    const float* logits;
    int32_t* ids_w;
    float* tw_w;
    // timing, through events attached to kernel dispatches (hipExtLaunchKernel:
    // no marker packet between kernels): ev_first_start to the forward's first
    // kernel (recorded when it starts), ev_stage_end to the current stage's
    // last kernel (recorded when it ends); null when not timed
    hipEvent_t ev_first_start;
    hipEvent_t ev_stage_end;
};

constexpr int kGemmBM = 128;

int grouped_max_tiles(int R, int E);
// MX products of the backward on the grouped GEMM kernel: C (fp32 or bf16
// [R][N], sorted route rows; bf16 only without gather) = rows of A (e4m3, K bytes each, with E8M0 bytes per 32
// in the MX scale order; the tokens perm[i] / k of an x-shaped A when gather)
// times the packed B (N x K, moe_pack layout) of each row's expert.
struct MxProduct {
    const uint8_t* A;
    const uint8_t* sa;
    long a_rows;                // rows addressable in A and sa
    int K, N;
    const uint8_t* B;
    const uint8_t* swx;         // packed weight scale dwords
    bool gather;
    const int32_t* perm;
    int k;
    const int32_t* tiles;
    const int32_t* ntiles;
    const int32_t* offsets;
    int max_tiles;
    void* C;
    bool out_f32;
    long R;
    hipEvent_t ev_end;
};
hipError_t launch_grouped_mx_y(const MxProduct& q, hipStream_t st);

// backward.hip
hipError_t launch_mx_pack_weights(const uint16_t* src, int E, int K, int N, bool along_k, bool gate_up,
                                  uint8_t* packed, uint8_t* packed_s, uint8_t* plain, uint8_t* plain_s,
                                  hipStream_t st);
hipError_t launch_swiglu_fwd(const float* gu, long R, int I, float* h32, uint8_t* hq, uint8_t* sh,
                             hipEvent_t ev_end, hipStream_t st);
hipError_t launch_dy(const uint16_t* dout, const float* tw, const int32_t* perm, int k, const uint16_t* y, long R,
                     int H, uint8_t* dyq, uint8_t* sdy, float* dgate, hipEvent_t ev_end, hipStream_t st);
hipError_t launch_swiglu_bwd(const float* gu, const float* dh, long R, int I, float* dgu, uint8_t* dguq,
                             uint8_t* sdgu, hipEvent_t ev_end, hipStream_t st);
hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, int32_t* seg, int nseg, hipStream_t st);
// src_kind 0: x bf16 [T][M] through perm; 1: gate * dout (dout bf16 [T][M]);
// 2: fp32 [R][M] in sorted order
hipError_t launch_dim1(int src_kind, const void* src, const uint16_t* dout, const float* tw, const int32_t* perm,
                       int k, const int32_t* offsets, const int32_t* poff, const int32_t* seg, int E, int M, long Rp,
                       long ldo, long lds_, uint8_t* out, uint8_t* sout, hipEvent_t ev_end, hipStream_t st);
hipError_t launch_wgrad(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, long ldo, long lds_,
                        const int32_t* poff, int E, int M, int N, uint16_t* C, hipEvent_t ev_end, hipStream_t st);
hipError_t launch_fill_f32(float* p, long n, float v, hipStream_t st);
hipError_t launch_route_grad(const int32_t* ids, const float* tw, const float* dgate, int T, int E, int k,
                             float* dlogits, hipStream_t st);

hipError_t launch_forward_init(const FwdPlan& p, bool build_tiles, hipStream_t st);
hipError_t launch_quant_x(const FwdPlan& p, hipStream_t st);
hipError_t launch_quant_h(const FwdPlan& p, hipStream_t st);
hipError_t launch_grouped_gate_up(const FwdPlan& p, hipStream_t st);
hipError_t launch_grouped_down(const FwdPlan& p, hipStream_t st);
hipError_t launch_combine(const FwdPlan& p, hipStream_t st);
// workgroups sharing one route-direct Gate/Up 32-row block pair (1, 2 or 4)
int rd_gate_up_split(int T, int H, int I, int k, int quant);
hipError_t launch_route_direct_gate_up(const FwdPlan& p, hipStream_t st);
// (slot, K part) items of one route-direct Down output block
int rd_down_items(int T, int H, int I, int k, int quant);
hipError_t launch_route_direct_down(const FwdPlan& p, hipStream_t st);
// the route-direct launch shape for a call (host-only)
struct RdLaunchInfo {
    int gu_split, gu_waves, down_form, down_parts;
};
RdLaunchInfo rd_launch_info(int T, int H, int I, int k, int quant);

}  // namespace moe
