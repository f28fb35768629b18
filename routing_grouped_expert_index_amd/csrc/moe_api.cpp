// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace sizing and carving, the route-direct / grouped dispatch rule, and
// the launch sequence of each path.  No allocation, no synchronisation, no
// device-to-host copy.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "moe.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Dispatch: the route-direct path wins while the batch is so small that many
// experts receive no route ("perf: add small-batch route MMA for MoE", Motivation
// and Dispatch).  The bound comes from measuring both paths, forced, at batch
// 1-16 and top-k 8 on this GPU (cold weights): with E=128, H=2048, I=768 bf16
// route-direct is faster up to about 112 routes (0.85 E); with E=192, H=4096,
// I=192 FP8 per-tensor still at 128 routes (0.67 E, the largest measured).
// Rule: T*k <= 3E/4 and T <= 16 (the measured range).
constexpr int kRouteDirectMaxTokens = 16;

// Route-direct kernels stage one activation row in LDS: H * elem <= 8192 bytes
// for Gate/Up, I * elem <= 2048 bytes for Down.
bool rd_shape_ok(int H, int I, int k, int quant) {
    const int elem = quant == MOE_BF16 ? 2 : 1;
    (void)k;
    return (long)H * elem <= 8192 && (long)I * elem <= 2048;
}

int check_shape(int T, int H, int I, int E, int k, int quant) {
    if (T < 0 || H <= 0 || I <= 0) return fail(MOE_ERR_INVALID_ARG, "T=%d H=%d I=%d: sizes must be positive (T >= 0)", T, H, I);
    if (k < 1 || E < k || E > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "need 1 <= k <= E <= %d (k=%d, E=%d)", moe::kMaxExperts, k, E);
    if (quant < MOE_BF16 || quant > MOE_FP8_MX32) return fail(MOE_ERR_INVALID_ARG, "unknown quant %d", quant);
    if ((long)T * k >= (1L << 31) || (long)T * H >= (1L << 31))
        return fail(MOE_ERR_UNSUPPORTED, "T*k and T*H must fit in int32");
    // The grouped GEMMs address the gathered x (at most 4 GiB when T*H < 2^31)
    // and the per-row scale tables with 32-bit offsets; h and y are addressed
    // from a 64-bit base per row tile, so their size is not limited here.
    if ((long)T * k * I >= (1L << 36))
        return fail(MOE_ERR_UNSUPPORTED, "T*k*I = %ld must be below 2^36", (long)T * k * I);
    if (H % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "H=%d: H must be a multiple of 64", H);
    if (quant == MOE_FP8_BLOCK128 && H % 128 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "H=%d: block128 needs H a multiple of 128", H);
    if (I % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "I=%d: I must be a multiple of 64", I);
    if (quant == MOE_FP8_BLOCK128 && I % 128 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "I=%d: block128 needs I a multiple of 128", I);
    if (quant == MOE_FP8_BLOCK128 && (H > 8192 || I > 8192))
        return fail(MOE_ERR_UNSUPPORTED, "block128: H and I up to 8192 (64 scale blocks along K)");
    if (quant == MOE_FP8_MX32 && (H % 256 != 0 || I % 256 != 0 || H > 8192 || I > 8192))
        return fail(MOE_ERR_UNSUPPORTED, "MX: H and I multiples of 256, up to 8192 (H=%d, I=%d)", H, I);
    if ((long)E * H * 2 * I >= (1L << 40)) return fail(MOE_ERR_UNSUPPORTED, "weights too large");
    return MOE_OK;
}

int resolve_path(int T, int H, int I, int E, int k, int quant, int path) {
    if (path == MOE_PATH_AUTO) {
        const bool small = T <= kRouteDirectMaxTokens && 4L * T * k <= 3L * E;
        return (small && rd_shape_ok(H, I, k, quant)) ? MOE_PATH_ROUTE_DIRECT : MOE_PATH_GROUPED;
    }
    if (path == MOE_PATH_GROUPED) return path;
    if (path == MOE_PATH_ROUTE_DIRECT) {
        if (!rd_shape_ok(H, I, k, quant))
            return fail(MOE_ERR_UNSUPPORTED,
                        "route-direct path: H*elem <= 8192 and I*elem <= 2048 bytes");
        return path;
    }
    return fail(MOE_ERR_INVALID_ARG, "unknown path %d", path);
}

struct Layout {
    size_t tiles, ntiles, amax, scal, xq, sx, h, hq, sh, y, rd_hmax, rd_part, rd_cnt, total;
};

Layout layout(int T, int H, int I, int E, int k, int quant, int path) {
    Layout L{};
    const size_t R = (size_t)T * k;
    const bool grouped = path == MOE_PATH_GROUPED;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return bytes ? at : (size_t)-1;
    };
    L.tiles = take(grouped ? sizeof(int32_t) * 2 * (size_t)moe::grouped_max_tiles((int)R, E) : 0);
    L.ntiles = take(grouped ? sizeof(int32_t) : 0);
    L.amax = take(2 * sizeof(uint32_t));
    L.scal = take(2 * sizeof(float));
    // (route-direct: the Gate/Up kernel leaves the codes of each token's x row
    // here too, for inspection; it reads them from LDS)
    L.xq = take(quant != MOE_BF16 ? (size_t)T * H : 0);
    L.sx = take(quant == MOE_FP8_BLOCK128 ? sizeof(float) * (size_t)T * (H / 128)
                : quant == MOE_FP8_MX32 ? (size_t)T * (H / 32) : 0);
    size_t hbytes = 0;
    if (quant == MOE_BF16) hbytes = R * I * 2;
    else if (quant == MOE_FP8_PER_TENSOR || !grouped) hbytes = R * I * 4;
    L.h = take(hbytes);
    L.hq = take(grouped && quant != MOE_BF16 ? R * I : 0);
    L.sh = take(quant == MOE_FP8_BLOCK128 ? sizeof(float) * R * (I / 128)
                : quant == MOE_FP8_MX32 ? R * (I / 32) : 0);
    L.y = take(grouped ? R * H * 2 : 0);
    const size_t rd_blocks = grouped ? 0 : (size_t)T * (H / 32);
    L.rd_hmax = take(!grouped && quant == MOE_FP8_PER_TENSOR
                         ? sizeof(float) * R * (I / 32) * moe::rd_gate_up_split(T, H, I, k, quant)
                         : 0);
    L.rd_part = take(rd_blocks * sizeof(float) * 32 * (size_t)(grouped ? 0 : moe::rd_down_items(T, H, I, k, quant)));
    L.rd_cnt = take(rd_blocks * sizeof(int32_t));
    L.total = off;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) {
    return off == (size_t)-1 ? nullptr : reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace moe {
int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}
}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_err; }

size_t moe_route_workspace_size(int T, int E, int k) {
    if (T < 0 || k < 1 || E < k || E > moe::kMaxExperts) return 0;
    return moe::route_workspace_bytes(T, E, k);
}

int moe_route(const float* logits, int T, int E, int k, moe_routes* out, void* ws, size_t ws_bytes,
              void* stream) {
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if (T < 0 || k < 1 || E < k || E > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "need T >= 0 and 1 <= k <= E <= %d (T=%d k=%d E=%d)",
                    moe::kMaxExperts, T, k, E);
    if ((long)T * k >= (1L << 31) || (long)T * E >= (1L << 31))
        return fail(MOE_ERR_UNSUPPORTED, "T*k and T*E must fit in int32");
    if (!out->expert_counts || !out->expert_offsets || (T > 0 && (!logits || !out->topk_ids ||
        !out->topk_weights || !out->perm || !out->route_pos)))
        return fail(MOE_ERR_INVALID_ARG, "null pointer among logits / routes members");
    const void* ptrs[] = {logits, out->topk_ids, out->topk_weights, out->expert_counts,
                          out->expert_offsets, out->perm, out->route_pos};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const size_t need = moe::route_workspace_bytes(T, E, k);
    if (ws_bytes < need || (need && !ws))
        return fail(MOE_ERR_WORKSPACE, "route workspace: need %zu bytes, got %zu", need, ws_bytes);
    out->T = T;
    out->E = E;
    out->k = k;
    const moe::RouteOut o{out->topk_ids, out->topk_weights, out->expert_counts, out->expert_offsets,
                          out->perm, out->route_pos};
    const int rc = hip_status(moe::launch_route(logits, T, E, k, o, ws, static_cast<hipStream_t>(stream)),
                              "moe_route launch");
    return rc == MOE_OK ? ok() : rc;
}

static bool route_project_shape_ok(int T, int H, int E, int k) {
    return T >= 0 && k >= 1 && E >= k && E <= moe::kMaxExperts && H >= 64 && H % 64 == 0 &&
           (long)T * k < (1L << 31) && (long)T * E < (1L << 31) && (long)T * H < (1L << 31);
}

size_t moe_route_project_workspace_size(int T, int H, int E, int k) {
    if (!route_project_shape_ok(T, H, E, k)) return 0;
    return moe::route_project_plan(T, H, E, k).ws_bytes;
}

int moe_route_project(const void* x, const float* w_router, int T, int H, int E, int k, float* logits,
                      moe_routes* out, void* ws, size_t ws_bytes, void* stream) {
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if (T < 0 || k < 1 || E < k || E > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "need T >= 0 and 1 <= k <= E <= %d (T=%d k=%d E=%d)",
                    moe::kMaxExperts, T, k, E);
    if (H < 64 || H % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "H must be a positive multiple of 64 (H=%d)", H);
    if (!route_project_shape_ok(T, H, E, k))
        return fail(MOE_ERR_UNSUPPORTED, "T*k, T*E and T*H must fit in int32");
    if (!out->expert_counts || !out->expert_offsets || (T > 0 && (!x || !w_router || !logits ||
        !out->topk_ids || !out->topk_weights || !out->perm || !out->route_pos)))
        return fail(MOE_ERR_INVALID_ARG, "null pointer among x / w_router / logits / routes members");
    const void* ptrs[] = {x, w_router, logits, ws, out->topk_ids, out->topk_weights, out->expert_counts,
                          out->expert_offsets, out->perm, out->route_pos};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const size_t need = T > 0 ? moe::route_project_plan(T, H, E, k).ws_bytes : 0;
    if (ws_bytes < need || (need && !ws))
        return fail(MOE_ERR_WORKSPACE, "route_project workspace: need %zu bytes, got %zu", need, ws_bytes);
    out->T = T;
    out->E = E;
    out->k = k;
    const moe::RouteOut o{out->topk_ids, out->topk_weights, out->expert_counts, out->expert_offsets,
                          out->perm, out->route_pos};
    const int rc = hip_status(moe::launch_route_project(static_cast<const uint16_t*>(x), w_router, T, H, E, k,
                                                        logits, o, ws, static_cast<hipStream_t>(stream)),
                              "moe_route_project launch");
    return rc == MOE_OK ? ok() : rc;
}

static int pack_weights_impl(const void* w_gate_up, const void* w_down, int E, int H, int I, int quant,
                             void* packed_gate_up, void* packed_down, void* stream) {
    if (E < 1 || E > moe::kMaxExperts || H <= 0 || I <= 0)
        return fail(MOE_ERR_INVALID_ARG, "bad sizes E=%d H=%d I=%d", E, H, I);
    if (quant < MOE_BF16 || quant > MOE_FP8_MX32) return fail(MOE_ERR_INVALID_ARG, "unknown quant %d", quant);
    if (I % 16 != 0) return fail(MOE_ERR_UNSUPPORTED, "I must be a multiple of 16");
    if (quant == MOE_FP8_MX32 && (H % 256 != 0 || I % 256 != 0))
        return fail(MOE_ERR_UNSUPPORTED, "MX: H and I multiples of 256 (H=%d, I=%d)", H, I);
    if (!w_gate_up || !w_down || !packed_gate_up || !packed_down)
        return fail(MOE_ERR_INVALID_ARG, "null weight pointer");
    if (w_gate_up == packed_gate_up || w_down == packed_down)
        return fail(MOE_ERR_INVALID_ARG, "packing cannot run in place");
    const int elem = quant == MOE_BF16 ? 2 : 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc;
    if (quant == MOE_FP8_MX32) {
        rc = hip_status(moe::launch_pack_mx(w_gate_up, packed_gate_up, E, H, 2 * I, I, true, st), "pack gate_up");
        if (rc != MOE_OK) return rc;
        rc = hip_status(moe::launch_pack_mx(w_down, packed_down, E, I, H, I, false, st), "pack down");
        return rc == MOE_OK ? ok() : rc;
    }
    rc = hip_status(moe::launch_pack_gate_up(w_gate_up, packed_gate_up, E, H, I, elem, st), "pack gate_up");
    if (rc != MOE_OK) return rc;
    rc = hip_status(moe::launch_pack_down(w_down, packed_down, E, H, I, elem, st), "pack down");
    return rc == MOE_OK ? ok() : rc;
}

int moe_pack_weights(const void* w_gate_up, const void* w_down, int E, int H, int I, int quant,
                     void* packed_gate_up, void* packed_down, moe_packed_weights* packed, void* stream) {
    if (!packed) return fail(MOE_ERR_INVALID_ARG, "packed (the descriptor to fill) is NULL");
    packed->tag = 0;
    const int rc = pack_weights_impl(w_gate_up, w_down, E, H, I, quant, packed_gate_up, packed_down, stream);
    if (rc != MOE_OK) return rc;
    packed->gate_up = packed_gate_up;
    packed->down = packed_down;
    packed->E = E;
    packed->H = H;
    packed->I = I;
    packed->quant = quant;
    packed->tag = MOE_PACKED_TAG;
    return ok();
}

int moe_pack_mx_scales(const uint8_t* s_gate_up, const uint8_t* s_down, int E, int H, int I,
                       uint8_t* packed_s_gate_up, uint8_t* packed_s_down, void* stream) {
    if (E < 1 || E > moe::kMaxExperts || H <= 0 || I <= 0)
        return fail(MOE_ERR_INVALID_ARG, "bad sizes E=%d H=%d I=%d", E, H, I);
    if (H % 256 != 0 || I % 256 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "MX: H and I multiples of 256 (H=%d, I=%d)", H, I);
    if (!s_gate_up || !s_down || !packed_s_gate_up || !packed_s_down)
        return fail(MOE_ERR_INVALID_ARG, "null scale pointer");
    if (s_gate_up == packed_s_gate_up || s_down == packed_s_down)
        return fail(MOE_ERR_INVALID_ARG, "packing cannot run in place");
    if (!aligned16(packed_s_gate_up) || !aligned16(packed_s_down))
        return fail(MOE_ERR_INVALID_ARG, "packed scale pointers must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = hip_status(moe::launch_pack_mx_scales(s_gate_up, packed_s_gate_up, E, H, 2 * I, I, true, st),
                        "pack gate_up scales");
    if (rc != MOE_OK) return rc;
    rc = hip_status(moe::launch_pack_mx_scales(s_down, packed_s_down, E, I, H, I, false, st), "pack down scales");
    return rc == MOE_OK ? ok() : rc;
}

int moe_select_path(int T, int H, int I, int E, int k, int quant, int path) {
    const int rc = check_shape(T, H, I, E, k, quant);
    if (rc != MOE_OK) return rc;
    return resolve_path(T, H, I, E, k, quant, path);
}

size_t moe_forward_workspace_size(int T, int H, int I, int E, int k, int quant, int path) {
    if (check_shape(T, H, I, E, k, quant) != MOE_OK) return 0;
    const int p = resolve_path(T, H, I, E, k, quant, path);
    if (p < 0) return 0;
    return layout(T, H, I, E, k, quant, p).total;
}

int moe_forward_workspace_views(int T, int H, int I, int E, int k, int quant, int path, moe_ws_views* out) {
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    out->x_codes = out->x_scales = out->h_codes = out->h_scales = -1;
    int rc = check_shape(T, H, I, E, k, quant);
    if (rc != MOE_OK) return rc;
    const int p = resolve_path(T, H, I, E, k, quant, path);
    if (p < 0) return p;
    if (quant == MOE_BF16) return ok();
    const Layout L = layout(T, H, I, E, k, quant, p);
    auto off = [](size_t v) { return v == (size_t)-1 ? (int64_t)-1 : (int64_t)v; };
    out->x_codes = off(L.xq);
    out->x_scales = quant == MOE_FP8_PER_TENSOR ? off(L.scal) : off(L.sx);
    out->h_codes = p == MOE_PATH_GROUPED ? off(L.hq) : -1;
    out->h_scales = quant == MOE_FP8_PER_TENSOR ? off(L.scal) + (int64_t)sizeof(float) : off(L.sh);
    return ok();
}

int moe_forward_launch_info(int T, int H, int I, int E, int k, int quant, int path, moe_launch_info* out) {
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    *out = moe_launch_info{};
    int rc = check_shape(T, H, I, E, k, quant);
    if (rc != MOE_OK) return rc;
    const int p = resolve_path(T, H, I, E, k, quant, path);
    if (p < 0) return p;
    out->path = p;
    if (p == MOE_PATH_ROUTE_DIRECT) {
        const moe::RdLaunchInfo li = moe::rd_launch_info(T, H, I, k, quant);
        out->gate_up_split = li.gu_split;
        out->gate_up_waves = li.gu_waves;
        out->down_form = li.down_form;
        out->down_parts = li.down_parts;
    }
    return ok();
}

static int forward_impl(const void* x, const moe_routes* routes, const moe_packed_weights* w,
                        const moe_scales* scales, void* out, int H, int I,
                        int quant, int path, const moe_ep* ep, void* ws, size_t ws_bytes, void* stream,
                        void** events, int n_events, int* n_stages, const char** stage_names,
                        const float* logits = nullptr, void* ev_start = nullptr, void* ev_end = nullptr) {
    if (!routes) return fail(MOE_ERR_INVALID_ARG, "routes is NULL");
    const int T = routes->T, E = routes->E, k = routes->k;
    int rc = check_shape(T, H, I, E, k, quant);
    if (rc != MOE_OK) return rc;
    const int e0 = ep ? ep->expert_begin : 0, nloc = ep ? ep->num_experts : E, acc = ep ? ep->accumulate : 0;
    if (e0 < 0 || nloc < 1 || (long)e0 + nloc > E || (acc != 0 && acc != 1))
        return fail(MOE_ERR_INVALID_ARG, "expert slice [%d, %d+%d) must lie in [0, %d) and accumulate be 0 or 1",
                    e0, e0, nloc, E);
    // the packed weights must be the descriptor moe_pack_weights filled, for
    // this call's experts, shape and format (checked before anything launches)
    if (w && w->tag != MOE_PACKED_TAG)
        return fail(MOE_ERR_INVALID_ARG, "w was not filled by moe_pack_weights");
    if (w && (w->E != nloc || w->H != H || w->I != I || w->quant != quant))
        return fail(MOE_ERR_INVALID_ARG,
                    "weights packed for E=%d H=%d I=%d quant=%d, but the call has E=%d H=%d I=%d quant=%d",
                    w->E, w->H, w->I, w->quant, nloc, H, I, quant);
    const int p = resolve_path(T, H, I, E, k, quant, path);
    if (p < 0) return p;
    if (logits && p != MOE_PATH_ROUTE_DIRECT)
        return fail(MOE_ERR_UNSUPPORTED, "moe_decode_forward runs the route-direct path only (T=%d, E=%d, k=%d)", T, E, k);
    if (logits && T > 0 && !aligned16(logits)) return fail(MOE_ERR_INVALID_ARG, "logits must be 16-byte aligned");
    if (T == 0) {
        if (n_stages) *n_stages = 0;
        if (stage_names) *stage_names = "";
        return ok();
    }
    if (!w) return fail(MOE_ERR_INVALID_ARG, "w (the packed weights) is NULL");
    const void* packed_gate_up = w->gate_up;
    const void* packed_down = w->down;
    if (!x || !out || !packed_gate_up || !packed_down || !routes->topk_ids || !routes->topk_weights)
        return fail(MOE_ERR_INVALID_ARG, "null pointer among x / out / weights / routes");
    if (p == MOE_PATH_GROUPED && (!routes->expert_offsets || !routes->perm || !routes->route_pos))
        return fail(MOE_ERR_INVALID_ARG, "grouped path needs routes->expert_offsets, perm and route_pos");
    if (quant != MOE_BF16 && (!scales || !scales->w_gate_up_scale || !scales->w_down_scale))
        return fail(MOE_ERR_INVALID_ARG, "FP8 quantisation needs both weight scale arrays");
    const void* ptrs[] = {x, out, packed_gate_up, packed_down, routes->topk_ids, routes->topk_weights,
                          routes->expert_offsets, routes->perm, routes->route_pos, ws};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const Layout L = layout(T, H, I, E, k, quant, p);
    if (ws_bytes < L.total || !ws)
        return fail(MOE_ERR_WORKSPACE, "forward workspace: need %zu bytes, got %zu", L.total, ws_bytes);

    moe::FwdPlan P{};
    P.T = T; P.H = H; P.I = I; P.E = E; P.k = k; P.R = T * k; P.quant = quant;
    P.x = static_cast<const uint16_t*>(x);
    P.ids = routes->topk_ids;
    P.tw = routes->topk_weights;
    P.offsets = routes->expert_offsets;
    P.perm = routes->perm;
    P.route_pos = routes->route_pos;
    P.wgu = packed_gate_up;
    P.wd = packed_down;
    P.s_gu = quant != MOE_BF16 ? scales->w_gate_up_scale : nullptr;
    P.s_d = quant != MOE_BF16 ? scales->w_down_scale : nullptr;
    P.out = static_cast<uint16_t*>(out);
    P.tiles = at<int32_t>(ws, L.tiles);
    P.ntiles = at<int32_t>(ws, L.ntiles);
    P.amax = at<uint32_t>(ws, L.amax);
    P.scal = at<float>(ws, L.scal);
    P.xq = at<uint8_t>(ws, L.xq);
    P.sx = at<float>(ws, L.sx);
    P.h = at<void>(ws, L.h);
    P.hq = at<uint8_t>(ws, L.hq);
    P.sh = at<float>(ws, L.sh);
    P.y = at<uint16_t>(ws, L.y);
    P.rd_hmax = at<float>(ws, L.rd_hmax);
    P.rd_part = at<float>(ws, L.rd_part);
    P.rd_cnt = at<int32_t>(ws, L.rd_cnt);
    P.max_tiles = moe::grouped_max_tiles(P.R, E);
    P.e0 = e0;
    P.nloc = nloc;
    P.acc = acc;
    P.logits = logits;
    P.ids_w = logits ? routes->topk_ids : nullptr;
    P.tw_w = logits ? routes->topk_weights : nullptr;
    // Timing events are attached to kernel dispatches (hipExtLaunchKernel), so
    // no marker packet sits between two kernels: profiled calls put events[0]
    // on the first kernel's start and events[i] on the end of stage i's last
    // kernel; timed calls put ev_start on the first kernel's start and ev_end
    // on the last kernel's end.
    P.ev_first_start = static_cast<hipEvent_t>(events && n_events > 0 ? events[0] : ev_start);

    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool grouped = p == MOE_PATH_GROUPED;
    int stage = 0;
    static thread_local char names[256];
    names[0] = '\0';
    auto mark = [&](const char* name) {
        if (name) {
            if (names[0]) strncat(names, ",", sizeof names - strlen(names) - 1);
            strncat(names, name, sizeof names - strlen(names) - 1);
        }
        ++stage;
    };
    auto stage_end = [&](bool last) -> hipEvent_t {
        if (events) return stage < n_events ? static_cast<hipEvent_t>(events[stage]) : nullptr;
        return last ? static_cast<hipEvent_t>(ev_end) : nullptr;
    };
    mark(nullptr);
#define MOE_STEP(call, what, last)                                      \
    do {                                                                \
        P.ev_stage_end = stage_end(last);                               \
        if ((rc = hip_status((call), what)) != MOE_OK) return rc;       \
        mark(what);                                                     \
    } while (0)
    if (grouped) {
        MOE_STEP(moe::launch_forward_init(P, true, st), "init", false);
        if (quant != MOE_BF16) MOE_STEP(moe::launch_quant_x(P, st), "quant_x", false);
        MOE_STEP(moe::launch_grouped_gate_up(P, st), "gate_up", false);
        if (quant == MOE_FP8_PER_TENSOR) MOE_STEP(moe::launch_quant_h(P, st), "quant_h", false);
        MOE_STEP(moe::launch_grouped_down(P, st), "down", false);
        MOE_STEP(moe::launch_combine(P, st), "combine", true);
    } else {
        // FP8 quantises x and h inside the route-direct kernels (per tensor: from
        // all of x and the Gate/Up workgroups' h maxima; blockwise and MX: per
        // token or route row and 128 or 32 channels, in the workgroup that uses
        // them)
        MOE_STEP(moe::launch_route_direct_gate_up(P, st), "rd_gate_up", false);
        MOE_STEP(moe::launch_route_direct_down(P, st), "rd_down_combine", true);
    }
#undef MOE_STEP
    if (n_stages) *n_stages = stage - 1;
    if (stage_names) *stage_names = names;
    return ok();
}

int moe_forward(const void* x, const moe_routes* routes, const moe_packed_weights* w,
                const moe_scales* scales, void* out, int H, int I,
                int quant, int path, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(x, routes, w, scales, out, H, I, quant, path, nullptr, ws,
                        ws_bytes, stream, nullptr, 0, nullptr, nullptr);
}

int moe_forward_ex(const void* x, const moe_routes* routes, const moe_packed_weights* w,
                   const moe_scales* scales, void* out, int H, int I,
                   int quant, int path, const moe_ep* ep, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(x, routes, w, scales, out, H, I, quant, path, ep, ws,
                        ws_bytes, stream, nullptr, 0, nullptr, nullptr);
}

int moe_decode_forward(const float* logits, const void* x, int T, int E, int k, moe_routes* routes,
                       const moe_packed_weights* w, const moe_scales* scales, void* out,
                       int H, int I, int quant, int path, const moe_ep* ep, void* ws, size_t ws_bytes,
                       void* stream) {
    if (!routes) return fail(MOE_ERR_INVALID_ARG, "routes is NULL");
    if (T > 0 && !logits) return fail(MOE_ERR_INVALID_ARG, "logits is NULL");
    routes->T = T;
    routes->E = E;
    routes->k = k;
    return forward_impl(x, routes, w, scales, out, H, I, quant, path, ep, ws, ws_bytes,
                        stream, nullptr, 0, nullptr, nullptr, logits ? logits : nullptr);
}

int moe_forward_timed(const void* x, const moe_routes* routes, const moe_packed_weights* w,
                      const moe_scales* scales, void* out, int H, int I, int quant, int path, void* ws,
                      size_t ws_bytes, void* stream, void* ev_start, void* ev_end) {
    return forward_impl(x, routes, w, scales, out, H, I, quant, path, nullptr, ws, ws_bytes, stream, nullptr, 0,
                        nullptr, nullptr, nullptr, ev_start, ev_end);
}

int moe_forward_profiled(const void* x, const moe_routes* routes, const moe_packed_weights* w,
                         const moe_scales* scales, void* out, int H, int I,
                         int quant, int path, void* ws, size_t ws_bytes, void* stream,
                         void** stage_events, int n_events, int* n_stages, const char** stage_names) {
    if (n_events < 0 || (n_events > 0 && !stage_events))
        return fail(MOE_ERR_INVALID_ARG, "stage_events must hold n_events handles");
    return forward_impl(x, routes, w, scales, out, H, I, quant, path, nullptr, ws,
                        ws_bytes, stream, stage_events, n_events, n_stages, stage_names);
}

}  // extern "C"

// ------------------------------------------------------------ MX backward --

namespace {

bool train_shape_ok(int H, int I, int E) {
    return H > 0 && I > 0 && E >= 1 && E <= moe::kMaxExperts && H % 256 == 0 && I % 256 == 0 && H <= 8192 &&
           I <= 8192 && (long)E * H * 2 * I < (1L << 40);
}

struct TrainLayout {
    size_t gu_f, gu_f_s, gu_k, gu_k_s, d_k, d_k_s, d_t, d_t_s, gu_t, gu_t_s, total;
};

TrainLayout train_layout(int E, int H, int I) {
    TrainLayout L{};
    const size_t w = (size_t)E * H * I;   // elements of W_down; W_gate_up has 2w
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at_ = off;
        off += align256(bytes);
        return at_;
    };
    L.gu_f = take(2 * w);
    L.gu_f_s = take(2 * w / 32);
    L.gu_k = take(2 * w);
    L.gu_k_s = take(2 * w / 32);
    L.d_k = take(w);
    L.d_k_s = take(w / 32);
    L.d_t = take(w);
    L.d_t_s = take(w / 32);
    L.gu_t = take(2 * w);
    L.gu_t_s = take(2 * w / 32);
    L.total = off;
    return L;
}

struct BwdLayout {
    size_t tiles, ntiles, amax, xq, sx, gu, h32, hq, sh, y, dyq, sdy, dh, dgu, dguq, sdgu, ones, poff, seg;
    size_t xT, sxT, dguT, sdguT, hT, shT, dyT, sdyT, total;
    long Rp;
};

// padded route positions of the weight-gradient operands: every expert's
// segment rounded up to 64, in whole 256-position scale-dword groups
long bwd_padded_routes(long R, int E) { return (R + 63L * E + 255) / 256 * 256; }

BwdLayout bwd_layout(int T, int H, int I, int E, int k) {
    BwdLayout L{};
    const size_t R = (size_t)T * k;
    L.Rp = bwd_padded_routes((long)R, E);
    const size_t Rp = (size_t)L.Rp, Rb = Rp / 32;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at_ = off;
        off += align256(bytes);
        return bytes ? at_ : (size_t)-1;
    };
    L.tiles = take(sizeof(int32_t) * 2 * (size_t)moe::grouped_max_tiles((int)R, E));
    L.ntiles = take(sizeof(int32_t));
    L.amax = take(2 * sizeof(uint32_t));
    L.xq = take((size_t)T * H);
    L.sx = take((size_t)T * (H / 32));
    L.gu = take(R * 2 * I * 4);
    L.h32 = take(R * I * 4);
    L.hq = take(R * I);
    L.sh = take(R * (I / 32));
    L.y = take(R * H * 2);          // the recomputed Down output, then the rows of dx (both bf16)
    L.dyq = take(R * H);
    L.sdy = take(R * (H / 32));
    L.dh = take(R * I * 4);
    L.dgu = take(R * 2 * I * 4);
    L.dguq = take(R * 2 * I);
    L.sdgu = take(R * (2 * I / 32));
    L.ones = take(R * 4);
    L.poff = take(sizeof(int32_t) * (size_t)(E + 1));
    L.seg = take(sizeof(int32_t) * (size_t)(L.Rp / 64));
    L.xT = take((size_t)H * Rp);
    L.sxT = take((size_t)H * Rb);
    L.dguT = take((size_t)2 * I * Rp);
    L.sdguT = take((size_t)2 * I * Rb);
    L.hT = take((size_t)I * Rp);
    L.shT = take((size_t)I * Rb);
    L.dyT = take((size_t)H * Rp);
    L.sdyT = take((size_t)H * Rb);
    L.total = off;
    return L;
}

int check_train_shape(int T, int H, int I, int E, int k) {
    if (T < 0 || k < 1 || E < k || E > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "need T >= 0 and 1 <= k <= E <= %d (T=%d k=%d E=%d)", moe::kMaxExperts, T, k,
                    E);
    if (!train_shape_ok(H, I, E))
        return fail(MOE_ERR_UNSUPPORTED, "MX backward: H and I multiples of 256 up to 8192 (H=%d, I=%d)", H, I);
    const long R = (long)T * k;
    if (R >= (1L << 31) || (long)T * H >= (1L << 31) || R * 2 * I >= (1L << 31) || R * H >= (1L << 31))
        return fail(MOE_ERR_UNSUPPORTED, "MX backward: T*k*H and T*k*2I must stay below 2^31");
    if ((long)H * bwd_padded_routes(R, E) >= (1L << 40))
        return fail(MOE_ERR_UNSUPPORTED, "MX backward: transposed operands too large");
    return MOE_OK;
}

int backward_impl(const void* x, const moe_routes* routes, const moe_mx_train_weights* w, const void* dout,
                  void* dx, float* dgate, void* dw_gate_up, void* dw_down, void* ws, size_t ws_bytes, void* stream,
                  void** events, int n_events, int* n_stages, const char** stage_names) {
    if (!routes || !w) return fail(MOE_ERR_INVALID_ARG, "routes or w is NULL");
    const int T = routes->T, E = routes->E, k = routes->k, H = w->H, I = w->I;
    int rc = check_train_shape(T, H, I, E, k);
    if (rc != MOE_OK) return rc;
    if (w->tag != MOE_TRAIN_TAG) return fail(MOE_ERR_INVALID_ARG, "w was not filled by moe_prepare_mx_train_weights");
    if (w->E != E) return fail(MOE_ERR_INVALID_ARG, "weights prepared for E=%d, routes have E=%d", w->E, E);
    if (!dw_gate_up || !dw_down || !routes->expert_offsets)
        return fail(MOE_ERR_INVALID_ARG, "null pointer among dw_gate_up / dw_down / routes->expert_offsets");
    if (T > 0 && (!x || !dout || !dx || !dgate || !routes->topk_weights || !routes->perm || !routes->route_pos))
        return fail(MOE_ERR_INVALID_ARG, "null pointer among x / dout / dx / dgate / routes");
    const void* ptrs[] = {x, dout, dx, dgate, dw_gate_up, dw_down, routes->topk_weights, routes->expert_offsets,
                          routes->perm, routes->route_pos, ws};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const BwdLayout L = bwd_layout(T, H, I, E, k);
    if (ws_bytes < L.total || !ws)
        return fail(MOE_ERR_WORKSPACE, "backward workspace: need %zu bytes, got %zu", L.total, ws_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const long R = (long)T * k, Rp = L.Rp, Rb = Rp / 32;
    int32_t* poff = at<int32_t>(ws, L.poff);
    int32_t* seg = at<int32_t>(ws, L.seg);

    int stage = 0;
    static thread_local char names[256];
    names[0] = '\0';
    auto ev = [&]() -> hipEvent_t {
        return events && stage + 1 < n_events ? static_cast<hipEvent_t>(events[stage + 1]) : nullptr;
    };
    auto mark = [&](const char* name) {
        if (names[0]) strncat(names, ",", sizeof names - strlen(names) - 1);
        strncat(names, name, sizeof names - strlen(names) - 1);
        ++stage;
    };
#define MOE_BSTEP(call, what)                                           \
    do {                                                                \
        if ((rc = hip_status((call), what)) != MOE_OK) return rc;       \
        mark(what);                                                     \
    } while (0)

    moe::FwdPlan P{};
    P.T = T; P.H = H; P.I = I; P.E = E; P.k = k; P.R = (int)R; P.quant = MOE_FP8_MX32;
    P.x = static_cast<const uint16_t*>(x);
    P.ids = routes->topk_ids;
    P.tw = at<float>(ws, L.ones);
    P.offsets = routes->expert_offsets;
    P.perm = routes->perm;
    P.route_pos = routes->route_pos;
    P.out = static_cast<uint16_t*>(dx);
    P.tiles = at<int32_t>(ws, L.tiles);
    P.ntiles = at<int32_t>(ws, L.ntiles);
    P.amax = at<uint32_t>(ws, L.amax);
    P.xq = at<uint8_t>(ws, L.xq);
    P.sx = at<float>(ws, L.sx);
    P.y = at<uint16_t>(ws, L.y);   // (the combine reads the bf16 rows of dx there)
    P.max_tiles = moe::grouped_max_tiles((int)R, E);
    P.e0 = 0;
    P.nloc = E;
    P.acc = 0;
    P.ev_first_start = static_cast<hipEvent_t>(events && n_events > 0 ? events[0] : nullptr);

    float* gu = at<float>(ws, L.gu);
    float* h32 = at<float>(ws, L.h32);
    uint8_t* hq = at<uint8_t>(ws, L.hq);
    uint8_t* sh = at<uint8_t>(ws, L.sh);
    uint8_t* dyq = at<uint8_t>(ws, L.dyq);
    uint8_t* sdy = at<uint8_t>(ws, L.sdy);
    float* dh = at<float>(ws, L.dh);
    float* dgu = at<float>(ws, L.dgu);
    uint8_t* dguq = at<uint8_t>(ws, L.dguq);
    uint8_t* sdgu = at<uint8_t>(ws, L.sdgu);
    const uint16_t* dout16 = static_cast<const uint16_t*>(dout);

    if (R > 0) {
        P.ev_stage_end = ev();
        MOE_BSTEP(moe::launch_forward_init(P, true, st), "init");
        P.ev_first_start = nullptr;
        P.ev_stage_end = ev();
        MOE_BSTEP(moe::launch_quant_x(P, st), "quant_x");
        auto product = [&](const uint8_t* A, const uint8_t* sa, long a_rows, int K, int N, const void* B,
                           const uint8_t* swx, bool gather, void* C, bool f32) {
            moe::MxProduct q{};
            q.A = A; q.sa = sa; q.a_rows = a_rows; q.K = K; q.N = N;
            q.B = static_cast<const uint8_t*>(B); q.swx = swx; q.gather = gather;
            q.perm = routes->perm; q.k = k; q.tiles = P.tiles; q.ntiles = P.ntiles; q.offsets = P.offsets;
            q.max_tiles = P.max_tiles; q.C = C; q.out_f32 = f32; q.R = R; q.ev_end = ev();
            return moe::launch_grouped_mx_y(q, st);
        };
        // forward recomputation: [g | u] = x W_gate_up, h, y = h W_down
        MOE_BSTEP(product(P.xq, reinterpret_cast<const uint8_t*>(P.sx), T, H, 2 * I, w->gate_up_k,
                          w->gate_up_k_scales, true, gu, true),
                  "gate_up");
        MOE_BSTEP(moe::launch_swiglu_fwd(gu, R, I, h32, hq, sh, ev(), st), "swiglu");
        MOE_BSTEP(product(hq, sh, R, I, H, w->down_k, w->down_k_scales, false, P.y, false), "down");
        // dy = gate * dout, the gates' gradient, dh = dy W_down^T
        MOE_BSTEP(moe::launch_dy(dout16, routes->topk_weights, routes->perm, k, P.y, R, H, dyq, sdy, dgate, ev(), st),
                  "dy");
        MOE_BSTEP(product(dyq, sdy, R, H, I, w->down_t, w->down_t_scales, false, dh, true), "dh");
        MOE_BSTEP(moe::launch_swiglu_bwd(gu, dh, R, I, dgu, dguq, sdgu, ev(), st), "swiglu_bwd");
        // dx rows = dGU W_gate_up^T (into y's space), summed per token with unit weights
        MOE_BSTEP(product(dguq, sdgu, R, 2 * I, H, w->gate_up_t, w->gate_up_t_scales, false, P.y, false), "dx_rows");
        if ((rc = hip_status(moe::launch_fill_f32(at<float>(ws, L.ones), R, 1.0f, st), "fill")) != MOE_OK) return rc;
        P.ev_stage_end = ev();
        MOE_BSTEP(moe::launch_combine(P, st), "combine");
    }
    // weight gradients: each expert's routes padded to 64 (offsets built here),
    // the four operands cast along the routes, then the per-expert products
    if ((rc = hip_status(moe::launch_pad_offsets(routes->expert_offsets, E, poff, seg, (int)(Rp / 64), st), "pad_offsets")) != MOE_OK)
        return rc;
    uint8_t* xT = at<uint8_t>(ws, L.xT);
    uint8_t* sxT = at<uint8_t>(ws, L.sxT);
    uint8_t* dguT = at<uint8_t>(ws, L.dguT);
    uint8_t* sdguT = at<uint8_t>(ws, L.sdguT);
    uint8_t* hT = at<uint8_t>(ws, L.hT);
    uint8_t* shT = at<uint8_t>(ws, L.shT);
    uint8_t* dyT = at<uint8_t>(ws, L.dyT);
    uint8_t* sdyT = at<uint8_t>(ws, L.sdyT);
    if (R > 0) {
        const int32_t* offs = routes->expert_offsets;
        const float* tw = routes->topk_weights;
        if ((rc = hip_status(moe::launch_dim1(0, x, nullptr, nullptr, routes->perm, k, offs, poff, seg, E, H, Rp, Rp, Rb,
                                              xT, sxT, nullptr, st), "dim1 x")) != MOE_OK)
            return rc;
        if ((rc = hip_status(moe::launch_dim1(2, dgu, nullptr, nullptr, routes->perm, k, offs, poff, seg, E, 2 * I, Rp, Rp,
                                              Rb, dguT, sdguT, nullptr, st), "dim1 dGU")) != MOE_OK)
            return rc;
        if ((rc = hip_status(moe::launch_dim1(2, h32, nullptr, nullptr, routes->perm, k, offs, poff, seg, E, I, Rp, Rp, Rb,
                                              hT, shT, nullptr, st), "dim1 h")) != MOE_OK)
            return rc;
        MOE_BSTEP(moe::launch_dim1(1, nullptr, dout16, tw, routes->perm, k, offs, poff, seg, E, H, Rp, Rp, Rb, dyT, sdyT,
                                   ev(), st),
                  "dim1");
    }
    MOE_BSTEP(moe::launch_wgrad(xT, sxT, dguT, sdguT, Rp, Rb, poff, E, H, 2 * I, static_cast<uint16_t*>(dw_gate_up),
                                ev(), st),
              "wgrad_gate_up");
    MOE_BSTEP(moe::launch_wgrad(hT, shT, dyT, sdyT, Rp, Rb, poff, E, I, H, static_cast<uint16_t*>(dw_down), ev(), st),
              "wgrad_down");
#undef MOE_BSTEP
    if (n_stages) *n_stages = stage;
    if (stage_names) *stage_names = names;
    return ok();
}

}  // namespace

extern "C" {

size_t moe_mx_train_weights_size(int E, int H, int I) {
    if (!train_shape_ok(H, I, E)) return 0;
    return train_layout(E, H, I).total;
}

int moe_prepare_mx_train_weights(const void* w_gate_up, const void* w_down, int E, int H, int I, void* buf,
                                 size_t buf_bytes, moe_mx_train_weights* out, void* stream) {
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    out->tag = 0;
    out->forward.tag = 0;
    if (!train_shape_ok(H, I, E))
        return fail(MOE_ERR_UNSUPPORTED, "MX backward: H and I multiples of 256 up to 8192, 1 <= E <= %d",
                    moe::kMaxExperts);
    if (!w_gate_up || !w_down || !buf) return fail(MOE_ERR_INVALID_ARG, "null pointer among weights / buf");
    if (!aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(buf))
        return fail(MOE_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const TrainLayout L = train_layout(E, H, I);
    if (buf_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "need %zu bytes, got %zu", L.total, buf_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* b = static_cast<uint8_t*>(buf);
    const uint16_t* wgu = static_cast<const uint16_t*>(w_gate_up);
    const uint16_t* wd = static_cast<const uint16_t*>(w_down);
    // (src, K, N, along_k) -> the packed set (N rows of K) and its packed scales, one pass
    auto one = [&](const uint16_t* src, int K, int N, bool along_k, size_t dst, size_t dst_s) -> int {
        return hip_status(moe::launch_mx_pack_weights(src, E, K, N, along_k, false, b + dst, b + dst_s, nullptr,
                                                      nullptr, st),
                          "mx pack");
    };
    int rc;
    // W_gate_up along H, once: the forward's interleaved set and the plain set of the recomputation
    if ((rc = hip_status(moe::launch_mx_pack_weights(wgu, E, H, 2 * I, true, true, b + L.gu_f, b + L.gu_f_s,
                                                     b + L.gu_k, b + L.gu_k_s, st),
                         "mx pack")) != MOE_OK)
        return rc;
    if ((rc = one(wd, I, H, true, L.d_k, L.d_k_s)) != MOE_OK) return rc;            // forward Down: along I
    if ((rc = one(wd, H, I, false, L.d_t, L.d_t_s)) != MOE_OK) return rc;           // W_down^T: along H
    if ((rc = one(wgu, 2 * I, H, false, L.gu_t, L.gu_t_s)) != MOE_OK) return rc;    // W_gate_up^T: along 2I
    out->gate_up_k = b + L.gu_k;
    out->gate_up_k_scales = b + L.gu_k_s;
    out->down_k = b + L.d_k;
    out->down_k_scales = b + L.d_k_s;
    out->down_t = b + L.d_t;
    out->down_t_scales = b + L.d_t_s;
    out->gate_up_t = b + L.gu_t;
    out->gate_up_t_scales = b + L.gu_t_s;
    out->E = E;
    out->H = H;
    out->I = I;
    // the MX forward's weights: the interleaved Gate/Up set and the Down set
    out->forward.gate_up = b + L.gu_f;
    out->forward.down = b + L.d_k;
    out->forward.E = E;
    out->forward.H = H;
    out->forward.I = I;
    out->forward.quant = MOE_FP8_MX32;
    out->forward.tag = MOE_PACKED_TAG;
    out->forward_scales.w_gate_up_scale = reinterpret_cast<const float*>(b + L.gu_f_s);
    out->forward_scales.w_down_scale = reinterpret_cast<const float*>(b + L.d_k_s);
    out->tag = MOE_TRAIN_TAG;
    return ok();
}

size_t moe_backward_workspace_size(int T, int H, int I, int E, int k) {
    if (check_train_shape(T, H, I, E, k) != MOE_OK) return 0;
    return bwd_layout(T, H, I, E, k).total;
}

int moe_backward(const void* x, const moe_routes* routes, const moe_mx_train_weights* w, const void* dout, void* dx,
                 float* dgate, void* dw_gate_up, void* dw_down, void* ws, size_t ws_bytes, void* stream) {
    return backward_impl(x, routes, w, dout, dx, dgate, dw_gate_up, dw_down, ws, ws_bytes, stream, nullptr, 0,
                         nullptr, nullptr);
}

int moe_route_backward(const moe_routes* routes, const float* dgate, float* dlogits, void* stream) {
    if (!routes) return fail(MOE_ERR_INVALID_ARG, "routes is NULL");
    const int T = routes->T, E = routes->E, k = routes->k;
    if (T < 0 || k < 1 || E < k || E > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "need T >= 0 and 1 <= k <= E <= %d (T=%d k=%d E=%d)", moe::kMaxExperts, T, k,
                    E);
    if ((long)T * E >= (1L << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*E must fit in int32");
    if (T == 0) return ok();
    if (!dgate || !dlogits || !routes->topk_ids || !routes->topk_weights)
        return fail(MOE_ERR_INVALID_ARG, "null pointer among dgate / dlogits / routes");
    const void* ptrs[] = {dgate, dlogits, routes->topk_ids, routes->topk_weights};
    for (const void* q : ptrs)
        if (!aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const int rc = hip_status(moe::launch_route_grad(routes->topk_ids, routes->topk_weights, dgate, T, E, k, dlogits,
                                                     static_cast<hipStream_t>(stream)),
                              "moe_route_backward launch");
    return rc == MOE_OK ? ok() : rc;
}

int moe_backward_profiled(const void* x, const moe_routes* routes, const moe_mx_train_weights* w, const void* dout,
                          void* dx, float* dgate, void* dw_gate_up, void* dw_down, void* ws, size_t ws_bytes,
                          void* stream, void** events, int n_events, int* n_stages, const char** stage_names) {
    return backward_impl(x, routes, w, dout, dx, dgate, dw_gate_up, dw_down, ws, ws_bytes, stream, events, n_events,
                         n_stages, stage_names);
}

}  // extern "C"
