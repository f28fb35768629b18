/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE FFN forward library.
 *
 * The library computes the forward pass of a token-choice Mixture-of-Experts
 * SwiGLU FFN layer on one GPU:
 *
 *   routing   top-k over the router logits, softmax gates renormalised over the
 *             k picks, then the routes grouped by expert: per-expert counts,
 *             their exclusive prefix and a stable permutation of route ids
 *             ("Port necessary FBGEMM MoE kernels", Summary: index_shuffling;
 *              "perf: add small-batch route MMA for MoE", Motivation:
 *              count/sort and prefix of the grouped pipeline);
 *   forward   Gate/Up projection, SwiGLU, optional FP8 requantisation, Down
 *             projection and the top-k weighted combine, either over the
 *             expert-grouped routes (grouped GEMMs) or straight from the routes
 *             for small decode batches ("perf: add small-batch route MMA for
 *             MoE", Summary, Motivation and Dispatch);
 *   also      router scores x W_r fused with the routing (moe_route_project),
 *             an expert slice and a shared output (moe_forward_ex), a decode
 *             batch with the routing folded into its first kernel
 *             (moe_decode_forward), and MX FP8 weights (MOE_FP8_MX32,
 *             moe_pack_mx_scales).
 *
 * Conventions for every entry point:
 *   - Every pointer is a device pointer (HIP global memory of the current
 *     device) unless stated otherwise; every buffer is allocated and owned by
 *     the caller.  The library never allocates or frees device memory, never
 *     synchronises the stream and never copies device data to the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued on it in order, so calls can be captured in a HIP
 *     graph.
 *   - Return value: MOE_OK (0) or a negative moe_status.  On error nothing has
 *     been enqueued (argument checks run before any launch) except for
 *     MOE_ERR_HIP, which reports a failed launch.  moe_last_error() gives a
 *     message for the calling thread's last error.
 *   - Device contents are never validated (that would need a synchronisation):
 *     routes that moe_route did not produce (for example ids >= E) give
 *     undefined results.
 *   - Pointers must be 16-byte aligned.
 *   - Calls that share a workspace must be ordered on one stream (or
 *     otherwise not run at the same time).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, k > E, negative sizes, ... */
    MOE_ERR_UNSUPPORTED = -2,   /* shape or quantisation the library does not handle */
    MOE_ERR_WORKSPACE = -3,     /* workspace smaller than the *_workspace_size query */
    MOE_ERR_HIP = -4            /* a kernel launch failed */
} moe_status;

typedef enum {
    MOE_BF16 = 0,               /* bf16 x and weights, fp32 accumulation */
    MOE_FP8_PER_TENSOR = 1,     /* e4m3 weights with one fp32 scale per expert tensor;
                                   x and h quantised on device with one scale each */
    MOE_FP8_BLOCK128 = 2,       /* e4m3 weights with fp32 scales per 128x128 block;
                                   x and h quantised per row per 128 channels */
    MOE_FP8_MX32 = 3            /* MX: e4m3 weights with one E8M0 (power-of-two) scale
                                   per 32 rows of K per output column; x and h
                                   quantised per row per 32 channels; grouped path
                                   only, H and I multiples of 256 */
} moe_quant;

typedef enum {
    MOE_PATH_AUTO = 0,          /* the dispatch rule picks (see moe_select_path) */
    MOE_PATH_GROUPED = 1,       /* sort by expert, grouped MFMA GEMMs */
    MOE_PATH_ROUTE_DIRECT = 2   /* per-route weight streaming, no sort or gather */
} moe_path;

/* Routes of T tokens over E experts, k per token.  Device arrays, int32 unless
 * noted, all caller-allocated:
 *   topk_ids       [T,k]  slot j = the j-th largest logit; equal logits (exact
 *                         fp32 equality, -0 == +0) go to the lower expert id
 *   topk_weights   [T,k]  fp32 gates: softmax over all E renormalised over the
 *                         k picks (= exp(l_j - max) / sum over picks)
 *   expert_counts  [E]    routes per expert
 *   expert_offsets [E+1]  exclusive prefix of the counts; offsets[E] = T*k
 *   perm           [T*k]  route ids r = t*k + j ordered by (expert, r)
 *   route_pos      [T*k]  inverse of perm: perm[route_pos[r]] = r           */
typedef struct {
    int32_t *topk_ids;
    float *topk_weights;
    int32_t *expert_counts;
    int32_t *expert_offsets;
    int32_t *perm;
    int32_t *route_pos;
    int32_t T, E, k;
} moe_routes;

/* FP8 weight scales (device arrays; NULL members for MOE_BF16):
 *   per-tensor: fp32 w_gate_up_scale [E], w_down_scale [E]
 *   block128:   fp32 w_gate_up_scale [E][H/128][2I/128], w_down_scale [E][I/128][H/128]
 *               (the layout of the unpacked weights)
 *   MX:         E8M0 bytes re-laid by moe_pack_mx_scales (the members point to
 *               those bytes; the float type is only the struct's) */
typedef struct {
    const float *w_gate_up_scale;
    const float *w_down_scale;
} moe_scales;

/* Bytes of workspace moe_route needs (0 is a valid answer: pass ws = NULL). */
size_t moe_route_workspace_size(int T, int E, int k);

/* Routing ("perf: add small-batch route MMA for MoE", Summary: routes are
 * token/top-k; "Port necessary FBGEMM MoE kernels", Summary: index_shuffling).
 * logits: fp32 [T,E], row-major.  Requires 1 <= k <= E <= 512, T >= 0 and
 * T*k < 2^31; out->T/E/k are set by this call.  T = 0 writes zero counts and
 * offsets.  NaN logits are not supported. */
int moe_route(const float *logits, int T, int E, int k, moe_routes *out,
              void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace moe_route_project needs (> 0 for T > 0). */
size_t moe_route_project_workspace_size(int T, int H, int E, int k);

/* Router scores and routing in one call: logits = x W_r, then exactly what
 * moe_route computes from those logits.  The pages route every token by the
 * top-k of its per-expert scores ("Port necessary FBGEMM MoE kernels",
 * Benchmarks: the MoE module of 16 experts, top 8) without printing the
 * router; here it is a bias-free linear map.
 *   x        bf16 [T,H] row-major; H a positive multiple of 64
 *   w_router fp32 [H,E] row-major
 *   logits   fp32 [T,E], written: sum over h of x[t,h] * w_router[h,e] in
 *            fp32, in an order fixed by (T, H, E) -- repeated calls give the
 *            same bits; the routes are taken from exactly these values
 *   out      as for moe_route (out->T/E/k are set by this call)
 * For small T the scores and the routing run in one launch: its workgroups
 * meet through an arrival counter in the first 256 bytes of ws, which must be
 * zero before the first call with a given workspace (e.g. zero-filled when
 * allocated); every call leaves it zero.  Calls that share a workspace must
 * not run concurrently.  T = 0 writes zero counts and offsets only. */
int moe_route_project(const void *x, const float *w_router, int T, int H, int E, int k,
                      float *logits, moe_routes *out, void *ws, size_t ws_bytes, void *stream);

/* Expert weights as moe_pack_weights re-laid them, with the shape and format
 * they were packed for.  moe_pack_weights fills every member; the forward
 * entry points compare E, H, I, quant and tag with the call (E: the routes'
 * E, or the slice's num_experts) and return MOE_ERR_INVALID_ARG on any
 * mismatch before anything is enqueued, so raw [E,H,2I] / [E,I,H] weights or
 * weights packed for another shape cannot reach the kernels by mistake.  The
 * struct lives in host memory; the two buffers stay owned by the caller. */
#define MOE_PACKED_TAG 0x4d6f4557u
typedef struct {
    const void *gate_up;   /* device: packed Gate/Up weights (E*H*2I elements) */
    const void *down;      /* device: packed Down weights (E*I*H elements) */
    int32_t E, H, I;       /* the packed shape */
    int32_t quant;         /* moe_quant the weights were packed for */
    uint32_t tag;          /* MOE_PACKED_TAG once moe_pack_weights succeeded */
} moe_packed_weights;

/* Weight re-layout, once per weight set (not per forward call).
 *   w_gate_up [E][H][2I] (gate = columns [0,I), up = columns [I,2I)) and
 *   w_down [E][I][H], bf16 (2 bytes) or e4m3 codes (1 byte), row-major
 * -> packed_gate_up and packed_down, each the same size as its source, K
 * (the reduction dimension) contiguous, gate and up columns interleaved in
 * groups of 16.  The forward entry points read only the packed form, through
 * the descriptor `packed` this call fills (host memory, not NULL; on error its
 * tag is cleared).  Scales are not re-laid out (MX: moe_pack_mx_scales). */
int moe_pack_weights(const void *w_gate_up, const void *w_down, int E, int H, int I,
                     int quant, void *packed_gate_up, void *packed_down,
                     moe_packed_weights *packed, void *stream);

/* MX scale re-layout, once per weight set ("[mxfp8 moe training] add per group
 * blocked scale kernels", Summary: scales re-laid for the block-scaled matrix
 * instruction on device).
 *   s_gate_up [E][H/32][2I] and s_down [E][I/32][H]: E8M0 bytes, one per 32
 *   rows of K and output column (2^(b-127)), the layout of the unpacked weights
 * -> packed_s_gate_up, packed_s_down, each the same size as its source, the
 * order in which the MX GEMM feeds its scaled MFMAs.  H and I multiples of 256. */
int moe_pack_mx_scales(const uint8_t *s_gate_up, const uint8_t *s_down, int E, int H, int I,
                       uint8_t *packed_s_gate_up, uint8_t *packed_s_down, void *stream);

/* The path MOE_PATH_AUTO takes for this shape, or a negative moe_status if
 * the requested path cannot run it.  Host-only; no GPU call.
 * ("perf: add small-batch route MMA for MoE", Dispatch.)  AUTO takes the
 * route-direct path while T*k <= 3E/4 and T <= 16 and the shape fits it
 * (the bound measured on MI355X with both paths forced), else grouped; the
 * same rule for every quantisation, MX included. */
int moe_select_path(int T, int H, int I, int E, int k, int quant, int path);

/* Bytes of workspace moe_forward needs for this shape, quantisation and path. */
size_t moe_forward_workspace_size(int T, int H, int I, int E, int k, int quant, int path);

/* Where a forward call leaves its FP8 quantised activations in the workspace,
 * as byte offsets from ws (-1 where the call keeps no such array).  After a
 * moe_forward / moe_forward_ex / moe_decode_forward call with this shape,
 * quantisation and path, and until the next call that uses the workspace:
 *   x_codes   e4m3 [T,H], the codes the Gate/Up projection consumed (both paths;
 *             route-direct: rows of tokens with a route into the call's
 *             expert slice, or every row with the routing folded in)
 *   x_scales  per-tensor fp32 [1]; block128 fp32 [T,H/128]; MX E8M0 bytes
 *             [T,H/32], group c of a row at byte 8(c/8) + 4(c%2) + (c%8)/2
 *   h_codes   grouped path: e4m3 [T*k,I], row i = the route at sorted position i
 *   h_scales  per-tensor fp32 [1] (both paths); block128 fp32 [T*k,I/128],
 *             sorted order (grouped) or route order r = t*k + j (route-direct);
 *             MX E8M0 [T*k,I/32], sorted order (grouped) or route order
 *             (route-direct), bytes ordered as x_scales
 * ("perf: add small-batch route MMA for MoE", Summary: the activation and
 * Down-input quantisation; exposed so callers and tests can inspect the
 * codes.)  bf16 has none of them.  Returns MOE_OK or the shape's error. */
typedef struct {
    int64_t x_codes, x_scales, h_codes, h_scales;
} moe_ws_views;
int moe_forward_workspace_views(int T, int H, int I, int E, int k, int quant, int path, moe_ws_views *out);

/* The launch shape a forward call with these arguments takes (host-only; the
 * route-direct shape depends on the current device's occupancy figures, so
 * call it with the device the forward will run on current):
 *   path            MOE_PATH_GROUPED or MOE_PATH_ROUTE_DIRECT
 *   gate_up_split   route-direct: workgroups sharing one 32-row block pair of
 *                   the Gate/Up weights (1, 2 or 4); 0 on the grouped path
 *   gate_up_waves   route-direct: waves per Gate/Up workgroup
 *   down_form       route-direct: 0 = K split over workgroups with a
 *                   last-arriver sum, 1 = one workgroup per output block
 *   down_parts      route-direct: K parts per route slot of the Down step
 * ("perf: add small-batch route MMA for MoE", Dispatch: the fast path's
 * launch depends on the shape.) */
typedef struct {
    int32_t path, gate_up_split, gate_up_waves, down_form, down_parts;
} moe_launch_info;
int moe_forward_launch_info(int T, int H, int I, int E, int k, int quant, int path, moe_launch_info *out);

/* Layer forward ("perf: add small-batch route MMA for MoE", Motivation and
 * Summary; "Port necessary FBGEMM MoE kernels", Summary: scatter_add):
 *   out[t] = sum_j topk_weights[t,j] * FFN_{topk_ids[t,j]}(x[t])
 *   FFN_e(v) = (silu(v W_gate[e]) * (v W_up[e])) W_down[e]
 * x: bf16 [T,H]; out: bf16 [T,H], fully overwritten; routes: from moe_route
 * (same T, E, k); w: the descriptor moe_pack_weights filled (its E, H, I and
 * quant must equal the routes' E and this call's H, I and quant).
 * FP8: x is quantised on device (per-tensor: one scale amax/448 for all of x;
 * block128: per token per 128 channels; MX: per token per 32 channels, E8M0
 * scale 2^(floor(log2 amax) - 8)); the SwiGLU output h is requantised the
 * same way before Down (per-tensor: one scale for all T*k rows).
 * The combine sums the k routes of a token in a fixed order in fp32 and
 * rounds to bf16 once: repeated calls give identical bits.
 * Shapes: H % 64 == 0, I % 64 == 0 (block128: both % 128; MX: both % 256); T*H < 2^31
 * and T*k*I < 2^36 (the grouped path addresses x with 32-bit offsets and
 * every sorted-row buffer -- h, y -- from a 64-bit base per row tile, so
 * intermediates of many GiB are fine); the route-direct path also needs
 * H*elem <= 8192 bytes and I*elem <= 2048 bytes.  Shapes outside these limits
 * give MOE_ERR_UNSUPPORTED before anything is enqueued. */
int moe_forward(const void *x, const moe_routes *routes, const moe_packed_weights *w,
                const moe_scales *scales, void *out, int H, int I,
                int quant, int path, void *ws, size_t ws_bytes, void *stream);

/* Expert-parallel slice and shared output for moe_forward_ex ("perf: add
 * small-batch route MMA for MoE", Summary: the fast path preserves EP
 * routing and shared output).  The routes stay global (moe_route over all E
 * experts); this call holds experts [expert_begin, expert_begin +
 * num_experts) only -- the packed weights (packed with E = num_experts) and
 * the scales cover exactly those, expert expert_begin + i at index i -- and
 * computes only the
 * routes to them:
 *   sum[t] = sum over j with topk_ids[t,j] in the slice of
 *            topk_weights[t,j] * FFN_{topk_ids[t,j]}(x[t])
 * FP8 per-tensor: the h scale is the amax over this call's routes (the only
 * h it sees); x's scale still covers all of x.
 * accumulate 0: out = bf16(sum); 1: out = bf16(out + sum), one rounding (a
 * shared output, e.g. the partial sums of several expert slices). */
typedef struct {
    int32_t expert_begin;   /* >= 0 */
    int32_t num_experts;    /* >= 1, expert_begin + num_experts <= routes->E */
    int32_t accumulate;     /* 0 or 1 */
} moe_ep;

/* moe_forward for an expert slice and/or into a shared output; ep may be
 * NULL (all experts, out overwritten: exactly moe_forward).  The workspace
 * is moe_forward_workspace_size with the routes' E.  AUTO picks the path
 * from the routes' T, E and k as for moe_forward.  Invalid ep fields give
 * MOE_ERR_INVALID_ARG. */
int moe_forward_ex(const void *x, const moe_routes *routes, const moe_packed_weights *w,
                   const moe_scales *scales, void *out, int H, int I,
                   int quant, int path, const moe_ep *ep, void *ws, size_t ws_bytes, void *stream);

/* Decode batch in one call: the routing folded into the route-direct Gate/Up
 * kernel ("perf: add small-batch route MMA for MoE", Summary: the fast path
 * reads each route's expert straight from the token's top-k; Motivation: the
 * route-order pipeline starts from the top-k routes).  Every Gate/Up workgroup
 * takes its route's expert from the top-k of its token's logits (fp32 [T,E],
 * as moe_route reads them), so no routing launch precedes the layer.
 *   routes: caller-allocated as for moe_route; this call sets T/E/k and writes
 *           topk_ids and topk_weights (the same bits moe_route writes);
 *           expert_counts, expert_offsets, perm and route_pos are not used and
 *           not written (may be NULL).
 *   everything else as for moe_forward_ex (ep may be NULL).
 * The path (AUTO or forced) must be the route-direct one, else
 * MOE_ERR_UNSUPPORTED: larger batches use moe_route + moe_forward.  The
 * workspace is moe_forward_workspace_size(T, H, I, E, k, quant, path). */
int moe_decode_forward(const float *logits, const void *x, int T, int E, int k, moe_routes *routes,
                       const moe_packed_weights *w, const moe_scales *scales, void *out,
                       int H, int I, int quant, int path, const moe_ep *ep, void *ws, size_t ws_bytes,
                       void *stream);

/* moe_decode_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same launches and results as moe_decode_forward, with the
 * workspace taken from a 16 MiB device array inside this library (each GPU
 * the library runs on holds its own copy until the process ends; the call
 * itself allocates nothing).  A call whose workspace
 * (moe_forward_workspace_size for its shape, route-direct path) exceeds
 * 16 MiB returns MOE_ERR_UNSUPPORTED before anything is enqueued; every
 * decode batch up to 16 tokens at the layer shapes measured here needs
 * under 6 MiB.  All calls on one GPU share that array: calls that overlap
 * on one GPU (other streams, other threads) race; order them on one stream.
 * The array keeps the last call's contents; nothing in it needs to start at
 * zero (the kernels reset their own counters each call).  Arguments and
 * errors otherwise as for moe_decode_forward. */
int moe_decode_forward_noalloc(const float *logits, const void *x, int T, int E, int k, moe_routes *routes,
                               const moe_packed_weights *w, const moe_scales *scales, void *out,
                               int H, int I, int quant, int path, const moe_ep *ep, void *stream);

/* moe_forward with its device time: exactly moe_forward's launches, with
 * ev_start attached to the first kernel's dispatch (recorded when that kernel
 * starts) and ev_end to the last kernel's (recorded when it ends) --
 * hipExtLaunchKernel's dispatch events, so no marker packet sits between the
 * kernels.  hipEventElapsedTime(ev_start, ev_end) is then the span from the
 * first kernel's start to the last kernel's end on the device, the quantity
 * a kernel trace reports.  Both events are caller-created hipEvent_t handles
 * (either may be NULL); T = 0 launches nothing and records neither.
 * (For benchmarks: "perf: add small-batch route MMA for MoE", Performance.) */
int moe_forward_timed(const void *x, const moe_routes *routes, const moe_packed_weights *w,
                      const moe_scales *scales, void *out, int H, int I, int quant, int path,
                      void *ws, size_t ws_bytes, void *stream, void *ev_start, void *ev_end);

/* moe_forward with stage timing for profilers and benchmarks: the same
 * kernels, with stage_events[0] attached to the first kernel's dispatch
 * (recorded when it starts) and stage_events[i] to the dispatch of stage i's
 * last kernel (recorded when it ends), through hipExtLaunchKernel, so no
 * marker packet sits between two kernels and the timing does not slow the
 * stream; stage_events[i] - stage_events[i-1] is then stage i's device time
 * (from the end of the previous stage, the kernels running back to back).
 * stage_events holds n_events caller-created hipEvent_t handles; stages past
 * them and NULL entries take no event.  No synchronisation.  *n_stages
 * receives the number of stages and stage_names (may be NULL) a
 * comma-separated list of their names, e.g. "init,gate_up,down,combine" for
 * the bf16 grouped path. */
int moe_forward_profiled(const void *x, const moe_routes *routes, const moe_packed_weights *w,
                         const moe_scales *scales, void *out, int H,
                         int I, int quant, int path, void *ws, size_t ws_bytes, void *stream,
                         void **stage_events, int n_events, int *n_stages,
                         const char **stage_names);

/* ---------------------------------------------------- MX training backward --
 * The layer's gradients under the MX training recipe of "[mxfp8 moe training]
 * add per group blocked scale kernels" (Summary and its stacked pull requests:
 * the "dim1" cast in the backward, per-expert weight scales, per-group padded
 * scale rows).  Every backward product runs on MX operands (e4m3 codes, one
 * E8M0 scale per 32 values) quantised along its own reduction dimension:
 *   dh  = dy W_down^T, dy = gate * dout          (operands along H)
 *   dx  = sum over the token's routes of dGU W_gate_up^T, dGU = [dgate | dup]
 *         the SwiGLU backward                     (operands along 2I)
 *   dW_down[e]    = h_e^T dy_e, dW_gate_up[e] = x_e^T dGU_e  (operands along
 *         expert e's routes in sorted order, 32 per scale, each expert's
 *         segment zero-padded to 64 at offsets built on the device)
 *   dgate[r] = <dout[t], y_r>, y_r route r's Down output before its gate.
 * The quantisers pass gradients through unchanged.  The forward quantities
 * (g, u, h, y) are recomputed from x and the weights, as the MX forward
 * computes them.  Grouped path only; H and I multiples of 256, up to 8192.
 *
 * Weight preparation, once per weight update: from bf16 master weights
 * w_gate_up [E][H][2I] and w_down [E][I][H], in one pass each, four packed
 * MX operand sets (the moe_pack_weights layout, plain column order) --
 * W_gate_up along H and W_down along I (the recomputed forward), W_down^T
 * along H and W_gate_up^T along 2I (the input gradients) -- in buf (device,
 * moe_mx_train_weights_size bytes, caller-owned; 0 for an unsupported
 * shape), described by *out (host; its tag is cleared on error).  The same
 * pass also lays out W_gate_up along H with gate and up interleaved, which
 * with the W_down set is the MX forward's weights (out->forward,
 * out->forward_scales).  Enqueued on stream; no synchronisation. */
#define MOE_TRAIN_TAG 0x4d6f4542u
typedef struct {
    const void *gate_up_k;              /* W_gate_up along H: N = 2I, K = H */
    const uint8_t *gate_up_k_scales;
    const void *down_k;                 /* W_down along I: N = H, K = I */
    const uint8_t *down_k_scales;
    const void *down_t;                 /* W_down^T along H: N = I, K = H */
    const uint8_t *down_t_scales;
    const void *gate_up_t;              /* W_gate_up^T along 2I: N = H, K = 2I */
    const uint8_t *gate_up_t_scales;
    int32_t E, H, I;
    uint32_t tag;                       /* MOE_TRAIN_TAG once prepared */
    /* the MX forward of the same weights (W_gate_up along H with gate and up
     * interleaved as moe_pack_weights lays them, W_down along I): pass them to
     * moe_forward with quant MOE_FP8_MX32, so a training step runs its forward
     * and its backward from one preparation */
    moe_packed_weights forward;
    moe_scales forward_scales;
} moe_mx_train_weights;

size_t moe_mx_train_weights_size(int E, int H, int I);
int moe_prepare_mx_train_weights(const void *w_gate_up, const void *w_down, int E, int H, int I, void *buf,
                                 size_t buf_bytes, moe_mx_train_weights *out, void *stream);

/* Bytes of workspace moe_backward needs (0 for an unsupported shape). */
size_t moe_backward_workspace_size(int T, int H, int I, int E, int k);

/* Gradients of the layer for the upstream gradient dout (bf16 [T][H]):
 *   x       bf16 [T][H], the forward's input
 *   routes  moe_route's output for the forward (expert_offsets, perm,
 *           route_pos and topk_weights are read)
 *   w       moe_prepare_mx_train_weights' descriptor (its E must be the
 *           routes' E)
 *   dx      bf16 [T][H]; dgate fp32 [T][k] (route r = t*k + j);
 *   dw_gate_up bf16 [E][H][2I], dw_down bf16 [E][I][H], the master
 *           weights' type (zero for an expert without routes)
 * All pointers device, 16-byte aligned, caller-owned; ws as sized above.
 * Returns MOE_ERR_INVALID_ARG / UNSUPPORTED / WORKSPACE before anything is
 * enqueued, MOE_ERR_HIP if a launch fails.  Deterministic: every sum runs in
 * a fixed order.  No synchronisation. */
int moe_backward(const void *x, const moe_routes *routes, const moe_mx_train_weights *w, const void *dout,
                 void *dx, float *dgate, void *dw_gate_up, void *dw_down, void *ws, size_t ws_bytes,
                 void *stream);

/* moe_backward with stage events, as moe_forward_profiled: stage_events[0]
 * on the first kernel's start, stage_events[i] on the end of stage i's last
 * kernel; the stages are "init,quant_x,gate_up,swiglu,down,dy,dh,swiglu_bwd,
 * dx_rows,combine,dim1,wgrad_gate_up,wgrad_down" (T = 0: the last two). */
int moe_backward_profiled(const void *x, const moe_routes *routes, const moe_mx_train_weights *w,
                          const void *dout, void *dx, float *dgate, void *dw_gate_up, void *dw_down, void *ws,
                          size_t ws_bytes, void *stream, void **stage_events, int n_events, int *n_stages,
                          const char **stage_names);

/* The gates' gradient taken to the router logits: dlogits fp32 [T][E] for
 * dgate fp32 [T][k] (moe_backward's gate gradient) and the routes moe_route
 * returned (topk_ids, topk_weights, T, E, k are read).  The gates are the
 * softmax over the k picked logits ("perf: add small-batch route MMA for
 * MoE", Summary: routes are token/top-k; the renormalised softmax of the
 * routing) and the picks are piecewise constant, so every entry is zero
 * except dlogits[t][ids[t][j]] = w_j (g_j - sum_i w_i g_i).  Device pointers,
 * 16-byte aligned, caller-owned; host validation before any launch; T = 0
 * launches nothing.  No synchronisation. */
int moe_route_backward(const moe_routes *routes, const float *dgate, float *dlogits, void *stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
