/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the forward pass of a
 * token-choice Mixture-of-Experts SwiGLU FFN layer, written from the plain
 * definition of what the layer computes.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load this library; the GPU product path
 * never calls it and shares no code, header or table with it.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "Port necessary FBGEMM MoE kernels" (world_engine pull request):
 *       Summary -- the layer's index shuffling (per-expert grouping of token
 *       routes) and the top-k weighted scatter-add back into tokens.
 *  [P3] "perf: add small-batch route MMA for MoE" (hpc-ops pull request):
 *       Motivation -- the grouped pipeline count/sort -> gather -> prefix ->
 *       Gate/Up GEMM -> activation/quantisation -> Down GEMM -> top-k
 *       reduction, and the route-order pipeline that reaches the same result
 *       without the sort;  Summary -- SwiGLU, FP8 per-tensor and 128x128
 *       blockwise quantisation, Down-input FP8 requantisation.
 *
 * Everything here is computed per token with no sort (the sorted form is
 * derived separately in oracle_route), in IEEE double, with the method's
 * quantisation decisions taken in fp32 as the method takes them.
 *
 * Readings taken where the pages are silent:
 *  - top-k selects on the fp32 logits, descending, exact fp32 equality (so -0
 *    equals +0) broken to the lower expert id; slot j is the j-th pick;
 *  - gates are the softmax over all E experts renormalised over the k picks;
 *  - the Gate/Up weight [H, 2I] holds the gate in columns [0, I) and the up
 *    projection in columns [I, 2I); h = silu(gate) * up, silu(z) = z/(1+e^-z);
 *  - e4m3 is the OCP e4m3fn format (bias 7, max 448, no infinities), encoded
 *    round-to-nearest-even and saturated to +-448 (never NaN);
 *  - a scale is amax/448 in fp32 (1 when amax is 0); a code is e4m3(v / s)
 *    with v / s a true fp32 division;
 *  - per-tensor: one scale for all of x [T,H] and one for all of h [T*k, I];
 *    blockwise: one scale per token per 128 channels (x) and per route row per
 *    128 channels (h); weight scales are given with the weights;
 *  - the combine sums j = 0..k-1 in ascending order;
 *  - MX ("[mxfp8 moe training] add per group blocked scale kernels", Summary:
 *    mxfp8 scales): one power-of-two scale per 32 consecutive values along K,
 *    stored as an E8M0 byte b (scale 2^(b-127)); a group's scale is
 *    2^(floor(log2 amax) - 8), 8 being the largest exponent of e4m3 (the OCP
 *    MX rule), byte 0 for an all-zero group, bytes clamped to [0, 254]; codes
 *    are e4m3(v / scale) as above.  Weights come with their scales per 32 rows
 *    of K per output column; x is quantised per token and h per route row,
 *    each per 32 channels.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BF16 0
#define ORC_FP8_PER_TENSOR 1
#define ORC_FP8_BLOCK128 2
#define ORC_FP8_MX32 3

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- codecs -- */

/* bf16 is the upper half of an IEEE binary32. */
float oracle_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP e4m3fn: s.eeee.mmm, bias 7.  e == 0 are subnormals m * 2^-9; otherwise
 * (1 + m/8) * 2^(e-7) = (8 + m) * 2^(e-10).  s.1111.111 is NaN. */
double oracle_e4m3_decode(uint8_t q) {
    int s = q >> 7, e = (q >> 3) & 15, m = q & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Round-to-nearest-even onto the e4m3fn grid, saturating at +-448.  The
 * spacing of the grid is 2^-9 below 2^-6 and 2^(floor(log2|v|) - 3) above. */
uint8_t oracle_e4m3_encode(float f) {
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f), quantum, n, fl, r, v;
    int ex;
    if (isnan(f)) return 0x7f;
    if (a >= 448.0) return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
        quantum = ldexp(1.0, ex - 1 - 3);
    }
    n = a / quantum;                   /* exact: division by a power of two */
    fl = floor(n);
    if (n - fl > 0.5) r = fl + 1.0;
    else if (n - fl < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;   /* tie: even mantissa */
    v = r * quantum;                   /* <= 448 because a < 448 */
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -6)) {
        return sign | (uint8_t)(v / ldexp(1.0, -9));   /* subnormal m */
    }
    frexp(v, &ex);
    {
        int E = ex - 1;                                  /* floor(log2 v) */
        int m = (int)(v / ldexp(1.0, E - 3)) - 8;
        return sign | (uint8_t)(((E + 7) << 3) | m);
    }
}

/* Scale of a quantisation group: amax / 448 in fp32, or 1 for an all-zero group. */
float oracle_scale_from_amax(float amax) {
    return amax > 0.0f ? amax / 448.0f : 1.0f;
}

/* E8M0 byte of an MX group with largest magnitude amax (see the header). */
uint8_t oracle_mx_scale_byte(float amax) {
    int ex, b;
    if (!(amax > 0.0f)) return 0;
    frexp((double)amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    b = (ex - 1) - 8 + 127;
    return (uint8_t)(b < 0 ? 0 : b > 254 ? 254 : b);
}

double oracle_e8m0_decode(uint8_t b) { return ldexp(1.0, (int)b - 127); }

/* MX-quantise n fp32 values as one group; returns the E8M0 byte.  v / scale is
 * exact (a power of two), so the codes are those of the values themselves. */
uint8_t oracle_quantise_group_mx(const float *v, long n, uint8_t *q) {
    float amax = 0.0f;
    uint8_t b;
    long i;
    for (i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    b = oracle_mx_scale_byte(amax);
    for (i = 0; i < n; ++i) q[i] = oracle_e4m3_encode((float)((double)v[i] / oracle_e8m0_decode(b)));
    return b;
}

/* Quantise n fp32 values with one scale; returns the scale. */
float oracle_quantise_group(const float *v, long n, uint8_t *q) {
    float amax = 0.0f, s;
    long i;
    for (i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    s = oracle_scale_from_amax(amax);
    for (i = 0; i < n; ++i) q[i] = oracle_e4m3_encode(v[i] / s);
    return s;
}

/* ---------------------------------------------------------------- router -- */

/* Router scores of a bias-free linear router: logits[t][e] = sum over h of
 * x[t][h] * w_r[h][e], with x bf16 [T, H] and w_r fp32 [H, E] row-major.  Each
 * product is exact in double (8 + 24 significand bits); the sum runs over
 * ascending h in double and is rounded once to fp32.  The pages route each
 * token by the top-k of its per-expert scores ("Port necessary FBGEMM MoE
 * kernels", Benchmarks: the MoE module of 16 experts, top 8) without printing
 * the router itself; this linear map is the plainest reading. */
void oracle_router_logits(const uint16_t *x, const float *w_r, int T, int H, int E, float *logits) {
    int t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        int e, h;
        for (e = 0; e < E; ++e) {
            double s = 0.0;
            for (h = 0; h < H; ++h)
                s += (double)oracle_bf16_decode(x[(long)t * H + h]) * (double)w_r[(long)h * E + e];
            logits[(long)t * E + e] = (float)s;
        }
    }
}

/* --------------------------------------------------------------- routing -- */

/* Token-choice routing.  For each token: pick k experts greedily by largest
 * logit (ties to the lower id), gates = softmax over E renormalised over the
 * picks.  Then the grouped form [P1 Summary "index shuffling"; P3 Motivation
 * "count/sort", "prefix"]: per-expert counts, their exclusive prefix (E+1
 * entries), and the route ids r = t*k + j listed expert by expert, in
 * increasing r inside each expert (a counting sort), with its inverse. */
void oracle_route(const float *logits, int T, int E, int k,
                  int32_t *ids, float *weights, int32_t *counts,
                  int32_t *offsets, int32_t *perm, int32_t *route_pos) {
    long R = (long)T * k, r;
    int t, e;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        const float *l = logits + (long)t * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        double m, z = 0.0, zs = 0.0;
        int j, i;
        for (j = 0; j < k; ++j) {
            int best = -1;
            for (i = 0; i < E; ++i) {
                if (taken[i]) continue;
                if (best < 0 || l[i] > l[best]) best = i;   /* '>' keeps the lower id on ties */
            }
            taken[best] = 1;
            ids[(long)t * k + j] = best;
        }
        m = l[0];
        for (i = 1; i < E; ++i) if (l[i] > m) m = l[i];
        for (i = 0; i < E; ++i) z += exp((double)l[i] - m);
        for (j = 0; j < k; ++j) zs += exp((double)l[ids[(long)t * k + j]] - m) / z;
        for (j = 0; j < k; ++j) {
            double p = exp((double)l[ids[(long)t * k + j]] - m) / z;
            weights[(long)t * k + j] = (float)(p / zs);
        }
        free(taken);
    }
    for (e = 0; e < E; ++e) counts[e] = 0;
    for (r = 0; r < R; ++r) counts[ids[r]]++;
    offsets[0] = 0;
    for (e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    {
        int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
        for (e = 0; e < E; ++e) next[e] = offsets[e];
        for (r = 0; r < R; ++r) perm[next[ids[r]]++] = (int32_t)r;
        free(next);
    }
    for (r = 0; r < R; ++r) route_pos[perm[r]] = (int32_t)r;
}

/* --------------------------------------------------------------- forward -- */

typedef struct {
    int T, H, I, E, k, quant;
    const uint16_t *x;        /* bf16 [T, H] */
    const void *w_gu;         /* [E, H, 2I] bf16 or e4m3 */
    const void *w_d;          /* [E, I, H]  bf16 or e4m3 */
    const float *s_gu;        /* per-tensor [E]; block128 [E, H/128, 2I/128] */
    const float *s_d;         /* per-tensor [E]; block128 [E, I/128, H/128] */
    float s_x;                /* per-tensor activation scale */
    const float *s_x_blk;     /* block128 activation scales [T, H/128] */
    const uint8_t *mx_x;      /* MX activation scale bytes [T, H/32] */
    const uint8_t *q_x;       /* fp8 activation codes [T, H] */
} orc_layer;

/* Every e4m3 code and E8M0 byte decoded once (the same decoders, looked up
 * instead of called per weight: the layer reads each weight once per route). */
static double e4m3_tab[256], e8m0_tab[256];

static void decode_tables(void) {
    int c;
    for (c = 0; c < 256; ++c) {
        e4m3_tab[c] = oracle_e4m3_decode((uint8_t)c);
        e8m0_tab[c] = oracle_e8m0_decode((uint8_t)c);
    }
}

static double w_gu_at(const orc_layer *L, int e, int h, int n) {
    long idx = ((long)e * L->H + h) * (2L * L->I) + n;
    if (L->quant == ORC_BF16) return oracle_bf16_decode(((const uint16_t *)L->w_gu)[idx]);
    {
        double q = e4m3_tab[((const uint8_t *)L->w_gu)[idx]];
        if (L->quant == ORC_FP8_MX32)   /* bytes [E][H/32][2I] */
            return q * e8m0_tab[((const uint8_t *)L->s_gu)[((long)e * (L->H / 32) + h / 32) * (2L * L->I) + n]];
        if (L->quant == ORC_FP8_PER_TENSOR) return q * L->s_gu[e];
        return q * L->s_gu[((long)e * (L->H / 128) + h / 128) * (2L * L->I / 128) + n / 128];
    }
}

static double w_d_at(const orc_layer *L, int e, int i, int n) {
    long idx = ((long)e * L->I + i) * L->H + n;
    if (L->quant == ORC_BF16) return oracle_bf16_decode(((const uint16_t *)L->w_d)[idx]);
    {
        double q = e4m3_tab[((const uint8_t *)L->w_d)[idx]];
        if (L->quant == ORC_FP8_MX32)   /* bytes [E][I/32][H] */
            return q * e8m0_tab[((const uint8_t *)L->s_d)[((long)e * (L->I / 32) + i / 32) * L->H + n]];
        if (L->quant == ORC_FP8_PER_TENSOR) return q * L->s_d[e];
        return q * L->s_d[((long)e * (L->I / 128) + i / 128) * (L->H / 128) + n / 128];
    }
}

/* The activation entering the Gate/Up projection for token t. */
static void activation(const orc_layer *L, int t, double *a) {
    int h;
    for (h = 0; h < L->H; ++h) {
        long idx = (long)t * L->H + h;
        if (L->quant == ORC_BF16) a[h] = oracle_bf16_decode(L->x[idx]);
        else if (L->quant == ORC_FP8_PER_TENSOR) a[h] = oracle_e4m3_decode(L->q_x[idx]) * L->s_x;
        else if (L->quant == ORC_FP8_MX32)
            a[h] = oracle_e4m3_decode(L->q_x[idx]) * oracle_e8m0_decode(L->mx_x[(long)t * (L->H / 32) + h / 32]);
        else a[h] = oracle_e4m3_decode(L->q_x[idx]) * L->s_x_blk[(long)t * (L->H / 128) + h / 128];
    }
}

/* h = silu(a W_gate) * (a W_up) for one route, in double. */
static void gate_up_swiglu(const orc_layer *L, int e, const double *a, double *h_out, double *acc) {
    int h, n, I2 = 2 * L->I;
    for (n = 0; n < I2; ++n) acc[n] = 0.0;
    for (h = 0; h < L->H; ++h) {
        double ah = a[h];
        if (ah == 0.0) continue;
        for (n = 0; n < I2; ++n) acc[n] += ah * w_gu_at(L, e, h, n);
    }
    for (n = 0; n < L->I; ++n) {
        double g = acc[n], u = acc[L->I + n];
        h_out[n] = g / (1.0 + exp(-g)) * u;
    }
}

/* y = h W_down for one route. */
static void down(const orc_layer *L, int e, const double *h, double *y) {
    int i, n;
    for (n = 0; n < L->H; ++n) y[n] = 0.0;
    for (i = 0; i < L->I; ++i) {
        double hi = h[i];
        if (hi == 0.0) continue;
        for (n = 0; n < L->H; ++n) y[n] += hi * w_d_at(L, e, i, n);
    }
}

/*
 * Layer output for the tokens listed in tok (n_tok of them; tok == NULL means
 * all T tokens in order), written to out[n_tok, H] in double.
 * x: bf16 [T,H]; ids/weights: [T,k] as produced by oracle_route.
 * quant 1 (per-tensor) needs h of every route for its scale, so it runs the
 * Gate/Up pass over all T tokens first, whatever tok lists.
 * Returns 0, or -1 on an unsupported shape or an allocation failure.
 */
int oracle_forward_ep(const uint16_t *x, int T, int H, int I, int E, int k,
                      const int32_t *ids, const float *weights,
                      const void *w_gu, const void *w_d,
                      const float *s_gu, const float *s_d, int quant, int e0, int n_local,
                      const int32_t *tok, int n_tok, double *out);

int oracle_forward(const uint16_t *x, int T, int H, int I, int E, int k,
                   const int32_t *ids, const float *weights,
                   const void *w_gu, const void *w_d,
                   const float *s_gu, const float *s_d, int quant,
                   const int32_t *tok, int n_tok, double *out) {
    return oracle_forward_ep(x, T, H, I, E, k, ids, weights, w_gu, w_d, s_gu, s_d, quant, 0, E, tok,
                             n_tok, out);
}

/*
 * Expert-parallel form [P3 Summary: the fast path "preserves EP routing" and
 * "shared output"]: the weights and scales hold experts [e0, e0 + n_local)
 * only (expert e at index e - e0); routes to other experts contribute nothing,
 * so out[t] is the gate-weighted sum over token t's local routes.  The
 * per-tensor h scale is the amax over the local routes' h, the only h such a
 * call sees.  (Adding the sum into an existing output is left to the caller.)
 */
int oracle_forward_ep(const uint16_t *x, int T, int H, int I, int E, int k,
                      const int32_t *ids, const float *weights,
                      const void *w_gu, const void *w_d,
                      const float *s_gu, const float *s_d, int quant, int e0, int n_local,
                      const int32_t *tok, int n_tok, double *out) {
    orc_layer L;
    uint8_t *q_x = NULL;
    float *s_x_blk = NULL, *h_all = NULL, s_h = 1.0f;
    uint8_t *mx_x = NULL;
    double *hq_all = NULL;
    int bad = 0, ti;
    long i;
    (void)E;
    if (quant < 0 || quant > 3) return -1;
    if (e0 < 0 || n_local < 1) return -1;
    if (quant == ORC_FP8_BLOCK128 && (H % 128 || I % 128)) return -1;
    if (quant == ORC_FP8_MX32 && (H % 32 || I % 32)) return -1;
    memset(&L, 0, sizeof L);
    L.T = T; L.H = H; L.I = I; L.E = E; L.k = k; L.quant = quant;
    L.x = x; L.w_gu = w_gu; L.w_d = w_d; L.s_gu = s_gu; L.s_d = s_d;
    if (n_tok == 0 || T == 0) return 0;
    decode_tables();

    /* activation quantisation [P3 Summary: FP8 activations before each GEMM] */
    if (quant != ORC_BF16) {
        q_x = (uint8_t *)malloc((size_t)T * H);
        if (!q_x) return -1;
        if (quant == ORC_FP8_PER_TENSOR) {
            float *xf = (float *)malloc(sizeof(float) * (size_t)T * H);
            if (!xf) { free(q_x); return -1; }
            for (i = 0; i < (long)T * H; ++i) xf[i] = oracle_bf16_decode(x[i]);
            L.s_x = oracle_quantise_group(xf, (long)T * H, q_x);
            free(xf);
        } else if (quant == ORC_FP8_MX32) {
            int nb = H / 32, t, c, j;
            mx_x = (uint8_t *)malloc((size_t)T * nb);
            if (!mx_x) { free(q_x); return -1; }
            for (t = 0; t < T; ++t)
                for (c = 0; c < nb; ++c) {
                    float v[32];
                    for (j = 0; j < 32; ++j) v[j] = oracle_bf16_decode(x[(long)t * H + c * 32 + j]);
                    mx_x[(long)t * nb + c] = oracle_quantise_group_mx(v, 32, q_x + (long)t * H + c * 32);
                }
            L.mx_x = mx_x;
        } else {
            int nb = H / 128, t, c, j;
            s_x_blk = (float *)malloc(sizeof(float) * (size_t)T * nb);
            if (!s_x_blk) { free(q_x); return -1; }
            for (t = 0; t < T; ++t)
                for (c = 0; c < nb; ++c) {
                    float v[128];
                    for (j = 0; j < 128; ++j) v[j] = oracle_bf16_decode(x[(long)t * H + c * 128 + j]);
                    s_x_blk[(long)t * nb + c] = oracle_quantise_group(v, 128, q_x + (long)t * H + c * 128);
                }
            L.s_x_blk = s_x_blk;
        }
        L.q_x = q_x;
    }

    /* per-tensor Down-input requantisation needs every route's h first */
    if (quant == ORC_FP8_PER_TENSOR) {
        long R = (long)T * k, nl = 0, r;
        long *slot = (long *)malloc(sizeof(long) * (size_t)(R > 0 ? R : 1));   /* route -> local h row */
        uint8_t *q_h;
        if (!slot) { free(q_x); return -1; }
        for (r = 0; r < R; ++r) slot[r] = (ids[r] >= e0 && ids[r] < e0 + n_local) ? nl++ : -1;
        h_all = (float *)malloc(sizeof(float) * (size_t)(nl > 0 ? nl : 1) * I);
        q_h = (uint8_t *)malloc((size_t)(nl > 0 ? nl : 1) * I);
        if (!h_all || !q_h) { free(h_all); free(q_h); free(q_x); free(slot); return -1; }
#pragma omp parallel for schedule(dynamic)
        for (ti = 0; ti < T; ++ti) {
            double *a = (double *)malloc(sizeof(double) * (size_t)H);
            double *acc = (double *)malloc(sizeof(double) * 2 * (size_t)I);
            double *hr = (double *)malloc(sizeof(double) * (size_t)I);
            int j, n;
            activation(&L, ti, a);
            for (j = 0; j < k; ++j) {
                long rr = (long)ti * k + j;
                if (slot[rr] < 0) continue;
                gate_up_swiglu(&L, ids[rr] - e0, a, hr, acc);
                /* the quantiser sees h as fp32, the width the method holds it in */
                for (n = 0; n < I; ++n) h_all[slot[rr] * I + n] = (float)hr[n];
            }
            free(a); free(acc); free(hr);
        }
        s_h = nl > 0 ? oracle_quantise_group(h_all, nl * I, q_h) : 1.0f;
        free(h_all);
        h_all = NULL;
        hq_all = (double *)malloc(sizeof(double) * (size_t)R * I);
        if (!hq_all) { free(q_h); free(q_x); free(slot); return -1; }
        for (r = 0; r < R; ++r)
            for (i = 0; i < I; ++i)
                hq_all[r * I + i] = slot[r] < 0 ? 0.0 : oracle_e4m3_decode(q_h[slot[r] * I + i]) * s_h;
        free(q_h);
        free(slot);
    }

#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (ti = 0; ti < n_tok; ++ti) {
        int t = tok ? tok[ti] : ti, j, n, c;
        double *a = (double *)malloc(sizeof(double) * (size_t)H);
        double *acc = (double *)malloc(sizeof(double) * 2 * (size_t)I);
        double *hd = (double *)malloc(sizeof(double) * (size_t)I);
        double *y = (double *)malloc(sizeof(double) * (size_t)H);
        double *h = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = out + (long)ti * H;
        if (!a || !acc || !hd || !y || !h || t < 0 || t >= T) {
            bad |= 1;
        } else {
            for (n = 0; n < H; ++n) o[n] = 0.0;
            if (quant != ORC_FP8_PER_TENSOR) activation(&L, t, a);
            for (j = 0; j < k; ++j) {
                long r = (long)t * k + j;
                int e = ids[r] - e0;   /* index into this call's experts */
                if (e < 0 || e >= n_local) continue;   /* another rank's expert */
                if (quant == ORC_FP8_PER_TENSOR) {
                    for (n = 0; n < I; ++n) hd[n] = hq_all[r * I + n];
                } else {
                    gate_up_swiglu(&L, e, a, h, acc);
                    if (quant == ORC_FP8_BLOCK128) {
                        uint8_t q[128];
                        float hf[128];
                        for (c = 0; c < I / 128; ++c) {
                            float s;
                            for (n = 0; n < 128; ++n) hf[n] = (float)h[c * 128 + n];
                            s = oracle_quantise_group(hf, 128, q);
                            for (n = 0; n < 128; ++n) hd[c * 128 + n] = oracle_e4m3_decode(q[n]) * s;
                        }
                    } else if (quant == ORC_FP8_MX32) {
                        uint8_t q[32];
                        float hf[32];
                        for (c = 0; c < I / 32; ++c) {
                            uint8_t b;
                            for (n = 0; n < 32; ++n) hf[n] = (float)h[c * 32 + n];
                            b = oracle_quantise_group_mx(hf, 32, q);
                            for (n = 0; n < 32; ++n) hd[c * 32 + n] = oracle_e4m3_decode(q[n]) * oracle_e8m0_decode(b);
                        }
                    } else {
                        for (n = 0; n < I; ++n) hd[n] = h[n];
                    }
                }
                down(&L, e, hd, y);
                /* top-k weighted combine [P1 Summary "scatter_add"; P3 Motivation "top-k reduction"] */
                for (n = 0; n < H; ++n) o[n] += (double)weights[r] * y[n];
            }
        }
        free(a); free(acc); free(hd); free(y); free(h);
    }
    free(q_x); free(s_x_blk); free(mx_x); free(h_all); free(hq_all);
    return bad ? -1 : 0;
}

/* The quantised activations exactly as the method defines them, exposed so
 * the tests can compare codes: per-tensor writes one scale, block128 writes
 * [T, H/128] scales, MX writes [T, H/32] E8M0 bytes (into `scales` viewed as
 * bytes). */
int oracle_quantise_activations(const uint16_t *x, int T, int H, int quant,
                                uint8_t *q, float *scales) {
    long i;
    if (quant == ORC_FP8_PER_TENSOR) {
        float *xf = (float *)malloc(sizeof(float) * ((size_t)T * H + 1));
        if (!xf) return -1;
        for (i = 0; i < (long)T * H; ++i) xf[i] = oracle_bf16_decode(x[i]);
        scales[0] = oracle_quantise_group(xf, (long)T * H, q);
        free(xf);
        return 0;
    }
    if (quant == ORC_FP8_MX32) {
        int t, c, j, nb = H / 32;
        if (H % 32) return -1;
        for (t = 0; t < T; ++t)
            for (c = 0; c < nb; ++c) {
                float v[32];
                for (j = 0; j < 32; ++j) v[j] = oracle_bf16_decode(x[(long)t * H + c * 32 + j]);
                ((uint8_t *)scales)[(long)t * nb + c] = oracle_quantise_group_mx(v, 32, q + (long)t * H + c * 32);
            }
        return 0;
    }
    if (quant == ORC_FP8_BLOCK128) {
        int t, c, j, nb = H / 128;
        if (H % 128) return -1;
        for (t = 0; t < T; ++t)
            for (c = 0; c < nb; ++c) {
                float v[128];
                for (j = 0; j < 128; ++j) v[j] = oracle_bf16_decode(x[(long)t * H + c * 128 + j]);
                scales[(long)t * nb + c] = oracle_quantise_group(v, 128, q + (long)t * H + c * 128);
            }
        return 0;
    }
    return -1;
}

/*
 * The SwiGLU output h = silu(a W_gate) * (a W_up) of the listed routes, in
 * double, where a is the token's activation as the Gate/Up projection sees it
 * (bf16 x, or x quantised as oracle_quantise_activations defines it) [P3
 * Motivation: the Gate/Up GEMM, then the activation; Summary: FP8 activations
 * before each GEMM].  This is the tensor the Down-input quantisation takes
 * its scales over (per-tensor: amax over all routes; blockwise: per route row
 * per 128 channels; MX: per 32), exposed so tests can derive those scales.
 * routes: n route ids r = t*k + j (NULL: all T*k in order); out [n, I].
 * Returns 0, or -1 on an unsupported shape or an allocation failure.
 */
int oracle_gate_up_h(const uint16_t *x, int T, int H, int I, int E, int k, const int32_t *ids,
                     const void *w_gu, const float *s_gu, int quant, const int32_t *routes, long n,
                     double *out) {
    orc_layer L;
    uint8_t *q_x = NULL;
    float *scales = NULL;
    long R = (long)T * k, ri;
    int bad = 0;
    if (quant < 0 || quant > 3 || T < 0) return -1;
    if ((quant == ORC_FP8_BLOCK128 && H % 128) || (quant == ORC_FP8_MX32 && H % 32)) return -1;
    memset(&L, 0, sizeof L);
    L.T = T; L.H = H; L.I = I; L.E = E; L.k = k; L.quant = quant;
    L.x = x; L.w_gu = w_gu; L.s_gu = s_gu;
    if (quant != ORC_BF16) {
        long ns = quant == ORC_FP8_PER_TENSOR ? 1 : quant == ORC_FP8_BLOCK128 ? (long)T * (H / 128) : 0;
        q_x = (uint8_t *)malloc((size_t)T * H + 1);
        /* MX scale bytes are held in a float buffer of the same byte count or more */
        scales = (float *)malloc(sizeof(float) * (size_t)(ns > 0 ? ns : (long)T * (H / 32) / 4 + 1));
        if (!q_x || !scales || oracle_quantise_activations(x, T, H, quant, q_x, scales) != 0) {
            free(q_x); free(scales);
            return -1;
        }
        L.q_x = q_x;
        if (quant == ORC_FP8_PER_TENSOR) L.s_x = scales[0];
        else if (quant == ORC_FP8_BLOCK128) L.s_x_blk = scales;
        else L.mx_x = (const uint8_t *)scales;
    }
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (ri = 0; ri < n; ++ri) {
        long r = routes ? routes[ri] : ri;
        double *a = (double *)malloc(sizeof(double) * (size_t)H);
        double *acc = (double *)malloc(sizeof(double) * 2 * (size_t)I);
        if (!a || !acc || r < 0 || r >= R || ids[r] < 0 || ids[r] >= E) {
            bad |= 1;
        } else {
            activation(&L, (int)(r / k), a);
            gate_up_swiglu(&L, ids[r], a, out + ri * (long)I, acc);
        }
        free(a); free(acc);
    }
    free(q_x); free(scales);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------- backward -- */

/*
 * Gradients of the layer for an upstream gradient dout [T, H] (bf16), under
 * the MX training recipe of [P2] ("[mxfp8 moe training] add per group blocked
 * scale kernels": Summary and its stacked pull requests -- the "dim1" cast in
 * the backward, per-expert 3-D weight scales, per-group padded scale rows).
 * The gradients themselves are the chain rule through the forward above;
 * the readings taken where the pages are silent:
 *  - the forward is the MX forward with the weights quantised from bf16
 *    master weights along K (W_gate_up along H per output column, W_down
 *    along I), x per token along H and h per route along I;
 *  - every backward product takes MX operands quantised along its own
 *    reduction dimension, 32 values per scale: the input-gradient products
 *    along the forward's output dimension (dy and W_down along H, dGU =
 *    [dgate | dup] and W_gate_up along 2I), the weight-gradient products along
 *    the routes of one expert in ascending route order (the stable sort's
 *    order), 32 routes per group, an expert's last group padded with zeros;
 *  - the quantisers pass gradients through unchanged (straight-through);
 *  - the quantisers see fp32 values: dy = fp32(gate) * fp32(dout) rounded to
 *    fp32, h = fp32(silu(g) u), dGU rounded to fp32, x as its bf16 value;
 *  - silu'(g) = sigma(g) (1 + g (1 - sigma(g)));
 *  - dgate_r = sum over n of dout[t][n] y_r[n], y_r the route's Down output
 *    before the gate weighting; dx[t] = the sum of the token's route input
 *    gradients over j ascending.
 * exact = 1 switches every quantiser off (the bf16 inputs in double
 * throughout): the plain calculus, which the tests compare with autograd.
 *
 * x, dout: bf16 [T, H]; ids, weights: [T, k]; w_gu bf16 [E, H, 2I]; w_d bf16
 * [E, I, H].  tok (n_tok distinct tokens) selects the rows of dx [n_tok, H]
 * and dgate [n_tok, k]; exps (n_exp experts) the slabs of dw_gu [n_exp, H, 2I]
 * and dw_d [n_exp, I, H].  Returns 0, or -1 on a bad argument or allocation
 * failure.
 */
static void mx_group_deq(const float *v, double *out) {
    uint8_t q[32];
    uint8_t b = oracle_quantise_group_mx(v, 32, q);
    double s = oracle_e8m0_decode(b);
    int j;
    for (j = 0; j < 32; ++j) out[j] = oracle_e4m3_decode(q[j]) * s;
}

/* n values of a row (n a multiple of 32), each group of 32 MX-quantised and
 * returned dequantised; v holds fp32 values */
static void mx_row_deq(const float *v, long n, double *out) {
    long c;
    for (c = 0; c < n; c += 32) mx_group_deq(v + c, out + c);
}

static double silu_d(double z) { return z / (1.0 + exp(-z)); }

int oracle_backward_mx(const uint16_t *x, int T, int H, int I, int E, int k,
                       const int32_t *ids, const float *weights,
                       const uint16_t *w_gu, const uint16_t *w_d, const uint16_t *dout, int exact,
                       const int32_t *tok, int n_tok, const int32_t *exps, int n_exp,
                       double *dx, double *dgate, double *dw_gu, double *dw_d) {
    long R = (long)T * k, r;
    int I2 = 2 * I, bad = 0, e, i;
    double *xa = NULL, *da = NULL;
    long *slot = NULL;
    int *exp_slot = NULL;
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || n_tok < 0 || n_exp < 0) return -1;
    if (!exact && (H % 32 || I % 32)) return -1;
    slot = (long *)malloc(sizeof(long) * (size_t)(R > 0 ? R : 1));
    exp_slot = (int *)malloc(sizeof(int) * (size_t)E);
    xa = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * H);
    da = (double *)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1) * k * H);
    if (!slot || !exp_slot || !xa || !da) { bad = 1; goto done; }
    for (r = 0; r < R; ++r) {
        slot[r] = -1;
        if (ids[r] < 0 || ids[r] >= E) { bad = 1; goto done; }
    }
    for (i = 0; i < n_tok; ++i) {
        int j;
        if (tok[i] < 0 || tok[i] >= T) { bad = 1; goto done; }
        for (j = 0; j < k; ++j) slot[(long)tok[i] * k + j] = (long)i * k + j;
    }
    for (e = 0; e < E; ++e) exp_slot[e] = -1;
    for (i = 0; i < n_exp; ++i) {
        if (exps[i] < 0 || exps[i] >= E) { bad = 1; goto done; }
        exp_slot[exps[i]] = i;
    }
    /* the Gate/Up input: x quantised per token along H (MX), or x itself */
    {
        int t, c;
        for (t = 0; t < T; ++t) {
            float v[32];
            for (c = 0; c < H; c += 32) {
                int j;
                for (j = 0; j < 32 && c + j < H; ++j) v[j] = oracle_bf16_decode(x[(long)t * H + c + j]);
                if (exact) for (j = 0; j < 32 && c + j < H; ++j) xa[(long)t * H + c + j] = v[j];
                else mx_group_deq(v, xa + (long)t * H + c);
            }
        }
    }

#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (e = 0; e < E; ++e) {
        long n_e = 0, p, need = 0, r;
        int es = exp_slot[e], h, c, n, ii, g;
        double *WgK = NULL, *Wg2 = NULL, *WdK = NULL, *WdH = NULL;
        double *gu = NULL, *hq = NULL, *y = NULL, *dyq = NULL, *dh = NULL, *dgu = NULL;
        float *fv = NULL;
        double *xs = NULL, *hs = NULL, *dys = NULL, *dgs = NULL;   /* per route of e, for the weight gradients */
        long *rl = NULL;
        for (r = 0; r < R; ++r)
            if (ids[r] == e) {
                ++n_e;
                if (slot[r] >= 0) need = 1;
            }
        if (!need && es < 0) continue;
        WgK = (double *)malloc(sizeof(double) * (size_t)H * I2);
        Wg2 = (double *)malloc(sizeof(double) * (size_t)H * I2);
        WdK = (double *)malloc(sizeof(double) * (size_t)I * H);
        WdH = (double *)malloc(sizeof(double) * (size_t)I * H);
        gu = (double *)malloc(sizeof(double) * (size_t)I2);
        hq = (double *)malloc(sizeof(double) * (size_t)I);
        y = (double *)malloc(sizeof(double) * (size_t)H);
        dyq = (double *)malloc(sizeof(double) * (size_t)H);
        dh = (double *)malloc(sizeof(double) * (size_t)I);
        dgu = (double *)malloc(sizeof(double) * (size_t)I2);
        fv = (float *)malloc(sizeof(float) * (size_t)(H > I2 ? H : I2));
        rl = (long *)malloc(sizeof(long) * (size_t)(n_e > 0 ? n_e : 1));
        if (es >= 0) {
            xs = (double *)malloc(sizeof(double) * (size_t)(n_e > 0 ? n_e : 1) * H);
            hs = (double *)malloc(sizeof(double) * (size_t)(n_e > 0 ? n_e : 1) * I);
            dys = (double *)malloc(sizeof(double) * (size_t)(n_e > 0 ? n_e : 1) * H);
            dgs = (double *)malloc(sizeof(double) * (size_t)(n_e > 0 ? n_e : 1) * I2);
        }
        if (!WgK || !Wg2 || !WdK || !WdH || !gu || !hq || !y || !dyq || !dh || !dgu || !fv || !rl ||
            (es >= 0 && (!xs || !hs || !dys || !dgs))) {
            bad |= 1;
            goto next_e;
        }
        /* the expert's weights as each product sees them */
        {
            const uint16_t *wg = w_gu + (long)e * H * I2, *wd = w_d + (long)e * I * H;
            float v[32];
            double o[32];
            int j;
            for (h = 0; h < H; ++h)
                for (c = 0; c < I2; ++c) WgK[(long)h * I2 + c] = Wg2[(long)h * I2 + c] = oracle_bf16_decode(wg[(long)h * I2 + c]);
            for (ii = 0; ii < I; ++ii)
                for (n = 0; n < H; ++n) WdK[(long)ii * H + n] = WdH[(long)ii * H + n] = oracle_bf16_decode(wd[(long)ii * H + n]);
            if (!exact) {
                for (c = 0; c < I2; ++c)          /* forward: W_gate_up along H */
                    for (h = 0; h < H; h += 32) {
                        for (j = 0; j < 32; ++j) v[j] = oracle_bf16_decode(wg[(long)(h + j) * I2 + c]);
                        mx_group_deq(v, o);
                        for (j = 0; j < 32; ++j) WgK[(long)(h + j) * I2 + c] = o[j];
                    }
                for (h = 0; h < H; ++h)           /* input gradient: W_gate_up along 2I */
                    for (c = 0; c < I2; c += 32) {
                        for (j = 0; j < 32; ++j) v[j] = oracle_bf16_decode(wg[(long)h * I2 + c + j]);
                        mx_group_deq(v, Wg2 + (long)h * I2 + c);
                    }
                for (n = 0; n < H; ++n)           /* forward: W_down along I */
                    for (ii = 0; ii < I; ii += 32) {
                        for (j = 0; j < 32; ++j) v[j] = oracle_bf16_decode(wd[(long)(ii + j) * H + n]);
                        mx_group_deq(v, o);
                        for (j = 0; j < 32; ++j) WdK[(long)(ii + j) * H + n] = o[j];
                    }
                for (ii = 0; ii < I; ++ii)        /* input gradient: W_down along H */
                    for (n = 0; n < H; n += 32) {
                        for (j = 0; j < 32; ++j) v[j] = oracle_bf16_decode(wd[(long)ii * H + n + j]);
                        mx_group_deq(v, WdH + (long)ii * H + n);
                    }
            }
        }
        /* every route of e in ascending route order */
        p = 0;
        for (r = 0; r < R; ++r) {
            int t, j;
            const double *a;
            double dgr, wr;
            if (ids[r] != e) continue;
            rl[p] = r;
            if (slot[r] < 0 && es < 0) { ++p; continue; }
            t = (int)(r / k);
            j = (int)(r % k);
            (void)j;
            a = xa + (long)t * H;
            wr = (double)weights[r];
            /* forward: [g | u] = a W_gate_up, h = silu(g) u, y = h W_down */
            for (c = 0; c < I2; ++c) gu[c] = 0.0;
            for (h = 0; h < H; ++h) {
                double ah = a[h];
                const double *wrow = WgK + (long)h * I2;
                for (c = 0; c < I2; ++c) gu[c] += ah * wrow[c];
            }
            for (ii = 0; ii < I; ++ii) fv[ii] = (float)(silu_d(gu[ii]) * gu[I + ii]);
            if (es >= 0)
                for (ii = 0; ii < I; ++ii) hs[p * I + ii] = exact ? silu_d(gu[ii]) * gu[I + ii] : fv[ii];
            if (exact) for (ii = 0; ii < I; ++ii) hq[ii] = silu_d(gu[ii]) * gu[I + ii];
            else mx_row_deq(fv, I, hq);
            for (n = 0; n < H; ++n) y[n] = 0.0;
            for (ii = 0; ii < I; ++ii) {
                double hv = hq[ii];
                const double *wrow = WdK + (long)ii * H;
                for (n = 0; n < H; ++n) y[n] += hv * wrow[n];
            }
            /* the gate's gradient */
            dgr = 0.0;
            for (n = 0; n < H; ++n) dgr += (double)oracle_bf16_decode(dout[(long)t * H + n]) * y[n];
            /* dy = gate * dout; dh = dy W_down^T */
            {
                float *dyf = fv;
                for (n = 0; n < H; ++n) dyf[n] = weights[r] * oracle_bf16_decode(dout[(long)t * H + n]);
                if (es >= 0)
                    for (n = 0; n < H; ++n) dys[p * H + n] = exact ? wr * oracle_bf16_decode(dout[(long)t * H + n]) : dyf[n];
                if (exact) for (n = 0; n < H; ++n) dyq[n] = wr * oracle_bf16_decode(dout[(long)t * H + n]);
                else mx_row_deq(dyf, H, dyq);
            }
            for (ii = 0; ii < I; ++ii) {
                double s = 0.0;
                const double *wrow = WdH + (long)ii * H;
                for (n = 0; n < H; ++n) s += dyq[n] * wrow[n];
                dh[ii] = s;
            }
            /* SwiGLU backward, then dGU = [dgate | dup] */
            for (ii = 0; ii < I; ++ii) {
                double gv = gu[ii], uv = gu[I + ii];
                double sg = 1.0 / (1.0 + exp(-gv));
                dgu[ii] = dh[ii] * uv * sg * (1.0 + gv * (1.0 - sg));
                dgu[I + ii] = dh[ii] * gv * sg;
            }
            if (es >= 0) {
                for (h = 0; h < H; ++h) xs[p * H + h] = oracle_bf16_decode(x[(long)t * H + h]);
                for (c = 0; c < I2; ++c) dgs[p * I2 + c] = exact ? dgu[c] : (double)(float)dgu[c];
            }
            /* da = dGU W_gate_up^T, for the listed tokens */
            if (slot[r] >= 0) {
                double *dar = da + slot[r] * H;
                if (!exact) {
                    for (c = 0; c < I2; ++c) fv[c] = (float)dgu[c];
                    mx_row_deq(fv, I2, dgu);
                }
                for (h = 0; h < H; ++h) {
                    double s = 0.0;
                    const double *wrow = Wg2 + (long)h * I2;
                    for (c = 0; c < I2; ++c) s += dgu[c] * wrow[c];
                    dar[h] = s;
                }
                dgate[slot[r]] = dgr;
            }
            ++p;
        }
        /* weight gradients of e: products over its routes, the operands
         * quantised along the routes (the "dim1" cast) */
        if (es >= 0) {
            double *ow = dw_gu + (long)es * H * I2, *od = dw_d + (long)es * I * H;
            long ng = (n_e + 31) / 32, np = ng * 32;
            double *cq = (double *)malloc(sizeof(double) * (size_t)(np > 0 ? np : 1) * (H > I2 ? H : I2));
            double *cq2 = (double *)malloc(sizeof(double) * (size_t)(np > 0 ? np : 1) * (H > I2 ? H : I2));
            if (!cq || !cq2) {
                bad |= 1;
            } else {
                /* column-quantise src [n_e][m] into dst [np][m] (zero rows past n_e) */
#define ORC_DIM1(src, m, dst)                                                        \
                for (c = 0; c < (m); ++c)                                            \
                    for (g = 0; g < ng; ++g) {                                       \
                        float v[32];                                                 \
                        double o[32];                                                \
                        int j;                                                       \
                        for (j = 0; j < 32; ++j) {                                   \
                            long pp = (long)g * 32 + j;                              \
                            v[j] = pp < n_e ? (float)(src)[pp * (m) + c] : 0.0f;     \
                        }                                                            \
                        if (exact) for (j = 0; j < 32; ++j) {                        \
                            long pp = (long)g * 32 + j;                              \
                            o[j] = pp < n_e ? (src)[pp * (m) + c] : 0.0;             \
                        }                                                            \
                        else mx_group_deq(v, o);                                     \
                        for (j = 0; j < 32; ++j) (dst)[((long)g * 32 + j) * (m) + c] = o[j]; \
                    }
                ORC_DIM1(xs, H, cq)
                ORC_DIM1(dgs, I2, cq2)
                for (h = 0; h < H; ++h)
                    for (c = 0; c < I2; ++c) {
                        double s = 0.0;
                        for (p = 0; p < np; ++p) s += cq[p * H + h] * cq2[p * I2 + c];
                        ow[(long)h * I2 + c] = s;
                    }
                ORC_DIM1(hs, I, cq)
                ORC_DIM1(dys, H, cq2)
                for (ii = 0; ii < I; ++ii)
                    for (n = 0; n < H; ++n) {
                        double s = 0.0;
                        for (p = 0; p < np; ++p) s += cq[p * I + ii] * cq2[p * H + n];
                        od[(long)ii * H + n] = s;
                    }
#undef ORC_DIM1
            }
            free(cq); free(cq2);
        }
    next_e:
        free(WgK); free(Wg2); free(WdK); free(WdH); free(gu); free(hq); free(y); free(dyq);
        free(dh); free(dgu); free(fv); free(rl); free(xs); free(hs); free(dys); free(dgs);
    }
    if (bad) goto done;
    /* dx: the token's route input gradients summed over j ascending */
    for (i = 0; i < n_tok; ++i) {
        int j, h;
        for (h = 0; h < H; ++h) {
            double s = 0.0;
            for (j = 0; j < k; ++j) s += da[((long)i * k + j) * H + h];
            dx[(long)i * H + h] = s;
        }
    }
done:
    free(slot); free(exp_slot); free(xa); free(da);
    return bad ? -1 : 0;
}

/*
 * Gradient of the routing's gates with respect to the logits, for an upstream
 * gradient dgate [T, k] of the gates (the layer backward returns it).  The
 * gates are the softmax over all E renormalised over the k picks, which is the
 * softmax over the picked logits alone; the picks themselves are a piecewise
 * constant function of the logits, so only the picked entries get a gradient:
 * dl[t][ids[t][j]] = w_j (g_j - sum_i w_i g_i), everything else 0, with w the
 * routing's fp32 gates (the pages print no formula for this gradient).
 * dlogits [T, E] in double.  Returns 0, or -1 on a bad id.
 */
int oracle_route_backward(const int32_t *ids, const float *weights, const float *dgate, int T, int E, int k,
                          double *dlogits) {
    int t, j;
    for (t = 0; t < T; ++t) {
        double s = 0.0;
        double *row = dlogits + (long)t * E;
        for (j = 0; j < E; ++j) row[j] = 0.0;
        for (j = 0; j < k; ++j) s += (double)weights[(long)t * k + j] * (double)dgate[(long)t * k + j];
        for (j = 0; j < k; ++j) {
            long r = (long)t * k + j;
            if (ids[r] < 0 || ids[r] >= E) return -1;
            row[ids[r]] += (double)weights[r] * ((double)dgate[r] - s);
        }
    }
    return 0;
}
