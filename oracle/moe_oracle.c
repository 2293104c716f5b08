/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle for the routed mixture-of-experts
 * forward ("Experts backends" page).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant with the HIP library: it decodes every input format itself and
 * computes every step in fp64, one token and one selected expert at a time.
 *
 * What is computed (page "Experts backends"):
 *   - opening paragraph: for each token a router selects k experts, the hidden
 *     state is projected through the selected experts' parameters and the
 *     results are aggregated with the routing weights;
 *   - backend table, rows grouped_mm / deepgemm: tokens are ordered by their
 *     selected expert before one grouped GEMM;
 *   - backend table, row deepgemm_megamoe, and section "SonicMoE": each expert is
 *     a gated MLP -- up projection, gated activation, down projection; the
 *     gate is silu, gelu or relu (SwiGLU / GeGLU / ReGLU, section "SonicMoE");
 *   - paragraph under the backend table and section "FP8 and FP4 quantized
 *     experts": FP8 experts carry float32 or UE8M0 block scales, FP4 experts
 *     are int8-packed with UE8M0 scales, and activations are quantized with
 *     dynamic per-row scales (static per-tensor scales are rejected).
 *
 * Readings where the page is silent (the page gives no formula for the router,
 * no shapes and no block size):
 *   - score = softmax over all E experts, or a logistic sigmoid, of
 *     key[e] = x . W_r[e] + bias[e]; selection is on key itself, descending,
 *     ties to the lowest expert index; slots are in selection order;
 *   - optional renormalisation of the k selected scores to sum 1, then a
 *     multiplicative routed scale;
 *   - stable order within an expert: ascending (token, slot);
 *   - gated activation: a_j = act(g_j) * u_j with g = x W_gate^T, u = x W_up^T,
 *     no biases; silu(g) = g / (1 + e^-g), gelu(g) = g * Phi(g) with Phi the
 *     standard normal CDF (the exact form, 0.5 g (1 + erf(g / sqrt 2)); the
 *     page names gelu without saying which form), relu(g) = max(g, 0);
 *   - routing weight applied after the down projection;
 *   - FP8: OCP e4m3 ("fn": no infinities, 0x7f/0xff are NaN, max 448), weight
 *     block 128 x 128, activation group = 128 consecutive channels of one row,
 *     scale s = fl32(amax / 448), code = RNE_e4m3(fl32(v / s)) saturated at
 *     448, amax = 0 -> all codes 0.  The intermediate a (the SwiGLU output) is
 *     quantized the same way before the down projection.
 *   - FP4: OCP e2m1 codes, two per byte along K (even K in the low nibble),
 *     one UE8M0 scale per row per 32 consecutive K (the OCP MX block; the page
 *     gives no FP4 block size); activations as for FP8 (e4m3, per row per 128).
 *
 * Pins: every function here is checked by the CPU tests against closed forms,
 * library routines on special cases, brute force on tiny inputs and a worked
 * example computed by hand (tests/golden).  No function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* element formats understood by the oracle */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_E2M1 = 3 };
/* FP4 weight scale block: one UE8M0 scale per row per 32 consecutive K */
#define ORC_FP4_BLOCK 32
/* score functions */
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };
/* fp8 weight-scale formats */
enum { ORC_SCALE_NONE = 0, ORC_SCALE_F32 = 1, ORC_SCALE_UE8M0 = 2 };
/* gate activation of the gated MLP */
enum { ORC_GATE_SILU = 0, ORC_GATE_GELU = 1, ORC_GATE_RELU = 2 };

/* ------------------------------------------------------------------ decoders */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit float E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the two codes
 * with all exponent and mantissa bits set are NaN; there is no infinity. */
double orc_e4m3_to_f64(uint8_t code)
{
    int sign = code >> 7;
    int ex = (code >> 3) & 0xF;
    int man = code & 0x7;
    double v;
    if (ex == 0xF && man == 0x7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)man / 8.0, -6);
    else
        v = ldexp(1.0 + (double)man / 8.0, ex - 7);
    return sign ? -v : v;
}

/* OCP 4-bit float E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit;
 * exponent field 0 holds the subnormal m * 0.5; no NaN or infinity.  Values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.  `code` is one nibble. */
double orc_e2m1_to_f64(uint8_t code)
{
    int sign = (code >> 3) & 1;
    int ex = (code >> 1) & 3;
    int man = code & 1;
    double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return sign ? -v : v;
}

/* OCP E8M0 scale: an unsigned biased exponent, value 2^(b - 127); 0xff is NaN. */
double orc_e8m0_to_f64(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* Round v to the nearest finite E4M3 value, ties to the code with an even
 * mantissa (round-to-nearest-even), magnitudes beyond the largest finite value
 * saturating to +-448.  Written as an exhaustive search over the 127 finite
 * non-negative codes so that it can be checked by eye. */
uint8_t orc_e4m3_encode(double v)
{
    double a = fabs(v);
    if (a > 448.0)
        a = 448.0; /* saturation */
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(orc_e4m3_to_f64((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    if (best == 0)
        return 0; /* +0 whatever the sign of v */
    return (uint8_t)(v < 0 ? (0x80 | best) : best);
}

static double decode_elem(const void *base, int dt, int64_t idx)
{
    switch (dt) {
    case ORC_F32: return (double)((const float *)base)[idx];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)base)[idx]);
    case ORC_E4M3: return orc_e4m3_to_f64(((const uint8_t *)base)[idx]);
    default: return NAN;
    }
}

/* ------------------------------------------------------- activation grouping */

/* Dynamic quantization of one group of n values (one row, n consecutive
 * channels) and its dequantization, as read from section "FP8 and FP4 quantized
 * experts" (dynamic per-row activation scales).  deq[i] = code_i * s.  codes
 * and scale may be NULL. */
void orc_quant_group(const double *v, int n, double *deq, uint8_t *codes, float *scale)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    if (amax == 0.0) {
        for (int i = 0; i < n; ++i) {
            deq[i] = 0.0;
            if (codes) codes[i] = 0;
        }
        if (scale) *scale = 1.0f;
        return;
    }
    float s = (float)(amax / 448.0);
    for (int i = 0; i < n; ++i) {
        float r = (float)(v[i] / (double)s);
        uint8_t c = orc_e4m3_encode((double)r);
        deq[i] = orc_e4m3_to_f64(c) * (double)s;
        if (codes) codes[i] = c;
    }
    if (scale) *scale = s;
}

/* ------------------------------------------------------------------- routing */

/* Router of the opening paragraph: logits, key, top-k selection, weights.
 *   x      [T,H] in format xdt;  w_r [E,H] in format wdt;  bias [E] fp32 or NULL
 *   ids    [T,k] out, selected experts in slot order (descending key,
 *          ties to the lowest expert index)
 *   w      [T,k] out, routing weights
 *   keys   [T,E] out or NULL: z + bias, in fp64 */
void orc_route(int64_t T, int H, int E, int k,
               const void *x, int xdt, const void *w_r, int wdt, const float *bias,
               int score, int renormalize, double routed_scale,
               int32_t *ids, double *w, double *keys_out)
{
    int64_t t;
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < T; ++t) {
        double *key = (double *)malloc(sizeof(double) * (size_t)E);
        char *taken = (char *)calloc((size_t)E, 1);
        for (int e = 0; e < E; ++e) {
            double z = 0.0;
            for (int h = 0; h < H; ++h)
                z += decode_elem(x, xdt, t * H + h) * decode_elem(w_r, wdt, (int64_t)e * H + h);
            key[e] = z + (bias ? (double)bias[e] : 0.0);
            if (keys_out) keys_out[t * E + e] = key[e];
        }
        /* selection: k passes, each taking the largest remaining key; a strict
         * comparison keeps the lowest index among equal keys */
        for (int i = 0; i < k; ++i) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || key[e] > key[best]) best = e;
            }
            taken[best] = 1;
            ids[t * k + i] = best;
        }
        /* scores of the selected experts */
        double m = key[0];
        for (int e = 1; e < E; ++e) if (key[e] > m) m = key[e];
        double denom = 0.0;
        if (score == ORC_SOFTMAX)
            for (int e = 0; e < E; ++e) denom += exp(key[e] - m);
        double sum = 0.0;
        for (int i = 0; i < k; ++i) {
            double kv = key[ids[t * k + i]];
            double s = (score == ORC_SOFTMAX) ? exp(kv - m) / denom : 1.0 / (1.0 + exp(-kv));
            w[t * k + i] = s;
            sum += s;
        }
        for (int i = 0; i < k; ++i) {
            if (renormalize) w[t * k + i] /= sum;
            w[t * k + i] *= routed_scale;
        }
        free(key);
        free(taken);
    }
}

/* --------------------------------------------------------------- permutation */

/* Ordering of tokens by selected expert (backend table, grouped_mm row):
 * counts[e] pairs per expert; offsets[e] = exclusive prefix sum (E+1 entries);
 * stable order inside an expert, visiting (t, i) t-major;
 * perm[row] = t*k + i and inv[t*k + i] = row. */
void orc_permute(int64_t T, int k, int E, const int32_t *ids,
                 int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv)
{
    int64_t P = T * k;
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < P; ++p) counts[ids[p]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t p = 0; p < P; ++p) {
        int e = ids[p];
        int32_t row = offsets[e] + fill[e]++;
        perm[row] = (int32_t)p;
        inv[p] = row;
    }
    free(fill);
}

/* ------------------------------------------------------------------- experts */

typedef struct {
    int32_t H, I, E;
    int32_t wdt;        /* ORC_F32, ORC_BF16, ORC_E4M3 or ORC_E2M1 for all three matrices */
    int32_t scale_fmt;  /* ORC_SCALE_*; used only with ORC_E4M3 */
    int32_t block;      /* weight block edge and activation group size (fp8) */
    int32_t act_fp8;    /* quantize x and a per row per `block` channels */
    int32_t gate;       /* ORC_GATE_* */
    const void *w_gate; /* [E, I, H] */
    const void *w_up;   /* [E, I, H] */
    const void *w_down; /* [E, H, I] */
    const void *s_gate; /* [E, I/block, H/block] fp32 or e8m0 bytes */
    const void *s_up;   /* [E, I/block, H/block] */
    const void *s_down; /* [E, H/block, I/block] */
} orc_experts;

static double block_scale(const orc_experts *W, const void *s, int e, int r, int c, int rows, int cols)
{
    int br = rows / W->block, bc = cols / W->block;
    int64_t idx = ((int64_t)e * br + r / W->block) * bc + c / W->block;
    if (W->scale_fmt == ORC_SCALE_F32) return (double)((const float *)s)[idx];
    if (W->scale_fmt == ORC_SCALE_UE8M0) return orc_e8m0_to_f64(((const uint8_t *)s)[idx]);
    return 1.0;
}

/* one weight element of matrix m [E, rows, cols] as an exact fp64 value.
 * E2M1 ("int8-packed" FP4, paragraph under the backend table): two codes per
 * byte along cols, the even column in the low nibble, times the UE8M0 scale of
 * its (row, 32-column) block, s [E, rows, cols / 32]. */
static double weight(const orc_experts *W, const void *m, const void *s, int e, int r, int c,
                     int rows, int cols)
{
    if (W->wdt == ORC_E2M1) {
        int64_t idx = ((int64_t)e * rows + r) * cols + c;
        uint8_t byte = ((const uint8_t *)m)[idx / 2];
        double v = orc_e2m1_to_f64((c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15));
        int64_t sidx = ((int64_t)e * rows + r) * (cols / ORC_FP4_BLOCK) + c / ORC_FP4_BLOCK;
        return v * orc_e8m0_to_f64(((const uint8_t *)s)[sidx]);
    }
    double v = decode_elem(m, W->wdt, ((int64_t)e * rows + r) * cols + c);
    if (W->wdt == ORC_E4M3) v *= block_scale(W, s, e, r, c, rows, cols);
    return v;
}

static void quant_row(const orc_experts *W, const double *v, int n, double *out)
{
    for (int g = 0; g < n; g += W->block)
        orc_quant_group(v + g, W->block, out + g, NULL, NULL);
}

/* gate activation (section "SonicMoE": silu, gelu or relu) */
static double gate_act(int gate, double g)
{
    if (gate == ORC_GATE_GELU) return 0.5 * g * (1.0 + erf(g / sqrt(2.0)));
    if (gate == ORC_GATE_RELU) return g > 0.0 ? g : 0.0;
    return g / (1.0 + exp(-g));
}

/* Gated MLP of expert e on one row xin[H]:
 *   x^ = Q(x) (fp8 only), g = W_gate x^, u = W_up x^, a = act(g) * u,
 *   a^ = Q(a) (fp8 only), y = W_down a^.
 * h_out[I] (may be NULL) receives a^, y[H] receives y. */
void orc_expert_row(const orc_experts *W, int e, const double *xin, double *h_out, double *y)
{
    int H = W->H, I = W->I;
    double *xq = (double *)malloc(sizeof(double) * (size_t)H);
    double *a = (double *)malloc(sizeof(double) * (size_t)I);
    double *aq = (double *)malloc(sizeof(double) * (size_t)I);
    if (W->act_fp8) quant_row(W, xin, H, xq);
    else memcpy(xq, xin, sizeof(double) * (size_t)H);
    for (int j = 0; j < I; ++j) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            g += xq[h] * weight(W, W->w_gate, W->s_gate, e, j, h, I, H);
            u += xq[h] * weight(W, W->w_up, W->s_up, e, j, h, I, H);
        }
        a[j] = gate_act(W->gate, g) * u;
    }
    if (W->act_fp8) quant_row(W, a, I, aq);
    else memcpy(aq, a, sizeof(double) * (size_t)I);
    if (h_out) memcpy(h_out, aq, sizeof(double) * (size_t)I);
    for (int o = 0; o < H; ++o) {
        double acc = 0.0;
        for (int j = 0; j < I; ++j)
            acc += aq[j] * weight(W, W->w_down, W->s_down, e, o, j, H, I);
        y[o] = acc;
    }
    free(xq);
    free(a);
    free(aq);
}

/* Weighted aggregation of the opening paragraph for a list of tokens:
 *   out[n, :] = sum_i w[t, i] * y(t, i),  t = tokens[n],
 * where y(t, i) is the gated MLP of expert ids[t, i] on row x[t].  x is [T,H]
 * in format xdt; ids, w are [T,k]; out is [ntok, H] fp64. */
void orc_combine_tokens(const orc_experts *W, int k, const void *x, int xdt,
                        const int32_t *ids, const double *w,
                        const int64_t *tokens, int64_t ntok, double *out)
{
    int H = W->H;
    int64_t n;
#pragma omp parallel for schedule(dynamic, 1)
    for (n = 0; n < ntok; ++n) {
        int64_t t = tokens[n];
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *y = (double *)malloc(sizeof(double) * (size_t)H);
        for (int h = 0; h < H; ++h) xr[h] = decode_elem(x, xdt, t * H + h);
        for (int h = 0; h < H; ++h) out[n * H + h] = 0.0;
        for (int i = 0; i < k; ++i) {
            orc_expert_row(W, ids[t * k + i], xr, NULL, y);
            for (int h = 0; h < H; ++h) out[n * H + h] += w[t * k + i] * y[h];
        }
        free(xr);
        free(y);
    }
}

/* Expert outputs for a list of (token, expert) pairs, without the routing
 * weight: h[n, :] = a^ and y[n, :] = y for the pair (tokens[n], experts[n]).
 * Either output may be NULL. */
void orc_expert_pairs(const orc_experts *W, const void *x, int xdt,
                      const int64_t *tokens, const int32_t *experts, int64_t npairs,
                      double *h, double *y)
{
    int H = W->H, I = W->I;
    int64_t n;
#pragma omp parallel for schedule(dynamic, 1)
    for (n = 0; n < npairs; ++n) {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *hr = (double *)malloc(sizeof(double) * (size_t)I);
        double *yr = (double *)malloc(sizeof(double) * (size_t)H);
        for (int q = 0; q < H; ++q) xr[q] = decode_elem(x, xdt, tokens[n] * H + q);
        orc_expert_row(W, experts[n], xr, hr, yr);
        if (h) memcpy(h + n * I, hr, sizeof(double) * (size_t)I);
        if (y) memcpy(y + n * H, yr, sizeof(double) * (size_t)H);
        free(xr);
        free(hr);
        free(yr);
    }
}

/* Quantization of whole rows (x for the fp8 experts): codes [rows, n] and
 * scales [rows, n/group], as the per-row dynamic scheme reads. */
void orc_quant_rows(const void *x, int xdt, int64_t rows, int n, int group,
                    uint8_t *codes, float *scales)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        double *v = (double *)malloc(sizeof(double) * (size_t)group);
        double *d = (double *)malloc(sizeof(double) * (size_t)group);
        for (int g = 0; g < n / group; ++g) {
            for (int i = 0; i < group; ++i) v[i] = decode_elem(x, xdt, r * n + g * group + i);
            orc_quant_group(v, group, d, codes + r * n + g * group, scales + r * (n / group) + g);
        }
        free(v);
        free(d);
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
