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
 *   - opening paragraph: each token's router scores pick k experts, each
 *     picked expert transforms the token's hidden state with its own weights,
 *     and the k results are added up, each scaled by its routing weight;
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
 *     ties to the lowest expert index; slots are in selection order; a NaN
 *     key ranks as -inf (the page says nothing of non-finite inputs);
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
 * Backward (section "SonicMoE": training of the gated-MLP experts): the
 * gradients of every input and parameter for a given output gradient, with the
 * top-k selection held fixed (orc_bwd_tokens, orc_bwd_expert_rows,
 * orc_bwd_router; formulas in the comment above them).
 *
 * Pins: every function here is checked by the CPU tests against closed forms,
 * library routines on special cases, brute force on tiny inputs and a worked
 * example computed by hand (tests/golden); the backward against central finite
 * differences of this file's forward and a dense autograd formulation.  No
 * function is "parity unpinned".
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
            /* a NaN key (a NaN among the token's or the router's values)
             * ranks as -inf: below every number, tied with -inf, so the
             * lowest untaken index wins among such keys */
            if (isnan(key[e])) key[e] = -INFINITY;
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

/* ------------------------------------------------------------------ backward */

/* Backward of the layer ("Experts backends", section "SonicMoE": the page
 * names training of the gated-MLP experts as SonicMoE's focus; the gradient
 * formulas are those of the forward above differentiated by hand).  Given the
 * gradient dout[T,H] of the output, with the selection ids held fixed (the
 * top-k choice is piecewise constant in the inputs):
 *   dw[t,i]  = dout_t . y(t,i)                         (routing weight)
 *   dy       = w[t,i] dout_t,  da = W_down^T dy
 *   dg       = da * u * act'(g),  du = da * act(g)
 *   dx_t     = sum_i (W_gate^T dg + W_up^T du) + sum_e dkey[t,e] W_r[e]
 *   dW_down[e] = sum over the pairs of e of dy a^T, dW_gate[e] = sum dg x^T,
 *   dW_up[e] = sum du x^T,  dW_r = dkey^T x,  dbias = sum_t dkey[t,:]
 * where dkey is the gradient of the router key through the score function,
 * the renormalisation and the routed scale.  Experts in F32 or BF16 only (no
 * quantizer in the backward). */

/* derivative of the gate activation */
static double gate_act_deriv(int gate, double g)
{
    if (gate == ORC_GATE_GELU) {
        double Phi = 0.5 * (1.0 + erf(g / sqrt(2.0)));
        double phi = exp(-0.5 * g * g) / sqrt(2.0 * 3.14159265358979323846);
        return Phi + g * phi;
    }
    if (gate == ORC_GATE_RELU) return g > 0.0 ? 1.0 : 0.0;
    double sg = 1.0 / (1.0 + exp(-g));
    return sg * (1.0 + g * (1.0 - sg));
}

/* g, u and a = act(g) * u of expert e on the fp64 row xr */
static void expert_gua(const orc_experts *W, int e, const double *xr, double *g, double *u, double *a)
{
    int H = W->H, I = W->I;
    for (int j = 0; j < I; ++j) {
        double gj = 0.0, uj = 0.0;
        for (int h = 0; h < H; ++h) {
            gj += xr[h] * weight(W, W->w_gate, W->s_gate, e, j, h, I, H);
            uj += xr[h] * weight(W, W->w_up, W->s_up, e, j, h, I, H);
        }
        g[j] = gj;
        u[j] = uj;
        a[j] = gate_act(W->gate, gj) * uj;
    }
}

/* da = W_down[e]^T dy */
static void down_transpose(const orc_experts *W, int e, const double *dy, double *da)
{
    int H = W->H, I = W->I;
    for (int j = 0; j < I; ++j) {
        double s = 0.0;
        for (int o = 0; o < H; ++o) s += dy[o] * weight(W, W->w_down, W->s_down, e, o, j, H, I);
        da[j] = s;
    }
}

/* Token-side gradients for a list of tokens.  keys [T,E] are the router keys
 * (logits plus bias), ids and w [T,k] the selection and routing weights of the
 * forward; dout [T,H] fp64.  Out, per listed token n: dx [n,H], dw [n,k],
 * dkey [n,E] (any may be NULL except dx). */
void orc_bwd_tokens(const orc_experts *W, int64_t T, int k, const void *x, int xdt,
                    const void *w_r, int wdt, int score, int renormalize, double routed_scale,
                    const double *keys, const int32_t *ids, const double *w, const double *dout,
                    const int64_t *tokens, int64_t ntok, double *dx, double *dw_out, double *dkey_out)
{
    int H = W->H, I = W->I, E = W->E;
    int64_t n;
    (void)T;
#pragma omp parallel for schedule(dynamic, 1)
    for (n = 0; n < ntok; ++n) {
        int64_t t = tokens[n];
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        double *da = (double *)malloc(sizeof(double) * (size_t)I);
        double *dy = (double *)malloc(sizeof(double) * (size_t)H);
        double *dwt = (double *)malloc(sizeof(double) * (size_t)k);
        double *s = (double *)malloc(sizeof(double) * (size_t)E);
        double *ds = (double *)calloc((size_t)E, sizeof(double));
        double *dkey = (double *)malloc(sizeof(double) * (size_t)E);
        double *dxr = dx + n * H;
        const double *dot = dout + t * H;
        for (int h = 0; h < H; ++h) {
            xr[h] = decode_elem(x, xdt, t * H + h);
            dxr[h] = 0.0;
        }
        for (int i = 0; i < k; ++i) {
            int e = ids[t * k + i];
            double wi = w[t * k + i];
            expert_gua(W, e, xr, g, u, a);
            /* dw = dout . y with y = W_down a */
            double d = 0.0;
            for (int o = 0; o < H; ++o) {
                double yo = 0.0;
                for (int j = 0; j < I; ++j) yo += a[j] * weight(W, W->w_down, W->s_down, e, o, j, H, I);
                d += dot[o] * yo;
            }
            dwt[i] = d;
            for (int o = 0; o < H; ++o) dy[o] = wi * dot[o];
            down_transpose(W, e, dy, da);
            for (int j = 0; j < I; ++j) {
                double dg = da[j] * u[j] * gate_act_deriv(W->gate, g[j]);
                double du = da[j] * gate_act(W->gate, g[j]);
                for (int h = 0; h < H; ++h)
                    dxr[h] += dg * weight(W, W->w_gate, W->s_gate, e, j, h, I, H) +
                              du * weight(W, W->w_up, W->s_up, e, j, h, I, H);
            }
        }
        /* scores of all experts (softmax over all E, or sigmoid) */
        const double *key = keys + t * E;
        if (score == ORC_SOFTMAX) {
            double m = key[0], den = 0.0;
            for (int e = 1; e < E; ++e) if (key[e] > m) m = key[e];
            for (int e = 0; e < E; ++e) den += exp(key[e] - m);
            for (int e = 0; e < E; ++e) s[e] = exp(key[e] - m) / den;
        } else {
            for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + exp(-key[e]));
        }
        /* through the routed scale and the renormalisation: w_i = c s_i / S */
        double S = 0.0, dws = 0.0;
        for (int i = 0; i < k; ++i) {
            S += s[ids[t * k + i]];
            dws += dwt[i] * s[ids[t * k + i]];
        }
        for (int i = 0; i < k; ++i) {
            int e = ids[t * k + i];
            ds[e] = renormalize ? routed_scale * (dwt[i] / S - dws / (S * S)) : routed_scale * dwt[i];
        }
        /* through the score function */
        if (score == ORC_SOFTMAX) {
            double sds = 0.0;
            for (int e = 0; e < E; ++e) sds += s[e] * ds[e];
            for (int e = 0; e < E; ++e) dkey[e] = s[e] * (ds[e] - sds);
        } else {
            for (int e = 0; e < E; ++e) dkey[e] = ds[e] * s[e] * (1.0 - s[e]);
        }
        for (int e = 0; e < E; ++e)
            for (int h = 0; h < H; ++h) dxr[h] += dkey[e] * decode_elem(w_r, wdt, (int64_t)e * H + h);
        if (dw_out) memcpy(dw_out + n * k, dwt, sizeof(double) * (size_t)k);
        if (dkey_out) memcpy(dkey_out + n * E, dkey, sizeof(double) * (size_t)E);
        free(xr); free(g); free(u); free(a); free(da); free(dy); free(dwt); free(s); free(ds); free(dkey);
    }
}

/* Rows of one expert's weight gradient, summed over that expert's (token,
 * slot) pairs in token-major order.  which: 0 dW_gate [I,H], 1 dW_up [I,H],
 * 2 dW_down [H,I]; rows [nrows] are row indices of that matrix; out
 * [nrows, cols] fp64.  The per-pair vectors (a, or dg / du) are computed
 * first, then each requested row is a sum of outer-product rows. */
void orc_bwd_expert_rows(const orc_experts *W, int which, int e, const int32_t *rows, int nrows,
                         int64_t T, int k, const void *x, int xdt, const int32_t *ids, const double *w,
                         const double *dout, double *out)
{
    int H = W->H, I = W->I;
    int cols = which == 2 ? I : H;
    int64_t np_ = 0, q;
    int r;
    for (int64_t p = 0; p < T * k; ++p) np_ += ids[p] == e;
    int64_t *pairs = (int64_t *)malloc(sizeof(int64_t) * (size_t)(np_ + 1));
    np_ = 0;
    for (int64_t p = 0; p < T * k; ++p) if (ids[p] == e) pairs[np_++] = p;
    /* per pair: a (down) or the channel gradient d = dg or du (gate / up), [np_, I] */
    double *vec = (double *)malloc(sizeof(double) * (size_t)(np_ * I + 1));
#pragma omp parallel for schedule(dynamic, 1)
    for (q = 0; q < np_; ++q) {
        int64_t t = pairs[q] / k;
        double wi = w[pairs[q]];
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        double *dy = (double *)malloc(sizeof(double) * (size_t)H);
        double *da = (double *)malloc(sizeof(double) * (size_t)I);
        double *v = vec + q * I;
        for (int h = 0; h < H; ++h) xr[h] = decode_elem(x, xdt, t * H + h);
        expert_gua(W, e, xr, g, u, a);
        if (which == 2) {
            memcpy(v, a, sizeof(double) * (size_t)I);
        } else {
            for (int o = 0; o < H; ++o) dy[o] = wi * dout[t * H + o];
            down_transpose(W, e, dy, da);
            for (int j = 0; j < I; ++j)
                v[j] = which == 0 ? da[j] * u[j] * gate_act_deriv(W->gate, g[j]) : da[j] * gate_act(W->gate, g[j]);
        }
        free(xr); free(g); free(u); free(a); free(dy); free(da);
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (r = 0; r < nrows; ++r) {
        double *orow = out + (int64_t)r * cols;
        int row = rows[r];
        for (int c = 0; c < cols; ++c) orow[c] = 0.0;
        for (int64_t q2 = 0; q2 < np_; ++q2) {
            int64_t t = pairs[q2] / k;
            if (which == 2) {
                /* dW_down[o, :] += dy[o] a with dy = w dout_t */
                double dyo = w[pairs[q2]] * dout[t * H + row];
                for (int j = 0; j < I; ++j) orow[j] += dyo * vec[q2 * I + j];
            } else {
                /* dW_gate[j, :] += dg[j] x_t  (dW_up: du[j] x_t) */
                double d = vec[q2 * I + row];
                for (int h = 0; h < H; ++h) orow[h] += d * decode_elem(x, xdt, t * H + h);
            }
        }
    }
    free(pairs);
    free(vec);
}

/* Router parameter gradients from dkey [T,E]: dW_r [E,H] = dkey^T x and
 * dbias [E] = column sums of dkey, both summed in token order. */
void orc_bwd_router(int64_t T, int H, int E, const void *x, int xdt, const double *dkey,
                    double *dwr, double *dbias)
{
    int e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < E; ++e) {
        double b = 0.0;
        for (int h = 0; h < H; ++h) dwr[(int64_t)e * H + h] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double d = dkey[t * E + e];
            b += d;
            for (int h = 0; h < H; ++h) dwr[(int64_t)e * H + h] += d * decode_elem(x, xdt, t * H + h);
        }
        dbias[e] = b;
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
