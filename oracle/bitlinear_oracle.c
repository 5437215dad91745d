/*
 * bitlinear_oracle.c -- plain, slow CPU oracle of the BitNet b1.58 BitLinear path.
 *
 * TEST INFRASTRUCTURE. This is the independent reference that the HIP path is
 * checked against. Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it. The product library neither links nor calls it,
 * and the two share no code, header, table or constant.
 *
 * Pages this follows (title, then section):
 *  [BN] "BitNet Model - Complete Inference Pipeline" (Hesper API, Models.BitNet):
 *       "Model Configurations", "Memory Footprint (BitNet-3B with TQ2_0)",
 *       "Text Generation / Greedy Decoding", "GPU Argmax" (argmaxKernel).
 *  [TB] "Transformer Block" (Hesper API, Layers.TransformerBlock):
 *       "Feed-Forward Network (FFN)", "Memory Layout", "Layer Structure"
 *       (ffnNorm, ffnGate, ffnUp, ffnSubNorm, ffnDown), "Forward Pass" steps 4-8.
 *  [CA] "Add Support for BitNet Architecture Inference" (candle PR 2664): the
 *       reply that lists the changes -- an RMSNorm in front of every BitLinear,
 *       and the activation_quant / weight_quant pair.
 *  The pages name the quantizers but print no formula. They follow the BitNet
 *  b1.58 method that [BN] and [TB] reference (arXiv 2402.17764): one absmean
 *  scale per weight tensor with weights rounded to {-1, 0, +1}, and per-token
 *  absmax scaling of activations to 8-bit integers, integer accumulation, one
 *  float rescale at the end.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - Rounding is round-half-to-even (nearbyint in the default FP mode).
 *  - Activation codes are clamped to [-128, 127]; the absmax element lands on
 *    +-127, so -128 never occurs.
 *  - The floor on absmax and on mean|W| is 1e-5.
 *  - TQ2_0 byte layout: code c = t + 1 in {0, 1, 2}, four 2-bit fields per byte,
 *    least significant field first; byte i of a row holds k = 4i .. 4i+3.
 *    Code 3 is invalid. Weights are stored W[N_out][K_in], K contiguous.
 *  - RMSNorm: y = fl32(fl32(x * r) * g), r = fl32(1 / sqrt(ss / K + eps)) taken
 *    in fp64; ss is the fp64 sum of squares in one fixed order: 512 strided
 *    partials (partial l sums k = l, l+512, ... ascending), then a pairwise
 *    xor-butterfly over the partials with offsets 1, 2, 4, ..., 256.
 *  - Dequant: inv = fl32(1 / fl32(s_a * s_w)) once per (token, tensor), then
 *    y = fl32((float)acc * inv).
 *  - FFN: h = fl32(fl32(relu(gate) * relu(gate)) * up), then the sub-norm and
 *    activation quant of h, then the down projection. No residual inside.
 *  - Argmax ties go to the lowest index.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (OpenMP only splits independent
 * rows/tokens; every result is the same for any thread count).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EPS_FLOOR 1e-5
#define ORACLE_PARTIALS 512

int ref_abi_version(void) { return 1; }

/* Threads of the row-parallel loops (OpenMP); results do not depend on it.
 * n <= 0 leaves the current setting. Returns the setting in effect. */
int ref_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* weight_quant ([CA] weight_quant; absmean ternary rounding of the b1.58
 * method): s_w = 1 / mean|W| over the whole tensor, t = clamp(rne(W * s_w)).
 * mean|W| is an fp64 sum in row-major order divided by N*K; s_w is the fp64
 * reciprocal rounded once to fp32; each W*s_w is an fp32 product.           */
int ref_weight_quant(const float *w, int64_t n, int64_t k, int8_t *t, float *s_w)
{
    if (n <= 0 || k <= 0) return -2;
    double sum = 0.0;
    for (int64_t i = 0; i < n * k; i++) {
        if (!isfinite(w[i])) return -4;
        sum += fabs((double)w[i]);
    }
    double mean = sum / (double)(n * k);
    if (mean < ORACLE_EPS_FLOOR) mean = ORACLE_EPS_FLOOR;
    float scale = (float)(1.0 / mean);
    *s_w = scale;
    for (int64_t i = 0; i < n * k; i++) {
        float v = w[i] * scale;
        float r = nearbyintf(v);
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        t[i] = (int8_t)r;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* TQ2_0 codec ([BN] "Memory Footprint": 0.25 byte per weight; layout is the
 * reading stated in the header). pack: P[n][i] = sum_j (t[n][4i+j] + 1) << 2j. */
int ref_pack(const int8_t *t, int64_t n, int64_t k, uint8_t *packed)
{
    if (n <= 0 || k <= 0) return -2;
    if (k % 4 != 0) return -2;
    for (int64_t i = 0; i < n * k; i++)
        if (t[i] < -1 || t[i] > 1) return -4;
    int64_t kb = k / 4;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t i = 0; i < kb; i++) {
            unsigned byte = 0;
            for (int j = 0; j < 4; j++) {
                unsigned code = (unsigned)(t[r * k + 4 * i + j] + 1);
                byte |= code << (2 * j);
            }
            packed[r * kb + i] = (uint8_t)byte;
        }
    }
    return 0;
}

/* unpack: inverse of ref_pack; a field holding code 3 is rejected (-4). */
int ref_unpack(const uint8_t *packed, int64_t n, int64_t k, int8_t *t)
{
    if (n <= 0 || k <= 0 || k % 4 != 0) return -2;
    int64_t kb = k / 4;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t i = 0; i < kb; i++) {
            unsigned byte = packed[r * kb + i];
            for (int j = 0; j < 4; j++) {
                unsigned code = (byte >> (2 * j)) & 3u;
                if (code == 3u) return -4;
                t[r * k + 4 * i + j] = (int8_t)((int)code - 1);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm sum of squares in the fixed order stated in the header. Each x^2 is
 * exact in fp64 (a 24-bit significand squared fits in 53 bits).              */
double ref_sumsq(const float *x, int64_t k)
{
    double p[ORACLE_PARTIALS], c[ORACLE_PARTIALS];
    for (int l = 0; l < ORACLE_PARTIALS; l++) p[l] = 0.0;
    for (int64_t i = 0; i < k; i++) {
        double v = (double)x[i];
        p[i % ORACLE_PARTIALS] += v * v;
    }
    for (int off = 1; off < ORACLE_PARTIALS; off *= 2) {
        memcpy(c, p, sizeof p);
        for (int l = 0; l < ORACLE_PARTIALS; l++) p[l] = c[l] + c[l ^ off];
    }
    return p[0];
}

/* RMSNorm ([TB] "Layer Structure": attnNorm/ffnNorm/ffnSubNorm; [CA]: a norm in
 * front of every BitLinear). y[m][k] = fl32(fl32(x * r) * g[k]). g == NULL is
 * not allowed here (the caller skips the norm instead).                       */
int ref_rmsnorm(const float *x, const float *g, float eps, int64_t m, int64_t k, float *y)
{
    if (m <= 0 || k <= 0 || !g) return -2;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t row = 0; row < m; row++) {
        const float *xr = x + row * k;
        for (int64_t i = 0; i < k; i++)
            if (!isfinite(xr[i])) bad = 1;
        double ss = ref_sumsq(xr, k);
        double r64 = 1.0 / sqrt(ss / (double)k + (double)eps);
        float r = (float)r64;
        for (int64_t i = 0; i < k; i++) {
            float a = xr[i] * r;
            y[row * k + i] = a * g[i];
        }
    }
    return bad ? -4 : 0;
}

/* activation_quant ([CA]; per-token absmax of the b1.58 method):
 * s_a = fl32(127 / max(absmax, 1e-5)), q = clamp(rne(fl32(y * s_a)), -128, 127),
 * qsum = sum of q in int32.                                                   */
int ref_activation_quant(const float *y, int64_t m, int64_t k, int8_t *q, float *s_a, int32_t *qsum)
{
    if (m <= 0 || k <= 0) return -2;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t row = 0; row < m; row++) {
        const float *yr = y + row * k;
        float amax = 0.0f;
        for (int64_t i = 0; i < k; i++) {
            if (!isfinite(yr[i])) bad = 1;
            float a = fabsf(yr[i]);
            if (a > amax) amax = a;
        }
        float floor_ = (float)ORACLE_EPS_FLOOR;
        float scale = 127.0f / (amax > floor_ ? amax : floor_);
        s_a[row] = scale;
        int32_t sum = 0;
        for (int64_t i = 0; i < k; i++) {
            float v = yr[i] * scale;
            float r = nearbyintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -128.0f) r = -128.0f;
            int8_t qi = (int8_t)r;
            q[row * k + i] = qi;
            sum += qi;
        }
        if (qsum) qsum[row] = sum;
    }
    return bad ? -4 : 0;
}

/* ------------------------------------------------------------------------ */
/* Ternary x int8 matmul: acc[m][n] = sum_k t[n][k] * q[m][k], exact in int32
 * (|acc| <= 127 K < 2^31 for every K this path sees).                        */
int ref_matmul_i32(const int8_t *t, const int8_t *q, int64_t m, int64_t n, int64_t k, int32_t *acc)
{
    if (m <= 0 || n <= 0 || k <= 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t col = 0; col < n; col++) {
        const int8_t *tr = t + col * k;
        for (int64_t row = 0; row < m; row++) {
            const int8_t *qr = q + row * k;
            int32_t s = 0;
            for (int64_t i = 0; i < k; i++) s += (int32_t)tr[i] * (int32_t)qr[i];
            acc[row * n + col] = s;
        }
    }
    return 0;
}

/* Dequant: one float rescale by 1/(s_a * s_w) per (token, tensor).           */
int ref_dequant(const int32_t *acc, const float *s_a, float s_w, int64_t m, int64_t n, float *y)
{
    if (m <= 0 || n <= 0) return -2;
    for (int64_t row = 0; row < m; row++) {
        float prod = s_a[row] * s_w;
        float inv = 1.0f / prod;
        for (int64_t col = 0; col < n; col++) y[row * n + col] = (float)acc[row * n + col] * inv;
    }
    return 0;
}

/* One BitLinear on quantized activations: unpack, exact matmul, dequant.
 * acc may be NULL.                                                            */
int ref_bitlinear(const uint8_t *packed, float s_w, int64_t n, int64_t k, const int8_t *q,
                  const float *s_a, int64_t m, float *y, int32_t *acc)
{
    if (m <= 0 || n <= 0 || k <= 0 || k % 4 != 0) return -2;
    int8_t *t = (int8_t *)malloc((size_t)(n * k));
    int32_t *a = acc ? acc : (int32_t *)malloc((size_t)(m * n) * sizeof(int32_t));
    if (!t || !a) {
        free(t);
        if (!acc) free(a);
        return -7;
    }
    int rc = ref_unpack(packed, n, k, t);
    if (rc == 0) rc = ref_matmul_i32(t, q, m, n, k, a);
    if (rc == 0) rc = ref_dequant(a, s_a, s_w, m, n, y);
    free(t);
    if (!acc) free(a);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* FFN gating ([TB] "Feed-Forward Network (FFN)": the gate goes through a
 * squared ReLU, then multiplies the up projection elementwise).             */
void ref_relu2_mul(const float *gate, const float *up, int64_t count, float *h)
{
    for (int64_t i = 0; i < count; i++) {
        float g = gate[i] > 0.0f ? gate[i] : 0.0f;
        float g2 = g * g;
        h[i] = g2 * up[i];
    }
}

/* Residual add ([TB] "Forward Pass" steps 3 and 9): x = fl32(x + d).        */
void ref_residual_add(float *x, const float *d, int64_t count)
{
    for (int64_t i = 0; i < count; i++) x[i] = x[i] + d[i];
}

/* Greedy token choice ([BN] "Greedy Decoding", "GPU Argmax"): per row, the
 * lowest index holding the maximum accumulator.                              */
int ref_argmax_rows(const int32_t *acc, int64_t m, int64_t n, int32_t *idx)
{
    if (m <= 0 || n <= 0) return -2;
    for (int64_t row = 0; row < m; row++) {
        const int32_t *a = acc + row * n;
        int64_t best = 0;
        for (int64_t col = 1; col < n; col++)
            if (a[col] > a[best]) best = col;
        idx[row] = (int32_t)best;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Ternary embedding lookup ([BN] "Architecture": the embedding layer is TQ2_0
 * quantized; "Memory Footprint": 50000 x 2560 x 0.25 bytes). Row tokens[r] of
 * the packed table, dequantized like every ternary tensor, W = t / s_e:
 * x[r][k] = fl32(t / s_e). A token id outside [0, vocab) gives a zero row.    */
int ref_embed(const uint8_t *table, float s_e, int64_t vocab, int64_t d, const int32_t *tokens, int64_t m,
              float *x)
{
    if (vocab <= 0 || d <= 0 || m <= 0 || d % 4 != 0) return -2;
    if (!(s_e > 0.0f)) return -4;
    int8_t *t = (int8_t *)malloc((size_t)d);
    if (!t) return -7;
    int rc = 0;
    for (int64_t r = 0; r < m && rc == 0; r++) {
        const int64_t tok = tokens[r];
        if (tok < 0 || tok >= vocab) {
            for (int64_t k = 0; k < d; k++) x[r * d + k] = 0.0f;
            continue;
        }
        rc = ref_unpack(table + tok * (d / 4), 1, d, t);
        for (int64_t k = 0; k < d && rc == 0; k++) x[r * d + k] = (float)t[k] / s_e;
    }
    free(t);
    return rc;
}

/* Repetition penalty, then the greedy choice ([BN] "GPU Argmax":
 * repetitionPenaltyKernel penalises the logit of every previous token in
 * place, gpuArgmaxWithPenalty then takes the argmax; "Text Generation":
 * repetitionPenalty = 1.1 by default). Per row r, every distinct token id v of
 * hist[r][0 .. hist_len[r]) with 0 <= v < n has its logit l replaced, once, by
 * fl32(l / penalty) if l > 0 and by fl32(l * penalty) otherwise; ids outside
 * [0, n) are ignored. idx[r] = the lowest n holding the largest penalised
 * logit. logits is updated in place.                                          */
int ref_penalty_argmax(float *logits, int64_t m, int64_t n, const int32_t *hist, int64_t hist_stride,
                       const int32_t *hist_len, float penalty, int32_t *idx)
{
    if (m <= 0 || n <= 0 || hist_stride < 0) return -2;
    if (!(penalty > 0.0f)) return -4;
    unsigned char *seen = (unsigned char *)malloc((size_t)n);
    if (!seen) return -7;
    for (int64_t r = 0; r < m; r++) {
        float *l = logits + r * n;
        memset(seen, 0, (size_t)n);
        int64_t len = hist_len ? hist_len[r] : 0;
        if (len > hist_stride) len = hist_stride;
        for (int64_t i = 0; i < len; i++) {
            const int64_t v = hist[r * hist_stride + i];
            if (v < 0 || v >= n || seen[v]) continue;
            seen[v] = 1;
            l[v] = l[v] > 0.0f ? l[v] / penalty : l[v] * penalty;
        }
        int64_t best = 0;
        for (int64_t c = 1; c < n; c++)
            if (l[c] > l[best]) best = c;
        idx[r] = (int32_t)best;
    }
    free(seen);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Top-k and nucleus (top-p) sampling ([BN] "Text Generation": Top-k Sampling,
 * Nucleus (Top-p) Sampling; sampleTopK / sampleNucleus with a temperature and
 * a random number generator). The random numbers are inputs: u[r] uniform in
 * [0, 1), one per row. Readings (the pages give the steps, not the arithmetic):
 *  - tokens are taken in the pages' sorted order: descending logit, the lower
 *    index first among equal logits;
 *  - the softmax weight of token i is e^((l_i - l_max) / T), with the
 *    exponential below, rounded to a fixed-point integer with 40 fractional
 *    bits (weights below 2^-41 of the largest become 0), so every sum of
 *    weights is exact whatever its order;
 *  - top-k keeps the first min(k, n) tokens of the sorted order;
 *  - the nucleus is the shortest prefix of the sorted order whose weight
 *    reaches ceil(p * Z), Z the total weight (the smallest set with cumulative
 *    probability >= p of sampleNucleus; at least one token);
 *  - sampling draws r = floor(u * M), M the kept weight, and picks the first
 *    kept token in sorted order whose cumulative weight exceeds r.            */

/* e^x for x in [-32, 0] in fp64: Cody-Waite range reduction x = k ln2 + r
 * (ln2 split into a 32-significant-bit head, so k * head is exact, and a
 * tail), e^r from its Taylor series through r^13 / 13! by Horner's rule
 * (|r| <= 0.35: truncation below 2^-58), then the exact scaling by 2^k.
 * Below -32 the result is 0 (it would round to a zero weight anyway).       */
static const double ORACLE_LN2_HEAD = 0x1.62e42fee00000p-1;
static const double ORACLE_LN2_TAIL = 0x1.a39ef35793c76p-33;
static const double ORACLE_INV_LN2 = 0x1.71547652b82fep+0;

double ref_exp_neg(double x)
{
    if (x < -32.0) return 0.0;
    const double k = nearbyint(x * ORACLE_INV_LN2);
    const double r = (x - k * ORACLE_LN2_HEAD) - k * ORACLE_LN2_TAIL;
    /* coefficients 1 / j! for j = 13 .. 0 */
    static const double inv_fact[14] = {1.0,
                                        1.0,
                                        1.0 / 2.0,
                                        1.0 / 6.0,
                                        1.0 / 24.0,
                                        1.0 / 120.0,
                                        1.0 / 720.0,
                                        1.0 / 5040.0,
                                        1.0 / 40320.0,
                                        1.0 / 362880.0,
                                        1.0 / 3628800.0,
                                        1.0 / 39916800.0,
                                        1.0 / 479001600.0,
                                        1.0 / 6227020800.0};
    double poly = inv_fact[13];
    for (int j = 12; j >= 0; j--) poly = poly * r + inv_fact[j];
    return ldexp(poly, (int)k);
}

static const float *sample_row_logits;

static int sample_order_cmp(const void *pa, const void *pb)
{
    const int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    const float la = sample_row_logits[a], lb = sample_row_logits[b];
    if (la != lb) return la > lb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* mode 0: top-k with k; mode 1: nucleus with p. idx[r] = the sampled token.  */
int ref_sample(const float *logits, int64_t m, int64_t n, int mode, int64_t k, float p, float temperature,
               const double *u, int32_t *idx)
{
    if (m <= 0 || n <= 0 || (mode != 0 && mode != 1)) return -2;
    if (!(temperature > 0.0f) || (mode == 0 && k <= 0) || (mode == 1 && !(p > 0.0f))) return -4;
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    int64_t *w = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!order || !w) {
        free(order);
        free(w);
        return -7;
    }
    for (int64_t row = 0; row < m; row++) {
        const float *l = logits + row * n;
        float lmax = l[0];
        for (int64_t i = 1; i < n; i++)
            if (l[i] > lmax) lmax = l[i];
        int64_t total = 0;
        for (int64_t i = 0; i < n; i++) {
            const double x = ((double)l[i] - (double)lmax) / (double)temperature;
            w[i] = (int64_t)nearbyint(ldexp(ref_exp_neg(x), 40));
            total += w[i];
        }
        for (int64_t i = 0; i < n; i++) order[i] = i;
        sample_row_logits = l;
        qsort(order, (size_t)n, sizeof(int64_t), sample_order_cmp);
        int64_t kept = 0; /* number of kept tokens (a prefix of order) */
        if (mode == 0) {
            kept = k < n ? k : n;
        } else {
            double tgt = ceil((double)p * (double)total);
            int64_t target = tgt > (double)total ? total : (int64_t)tgt;
            if (target < 1) target = 1;
            int64_t cum = 0;
            while (kept < n && cum < target) cum += w[order[kept++]];
        }
        int64_t mass = 0;
        for (int64_t j = 0; j < kept; j++) mass += w[order[j]];
        double rd = floor(u[row] * (double)mass);
        int64_t r = rd < 0.0 ? 0 : (rd >= (double)mass ? mass - 1 : (int64_t)rd);
        int64_t cum = 0, chosen = order[0];
        for (int64_t j = 0; j < kept; j++) {
            cum += w[order[j]];
            if (cum > r) {
                chosen = order[j];
                break;
            }
        }
        idx[row] = (int32_t)chosen;
    }
    free(order);
    free(w);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Single-token attention with a KV cache and rotary position embedding
 * ([BN] "KV Cache State", forwardSingleToken; [TB] "Forward Pass with KV
 * Cache", forwardWithCache; Config: numHeads, headDim, ropeBase). Readings:
 * heads h = 0 .. H-1 own columns h * hd .. h * hd + hd - 1 of q, k and v
 * (hd = d / H, numKVHeads = H); the rotation is RoFormer's: within a head the
 * pairs (x[2i], x[2i+1]) turn by the angle pos * theta_i, theta_i =
 * base^(-2i / hd); the rotated k and v of position pos join the cache, and the
 * head's output is softmax(q . K^T / sqrt(hd)) V over positions 0 .. pos.     */

/* cos / sin table [max_pos][hd / 2]: theta_i = pow(base, -(2 i) / hd) and the
 * angle pos * theta_i in fp64, cos and sin in fp64, each rounded once to fp32. */
int ref_rope_table(double base, int64_t hd, int64_t max_pos, float *cos_t, float *sin_t)
{
    if (hd <= 0 || hd % 2 != 0 || max_pos <= 0 || !(base > 1.0)) return -2;
    for (int64_t p = 0; p < max_pos; p++)
        for (int64_t i = 0; i < hd / 2; i++) {
            const double theta = pow(base, -(double)(2 * i) / (double)hd);
            const double ang = (double)p * theta;
            cos_t[p * (hd / 2) + i] = (float)cos(ang);
            sin_t[p * (hd / 2) + i] = (float)sin(ang);
        }
    return 0;
}

/* Rotation of one head vector in fp32 with the table row c, s (hd / 2 each):
 * (a, b) -> (fl32(fl32(a c) - fl32(b s)), fl32(fl32(a s) + fl32(b c))).      */
void ref_rope_apply(float *x, const float *c, const float *s, int64_t hd)
{
    for (int64_t i = 0; i < hd / 2; i++) {
        const float a = x[2 * i], b = x[2 * i + 1];
        const float ac = a * c[i], bs = b * s[i], as = a * s[i], bc = b * c[i];
        x[2 * i] = ac - bs;
        x[2 * i + 1] = as + bc;
    }
}

/* Attention of one query per sequence over cache positions 0 .. pos, in fp64
 * (scores, softmax, weighted sum), rounded once to fp32.
 *   q : [m][H][hd] (rotated); k_cache, v_cache : [m][H][max_seq][hd];
 *   out : [m][H * hd].                                                        */
int ref_attention(const float *q, const float *k_cache, const float *v_cache, int64_t m, int64_t heads, int64_t hd,
                  int64_t max_seq, int64_t pos, float *out)
{
    if (m <= 0 || heads <= 0 || hd <= 0 || pos < 0 || pos >= max_seq) return -2;
    double *sc = (double *)malloc(sizeof(double) * (size_t)(pos + 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)hd);
    if (!sc || !acc) {
        free(sc);
        free(acc);
        return -7;
    }
    const double scale = 1.0 / sqrt((double)hd);
    for (int64_t r = 0; r < m; r++)
        for (int64_t h = 0; h < heads; h++) {
            const float *qh = q + (r * heads + h) * hd;
            const float *K = k_cache + ((r * heads + h) * max_seq) * hd;
            const float *V = v_cache + ((r * heads + h) * max_seq) * hd;
            double mx = -INFINITY;
            for (int64_t j = 0; j <= pos; j++) {
                double dot = 0.0;
                for (int64_t i = 0; i < hd; i++) dot += (double)qh[i] * (double)K[j * hd + i];
                sc[j] = dot * scale;
                if (sc[j] > mx) mx = sc[j];
            }
            double den = 0.0;
            for (int64_t i = 0; i < hd; i++) acc[i] = 0.0;
            for (int64_t j = 0; j <= pos; j++) {
                const double e = exp(sc[j] - mx);
                den += e;
                for (int64_t i = 0; i < hd; i++) acc[i] += e * (double)V[j * hd + i];
            }
            for (int64_t i = 0; i < hd; i++) out[r * heads * hd + h * hd + i] = (float)(acc[i] / den);
        }
    free(sc);
    free(acc);
    return 0;
}
