/*
 * csa2_oracle.c -- plain CPU reference of the CSA2 hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg
 * do.  It shares no source, header, table or helper with the HIP library.
 *
 * Every quantity is computed in IEEE binary64 with a fixed, sequential order of
 * operations; the file is compiled with -O2 -fno-fast-math -ffp-contract=off so
 * that no multiply-add is fused and no sum is reordered.  Inputs (fp32, bf16,
 * FP4 E2M1 codes with E4M3 scales) convert exactly to binary64.
 *
 * Sources (the pages this follows; formulas on them were lost in extraction,
 * so each step states the reading it takes):
 *  - "读完这篇，你就搞懂 DeepSeek v4 了" (note.crab.center), section
 *    "闪电索引机制（对应步骤二）", eq. (8): per-token relevance of every
 *    compressed entry, one score per indexer head, heads weighted and summed,
 *    the k most relevant entries kept.  Same idea as DSA of V3.2, whose
 *    published definition puts a ReLU on each head's dot product.
 *  - same page, "注意力计算（对应步骤三）", eq. (9): standard attention in which
 *    the k selected compressed entries are one shared matrix C used for both
 *    keys and values by every query head.
 *  - same page, HCA "压缩机制" paragraphs with eqs. (10), (11), which define the
 *    CSA compression by contrast: groups of m tokens, two consecutive groups
 *    concatenated, a softmax weight S over Z = projection + learnable bias B,
 *    applied to the value projection C.
 *  - "Recall之王 祭出Reuse" (10100.com), section "把KV Cache压到极致的几把杀手锏":
 *    FP4 main KV = E2M1 values with one E4M3 scale per 16 channels; the
 *    hierarchical indexer in which Reindex layers score only the candidate
 *    pool (at most 16,384 positions) chosen by the Full layer.
 *  - video transcript on V4.1 Flash (prism.simon-ai.net), the passage that
 *    introduces CSA2's Full / Reindex / Reuse layer modes.
 *
 * The E2M1 and E4M3 element formats follow the OCP Microscaling Formats (MX)
 * v1.0 and OCP 8-bit Floating Point (OFP8) specifications.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_F32 0
#define ORA_BF16 1
#define ORA_FP4 2

/* ---------------------------------------------------------------- formats */

static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of a binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element i of a plain (fp32 or bf16) array. */
static double elem(const void *base, int dt, int64_t i)
{
    if (dt == ORA_F32)
        return (double)((const float *)base)[i];
    return bf16_bits_to_double(((const uint16_t *)base)[i]);
}

/* OCP MX FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
 * Exponent field 0 is subnormal: magnitude = 0.5 * mantissa. */
double ora_e2m1(unsigned code)
{
    unsigned e = (code >> 1) & 3u, mbit = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)mbit : ldexp(1.0 + 0.5 * (double)mbit, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

/* OCP OFP8 E4M3 ("FN"): bias 7, no infinities, S.1111.111 is NaN.
 * Exponent field 0 is subnormal: magnitude = 2^-6 * mantissa/8. */
double ora_e4m3(unsigned byte)
{
    unsigned e = (byte >> 3) & 15u, mant = byte & 7u;
    if (e == 15u && mant == 7u)
        return NAN;
    double mag = (e == 0) ? ldexp((double)mant / 8.0, -6) : ldexp(1.0 + (double)mant / 8.0, (int)e - 7);
    return (byte & 0x80u) ? -mag : mag;
}

/* An FP4 row's scale byte as a value.  E4M3FN's NaN code (S.1111.111) is not a
 * scale any quantizer writes (the largest finite magnitude is 448 = S.1111.110);
 * reading taken for it: the scale saturates to +-448, the largest finite value
 * of the format, so that a corrupted byte cannot turn a whole group, or every
 * score and attention output that touches it, into NaN.  Every other byte is
 * its E4M3FN value. */
double ora_fp4_scale(unsigned byte)
{
    double s = ora_e4m3(byte);
    if (isnan(s))
        return (byte & 0x80u) ? -448.0 : 448.0;
    return s;
}

/* Bytes per stored KV row of width D in format dt. An FP4 row is D/2 code
 * bytes (channel 2i in the low nibble of byte i, channel 2i+1 in the high
 * nibble) followed by D/16 E4M3 scale bytes (scale b covers channels
 * 16b..16b+15). */
static int64_t row_bytes(int dt, int D)
{
    if (dt == ORA_F32)
        return 4 * (int64_t)D;
    if (dt == ORA_BF16)
        return 2 * (int64_t)D;
    return (int64_t)D / 2 + (int64_t)D / 16;
}

/* Decode one stored row into D doubles. */
void ora_decode_row(const void *row, int dt, int D, double *out)
{
    if (dt == ORA_FP4) {
        const uint8_t *codes = (const uint8_t *)row;
        const uint8_t *scales = codes + D / 2;
        for (int c = 0; c < D; c++) {
            uint8_t byte = codes[c / 2];
            unsigned code = (c % 2 == 0) ? (byte & 15u) : (byte >> 4);
            out[c] = ora_e2m1(code) * ora_fp4_scale(scales[c / 16]);
        }
        return;
    }
    for (int c = 0; c < D; c++)
        out[c] = elem(row, dt, c);
}

static const void *row_ptr(const void *base, int dt, int D, int64_t row)
{
    return (const uint8_t *)base + row * row_bytes(dt, D);
}

/* ---------------------------------------------------------- compression */

/*
 * Token compression (the CSA step the page defines by contrast with HCA):
 * entry i pools the window of the previous group of m tokens and its own group
 * of m tokens (two groups concatenated).  For every channel c:
 *   l_t[c] = sum_d x_t[d] * wz[d][c]  +  bias[r][c],   r = window position 0..2m-1
 *   p_t[c] = exp(l_t[c] - max_t l[c]) / sum_t exp(l_t[c] - max_t l[c])
 *   E_i[c] = sum_t p_t[c] * x_t[c]
 * The raw token row x_t is the value that gets pooled.  Window positions before
 * token 0 are masked (entry 0 pools only its own group).
 *
 * halo = 1: x holds m tokens of the previous group followed by n_out*m tokens,
 *           so entry i's window is x rows [i*m, i*m + 2m).
 * halo = 0: x holds n_out*m tokens from token 0; entry i's window is x rows
 *           [(i-1)*m, (i+1)*m), clipped at row 0.
 * out: [n_out, D] doubles.
 */
void ora_compress(const void *x, int dt, int64_t n_out, int D, int m, int halo, const void *wz,
                  const float *bias, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_out; i++) {
        int W = 2 * m;
        double *logit = (double *)malloc(sizeof(double) * (size_t)W);
        for (int c = 0; c < D; c++) {
            int64_t first_row = halo ? i * m : (i - 1) * m; /* x row of window position 0 */
            int have_any = 0;
            double mx = 0.0;
            for (int r = 0; r < W; r++) {
                int64_t t = first_row + r;
                if (t < 0) {
                    logit[r] = -INFINITY; /* masked: before token 0 */
                    continue;
                }
                double z = 0.0;
                for (int d = 0; d < D; d++)
                    z = z + elem(x, dt, t * D + d) * elem(wz, dt, (int64_t)d * D + c);
                logit[r] = z + (double)bias[(int64_t)r * D + c];
                if (!have_any || logit[r] > mx)
                    mx = logit[r];
                have_any = 1;
            }
            double denom = 0.0;
            for (int r = 0; r < W; r++)
                if (first_row + r >= 0)
                    denom = denom + exp(logit[r] - mx);
            double acc = 0.0;
            for (int r = 0; r < W; r++) {
                int64_t t = first_row + r;
                if (t < 0)
                    continue;
                double p = exp(logit[r] - mx) / denom;
                acc = acc + p * elem(x, dt, t * D + c);
            }
            out[i * D + c] = acc;
        }
        free(logit);
    }
}

/* -------------------------------------------------------------- indexer */

/*
 * Lightning-indexer score of compressed entry j for one query token:
 *   d_h  = sum_{d=0}^{dI-1} qI[h][d] * kI[j][d]       (sequential, from +0.0)
 *   r_h  = d_h > 0 ? d_h : +0.0                        (ReLU)
 *   t_h  = w_h * r_h                                   (rounded product, not fused)
 *   s(j) = sum_{h=0}^{HI-1} t_h                        (sequential, from +0.0)
 * One key row per entry is shared by all indexer heads; q and w are per head.
 *
 * Visibility: with q_pos, a query at absolute position t sees entry j only if
 * its whole group is in the past, (j+1)*m <= t+1.  Without q_pos every entry
 * is visible.  With cand, slot p scores entry cand[p] (-1 = empty slot).
 * An invisible entry or empty slot scores -inf.
 *
 * qI [B,Q,HI,dI], w [B,Q,HI], kI [B,N,dI], out [B,Q,n] with n = cand ? P : N.
 */
void ora_index_score(const void *qI, const float *w, const void *kI, int dt, int B, int Q, int HI, int dI,
                     int64_t N, const int64_t *q_pos, int m, const int32_t *cand, int P, double *out)
{
    int64_t n = cand ? (int64_t)P : N;
    int64_t total = (int64_t)B * Q * n;
#pragma omp parallel for schedule(static)
    for (int64_t flat = 0; flat < total; flat++) {
        int64_t bq = flat / n, slot = flat % n;
        int64_t b = bq / Q;
        int64_t j = cand ? (int64_t)cand[bq * P + slot] : slot;
        if (j < 0 || (q_pos && (j + 1) * (int64_t)m > q_pos[bq] + 1)) {
            out[flat] = -INFINITY;
            continue;
        }
        double s = 0.0;
        for (int h = 0; h < HI; h++) {
            double dot = 0.0;
            for (int d = 0; d < dI; d++)
                dot = dot + elem(qI, dt, (bq * HI + h) * dI + d) * elem(kI, dt, (b * N + j) * dI + d);
            double r = dot > 0.0 ? dot : 0.0;
            double t = (double)w[bq * HI + h] * r;
            s = s + t;
        }
        out[flat] = s;
    }
}

/* ------------------------------------------------------- bf16 score keys */

/*
 * "读完这篇，你就搞懂 DeepSeek v4 了", the passage on V4's FP4 quantization-aware
 * training: the lightning indexer's score is quantized only down to BF16,
 * because the top-k ranking is sensitive to it.  Reading taken: the value
 * that top-k ranks is the binary64 score of the formula rounded once to
 * bfloat16 (8 exponent bits like binary32, 8 significant bits), to nearest
 * with ties to the even significand, directly from binary64 (never through
 * binary32, which could round twice); magnitudes that round past the largest
 * finite bfloat16 become infinite with their sign; zero, infinities and NaN
 * are kept.  Equal rounded scores are then ordered by entry index, as any tie.
 *
 * Method: the spacing of bfloat16 values around |x| is 2^(e-7) for the
 * binade [2^e, 2^(e+1)), and 2^-133 below 2^-126 (subnormals); |x| divided
 * by that spacing (exact: a power of two) is rounded to the nearest integer,
 * ties to even, by nearbyint in the default rounding mode, and scaled back.
 */
double ora_round_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    int e2;
    frexp(fabs(x), &e2); /* |x| in [2^(e2-1), 2^e2) */
    int lead = e2 - 1;
    if (lead < -126)
        lead = -126;
    double spacing = ldexp(1.0, lead - 7);
    double r = nearbyint(fabs(x) / spacing) * spacing;
    if (r >= ldexp(1.0, 128))
        r = INFINITY;
    return x < 0.0 ? -r : r;
}

void ora_round_bf16_array(const double *x, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = ora_round_bf16(x[i]);
}

/* ------------------------------------------------------------- selection */

typedef struct {
    double s;
    int32_t j;
} scored;

/* Rank order: higher score first; equal scores, lower entry index first. */
static int by_score_then_index(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->s > b->s)
        return -1;
    if (a->s < b->s)
        return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int by_index(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    return (a->j > b->j) - (a->j < b->j);
}

/*
 * Top-k per query over scores [BQ, n]: rank the selectable slots (score not
 * -inf, cand entry not -1) by (score descending, entry index ascending), keep
 * the first min(k, selectable), and write their entry indices in ascending
 * order, padded with -1.  The entry index of slot p is cand[p] when cand is
 * given, else p.  count[q] = number kept.
 */
void ora_topk(const double *scores, int64_t BQ, int64_t n, const int32_t *cand, int k, int32_t *idx,
              int32_t *count)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < BQ; q++) {
        scored *list = (scored *)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
        int64_t cnt = 0;
        for (int64_t p = 0; p < n; p++) {
            double s = scores[q * n + p];
            int32_t j = cand ? cand[q * n + p] : (int32_t)p;
            if (s == -INFINITY || j < 0)
                continue;
            list[cnt].s = s;
            list[cnt].j = j;
            cnt++;
        }
        qsort(list, (size_t)cnt, sizeof(scored), by_score_then_index);
        int64_t keep = cnt < k ? cnt : k;
        qsort(list, (size_t)keep, sizeof(scored), by_index);
        for (int64_t t = 0; t < k; t++)
            idx[q * k + t] = t < keep ? list[t].j : -1;
        if (count)
            count[q] = (int32_t)keep;
        free(list);
    }
}

/* ------------------------------------------------------------- attention */

/*
 * Shared-KV sparse attention for every query head h over the listed entries
 * (idx [BQ,k], -1 entries skipped).  C_j is the decoded KV row, used as both
 * key and value by all heads:
 *   a_j  = scale * sum_d q[h][d] * C_j[d]
 *   mu   = max_j a_j,  e_j = exp(a_j - mu),  Z = sum_j e_j
 *   o[h] = (sum_j e_j * C_j) / Z,   lse[h] = mu + ln Z
 * No listed entry: o = 0 and lse = -inf.
 * q [B,Q,H,D], kv rows [B,N,row], out [B,Q,H,D] and lse [B,Q,H] in doubles.
 */
void ora_sparse_attn(const void *q, int q_dt, const void *kv, int kv_dt, int B, int Q, int H, int D, int64_t N,
                     const int32_t *idx, int k, double scale, double *out, double *lse)
{
    int64_t BQ = (int64_t)B * Q;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bq = 0; bq < BQ; bq++) {
        int64_t b = bq / Q;
        double *C = (double *)malloc(sizeof(double) * (size_t)k * (size_t)D + 8);
        double *a = (double *)malloc(sizeof(double) * (size_t)k + 8);
        double *num = (double *)malloc(sizeof(double) * (size_t)D);
        int cnt = 0;
        for (int t = 0; t < k; t++) {
            int32_t j = idx[bq * k + t];
            if (j < 0)
                continue;
            ora_decode_row(row_ptr(kv, kv_dt, D, b * N + j), kv_dt, D, C + (int64_t)cnt * D);
            cnt++;
        }
        for (int h = 0; h < H; h++) {
            double *o = out + (bq * H + h) * D;
            if (cnt == 0) {
                for (int d = 0; d < D; d++)
                    o[d] = 0.0;
                lse[bq * H + h] = -INFINITY;
                continue;
            }
            double mu = 0.0;
            for (int t = 0; t < cnt; t++) {
                double dot = 0.0;
                for (int d = 0; d < D; d++)
                    dot = dot + elem(q, q_dt, (bq * H + h) * D + d) * C[(int64_t)t * D + d];
                a[t] = scale * dot;
                if (t == 0 || a[t] > mu)
                    mu = a[t];
            }
            double Z = 0.0;
            for (int d = 0; d < D; d++)
                num[d] = 0.0;
            for (int t = 0; t < cnt; t++) {
                double e = exp(a[t] - mu);
                Z = Z + e;
                for (int d = 0; d < D; d++)
                    num[d] = num[d] + e * C[(int64_t)t * D + d];
            }
            for (int d = 0; d < D; d++)
                o[d] = num[d] / Z;
            lse[bq * H + h] = mu + log(Z);
        }
        free(C);
        free(a);
        free(num);
    }
}

/* ------------------------------------------------------------ SWA branch */

/*
 * Window list of the sliding-window branch: the W most recent token
 * positions up to and including the query's own, p - W + 1 .. p in
 * ascending order, those below 0 given as -1.
 * Video transcript on V4.1 Flash (prism.simon-ai.net), the passages on the
 * SWA branch: a 128-token window per layer, kept uncompressed and never shared
 * across layers.  The window's exact edge is not stated; this reading counts
 * the query's own token as the newest of the W.
 */
void ora_window_idx(const int64_t *q_pos, int64_t BQ, int W, int32_t *idx)
{
    for (int64_t bq = 0; bq < BQ; bq++)
        for (int i = 0; i < W; i++) {
            int64_t j = q_pos[bq] - (int64_t)W + 1 + i;
            idx[bq * W + i] = j < 0 ? -1 : (int32_t)j;
        }
}

/*
 * Merge of two attention results over disjoint entry sets into the result of
 * one softmax over their union (the CSA2 branch and the SWA branch).  With
 * lse the log of each branch's softmax denominator:
 *   M = max(lse_a, lse_b),  u = exp(lse_a - M),  v = exp(lse_b - M)
 *   out = (u o_a + v o_b) / (u + v),   lse = M + ln(u + v)
 * A branch with lse = -inf (no entry) has weight 0; both empty: out = 0,
 * lse = -inf.  The pages do not state how the branches are combined; this is
 * the reading in which both sets enter a single softmax.
 * R rows of D values each, all arrays in doubles.
 */
void ora_merge_attn(const double *o_a, const double *lse_a, const double *o_b, const double *lse_b, int64_t R,
                    int D, double *out, double *lse)
{
    for (int64_t r = 0; r < R; r++) {
        double la = lse_a[r], lb = lse_b[r];
        double *o = out + r * D;
        if (la == -INFINITY && lb == -INFINITY) {
            for (int d = 0; d < D; d++)
                o[d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double M = la > lb ? la : lb;
        double u = exp(la - M), v = exp(lb - M);
        double s = u + v;
        for (int d = 0; d < D; d++)
            o[d] = (u * o_a[r * D + d] + v * o_b[r * D + d]) / s;
        lse[r] = M + log(s);
    }
}

/* ---------------------------------------------------- FP4 cache writes */

/*
 * FP4 quantizer for main-KV cache writes ("Recall之王 祭出Reuse", section
 * "把KV Cache压到极致的几把杀手锏": the main KV is stored as E2M1 values with
 * one E4M3 scale per 16 channels).  The pages do not say how the scale and
 * codes are chosen; the reading taken, per group of 16 channels:
 *   scale s = the smallest non-negative E4M3 value with 6 s >= max |x|
 *             (6 is the largest E2M1 magnitude, so no code saturates),
 *             448 if no such value exists (then codes saturate at 6);
 *   code    = the E2M1 value nearest to x / s, ties to the even code
 *             (mantissa bit 0), the sign of x in bit 3 (a zero is +0);
 *             with s = 0 every code is 0.
 * Every comparison is exact in binary64: 6 s and (midpoint * s) have at most
 * seven significant bits.  x: n rows of D values in dt (CSA2_F32 or BF16);
 * out: n FP4 rows (layout as ora_decode_row).
 */
void ora_quantize_fp4(const void *x, int dt, int64_t n, int D, uint8_t *out)
{
    const int64_t rb = row_bytes(ORA_FP4, D);
    for (int64_t r = 0; r < n; r++) {
        uint8_t *codes = out + r * rb;
        uint8_t *scales = codes + D / 2;
        for (int g = 0; g < D / 16; g++) {
            double v[16], amax = 0.0;
            for (int i = 0; i < 16; i++) {
                v[i] = elem(x, dt, r * D + g * 16 + i);
                if (fabs(v[i]) > amax)
                    amax = fabs(v[i]);
            }
            /* the smallest E4M3 byte (0x00 .. 0x7E, increasing values) with 6 s >= amax */
            unsigned sb = 0x7Eu;
            for (unsigned b = 0; b <= 0x7Eu; b++)
                if (6.0 * ora_e4m3(b) >= amax) {
                    sb = b;
                    break;
                }
            double s = ora_e4m3(sb);
            scales[g] = (uint8_t)sb;
            for (int i = 0; i < 16; i++) {
                unsigned best = 0;
                if (s > 0.0) {
                    /* nearest of the 8 magnitudes; on a tie the even code */
                    double a = fabs(v[i]), bd = INFINITY;
                    for (unsigned c = 0; c < 8; c++) {
                        double d = fabs(a - ora_e2m1(c) * s);
                        if (d < bd || (d == bd && (c & 1u) == 0)) {
                            bd = d;
                            best = c;
                        }
                    }
                    if (v[i] < 0.0 && best != 0)
                        best |= 8u;
                }
                int c = g * 16 + i;
                if (c % 2 == 0)
                    codes[c / 2] = (uint8_t)best;
                else
                    codes[c / 2] |= (uint8_t)(best << 4);
            }
        }
    }
}
