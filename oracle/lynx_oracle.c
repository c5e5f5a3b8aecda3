/*
 * Lynx progressive KV-cache quantization: CPU ORACLE (test infrastructure).
 *
 * This file is the plain, slow, obviously-correct definition that the GPU
 * library is checked against.  It is NOT part of the product path: only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * it.  It shares no code, header, table or constant generator with the HIP
 * library under long_context_serving_amd/.
 *
 * Source: "Lynx: the KV cache does not have to arrive whole" (a reading of
 * Han et al., "Lynx: Progressive Speculative Quantization for accelerating
 * KV Transfer in Long-Context Inference"), section 3 "The quantizer".
 * In that section's order, per page of 256 tokens:
 *   - per channel, the page's smallest value and its span rescale the
 *     channel onto [0,1];
 *   - each channel's page is cut into C = 32-token chunks; every chunk is
 *     shifted by its own mean and scaled by its own largest deviation, so an
 *     extreme value only coarsens its own chunk;
 *   - a logarithmic alpha-law curve sends the magnitude onto 127 levels,
 *     keeping the sign even for values whose magnitude rounds to level 0;
 *   - the 8-bit code is cut into a high nibble (the anchor, which fixes a
 *     geometric interval, i.e. an order of magnitude) and a low nibble (the
 *     residual, a position inside that interval); +7 is the round-half-down
 *     centre of the 16 codes an anchor spans.
 * Section 4 "Speculation at the communication boundary": a draft decodes
 * from the anchor stream alone, the refined cache (Q_full) from both nibbles.
 * Attention (page "LLM KV cache quantization", section "The architecture:
 * every piece explained"): scaled dot products of the query with every
 * cached key, a softmax over them, and the probability-weighted sum of the
 * cached values, all downstream of the dequantized cache.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   the scales are plain fp32 values: the page range is the fp32 difference
 *   max - min, the chunk max-abs the largest |x' - mean| of the chunk;
 *   alpha = 255 (mu-law constant); F(u) = ln(1+alpha u)/ln(1+alpha);
 *   magnitude m = floor(127 F(|y|) + 1/2) in 0..127;
 *   code q = m for y >= 0, q = -m-1 (= ~m) for y < 0;
 *   anchor a = q >> 4 (arithmetic), residual r = q & 15;
 *   draft code = 16 a + 7, full code = 16 a + r;
 *   yhat = sign * ((1+alpha)^(m/127) - 1)/alpha;
 *   xhat = min + range * (mean + maxabs * yhat).
 * Numeric contract for the statistics (so that codes are reproducible
 * bit for bit): every step below marked "fp32" is one IEEE single-precision
 * operation rounded to nearest even, with no fused multiply-add (this file
 * is compiled with -ffp-contract=off), and the chunk mean is the exact sum
 * of the chunk's 32 normalised values divided by 32, rounded once to fp32.
 * Everything else is evaluated in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_PAGE 256
#define OR_CHUNK 32
#define OR_NCHUNK (OR_PAGE / OR_CHUNK)
#define OR_LEVELS 127
#define OR_ALPHA 255.0

/* Flag bits written per element by oracle_encode. */
#define OR_FLAG_NEAR_HALF 1u   /* 127 F(u) within 2^-20 of a half-level  */
#define OR_FLAG_SUM_INEXACT 2u /* a nonzero x' below 2^-24 in the chunk */

static float bf16_to_float(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

/* tau(u) = 127 * ln(1 + alpha u) / ln(1 + alpha), in double precision. */
static double tau_of(float u)
{
    return (double)OR_LEVELS * log1p(OR_ALPHA * (double)u) / log1p(OR_ALPHA);
}

/* Magnitude level of |y| = u in [0,1] by rounding tau half up; sets *near
 * when tau lies within 2^-20 of a rounding boundary k + 1/2. */
static int magnitude_of(float u, int *near)
{
    double t = tau_of(u);
    double fl = floor(t);
    int m = (int)floor(t + 0.5);
    if (m < 0) m = 0;
    if (m > OR_LEVELS) m = OR_LEVELS;
    *near = fabs(t - (fl + 0.5)) < 0x1p-20;
    return m;
}

/* Sign-aware code: q = m for non-negative values, ~m = -m-1 for negative. */
static int code_of(float u, int negative, int *near)
{
    int m = magnitude_of(u, near);
    return negative ? -m - 1 : m;
}

/* Inverse map: yhat for an 8-bit code q in [-128, 127]. */
static double yhat_of(int q)
{
    int m = q >= 0 ? q : -q - 1;
    double g = (pow(1.0 + OR_ALPHA, (double)m / OR_LEVELS) - 1.0) / OR_ALPHA;
    return q >= 0 ? g : -g;
}

/* Exact sum of non-negative finite fp32 values, held as a 192-bit integer
 * in units of 2^-149 (the smallest fp32 denormal): a value below 2 is at
 * most 2^150 units, so 32 of them stay below 2^155. */
typedef struct {
    uint64_t w[3];
} exact_sum;

static void exact_sum_add(exact_sum *a, float f)
{
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    const uint32_t e = b >> 23;                    /* sign bit is 0 */
    uint64_t m = b & 0x7FFFFFu;
    int shift = 0;
    if (e != 0) {                                  /* normal: (2^23 + m) 2^(e-150) */
        m |= 0x800000u;
        shift = (int)e - 1;
    }
    /* add m << shift (m < 2^24, shift <= 127) */
    const int word = shift / 64, off = shift % 64;
    uint64_t add[3] = {0, 0, 0};
    add[word] = m << off;
    if (off > 40 && word < 2) add[word + 1] = m >> (64 - off);
    uint64_t carry = 0;
    for (int i = 0; i < 3; ++i) {
        const uint64_t t = a->w[i] + carry;
        const uint64_t c1 = t < carry;
        const uint64_t r = t + add[i];
        carry = c1 + (r < t);
        a->w[i] = r;
    }
}

/* bit i of the 192-bit integer */
static int exact_sum_bit(const exact_sum *a, int i)
{
    return (int)((a->w[i / 64] >> (i % 64)) & 1u);
}

/* fp32 value of sum * 2^-149 / 32, rounded once to nearest even. */
static float exact_sum_mean32(const exact_sum *a)
{
    int top = -1;
    for (int i = 191; i >= 0; --i)
        if (exact_sum_bit(a, i)) { top = i; break; }
    if (top < 0) return 0.0f;
    /* the value is sum * 2^-154; keep 24 significant bits, or the
     * denormal quantum 2^-149 (= 2^5 units of the sum) below 2^-126 */
    const int drop = top - 23 > 5 ? top - 23 : 5;
    uint64_t kept = 0;
    for (int i = top; i >= drop; --i) kept = (kept << 1) | (uint64_t)exact_sum_bit(a, i);
    const int half = exact_sum_bit(a, drop - 1);
    int sticky = 0;
    for (int i = drop - 2; i >= 0; --i) sticky |= exact_sum_bit(a, i);
    if (half && (sticky || (kept & 1u))) ++kept;   /* round half to even */
    return (float)ldexp((double)kept, drop - 154);  /* exact: kept <= 2^24 */
}

static int nthreads_or_default(int32_t n)
{
#ifdef _OPENMP
    return n > 0 ? n : omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

int32_t oracle_max_threads(void)
{
    return nthreads_or_default(0);
}

/* ---------------------------------------------------------------------------
 * Encoder.  Input x: bf16 bit patterns, layout [P][256][H][D] (a page is 256
 * tokens x KV heads x head_dim, in paged order).  Outputs:
 *   codes        int8  [P][256][H][D]   signed 8-bit code q
 *   page_min     fp32  [P][H][D]
 *   page_range   fp32  [P][H][D]
 *   chunk_mean   fp32  [P][H][8][D]
 *   chunk_maxabs fp32  [P][H][8][D]
 *   flags        uint8 [P][256][H][D]   OR_FLAG_* bits (may be NULL)
 * ------------------------------------------------------------------------- */
static void encode_channel(const uint16_t *x, int64_t p, int32_t h, int32_t d,
                           int32_t H, int32_t D, int8_t *codes,
                           float *page_min, float *page_range,
                           float *chunk_mean, float *chunk_maxabs,
                           uint8_t *flags)
{
    float v[OR_PAGE], xn[OR_PAGE];
    const int64_t row = (int64_t)H * D;
    const int64_t base = p * OR_PAGE * row + (int64_t)h * D + d;

    for (int t = 0; t < OR_PAGE; ++t)
        v[t] = bf16_to_float(x[base + t * row]);

    /* Page-level normalisation: per channel min and range over the page. */
    float mn = v[0], mx = v[0];
    for (int t = 1; t < OR_PAGE; ++t) {
        if (v[t] < mn) mn = v[t];
        if (v[t] > mx) mx = v[t];
    }
    float rg = mx - mn;                          /* fp32 */
    float inv_rg = rg > 0.0f ? 1.0f / rg : 0.0f; /* fp32, correctly rounded */
    for (int t = 0; t < OR_PAGE; ++t) {
        float diff = v[t] - mn;                  /* fp32 */
        xn[t] = diff * inv_rg;                   /* fp32 */
    }
    const int64_t sidx = ((p * H + h) * (int64_t)D) + d;
    page_min[sidx] = mn;
    page_range[sidx] = rg;

    /* Chunk-wise outlier isolation, C = 32 consecutive tokens. */
    for (int c = 0; c < OR_NCHUNK; ++c) {
        const int t0 = c * OR_CHUNK;
        /* a nonzero term below 2^-24 is flagged: a double-precision sum of
         * such a chunk need not be exact (its terms span more than 53 bits) */
        int inexact = 0;
        exact_sum sum = {{0, 0, 0}};
        for (int t = t0; t < t0 + OR_CHUNK; ++t) {
            if (xn[t] != 0.0f && xn[t] < 0x1p-24f) inexact = 1;
            exact_sum_add(&sum, xn[t]);
        }
        float mu = exact_sum_mean32(&sum);         /* one rounding */
        float dv[OR_CHUNK];
        float s = 0.0f;
        for (int i = 0; i < OR_CHUNK; ++i) {
            dv[i] = xn[t0 + i] - mu;               /* fp32 */
            float a = fabsf(dv[i]);
            if (a > s) s = a;
        }
        float inv_s = s > 0.0f ? 1.0f / s : 0.0f;  /* fp32, correctly rounded */
        const int64_t cidx = (((p * H + h) * OR_NCHUNK + c) * (int64_t)D) + d;
        chunk_mean[cidx] = mu;
        chunk_maxabs[cidx] = s;

        for (int i = 0; i < OR_CHUNK; ++i) {
            float u = fabsf(dv[i]) * inv_s;        /* fp32 */
            if (u > 1.0f) u = 1.0f;
            int near = 0;
            int q = code_of(u, dv[i] < 0.0f, &near);
            const int64_t e = base + (int64_t)(t0 + i) * row;
            codes[e] = (int8_t)q;
            if (flags)
                flags[e] = (uint8_t)((near ? OR_FLAG_NEAR_HALF : 0u) |
                                     (inexact ? OR_FLAG_SUM_INEXACT : 0u));
        }
    }
}

int32_t oracle_encode(const uint16_t *x, int64_t num_pages, int32_t H,
                      int32_t D, int8_t *codes, float *page_min,
                      float *page_range, float *chunk_mean,
                      float *chunk_maxabs, uint8_t *flags, int32_t nthreads)
{
    if (!x || !codes || !page_min || !page_range || !chunk_mean ||
        !chunk_maxabs || num_pages < 0 || H < 1 || D < 1)
        return -1;
    const int64_t units = num_pages * H;
    const int nt = nthreads_or_default(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t p = u / H;
        const int32_t h = (int32_t)(u % H);
        for (int32_t d = 0; d < D; ++d)
            encode_channel(x, p, h, d, H, D, codes, page_min, page_range,
                           chunk_mean, chunk_maxabs, flags);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Per-element maps, exposed for the pins.
 * ------------------------------------------------------------------------- */
void oracle_tau(const float *u, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = tau_of(u[i]);
}

/* codes from (u, negative) pairs; flag = near-half-level indicator */
void oracle_codes(const float *u, const uint8_t *negative, int64_t n,
                  int8_t *q, uint8_t *flag, int32_t nthreads)
{
    const int nt = nthreads_or_default(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n; ++i) {
        int near = 0;
        q[i] = (int8_t)code_of(u[i], negative ? negative[i] != 0 : 0, &near);
        if (flag) flag[i] = (uint8_t)near;
    }
}

void oracle_yhat(const int32_t *q, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = yhat_of(q[i]);
}

/* The cut: anchor = q >> 4 (arithmetic shift, -8..7), residual = q & 15. */
void oracle_split(const int8_t *q, int64_t n, int8_t *anchor,
                  uint8_t *residual)
{
    for (int64_t i = 0; i < n; ++i) {
        int v = q[i];
        anchor[i] = (int8_t)(v >> 4);
        residual[i] = (uint8_t)(v & 15);
    }
}

/* Full code 16 a + r; draft code 16 a + 7 (residual NULL). */
void oracle_join(const int8_t *anchor, const uint8_t *residual, int64_t n,
                 int32_t *q)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = 16 * (int32_t)anchor[i] + (residual ? (int32_t)residual[i] : 7);
}

/* ---------------------------------------------------------------------------
 * Other cuts of the 8-bit code (section 3 cuts it 4 + 4; section 7 of the
 * page lists 6 + 2, 2 + 6 and 5 + 3 as untried).  A b + (8 - b) cut keeps
 * the top b bits as the anchor (arithmetic shift: -2^(b-1) .. 2^(b-1) - 1)
 * and the low 8 - b bits as the residual; the draft code of anchor a is
 * a * 2^(8-b) + 2^(7-b) - 1, the round-half-down centre of the anchor's
 * 2^(8-b) codes (16 a + 7 for the 4 + 4 cut; the anchor itself for 8 + 0).
 * ------------------------------------------------------------------------- */
static int draft_offset(int anchor_bits)
{
    const int rb = 8 - anchor_bits;
    return rb > 0 ? (1 << (rb - 1)) - 1 : 0;
}

int32_t oracle_split_bits(const int8_t *q, int64_t n, int32_t anchor_bits,
                          int8_t *anchor, uint8_t *residual)
{
    if (anchor_bits < 1 || anchor_bits > 8) return -1;
    const int rb = 8 - anchor_bits;
    for (int64_t i = 0; i < n; ++i) {
        const int v = q[i];
        anchor[i] = (int8_t)(v >> rb);
        residual[i] = (uint8_t)(v & ((1 << rb) - 1));
    }
    return 0;
}

/* Full code a * 2^(8-b) + r; draft code with the centre (residual NULL). */
int32_t oracle_join_bits(const int8_t *anchor, const uint8_t *residual,
                         int64_t n, int32_t anchor_bits, int32_t *q)
{
    if (anchor_bits < 1 || anchor_bits > 8) return -1;
    const int rb = 8 - anchor_bits;
    const int mid = draft_offset(anchor_bits);
    for (int64_t i = 0; i < n; ++i)
        q[i] = (int32_t)anchor[i] * (1 << rb) + (residual ? (int32_t)residual[i] : mid);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Dequantizer.  anchor int8 [P][256][H][D] in -8..7; residual uint8 same
 * shape in 0..15, or NULL for the anchor-only (draft) reconstruction.
 * Scales as written by oracle_encode.  Output double [P][256][H][D].
 * ------------------------------------------------------------------------- */
int32_t oracle_dequant(const int8_t *anchor, const uint8_t *residual,
                       const float *page_min, const float *page_range,
                       const float *chunk_mean, const float *chunk_maxabs,
                       int64_t num_pages, int32_t H, int32_t D, double *out,
                       int32_t nthreads)
{
    if (!anchor || !page_min || !page_range || !chunk_mean || !chunk_maxabs ||
        !out || num_pages < 0 || H < 1 || D < 1)
        return -1;
    const int64_t row = (int64_t)H * D;
    const int64_t units = num_pages * OR_PAGE;
    const int nt = nthreads_or_default(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t p = u / OR_PAGE;
        const int t = (int)(u % OR_PAGE);
        const int c = t / OR_CHUNK;
        for (int32_t h = 0; h < H; ++h) {
            for (int32_t d = 0; d < D; ++d) {
                const int64_t e = u * row + (int64_t)h * D + d;
                const int q = 16 * (int)anchor[e] +
                              (residual ? (int)residual[e] : 7);
                const int64_t sidx = (p * H + h) * (int64_t)D + d;
                const int64_t cidx = ((p * H + h) * OR_NCHUNK + c) * (int64_t)D + d;
                const double yh = yhat_of(q);
                out[e] = (double)page_min[sidx] +
                         (double)page_range[sidx] *
                             ((double)chunk_mean[cidx] +
                              (double)chunk_maxabs[cidx] * yh);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Dequantizer of a b + (8 - b) cut: anchor int8 [P][256][H][D] in
 * -2^(b-1) .. 2^(b-1) - 1; residual uint8 in 0 .. 2^(8-b) - 1, or NULL for
 * the draft.  Same scales and output as oracle_dequant.
 * ------------------------------------------------------------------------- */
int32_t oracle_dequant_bits(const int8_t *anchor, const uint8_t *residual,
                            int32_t anchor_bits, const float *page_min,
                            const float *page_range, const float *chunk_mean,
                            const float *chunk_maxabs, int64_t num_pages,
                            int32_t H, int32_t D, double *out, int32_t nthreads)
{
    if (!anchor || !page_min || !page_range || !chunk_mean || !chunk_maxabs ||
        !out || num_pages < 0 || H < 1 || D < 1 || anchor_bits < 1 ||
        anchor_bits > 8)
        return -1;
    const int rb = 8 - anchor_bits;
    const int mid = draft_offset(anchor_bits);
    const int64_t row = (int64_t)H * D;
    const int64_t units = num_pages * OR_PAGE;
    const int nt = nthreads_or_default(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t p = u / OR_PAGE;
        const int t = (int)(u % OR_PAGE);
        const int c = t / OR_CHUNK;
        for (int32_t h = 0; h < H; ++h) {
            for (int32_t d = 0; d < D; ++d) {
                const int64_t e = u * row + (int64_t)h * D + d;
                const int q = (int)anchor[e] * (1 << rb) + (residual ? (int)residual[e] : mid);
                const int64_t sidx = (p * H + h) * (int64_t)D + d;
                const int64_t cidx = ((p * H + h) * OR_NCHUNK + c) * (int64_t)D + d;
                out[e] = (double)page_min[sidx] +
                         (double)page_range[sidx] *
                             ((double)chunk_mean[cidx] +
                              (double)chunk_maxabs[cidx] * yhat_of(q));
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Single-query GQA decode attention, brute force in double precision.
 *   q   [B][Hq][D]
 *   k,v [B][T][H][D]    (already dequantized)
 *   out [B][Hq][D]
 *   logits [B][Hq][T]   scaled scores before softmax (may be NULL)
 * Query head j reads KV head j / (Hq / H).  No mask: one query token
 * attends to every cached token.
 * ------------------------------------------------------------------------- */
int32_t oracle_attention(const double *q, const double *k, const double *v,
                         int32_t B, int64_t T, int32_t H, int32_t Hq,
                         int32_t D, double sm_scale, double *out,
                         double *logits, int32_t nthreads)
{
    if (!q || !k || !v || !out || B < 0 || T < 1 || H < 1 || Hq < H ||
        Hq % H != 0 || D < 1)
        return -1;
    const int32_t g = Hq / H;
    const int nt = nthreads_or_default(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double *s = (double *)malloc((size_t)T * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t bj = 0; bj < (int64_t)B * Hq; ++bj) {
            const int32_t b = (int32_t)(bj / Hq), j = (int32_t)(bj % Hq);
            const int32_t h = j / g;
            const double *qv = q + ((int64_t)b * Hq + j) * D;
            double mx = -INFINITY;
            for (int64_t t = 0; t < T; ++t) {
                const double *kv = k + (((int64_t)b * T + t) * H + h) * D;
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d) acc += qv[d] * kv[d];
                s[t] = sm_scale * acc;
                if (s[t] > mx) mx = s[t];
            }
            if (logits)
                memcpy(logits + ((int64_t)b * Hq + j) * T, s,
                       (size_t)T * sizeof(double));
            double z = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                s[t] = exp(s[t] - mx);
                z += s[t];
            }
            double *o = out + ((int64_t)b * Hq + j) * D;
            for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double p = s[t] / z;
                const double *vv = v + (((int64_t)b * T + t) * H + h) * D;
                for (int32_t d = 0; d < D; ++d) o[d] += p * vv[d];
            }
        }
        free(s);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Attention of several query tokens per request, each over a prefix of the
 * cached sequence, brute force in double precision.  This is the verify
 * pass of speculative decoding (page "Lynx: the KV cache does not have to
 * arrive whole", section 4: drafts run on the anchor stream, the refined
 * cache Q_full verifies them): the Tq speculative tokens are scored at once,
 * token i seeing the cache and the speculative tokens up to itself.
 *   q       [B][Tq][Hq][D]
 *   k,v     [B][T][H][D]      (dequantized pages followed by the bf16 tail)
 *   visible [B][Tq]           tokens 0 .. visible-1 are seen (1 <= visible <= T)
 *   out     [B][Tq][Hq][D]
 * Query head j reads KV head j / (Hq / H).
 * ------------------------------------------------------------------------- */
int32_t oracle_prefix_attention(const double *q, const double *k, const double *v,
                                const int64_t *visible, int32_t B, int32_t Tq,
                                int64_t T, int32_t H, int32_t Hq, int32_t D,
                                double sm_scale, double *out, int32_t nthreads)
{
    if (!q || !k || !v || !visible || !out || B < 0 || Tq < 1 || T < 1 || H < 1 ||
        Hq < H || Hq % H != 0 || D < 1)
        return -1;
    for (int64_t i = 0; i < (int64_t)B * Tq; ++i)
        if (visible[i] < 1 || visible[i] > T) return -1;
    const int32_t g = Hq / H;
    const int nt = nthreads_or_default(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double *s = (double *)malloc((size_t)T * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t row = 0; row < (int64_t)B * Tq * Hq; ++row) {
            const int64_t bi = row / Hq;             /* b * Tq + i */
            const int32_t j = (int32_t)(row % Hq);
            const int32_t b = (int32_t)(bi / Tq);
            const int32_t h = j / g;
            const int64_t n = visible[bi];
            const double *qv = q + row * D;
            double mx = -INFINITY;
            for (int64_t t = 0; t < n; ++t) {
                const double *kv = k + (((int64_t)b * T + t) * H + h) * D;
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d) acc += qv[d] * kv[d];
                s[t] = sm_scale * acc;
                if (s[t] > mx) mx = s[t];
            }
            double z = 0.0;
            for (int64_t t = 0; t < n; ++t) {
                s[t] = exp(s[t] - mx);
                z += s[t];
            }
            double *o = out + row * D;
            for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < n; ++t) {
                const double p = s[t] / z;
                const double *vv = v + (((int64_t)b * T + t) * H + h) * D;
                for (int32_t d = 0; d < D; ++d) o[d] += p * vv[d];
            }
        }
        free(s);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Baseline for the effective-bin check of section 2 ("Not all bits are
 * equal"): a uniform B-bit grid shared by all columns of a row.
 * x [rows][cols] fp32; codes [rows][cols] int32 in 0 .. 2^bits - 1.
 * ------------------------------------------------------------------------- */
void oracle_uniform_codes(const float *x, int64_t rows, int64_t cols,
                          int32_t bits, int32_t *codes)
{
    const double top = (double)((1 << bits) - 1);
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * cols;
        double lo = xr[0], hi = xr[0];
        for (int64_t c = 1; c < cols; ++c) {
            if (xr[c] < lo) lo = xr[c];
            if (xr[c] > hi) hi = xr[c];
        }
        const double step = hi > lo ? (hi - lo) / top : 1.0;
        for (int64_t c = 0; c < cols; ++c)
            codes[r * cols + c] = (int32_t)floor(((double)xr[c] - lo) / step + 0.5);
    }
}
