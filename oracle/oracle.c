/*
 * Oracle for the sparse-attention indexer: paged MQA logits and per-row top-k.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header, table or constant with the HIP
 * library: its decoders, page translation and selection are written here from
 * the definitions alone, in plain loops, accumulating in double precision.
 *
 * What it computes (sources are the four pull-request pages the method is
 * described on):
 *   - The indexer score ("mqa-logits") of one query row against one K token:
 *       logit = sum_h w[h] * max(0, k_scale * (q_h . k))
 *     over a single-head K cache. The pages name the op (ROCm/ATOM PR #1709
 *     "Add fp4 indexer fo dsv4", commit messages on the FP4 mqa-logits kernel
 *     and on indexer_score_topk; vllm-project/DeepGEMM PR #14, summary, "FP8
 *     paged-MQA logits") but do not print the formula; the formula above is
 *     the stated problem this library is built for.
 *   - The page walk: logical token t of a sequence lives in physical page
 *     block_table[t / page_size] at slot t % page_size, i.e. cache row
 *     phys * page_size + slot (ATOM PR #1709, commit on the HCA k2-aware
 *     offsets, which names this "//capacity, %capacity, phys*capacity+slot"
 *     pattern as the correct one).
 *   - The per-row top-k: the min(k, E) largest logits of a row, ties to the
 *     lower token index, padded with -1 (ATOM PR #1709, commit on routing
 *     indexer_score_topk; "seq-local" output of the FP4 prefill path).
 *
 * Storage formats decoded here (closed forms from the format definitions):
 *   - OCP FP8 E4M3FN byte: sign, 4-bit exponent (bias 7), 3-bit mantissa;
 *     exponent 15 with mantissa 7 is NaN, there is no infinity. The KV cache
 *     is fp8_e4m3 (sglang PR #11993 "Accelerate deepseek fp4 b200 ci",
 *     summary of changes).
 *   - OCP E2M1 nibble: sign, 2-bit exponent (bias 1), 1-bit mantissa.
 *   - OCP E8M0 byte: 2^(byte-127); 0xFF is NaN.
 *   The MXFP4 cache is a uint8 tensor with two E2M1 values per byte (ATOM PR
 *   #1709, commit on the forward_pre split: FP4 is selected by a uint8 kv
 *   cache). Reading adopted where the pages are silent: the low nibble holds
 *   the even element, and one E8M0 scale covers 32 consecutive elements. This
 *   reading is parity unpinned by the pages (only by the round trip against the
 *   input quantizer).
 *
 * Row windows (visible length E_r of query row r):
 *   - decode with next_n rows per sequence: row r = b*next_n + j sees
 *     E_r = max(0, len_b - (next_n-1-j)) (reading adopted: the last row of a
 *     sequence sees the whole context, each earlier row one token less);
 *   - prefill: E_r = visible_end[r], given per row.
 *   - ragged decode: sequence b owns the packed rows [off[b], off[b+1]) and
 *     its row j sees max(0, len_b - (n_b-1-j)), the rule above with next_n
 *     replaced by the sequence's own row count (section at the end).
 *
 * Also here, each in its own section below with its readings: the K-cache
 * writer's encoders (FP8 row scale amax/448, E4M3 nearest with ties to even;
 * MXFP4 per-32 OCP MX exponent and E2M1 nearest with ties to even) and the
 * query quantizer with the weight fold.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_FP8 1
#define ORC_MXFP4 2

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_BAD_PAGE 2

/* Threads the row loops use (1 without OpenMP). */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- decoders */

double orc_dec_fp8_e4m3(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ((double)m / 8.0) * ldexp(1.0, -6); /* subnormal */
    else
        v = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
    return s ? -v : v;
}

double orc_dec_e2m1(uint8_t nibble)
{
    int s = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int m = nibble & 1;
    double v;
    if (e == 0)
        v = (double)m * 0.5; /* subnormal: 0 or 0.5 */
    else
        v = (1.0 + (double)m / 2.0) * ldexp(1.0, e - 1);
    return s ? -v : v;
}

double orc_dec_e8m0(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

static float orc_load_f32(const uint8_t *p)
{
    float f;
    memcpy(&f, p, sizeof f);
    return f;
}

/* ------------------------------------------------------ dequantized operands */

/* Query row r, head h, as D real numbers. FP8: code * per-row fp32 scale (a
 * null scale means 1). MXFP4: code * e8m0 scale of its 32-element block. */
static void orc_query_head(int dtype, const uint8_t *q, const uint8_t *q_scale,
                           int64_t r, int h, int H, int D, double *out)
{
    int d;
    if (dtype == ORC_FP8) {
        const uint8_t *row = q + ((int64_t)r * H + h) * D;
        double s = q_scale ? (double)orc_load_f32(q_scale + 4 * r) : 1.0;
        for (d = 0; d < D; ++d)
            out[d] = orc_dec_fp8_e4m3(row[d]) * s;
    } else {
        const uint8_t *row = q + ((int64_t)r * H + h) * (D / 2);
        const uint8_t *sc = q_scale + ((int64_t)r * H + h) * (D / 32);
        for (d = 0; d < D; ++d) {
            uint8_t byte = row[d / 2];
            uint8_t nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[d] = orc_dec_e2m1(nib) * orc_dec_e8m0(sc[d / 32]);
        }
    }
}

/* Logical token t of the sequence whose block-table row is bt, as D real
 * numbers with its stored scale applied. Returns ORC_BAD_PAGE when the
 * block-table entry is not a page of the pool. */
static int orc_key_token(int dtype, const uint8_t *kdata, int64_t page_stride,
                         int64_t row_stride, const uint8_t *kscale,
                         int64_t scale_page_stride, int64_t scale_row_stride,
                         int page_size, int64_t num_pages, const int32_t *bt,
                         int64_t t, int D, double *out)
{
    int64_t logical_page = t / page_size;
    int64_t slot = t % page_size;
    int64_t phys = bt[logical_page];
    const uint8_t *row, *srow;
    int d;
    if (phys < 0 || phys >= num_pages)
        return ORC_BAD_PAGE;
    row = kdata + phys * page_stride + slot * row_stride;
    srow = kscale + phys * scale_page_stride + slot * scale_row_stride;
    if (dtype == ORC_FP8) {
        double s = (double)orc_load_f32(srow);
        for (d = 0; d < D; ++d)
            out[d] = orc_dec_fp8_e4m3(row[d]) * s;
    } else {
        for (d = 0; d < D; ++d) {
            uint8_t byte = row[d / 2];
            uint8_t nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[d] = orc_dec_e2m1(nib) * orc_dec_e8m0(srow[d / 32]);
        }
    }
    return ORC_OK;
}

/* One logit: sum over heads of w[h] * max(0, q_h . k). */
static double orc_score(const double *qf /* [H][D] */, const double *kf,
                        const float *w_row, int H, int D)
{
    double logit = 0.0;
    int h, d;
    for (h = 0; h < H; ++h) {
        double s = 0.0;
        for (d = 0; d < D; ++d)
            s += qf[(int64_t)h * D + d] * kf[d];
        if (s > 0.0)
            logit += (double)w_row[h] * s;
    }
    return logit;
}

/* Scores one query row against tokens [0, E) of the sequence with block-table
 * row bt; writes out[0..W), with -inf at t >= E. */
static int orc_row(int dtype, const uint8_t *q, const uint8_t *q_scale,
                   const float *w, int H, int D, int64_t r, const uint8_t *kdata,
                   int64_t page_stride, int64_t row_stride, const uint8_t *kscale,
                   int64_t scale_page_stride, int64_t scale_row_stride,
                   int page_size, int64_t num_pages, const int32_t *bt, int64_t E,
                   int64_t W, double *out)
{
    double *qf = (double *)malloc(sizeof(double) * (size_t)H * (size_t)D);
    double *kf = (double *)malloc(sizeof(double) * (size_t)D);
    int64_t t;
    int h, rc = ORC_OK;
    if (!qf || !kf) {
        free(qf);
        free(kf);
        return ORC_BAD_ARG;
    }
    for (h = 0; h < H; ++h)
        orc_query_head(dtype, q, q_scale, r, h, H, D, qf + (int64_t)h * D);
    for (t = 0; t < W; ++t)
        out[t] = -INFINITY;
    for (t = 0; t < E && t < W; ++t) {
        rc = orc_key_token(dtype, kdata, page_stride, row_stride, kscale,
                           scale_page_stride, scale_row_stride, page_size,
                           num_pages, bt, t, D, kf);
        if (rc != ORC_OK)
            break;
        out[t] = orc_score(qf, kf, w + r * H, H, D);
    }
    free(qf);
    free(kf);
    return rc;
}

static int orc_check_common(int dtype, int H, int D, int page_size)
{
    if (dtype != ORC_FP8 && dtype != ORC_MXFP4)
        return ORC_BAD_ARG;
    if (H < 1 || D < 1 || page_size < 1)
        return ORC_BAD_ARG;
    if (dtype == ORC_MXFP4 && D % 32 != 0)
        return ORC_BAD_ARG;
    return ORC_OK;
}

/*
 * Decode: B sequences with next_n query rows each (row r = b*next_n + j).
 * Computes the listed rows only (rows[i], i < nrows) into out[i][0..W), and
 * their visible lengths into E_out[i].
 */
int orc_decode_logits(int dtype, const uint8_t *q, const uint8_t *q_scale,
                      const float *w, int H, int D, const uint8_t *kdata,
                      int64_t page_stride, int64_t row_stride,
                      const uint8_t *kscale, int64_t scale_page_stride,
                      int64_t scale_row_stride, int page_size, int64_t num_pages,
                      const int32_t *block_tables, int64_t bt_stride,
                      const int32_t *lens, int B, int next_n, const int64_t *rows,
                      int64_t nrows, int64_t W, double *out, int64_t *E_out)
{
    int64_t i;
    int rc_all = ORC_OK;
    if (orc_check_common(dtype, H, D, page_size) != ORC_OK || next_n < 1)
        return ORC_BAD_ARG;
    for (i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= (int64_t)B * next_n)
            return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        int64_t b = r / next_n;
        int64_t j = r % next_n;
        int64_t E = (int64_t)lens[b] - (next_n - 1 - j);
        int rc;
        if (E < 0)
            E = 0;
        E_out[i] = E;
        rc = orc_row(dtype, q, q_scale, w, H, D, r, kdata, page_stride,
                     row_stride, kscale, scale_page_stride, scale_row_stride,
                     page_size, num_pages, block_tables + b * bt_stride, E, W,
                     out + i * W);
        if (rc != ORC_OK) {
#pragma omp critical
            rc_all = rc;
        }
    }
    return rc_all;
}

/*
 * Prefill: T query rows of one sequence; row r sees visible_end[r] tokens.
 * Computes the listed rows only.
 */
int orc_prefill_logits(int dtype, const uint8_t *q, const uint8_t *q_scale,
                       const float *w, int H, int D, const uint8_t *kdata,
                       int64_t page_stride, int64_t row_stride,
                       const uint8_t *kscale, int64_t scale_page_stride,
                       int64_t scale_row_stride, int page_size,
                       int64_t num_pages, const int32_t *block_table,
                       const int32_t *visible_end, int64_t T, const int64_t *rows,
                       int64_t nrows, int64_t W, double *out, int64_t *E_out)
{
    int64_t i;
    int rc_all = ORC_OK;
    if (orc_check_common(dtype, H, D, page_size) != ORC_OK)
        return ORC_BAD_ARG;
    for (i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= T)
            return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        int64_t E = visible_end[r] < 0 ? 0 : visible_end[r];
        int rc;
        E_out[i] = E;
        rc = orc_row(dtype, q, q_scale, w, H, D, r, kdata, page_stride,
                     row_stride, kscale, scale_page_stride, scale_row_stride,
                     page_size, num_pages, block_table, E, W, out + i * W);
        if (rc != ORC_OK) {
#pragma omp critical
            rc_all = rc;
        }
    }
    return rc_all;
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
    double v;
    int64_t t;
} orc_item;

/* Larger value first; equal values (including -0 against +0, which compare
 * equal) go to the lower token index first. */
static int orc_item_cmp(const void *a, const void *b)
{
    const orc_item *x = (const orc_item *)a;
    const orc_item *y = (const orc_item *)b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    if (x->t < y->t)
        return -1;
    if (x->t > y->t)
        return 1;
    return 0;
}

static int orc_topk_items(orc_item *items, int64_t E, int k, int32_t *out)
{
    int64_t n = E < k ? E : k;
    int64_t i;
    qsort(items, (size_t)E, sizeof(orc_item), orc_item_cmp);
    for (i = 0; i < n; ++i)
        out[i] = (int32_t)items[i].t;
    for (i = n; i < k; ++i)
        out[i] = -1;
    return ORC_OK;
}

/* Top-k of one row of double logits v[0..E): token indices, largest first. */
int orc_topk_f64(const double *v, int64_t E, int k, int32_t *out)
{
    orc_item *items;
    int64_t t;
    int rc;
    if (E < 0 || k < 1)
        return ORC_BAD_ARG;
    items = (orc_item *)malloc(sizeof(orc_item) * (size_t)(E > 0 ? E : 1));
    if (!items)
        return ORC_BAD_ARG;
    for (t = 0; t < E; ++t) {
        items[t].v = v[t];
        items[t].t = t;
    }
    rc = orc_topk_items(items, E, k, out);
    free(items);
    return rc;
}

/* Top-k of one row of float logits; the ordering is decided on the float
 * values themselves (exactly representable in double). */
int orc_topk_f32(const float *v, int64_t E, int k, int32_t *out)
{
    orc_item *items;
    int64_t t;
    int rc;
    if (E < 0 || k < 1)
        return ORC_BAD_ARG;
    items = (orc_item *)malloc(sizeof(orc_item) * (size_t)(E > 0 ? E : 1));
    if (!items)
        return ORC_BAD_ARG;
    for (t = 0; t < E; ++t) {
        items[t].v = (double)v[t];
        items[t].t = t;
    }
    rc = orc_topk_items(items, E, k, out);
    free(items);
    return rc;
}

/* Many rows of float logits (row stride W), each with its own length. */
int orc_topk_rows_f32(const float *logits, int64_t W, const int64_t *E,
                      int64_t nrows, int k, int32_t *out)
{
    int64_t i;
    int rc_all = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        int rc = orc_topk_f32(logits + i * W, E[i], k, out + i * k);
        if (rc != ORC_OK) {
#pragma omp critical
            rc_all = rc;
        }
    }
    return rc_all;
}

/* --------------------------------------------------------- K-cache writer */
/*
 * The step before the scores: new K rows are quantized to the cache's storage
 * format and scattered into their pages (ATOM PR #1709 names "FP4 mqa-logits /
 * scatter kernels" in the commit that adds the FP4 indexer flag). The pages do
 * not print the quantizer; the readings adopted (and used by the input
 * generator the scoring tests run on) are:
 *   - FP8: one fp32 scale per row, amax / 448 computed in single precision
 *     (1 for an all-zero row); codes are the E4M3FN value nearest to
 *     x / scale (single-precision quotient), ties to the even code, the sign
 *     kept (so -0 and small negatives give 0x80).
 *   - MXFP4 (OCP MX): per 32-element block the shared exponent
 *     e = floor(log2(amax)) - 2 (2 = the largest E2M1 exponent), clamped to
 *     [-127, 127] (0 for an all-zero block), stored as the E8M0 byte e + 127;
 *     codes are the E2M1 magnitude nearest to |x| * 2^-e, ties to the even
 *     code, saturating at 6, with the sign bit set only for a nonzero code;
 *     the even element goes to the low nibble.
 * Both encoders search the decoders' value tables: no bit tricks.
 */

/* Nearest E4M3FN code to y (single precision), ties to the even code. */
uint8_t orc_enc_fp8_e4m3(float y)
{
    const double a = fabs((double)y);
    int best = 0;
    double best_d = INFINITY;
    int c;
    for (c = 0; c < 0x7F; ++c) { /* 0x7F is NaN */
        const double v = orc_dec_fp8_e4m3((uint8_t)c);
        const double d = fabs(v - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* Nearest E2M1 magnitude code (0..7) to a >= 0, ties to the even code,
 * saturating at the largest magnitude. */
static int orc_enc_e2m1_mag(double a)
{
    int best = 0, c;
    double best_d = INFINITY;
    for (c = 0; c < 8; ++c) {
        const double d = fabs(orc_dec_e2m1((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* One row of D values to FP8 codes + fp32 scale. */
void orc_quant_fp8_row(const float *x, int D, uint8_t *codes, float *scale)
{
    float amax = 0.f, s;
    int i;
    for (i = 0; i < D; ++i)
        amax = fabsf(x[i]) > amax ? fabsf(x[i]) : amax;
    s = amax > 0.f ? amax / 448.0f : 1.0f;
    for (i = 0; i < D; ++i)
        codes[i] = orc_enc_fp8_e4m3(x[i] / s);
    *scale = s;
}

/* One row of D values (a multiple of 32) to packed E2M1 + E8M0 bytes. */
void orc_quant_mxfp4_row(const float *x, int D, uint8_t *packed, uint8_t *scales)
{
    int b, i;
    memset(packed, 0, (size_t)D / 2);
    for (b = 0; b < D / 32; ++b) {
        const float *blk = x + 32 * b;
        float amax = 0.f;
        int e = 0, ex;
        for (i = 0; i < 32; ++i)
            amax = fabsf(blk[i]) > amax ? fabsf(blk[i]) : amax;
        if (amax > 0.f) {
            (void)frexpf(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1) */
            e = ex - 1 - 2;
            e = e < -127 ? -127 : (e > 127 ? 127 : e);
        }
        scales[b] = (uint8_t)(e + 127);
        for (i = 0; i < 32; ++i) {
            const float y = ldexpf(blk[i], -e);
            int c = orc_enc_e2m1_mag(fabs((double)y));
            if (y < 0.f && c > 0)
                c |= 8;
            packed[(32 * b + i) / 2] |= (uint8_t)(((i & 1) ? c << 4 : c));
        }
    }
}

/* Writes N rows (row stride ld floats) into a cache image: row t goes to
 * slot_mapping[t] = page * P + slot (skipped when negative or past the pool),
 * its bytes at data + page*page_stride + slot*row_stride and its scale at
 * scale + page*scale_page_stride + slot*scale_row_stride. */
int orc_kv_write(int dtype, const float *k, int64_t ld, int64_t N, int D,
                 const int64_t *slot_mapping, int P, int64_t num_pages,
                 uint8_t *data, int64_t page_stride, int64_t row_stride,
                 uint8_t *scale, int64_t scale_page_stride, int64_t scale_row_stride)
{
    int64_t t;
    uint8_t codes[256];
    uint8_t sc[8];
    if ((dtype != ORC_FP8 && dtype != ORC_MXFP4) || D < 32 || D > 256 || D % 32 || P < 1)
        return ORC_BAD_ARG;
    for (t = 0; t < N; ++t) {
        const int64_t s = slot_mapping[t];
        int64_t pg, sl;
        if (s < 0)
            continue;
        pg = s / P;
        sl = s % P;
        if (pg >= num_pages)
            continue;
        if (dtype == ORC_FP8) {
            float f;
            orc_quant_fp8_row(k + t * ld, D, codes, &f);
            memcpy(data + pg * page_stride + sl * row_stride, codes, (size_t)D);
            memcpy(scale + pg * scale_page_stride + sl * scale_row_stride, &f, 4);
        } else {
            orc_quant_mxfp4_row(k + t * ld, D, codes, sc);
            memcpy(data + pg * page_stride + sl * row_stride, codes, (size_t)D / 2);
            memcpy(scale + pg * scale_page_stride + sl * scale_row_stride, sc, (size_t)D / 32);
        }
    }
    return ORC_OK;
}

/* ---- Query quantization with the weight fold (ATOM PR #1709, commit on the
 * forward_pre / score_topk_from split: forward_pre returns the quantized q and
 * the weights; the FP4 path keeps its q scales beside them).
 * Readings: FP8 takes one scale per query row over all H*D values (the row
 * quantizer above on a row of H*D); with fold != 0 that scale goes into the
 * weights, w_out = (w*s)*c in single precision, and q_scale is not written;
 * otherwise q_scale[r] = s and w_out = w*c. MXFP4 takes the block quantizer
 * above on the row of H*D values (blocks of 32 never straddle a head since D
 * is a multiple of 32) and w_out = w*c. */
int orc_quantize_query(int dtype, const float *x, int64_t ld, int64_t R, int H, int D,
                       const float *w, float c, int fold, uint8_t *q, void *q_scale,
                       float *w_out)
{
    int64_t r;
    int h;
    const int n = H * D;
    if (dtype != ORC_FP8 && dtype != ORC_MXFP4)
        return ORC_BAD_ARG;
    if (n % 32 || R < 0)
        return ORC_BAD_ARG;
    for (r = 0; r < R; ++r) {
        const float *xr = x + r * ld;
        if (dtype == ORC_FP8) {
            float s;
            orc_quant_fp8_row(xr, n, q + r * n, &s);
            for (h = 0; h < H; ++h)
                w_out[r * H + h] = fold ? (w[r * H + h] * s) * c : w[r * H + h] * c;
            if (!fold)
                ((float *)q_scale)[r] = s;
        } else {
            orc_quant_mxfp4_row(xr, n, q + r * (n / 2), (uint8_t *)q_scale + r * (n / 32));
            for (h = 0; h < H; ++h)
                w_out[r * H + h] = w[r * H + h] * c;
        }
    }
    return ORC_OK;
}

/* ---- Ragged decode (ATOM PR #1709, commits on the ragged varlen windows:
 * sequence b's draft rows see windows ending at its committed length; a
 * rectangular step is the uniform case). Reading: sequence b owns the packed
 * rows [off[b], off[b+1]) (n_b of them) and its row j sees
 * max(0, lens[b] - (n_b - 1 - j)) keys, the rectangular rule with next_n
 * replaced by n_b. */

/* Sequence owning row r, or -1; by a linear walk over the offsets. */
static int64_t orc_row_owner(const int32_t *off, int B, int64_t r)
{
    int b;
    for (b = 0; b < B; ++b)
        if (off[b] <= r && r < off[b + 1])
            return b;
    return -1;
}

/* Visible ends of rows [0, R): the rule above; rows no sequence owns get 0. */
int orc_varlen_windows(const int32_t *lens, const int32_t *off, int B, int64_t R,
                       int64_t *E_out)
{
    int64_t r;
    int b;
    for (b = 0; b < B; ++b)
        if (off[b] < 0 || off[b + 1] < off[b])
            return ORC_BAD_ARG;
    for (r = 0; r < R; ++r) {
        const int64_t o = orc_row_owner(off, B, r);
        int64_t E = 0;
        if (o >= 0) {
            const int64_t n = off[o + 1] - off[o];
            const int64_t j = r - off[o];
            E = (int64_t)lens[o] - (n - 1 - j);
            if (E < 0)
                E = 0;
        }
        E_out[r] = E;
    }
    return ORC_OK;
}

/* Logits of the listed packed rows of a ragged decode step (rows no sequence
 * owns have E = 0 and an all -inf output). */
int orc_varlen_logits(int dtype, const uint8_t *q, const uint8_t *q_scale,
                      const float *w, int H, int D, const uint8_t *kdata,
                      int64_t page_stride, int64_t row_stride,
                      const uint8_t *kscale, int64_t scale_page_stride,
                      int64_t scale_row_stride, int page_size, int64_t num_pages,
                      const int32_t *block_tables, int64_t bt_stride,
                      const int32_t *lens, const int32_t *off, int B, int64_t R,
                      const int64_t *rows, int64_t nrows, int64_t W, double *out,
                      int64_t *E_out)
{
    int64_t i;
    int rc_all = ORC_OK;
    int64_t *Eall;
    if (orc_check_common(dtype, H, D, page_size) != ORC_OK)
        return ORC_BAD_ARG;
    for (i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= R)
            return ORC_BAD_ARG;
    Eall = (int64_t *)malloc((size_t)(R > 0 ? R : 1) * sizeof(int64_t));
    if (!Eall)
        return ORC_BAD_ARG;
    if (orc_varlen_windows(lens, off, B, R, Eall) != ORC_OK) {
        free(Eall);
        return ORC_BAD_ARG;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        const int64_t r = rows[i];
        const int64_t b = orc_row_owner(off, B, r);
        int rc;
        int64_t t;
        E_out[i] = Eall[r];
        if (b < 0) {
            for (t = 0; t < W; ++t)
                out[i * W + t] = -INFINITY;
            continue;
        }
        rc = orc_row(dtype, q, q_scale, w, H, D, r, kdata, page_stride, row_stride, kscale,
                     scale_page_stride, scale_row_stride, page_size, num_pages,
                     block_tables + b * bt_stride, Eall[r], W, out + i * W);
        if (rc != ORC_OK) {
#pragma omp critical
            rc_all = rc;
        }
    }
    free(Eall);
    return rc_all;
}

/* ---- Sparse attention over the selected tokens (the consumer of the
 * top-k: flashinfer PR #3269 "Add DeepSeek V4 sparse MLA TRTLLM-GEN
 * kernels", summary and review: a decode over dynamic per-row top-k lengths
 * with 512-dim QK and V, i.e. MLA where the values are the same latent rows
 * as the keys). Reading (the pages give only the API surface): row r of
 * sequence b = r / next_n with n = min(topk_lens[r], k) entries of
 * indices[r][.], entries < 0 skipped; for head h
 *     s_i = scale * (q[r][h] . c[t_i]),   out[r][h] = sum_i softmax(s)_i c[t_i]
 * with c[t] the bf16 latent row of sequence-local token t through the block
 * table; lse[r][h] = log sum_i exp(s_i). No selected token: out = 0,
 * lse = -inf. Everything in double precision from the bf16 inputs. */

static double orc_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

int orc_sparse_mla(const uint16_t *q, int64_t R, int H, int D,
                   const uint8_t *kv, int64_t page_stride, int64_t row_stride, int page_size,
                   int64_t num_pages, const int32_t *block_tables, int64_t bt_stride,
                   int next_n, const int32_t *indices, int64_t k, const int32_t *topk_lens,
                   double scale, double *out, double *lse)
{
    int64_t r;
    int rc_all = ORC_OK;
    if (R < 0 || H < 1 || D < 1 || page_size < 1 || next_n < 1 || k < 0)
        return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < R; ++r) {
        const int64_t b = r / next_n;
        int64_t n = topk_lens[r] < k ? topk_lens[r] : k;
        double *c = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)D);
        int64_t *ok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
        int64_t i, m = 0;
        int h, d;
        if (!c || !ok) {
#pragma omp critical
            rc_all = ORC_BAD_ARG;
            free(c);
            free(ok);
            continue;
        }
        if (n < 0)
            n = 0;
        /* gather the selected latent rows */
        for (i = 0; i < n; ++i) {
            const int32_t t = indices[r * k + i];
            int64_t lp, pg;
            const uint8_t *row;
            if (t < 0)
                continue;
            lp = t / page_size;
            if (lp >= bt_stride) {
#pragma omp critical
                rc_all = ORC_BAD_PAGE;
                continue;
            }
            pg = block_tables[b * bt_stride + lp];
            if (pg < 0 || pg >= num_pages) {
#pragma omp critical
                rc_all = ORC_BAD_PAGE;
                continue;
            }
            row = kv + pg * page_stride + (int64_t)(t % page_size) * row_stride;
            for (d = 0; d < D; ++d) {
                uint16_t v;
                memcpy(&v, row + 2 * d, 2);
                c[m * D + d] = orc_bf16(v);
            }
            ok[m++] = i;
        }
        for (h = 0; h < H; ++h) {
            const uint16_t *qh = q + (r * H + h) * (int64_t)D;
            double *o = out + (r * H + h) * (int64_t)D;
            double mx = -INFINITY, sum = 0.0;
            double *s = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
            for (d = 0; d < D; ++d)
                o[d] = 0.0;
            if (!s) {
#pragma omp critical
                rc_all = ORC_BAD_ARG;
                continue;
            }
            for (i = 0; i < m; ++i) {
                double acc = 0.0;
                for (d = 0; d < D; ++d)
                    acc += orc_bf16(qh[d]) * c[i * D + d];
                s[i] = scale * acc;
                mx = s[i] > mx ? s[i] : mx;
            }
            for (i = 0; i < m; ++i)
                sum += exp(s[i] - mx);
            for (i = 0; i < m; ++i) {
                const double p = exp(s[i] - mx) / sum;
                for (d = 0; d < D; ++d)
                    o[d] += p * c[i * D + d];
            }
            if (lse)
                lse[r * H + h] = m > 0 ? mx + log(sum) : -INFINITY;
            free(s);
        }
        free(c);
        free(ok);
    }
    return rc_all;
}
