/*
 * oracle.c -- plain, slow float64 CPU reference of the fused row-wise
 * vocabulary-softmax loss.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library, and nothing in the product path
 * calls it.
 *
 * Every function is the plain definition written out in float64: one scalar
 * loop per row, indices in natural order, no blocking or fusion.  OpenMP
 * splits independent rows across host threads and changes no arithmetic.
 *
 * Inputs are the exact bytes the GPU receives.  float32 logits are widened
 * exactly; bf16 logits (raw uint16 bit patterns) are widened exactly as
 * bits << 16.
 *
 * Sources (the pages):
 *   [CE]  aprender-train 0.36.0, entrenar/autograd/wgpu_cross_entropy.rs:
 *         module doc (forward and backward formulas), CEForwardParams and
 *         CEBackwardParams (the loss range and scale), read_loss (the mean
 *         over the loss range), forward_async (loss and logsumexp per row),
 *         backward (gradient written in place from the saved logsumexp).
 *   [KL]  cortiq-engine 0.8.21, src/gpu_wgpu/train_head.rs: module doc (the
 *         distillation loss and its gradient), the kl_rows kernel, the
 *         topk_rows kernel (teacher top-k with probabilities renormalised
 *         over the k), the acc_add kernel (slice gradient sum).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Value j of a row given as raw bytes, widened exactly to float64. */
static double widen(const void *row, int dtype, int64_t j)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)row)[j];
    uint32_t bits = (uint32_t)((const uint16_t *)row)[j] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static const void *row_ptr(const void *base, int dtype, int64_t i, int64_t V)
{
    size_t elt = dtype == ORACLE_F32 ? 4 : 2;
    return (const char *)base + (size_t)i * (size_t)V * elt;
}

/*
 * Loss range [CE: CEForwardParams / read_loss]: a row takes part in the loss
 * when start <= r mod seq_len < end.  seq_len <= 0 means every row does.
 */
static int in_loss(int64_t r, int64_t seq_len, int64_t start, int64_t end)
{
    if (seq_len <= 0)
        return 1;
    int64_t p = r % seq_len;
    return start <= p && p < end;
}

/*
 * logsumexp of one row [KL: module doc, log p_S = s - logsumexp(s); CE:
 * module doc]: m = max_j s_j, then m + ln sum_j exp(s_j - m), summed in
 * index order.
 */
double oracle_row_lse(const void *row, int dtype, int64_t V)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j) {
        double s = widen(row, dtype, j);
        if (s > m)
            m = s;
    }
    double z = 0.0;
    for (int64_t j = 0; j < V; ++j)
        z += exp(widen(row, dtype, j) - m);
    return m + log(z);
}

/*
 * Cross-entropy forward and backward [CE: module doc, backward]:
 *   loss_r = logsumexp(s) - s_label
 *   grad_rj = scale * (softmax(s)_j - [j == label])
 * Rows outside the loss range get loss 0, lse 0 and gradient 0: read_loss
 * sums every row's loss and divides by the number of rows in the range, so
 * the loss of a row outside it must be 0, and the gradient of that mean is 0
 * there.
 *
 * rows: nrows rows of V logits, contiguous.  row_index[i] is the global row
 * number of row i (used only for the loss-range test); NULL means i.
 * grad may be NULL (loss and lse only).
 */
void oracle_ce(const void *logits, int dtype, const uint32_t *labels,
               int64_t nrows, int64_t V, const int64_t *row_index,
               int64_t seq_len, int64_t start, int64_t end, double scale,
               double *loss, double *lse, double *grad)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const void *row = row_ptr(logits, dtype, i, V);
        int64_t r = row_index ? row_index[i] : i;
        double *g = grad ? grad + i * V : NULL;
        if (!in_loss(r, seq_len, start, end)) {
            loss[i] = 0.0;
            lse[i] = 0.0;
            if (g)
                for (int64_t j = 0; j < V; ++j)
                    g[j] = 0.0;
            continue;
        }
        double L = oracle_row_lse(row, dtype, V);
        int64_t label = (int64_t)labels[i];
        loss[i] = L - widen(row, dtype, label);
        lse[i] = L;
        if (g)
            for (int64_t j = 0; j < V; ++j) {
                double onehot = (j == label) ? 1.0 : 0.0;
                g[j] = scale * (exp(widen(row, dtype, j) - L) - onehot);
            }
    }
}

/*
 * Cross-entropy backward from a saved logsumexp [CE: backward, which takes
 * the logsumexp the forward pass stored instead of reducing the row again]:
 *   grad_rj = scale * (exp(s_j - lse_r) - [j == label])
 * lse_r is the given float32 value, widened exactly and used as given.
 * Rows outside the loss range get gradient 0, as in oracle_ce.
 */
void oracle_ce_bwd(const void *logits, int dtype, const uint32_t *labels, const float *lse,
                   int64_t nrows, int64_t V, const int64_t *row_index, int64_t seq_len,
                   int64_t start, int64_t end, double scale, double *grad)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const void *row = row_ptr(logits, dtype, i, V);
        int64_t r = row_index ? row_index[i] : i;
        double *g = grad + i * V;
        if (!in_loss(r, seq_len, start, end)) {
            for (int64_t j = 0; j < V; ++j)
                g[j] = 0.0;
            continue;
        }
        double L = (double)lse[i];
        int64_t label = (int64_t)labels[i];
        for (int64_t j = 0; j < V; ++j) {
            double onehot = (j == label) ? 1.0 : 0.0;
            g[j] = scale * (exp(widen(row, dtype, j) - L) - onehot);
        }
    }
}

/*
 * Mean loss [CE: read_loss]: the sum of the loss over every row (rows
 * outside the range hold 0 after the forward) divided by the number of rows
 * in the loss range, or 0 when the range holds no row.  Summed in index
 * order.
 */
double oracle_loss_mean(const float *loss, int64_t nrows, int64_t seq_len, int64_t start,
                        int64_t end)
{
    double sum = 0.0;
    int64_t count = 0;
    for (int64_t i = 0; i < nrows; ++i) {
        sum += (double)loss[i];
        count += in_loss(i, seq_len, start, end);
    }
    return count > 0 ? sum / (double)count : 0.0;
}

/*
 * Distillation KL forward and backward [KL: module doc, kl_rows]:
 *   loss_r = sum over q with p_q > 0 of p_q * (ln p_q - (s_{id_q} - lse))
 *   grad_rj = coef * (softmax(s)_j - t_j),  t_j = sum of p_q over q: id_q == j
 * Terms with p_q = 0 add nothing (0 ln 0 = 0).  The teacher probabilities are
 * used exactly as given (no renormalisation).  Rows outside the loss range
 * get loss 0, lse 0 and gradient 0, as for the cross-entropy.
 *
 * ids, probs: nrows x k, the rows matching the logits rows.
 */
void oracle_kl(const void *logits, int dtype, const uint32_t *ids,
               const float *probs, int64_t k, int64_t nrows, int64_t V,
               const int64_t *row_index, int64_t seq_len, int64_t start,
               int64_t end, double coef, double *loss, double *lse,
               double *grad)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const void *row = row_ptr(logits, dtype, i, V);
        int64_t r = row_index ? row_index[i] : i;
        double *g = grad ? grad + i * V : NULL;
        if (!in_loss(r, seq_len, start, end)) {
            loss[i] = 0.0;
            lse[i] = 0.0;
            if (g)
                for (int64_t j = 0; j < V; ++j)
                    g[j] = 0.0;
            continue;
        }
        double L = oracle_row_lse(row, dtype, V);
        const uint32_t *id = ids + i * k;
        const float *p = probs + i * k;
        double acc = 0.0;
        for (int64_t q = 0; q < k; ++q) {
            double pq = (double)p[q];
            if (pq > 0.0)
                acc += pq * (log(pq) - (widen(row, dtype, (int64_t)id[q]) - L));
        }
        loss[i] = acc;
        lse[i] = L;
        if (g) {
            double *t = calloc((size_t)V, sizeof(double));
            for (int64_t q = 0; q < k; ++q)
                t[id[q]] += (double)p[q];
            for (int64_t j = 0; j < V; ++j)
                g[j] = coef * (exp(widen(row, dtype, j) - L) - t[j]);
            free(t);
        }
    }
}

typedef struct {
    double v;
    int64_t id;
} keyed;

/* Order for the teacher top-k: larger value first, then lower id first.
 * -0 and +0 compare equal, so they tie and the lower id wins. */
static int by_value_desc_id_asc(const void *a, const void *b)
{
    const keyed *x = a, *y = b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    return (x->id > y->id) - (x->id < y->id);
}

/*
 * Teacher top-k with renormalised probabilities [KL: topk_rows]:
 * ids = the k entries of the row that come first in the order (value
 * descending, id ascending); probs_q = exp(v_q - v_0) / sum_{q'<k}
 * exp(v_q' - v_0), v_0 the largest value: the softmax restricted to the k.
 * The whole row is sorted (a library sort) and the first k are kept.
 */
void oracle_topk(const void *logits, int dtype, int64_t nrows, int64_t V,
                 int64_t k, uint32_t *ids, double *probs)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const void *row = row_ptr(logits, dtype, i, V);
        keyed *e = malloc((size_t)V * sizeof(keyed));
        for (int64_t j = 0; j < V; ++j) {
            e[j].v = widen(row, dtype, j);
            e[j].id = j;
        }
        qsort(e, (size_t)V, sizeof(keyed), by_value_desc_id_asc);
        double v0 = e[0].v;
        double z = 0.0;
        for (int64_t q = 0; q < k; ++q)
            z += exp(e[q].v - v0);
        for (int64_t q = 0; q < k; ++q) {
            ids[i * k + q] = (uint32_t)e[q].id;
            probs[i * k + q] = exp(e[q].v - v0) / z;
        }
        free(e);
    }
}

/*
 * Slice accumulate [KL: acc_add]: out_i = dst_i + src_i for i < n, the
 * float32 sum.  Formed in float64 and rounded once to float32, which equals
 * the correctly rounded float32 sum (double has at least 2*24+2 bits, so the
 * double rounding is harmless).
 */
void oracle_acc(const float *dst, const float *src, int64_t n, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)((double)dst[i] + (double)src[i]);
}

/*
 * Host threads the row loops use: the OpenMP runtime's current maximum, and
 * a setter (n >= 1) for timing the oracle on a chosen number of cores.
 * Neither changes any arithmetic.
 */
int oracle_threads(void)
{
    return omp_get_max_threads();
}

void oracle_set_threads(int n)
{
    omp_set_num_threads(n >= 1 ? n : 1);
}
