/*
 * Float64 CPU oracle for the online-softmax attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the HIP path is checked against.  Only the test suite, the
 * smoke check and the bench's CPU-baseline leg may load it.  It shares no
 * code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * Everything is computed in IEEE double from the exact stored input values
 * (bf16 or fp32 widened to double by the caller).  There is no blocking, no
 * fusion and no reordering beyond the definitions cited at each function.
 * Rows are independent, so an OpenMP parallel-for over rows is the only
 * concurrency.
 *
 * Built with:  gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/*
 * Safe softmax in three passes, row by row.
 * Source: "Online Softmax and Flash Attention" page, section "Safe softmax",
 * eq. (2) and its three-pass description (max, sum of exponentials, divide);
 * "从原始Softmax到在线Softmax" page, "softmax形式推导" (p_j = e^{z_j-m}/sum_k e^{z_k-m}).
 * x, y: row-major [rows, n], n >= 1.
 */
void oracle_softmax_f64(const double *x, double *y, int64_t rows, int64_t n)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double *yr = y + r * n;
        /* pass 1: the maximum */
        double m = xr[0];
        for (int64_t j = 1; j < n; ++j)
            if (xr[j] > m) m = xr[j];
        /* pass 2: the sum of shifted exponentials */
        double s = 0.0;
        for (int64_t j = 0; j < n; ++j)
            s += exp(xr[j] - m);
        /* pass 3: divide */
        for (int64_t j = 0; j < n; ++j)
            yr[j] = exp(xr[j] - m) / s;
    }
}

/*
 * Log-sum-exp of each row: LSE(z) = m + log sum_k e^{z_k - m}.
 * Source: "从原始Softmax到在线Softmax" page, "softmax形式推导" (log-softmax and
 * LSE definitions).
 */
void oracle_logsumexp_f64(const double *x, double *lse, int64_t rows, int64_t n)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double m = xr[0];
        for (int64_t j = 1; j < n; ++j)
            if (xr[j] > m) m = xr[j];
        double s = 0.0;
        for (int64_t j = 0; j < n; ++j)
            s += exp(xr[j] - m);
        lse[r] = m + log(s);
    }
}

/*
 * Softmax cross-entropy of each row against its class label, and the row LSE.
 * Source: "从原始Softmax到在线Softmax" page, section "softmax实际代码实现" (the
 * cross-entropy loss: row max, shifted exponentials and their sum, log
 * probabilities z - max - log(sum), the label's entry, negated) and the
 * log-softmax / LSE definitions of "softmax形式推导".
 * x: row-major [rows, n], n >= 1; labels: [rows].  A label outside [0, n) has
 * no log probability: its loss is NaN.
 */
void oracle_xent_f64(const double *x, const int64_t *labels, double *loss, double *lse, int64_t rows, int64_t n)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double m = xr[0];
        for (int64_t j = 1; j < n; ++j)
            if (xr[j] > m) m = xr[j];
        double s = 0.0;
        for (int64_t j = 0; j < n; ++j)
            s += exp(xr[j] - m);
        const double log_sum = log(s);
        lse[r] = m + log_sum;
        const int64_t c = labels[r];
        if (c < 0 || c >= n) {
            loss[r] = NAN;
        } else {
            const double log_prob = xr[c] - m - log_sum;
            loss[r] = -log_prob;
        }
    }
}

/*
 * The one-pass normaliser: the pair (m, s) of a prefix of the row -- its
 * maximum and the sum of e^{x - m} over it -- extended by one element at a
 * time, m' = max(m, x_i) and s' = s e^{m - m'} + e^{x_i - m'}.  The empty
 * prefix is (m, s) = (-inf, 0) and contributes nothing when it is carried to
 * the first finite maximum; leading -inf elements leave it empty.
 * Source: "Online Softmax and Flash Attention" page, section "Online softmax",
 * eq. (3)-(5); "Softmax与Flash-Attention" page, "online-softmax 推导".
 * Writes the final m_N and s_N of each row.  Kept only to check that s_N equals
 * the two-pass denominator (eq. (6)-(7)); the attention oracle does not use it.
 */
void oracle_online_normalizer_f64(const double *x, double *m_out, double *s_out,
                                  int64_t rows, int64_t n)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double m = -INFINITY; /* the empty prefix */
        double s = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double m_next = xr[i] > m ? xr[i] : m;
            if (m_next == -INFINITY)
                continue;
            const double carried = m == -INFINITY ? 0.0 : s * exp(m - m_next);
            s = carried + exp(xr[i] - m_next);
            m = m_next;
        }
        m_out[r] = m;
        s_out[r] = s;
    }
}

/*
 * Exact attention for selected query rows.
 *
 * Definition: A = softmax(mask(Q K^T * scale)) V, per head, with Q [N,d],
 * K and V [M,d].  Source: "Online Softmax and Flash Attention" page, eq. (8)
 * (shapes stated under it) and the 1/sqrt(K) scale folded into the product;
 * three-pass safe softmax as above; LSE from the "softmax形式推导" section
 * of the "从原始Softmax到在线Softmax" page.
 *
 * mask() (the page leaves it open): key j of batch b is masked for query i
 * when
 *   - j >= kv_len[b]            (kv_len != NULL: the batch's valid key count),
 *   - j > i                     (causal_mode 1: key index greater than query
 *                                index, counted from 0 in both),
 *   - j > i + (M - N)           (causal_mode 2: the same, aligned at the last
 *                                query and the last key).
 * The visible keys of a row are therefore a prefix [0, visible).  A row with
 * no visible key has an empty sum: o = 0 and LSE = -inf.
 *
 * Additive bias (optional; the elementwise mask() read as "add a term to
 * each score"): s_ij = scale * <q_i, k_j> + bias[b*bias_sb + h*bias_sh +
 * i*bias_sn + j], strides in elements, 0 to broadcast.  A bias of -inf masks
 * its key; a row whose visible scores are all -inf is treated as one with no
 * visible key.
 *
 * q: [B,H,N,d], k and v: [B,H,M,d], contiguous.  rows: flat indices
 * r = (b*H + h)*N + i.  Outputs: o_rows [nrows, d], lse_rows [nrows] (natural
 * log over the scaled, masked scores).
 */
void oracle_attn_masked_rows_f64(const double *q, const double *k, const double *v,
                                 int64_t B, int64_t H, int64_t N, int64_t M, int64_t d,
                                 double scale, int causal_mode, const int64_t *kv_len,
                                 const double *bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_sn,
                                 const int64_t *rows, int64_t nrows,
                                 double *o_rows, double *lse_rows)
{
    (void)B;
    int64_t t;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)M * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (t = 0; t < nrows; ++t) {
            int64_t r = rows[t];
            int64_t bh = r / N;
            int64_t i = r % N;
            const double *qi = q + r * d;
            const double *kh = k + bh * M * d;
            const double *vh = v + bh * M * d;
            double *oi = o_rows + t * d;
            /* The visible keys of row i are a prefix [0, visible). */
            int64_t visible = M;
            if (kv_len && kv_len[bh / H] < visible) visible = kv_len[bh / H] > 0 ? kv_len[bh / H] : 0;
            if (causal_mode == 1 && i + 1 < visible) visible = i + 1;
            if (causal_mode == 2 && i + 1 + (M - N) < visible) visible = i + 1 + (M - N) > 0 ? i + 1 + (M - N) : 0;
            if (visible == 0) {
                /* No visible key: an empty sum; o = 0 and LSE = log 0. */
                for (int64_t c = 0; c < d; ++c)
                    oi[c] = 0.0;
                lse_rows[t] = -INFINITY;
                continue;
            }

            /* scores s_j = scale * <q_i, k_j> (+ bias_ij) for the visible keys */
            const double *brow = bias ? bias + (bh / H) * bias_sb + (bh % H) * bias_sh + i * bias_sn : NULL;
            for (int64_t j = 0; j < visible; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc += qi[c] * kh[j * d + c];
                s[j] = scale * acc;
                if (brow)
                    s[j] += brow[j];
            }
            /* pass 1: max */
            double m = s[0];
            for (int64_t j = 1; j < visible; ++j)
                if (s[j] > m) m = s[j];
            if (m == -INFINITY) {
                /* Every visible score is -inf (a bias of -inf masks its key):
                   as with no visible key. */
                for (int64_t c = 0; c < d; ++c)
                    oi[c] = 0.0;
                lse_rows[t] = m;
                continue;
            }
            /* pass 2: sum of shifted exponentials */
            double l = 0.0;
            for (int64_t j = 0; j < visible; ++j)
                l += exp(s[j] - m);
            /* pass 3: probabilities times V */
            for (int64_t c = 0; c < d; ++c)
                oi[c] = 0.0;
            for (int64_t j = 0; j < visible; ++j) {
                double p = exp(s[j] - m) / l;
                for (int64_t c = 0; c < d; ++c)
                    oi[c] += p * vh[j * d + c];
            }
            lse_rows[t] = m + log(l);
        }
        free(s);
    }
}

/* No mask (causal = 0) or the top-left causal mask (causal != 0). */
void oracle_attn_rows_f64(const double *q, const double *k, const double *v,
                          int64_t B, int64_t H, int64_t N, int64_t M, int64_t d,
                          double scale, int causal,
                          const int64_t *rows, int64_t nrows,
                          double *o_rows, double *lse_rows)
{
    oracle_attn_masked_rows_f64(q, k, v, B, H, N, M, d, scale, causal ? 1 : 0, NULL, NULL, 0, 0, 0, rows, nrows,
                                o_rows, lse_rows);
}

/* All rows of all heads: o [B,H,N,d], lse [B,H,N]. */
void oracle_attn_f64(const double *q, const double *k, const double *v,
                     double *o, double *lse,
                     int64_t B, int64_t H, int64_t N, int64_t M, int64_t d,
                     double scale, int causal)
{
    int64_t total = B * H * N;
    int64_t *rows = (int64_t *)malloc((size_t)(total > 0 ? total : 1) * sizeof(int64_t));
    for (int64_t r = 0; r < total; ++r)
        rows[r] = r;
    oracle_attn_rows_f64(q, k, v, B, H, N, M, d, scale, causal, rows, total, o, lse);
    free(rows);
}

/* Threads OpenMP will use for the calls above. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
