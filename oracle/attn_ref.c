/*
 * FP64 reference attention -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the oracle against which the GPU attention library is checked.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header or constant with the GPU library.
 *
 * What it computes is the plain definition of scaled-dot-product attention
 * as given on the page "Ch.04 Attention optimisation: FlashAttention and
 * sparse attention" (mdooai.com), sections "Core formula" and "Key points of
 * the formulas":
 *
 *     S_ij = scale * (q_i . k_j)           (scale = 1/sqrt(d_k) by default)
 *     A_i: = softmax_j(S_i:),  sum_j A_ij = 1
 *     O_i  = sum_j A_ij v_j                (O = A V)
 *
 * and the same page's sparse-attention rule: for a key j outside the allowed
 * set of query i the logit is set to -infinity before the softmax, so A_ij = 0.
 * The FlashAttention summary page ("FlashAttention: Fast and Memory-Efficient
 * Exact Attention with IO-Awareness", ai-paper-library, Summary and Method)
 * states the tiled method is exact, i.e. it reaches this same result; the
 * oracle is therefore the definition itself, written out with S (and A, in
 * place) materialised, with no tiling and no online softmax.
 *
 * Allowed-set readings where the pages are silent:
 *   causal      : key j allowed for query i iff j <= i
 *   key padding : key j allowed iff j < key_len[b]
 *   block mask  : key j allowed iff mask[(i / blk) * nkb + (j / blk)] != 0,
 *                 nkb = ceil(N / blk); the mask is shared by every (b, h)
 *   a row with no allowed key gets O_i = 0 and LSE_i = -infinity.
 * The row maximum is subtracted before exp (a rewrite that leaves the softmax
 * unchanged) so that large logits do not overflow.
 * LSE_i = log(sum_j exp(S_ij)) in natural log.
 *
 * Layout: q, o are contiguous [B, H, N, d]; k, v are [B, H, N, d] (or
 * [B, Hkv, N, d] for the grouped-query entry points); lse is [B, H, N].
 * Build: gcc -O3 -march=native -std=c11 -fopenmp -shared -fPIC (oracle/build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static int key_allowed(int64_t i, int64_t j, int64_t b, int causal,
                       const int32_t *key_len, const uint8_t *block_mask,
                       int64_t blk, int64_t nkb)
{
    if (causal && j > i) return 0;
    if (key_len && j >= (int64_t)key_len[b]) return 0;
    if (block_mask && block_mask[(i / blk) * nkb + (j / blk)] == 0) return 0;
    return 1;
}

/* Softmax of one materialised row s[0..N) in place (s becomes the row of A),
 * then o = A_row V and the row's logsumexp.  Returns nothing; a row whose
 * logits are all -inf gives o = 0, lse = -inf. */
static void softmax_row_times_v(double *s, const double *vh, double *o,
                                double *lse, int64_t N, int64_t d)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j)
        if (s[j] > m) m = s[j];
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    if (m == -INFINITY) {
        for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        s[j] = exp(s[j] - m); /* exp(-inf) = 0 for masked keys */
        l += s[j];
    }
    for (int64_t j = 0; j < N; ++j) s[j] /= l;
    for (int64_t j = 0; j < N; ++j) {
        if (s[j] == 0.0) continue;
        const double *vj = vh + j * d;
        for (int64_t c = 0; c < d; ++c) o[c] += s[j] * vj[c];
    }
    *lse = m + log(l);
}

static void score_row(double *s, const double *qi, const double *kh, int64_t i,
                      int64_t b, int64_t N, int64_t d, double scale, int causal,
                      const int32_t *key_len, const uint8_t *block_mask,
                      int64_t blk, int64_t nkb)
{
    for (int64_t j = 0; j < N; ++j) {
        if (!key_allowed(i, j, b, causal, key_len, block_mask, blk, nkb)) {
            s[j] = -INFINITY;
            continue;
        }
        const double *kj = kh + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
        s[j] = scale * dot;
    }
}

static int check_args(const double *q, const double *k, const double *v,
                      int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                      const uint8_t *block_mask, int64_t blk)
{
    if (!q || !k || !v) return 1;
    if (B < 0 || H < 0 || N < 0 || d <= 0) return 2;
    if (Hkv <= 0 || H % Hkv != 0) return 2;
    if (block_mask && blk <= 0) return 2;
    return 0;
}

/* Key/value head used by query head h of batch entry b when the H query
 * heads share Hkv key/value heads in consecutive groups of H / Hkv
 * (grouped-query attention, on the page on FlashAttention-2 adoption,
 * tcdigital.jp, section on the synergy with MQA/GQA; Hkv = H is plain
 * multi-head attention).  k and v are [B, Hkv, N, d]. */
static int64_t kv_head(int64_t b, int64_t h, int64_t H, int64_t Hkv)
{
    return b * Hkv + h / (H / Hkv);
}

/* Full evaluation: every (b, h) head, S materialised as an N x N array of
 * doubles one head at a time (A overwrites S in place).  Returns 0 on success,
 * non-zero on bad arguments or allocation failure. */
int attn_ref_gqa_f64(const double *q, const double *k, const double *v, double *o,
                     double *lse, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                     int64_t d, double scale, int causal, const int32_t *key_len,
                     const uint8_t *block_mask, int64_t blk)
{
    int rc = check_args(q, k, v, B, H, Hkv, N, d, block_mask, blk);
    if (rc) return rc;
    if (!o || !lse) return 1;
    if (N == 0) return 0;
    const int64_t nkb = block_mask ? (N + blk - 1) / blk : 0;
    double *S = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    if (!S) return 3;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t head = (b * H + h) * N, kvh = kv_head(b, h, H, Hkv) * N;
            const double *qh = q + head * d, *kh = k + kvh * d, *vh = v + kvh * d;
            double *oh = o + head * d, *lh = lse + head;
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t i = 0; i < N; ++i)
                score_row(S + i * N, qh + i * d, kh, i, b, N, d, scale, causal,
                          key_len, block_mask, blk, nkb);
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t i = 0; i < N; ++i)
                softmax_row_times_v(S + i * N, vh, oh + i * d, lh + i, N, d);
        }
    }
    free(S);
    return 0;
}

/* Plain multi-head attention: one key/value head per query head. */
int attn_ref_f64(const double *q, const double *k, const double *v, double *o,
                 double *lse, int64_t B, int64_t H, int64_t N, int64_t d,
                 double scale, int causal, const int32_t *key_len,
                 const uint8_t *block_mask, int64_t blk)
{
    return attn_ref_gqa_f64(q, k, v, o, lse, B, H, H, N, d, scale, causal,
                            key_len, block_mask, blk);
}

/* Sampled evaluation: only the query rows listed in rows[] are computed.
 * rows[r] is a flat row index (b * H + h) * N + i.  o_rows is [n_rows, d],
 * lse_rows is [n_rows].  Each row is the same definition as above, with that
 * row of S materialised on its own. */
int attn_ref_rows_gqa_f64(const double *q, const double *k, const double *v,
                          int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                          double scale, int causal, const int32_t *key_len,
                          const uint8_t *block_mask, int64_t blk,
                          const int64_t *rows, int64_t n_rows, double *o_rows,
                          double *lse_rows)
{
    int rc = check_args(q, k, v, B, H, Hkv, N, d, block_mask, blk);
    if (rc) return rc;
    if (n_rows > 0 && (!rows || !o_rows || !lse_rows)) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * H * N) return 2;
    if (n_rows == 0) return 0;
    const int64_t nkb = block_mask ? (N + blk - 1) / blk : 0;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            const int64_t flat = rows[r];
            const int64_t head = flat / N, i = flat % N, b = head / H;
            const int64_t kvh = kv_head(b, head - b * H, H, Hkv);
            const double *kh = k + kvh * N * d, *vh = v + kvh * N * d;
            score_row(s, q + flat * d, kh, i, b, N, d, scale, causal, key_len,
                      block_mask, blk, nkb);
            softmax_row_times_v(s, vh, o_rows + r * d, lse_rows + r, N, d);
        }
        free(s);
    }
    return failed ? 3 : 0;
}

int attn_ref_rows_f64(const double *q, const double *k, const double *v,
                      int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                      int causal, const int32_t *key_len,
                      const uint8_t *block_mask, int64_t blk,
                      const int64_t *rows, int64_t n_rows, double *o_rows,
                      double *lse_rows)
{
    return attn_ref_rows_gqa_f64(q, k, v, B, H, H, N, d, scale, causal, key_len,
                                 block_mask, blk, rows, n_rows, o_rows, lse_rows);
}

/* Gradients of the definition (backward pass) -- not printed on the pages,
 * which give only the forward definition; this is its derivative, written
 * out plainly.  With the loss L = sum_{i,c} dO_ic O_ic (so dL/dO = dO):
 *     A_ij  = softmax_j(S_ij)               (0 for disallowed keys)
 *     dV_j  = sum_i A_ij dO_i
 *     dA_ij = dO_i . V_j
 *     D_i   = dO_i . O_i  (= sum_j A_ij dA_ij)
 *     dS_ij = A_ij (dA_ij - D_i)
 *     dQ_i  = scale * sum_j dS_ij K_j
 *     dK_j  = scale * sum_i dS_ij Q_i
 * With grouped key/value heads, dK and dV of a key/value head sum the
 * contributions of every query head of its group.  One head at a time, A
 * (then dS, in place) materialised as an N x N array of doubles.  dq is
 * [B, H, N, d]; dk and dv are [B, Hkv, N, d] and are overwritten. */
int attn_bwd_ref_gqa_f64(const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk, double *dv,
                         int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                         double scale, int causal, const int32_t *key_len,
                         const uint8_t *block_mask, int64_t blk)
{
    int rc = check_args(q, k, v, B, H, Hkv, N, d, block_mask, blk);
    if (rc) return rc;
    if (!dout || !dq || !dk || !dv) return 1;
    for (int64_t x = 0; x < B * H * N * d; ++x) dq[x] = 0.0;
    for (int64_t x = 0; x < B * Hkv * N * d; ++x) dk[x] = dv[x] = 0.0;
    if (N == 0) return 0;
    const int64_t nkb = block_mask ? (N + blk - 1) / blk : 0;
    double *A = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    double *O = (double *)malloc((size_t)N * (size_t)d * sizeof(double));
    double *Dr = (double *)malloc((size_t)N * sizeof(double));
    if (!A || !O || !Dr) {
        free(A);
        free(O);
        free(Dr);
        return 3;
    }
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t head = (b * H + h) * N, kvh = kv_head(b, h, H, Hkv) * N;
            const double *qh = q + head * d, *kh = k + kvh * d, *vh = v + kvh * d;
            const double *doh = dout + head * d;
            double *dqh = dq + head * d, *dkh = dk + kvh * d, *dvh = dv + kvh * d;
            /* A and O (the forward definition), D_i = dO_i . O_i */
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t i = 0; i < N; ++i) {
                double lse_unused;
                score_row(A + i * N, qh + i * d, kh, i, b, N, d, scale, causal,
                          key_len, block_mask, blk, nkb);
                softmax_row_times_v(A + i * N, vh, O + i * d, &lse_unused, N, d);
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c) acc += doh[i * d + c] * O[i * d + c];
                Dr[i] = acc;
            }
            /* dV_j += sum_i A_ij dO_i */
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t j = 0; j < N; ++j) {
                for (int64_t i = 0; i < N; ++i) {
                    const double a = A[i * N + j];
                    if (a == 0.0) continue;
                    for (int64_t c = 0; c < d; ++c) dvh[j * d + c] += a * doh[i * d + c];
                }
            }
            /* dS_ij = A_ij (dO_i . V_j - D_i), in place of A */
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t i = 0; i < N; ++i) {
                for (int64_t j = 0; j < N; ++j) {
                    const double a = A[i * N + j];
                    if (a == 0.0) continue;
                    double da = 0.0;
                    for (int64_t c = 0; c < d; ++c) da += doh[i * d + c] * vh[j * d + c];
                    A[i * N + j] = a * (da - Dr[i]);
                }
            }
            /* dQ_i = scale sum_j dS_ij K_j */
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t i = 0; i < N; ++i)
                for (int64_t j = 0; j < N; ++j) {
                    const double ds = A[i * N + j];
                    if (ds == 0.0) continue;
                    for (int64_t c = 0; c < d; ++c) dqh[i * d + c] += scale * ds * kh[j * d + c];
                }
            /* dK_j += scale sum_i dS_ij Q_i */
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t j = 0; j < N; ++j)
                for (int64_t i = 0; i < N; ++i) {
                    const double ds = A[i * N + j];
                    if (ds == 0.0) continue;
                    for (int64_t c = 0; c < d; ++c) dkh[j * d + c] += scale * ds * qh[i * d + c];
                }
        }
    }
    free(A);
    free(O);
    free(Dr);
    return 0;
}

/* Sampled gradients, by row: dQ_i for the query rows listed in rows[]
 * (flat index (b * H + h) * N + i), each from that row of A evaluated on its
 * own -- the same formulas as the full backward above, restricted to one
 * row:  D_i = dO_i . O_i,  dQ_i = scale * sum_j A_ij (dO_i . V_j - D_i) K_j.
 * dq_rows is [n_rows, d]. */
int attn_bwd_rows_gqa_f64(const double *q, const double *k, const double *v,
                          const double *dout, int64_t B, int64_t H, int64_t Hkv,
                          int64_t N, int64_t d, double scale, int causal,
                          const int32_t *key_len, const uint8_t *block_mask,
                          int64_t blk, const int64_t *rows, int64_t n_rows,
                          double *dq_rows)
{
    int rc = check_args(q, k, v, B, H, Hkv, N, d, block_mask, blk);
    if (rc) return rc;
    if (!dout || (n_rows > 0 && (!rows || !dq_rows))) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * H * N) return 2;
    if (n_rows == 0) return 0;
    const int64_t nkb = block_mask ? (N + blk - 1) / blk : 0;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *o = (double *)malloc((size_t)d * sizeof(double));
        if (!s || !o) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s || !o) continue;
            const int64_t flat = rows[r];
            const int64_t head = flat / N, i = flat % N, b = head / H;
            const int64_t kvh = kv_head(b, head - b * H, H, Hkv);
            const double *kh = k + kvh * N * d, *vh = v + kvh * N * d;
            const double *doi = dout + flat * d;
            double lse_unused;
            score_row(s, q + flat * d, kh, i, b, N, d, scale, causal, key_len,
                      block_mask, blk, nkb);
            softmax_row_times_v(s, vh, o, &lse_unused, N, d);
            double Di = 0.0;
            for (int64_t c = 0; c < d; ++c) Di += doi[c] * o[c];
            double *dqi = dq_rows + r * d;
            for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                const double a = s[j];
                if (a == 0.0) continue;
                double da = 0.0;
                for (int64_t c = 0; c < d; ++c) da += doi[c] * vh[j * d + c];
                const double ds = a * (da - Di);
                for (int64_t c = 0; c < d; ++c) dqi[c] += scale * ds * kh[j * d + c];
            }
        }
        free(s);
        free(o);
    }
    return failed ? 3 : 0;
}

/* Sampled gradients, by key: dK_j and dV_j for the keys listed in cols[]
 * (flat index (b * Hkv + g) * N + j), summed over every query row of every
 * query head that reads key/value head g:
 *     dV_j = sum_i A_ij dO_i,   dK_j = scale * sum_i A_ij (dO_i . V_j - D_i) Q_i.
 * Each query row's A row, O_i and D_i are evaluated on their own, so the
 * cost is one forward pass of the query heads involved.  dk_cols and
 * dv_cols are [n_cols, d]. */
int attn_bwd_cols_gqa_f64(const double *q, const double *k, const double *v,
                          const double *dout, int64_t B, int64_t H, int64_t Hkv,
                          int64_t N, int64_t d, double scale, int causal,
                          const int32_t *key_len, const uint8_t *block_mask,
                          int64_t blk, const int64_t *cols, int64_t n_cols,
                          double *dk_cols, double *dv_cols)
{
    int rc = check_args(q, k, v, B, H, Hkv, N, d, block_mask, blk);
    if (rc) return rc;
    if (!dout || (n_cols > 0 && (!cols || !dk_cols || !dv_cols))) return 1;
    for (int64_t r = 0; r < n_cols; ++r)
        if (cols[r] < 0 || cols[r] >= B * Hkv * N) return 2;
    for (int64_t x = 0; x < n_cols * d; ++x) dk_cols[x] = dv_cols[x] = 0.0;
    if (n_cols == 0) return 0;
    const int64_t nkb = block_mask ? (N + blk - 1) / blk : 0, G = H / Hkv;
    int failed = 0;
    for (int64_t x = 0; x < B * Hkv; ++x) {
        int64_t any = 0;
        for (int64_t r = 0; r < n_cols; ++r) any |= cols[r] / N == x;
        if (!any) continue;
        const int64_t b = x / Hkv, g = x % Hkv;
        const double *kh = k + x * N * d, *vh = v + x * N * d;
        for (int64_t h = g * G; h < (g + 1) * G; ++h) {
            const int64_t head = (b * H + h) * N;
            const double *qh = q + head * d, *doh = dout + head * d;
#pragma omp parallel
            {
                double *s = (double *)malloc((size_t)N * sizeof(double));
                double *o = (double *)malloc((size_t)d * sizeof(double));
                double *acc = (double *)calloc((size_t)(2 * n_cols * d), sizeof(double));
                if (!s || !o || !acc) {
#pragma omp atomic write
                    failed = 1;
                }
#pragma omp for schedule(dynamic, 16)
                for (int64_t i = 0; i < N; ++i) {
                    if (!s || !o || !acc) continue;
                    double lse_unused;
                    score_row(s, qh + i * d, kh, i, b, N, d, scale, causal, key_len,
                              block_mask, blk, nkb);
                    softmax_row_times_v(s, vh, o, &lse_unused, N, d);
                    const double *doi = doh + i * d, *qi = qh + i * d;
                    double Di = 0.0;
                    for (int64_t c = 0; c < d; ++c) Di += doi[c] * o[c];
                    for (int64_t r = 0; r < n_cols; ++r) {
                        if (cols[r] / N != x) continue;
                        const int64_t j = cols[r] % N;
                        const double a = s[j];
                        if (a == 0.0) continue;
                        double da = 0.0;
                        for (int64_t c = 0; c < d; ++c) da += doi[c] * vh[j * d + c];
                        const double ds = a * (da - Di);
                        double *ak = acc + r * d, *av = acc + (n_cols + r) * d;
                        for (int64_t c = 0; c < d; ++c) {
                            av[c] += a * doi[c];
                            ak[c] += scale * ds * qi[c];
                        }
                    }
                }
                if (acc) {
#pragma omp critical
                    for (int64_t y = 0; y < n_cols * d; ++y) {
                        dk_cols[y] += acc[y];
                        dv_cols[y] += acc[n_cols * d + y];
                    }
                }
                free(s);
                free(o);
                free(acc);
            }
        }
    }
    return failed ? 3 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int attn_ref_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
