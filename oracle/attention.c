/*
 * oracle/attention.c -- TEST INFRASTRUCTURE ONLY. Plain, slow, fp64 CPU reference for exact
 * attention. Only the tests, the smoke check and the benchmark's CPU-baseline leg may load it;
 * the product path never does. It shares no code, header or constant with the HIP library.
 *
 * What it computes (the plain, materialised definition of attention, written out):
 *   s_ij = scale * sum_c q_ic * k_jc            for every key j the mask allows, else -inf
 *   m_i  = max_j s_ij
 *   O_i  = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i)
 *   LSE_i = m_i + ln(sum_j exp(s_ij - m_i))     (natural log)
 * Source: "ops-transformer" article on gitcode.csdn.net, section 二.1 "FlashAttention算子",
 * the listing of conventional attention (scores = Q K^T / sqrt(d_k), softmax over keys, then
 * the product with V). The tiled method on the same pages reaches this same result (it only
 * avoids storing the N x N score matrix), so the oracle is this definition and not the
 * tiled recurrence. The running-max subtraction is the numerically stable form of the same
 * softmax (zwxr.cn article, section 6.1, "softmax_stable" remedy for score overflow).
 *
 * Readings where the pages are silent or ambiguous (each one is also listed in the design
 * notes of the repository):
 *   - layout [B, H, N, d], contiguous; LSE [B, H, Nq];
 *   - causal keeps the diagonal (j <= i), aligned bottom-right when Nq != Nkv:
 *     query row i sits at absolute position i' = i + (Nkv - Nq);
 *   - sliding window + global keys ("ascend-transformer-boost" article, 场景三, sparse_config
 *     with window_size and global_tokens): causal window of W keys including the query's own
 *     position (i' - j < W) plus the first G key positions, still causal;
 *   - band attention (ops-transformer article on zwxr.cn, section 3.2, 带状注意力: each token
 *     attends the positions within +-w of it): |i' - j| <= w, on both sides of the query;
 *   - prefix LM ("ascend-transformer-boost" article, 场景三, names the variant only): keys
 *     j < P (the prefix) are visible to every query, later keys causally (j <= i');
 *   - block sparse (same article, names the variant only): a per-head layout of
 *     block x block tiles over (query index, key index); a key is visible when its tile is
 *     set; no shift between query and key positions;
 *   - a row with no visible key gives O = 0 and LSE = -inf.
 *
 * Inputs are float32 arrays that hold exactly the values the device sees (fp16 and bf16
 * values are exactly representable in float32); every product, sum and exponential is done
 * in double precision. No -ffast-math, no contraction into FMA (see oracle/build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Mask predicate: is key position j visible from a query at absolute position ip?
 * mode 0: all keys; mode 1: causal (j <= ip); mode 2: causal window of `window` keys
 * ending at ip, plus the first `n_global` positions (still causal); mode 3: band of
 * `window` positions on either side of ip; mode 4: prefix LM with a prefix of `n_global`
 * keys. */
static int key_visible(long ip, long j, int mode, long window, long n_global)
{
    if (mode == 0)
        return 1;
    if (mode == 1)
        return j <= ip;
    if (mode == 2)
        return j <= ip && ((ip - j) < window || j < n_global);
    if (mode == 3)
        return j >= ip - window && j <= ip + window;
    if (mode == 4) {
        const long prefix = n_global;
        return j < prefix || j - ip <= 0;
    }
    return 0;
}

/* One query row against `nkv` key/value rows given by pointers. `s` is scratch of nkv
 * doubles. Writes d outputs and the row's LSE. */
/* kvis: per-key visibility of this row (block sparse), or NULL to use the mask mode. */
static void attend_row(const float *q, const float *const *krow, const float *const *vrow,
                       long nkv, int d, double scale, long ip, int mode, long window,
                       long n_global, const unsigned char *kvis, double *s, double *out,
                       double *lse)
{
    double m = -INFINITY;
    long j;
    int c;

    for (j = 0; j < nkv; ++j) {
        double dot = 0.0;
        if (kvis ? !kvis[j] : !key_visible(ip, j, mode, window, n_global)) {
            s[j] = -INFINITY;
            continue;
        }
        for (c = 0; c < d; ++c)
            dot += (double)q[c] * (double)krow[j][c];
        s[j] = scale * dot;
        if (s[j] > m)
            m = s[j];
    }

    for (c = 0; c < d; ++c)
        out[c] = 0.0;
    if (m == -INFINITY) {
        *lse = -INFINITY;
        return;
    }

    {
        double l = 0.0;
        for (j = 0; j < nkv; ++j) {
            double e;
            if (s[j] == -INFINITY)
                continue;
            e = exp(s[j] - m);
            l += e;
            for (c = 0; c < d; ++c)
                out[c] += e * (double)vrow[j][c];
        }
        for (c = 0; c < d; ++c)
            out[c] /= l;
        *lse = m + log(l);
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Attention over contiguous [B,H,N,d] tensors for a list of query rows.
 * rows: flat indices ((b*H + h)*Nq + i); if NULL, every row in order.
 * o: nrows x d doubles; lse: nrows doubles. Returns 0, or -1 on bad arguments / no memory.
 */
int oracle_attention_rows(const float *q, const float *k, const float *v, int B, int H,
                          long Nq, long Nkv, int d, double scale, int mode, long window,
                          long n_global, const int64_t *rows, long nrows, double *o,
                          double *lse)
{
    int failed = 0;
    if (B < 1 || H < 1 || Nq < 1 || Nkv < 1 || d < 1 || mode < 0 || mode > 4)
        return -1;
    if (rows == NULL)
        nrows = (long)B * H * Nq;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nkv);
        const float **kp = (const float **)malloc(sizeof(float *) * (size_t)Nkv);
        const float **vp = (const float **)malloc(sizeof(float *) * (size_t)Nkv);
        long r;
        if (s == NULL || kp == NULL || vp == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (r = 0; r < nrows; ++r) {
                int64_t flat = rows ? rows[r] : (int64_t)r;
                long i = (long)(flat % Nq);
                long bh = (long)(flat / Nq);
                const float *kb = k + (size_t)bh * Nkv * d;
                const float *vb = v + (size_t)bh * Nkv * d;
                long j;
                for (j = 0; j < Nkv; ++j) {
                    kp[j] = kb + (size_t)j * d;
                    vp[j] = vb + (size_t)j * d;
                }
                attend_row(q + (size_t)flat * d, kp, vp, Nkv, d, scale, i + (Nkv - Nq), mode,
                           window, n_global, NULL, s, o + (size_t)r * d, lse + r);
            }
        }
        free(s);
        free((void *)kp);
        free((void *)vp);
    }
    return failed ? -1 : 0;
}

/*
 * Block-sparse attention over contiguous [B,H,N,d] tensors for a list of query rows.
 * layout: [H][ceil(Nq/block)][ceil(Nkv/block)] bytes, nonzero = the tile of query block
 * i/block and key block j/block is visible (the same layout for every batch entry).
 * rows, o, lse as in oracle_attention_rows.
 */
int oracle_attention_block_sparse_rows(const float *q, const float *k, const float *v, int B,
                                       int H, long Nq, long Nkv, int d, double scale,
                                       const uint8_t *layout, long block, const int64_t *rows,
                                       long nrows, double *o, double *lse)
{
    int failed = 0;
    long nqb, nkb;
    if (B < 1 || H < 1 || Nq < 1 || Nkv < 1 || d < 1 || block < 1 || layout == NULL)
        return -1;
    nqb = (Nq + block - 1) / block;
    nkb = (Nkv + block - 1) / block;
    if (rows == NULL)
        nrows = (long)B * H * Nq;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nkv);
        unsigned char *vis = (unsigned char *)malloc((size_t)Nkv);
        const float **kp = (const float **)malloc(sizeof(float *) * (size_t)Nkv);
        const float **vp = (const float **)malloc(sizeof(float *) * (size_t)Nkv);
        long r;
        if (s == NULL || vis == NULL || kp == NULL || vp == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (r = 0; r < nrows; ++r) {
                int64_t flat = rows ? rows[r] : (int64_t)r;
                long i = (long)(flat % Nq);
                long bh = (long)(flat / Nq);
                long h = bh % H;
                const uint8_t *lrow = layout + ((size_t)h * nqb + (size_t)(i / block)) * nkb;
                const float *kb = k + (size_t)bh * Nkv * d;
                const float *vb = v + (size_t)bh * Nkv * d;
                long j;
                for (j = 0; j < Nkv; ++j) {
                    kp[j] = kb + (size_t)j * d;
                    vp[j] = vb + (size_t)j * d;
                    vis[j] = lrow[j / block] != 0;
                }
                attend_row(q + (size_t)flat * d, kp, vp, Nkv, d, scale, i, 0, 0, 0, vis, s,
                           o + (size_t)r * d, lse + r);
            }
        }
        free(s);
        free(vis);
        free((void *)kp);
        free((void *)vp);
    }
    return failed ? -1 : 0;
}

/*
 * Gradients of exact attention with respect to Q, K and V for an upstream gradient dO, in
 * fp64, from the plain definition (the pages stress that the score matrix is recomputed,
 * not stored, for the backward pass: ops-transformer article on zwxr.cn, section 2.2,
 * gradient checkpointing; here the oracle simply materialises each row again):
 *   P_ij  = exp(s_ij - m_i) / l_i                 (0 for hidden keys)
 *   D_i   = sum_c dO_ic O_ic                       (O from the same P)
 *   dP_ij = sum_c dO_ic v_jc
 *   dS_ij = P_ij (dP_ij - D_i)                     (softmax Jacobian)
 *   dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i
 * Masks as oracle_attention_rows, or (layout != NULL) the block layout of
 * oracle_attention_block_sparse_rows. All outputs [B,H,N,d] doubles. Parallel over (b, h).
 */
static int attention_backward(const float *q, const float *k, const float *v,
                              const float *dout, int B, int H, long Nq, long Nkv, int d,
                              double scale, int mode, long window, long n_global,
                              const uint8_t *layout, long block, double *dq, double *dk,
                              double *dv)
{
    int failed = 0;
    long bh;
    const long nqb = layout ? (Nq + block - 1) / block : 0;
    const long nkb = layout ? (Nkv + block - 1) / block : 0;
    memset(dk, 0, sizeof(double) * (size_t)B * H * Nkv * d);
    memset(dv, 0, sizeof(double) * (size_t)B * H * Nkv * d);

#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)Nkv);
        double *orow = (double *)malloc(sizeof(double) * (size_t)d);
        if (p == NULL || orow == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (bh = 0; bh < (long)B * H; ++bh) {
                const float *qb = q + (size_t)bh * Nq * d, *kb = k + (size_t)bh * Nkv * d;
                const float *vb = v + (size_t)bh * Nkv * d, *gb = dout + (size_t)bh * Nq * d;
                double *dqb = dq + (size_t)bh * Nq * d, *dkb = dk + (size_t)bh * Nkv * d;
                double *dvb = dv + (size_t)bh * Nkv * d;
                long i, j;
                int c;
                for (i = 0; i < Nq; ++i) {
                    const float *qi = qb + (size_t)i * d, *gi = gb + (size_t)i * d;
                    const long ip = i + (Nkv - Nq);
                    double m = -INFINITY, l = 0.0, D = 0.0;
                    const uint8_t *lrow =
                        layout ? layout + ((size_t)(bh % H) * nqb + (size_t)i / (size_t)block) * nkb
                               : NULL;
                    for (j = 0; j < Nkv; ++j) {
                        double dot = 0.0;
                        if (lrow ? lrow[j / block] == 0
                                 : !key_visible(ip, j, mode, window, n_global)) {
                            p[j] = -INFINITY;
                            continue;
                        }
                        for (c = 0; c < d; ++c)
                            dot += (double)qi[c] * (double)kb[(size_t)j * d + c];
                        p[j] = scale * dot;
                        if (p[j] > m)
                            m = p[j];
                    }
                    for (c = 0; c < d; ++c)
                        orow[c] = 0.0;
                    for (c = 0; c < d; ++c)
                        dqb[(size_t)i * d + c] = 0.0;
                    if (m == -INFINITY)
                        continue; /* no visible key: every gradient term is zero */
                    for (j = 0; j < Nkv; ++j) {
                        p[j] = (p[j] == -INFINITY) ? 0.0 : exp(p[j] - m);
                        l += p[j];
                    }
                    for (j = 0; j < Nkv; ++j) {
                        p[j] /= l;
                        if (p[j] == 0.0)
                            continue;
                        for (c = 0; c < d; ++c)
                            orow[c] += p[j] * (double)vb[(size_t)j * d + c];
                    }
                    for (c = 0; c < d; ++c)
                        D += (double)gi[c] * orow[c];
                    for (j = 0; j < Nkv; ++j) {
                        double dp = 0.0, ds;
                        if (p[j] == 0.0)
                            continue;
                        for (c = 0; c < d; ++c)
                            dp += (double)gi[c] * (double)vb[(size_t)j * d + c];
                        ds = p[j] * (dp - D);
                        for (c = 0; c < d; ++c) {
                            dqb[(size_t)i * d + c] += scale * ds * (double)kb[(size_t)j * d + c];
                            dkb[(size_t)j * d + c] += scale * ds * (double)qi[c];
                            dvb[(size_t)j * d + c] += p[j] * (double)gi[c];
                        }
                    }
                }
            }
        }
        free(p);
        free(orow);
    }
    return failed ? -1 : 0;
}

int oracle_attention_backward(const float *q, const float *k, const float *v, const float *dout,
                              int B, int H, long Nq, long Nkv, int d, double scale, int mode,
                              long window, long n_global, double *dq, double *dk, double *dv)
{
    if (B < 1 || H < 1 || Nq < 1 || Nkv < 1 || d < 1 || mode < 0 || mode > 4)
        return -1;
    return attention_backward(q, k, v, dout, B, H, Nq, Nkv, d, scale, mode, window, n_global,
                              NULL, 0, dq, dk, dv);
}

/* Gradients of block-sparse attention: layout [H, ceil(Nq/block), ceil(Nkv/block)], key j
 * visible from query row i of head h when layout[h][i/block][j/block] != 0 (the reading of
 * oracle_attention_block_sparse_rows); the arithmetic is the backward above. */
int oracle_attention_backward_block_sparse(const float *q, const float *k, const float *v,
                                           const float *dout, int B, int H, long Nq, long Nkv,
                                           int d, double scale, const uint8_t *layout,
                                           long block, double *dq, double *dk, double *dv)
{
    if (B < 1 || H < 1 || Nq < 1 || Nkv < 1 || d < 1 || block < 1 || layout == NULL)
        return -1;
    return attention_backward(q, k, v, dout, B, H, Nq, Nkv, d, scale, 0, 0, 0, layout, block,
                              dq, dk, dv);
}

/*
 * Single-token decode against a paged K/V cache ("ascend-transformer-boost" article, 场景二:
 * the cache is cut into fixed pages of page_size tokens; a sequence's pages need not be
 * contiguous). Pages are [num_pages, page_size, H, d]; logical token j of sequence s lives
 * in physical page page_table[s*max_pages + j/page_size], slot j % page_size. The query is
 * the newest token, so it sees all L_s keys. q: [S,H,d]; o: [S,H,d]; lse: [S,H].
 * Returns 0, or -1 on bad arguments (including a page id outside [0, num_pages)).
 */
int oracle_decode_paged(const float *q, const float *k_pages, const float *v_pages,
                        const int32_t *page_table, const int32_t *seq_lens, int S, int H, int d,
                        int page_size, int max_pages, long num_pages, double scale, double *o,
                        double *lse)
{
    int failed = 0;
    long r;
    if (S < 1 || H < 1 || d < 1 || page_size < 1 || max_pages < 1 || num_pages < 1)
        return -1;
    for (r = 0; r < S; ++r) {
        long L = seq_lens[r], p;
        if (L < 1 || L > (long)max_pages * page_size)
            return -1;
        for (p = 0; p < (L + page_size - 1) / page_size; ++p) {
            int32_t id = page_table[r * max_pages + p];
            if (id < 0 || id >= num_pages)
                return -1;
        }
    }

#pragma omp parallel
    {
        long Lmax = (long)max_pages * page_size;
        double *s = (double *)malloc(sizeof(double) * (size_t)Lmax);
        const float **kp = (const float **)malloc(sizeof(float *) * (size_t)Lmax);
        const float **vp = (const float **)malloc(sizeof(float *) * (size_t)Lmax);
        long t;
        if (s == NULL || kp == NULL || vp == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (t = 0; t < (long)S * H; ++t) {
                long sq = t / H, h = t % H, L = seq_lens[sq], j;
                for (j = 0; j < L; ++j) {
                    long page = page_table[sq * max_pages + j / page_size];
                    size_t off = (((size_t)page * page_size + (size_t)(j % page_size)) * H + h) * d;
                    kp[j] = k_pages + off;
                    vp[j] = v_pages + off;
                }
                attend_row(q + (size_t)t * d, kp, vp, L, d, scale, L - 1, 1, 0, 0, NULL, s,
                           o + (size_t)t * d, lse + t);
            }
        }
        free(s);
        free((void *)kp);
        free((void *)vp);
    }
    return failed ? -1 : 0;
}

/*
 * Paged multi-token (chunked) prefill: sequence s appends a chunk of q_lens[s] new tokens to
 * a cache that then holds L_s = seq_lens[s] tokens (the chunk included), stored in pages as
 * for oracle_decode_paged (the paged KV cache of the "ascend-transformer-boost" article,
 * 场景二). The chunk's tokens are the newest ones, so query row i of sequence s sits at
 * absolute position i + (L_s - q_lens[s]) and sees keys by `mode` exactly as in
 * oracle_attention_rows (bottom-right alignment; mode 1 is causal). q: [S, Qmax, H, d];
 * o: [S, Qmax, H, d]; lse: [S, Qmax, H]; rows i >= q_lens[s] are not written.
 * Returns 0, or -1 on bad arguments (including a page id outside [0, num_pages) or a chunk
 * longer than its sequence).
 */
int oracle_prefill_paged(const float *q, const float *k_pages, const float *v_pages,
                         const int32_t *page_table, const int32_t *seq_lens,
                         const int32_t *q_lens, int S, int Qmax, int H, int d, int page_size,
                         int max_pages, long num_pages, double scale, int mode, long window,
                         long n_global, double *o, double *lse)
{
    int failed = 0;
    long r;
    if (S < 1 || Qmax < 1 || H < 1 || d < 1 || page_size < 1 || max_pages < 1 ||
        num_pages < 1 || mode < 0 || mode > 4)
        return -1;
    for (r = 0; r < S; ++r) {
        long L = seq_lens[r], nq = q_lens[r], p;
        if (L < 1 || L > (long)max_pages * page_size || nq < 0 || nq > Qmax || nq > L)
            return -1;
        for (p = 0; p < (L + page_size - 1) / page_size; ++p) {
            int32_t id = page_table[r * max_pages + p];
            if (id < 0 || id >= num_pages)
                return -1;
        }
    }

#pragma omp parallel
    {
        long Lmax = (long)max_pages * page_size;
        double *s = (double *)malloc(sizeof(double) * (size_t)Lmax);
        const float **kp = (const float **)malloc(sizeof(float *) * (size_t)Lmax);
        const float **vp = (const float **)malloc(sizeof(float *) * (size_t)Lmax);
        long t;
        if (s == NULL || kp == NULL || vp == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (t = 0; t < (long)S * H; ++t) {
                long sq = t / H, h = t % H, L = seq_lens[sq], nq = q_lens[sq], j, i;
                for (j = 0; j < L; ++j) {  /* logical token j: page j / page_size, slot */
                    long pg = j / page_size, slot = j - pg * page_size;
                    size_t tok = (size_t)page_table[sq * max_pages + pg] * (size_t)page_size +
                                 (size_t)slot;
                    kp[j] = k_pages + (tok * (size_t)H + (size_t)h) * (size_t)d;
                    vp[j] = v_pages + (tok * (size_t)H + (size_t)h) * (size_t)d;
                }
                for (i = 0; i < nq; ++i) {
                    size_t row = ((size_t)sq * Qmax + (size_t)i) * H + (size_t)h;
                    attend_row(q + row * d, kp, vp, L, d, scale, i + (L - nq), mode, window,
                               n_global, NULL, s, o + row * d, lse + row);
                }
            }
        }
        free(s);
        free((void *)kp);
        free((void *)vp);
    }
    return failed ? -1 : 0;
}

/*
 * Merge of two attention results over disjoint key sets A and B of the same query rows.
 * With the row statistic lse = ln sum exp(score) over each set, the union has
 *   lse = ln(exp(lse_a) + exp(lse_b)),  o = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b,
 * which is how the "ascend-transformer-boost" article (场景四) can run the text queries'
 * attention to text keys and to image keys as separate calls and still get the result of
 * one call over both. A set without keys has lse = -inf and weight 0; a row with no key in
 * either set stays o = 0, lse = -inf. Inputs are the values the device holds (float32
 * copies); o_a, o_b, o: rows x d; lse_*: rows.
 */
void oracle_merge_lse(const float *o_a, const float *lse_a, const float *o_b,
                      const float *lse_b, long rows, int d, double *o, double *lse)
{
    long r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        double la = lse_a[r], lb = lse_b[r], m = la > lb ? la : lb, wa, wb, t;
        int c;
        if (m == -INFINITY) {
            for (c = 0; c < d; ++c)
                o[(size_t)r * d + c] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        wa = exp(la - m);
        wb = exp(lb - m);
        t = wa + wb;
        for (c = 0; c < d; ++c)
            o[(size_t)r * d + c] = (wa * (double)o_a[(size_t)r * d + c] +
                                    wb * (double)o_b[(size_t)r * d + c]) / t;
        lse[r] = m + log(t);
    }
}
