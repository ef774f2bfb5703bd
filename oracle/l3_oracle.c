/*
 * Reference oracle for the Large Lookup Layer (L^3) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 definition of
 * what the layer computes, used to check the GPU library.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the
 * GPU library never links, calls or includes anything from here, and this
 * file includes nothing from the GPU library.
 *
 * Source: "L^3: Large Lookup Layers" (Tseng & De Sa, ICML 2026), as summarised
 * on the papernotes.org page (section "整体框架", the layer equation), the
 * sciencestack.ai page (Fig. 2 caption), the gist.science pages (section
 * "Architecture Centrale" / "Architettura Core") and the kimjy99.github.io
 * page (section "Method", the layer equation and its dimension statement).
 *
 * For one token with hidden state x (d_in) and token ID t:
 *     K_t = rows [off[t], off[t+1]) of W_K      (d_t x d_in)
 *     V_t = the same rows of W_V                (d_t x d_emb)
 *     p   = softmax(K_t x)                      (d_t scores, softmax over them)
 *     o   = V_t^T p                             (d_emb)
 *     h   = W_up o                              (d_up;  W_up is d_up x d_emb)
 *     y   = LayerNorm(h) = (h - mean) / sqrt(var + eps) * gamma + beta
 *     out = W_mix [y ; x]                       (d_out; W_mix is d_out x (d_up+d_in))
 * Readings taken where the pages are silent or garbled (each documented with
 * the library): W_up is d_up x d_emb (the printed d_out x (d_up+d_emb) cannot
 * multiply a d_emb vector); the first d_up columns of W_mix act on y and the
 * last d_in on x (the stacked vector's order); no biases; no softmax
 * temperature; LayerNorm over the d_up features of one token with the biased
 * variance, learned gamma/beta and eps given by the caller; token IDs are
 * 0-based; the tables are the per-token slices concatenated in token-ID order.
 *
 * Every token is computed on its own (the layer mixes channels only, no
 * information crosses tokens), so the loop over tokens may run in any order;
 * OpenMP only splits that loop.  All arithmetic is double precision.
 *
 * l3o_backward is the gradient of the same function: the chain rule applied to
 * the steps above in reverse order, one token at a time, the parameter
 * gradients summed over the tokens.  The pages train the layer end to end
 * (papernotes.org page, section 训练策略; kimjy99.github.io page, section
 * "2. Efficient Training and Inference": sort, block-diagonal attention,
 * inverse sort), but print no gradient formulas; these are the plain
 * derivatives of the forward equations.  On request it also returns, per table
 * row, the size of the products that row's gradient is formed from (kmag, vmag):
 * the scale of the rounding error a finite-precision gradient carries in that
 * row, however much the products cancel.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define L3O_OK 0
#define L3O_BAD_OFFSETS (-2)
#define L3O_TOKEN_RANGE (-3)
#define L3O_NOMEM (-6)

/* Checks the allocation: off[0] = 0, 1 <= d_t <= k for every token, off[vocab] = v
 * (every token owns at least one and at most k embeddings; the budget is
 * v = sum_t d_t). */
int l3o_check_offsets(const int64_t *off, int64_t vocab, int64_t v, int32_t k)
{
    if (off[0] != 0) return L3O_BAD_OFFSETS;
    for (int64_t t = 0; t < vocab; ++t) {
        int64_t d = off[t + 1] - off[t];
        if (d < 1 || d > k) return L3O_BAD_OFFSETS;
    }
    if (off[vocab] != v) return L3O_BAD_OFFSETS;
    return L3O_OK;
}

/* One token of the layer.  `s` holds max_d doubles, `o` d_emb, `h` and `y` d_up. */
static void l3o_token(const double *x, int64_t t, const int64_t *off,
                      int64_t d_in, int64_t d_emb, int64_t d_up, int64_t d_out,
                      const double *WK, const double *WV, const double *Wup,
                      const double *gamma, const double *beta, double eps,
                      const double *Wmix, double *out,
                      double *s, double *o, double *h, double *y)
{
    const int64_t a = off[t];
    const int64_t d = off[t + 1] - off[t];

    /* scores: s_j = <K_t[j], x> */
    for (int64_t j = 0; j < d; ++j) {
        const double *kr = WK + (a + j) * d_in;
        double acc = 0.0;
        for (int64_t c = 0; c < d_in; ++c) acc += kr[c] * x[c];
        s[j] = acc;
    }
    /* softmax over the d_t scores (the max is subtracted before exp; this
     * leaves the value unchanged and keeps exp finite) */
    double mx = s[0];
    for (int64_t j = 1; j < d; ++j) if (s[j] > mx) mx = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < d; ++j) { s[j] = exp(s[j] - mx); z += s[j]; }
    for (int64_t j = 0; j < d; ++j) s[j] /= z;
    /* o = V_t^T p */
    for (int64_t c = 0; c < d_emb; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < d; ++j) {
        const double *vr = WV + (a + j) * d_emb;
        for (int64_t c = 0; c < d_emb; ++c) o[c] += s[j] * vr[c];
    }
    /* h = W_up o */
    for (int64_t r = 0; r < d_up; ++r) {
        const double *wr = Wup + r * d_emb;
        double acc = 0.0;
        for (int64_t c = 0; c < d_emb; ++c) acc += wr[c] * o[c];
        h[r] = acc;
    }
    /* y = LayerNorm(h) */
    double mean = 0.0;
    for (int64_t r = 0; r < d_up; ++r) mean += h[r];
    mean /= (double)d_up;
    double var = 0.0;
    for (int64_t r = 0; r < d_up; ++r) var += (h[r] - mean) * (h[r] - mean);
    var /= (double)d_up;
    const double inv = 1.0 / sqrt(var + eps);
    for (int64_t r = 0; r < d_up; ++r) y[r] = (h[r] - mean) * inv * gamma[r] + beta[r];
    /* out = W_mix [y ; x] */
    for (int64_t q = 0; q < d_out; ++q) {
        const double *wr = Wmix + q * (d_up + d_in);
        double acc = 0.0;
        for (int64_t r = 0; r < d_up; ++r) acc += wr[r] * y[r];
        for (int64_t c = 0; c < d_in; ++c) acc += wr[d_up + c] * x[c];
        out[q] = acc;
    }
}

/*
 * Forward over n tokens.  All matrices are row-major:
 *   x [n x d_in], WK [v x d_in], WV [v x d_emb], Wup [d_up x d_emb],
 *   gamma, beta [d_up], Wmix [d_out x (d_up + d_in)], out [n x d_out].
 * o_out [n x d_emb], h_out [n x d_up], y_out [n x d_up] receive the
 * intermediate stages when not NULL.  nthreads <= 0 uses the OpenMP default.
 * Returns 0, L3O_BAD_OFFSETS or L3O_TOKEN_RANGE (nothing is written then).
 */
int l3o_forward(int64_t n, int64_t vocab, int64_t v, int32_t k, const int64_t *off,
                int64_t d_in, int64_t d_emb, int64_t d_up, int64_t d_out,
                const double *x, const int32_t *ids,
                const double *WK, const double *WV, const double *Wup,
                const double *gamma, const double *beta, double eps,
                const double *Wmix, double *out,
                double *o_out, double *h_out, double *y_out, int nthreads)
{
    int rc = l3o_check_offsets(off, vocab, v, k);
    if (rc) return rc;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= vocab) return L3O_TOKEN_RANGE;
    int nt = 1;
#ifdef _OPENMP
    nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    /* per-thread scratch: scores (k), o (d_emb), h (d_up), y (d_up) */
    const int64_t per = (int64_t)k + d_emb + 2 * d_up;
    double *scratch = (double *)malloc(sizeof(double) * (size_t)(per * nt));
    if (!scratch) return L3O_NOMEM;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *s = scratch + per * tid;
        double *o = s + k;
        double *h = o + d_emb;
        double *y = h + d_up;
        l3o_token(x + i * d_in, ids[i], off, d_in, d_emb, d_up, d_out,
                  WK, WV, Wup, gamma, beta, eps, Wmix, out + i * d_out, s, o, h, y);
        if (o_out) for (int64_t c = 0; c < d_emb; ++c) o_out[i * d_emb + c] = o[c];
        if (h_out) for (int64_t r = 0; r < d_up; ++r) h_out[i * d_up + r] = h[r];
        if (y_out) for (int64_t r = 0; r < d_up; ++r) y_out[i * d_up + r] = y[r];
    }
    free(scratch);
    return L3O_OK;
}

/*
 * Backward over n tokens for the upstream gradient dout [n x d_out]: writes
 * (overwrites) dx [n x d_in], dWK [v x d_in], dWV [v x d_emb], dWup [d_up x d_emb],
 * dgamma, dbeta [d_up] and dWmix [d_out x (d_up + d_in)].  Single-threaded (the
 * parameter gradients are sums over tokens).  Per token, with W_mix = [W1 | W2],
 * yhat = (h - mean) / sqrt(var + eps) and y = yhat * gamma + beta:
 *     dWmix += dout [y ; x]^T          dy = W1^T dout      dx = W2^T dout
 *     dgamma += dy * yhat              dbeta += dy
 *     g = dy * gamma;  dh = rstd * (g - mean(g) - yhat * mean(g * yhat))
 *     dWup += dh o^T                   do = Wup^T dh
 *     dV_t[j] += p_j do                dp_j = <V_t[j], do>
 *     ds_j = p_j (dp_j - sum_k p_k dp_k)
 *     dK_t[j] += ds_j x                dx += sum_j ds_j K_t[j]
 */
int l3o_backward(int64_t n, int64_t vocab, int64_t v, int32_t k, const int64_t *off,
                 int64_t d_in, int64_t d_emb, int64_t d_up, int64_t d_out,
                 const double *x, const int32_t *ids,
                 const double *WK, const double *WV, const double *Wup,
                 const double *gamma, const double *beta, double eps,
                 const double *Wmix, const double *dout,
                 double *dx, double *dWK, double *dWV, double *dWup,
                 double *dgamma, double *dbeta, double *dWmix,
                 double *kmag, double *vmag)
{
    int rc = l3o_check_offsets(off, vocab, v, k);
    if (rc) return rc;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= vocab) return L3O_TOKEN_RANGE;
    const int64_t dz = d_up + d_in;
    for (int64_t e = 0; e < v * d_in; ++e) dWK[e] = 0.0;
    for (int64_t e = 0; e < v * d_emb; ++e) dWV[e] = 0.0;
    for (int64_t e = 0; e < d_up * d_emb; ++e) dWup[e] = 0.0;
    for (int64_t e = 0; e < d_up; ++e) dgamma[e] = dbeta[e] = 0.0;
    for (int64_t e = 0; e < d_out * dz; ++e) dWmix[e] = 0.0;
    if (kmag) for (int64_t e = 0; e < v; ++e) kmag[e] = 0.0;
    if (vmag) for (int64_t e = 0; e < v; ++e) vmag[e] = 0.0;
    /* scratch: p (k), dp (k), o (d_emb), do (d_emb), h, yhat, y, dy, dh (d_up), out (d_out) */
    double *p = (double *)malloc(sizeof(double) * (size_t)(2 * k + 2 * d_emb + 5 * d_up + d_out));
    if (!p) return L3O_NOMEM;
    double *dp = p + k, *o = dp + k, *dov = o + d_emb, *h = dov + d_emb;
    double *yh = h + d_up, *y = yh + d_up, *dy = y + d_up, *dh = dy + d_up, *tmp = dh + d_up;
    for (int64_t i = 0; i < n; ++i) {
        const double *xi = x + i * d_in, *go = dout + i * d_out;
        const int64_t t = ids[i], a = off[t], d = off[t + 1] - off[t];
        /* forward again: p, o, h, y (l3o_token; s doubles as p) */
        l3o_token(xi, t, off, d_in, d_emb, d_up, d_out, WK, WV, Wup, gamma, beta, eps, Wmix,
                  tmp, p, o, h, y);
        /* the normalised h (before gamma, beta) and 1 / sqrt(var + eps) */
        double mu = 0.0, ss = 0.0;
        for (int64_t r = 0; r < d_up; ++r) mu += h[r];
        mu /= (double)d_up;
        for (int64_t r = 0; r < d_up; ++r) { const double c = h[r] - mu; ss += c * c; }
        const double rstd = 1.0 / sqrt(ss / (double)d_up + eps);
        for (int64_t r = 0; r < d_up; ++r) yh[r] = (h[r] - mu) * rstd;
        /* out = W_mix [y ; x] */
        for (int64_t q = 0; q < d_out; ++q) {
            double *gr = dWmix + q * dz;
            for (int64_t r = 0; r < d_up; ++r) gr[r] += go[q] * y[r];
            for (int64_t c = 0; c < d_in; ++c) gr[d_up + c] += go[q] * xi[c];
        }
        for (int64_t r = 0; r < d_up; ++r) {
            double acc = 0.0;
            for (int64_t q = 0; q < d_out; ++q) acc += Wmix[q * dz + r] * go[q];
            dy[r] = acc;
        }
        for (int64_t c = 0; c < d_in; ++c) {
            double acc = 0.0;
            for (int64_t q = 0; q < d_out; ++q) acc += Wmix[q * dz + d_up + c] * go[q];
            dx[i * d_in + c] = acc;
        }
        /* y = yhat * gamma + beta, yhat = (h - mean) * rstd */
        double mg = 0.0, mgy = 0.0;
        for (int64_t r = 0; r < d_up; ++r) {
            dgamma[r] += dy[r] * yh[r];
            dbeta[r] += dy[r];
            const double g = dy[r] * gamma[r];
            mg += g;
            mgy += g * yh[r];
        }
        mg /= (double)d_up;
        mgy /= (double)d_up;
        for (int64_t r = 0; r < d_up; ++r) dh[r] = rstd * (dy[r] * gamma[r] - mg - yh[r] * mgy);
        /* h = W_up o */
        for (int64_t r = 0; r < d_up; ++r)
            for (int64_t c = 0; c < d_emb; ++c) dWup[r * d_emb + c] += dh[r] * o[c];
        for (int64_t c = 0; c < d_emb; ++c) {
            double acc = 0.0;
            for (int64_t r = 0; r < d_up; ++r) acc += Wup[r * d_emb + c] * dh[r];
            dov[c] = acc;
        }
        /* o = V_t^T p */
        double pdp = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            const double *vrow = WV + (a + j) * d_emb;
            double *gv = dWV + (a + j) * d_emb;
            double acc = 0.0;
            for (int64_t c = 0; c < d_emb; ++c) {
                gv[c] += p[j] * dov[c];
                acc += vrow[c] * dov[c];
            }
            dp[j] = acc;
            pdp += p[j] * acc;
        }
        /* magnitudes of the products behind each row's gradient.  dS_j is the
         * difference of two inner products, <V_j, do> and <o, do>; key row j gets
         * p_j (||V_j * do||_2 + ||o * do||_2) max_c |x_c| per token (the root sum of
         * squares of those products: the scale a rounding error in them takes, however
         * much the two cancel), value row j gets p_j max_c |do_c|. */
        if (kmag || vmag) {
            double od = 0.0, dmax = 0.0, xmax = 0.0;
            for (int64_t c = 0; c < d_emb; ++c) {
                od += (o[c] * dov[c]) * (o[c] * dov[c]);
                if (fabs(dov[c]) > dmax) dmax = fabs(dov[c]);
            }
            od = sqrt(od);
            for (int64_t c = 0; c < d_in; ++c) if (fabs(xi[c]) > xmax) xmax = fabs(xi[c]);
            for (int64_t j = 0; j < d; ++j) {
                const double *vrow = WV + (a + j) * d_emb;
                double vd = 0.0;
                for (int64_t c = 0; c < d_emb; ++c) vd += (vrow[c] * dov[c]) * (vrow[c] * dov[c]);
                if (kmag) kmag[a + j] += p[j] * (sqrt(vd) + od) * xmax;
                if (vmag) vmag[a + j] += p[j] * dmax;
            }
        }
        /* p = softmax(s), s_j = <K_t[j], x> */
        for (int64_t j = 0; j < d; ++j) {
            const double ds = p[j] * (dp[j] - pdp);
            const double *kr = WK + (a + j) * d_in;
            double *gk = dWK + (a + j) * d_in;
            for (int64_t c = 0; c < d_in; ++c) {
                gk[c] += ds * xi[c];
                dx[i * d_in + c] += ds * kr[c];
            }
        }
    }
    free(p);
    return L3O_OK;
}
