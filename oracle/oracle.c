/*
 * ORACLE for SparseConv2D on pruned token sequences -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct CPU loops in double precision.  Nothing in
 * the product path may link, load or call this file: only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark use it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes, and where that is defined ("SV-TAD: Native Sparse
 * Convolutions for Efficient Temporal Action Detection", paper notes page):
 *
 *   orc_build_index   Key Design 1 ("Static Neighbor Index Table"), the two
 *                     steps and the piecewise equation for N[k, j], for a
 *                     K x K neighbourhood (the Background's "K x K spatial
 *                     neighbors"; the page's tables and kernels use K = 3).
 *   orc_fwd           Key Design 2 ("Native Sparse 2D Convolution Kernels"),
 *                     the equation y_k = sum_j W_j x[N[k, j]] with N = -1 read
 *                     as zero padding, plus a per-channel bias.
 *   orc_bwd_dx        Key Design 2 names dedicated backward kernels but prints
 *   orc_bwd_dx_scatter no backward formula.  These are the adjoint of the
 *   orc_bwd_dw        forward map, obtained by differentiating the forward sum
 *   orc_bwd_db        (scatter form, dW, db) and by the mirror property of the
 *                     3x3 offsets (gather form of dX).
 *   orc_xattn_fwd     Key Design 3 ("Asymmetric Cross-Attention"): auxiliary
 *   orc_xattn_bwd     tokens are the queries, the down-projected sparse
 *                     visual tokens are both keys and values, and only the
 *                     auxiliary tokens are updated.  The page prints
 *                     X'_aux = CrossAttn(X'_vis) and nothing more; the
 *                     reading here is single-head scaled dot-product
 *                     attention with no further projections, the scores
 *                     scaled by 1/sqrt(d) unless another scale is given.
 *                     The backward is the chain rule through scores, row
 *                     softmax and the weighted sum.
 *   orc_adapter_fwd   The bottleneck adapter (Overall Architecture: adapters
 *   orc_adapter_bwd   with sparse spatial convolutions run on the pruned
 *                     tokens; Key Design 3: the visual features inside are
 *                     down-projected).  No further internals are printed;
 *                     the reading is the plain residual bottleneck
 *                     H1 = X Wd + bd, H2 = conv_K(H1) + bc,
 *                     Y = X + H2 Wu + bu, no activation.  A projection is
 *                     the K x K layer above with one tap and N[k][0] = k.
 *                     The backward is the chain rule through the three
 *                     layers and the residual.
 *
 * Readings of points the page leaves open:
 *   - K odd; tap order j = K*(dy+r) + (dx+r) with r = K/2 and dy, dx in
 *     [-r, r] (for K = 3: j = 3*(dy+1) + (dx+1)); the centre tap j = K*K/2
 *     is part of the K*K-column table; the mirror of tap j is K*K-1-j;
 *   - one map M per frame (the convolution is spatial, within a frame), the
 *     table holds global indices into the packed sequence;
 *   - cross-correlation convention: tap j of token k reads the token at
 *     (y_k + dy_j, x_k + dx_j) and applies W[j] to it;
 *   - row form: W[j] is C_in x C_out and y_k = sum_j x[N[k,j]] W[j] + b;
 *   - stride 1, zero padding r, no dilation;
 *   - out-of-range or duplicate coordinates are errors, never "last writer".
 *
 * Layouts (row-major, contiguous): X [n][Ci], Y [n][Co], N [n][K*K],
 * W [K*K][Ci][Co], b [Co], dW [K*K][Ci][Co], db [Co].  Flat coordinate
 * p = y * W + x; frame t holds tokens frame_offsets[t] .. frame_offsets[t+1]-1.
 *
 * Every function sums each output in a fixed order (tap ascending, then
 * channel ascending, or token ascending for dW/db), so results are
 * deterministic whatever the thread count.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_OK = 0, ORC_BAD_ARGS = 1, ORC_COORD_RANGE = 5, ORC_DUPLICATE = 6 };

int orc_threads(int want)
{
#ifdef _OPENMP
    if (want > 0) omp_set_num_threads(want);
    return omp_get_max_threads();
#else
    (void)want;
    return 1;
#endif
}

/* Key Design 1, step 1 then step 2, frame by frame.
 * M (nullable) receives [T][H][W] global token indices, -1 where no token. */
int orc_build_index(const int32_t *coords, const int32_t *frame_offsets,
                    int32_t T, int32_t H, int32_t W, int64_t n, int32_t K,
                    int32_t *N, int32_t *M)
{
    if (T < 0 || H <= 0 || W <= 0 || n < 0 || K < 1 || K % 2 == 0) return ORC_BAD_ARGS;
    const int taps = K * K, r = K / 2;
    if (frame_offsets[0] != 0 || frame_offsets[T] != n) return ORC_BAD_ARGS;
    int64_t cells = (int64_t)H * W;
    int32_t *map = (int32_t *)malloc(sizeof(int32_t) * (size_t)cells);
    if (!map) return ORC_BAD_ARGS;
    int status = ORC_OK;
    for (int32_t t = 0; t < T && status == ORC_OK; ++t) {
        int64_t beg = frame_offsets[t], end = frame_offsets[t + 1];
        if (end < beg) { status = ORC_BAD_ARGS; break; }
        /* step 1: the lookup array starts at -1 and each kept token k
         * writes its own index at its grid cell. */
        for (int64_t c = 0; c < cells; ++c) map[c] = -1;
        for (int64_t k = beg; k < end; ++k) {
            int32_t p = coords[k];
            if (p < 0 || p >= cells) { status = ORC_COORD_RANGE; break; }
            if (map[p] != -1) { status = ORC_DUPLICATE; break; }
            map[p] = (int32_t)k;
        }
        if (status != ORC_OK) break;
        /* step 2: for each kept token, read the map at the K*K offsets; a
         * cell outside the H x W grid reads as -1. */
        for (int64_t k = beg; k < end; ++k) {
            int32_t y = coords[k] / W, x = coords[k] % W;
            for (int j = 0; j < taps; ++j) {
                int32_t yy = y + (j / K - r), xx = x + (j % K - r);
                int32_t v = -1;
                if (yy >= 0 && yy < H && xx >= 0 && xx < W) v = map[yy * W + xx];
                N[k * taps + j] = v;
            }
        }
        if (M) memcpy(M + (int64_t)t * cells, map, sizeof(int32_t) * (size_t)cells);
    }
    free(map);
    return status;
}

/* Key Design 2: Y[k][o] = sum_j sum_i X[N[k,j]][i] * W[j][i][o] + b[o];
 * a tap whose entry is -1 contributes nothing (zero padding). */
void orc_fwd(const double *X, const int32_t *N, const double *Wt,
             const double *b, double *Y, int64_t n, int32_t Ci, int32_t Co, int32_t taps)
{
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n; ++k) {
        double *acc = Y + k * Co;
        for (int32_t o = 0; o < Co; ++o) acc[o] = 0.0;
        for (int j = 0; j < taps; ++j) {
            int32_t m = N[k * taps + j];
            if (m < 0) continue;
            const double *x = X + (int64_t)m * Ci;
            const double *w = Wt + (int64_t)j * Ci * Co;
            for (int32_t i = 0; i < Ci; ++i) {
                double xv = x[i];
                const double *wr = w + (int64_t)i * Co;
                for (int32_t o = 0; o < Co; ++o) acc[o] += xv * wr[o];
            }
        }
        if (b)
            for (int32_t o = 0; o < Co; ++o) acc[o] += b[o];
    }
}

/* Forward restricted to a list of output tokens (for sampled checks at
 * full size): Yr[r] = Y[rows[r]]. */
void orc_fwd_rows(const double *X, const int32_t *N, const double *Wt,
                  const double *b, const int64_t *rows, int64_t nrows,
                  double *Yr, int32_t Ci, int32_t Co, int32_t taps)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t k = rows[r];
        double *acc = Yr + r * Co;
        for (int32_t o = 0; o < Co; ++o) acc[o] = 0.0;
        for (int j = 0; j < taps; ++j) {
            int32_t m = N[k * taps + j];
            if (m < 0) continue;
            const double *x = X + (int64_t)m * Ci;
            const double *w = Wt + (int64_t)j * Ci * Co;
            for (int32_t i = 0; i < Ci; ++i) {
                double xv = x[i];
                const double *wr = w + (int64_t)i * Co;
                for (int32_t o = 0; o < Co; ++o) acc[o] += xv * wr[o];
            }
        }
        if (b)
            for (int32_t o = 0; o < Co; ++o) acc[o] += b[o];
    }
}

/* Gather form of the input gradient.  The K x K offsets mirror: token m
 * sits at offset j of token k exactly when k sits at offset taps-1-j of m
 * (the offset negated).  So the contributions that token k received in the
 * forward map through tap j come back to it through tap taps-1-j:
 *   dX[k][i] = sum_j sum_o dY[N[k,taps-1-j]][o] * W[j][i][o]. */
static void dx_gather_one(const double *dY, const int32_t *N, const double *Wt,
                          int64_t k, double *out, int32_t Ci, int32_t Co, int32_t taps)
{
    for (int32_t i = 0; i < Ci; ++i) out[i] = 0.0;
    for (int j = 0; j < taps; ++j) {
        int32_t m = N[k * taps + (taps - 1 - j)];
        if (m < 0) continue;
        const double *g = dY + (int64_t)m * Co;
        const double *w = Wt + (int64_t)j * Ci * Co;
        for (int32_t i = 0; i < Ci; ++i) {
            const double *wr = w + (int64_t)i * Co;
            double s = 0.0;
            for (int32_t o = 0; o < Co; ++o) s += g[o] * wr[o];
            out[i] += s;
        }
    }
}

void orc_bwd_dx(const double *dY, const int32_t *N, const double *Wt,
                double *dX, int64_t n, int32_t Ci, int32_t Co, int32_t taps)
{
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n; ++k) dx_gather_one(dY, N, Wt, k, dX + k * Ci, Ci, Co, taps);
}

void orc_bwd_dx_rows(const double *dY, const int32_t *N, const double *Wt,
                     const int64_t *rows, int64_t nrows, double *dXr,
                     int32_t Ci, int32_t Co, int32_t taps)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) dx_gather_one(dY, N, Wt, rows[r], dXr + r * Ci, Ci, Co, taps);
}

/* Scatter form: the literal adjoint of the forward sum.  Every forward term
 * Y[k] += X[m] W[j] (m = N[k,j]) sends dY[k] W[j]^T back to row m.
 * Parallel over input channels so that no two threads write one element. */
void orc_bwd_dx_scatter(const double *dY, const int32_t *N, const double *Wt,
                        double *dX, int64_t n, int32_t Ci, int32_t Co, int32_t taps)
{
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < Ci; ++i) {
        for (int64_t m = 0; m < n; ++m) dX[m * Ci + i] = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            const double *g = dY + k * Co;
            for (int j = 0; j < taps; ++j) {
                int32_t m = N[k * taps + j];
                if (m < 0) continue;
                const double *wr = Wt + ((int64_t)j * Ci + i) * Co;
                double s = 0.0;
                for (int32_t o = 0; o < Co; ++o) s += g[o] * wr[o];
                dX[(int64_t)m * Ci + i] += s;
            }
        }
    }
}

/* dW[j][i][o] = sum_k [N[k,j] >= 0] X[N[k,j]][i] * dY[k][o], k ascending. */
void orc_bwd_dw(const double *X, const int32_t *N, const double *dY,
                double *dW, int64_t n, int32_t Ci, int32_t Co, int32_t taps)
{
#pragma omp parallel for schedule(static)
    for (int64_t ji = 0; ji < (int64_t)taps * Ci; ++ji) {
        int j = (int)(ji / Ci);
        int32_t i = (int32_t)(ji % Ci);
        double *acc = dW + ji * Co;
        for (int32_t o = 0; o < Co; ++o) acc[o] = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            int32_t m = N[k * taps + j];
            if (m < 0) continue;
            double xv = X[(int64_t)m * Ci + i];
            const double *g = dY + k * Co;
            for (int32_t o = 0; o < Co; ++o) acc[o] += xv * g[o];
        }
    }
}

/* A chosen set of dW rows (j, i), each over all tokens: out[r][o] =
 * dW[j][i][o] with ji = rows[r] = j * Ci + i. */
void orc_bwd_dw_rows(const double *X, const int32_t *N, const double *dY,
                     const int64_t *rows, int64_t nrows, double *out,
                     int64_t n, int32_t Ci, int32_t Co, int32_t taps)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        int j = (int)(rows[r] / Ci);
        int32_t i = (int32_t)(rows[r] % Ci);
        double *acc = out + r * Co;
        for (int32_t o = 0; o < Co; ++o) acc[o] = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            int32_t m = N[k * taps + j];
            if (m < 0) continue;
            double xv = X[(int64_t)m * Ci + i];
            const double *g = dY + k * Co;
            for (int32_t o = 0; o < Co; ++o) acc[o] += xv * g[o];
        }
    }
}

/* db[o] = sum_k dY[k][o]: the bias enters every output row once. */
void orc_bwd_db(const double *dY, double *db, int64_t n, int32_t Co)
{
    for (int32_t o = 0; o < Co; ++o) db[o] = 0.0;
    for (int64_t k = 0; k < n; ++k)
        for (int32_t o = 0; o < Co; ++o) db[o] += dY[k * Co + o];
}

/* ------------------------------------------------------------------------
 * Asymmetric cross-attention (Key Design 3).  Q [m][d] auxiliary queries,
 * X [n][d] sparse visual tokens used as keys and as values:
 *   S[q][j] = scale * sum_c Q[q][c] X[j][c]
 *   P[q][j] = exp(S[q][j] - lse[q]),  lse[q] = log sum_j exp(S[q][j])
 *   O[q][c] = sum_j P[q][j] X[j][c]
 * The largest score is subtracted before exponentiating (the same value in
 * exact arithmetic).  With n == 0 there is nothing to attend to: O = 0 and
 * lse = -infinity.  Keys are visited in ascending order. */
void orc_xattn_fwd(const double *Q, const double *X, double *O, double *lse,
                   int64_t m, int64_t n, int32_t d, double scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < m; ++q) {
        const double *qv = Q + q * d;
        double *o = O + q * d;
        for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
        if (n == 0) { lse[q] = -1.0 / 0.0; continue; }
        double *srow = (double *)malloc((size_t)n * sizeof(double));
        double mx = -1.0 / 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int32_t c = 0; c < d; ++c) s += qv[c] * X[j * d + c];
            srow[j] = scale * s;
            if (srow[j] > mx) mx = srow[j];
        }
        double sum = 0.0;
        for (int64_t j = 0; j < n; ++j) sum += exp(srow[j] - mx);
        for (int64_t j = 0; j < n; ++j) {
            double pj = exp(srow[j] - mx) / sum;
            for (int32_t c = 0; c < d; ++c) o[c] += pj * X[j * d + c];
        }
        lse[q] = mx + log(sum);
        free(srow);
    }
}

/* Backward of orc_xattn_fwd for an upstream gradient dO [m][d]:
 *   dP[q][j] = sum_c dO[q][c] X[j][c]
 *   D[q]     = sum_j P[q][j] dP[q][j]         (= sum_c dO[q][c] O[q][c])
 *   dS[q][j] = P[q][j] (dP[q][j] - D[q])       (row softmax)
 *   dQ[q][c] = scale * sum_j dS[q][j] X[j][c]
 *   dX[j][c] = scale * sum_q dS[q][j] Q[q][c]  (X as keys)
 *            +         sum_q P[q][j] dO[q][c]  (X as values)
 * P is recomputed from Q and X here, not taken from the forward. */
void orc_xattn_bwd(const double *Q, const double *X, const double *dO,
                   double *dQ, double *dX, int64_t m, int64_t n, int32_t d,
                   double scale)
{
    double *P = (double *)malloc((size_t)(m * n + 1) * sizeof(double));
    double *dS = (double *)malloc((size_t)(m * n + 1) * sizeof(double));
    for (int64_t q = 0; q < m; ++q) {
        const double *qv = Q + q * d, *g = dO + q * d;
        double mx = -1.0 / 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int32_t c = 0; c < d; ++c) s += qv[c] * X[j * d + c];
            P[q * n + j] = scale * s;
            if (P[q * n + j] > mx) mx = P[q * n + j];
        }
        double sum = 0.0;
        for (int64_t j = 0; j < n; ++j) sum += exp(P[q * n + j] - mx);
        for (int64_t j = 0; j < n; ++j) P[q * n + j] = exp(P[q * n + j] - mx) / sum;
        double D = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double dp = 0.0;
            for (int32_t c = 0; c < d; ++c) dp += g[c] * X[j * d + c];
            dS[q * n + j] = dp;              /* dP for now */
            D += P[q * n + j] * dp;
        }
        for (int64_t j = 0; j < n; ++j) dS[q * n + j] = P[q * n + j] * (dS[q * n + j] - D);
        for (int32_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; ++j) acc += dS[q * n + j] * X[j * d + c];
            dQ[q * d + c] = scale * acc;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        for (int32_t c = 0; c < d; ++c) {
            double key = 0.0, val = 0.0;
            for (int64_t q = 0; q < m; ++q) {
                key += dS[q * n + j] * Q[q * d + c];
                val += P[q * n + j] * dO[q * d + c];
            }
            dX[j * d + c] = scale * key + val;
        }
    free(P);
    free(dS);
}

/* ------------------------------------------------------------------------
 * Bottleneck adapter: down-projection C -> r, K x K SparseConv2D r -> r,
 * up-projection r -> C, residual.  Wd [C][r], Wc [taps][r][r], Wu [r][C],
 * biases nullable; H1, H2 [n][r] and Y [n][C] written. */
static int32_t *identity_table(int64_t n)
{
    int32_t *I = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t k = 0; k < n; ++k) I[k] = (int32_t)k;
    return I;
}

void orc_adapter_fwd(const double *X, const int32_t *N, int64_t n, int32_t taps, int32_t C, int32_t r,
                     const double *Wd, const double *bd, const double *Wc, const double *bc,
                     const double *Wu, const double *bu, double *H1, double *H2, double *Y)
{
    int32_t *I = identity_table(n);
    orc_fwd(X, I, Wd, bd, H1, n, C, r, 1);
    orc_fwd(H1, N, Wc, bc, H2, n, r, r, taps);
    orc_fwd(H2, I, Wu, bu, Y, n, r, C, 1);
    for (int64_t e = 0; e < n * C; ++e) Y[e] += X[e];
    free(I);
}

/* Gradients of <Y, dY>:
 *   dWu = H2^T dY, dbu = sum_k dY[k], dH2 = dY Wu^T;
 *   dWc, dbc, dH1: the K x K layer's backward at (H1, dH2);
 *   dWd = X^T dH1, dbd = sum_k dH1[k], dX = dY + dH1 Wd^T.
 * H1 and H2 are recomputed from X. */
void orc_adapter_bwd(const double *X, const int32_t *N, int64_t n, int32_t taps, int32_t C, int32_t r,
                     const double *Wd, const double *bd, const double *Wc, const double *bc,
                     const double *Wu, const double *dY, double *dX, double *dWd, double *dbd,
                     double *dWc, double *dbc, double *dWu, double *dbu)
{
    const size_t hr = sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)r;
    double *H1 = (double *)malloc(hr), *H2 = (double *)malloc(hr);
    double *dH1 = (double *)malloc(hr), *dH2 = (double *)malloc(hr);
    int32_t *I = identity_table(n);
    orc_fwd(X, I, Wd, bd, H1, n, C, r, 1);
    orc_fwd(H1, N, Wc, bc, H2, n, r, r, taps);
    orc_bwd_dw(H2, I, dY, dWu, n, r, C, 1);
    orc_bwd_db(dY, dbu, n, C);
    orc_bwd_dx(dY, I, Wu, dH2, n, r, C, 1);
    orc_bwd_dw(H1, N, dH2, dWc, n, r, r, taps);
    orc_bwd_db(dH2, dbc, n, r);
    orc_bwd_dx(dH2, N, Wc, dH1, n, r, r, taps);
    orc_bwd_dw(X, I, dH1, dWd, n, C, r, 1);
    orc_bwd_db(dH1, dbd, n, r);
    orc_bwd_dx(dH1, I, Wd, dX, n, C, r, 1);
    for (int64_t e = 0; e < n * C; ++e) dX[e] += dY[e];
    free(I);
    free(H1);
    free(H2);
    free(dH1);
    free(dH2);
}
