/*
 * lnr_oracle.c -- fp64 CPU oracle for masked/causal attention softmax, LayerNorm, RMSNorm
 * and softmax cross-entropy over a vocabulary, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY. The product library never links, loads or calls this file.
 * Only the test suite, the smoke check and the CPU-baseline leg of the benchmark use it,
 * through oracle/__init__.py.
 *
 * Every function below is the plain textbook definition written with ordinary loops:
 *   - all arithmetic and all accumulation in double precision;
 *   - two-pass statistics (mean first, then the centred second moment), NOT the one-pass
 *     rewrite that the GPU kernels use, so the rewrite itself is under test;
 *   - inputs are double arrays holding the stored values exactly (fp16 and fp32 both widen
 *     to double without rounding); outputs are double and never rounded to a storage type.
 * OpenMP spreads independent rows (or independent column blocks) over threads. Each output
 * element is still produced by one thread summing in the natural index order, so the thread
 * count never changes a result.
 *
 * Sources (the pages this oracle follows):
 *   [L10]  "CMU 11-868 L10: Accelerating Transformers on GPUs, and Where LightSeq Finds the
 *          Time", section "Technique 2: rewrite the formula, drop a synchronization".
 *   [HW4]  "CMU 11-868 HW4: Softmax and LayerNorm as fused CUDA kernels", section
 *          "Problem structure and scoring" (softmax with attention mask and future-token
 *          mask; LayerNorm with epsilon inside the square root; LayerNorm backward as dinp
 *          plus dgamma/dbeta summed across rows) and section "Faster than what?" (the
 *          softmax(inp + mask) baseline, i.e. an additive mask).
 *   [FT]   "FastTransformer: Breaking the Compiler Ceiling via Architectural Co-Design",
 *          section 5.4 "Vectorized Pre-RMSNorm" (RMSNorm: no mean, one sum of squares).
 *   [L10]  section "Technique 1: kernel fusion, leaving only GEMMs to cuBLAS" (cross entropy
 *          is one of the custom reduce kernels; "bias + dropout + residual" one of the
 *          elementwise kernels, followed by LayerNorm) and "Inference: making beam search skip a
 *          sort" (a softmax over the whole vocabulary). The pages give no formula; the
 *          oracle is the textbook softmax cross-entropy (no label smoothing).
 * The softmax backward formula is never printed on the pages; it is the textbook Jacobian
 * of softmax (diag(y) - y y^T) applied to dy, and it is pinned by finite differences.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------------------------------
 * Attention softmax, forward. [HW4 "Problem structure and scoring"; L10 "Technique 2"]
 * One row r = (b, h, i) of the score tensor [B, H, Tq, Tk]:
 *   z_j = x_j + m_j           (additive attention mask, key-padding positions hold -inf)
 *   z_j = -inf  for j > i     (future tokens, when causal)
 *   M   = max_j z_j           (the first reduction: keeps exp from overflowing)
 *   e_j = exp(z_j - M),  S = sum_j e_j   (the second reduction)
 *   y_j = e_j / S
 * A row whose every position is masked (M = -inf) has no defined softmax; this oracle
 * returns zeros for it (the reading taken where the pages are silent).
 * ------------------------------------------------------------------------------------- */
static double masked_score(const double *x, const double *mrow, int64_t j, int64_t qi,
                           int causal)
{
    if (causal && j > qi)
        return -INFINITY;
    double z = x[j];
    if (mrow)
        z += mrow[j];
    return z;
}

static void softmax_fw_row(const double *x, const double *mrow, int64_t Tk, int64_t qi,
                           int causal, double *y)
{
    double M = -INFINITY;
    for (int64_t j = 0; j < Tk; ++j) {
        double z = masked_score(x, mrow, j, qi, causal);
        if (z > M)
            M = z;
    }
    if (M == -INFINITY) {
        for (int64_t j = 0; j < Tk; ++j)
            y[j] = 0.0;
        return;
    }
    double S = 0.0;
    for (int64_t j = 0; j < Tk; ++j) {
        double z = masked_score(x, mrow, j, qi, causal);
        double e = (z == -INFINITY) ? 0.0 : exp(z - M);
        y[j] = e;
        S += e;
    }
    for (int64_t j = 0; j < Tk; ++j)
        y[j] = y[j] / S;
}

/* Whole tensor: x, y are [B, H, Tq, Tk]; mask is [B, Tk] (broadcast over H and Tq) or NULL. */
ORACLE_API void lnr_oracle_softmax_fw(const double *x, const double *mask, int64_t B,
                                      int64_t H, int64_t Tq, int64_t Tk, int causal, double *y)
{
    const int64_t rows = B * H * Tq;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r / (H * Tq);
        const int64_t i = r % Tq;
        softmax_fw_row(x + r * Tk, mask ? mask + b * Tk : 0, Tk, i, causal, y + r * Tk);
    }
}

/* Selected rows: x, y are [nrows, Tk]; mask_rows is [nrows, Tk] (the mask row of each
 * selected row's batch) or NULL; qidx[r] is the query position i of selected row r. */
ORACLE_API void lnr_oracle_softmax_fw_rows(const double *x, const double *mask_rows,
                                           const int64_t *qidx, int64_t nrows, int64_t Tk,
                                           int causal, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r)
        softmax_fw_row(x + r * Tk, mask_rows ? mask_rows + r * Tk : 0, Tk, qidx[r], causal,
                       y + r * Tk);
}

/* ---------------------------------------------------------------------------------------
 * Attention softmax, backward. [HW4 "Problem structure and scoring" names the kernel]
 * For one row with forward output y and upstream gradient dy:
 *   t    = sum_j y_j * dy_j
 *   dx_j = y_j * (dy_j - t)
 * i.e. (diag(y) - y y^T) dy. Masked positions have y_j = 0 and therefore dx_j = 0.
 * y, dy, dx are [rows, Tk].
 * ------------------------------------------------------------------------------------- */
ORACLE_API void lnr_oracle_softmax_bw(const double *y, const double *dy, int64_t rows,
                                      int64_t Tk, double *dx)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *yr = y + r * Tk, *dyr = dy + r * Tk;
        double t = 0.0;
        for (int64_t j = 0; j < Tk; ++j)
            t += yr[j] * dyr[j];
        for (int64_t j = 0; j < Tk; ++j)
            dx[r * Tk + j] = yr[j] * (dyr[j] - t);
    }
}

/* ---------------------------------------------------------------------------------------
 * LayerNorm statistics of one row, two-pass definition. [L10 "Technique 2"; HW4]
 *   mu    = (1/C) sum_j x_j
 *   var   = (1/C) sum_j (x_j - mu)^2          (biased: a mean, as mu(x^2) is a mean)
 *   sigma = sqrt(var + eps)                    (eps inside the root, as on the HW4 page)
 * ------------------------------------------------------------------------------------- */
static void row_stats(const double *x, int64_t C, double eps, double *mu_out,
                      double *sigma_out)
{
    double s = 0.0;
    for (int64_t j = 0; j < C; ++j)
        s += x[j];
    const double mu = s / (double)C;
    double q = 0.0;
    for (int64_t j = 0; j < C; ++j) {
        const double d = x[j] - mu;
        q += d * d;
    }
    const double var = q / (double)C;
    *mu_out = mu;
    *sigma_out = sqrt(var + eps);
}

/* LayerNorm forward: y = gamma * (x - mu) / sigma + beta. x, y: [N, C]; gamma, beta: [C].
 * Also returns mu and 1/sigma per row (mean, rstd: [N]). */
ORACLE_API void lnr_oracle_layernorm_fw(const double *x, const double *gamma,
                                        const double *beta, int64_t N, int64_t C, double eps,
                                        double *y, double *mean, double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *xr = x + i * C;
        double mu, sigma;
        row_stats(xr, C, eps, &mu, &sigma);
        for (int64_t j = 0; j < C; ++j)
            y[i * C + j] = gamma[j] * ((xr[j] - mu) / sigma) + beta[j];
        mean[i] = mu;
        rstd[i] = 1.0 / sigma;
    }
}

/* ---------------------------------------------------------------------------------------
 * LayerNorm backward, input gradient. [L10 "Technique 2"; HW4 "Problem structure"]
 * With xhat_j = (x_j - mu)/sigma and g_j = gamma_j * dy_j, differentiating
 * y_j = gamma_j xhat_j + beta_j through mu and sigma (eps inside sigma) gives
 *   dx_j = (1/sigma) * ( g_j - (1/C) sum_k g_k - xhat_j * (1/C) sum_k g_k xhat_k ),
 * the two row sums that the L10 lecture rearranges to run in parallel. The statistics are
 * recomputed here from x in double, so the saved-statistics format cannot affect parity.
 * x, dy, dx: [N, C]; gamma: [C].
 * ------------------------------------------------------------------------------------- */
ORACLE_API void lnr_oracle_layernorm_bw_dx(const double *x, const double *dy,
                                           const double *gamma, int64_t N, int64_t C,
                                           double eps, double *dx)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *xr = x + i * C, *dyr = dy + i * C;
        double mu, sigma;
        row_stats(xr, C, eps, &mu, &sigma);
        double sum_g = 0.0, sum_gx = 0.0;
        for (int64_t j = 0; j < C; ++j) {
            const double xhat = (xr[j] - mu) / sigma;
            const double g = gamma[j] * dyr[j];
            sum_g += g;
            sum_gx += g * xhat;
        }
        const double a = sum_g / (double)C, b = sum_gx / (double)C;
        for (int64_t j = 0; j < C; ++j) {
            const double xhat = (xr[j] - mu) / sigma;
            const double g = gamma[j] * dyr[j];
            dx[i * C + j] = (g - a - xhat * b) / sigma;
        }
    }
}

/* ---------------------------------------------------------------------------------------
 * LayerNorm backward, parameter gradients: sums across rows. [HW4 "Problem structure"]
 *   dgamma_j = sum_i dy_ij * xhat_ij,   dbeta_j = sum_i dy_ij
 * Every column is summed over i = 0..N-1 in that order. Threads own disjoint blocks of
 * columns; that only chooses which thread does a column, not the order of its sum.
 * x, dy: [N, C]; dgamma, dbeta: [C]. mu/sigma per row are recomputed from x first.
 * ------------------------------------------------------------------------------------- */
ORACLE_API void lnr_oracle_layernorm_bw_dgamma_dbeta(const double *x, const double *dy,
                                                     int64_t N, int64_t C, double eps,
                                                     double *mu_ws, double *sigma_ws,
                                                     double *dgamma, double *dbeta)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i)
        row_stats(x + i * C, C, eps, &mu_ws[i], &sigma_ws[i]);

    const int64_t blk = 64;
#pragma omp parallel for schedule(static)
    for (int64_t jb = 0; jb < C; jb += blk) {
        const int64_t je = (jb + blk < C) ? jb + blk : C;
        for (int64_t j = jb; j < je; ++j) {
            dgamma[j] = 0.0;
            dbeta[j] = 0.0;
        }
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t j = jb; j < je; ++j) {
                const double xhat = (x[i * C + j] - mu_ws[i]) / sigma_ws[i];
                dgamma[j] += dy[i * C + j] * xhat;
                dbeta[j] += dy[i * C + j];
            }
        }
    }
}

/* ---------------------------------------------------------------------------------------
 * LayerNorm backward from given statistics. [L10 "Technique 2"; HW4 "Problem structure"]
 * The same formulas as above, with mu_i and 1/sigma_i taken from mean[i] and rstd[i] (the
 * values a forward pass saved) instead of being recomputed from x:
 *   xhat_ij = (x_ij - mean_i) * rstd_i,  g_ij = gamma_j * dy_ij
 *   dx_ij   = rstd_i * ( g_ij - (1/C) sum_k g_ik - xhat_ij * (1/C) sum_k g_ik xhat_ik )
 *   dgamma_j = sum_i dy_ij * xhat_ij,  dbeta_j = sum_i dy_ij
 * This is the function a backward kernel that receives saved statistics computes; with the
 * exact statistics it equals the recomputing version.
 * ------------------------------------------------------------------------------------- */
ORACLE_API void lnr_oracle_layernorm_bw_given_stats(const double *x, const double *dy,
                                                    const double *gamma, const double *mean,
                                                    const double *rstd, int64_t N, int64_t C,
                                                    double *dx, double *dgamma, double *dbeta)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *xr = x + i * C, *dyr = dy + i * C;
        double sum_g = 0.0, sum_gx = 0.0;
        for (int64_t j = 0; j < C; ++j) {
            const double xhat = (xr[j] - mean[i]) * rstd[i];
            const double g = gamma[j] * dyr[j];
            sum_g += g;
            sum_gx += g * xhat;
        }
        const double a = sum_g / (double)C, b = sum_gx / (double)C;
        for (int64_t j = 0; j < C; ++j) {
            const double xhat = (xr[j] - mean[i]) * rstd[i];
            const double g = gamma[j] * dyr[j];
            dx[i * C + j] = rstd[i] * (g - a - xhat * b);
        }
    }
    const int64_t blk = 64;
#pragma omp parallel for schedule(static)
    for (int64_t jb = 0; jb < C; jb += blk) {
        const int64_t je = (jb + blk < C) ? jb + blk : C;
        for (int64_t j = jb; j < je; ++j) {
            dgamma[j] = 0.0;
            dbeta[j] = 0.0;
        }
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t j = jb; j < je; ++j) {
                const double xhat = (x[i * C + j] - mean[i]) * rstd[i];
                dgamma[j] += dy[i * C + j] * xhat;
                dbeta[j] += dy[i * C + j];
            }
        }
    }
}

/* ---------------------------------------------------------------------------------------
 * RMSNorm (forward and input gradient). [FT section 5.4]
 *   rms = sqrt((1/C) sum_j x_j^2 + eps),  y_j = gamma_j * x_j / rms
 *   dx_j = (1/rms) * ( g_j - xhat_j * (1/C) sum_k g_k xhat_k ),  g = gamma*dy, xhat = x/rms
 *   dgamma_j = sum_i dy_ij * xhat_ij
 * ------------------------------------------------------------------------------------- */
ORACLE_API void lnr_oracle_rmsnorm_fw(const double *x, const double *gamma, int64_t N,
                                      int64_t C, double eps, double *y, double *rrms)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *xr = x + i * C;
        double q = 0.0;
        for (int64_t j = 0; j < C; ++j)
            q += xr[j] * xr[j];
        const double rms = sqrt(q / (double)C + eps);
        for (int64_t j = 0; j < C; ++j)
            y[i * C + j] = gamma[j] * (xr[j] / rms);
        rrms[i] = 1.0 / rms;
    }
}

ORACLE_API void lnr_oracle_rmsnorm_bw(const double *x, const double *dy, const double *gamma,
                                      int64_t N, int64_t C, double eps, double *dx,
                                      double *dgamma)
{
    double *rms = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    if (rms == NULL)
        abort();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *xr = x + i * C, *dyr = dy + i * C;
        double q = 0.0;
        for (int64_t j = 0; j < C; ++j)
            q += xr[j] * xr[j];
        rms[i] = sqrt(q / (double)C + eps);
        double sum_gx = 0.0;
        for (int64_t j = 0; j < C; ++j)
            sum_gx += gamma[j] * dyr[j] * (xr[j] / rms[i]);
        const double b = sum_gx / (double)C;
        for (int64_t j = 0; j < C; ++j)
            dx[i * C + j] = (gamma[j] * dyr[j] - (xr[j] / rms[i]) * b) / rms[i];
    }
    /* dgamma_j = sum over rows in row order, columns spread over threads. */
    const int64_t blk = 64;
#pragma omp parallel for schedule(static)
    for (int64_t jb = 0; jb < C; jb += blk) {
        const int64_t je = (jb + blk < C) ? jb + blk : C;
        for (int64_t j = jb; j < je; ++j)
            dgamma[j] = 0.0;
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = jb; j < je; ++j)
                dgamma[j] += dy[i * C + j] * (x[i * C + j] / rms[i]);
    }
    free(rms);
}

/* ---------------------------------------------------------------------------------------
 * RMSNorm backward from a given rstd. [FT section 5.4]
 * The chain rule through y_ij = gamma_j * x_ij * r_i with r_i = (mean_k x_ik^2 + eps)^(-1/2),
 * whose derivative is dr_i/dx_ik = -r_i^3 x_ik / C, evaluated with r_i taken from rstd[i]
 * (the value a forward pass saved) instead of recomputed from x:
 *   xhat_ij = x_ij * rstd_i,  g_ij = gamma_j * dy_ij
 *   dx_ij   = rstd_i * ( g_ij - xhat_ij * (1/C) sum_k g_ik xhat_ik )
 *   dgamma_j = sum_i dy_ij * xhat_ij
 * With the exact rstd it equals lnr_oracle_rmsnorm_bw.
 * ------------------------------------------------------------------------------------- */
ORACLE_API void lnr_oracle_rmsnorm_bw_given_rstd(const double *x, const double *dy,
                                                 const double *gamma, const double *rstd,
                                                 int64_t N, int64_t C, double *dx,
                                                 double *dgamma)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *xr = x + i * C, *dyr = dy + i * C;
        double sum_gx = 0.0;
        for (int64_t j = 0; j < C; ++j)
            sum_gx += gamma[j] * dyr[j] * (xr[j] * rstd[i]);
        const double b = sum_gx / (double)C;
        for (int64_t j = 0; j < C; ++j)
            dx[i * C + j] = rstd[i] * (gamma[j] * dyr[j] - (xr[j] * rstd[i]) * b);
    }
    const int64_t blk = 64;
#pragma omp parallel for schedule(static)
    for (int64_t jb = 0; jb < C; jb += blk) {
        const int64_t je = (jb + blk < C) ? jb + blk : C;
        for (int64_t j = jb; j < je; ++j)
            dgamma[j] = 0.0;
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = jb; j < je; ++j)
                dgamma[j] += dy[i * C + j] * (x[i * C + j] * rstd[i]);
    }
}

/* ---------------------------------------------------------------------------------------
 * Bias + dropout + residual, then LayerNorm. [L10 "Technique 1": "bias + dropout + residual"
 * is one of the elementwise kernels between the GEMMs, and LayerNorm follows it in the layer]
 * The dropout draws are an input: keep_ij is bit (j % 8) of mask[i * ceil(C/8) + j / 8]
 * (least significant bit first), p the drop probability (0 <= p < 1).
 *   s_ij = residual_ij + keep_ij * (x_ij + bias_j) / (1 - p)
 *   y    = LayerNorm(s) with gamma, beta, eps (two-pass statistics, as above)
 * Outputs s, y and the per-row mean and 1/sigma of s.
 * ------------------------------------------------------------------------------------- */
static int keep_bit(const unsigned char *mask, int64_t i, int64_t j, int64_t C)
{
    const int64_t mb = (C + 7) / 8;
    return (mask[i * mb + j / 8] >> (j % 8)) & 1;
}

ORACLE_API void lnr_oracle_bdr_ln_fw(const double *x, const double *residual, const double *bias,
                                     const unsigned char *mask, double p, const double *gamma,
                                     const double *beta, int64_t N, int64_t C, double eps,
                                     double *s, double *y, double *mean, double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        double *sr = s + i * C;
        for (int64_t j = 0; j < C; ++j)
            sr[j] = residual[i * C + j] +
                    (keep_bit(mask, i, j, C) ? (x[i * C + j] + bias[j]) / (1.0 - p) : 0.0);
        double mu = 0.0;
        for (int64_t j = 0; j < C; ++j)
            mu += sr[j];
        mu /= (double)C;
        double q = 0.0;
        for (int64_t j = 0; j < C; ++j)
            q += (sr[j] - mu) * (sr[j] - mu);
        const double sigma = sqrt(q / (double)C + eps);
        for (int64_t j = 0; j < C; ++j)
            y[i * C + j] = gamma[j] * ((sr[j] - mu) / sigma) + beta[j];
        mean[i] = mu;
        rstd[i] = 1.0 / sigma;
    }
}

/* Backward of the fused op from the saved s, mean and rstd. dy is the gradient of y; ds_extra
 * (may be NULL) is a gradient reaching s by another path. With ds the LayerNorm input
 * gradient (the given-statistics formula above) plus ds_extra:
 *   dresidual = ds,   dx_ij = ds_ij * keep_ij / (1 - p),   dbias_j = sum_i dx_ij,
 *   dgamma_j = sum_i dy_ij * shat_ij,   dbeta_j = sum_i dy_ij,  shat = (s - mean) * rstd. */
ORACLE_API void lnr_oracle_bdr_ln_bw(const double *s, const double *dy, const double *ds_extra,
                                     const unsigned char *mask, double p, const double *gamma,
                                     const double *mean, const double *rstd, int64_t N, int64_t C,
                                     double *dresidual, double *dx, double *dgamma,
                                     double *dbeta, double *dbias)
{
    /* ds from the LayerNorm backward on the saved statistics */
    lnr_oracle_layernorm_bw_given_stats(s, dy, gamma, mean, rstd, N, C, dresidual, dgamma, dbeta);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < C; ++j) {
            const double ds = dresidual[i * C + j] + (ds_extra ? ds_extra[i * C + j] : 0.0);
            dresidual[i * C + j] = ds;
            dx[i * C + j] = keep_bit(mask, i, j, C) ? ds / (1.0 - p) : 0.0;
        }
    const int64_t blk = 64;
#pragma omp parallel for schedule(static)
    for (int64_t jb = 0; jb < C; jb += blk) {
        const int64_t je = (jb + blk < C) ? jb + blk : C;
        for (int64_t j = jb; j < je; ++j)
            dbias[j] = 0.0;
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = jb; j < je; ++j)
                dbias[j] += dx[i * C + j];
    }
}

/* ---------------------------------------------------------------------------------------
 * Softmax cross-entropy over a vocabulary. [L10 "Technique 1"; textbook definition]
 * For row i with logits z_i[0..V) and target t_i:
 *   M_i   = max_j z_ij,   lse_i = M_i + log( sum_j exp(z_ij - M_i) )
 *   loss_i = lse_i - z_i,t_i
 * A row whose target equals ignore_index has loss 0 (its lse is still computed). A target
 * outside [0, V) that is not ignore_index gives loss NaN.
 * ------------------------------------------------------------------------------------- */
ORACLE_API void lnr_oracle_xent_fw(const double *z, const int64_t *target, int64_t N, int64_t V,
                                   int64_t ignore_index, double *loss, double *lse)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *zr = z + i * V;
        double M = -INFINITY;
        for (int64_t j = 0; j < V; ++j)
            if (zr[j] > M) M = zr[j];
        double S = 0.0;
        for (int64_t j = 0; j < V; ++j)
            S += exp(zr[j] - M);
        lse[i] = M + log(S);
        const int64_t t = target[i];
        if (t == ignore_index)
            loss[i] = 0.0;
        else if (t < 0 || t >= V)
            loss[i] = NAN;
        else
            loss[i] = lse[i] - zr[t];
    }
}

/* Cross-entropy backward from a given lse (the value a forward pass saved) and the upstream
 * gradient dloss_i of each row's loss:
 *   dz_ij = dloss_i * ( exp(z_ij - lse_i) - [j == t_i] )
 * (the derivative of lse - z_t: softmax minus the one-hot target). Rows whose target is
 * ignore_index get dz = 0; a target outside [0, V) otherwise gives a row of NaN. */
ORACLE_API void lnr_oracle_xent_bw_given_lse(const double *z, const int64_t *target,
                                             const double *lse, const double *dloss, int64_t N,
                                             int64_t V, int64_t ignore_index, double *dz)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const double *zr = z + i * V;
        const int64_t t = target[i];
        for (int64_t j = 0; j < V; ++j) {
            double d;
            if (t == ignore_index)
                d = 0.0;
            else if (t < 0 || t >= V)
                d = NAN;
            else
                d = dloss[i] * (exp(zr[j] - lse[i]) - (j == t ? 1.0 : 0.0));
            dz[i * V + j] = d;
        }
    }
}

/* Threads the OpenMP loops above will use (reported next to CPU timings). */
#ifdef _OPENMP
#include <omp.h>
#endif
ORACLE_API int lnr_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (timing only; results do not depend on it). */
ORACLE_API void lnr_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
