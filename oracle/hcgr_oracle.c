/*
 * hcgr_oracle.c -- plain, slow, fp64 CPU reference of the Hyper-Connection
 * Gated Residual (HCGR) op.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. The GPU library
 * shares no code, header, table or helper with it.
 *
 * Source of every formula: ROCm/aiter pull request #5913, "Two-stage
 * Hyper-Connection Gated Residual kernel", section "Technical Details", the
 * six per-token steps (COMBINE), (N), (G1), (G2), (MIX) and (INJ); and its
 * "Performance" section for the merged down/inject matrix with (1+w) folded
 * into its columns. Readings where the page leaves a point open:
 *   - R is stream-major: element (s, c) of the [HC x HS] residual sits at
 *     k = s*HS + c of the flattened row of length K = HC*HS.
 *   - eps is added to the mean of squares inside the square root.
 *   - Wnorm has HS entries shared by every stream (indexed by c), or, as a
 *     create-time option, K entries (indexed by k = s*HS + c).
 *   - the 1/HC scale sits inside SiLU, h = SiLU(lora / HC); inj_next is not
 *     scaled.
 *   - merged layout: rows 0..r-1 of Wm are Wd, rows r..r+HC-1 are Wi, the
 *     remaining rows up to n_pad are padding; the caller has already folded
 *     (1 + Wnorm) into the columns, so the down/inject products take
 *     R2 * rrms (without the (1 + Wnorm) factor), while MIX still uses the
 *     full xn = R2 * rrms * (1 + Wnorm).
 * Every bf16 input is widened exactly to double; every step runs in double
 * in the order the page lists, one token at a time.
 *
 * Besides the whole op, the same pull request's "PR Self-Review" section lists
 * a combine-only entry point and a mix entry point. Reading taken here (the
 * page names them without formulas): combine = (COMBINE) alone, giving R2;
 * mix = every other step applied to a residual that needs no injection, that
 * is R2 = R, giving rrms, inj_next and x. Both run through the loop below
 * with the other part switched off.
 *
 * Parity pins for each step live in the test-suite (closed forms, invariants
 * and one-hot special cases); none of them calls this file's arithmetic twice.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t hc;          /* number of residual streams HC            */
    int32_t hs;          /* width of one stream HS                   */
    int32_t r;           /* low-rank width of the down projection    */
    int32_t wnorm_full;  /* 0: Wnorm[HS] by channel; 1: Wnorm[K] by k */
    int32_t merged;      /* 0: separate Wd, Wi; 1: folded Wm[n_pad,K]  */
    int32_t n_pad;       /* rows of Wm when merged                    */
    double eps;          /* RMSNorm epsilon                           */
} hcgr_oracle_cfg;

/* Exact widening of a bf16 bit pattern: the 16 bits are the top half of an
 * IEEE-754 binary32 value. */
static double widen_bf16(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double* widen_all(const uint16_t* src, int64_t n)
{
    double* d = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!d) return NULL;
    for (int64_t i = 0; i < n; ++i) d[i] = widen_bf16(src[i]);
    return d;
}

static double logistic(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Which parts of the op run_tokens computes. */
enum { PART_COMBINE = 1, PART_MIX = 2 };

/* The op, or one of its two parts, for M tokens. With PART_COMBINE the
 * residual is R2 = R + y*iw; without it R2 = R (y and inj are not read).
 * With PART_MIX the steps N, G1, INJ, G2 and MIX follow; without it only R2
 * is produced (the weights are not read). */
static int run_tokens(const hcgr_oracle_cfg* cfg, int64_t M, int parts,
                      const uint16_t* R, const uint16_t* y,
                      const uint16_t* inj, int64_t ld_inj,
                      const uint16_t* wnorm, const uint16_t* wd,
                      const uint16_t* wi, const uint16_t* wu,
                      double* R2_out, double* rrms_out, double* inj_next_out,
                      double* x_out, double* xn_dbg, double* lora_dbg,
                      double* h_dbg, double* gate_dbg, double* G_dbg,
                      int nthreads)
{
    if (!cfg || M < 0 || cfg->hc < 1 || cfg->hs < 1 || cfg->r < 1)
        return -1;
    if ((parts & PART_COMBINE) && ld_inj < cfg->hc) return -1;
    if ((parts & PART_MIX) && cfg->merged && cfg->n_pad < cfg->r + cfg->hc) return -1;
    if (M == 0) return 0;
    const int HC = cfg->hc, HS = cfg->hs, RR = cfg->r;
    const int64_t K = (int64_t)HC * HS;
    const int64_t wlen = cfg->wnorm_full ? K : HS;
    const int64_t down_rows = cfg->merged ? cfg->n_pad : RR;
    const int mix = (parts & PART_MIX) != 0;

    double* Wn = mix ? widen_all(wnorm, wlen) : NULL;
    double* Wd = mix ? widen_all(wd, down_rows * K) : NULL;          /* Wd [r,K] or Wm [n_pad,K] */
    double* Wi = (mix && !cfg->merged) ? widen_all(wi, (int64_t)HC * K) : NULL;
    double* Wu = mix ? widen_all(wu, K * RR) : NULL;                 /* Wu [K,r]                 */
    if (mix && (!Wn || !Wd || !Wu || (!cfg->merged && !Wi))) {
        free(Wn); free(Wd); free(Wi); free(Wu);
        return -2;
    }
    int status = 0;
    /* nthreads > 0 sets this region's team size only (num_threads clause),
       so a one-thread call leaves later calls on every core */
#ifdef _OPENMP
    const int team = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif

#pragma omp parallel num_threads(team)
    {
        double* iw = (double*)malloc(sizeof(double) * HC);
        double* r2 = (double*)malloc(sizeof(double) * K);
        double* rr = (double*)malloc(sizeof(double) * HC);
        double* xn = (double*)malloc(sizeof(double) * K);
        double* u = (double*)malloc(sizeof(double) * K);
        double* lora = (double*)malloc(sizeof(double) * RR);
        double* h = (double*)malloc(sizeof(double) * RR);
        double* gate = (double*)malloc(sizeof(double) * K);
        double* G = (double*)malloc(sizeof(double) * K);
        int ok = iw && r2 && rr && xn && u && lora && h && gate && G;
        if (!ok) {
#pragma omp atomic write
            status = -2;
        }

#pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            if (!ok) continue;
            const uint16_t* Rm = R + m * K;
            if (parts & PART_COMBINE) {
                const uint16_t* ym = y + m * HS;
                const uint16_t* im = inj + m * ld_inj;
                /* (COMBINE) injection weights: iw[s] = 2 * sigmoid(inj[s] / HC) */
                for (int s = 0; s < HC; ++s)
                    iw[s] = 2.0 * logistic(widen_bf16(im[s]) / HC);
                /* (COMBINE) next residual: R2[s,c] = R[s,c] + y[c] * iw[s] */
                for (int s = 0; s < HC; ++s)
                    for (int c = 0; c < HS; ++c)
                        r2[(int64_t)s * HS + c] = widen_bf16(Rm[(int64_t)s * HS + c]) + widen_bf16(ym[c]) * iw[s];
            } else {
                /* mix entry: no injection, the residual is R itself */
                for (int64_t k = 0; k < K; ++k) r2[k] = widen_bf16(Rm[k]);
            }
            if (!mix) {
                if (R2_out) memcpy(R2_out + m * K, r2, sizeof(double) * K);
                continue;
            }

            /* (N) per-stream reciprocal RMS: rrms[s] = 1 / sqrt(mean_c R2[s,c]^2 + eps) */
            for (int s = 0; s < HC; ++s) {
                double sq = 0.0;
                for (int c = 0; c < HS; ++c) sq += r2[(int64_t)s * HS + c] * r2[(int64_t)s * HS + c];
                double ms = sq / HS;
                rr[s] = 1.0 / sqrt(ms + cfg->eps);
            }
            /* (N) xn[s,c] = R2[s,c] * rrms[s] * (1 + Wnorm) */
            for (int s = 0; s < HC; ++s)
                for (int c = 0; c < HS; ++c) {
                    int64_t k = (int64_t)s * HS + c;
                    double wn = cfg->wnorm_full ? Wn[k] : Wn[c];
                    xn[k] = r2[k] * rr[s] * (1.0 + wn);
                    u[k] = r2[k] * rr[s];
                }

            /* (G1) lora = xn . Wd^T over K; with the folded merged matrix the
             * (1 + Wnorm) factor already sits in the weight, so it takes u. */
            const double* act = cfg->merged ? u : xn;
            for (int j = 0; j < RR; ++j) {
                const double* wrow = Wd + (int64_t)j * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += act[k] * wrow[k];
                lora[j] = acc;
            }
            /* (INJ) inj_next = xn . Wi^T over K (no 1/HC scale) */
            for (int t = 0; t < HC; ++t) {
                const double* wrow = cfg->merged ? (Wd + (int64_t)(RR + t) * K) : (Wi + (int64_t)t * K);
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += act[k] * wrow[k];
                if (inj_next_out) inj_next_out[m * HC + t] = acc;
            }
            /* (G1) h = SiLU(lora / HC), SiLU(z) = z * sigmoid(z) */
            for (int j = 0; j < RR; ++j) {
                double zj = lora[j] / HC;
                h[j] = zj * logistic(zj);
            }

            /* (G2) gate = h . Wu^T over r; G = sigmoid(gate) */
            for (int64_t k = 0; k < K; ++k) {
                const double* wrow = Wu + k * RR;
                double acc = 0.0;
                for (int j = 0; j < RR; ++j) acc += h[j] * wrow[j];
                gate[k] = acc;
                G[k] = logistic(acc);
            }

            /* (MIX) x[c] = (1/HC) * sum_s G[s,c] * xn[s,c] */
            for (int c = 0; c < HS; ++c) {
                double acc = 0.0;
                for (int s = 0; s < HC; ++s) acc += G[(int64_t)s * HS + c] * xn[(int64_t)s * HS + c];
                if (x_out) x_out[m * HS + c] = acc / HC;
            }

            if (R2_out) memcpy(R2_out + m * K, r2, sizeof(double) * K);
            if (rrms_out) memcpy(rrms_out + m * HC, rr, sizeof(double) * HC);
            if (xn_dbg) memcpy(xn_dbg + m * K, xn, sizeof(double) * K);
            if (lora_dbg) memcpy(lora_dbg + m * RR, lora, sizeof(double) * RR);
            if (h_dbg) memcpy(h_dbg + m * RR, h, sizeof(double) * RR);
            if (gate_dbg) memcpy(gate_dbg + m * K, gate, sizeof(double) * K);
            if (G_dbg) memcpy(G_dbg + m * K, G, sizeof(double) * K);
        }
        free(iw); free(r2); free(rr); free(xn); free(u);
        free(lora); free(h); free(gate); free(G);
    }
    free(Wn); free(Wd); free(Wi); free(Wu);
    return status;
}

/* The whole op. Returns 0 on success, -1 on a bad argument, -2 on
 * allocation failure. Outputs (double, row-major): R2 [M,K], rrms [M,HC],
 * inj_next [M,HC], x [M,HS]. Optional intermediates (pass NULL to skip):
 * xn [M,K], lora [M,r], h [M,r], gate [M,K], G [M,K]. */
int hcgr_oracle_forward(const hcgr_oracle_cfg* cfg, int64_t M,
                        const uint16_t* R, const uint16_t* y,
                        const uint16_t* inj, int64_t ld_inj,
                        const uint16_t* wnorm, const uint16_t* wd,
                        const uint16_t* wi, const uint16_t* wu,
                        double* R2_out, double* rrms_out, double* inj_next_out,
                        double* x_out, double* xn_dbg, double* lora_dbg,
                        double* h_dbg, double* gate_dbg, double* G_dbg,
                        int nthreads)
{
    return run_tokens(cfg, M, PART_COMBINE | PART_MIX, R, y, inj, ld_inj, wnorm, wd, wi, wu,
                      R2_out, rrms_out, inj_next_out, x_out, xn_dbg, lora_dbg, h_dbg, gate_dbg,
                      G_dbg, nthreads);
}

/* (COMBINE) alone: R2 [M,K] from R, y and the (row stride ld_inj) logits. */
int hcgr_oracle_combine(const hcgr_oracle_cfg* cfg, int64_t M,
                        const uint16_t* R, const uint16_t* y,
                        const uint16_t* inj, int64_t ld_inj,
                        double* R2_out, int nthreads)
{
    return run_tokens(cfg, M, PART_COMBINE, R, y, inj, ld_inj, NULL, NULL, NULL, NULL,
                      R2_out, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, nthreads);
}

/* Every step but COMBINE, on a residual R [M,K] that is taken as R2:
 * rrms [M,HC], inj_next [M,HC], x [M,HS] (+ the optional intermediates). */
int hcgr_oracle_mix(const hcgr_oracle_cfg* cfg, int64_t M, const uint16_t* R,
                    const uint16_t* wnorm, const uint16_t* wd,
                    const uint16_t* wi, const uint16_t* wu,
                    double* rrms_out, double* inj_next_out, double* x_out,
                    double* xn_dbg, double* lora_dbg, double* h_dbg,
                    double* gate_dbg, double* G_dbg, int nthreads)
{
    return run_tokens(cfg, M, PART_MIX, R, NULL, NULL, 0, wnorm, wd, wi, wu,
                      NULL, rrms_out, inj_next_out, x_out, xn_dbg, lora_dbg, h_dbg, gate_dbg,
                      G_dbg, nthreads);
}

/* Number of threads an OpenMP parallel region of this library would use. */
int hcgr_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
