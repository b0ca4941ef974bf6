/*
 * kdn_oracle.c -- plain, sequential fp64 CPU oracle for the Kalman Delta
 * Network (KDN) mixer recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference that the
 * GPU library is checked against.  It shares no code, header, table or helper
 * with the HIP library under kalman_delta_network_amd/, and nothing in the
 * product path may load it: only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.
 *
 * Source of the equations: "Kalman Delta Networks: Uncertainty-aware
 * Associative Memory" (arXiv 2609.07816), summary page, section "方法步骤详情"
 * (method steps 1-5) and the English page, section 3 (Kalman view and its
 * diagonal restriction).  Every step below is the page's equation written out
 * one token at a time, in fp64, with no blocking, chunking or reordering:
 *
 *   predict    p_hat   = alpha^2 (.) p + omega                    (step 2)
 *   gain       kappa_i = p_hat_i k_i / (r + sum_j p_hat_j k_j^2)   (step 3)
 *   write      S       = diag(alpha) S + kappa (v - (diag(alpha) S)^T k)^T
 *                                                                 (step 4)
 *   read       o       = S^T q   (the post-write memory)          (step 4)
 *   posterior  u = (mu/r) k (.) k ;  p = p_hat / (1 + u (.) p_hat) (step 5)
 *
 * Isotropic variant (same section, last sentence): one uncertainty scalar b
 * per head, trace-projected prediction b_hat = a b + omega/d_k with
 * a = mean_i alpha_i^2 (alpha is a scalar per head-token here, so a =
 * alpha^2), scalar gain beta = b_hat/(r + b_hat |k|^2), kappa = beta k, and
 * the posterior precision increment averaged over the d_k channels:
 * b = b_hat / (1 + (mu/(d_k r)) |k|^2 b_hat).  That last formula is a reading
 * (the page does not print it); see the readings list of the repository.
 *
 * Isotropic variant with per-channel decay (the general form of the same
 * sentence): alpha has one decay per key channel, the memory decays by
 * diag(alpha), omega and r are scalars per head-token, and the trace
 * projection uses a = (1/d_k) sum_i alpha_i^2; gain and posterior as above.
 *
 * Inputs arrive as double arrays holding exactly the values the GPU receives
 * (bf16 and fp32 values widen to double without loss); all arithmetic is
 * double.
 * Layouts (row-major, contiguous):
 *   q, k, alpha, omega : [B,T,H,dk]   (isotropic alpha, omega: [B,T,H];
 *                                     per-channel-decay isotropic: omega [B,T,H])
 *   v, o               : [B,T,H,dv]
 *   r                  : [B,T,H]
 *   c0                 : [H]
 *   S0, S_T            : [B,H,dk,dv]
 *   p0, p_T            : [B,H,dk]     (isotropic: [B,H])
 * Optional per-token traces (NULL to skip), layout [B,T,H,dk]
 * (isotropic p_hat / p traces: [B,T,H]):
 *   tr_phat = predicted p_hat_t, tr_kappa = gain kappa_t, tr_p = posterior p_t.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stddef.h>

#define IDX_TOK(b, t, h, B, T, H) ((((size_t)(b) * (size_t)(T) + (size_t)(t)) * (size_t)(H)) + (size_t)(h))

/* One (b,h) recurrence of the Diagonal KDN, token by token. */
static void diag_head(int b, int h, int T, int H, int dk, int dv,
                      const double* q, const double* k, const double* v,
                      const double* alpha, const double* omega, const double* r,
                      const double* c0, double mu, const double* S0,
                      const double* p0, double* o, double* S_T, double* p_T,
                      double* tr_phat, double* tr_kappa, double* tr_p) {
    (void)T;
    const size_t state = ((size_t)b * H + h);
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* Sh = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* p = (double*)malloc(sizeof(double) * dk);
    double* ph = (double*)malloc(sizeof(double) * dk);
    double* kap = (double*)malloc(sizeof(double) * dk);
    double* delta = (double*)malloc(sizeof(double) * dv);

    /* initial state: S_0 = 0 and p_0 = c0[h] * 1 unless given */
    for (int i = 0; i < dk; ++i) {
        p[i] = p0 ? p0[state * dk + i] : (double)c0[h];
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] = S0 ? S0[state * (size_t)dk * dv + (size_t)i * dv + j] : 0.0;
    }

    for (int t = 0; t < T; ++t) {
        const size_t tok = IDX_TOK(b, t, h, 0, T, H);
        const double* kt = k + tok * dk;
        const double* qt = q + tok * dk;
        const double* vt = v + tok * dv;
        const double* at = alpha + tok * dk;
        const double* wt = omega + tok * dk;
        const double rt = (double)r[tok];

        /* predict: p_hat = alpha^2 p + omega */
        for (int i = 0; i < dk; ++i) {
            const double a = at[i];
            ph[i] = a * a * p[i] + (double)wt[i];
        }
        /* gain: kappa = p_hat k / (r + k^T (p_hat k)) */
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += ph[i] * (double)kt[i] * (double)kt[i];
        for (int i = 0; i < dk; ++i) kap[i] = ph[i] * (double)kt[i] / (rt + s);

        /* predicted mean S_hat = diag(alpha) S and innovation v - S_hat^T k */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) Sh[(size_t)i * dv + j] = (double)at[i] * S[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += Sh[(size_t)i * dv + j] * (double)kt[i];
            delta[j] = (double)vt[j] - pred;
        }
        /* residual write S = S_hat + kappa delta^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = Sh[(size_t)i * dv + j] + kap[i] * delta[j];
        /* readout from the written memory: o = S^T q */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * (double)qt[i];
            o[tok * dv + j] = acc;
        }
        /* mean-field posterior with information scale mu */
        for (int i = 0; i < dk; ++i) {
            const double u = (mu / rt) * (double)kt[i] * (double)kt[i];
            p[i] = ph[i] / (1.0 + u * ph[i]);
        }
        if (tr_phat) for (int i = 0; i < dk; ++i) tr_phat[tok * dk + i] = ph[i];
        if (tr_kappa) for (int i = 0; i < dk; ++i) tr_kappa[tok * dk + i] = kap[i];
        if (tr_p) for (int i = 0; i < dk; ++i) tr_p[tok * dk + i] = p[i];
    }

    for (int i = 0; i < dk; ++i) {
        if (p_T) p_T[state * dk + i] = p[i];
        if (S_T)
            for (int j = 0; j < dv; ++j)
                S_T[state * (size_t)dk * dv + (size_t)i * dv + j] = S[(size_t)i * dv + j];
    }
    free(S); free(Sh); free(p); free(ph); free(kap); free(delta);
}

/* One (b,h) recurrence of the Isotropic KDN (alpha, omega scalar per head-token). */
static void iso_head(int b, int h, int T, int H, int dk, int dv,
                     const double* q, const double* k, const double* v,
                     const double* alpha, const double* omega, const double* r,
                     const double* c0, double mu, const double* S0,
                     const double* p0, double* o, double* S_T, double* p_T,
                     double* tr_phat, double* tr_kappa, double* tr_p) {
    const size_t state = ((size_t)b * H + h);
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* delta = (double*)malloc(sizeof(double) * dv);
    double bcov = p0 ? p0[state] : (double)c0[h];
    for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = S0 ? S0[state * (size_t)dk * dv + e] : 0.0;

    for (int t = 0; t < T; ++t) {
        const size_t tok = IDX_TOK(b, t, h, 0, T, H);
        const double* kt = k + tok * dk;
        const double* qt = q + tok * dk;
        const double* vt = v + tok * dv;
        const double a = alpha[tok];
        const double w = omega[tok];
        const double rt = r[tok];

        /* trace-projected predict: b_hat = a b + omega/d_k, a = alpha^2 */
        const double bh = a * a * bcov + w / (double)dk;
        double n = 0.0;
        for (int i = 0; i < dk; ++i) n += (double)kt[i] * (double)kt[i];
        /* scalar gain beta = b_hat / (r + b_hat |k|^2), kappa = beta k */
        const double beta = bh / (rt + bh * n);
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += a * S[(size_t)i * dv + j] * (double)kt[i];
            delta[j] = (double)vt[j] - pred;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + beta * (double)kt[i] * delta[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * (double)qt[i];
            o[tok * dv + j] = acc;
        }
        /* posterior: precision increment (mu/r)|k|^2 averaged over d_k channels */
        bcov = bh / (1.0 + (mu / ((double)dk * rt)) * n * bh);
        if (tr_phat) tr_phat[tok] = bh;
        if (tr_kappa) for (int i = 0; i < dk; ++i) tr_kappa[tok * dk + i] = beta * (double)kt[i];
        if (tr_p) tr_p[tok] = bcov;
    }
    if (p_T) p_T[state] = bcov;
    if (S_T)
        for (size_t e = 0; e < (size_t)dk * dv; ++e) S_T[state * (size_t)dk * dv + e] = S[e];
    free(S); free(delta);
}

/* One (b,h) recurrence of the Isotropic KDN with per-channel decay: alpha
 * [.., dk], omega and r scalars per head-token. */
static void isoc_head(int b, int h, int T, int H, int dk, int dv,
                      const double* q, const double* k, const double* v,
                      const double* alpha, const double* omega, const double* r,
                      const double* c0, double mu, const double* S0,
                      const double* p0, double* o, double* S_T, double* p_T,
                      double* tr_phat, double* tr_kappa, double* tr_p) {
    const size_t state = ((size_t)b * H + h);
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* delta = (double*)malloc(sizeof(double) * dv);
    double bcov = p0 ? p0[state] : (double)c0[h];
    for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = S0 ? S0[state * (size_t)dk * dv + e] : 0.0;

    for (int t = 0; t < T; ++t) {
        const size_t tok = IDX_TOK(b, t, h, 0, T, H);
        const double* kt = k + tok * dk;
        const double* qt = q + tok * dk;
        const double* vt = v + tok * dv;
        const double* at = alpha + tok * dk;
        const double w = omega[tok];
        const double rt = r[tok];

        /* trace-projected predict: b_hat = a b + omega/d_k, a = mean_i alpha_i^2 */
        double a = 0.0;
        for (int i = 0; i < dk; ++i) a += (double)at[i] * (double)at[i];
        a /= (double)dk;
        const double bh = a * bcov + w / (double)dk;
        double n = 0.0;
        for (int i = 0; i < dk; ++i) n += (double)kt[i] * (double)kt[i];
        /* scalar gain beta = b_hat / (r + b_hat |k|^2), kappa = beta k */
        const double beta = bh / (rt + bh * n);
        /* predicted mean diag(alpha) S, innovation, residual write */
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += (double)at[i] * S[(size_t)i * dv + j] * (double)kt[i];
            delta[j] = (double)vt[j] - pred;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = (double)at[i] * S[(size_t)i * dv + j] + beta * (double)kt[i] * delta[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * (double)qt[i];
            o[tok * dv + j] = acc;
        }
        /* posterior: precision increment (mu/r)|k|^2 averaged over d_k channels */
        bcov = bh / (1.0 + (mu / ((double)dk * rt)) * n * bh);
        if (tr_phat) tr_phat[tok] = bh;
        if (tr_kappa) for (int i = 0; i < dk; ++i) tr_kappa[tok * dk + i] = beta * (double)kt[i];
        if (tr_p) tr_p[tok] = bcov;
    }
    if (p_T) p_T[state] = bcov;
    if (S_T)
        for (size_t e = 0; e < (size_t)dk * dv; ++e) S_T[state * (size_t)dk * dv + e] = S[e];
    free(S); free(delta);
}

typedef void (*head_fn)(int, int, int, int, int, int, const double*, const double*, const double*,
                        const double*, const double*, const double*, const double*, double,
                        const double*, const double*, double*, double*, double*, double*,
                        double*, double*);

static int run_heads(head_fn fn, int B, int T, int H, int dk, int dv,
                     const double* q, const double* k, const double* v, const double* alpha,
                     const double* omega, const double* r, const double* c0, double mu,
                     const double* S0, const double* p0, double* o, double* S_T, double* p_T,
                     double* tr_phat, double* tr_kappa, double* tr_p) {
    if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return 1;
    if (!q || !k || !v || !alpha || !omega || !r || !o) return 1;
    if (!c0 && !p0) return 1;
    const long units = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u)
        fn((int)(u / H), (int)(u % H), T, H, dk, dv, q, k, v, alpha, omega, r, c0, mu, S0, p0,
           o, S_T, p_T, tr_phat, tr_kappa, tr_p);
    return 0;
}

int kdn_oracle_forward_diag(int B, int T, int H, int dk, int dv,
                            const double* q, const double* k, const double* v,
                            const double* alpha, const double* omega, const double* r,
                            const double* c0, double mu, const double* S0, const double* p0,
                            double* o, double* S_T, double* p_T,
                            double* tr_phat, double* tr_kappa, double* tr_p) {
    return run_heads(diag_head, B, T, H, dk, dv, q, k, v, alpha, omega, r, c0, mu, S0, p0,
                     o, S_T, p_T, tr_phat, tr_kappa, tr_p);
}

int kdn_oracle_forward_iso(int B, int T, int H, int dk, int dv,
                           const double* q, const double* k, const double* v,
                           const double* alpha, const double* omega, const double* r,
                           const double* c0, double mu, const double* S0, const double* p0,
                           double* o, double* S_T, double* p_T,
                           double* tr_phat, double* tr_kappa, double* tr_p) {
    return run_heads(iso_head, B, T, H, dk, dv, q, k, v, alpha, omega, r, c0, mu, S0, p0,
                     o, S_T, p_T, tr_phat, tr_kappa, tr_p);
}

int kdn_oracle_forward_isoc(int B, int T, int H, int dk, int dv,
                            const double* q, const double* k, const double* v,
                            const double* alpha, const double* omega, const double* r,
                            const double* c0, double mu, const double* S0, const double* p0,
                            double* o, double* S_T, double* p_T,
                            double* tr_phat, double* tr_kappa, double* tr_p) {
    return run_heads(isoc_head, B, T, H, dk, dv, q, k, v, alpha, omega, r, c0, mu, S0, p0,
                     o, S_T, p_T, tr_phat, tr_kappa, tr_p);
}

/*
 * Single-token decode step: exactly one iteration of the recurrence on the
 * carried state (S, p), for N independent sequences.  S [N,H,dk,dv] and
 * p [N,H,dk] (isotropic [N,H]) are read and overwritten in place; token
 * inputs use the forward layouts with T = 1.
 */
static int step_common(head_fn fn, int pdim, int N, int H, int dk, int dv,
                       const double* q, const double* k, const double* v, const double* alpha,
                       const double* omega, const double* r, double mu, double* S, double* p,
                       double* o) {
    if (!S || !p) return 1;
    const size_t ns = (size_t)N * H * dk * dv, np_ = (size_t)N * H * pdim;
    double* S_in = (double*)malloc(sizeof(double) * (ns ? ns : 1));
    double* p_in = (double*)malloc(sizeof(double) * (np_ ? np_ : 1));
    memcpy(S_in, S, sizeof(double) * ns);
    memcpy(p_in, p, sizeof(double) * np_);
    const int rc = run_heads(fn, N, 1, H, dk, dv, q, k, v, alpha, omega, r, NULL, mu, S_in, p_in,
                             o, S, p, NULL, NULL, NULL);
    free(S_in); free(p_in);
    return rc;
}

int kdn_oracle_step_diag(int N, int H, int dk, int dv, const double* q, const double* k,
                         const double* v, const double* alpha, const double* omega, const double* r,
                         double mu, double* S, double* p, double* o) {
    return step_common(diag_head, dk, N, H, dk, dv, q, k, v, alpha, omega, r, mu, S, p, o);
}

int kdn_oracle_step_iso(int N, int H, int dk, int dv, const double* q, const double* k,
                        const double* v, const double* alpha, const double* omega, const double* r,
                        double mu, double* S, double* p, double* o) {
    return step_common(iso_head, 1, N, H, dk, dv, q, k, v, alpha, omega, r, mu, S, p, o);
}

int kdn_oracle_step_isoc(int N, int H, int dk, int dv, const double* q, const double* k,
                         const double* v, const double* alpha, const double* omega, const double* r,
                         double mu, double* S, double* p, double* o) {
    return step_common(isoc_head, 1, N, H, dk, dv, q, k, v, alpha, omega, r, mu, S, p, o);
}

/* Number of OpenMP threads the oracle's parallel loops use. */
#ifdef _OPENMP
#include <omp.h>
#endif
int kdn_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of OpenMP threads of the oracle's parallel loops (n >= 1). */
void kdn_oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Backward pass (reverse-mode adjoint of the recurrence above), for training.
 *
 * For cotangents dO [B,T,H,dv], dS_T [B,H,dk,dv] and dp_T [B,H,dk]
 * (isotropic forms [B,H]), both nullable (= 0), the scalar being
 * differentiated is
 *     L = sum dO (.) o + sum dS_T (.) S_T + sum dp_T (.) p_T,
 * and the outputs are dL/d(q, k, v, alpha, omega, r) in the input layouts,
 * dL/dS0 [B,H,dk,dv] and dL/dp0 [B,H,dk] (isotropic [B,H]).  When p0 is NULL
 * (p_0 = c0[h] on every channel) dL/dc0[h] is the sum of dL/dp0 over the
 * batch and the channels; dc0 [H] receives that sum in every case.
 *
 * Plain two-sweep form: a forward sweep stores every pre-token memory
 * S_{t-1} and uncertainty p_{t-1}; the reverse sweep walks t = T-1 .. 0 and
 * applies the chain rule to each equation of the token step in reverse
 * order (readout, residual write, predicted mean, gain, posterior,
 * predict).  `var` is 0 diagonal, 1 isotropic, 2 isotropic with
 * per-channel decay.
 */
static void backward_head(int var, int b, int h, int T, int H, int dk, int dv,
                          const double* q, const double* k, const double* v,
                          const double* alpha, const double* omega, const double* r,
                          const double* c0, double mu, const double* S0, const double* p0,
                          const double* dO, const double* dS_T, const double* dp_T,
                          double* dq, double* dkk, double* dvv, double* dalpha,
                          double* domega, double* dr, double* dS0, double* dp0) {
    const size_t state = ((size_t)b * H + h);
    const size_t SZ = (size_t)dk * dv;
    const int pd = var == 0 ? dk : 1;                  /* uncertainty entries */
    const int ad = var == 1 ? 1 : dk;                  /* decay entries per token */
    const int wd = var == 0 ? dk : 1;                  /* process-noise entries */
    double* Sall = (double*)malloc(sizeof(double) * SZ * ((size_t)T + 1));
    double* pall = (double*)malloc(sizeof(double) * (size_t)pd * ((size_t)T + 1));
    double* Sh = (double*)malloc(sizeof(double) * SZ);
    double* dS = (double*)malloc(sizeof(double) * SZ);
    double* dSh = (double*)malloc(sizeof(double) * SZ);
    double* ph = (double*)malloc(sizeof(double) * dk);
    double* kap = (double*)malloc(sizeof(double) * dk);
    double* dkap = (double*)malloc(sizeof(double) * dk);
    double* dp = (double*)malloc(sizeof(double) * pd);
    double* delta = (double*)malloc(sizeof(double) * dv);
    double* ddel = (double*)malloc(sizeof(double) * dv);

    /* ---- forward sweep: store S_{t-1}, p_{t-1} for every token ---- */
    for (size_t e = 0; e < SZ; ++e) Sall[e] = S0 ? S0[state * SZ + e] : 0.0;
    for (int i = 0; i < pd; ++i) pall[i] = p0 ? p0[state * pd + i] : c0[h];
    for (int t = 0; t < T; ++t) {
        const size_t tok = IDX_TOK(b, t, h, 0, T, H);
        const double* kt = k + tok * dk;
        const double* at = alpha + tok * ad;
        const double rt = r[tok];
        const double* S = Sall + SZ * t;
        double* Sn = Sall + SZ * (t + 1);
        const double* p = pall + (size_t)pd * t;
        double* pn = pall + (size_t)pd * (t + 1);
        if (var == 0) {
            double s = 0.0;
            for (int i = 0; i < dk; ++i) {
                ph[i] = at[i] * at[i] * p[i] + omega[tok * dk + i];
                s += ph[i] * kt[i] * kt[i];
            }
            for (int i = 0; i < dk; ++i) kap[i] = ph[i] * kt[i] / (rt + s);
            for (int i = 0; i < dk; ++i) pn[i] = ph[i] / (1.0 + (mu / rt) * kt[i] * kt[i] * ph[i]);
        } else {
            double a = 0.0, n = 0.0;
            if (var == 1) a = at[0] * at[0];
            else { for (int i = 0; i < dk; ++i) a += at[i] * at[i]; a /= dk; }
            for (int i = 0; i < dk; ++i) n += kt[i] * kt[i];
            const double bh = a * p[0] + omega[tok] / dk;
            const double beta = bh / (rt + bh * n);
            for (int i = 0; i < dk; ++i) kap[i] = beta * kt[i];
            pn[0] = bh / (1.0 + (mu / ((double)dk * rt)) * n * bh);
        }
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += at[var == 1 ? 0 : i] * S[(size_t)i * dv + j] * kt[i];
            delta[j] = v[tok * dv + j] - pred;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sn[(size_t)i * dv + j] = at[var == 1 ? 0 : i] * S[(size_t)i * dv + j] + kap[i] * delta[j];
    }

    /* ---- reverse sweep ---- */
    for (size_t e = 0; e < SZ; ++e) dS[e] = dS_T ? dS_T[state * SZ + e] : 0.0;
    for (int i = 0; i < pd; ++i) dp[i] = dp_T ? dp_T[state * pd + i] : 0.0;
    for (int t = T - 1; t >= 0; --t) {
        const size_t tok = IDX_TOK(b, t, h, 0, T, H);
        const double* kt = k + tok * dk;
        const double* qt = q + tok * dk;
        const double* at = alpha + tok * ad;
        const double* dot = dO ? dO + tok * dv : NULL;
        const double rt = r[tok];
        const double* S = Sall + SZ * t;        /* S_{t-1} */
        const double* Sn = Sall + SZ * (t + 1); /* S_t, the memory read out at t */
        const double* p = pall + (size_t)pd * t;
        const double* pn = pall + (size_t)pd * (t + 1);

        /* recompute the token's forward quantities from S_{t-1}, p_{t-1} */
        double s = 0.0, n = 0.0, a = 0.0, bh = 0.0, beta = 0.0;
        if (var == 0) {
            for (int i = 0; i < dk; ++i) {
                ph[i] = at[i] * at[i] * p[i] + omega[tok * dk + i];
                s += ph[i] * kt[i] * kt[i];
            }
            for (int i = 0; i < dk; ++i) kap[i] = ph[i] * kt[i] / (rt + s);
        } else {
            if (var == 1) a = at[0] * at[0];
            else { for (int i = 0; i < dk; ++i) a += at[i] * at[i]; a /= dk; }
            for (int i = 0; i < dk; ++i) n += kt[i] * kt[i];
            bh = a * p[0] + omega[tok] / dk;
            beta = bh / (rt + bh * n);
            for (int i = 0; i < dk; ++i) kap[i] = beta * kt[i];
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) Sh[(size_t)i * dv + j] = at[var == 1 ? 0 : i] * S[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += Sh[(size_t)i * dv + j] * kt[i];
            delta[j] = v[tok * dv + j] - pred;
        }

        /* readout o = S_t^T q */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                const double g = dot ? dot[j] : 0.0;
                acc += Sn[(size_t)i * dv + j] * g;
                dS[(size_t)i * dv + j] += qt[i] * g;
            }
            dq[tok * dk + i] = acc;
        }
        /* residual write S_t = S_hat + kappa delta^T, delta = v - S_hat^T k */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += dS[(size_t)i * dv + j] * kap[i];
            ddel[j] = acc;
            dvv[tok * dv + j] = acc;
        }
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0, acck = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += dS[(size_t)i * dv + j] * delta[j];
                dSh[(size_t)i * dv + j] = dS[(size_t)i * dv + j] - kt[i] * ddel[j];
                acck -= Sh[(size_t)i * dv + j] * ddel[j];
            }
            dkap[i] = acc;
            dkk[tok * dk + i] = acck;
        }
        /* predicted mean S_hat = diag(alpha) S_{t-1} (scalar alpha: alpha S_{t-1}) */
        double dasum = 0.0;
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += S[(size_t)i * dv + j] * dSh[(size_t)i * dv + j];
                dS[(size_t)i * dv + j] = at[var == 1 ? 0 : i] * dSh[(size_t)i * dv + j];
            }
            if (var == 1) dasum += acc;
            else dalpha[tok * dk + i] = acc;
        }

        if (var == 0) {
            /* gain kappa_i = p_hat_i k_i / d, d = r + sum p_hat k^2;
             * posterior p_i = p_hat_i / (1 + u_i p_hat_i), u_i = (mu/r) k_i^2;
             * predict p_hat = alpha^2 p + omega */
            const double d = rt + s;
            double dd = 0.0, drr = 0.0;
            for (int i = 0; i < dk; ++i) dd -= dkap[i] * kap[i] / d;
            for (int i = 0; i < dk; ++i) {
                const double u = (mu / rt) * kt[i] * kt[i];
                const double den = 1.0 + u * ph[i];
                const double du = -dp[i] * pn[i] * pn[i];
                const double dph = dp[i] / (den * den) + dkap[i] * kt[i] / d + dd * kt[i] * kt[i];
                drr += du * (-mu * kt[i] * kt[i] / (rt * rt));
                dkk[tok * dk + i] += dkap[i] * ph[i] / d + 2.0 * dd * ph[i] * kt[i]
                                     + 2.0 * du * (mu / rt) * kt[i];
                dalpha[tok * dk + i] += 2.0 * dph * at[i] * p[i];
                domega[tok * dk + i] = dph;
                dp[i] = dph * at[i] * at[i];
            }
            dr[tok] = dd + drr;
        } else {
            /* gain beta = b_hat / (r + b_hat n), n = |k|^2, kappa = beta k;
             * posterior b = b_hat / (1 + c n b_hat), c = mu / (d_k r);
             * predict b_hat = a b + omega / d_k */
            const double dg = rt + bh * n;
            const double c = mu / ((double)dk * rt);
            const double dpn = 1.0 + c * n * bh;
            const double bt = pn[0];
            double dbeta = 0.0;
            for (int i = 0; i < dk; ++i) dbeta += dkap[i] * kt[i];
            const double dbh = dbeta * rt / (dg * dg) + dp[0] / (dpn * dpn);
            const double dn = dbeta * (-bh * bh / (dg * dg)) - dp[0] * bt * bt * c;
            dr[tok] = dbeta * (-bh / (dg * dg)) + dp[0] * bt * bt * c * n / rt;
            for (int i = 0; i < dk; ++i) dkk[tok * dk + i] += beta * dkap[i] + 2.0 * dn * kt[i];
            if (var == 1) dalpha[tok] = dasum + 2.0 * dbh * at[0] * p[0];
            else for (int i = 0; i < dk; ++i) dalpha[tok * dk + i] += dbh * p[0] * 2.0 * at[i] / dk;
            domega[tok] = dbh / dk;
            dp[0] = dbh * a;
        }
    }
    for (size_t e = 0; e < SZ; ++e) dS0[state * SZ + e] = dS[e];
    for (int i = 0; i < pd; ++i) dp0[state * pd + i] = dp[i];
    free(Sall); free(pall); free(Sh); free(dS); free(dSh); free(ph); free(kap); free(dkap);
    free(dp); free(delta); free(ddel);
}

int kdn_oracle_backward(int var, int B, int T, int H, int dk, int dv,
                        const double* q, const double* k, const double* v,
                        const double* alpha, const double* omega, const double* r,
                        const double* c0, double mu, const double* S0, const double* p0,
                        const double* dO, const double* dS_T, const double* dp_T,
                        double* dq, double* dk_out, double* dv_out, double* dalpha,
                        double* domega, double* dr, double* dS0, double* dp0, double* dc0) {
    if (var < 0 || var > 2 || B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return 1;
    if (!q || !k || !v || !alpha || !omega || !r || (!c0 && !p0)) return 1;
    if (!dq || !dk_out || !dv_out || !dalpha || !domega || !dr || !dS0 || !dp0 || !dc0) return 1;
    const long units = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u)
        backward_head(var, (int)(u / H), (int)(u % H), T, H, dk, dv, q, k, v, alpha, omega, r, c0,
                      mu, S0, p0, dO, dS_T, dp_T, dq, dk_out, dv_out, dalpha, domega, dr, dS0, dp0);
    const int pd = var == 0 ? dk : 1;
    for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int b = 0; b < B; ++b)
            for (int i = 0; i < pd; ++i) acc += dp0[((size_t)b * H + h) * pd + i];
        dc0[h] = acc;
    }
    return 0;
}
