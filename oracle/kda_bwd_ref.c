/*
 * kda_bwd_ref.c -- fp64 CPU oracle for the gradients of the KDA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/ may load this library (it is built into the
 * same libkda_oracle.so as kda_ref.c).  It shares no code with the HIP library.
 *
 * What it computes.  The forward pass is the token recurrence of kda_ref.c (FlashKDA
 * README "Kernel API" table and the FLA-backend flags; article index "Delta Attention
 * Algorithm: linear-time recurrence"), per (sequence, head) chain, per token t:
 *   q^ = q / n_q, n_q = sqrt(|q|^2 + 1e-6);  k^ likewise         (l2norm switch)
 *   x_c = exp(A_log) (g_c + dt_bias_c), a_c = lb sigmoid(x_c)      (gate switch)
 *   alpha = exp(a);  beta = sigmoid(beta_logit)                    (sigmoid switch)
 *   S' = S_{t-1} Diag(alpha);  r = v - S' k^;  S_t = S' + beta r k^T;  o_t = scale S_t q^
 * The pages state no backward pass (the news digest: "forward pass only, no backward
 * yet"); this file is the reverse-mode derivative of that recurrence, written from the
 * chain rule.  Given dL/do_t (dout) and dL/dS_T (dht, or zero), with D = dL/dS_t:
 *   D  += scale do_t q^^T                          (read-out)
 *   dq^ = scale S_t^T do_t
 *   u   = D k^;  dv_t = beta u;  dbeta = u . r
 *   dk^ = beta (D^T r - S'^T u)
 *   dS' = D - beta u k^T
 *   dalpha_c = sum_v S_{t-1}[v][c] dS'[v][c];  D <- dS' Diag(alpha)   (the state before t)
 * and through the activations:
 *   da = dalpha alpha;  dx = da lb s (1 - s), s = sigmoid(x);  dg = dx exp(A_log);
 *   d dt_bias_c += dx_c exp(A_log);  dA_log += sum_c dx_c x_c;
 *   gate switch off (a = min(max(g, lb), 0)): dg = da where lb < g < 0, else 0;
 *   dbeta_logit = dbeta beta (1 - beta)  (sigmoid switch off: dbeta itself);
 *   dq = (dq^ - q^ (q^ . dq^)) / n_q     (l2norm switch off: dq^ itself), dk likewise.
 * dh0 = D after the first token.  dA_log and dt_bias gradients are summed over the
 * sequences (and tokens).  Every quantity is double; inputs are widened exactly.
 *
 * Pins (tests/test_oracle_bwd.py): the core derivative against exact forward-mode
 * derivatives in rational arithmetic (dual numbers over fractions.Fraction), the full
 * derivative against central finite differences of the forward oracle, closed forms
 * (pure decay with beta = 0), and the forward values it recomputes against kda_ref.c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BWD_DIM 128
#define BWD_EPS 1e-6
#define BWD_GATE_IN 1
#define BWD_L2_IN 2
#define BWD_SIG_IN 4

static double bwd_bf16(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double bwd_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * Reverse mode of the core recurrence (already-activated inputs, any K and V).
 *   alpha, kn, qn: [T][K]; beta: [T]; v: [T][V]; S0: [V][K]; dout: [T][V]; dST: [V][K] or NULL.
 *   Outputs (overwritten): dalpha, dkn, dqn [T][K]; dbeta [T]; dv [T][V]; dS0 [V][K].
 *   out (optional, [T][V]): the forward read-out, recomputed.
 * Returns 0, or 1 on bad sizes, 2 if memory runs out.
 */
int oracle_core_bwd(int64_t T, int64_t K, int64_t V, const double *alpha, const double *beta,
                    const double *kn, const double *qn, const double *v, double scale, const double *S0,
                    const double *dout, const double *dST, double *dalpha, double *dbeta, double *dkn,
                    double *dqn, double *dv, double *dS0, double *out)
{
    if (T < 0 || K < 1 || V < 1)
        return 1;
    const int64_t VK = V * K;
    /* states[t] = S_t, the state after t tokens (states[0] = S0) */
    double *states = (double *)malloc(sizeof(double) * (size_t)(T + 1) * (size_t)VK);
    double *Sp = (double *)malloc(sizeof(double) * (size_t)VK);
    double *D = (double *)malloc(sizeof(double) * (size_t)VK);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    if (!states || !Sp || !D || !r || !u) {
        free(states); free(Sp); free(D); free(r); free(u);
        return 2;
    }
    memcpy(states, S0, sizeof(double) * (size_t)VK);
    for (int64_t t = 0; t < T; ++t) {
        const double *Sprev = states + t * VK;
        double *S = states + (t + 1) * VK;
        const double *al = alpha + t * K, *kt = kn + t * K, *qt = qn + t * K, *vt = v + t * V;
        for (int64_t i = 0; i < V; ++i) {
            double pred = 0.0;
            for (int64_t c = 0; c < K; ++c)
                pred += Sprev[i * K + c] * al[c] * kt[c];
            const double ri = vt[i] - pred;
            for (int64_t c = 0; c < K; ++c)
                S[i * K + c] = Sprev[i * K + c] * al[c] + beta[t] * ri * kt[c];
        }
        if (out)
            for (int64_t i = 0; i < V; ++i) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c)
                    acc += S[i * K + c] * qt[c];
                out[t * V + i] = scale * acc;
            }
    }
    for (int64_t e = 0; e < VK; ++e)
        D[e] = dST ? dST[e] : 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
        const double *Sprev = states + t * VK;
        const double *S = states + (t + 1) * VK;
        const double *al = alpha + t * K, *kt = kn + t * K, *qt = qn + t * K, *vt = v + t * V;
        const double *dot = dout + t * V;
        const double bt = beta[t];
        /* forward quantities of token t */
        for (int64_t i = 0; i < V; ++i) {
            double pred = 0.0;
            for (int64_t c = 0; c < K; ++c) {
                Sp[i * K + c] = Sprev[i * K + c] * al[c];
                pred += Sp[i * K + c] * kt[c];
            }
            r[i] = vt[i] - pred;
        }
        /* read-out: o_t = scale S_t q^ */
        for (int64_t c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < V; ++i)
                acc += S[i * K + c] * dot[i];
            dqn[t * K + c] = scale * acc;
        }
        for (int64_t i = 0; i < V; ++i)
            for (int64_t c = 0; c < K; ++c)
                D[i * K + c] += scale * dot[i] * qt[c];
        /* delta-rule write: S_t = S' + beta r k^T, r = v - S' k^ */
        double db = 0.0;
        for (int64_t i = 0; i < V; ++i) {
            double acc = 0.0;
            for (int64_t c = 0; c < K; ++c)
                acc += D[i * K + c] * kt[c];
            u[i] = acc;
            dv[t * V + i] = bt * acc;
            db += acc * r[i];
        }
        dbeta[t] = db;
        for (int64_t c = 0; c < K; ++c) {
            double a1 = 0.0, a2 = 0.0;
            for (int64_t i = 0; i < V; ++i) {
                a1 += D[i * K + c] * r[i];
                a2 += Sp[i * K + c] * u[i];
            }
            dkn[t * K + c] = bt * (a1 - a2);
        }
        /* dS' = D - beta u k^T; decay: S' = S_{t-1} Diag(alpha) */
        for (int64_t c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < V; ++i) {
                const double dsp = D[i * K + c] - bt * u[i] * kt[c];
                acc += Sprev[i * K + c] * dsp;
                D[i * K + c] = dsp * al[c];
            }
            dalpha[t * K + c] = acc;
        }
    }
    memcpy(dS0, D, sizeof(double) * (size_t)VK);
    free(states); free(Sp); free(D); free(r); free(u);
    return 0;
}

/*
 * Gradients of the full forward pass (same argument meaning and layouts as oracle_kda_fwd
 * in kda_ref.c), host memory.
 *   dout: bf16 bits [B*T][H][128] (dL/dout); dht: NULL or fp32 [N][H][128][128] (dL/dfinal_state)
 *   Outputs (double, overwritten): dq, dk, dv, dg [B*T][H][128]; dbeta [B*T][H];
 *   dA_log [H]; ddt_bias [H][128] (both zero with the gate switch off);
 *   dh0 [N][H][128][128] (NULL = not written).
 * Returns 0 on success, nonzero on an argument error or when memory runs out.
 */
int oracle_kda_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                   const uint16_t *beta, double scale, const float *A_log, const float *dt_bias,
                   double lower_bound, int flags, const void *initial_state, int state_dtype,
                   const int64_t *cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t N,
                   const uint16_t *dout, const float *dht, double *dq, double *dk, double *dv,
                   double *dg, double *dbeta, double *dA_log, double *ddt_bias, double *dh0,
                   int nthreads)
{
    const int64_t D = BWD_DIM;
    if (B < 1 || T < 0 || H < 1 || (flags & ~7) != 0)
        return 1;
    if (cu_seqlens) {
        if (B != 1 || N < 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T)
            return 2;
        for (int64_t i = 0; i < N; ++i)
            if (cu_seqlens[i + 1] < cu_seqlens[i])
                return 2;
    } else {
        N = B;
    }
    if ((flags & BWD_GATE_IN) && (!A_log || !dt_bias))
        return 3;
    const int64_t n_chains = N * H;
    /* per-chain partial sums of the head parameters' gradients, summed in order below */
    double *pA = (double *)calloc((size_t)n_chains, sizeof(double));
    double *pdt = (double *)calloc((size_t)n_chains * D, sizeof(double));
    if (!pA || !pdt) {
        free(pA); free(pdt);
        return 4;
    }
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t chain = 0; chain < n_chains; ++chain) {
        const int64_t n = chain / H, h = chain % H;
        const int64_t t0 = cu_seqlens ? cu_seqlens[n] : n * T;
        const int64_t L = (cu_seqlens ? cu_seqlens[n + 1] : (n + 1) * T) - t0;
        const size_t LD = (size_t)(L > 0 ? L : 1) * D;
        double *alpha = malloc(sizeof(double) * LD), *kn = malloc(sizeof(double) * LD);
        double *qn = malloc(sizeof(double) * LD), *vv = malloc(sizeof(double) * LD);
        double *dd = malloc(sizeof(double) * LD), *bt = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *dalpha = malloc(sizeof(double) * LD), *dkn = malloc(sizeof(double) * LD);
        double *dqn = malloc(sizeof(double) * LD), *dvv = malloc(sizeof(double) * LD);
        double *dbt = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *nq = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1)), *nk = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *S0 = malloc(sizeof(double) * D * D), *dST = malloc(sizeof(double) * D * D);
        double *dS0 = malloc(sizeof(double) * D * D);
        if (!alpha || !kn || !qn || !vv || !dd || !bt || !dalpha || !dkn || !dqn || !dvv || !dbt || !nq ||
            !nk || !S0 || !dST || !dS0) {
            failed = 1;
        } else {
            const double eA = (flags & BWD_GATE_IN) ? exp((double)A_log[h]) : 0.0;
            for (int64_t s = 0; s < L; ++s) {
                const int64_t row = ((t0 + s) * H + h) * D;
                double ssq = 0.0, ssk = 0.0;
                for (int64_t c = 0; c < D; ++c) {
                    const double qc = bwd_bf16(q[row + c]), kc = bwd_bf16(k[row + c]);
                    ssq += qc * qc;
                    ssk += kc * kc;
                }
                nq[s] = (flags & BWD_L2_IN) ? sqrt(ssq + BWD_EPS) : 1.0;
                nk[s] = (flags & BWD_L2_IN) ? sqrt(ssk + BWD_EPS) : 1.0;
                for (int64_t c = 0; c < D; ++c) {
                    qn[s * D + c] = bwd_bf16(q[row + c]) / nq[s];
                    kn[s * D + c] = bwd_bf16(k[row + c]) / nk[s];
                    vv[s * D + c] = bwd_bf16(v[row + c]);
                    dd[s * D + c] = bwd_bf16(dout[row + c]);
                    const double gc = bwd_bf16(g[row + c]);
                    double a;
                    if (flags & BWD_GATE_IN) {
                        a = lower_bound * bwd_sigmoid(eA * (gc + (double)dt_bias[h * D + c]));
                    } else {
                        a = gc < lower_bound ? lower_bound : gc;
                        a = a > 0.0 ? 0.0 : a;
                    }
                    alpha[s * D + c] = exp(a);
                }
                const double braw = bwd_bf16(beta[(t0 + s) * H + h]);
                bt[s] = (flags & BWD_SIG_IN) ? bwd_sigmoid(braw) : braw;
            }
            for (int64_t e = 0; e < D * D; ++e) {
                double s0 = 0.0;
                if (initial_state) {
                    const int64_t idx = (n * H + h) * D * D + e;
                    if (state_dtype == 1)
                        s0 = bwd_bf16(((const uint16_t *)initial_state)[idx]);
                    else if (state_dtype == 2)
                        s0 = (double)((const float *)initial_state)[idx];
                    else if (state_dtype == 3)
                        s0 = ((const double *)initial_state)[idx];
                }
                S0[e] = s0;
                dST[e] = dht ? (double)dht[(n * H + h) * D * D + e] : 0.0;
            }
            if (oracle_core_bwd(L, D, D, alpha, bt, kn, qn, vv, scale, S0, dd, dST, dalpha, dbt, dkn, dqn,
                                dvv, dS0, NULL) != 0) {
                failed = 1;
            } else {
                for (int64_t s = 0; s < L; ++s) {
                    const int64_t row = ((t0 + s) * H + h) * D;
                    /* l2norm: dq = (dq^ - q^ (q^ . dq^)) / n */
                    double pq = 0.0, pk = 0.0;
                    for (int64_t c = 0; c < D; ++c) {
                        pq += qn[s * D + c] * dqn[s * D + c];
                        pk += kn[s * D + c] * dkn[s * D + c];
                    }
                    for (int64_t c = 0; c < D; ++c) {
                        if (flags & BWD_L2_IN) {
                            dq[row + c] = (dqn[s * D + c] - qn[s * D + c] * pq) / nq[s];
                            dk[row + c] = (dkn[s * D + c] - kn[s * D + c] * pk) / nk[s];
                        } else {
                            dq[row + c] = dqn[s * D + c];
                            dk[row + c] = dkn[s * D + c];
                        }
                        dv[row + c] = dvv[s * D + c];
                        /* gate: da = dalpha alpha */
                        const double da = dalpha[s * D + c] * alpha[s * D + c];
                        const double gc = bwd_bf16(g[row + c]);
                        if (flags & BWD_GATE_IN) {
                            const double x = eA * (gc + (double)dt_bias[h * D + c]);
                            const double sg = bwd_sigmoid(x);
                            const double dx = da * lower_bound * sg * (1.0 - sg);
                            dg[row + c] = dx * eA;
                            pdt[chain * D + c] += dx * eA;
                            pA[chain] += dx * x;
                        } else {
                            dg[row + c] = (gc > lower_bound && gc < 0.0) ? da : 0.0;
                        }
                    }
                    dbeta[(t0 + s) * H + h] = (flags & BWD_SIG_IN) ? dbt[s] * bt[s] * (1.0 - bt[s]) : dbt[s];
                }
                if (dh0)
                    memcpy(dh0 + (n * H + h) * D * D, dS0, sizeof(double) * D * D);
            }
        }
        free(alpha); free(kn); free(qn); free(vv); free(dd); free(bt); free(dalpha); free(dkn);
        free(dqn); free(dvv); free(dbt); free(nq); free(nk); free(S0); free(dST); free(dS0);
    }
    for (int64_t h = 0; h < H; ++h) {
        double a = 0.0;
        for (int64_t n = 0; n < N; ++n)
            a += pA[n * H + h];
        dA_log[h] = a;
        for (int64_t c = 0; c < D; ++c) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                s += pdt[(n * H + h) * D + c];
            ddt_bias[h * D + c] = s;
        }
    }
    free(pA);
    free(pdt);
    return failed ? 5 : 0;
}
