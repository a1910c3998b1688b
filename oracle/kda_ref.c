/*
 * kda_ref.c -- fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two are built separately.
 *
 * What it computes (token by token, one (sequence, head) chain at a time):
 *
 *   Sources.  "MoonshotAI/FlashKDA" repository page, README section "Kernel API"
 *   (argument table: q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
 *   initial_state, final_state, cu_seqlens; K = V = 128; state layout [.., V, K];
 *   dtype-match and varlen rules), README section "Using FlashKDA as an FLA
 *   backend" (flags use_gate_in_kernel, use_qk_l2norm_in_kernel,
 *   use_beta_sigmoid_in_kernel, safe_gate, transpose_state_layout), and the
 *   FlashKDA article index page ("Delta Attention Algorithm: linear-time
 *   recurrence", "lower_bound parameter", "Sigmoid in its gating path").
 *
 *   The pages print no formula.  The readings taken (each also listed in the
 *   design notes) are:
 *     1. q^ = q / sqrt(|q|^2 + 1e-6), k^ likewise           (l2norm flag; eps unpinned)
 *     2. a_c = lb * sigmoid(exp(A_log[h]) * (g_c + dt_bias[h,c]))   (gate reading R1;
 *        range (lb, 0] as the Kernel API table states for lower_bound)
 *        alpha_c = exp(a_c)
 *     3. beta = sigmoid(beta_logit)                           (Kernel API table, beta row)
 *     4. S[v][c] <- S[v][c] * alpha_c                          (decay first)
 *     5. r_v = v_t[v] - sum_c S[v][c] k^_c
 *     6. S[v][c] <- S[v][c] + beta * r_v * k^_c               (delta-rule write)
 *     7. out_t[v] = scale * sum_c S[v][c] q^_c                 (inclusive: sees token t)
 *   Equivalently S_t = S_{t-1} Diag(alpha_t) (I - beta_t k^ k^T) + beta_t v_t k^T.
 *
 *   Activation switches (the three use_*_in_kernel flags of the "Using FlashKDA as an
 *   FLA backend" section; the pages only name them).  With a switch off the library
 *   takes that input as already activated:
 *     gate off:   a_c = min(max(g_c, lb), 0)   (g holds the natural-log decay itself; A_log
 *                 and dt_bias are unused; it is held to the same range (lb, 0] the in-kernel
 *                 gate produces, the reading of safe_gate together with lower_bound)
 *     l2norm off: q^ = q, k^ = k as given
 *     sigmoid off: beta = beta as given
 *
 *   Inputs arrive as bf16 bit patterns (uint16) or fp32 and are widened exactly
 *   to double; every intermediate is double; nothing is rounded on the way out.
 *
 * Parity pins (tests/test_oracle_*.py): exact-rational brute force of steps 4-7,
 * dense 128x128 transition products, chunk-size independence of an independent
 * chunked form, beta = 0 pure-decay closed form, q = k / beta = 1 retrieval,
 * orthonormal-key overwrite, varlen = separate runs, split-and-resume, linearity,
 * gate and l2norm special values, and for the switches an exact-rational run with
 * every switch off and a pure-decay closed form of the pre-activated gate.  The gate
 * formula, eps, the decay/update order and the meaning of a switch that is off are
 * readings the pages do not pin ("parity unpinned" for those choices).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DIM 128
#define ORACLE_EPS 1e-6

/* activation switches: bit values of the forward pass's switch mask */
#define ORACLE_GATE_IN_KERNEL 1
#define ORACLE_QK_L2NORM_IN_KERNEL 2
#define ORACLE_BETA_SIGMOID_IN_KERNEL 4

enum { ORACLE_STATE_NONE = 0, ORACLE_STATE_BF16 = 1, ORACLE_STATE_FP32 = 2, ORACLE_STATE_FP64 = 3 };

/* bf16 bit pattern -> double, exact (bf16 is the upper half of an fp32). */
static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/* Log-decay of one channel (reading R1): lb * sigmoid(exp(A_log) * (g + dt_bias)). */
double oracle_gate(double g, double A_log, double dt_bias, double lower_bound)
{
    return lower_bound * oracle_sigmoid(exp(A_log) * (g + dt_bias));
}

/* Pre-activated gate (gate switch off): the given log-decay held to [lb, 0]. */
double oracle_gate_preactivated(double g, double lower_bound)
{
    double a = g < lower_bound ? lower_bound : g;
    return a > 0.0 ? 0.0 : a;
}

/* y = x / sqrt(sum x^2 + eps) */
void oracle_l2norm(const double *x, int64_t n, double eps, double *y)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int64_t i = 0; i < n; ++i)
        y[i] = x[i] * inv;
}

/*
 * Steps 4-7 for one chain with already-activated inputs, any K and V.
 *   alpha, kn, qn: [T][K]; beta: [T]; v: [T][V]; S: [V][K] in/out; out: [T][V] (may be NULL).
 */
int oracle_core(int64_t T, int64_t K, int64_t V, const double *alpha, const double *beta,
                const double *kn, const double *qn, const double *v, double scale, double *S,
                double *out)
{
    if (T < 0 || K < 1 || V < 1)
        return 1;
    for (int64_t t = 0; t < T; ++t) {
        const double *al = alpha + t * K;
        const double *kt = kn + t * K;
        const double *qt = qn + t * K;
        const double *vt = v + t * V;
        const double bt = beta[t];
        /* step 4: decay along the key channels */
        for (int64_t i = 0; i < V; ++i)
            for (int64_t c = 0; c < K; ++c)
                S[i * K + c] *= al[c];
        /* steps 5 and 6: delta-rule correction, one value row at a time */
        for (int64_t i = 0; i < V; ++i) {
            double pred = 0.0;
            for (int64_t c = 0; c < K; ++c)
                pred += S[i * K + c] * kt[c];
            double r = vt[i] - pred;
            for (int64_t c = 0; c < K; ++c)
                S[i * K + c] += bt * r * kt[c];
        }
        /* step 7: read-out with the updated state */
        if (out) {
            for (int64_t i = 0; i < V; ++i) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c)
                    acc += S[i * K + c] * qt[c];
                out[t * V + i] = scale * acc;
            }
        }
    }
    return 0;
}

/*
 * Full forward pass, same argument meaning as the library's kda_fwd, host memory.
 *   q, k, g: bf16 bits [B*T][H][128]; v: bf16 bits [B*T][H][128]; beta: bf16 bits [B*T][H]
 *   A_log: fp32 [H]; dt_bias: fp32 [H][128] (both may be NULL when the gate switch is off)
 *   flags: activation switches (ORACLE_*_IN_KERNEL bits; 7 = all activations in the pass)
 *   initial_state: NULL or [N][H][128][128] of state_dtype (bf16 bits, fp32 or fp64)
 *   cu_seqlens: NULL (then N = B, sequence b is batch row b) or int64 [N+1] with B == 1
 *   heads / n_heads: the subset of heads to compute (NULL = all, in order).  Outputs are
 *     laid out over the selected heads only:
 *       out:         double [B*T][n_sel][128]      (NULL = not written)
 *       final_state: double [N][n_sel][128][128]   (NULL = not written)
 *   nthreads <= 0 means the OpenMP default.
 * Returns 0 on success, nonzero on an argument error.
 */
static int kda_fwd_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                        const uint16_t *beta, double scale, const float *A_log, const float *dt_bias,
                        double lower_bound, int flags, const void *initial_state, int state_dtype,
                        const int64_t *cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t N,
                        const int32_t *heads, int64_t n_heads, double *out, double *final_state,
                        const uint16_t *out_cmp, double *stats, int nthreads)
{
    const int64_t D = ORACLE_DIM;
    if (B < 1 || T < 0 || H < 1)
        return 1;
    if (cu_seqlens) {
        if (B != 1 || N < 1)
            return 2;
        if (cu_seqlens[0] != 0 || cu_seqlens[N] != T)
            return 3;
        for (int64_t i = 0; i < N; ++i)
            if (cu_seqlens[i + 1] < cu_seqlens[i])
                return 3;
    } else {
        N = B;
    }
    if ((flags & ~7) != 0)
        return 5;
    if ((flags & ORACLE_GATE_IN_KERNEL) && (!A_log || !dt_bias))
        return 6;
    const int64_t n_sel = heads ? n_heads : H;
    if (n_sel < 1)
        return 4;
    const int64_t n_chains = N * n_sel;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t chain = 0; chain < n_chains; ++chain) {
        const int64_t n = chain / n_sel;
        const int64_t hs = chain % n_sel;
        const int64_t h = heads ? heads[hs] : hs;
        const int64_t t0 = cu_seqlens ? cu_seqlens[n] : n * T;
        const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : (n + 1) * T;

        double *S = (double *)malloc(sizeof(double) * D * D);
        double *alpha = (double *)malloc(sizeof(double) * D);
        double *kn = (double *)malloc(sizeof(double) * D);
        double *qn = (double *)malloc(sizeof(double) * D);
        double *tmp = (double *)malloc(sizeof(double) * D);
        double *vt = (double *)malloc(sizeof(double) * D);
        double *ot = (double *)malloc(sizeof(double) * D);

        /* initial state (V-major [v][c]), or zeros */
        const int64_t sbase = (n * H + h) * D * D;
        for (int64_t e = 0; e < D * D; ++e) {
            double s = 0.0;
            if (initial_state) {
                if (state_dtype == ORACLE_STATE_BF16)
                    s = bf16_bits_to_double(((const uint16_t *)initial_state)[sbase + e]);
                else if (state_dtype == ORACLE_STATE_FP32)
                    s = (double)((const float *)initial_state)[sbase + e];
                else if (state_dtype == ORACLE_STATE_FP64)
                    s = ((const double *)initial_state)[sbase + e];
            }
            S[e] = s;
        }

        if (stats)
            stats[3 * chain] = stats[3 * chain + 1] = stats[3 * chain + 2] = 0.0;
        const double Alog = (flags & ORACLE_GATE_IN_KERNEL) ? (double)A_log[h] : 0.0;
        for (int64_t t = t0; t < t1; ++t) {
            const int64_t row = (t * H + h) * D;
            /* step 1: l2-normalised query and key (or as given) */
            for (int64_t c = 0; c < D; ++c)
                tmp[c] = bf16_bits_to_double(q[row + c]);
            if (flags & ORACLE_QK_L2NORM_IN_KERNEL)
                oracle_l2norm(tmp, D, ORACLE_EPS, qn);
            else
                memcpy(qn, tmp, sizeof(double) * D);
            for (int64_t c = 0; c < D; ++c)
                tmp[c] = bf16_bits_to_double(k[row + c]);
            if (flags & ORACLE_QK_L2NORM_IN_KERNEL)
                oracle_l2norm(tmp, D, ORACLE_EPS, kn);
            else
                memcpy(kn, tmp, sizeof(double) * D);
            /* step 2: gate -> per-channel decay */
            for (int64_t c = 0; c < D; ++c) {
                const double gc = bf16_bits_to_double(g[row + c]);
                double a = (flags & ORACLE_GATE_IN_KERNEL)
                               ? oracle_gate(gc, Alog, (double)dt_bias[h * D + c], lower_bound)
                               : oracle_gate_preactivated(gc, lower_bound);
                alpha[c] = exp(a);
            }
            /* step 3: write strength */
            const double braw = bf16_bits_to_double(beta[t * H + h]);
            double bt = (flags & ORACLE_BETA_SIGMOID_IN_KERNEL) ? oracle_sigmoid(braw) : braw;
            for (int64_t c = 0; c < D; ++c)
                vt[c] = bf16_bits_to_double(v[row + c]);
            /* steps 4-7 */
            oracle_core(1, D, D, alpha, &bt, kn, qn, vt, scale, S, ot);
            if (out) {
                double *o = out + (t * n_sel + hs) * D;
                for (int64_t c = 0; c < D; ++c)
                    o[c] = ot[c];
            }
            if (out_cmp) {
                /* streaming comparison with a bf16 output of the full [B*T][H][128] layout */
                double *st = stats + 3 * chain;
                const uint16_t *oc = out_cmp + (t * H + h) * D;
                for (int64_t c = 0; c < D; ++c) {
                    const double e = bf16_bits_to_double(oc[c]) - ot[c];
                    const double ae = e < 0.0 ? -e : e;
                    if (!(ae <= st[0]))  /* also records a NaN */
                        st[0] = ae;
                    st[1] += e * e;
                    st[2] += ot[c] * ot[c];
                }
            }
        }
        if (final_state) {
            double *fs = final_state + (n * n_sel + hs) * D * D;
            memcpy(fs, S, sizeof(double) * D * D);
        }
        free(S);
        free(alpha);
        free(kn);
        free(qn);
        free(tmp);
        free(vt);
        free(ot);
    }
    return 0;
}

int oracle_kda_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                   const uint16_t *beta, double scale, const float *A_log, const float *dt_bias,
                   double lower_bound, int flags, const void *initial_state, int state_dtype,
                   const int64_t *cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t N,
                   const int32_t *heads, int64_t n_heads, double *out, double *final_state,
                   int nthreads)
{
    return kda_fwd_impl(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, flags, initial_state,
                        state_dtype, cu_seqlens, B, T, H, N, heads, n_heads, out, final_state, NULL,
                        NULL, nthreads);
}

/*
 * The same forward pass, comparing instead of storing the output: out_cmp holds another
 * implementation's output as bf16 bits in the full [B*T][H][128] layout, and for every
 * selected chain (sequence n, selected head hs; index n * n_sel + hs) stats receives
 * { max |out_cmp - out|, sum (out_cmp - out)^2, sum out^2 } with out the fp64 oracle
 * value.  The fp64 output itself is never stored, so very long sequences can be checked
 * in bounded memory.  final_state as in oracle_kda_fwd.  Test infrastructure only.
 */
int oracle_kda_fwd_compare(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                           const uint16_t *beta, double scale, const float *A_log, const float *dt_bias,
                           double lower_bound, int flags, const void *initial_state, int state_dtype,
                           const int64_t *cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t N,
                           const int32_t *heads, int64_t n_heads, const uint16_t *out_cmp,
                           double *stats, double *final_state, int nthreads)
{
    if (!out_cmp || !stats)
        return 7;
    return kda_fwd_impl(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, flags, initial_state,
                        state_dtype, cu_seqlens, B, T, H, N, heads, n_heads, NULL, final_state, out_cmp,
                        stats, nthreads);
}

/* Threads the OpenMP runtime would use by default (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
