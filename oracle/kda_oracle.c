/*
 * fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or table with the HIP library.
 *
 * What it computes (one sequence n, one head h, token by token, in order):
 *
 *   a   = exp(g_t)                 per key channel; a per-head gate is one
 *                                  scalar broadcast over the channels
 *   S  <- Diag(a) S                forget first, channel by channel
 *   r   = S^T k_t                  read what the key currently retrieves
 *   u   = beta_t (v_t - r)         the (scaled) delta
 *   S  <- S + k_t u^T              write only the delta
 *   o_t = S^T q_t                  read out after the write
 *
 * Sources, as read from the pages:
 *  - "From GPT-2 to Kimi K3" (molayo1419.me), section "DeltaNet: memory you can
 *    edit": read the value stored under the key, form the difference with the
 *    new value, add only the difference back (the delta rule).
 *  - same page, section "Gated DeltaNet: now it can forget": decay the old
 *    state first, then write precisely; alpha = 1 is plain DeltaNet, alpha = 0
 *    erases.
 *  - same page, section "KDA: Kimi's secret sauce" and "Kimi Linear
 *    architecture" (ttj.ttj.kr), section "KDA: a memo that erases and
 *    rewrites": the forget gate is a vector with one rate per state channel.
 *  - The write strength beta is not on the pages; it follows the stated KDA
 *    transition S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, which
 *    the six steps above reproduce exactly: expanding the product gives
 *    Diag(a)S + k * beta (v - (Diag(a)S)^T k).
 *
 * Conventions: S is d_k x d_v, row c = key channel c.  q, k, g are
 * [T, H, d_k] (g is [T, H] for a per-head gate), v and o are [T, H, d_v],
 * beta is [T, H], S0 and S_T are [N, H, d_k, d_v].  Sequences are packed
 * along T and delimited by cu_seqlens (N+1 offsets).  Inputs arrive as bf16
 * bit patterns, fp32 or fp64 and are widened exactly to fp64; all arithmetic
 * is fp64 with libm's exp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2 };

/* Widen element i of a bf16 / fp32 / fp64 array to fp64, exactly. */
static double widen(const void *p, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16) {
        uint32_t w = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F32)
        return (double)((const float *)p)[i];
    return ((const double *)p)[i];
}

int kda_oracle_version(void) { return 1; }

/*
 * Run the recurrence over every (sequence, head) pair.
 *
 *   S0      fp64 [N,H,dk,dv] or NULL (zeros)
 *   o       fp64 output rows; o_slot[t] (if o_slot != NULL) says which row of
 *           o token t goes to (-1 = not recorded); if o_slot == NULL, row t.
 *   S_T     fp64 [N,H,dk,dv] or NULL
 *   threads OpenMP threads (<= 0: runtime default)
 *
 * Returns 0, or -1 on a bad argument, -2 on allocation failure.
 */
int kda_oracle_recurrence(const void *q, const void *k, const void *v,
                          const void *g, const void *beta, int dtype,
                          const double *S0, const int64_t *cu_seqlens,
                          int32_t N, int32_t H, int32_t dk, int32_t dv,
                          int per_head_gate, double *o, const int64_t *o_slot,
                          double *S_T, int threads)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || N < 0 || H <= 0 ||
        dk <= 0 || dv <= 0 || dtype < 0 || dtype > 2)
        return -1;
    int64_t pairs = (int64_t)N * H;
    int failed = 0;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        int64_t n = p / H, h = p % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *a = (double *)malloc(sizeof(double) * (size_t)dk);
        double *kt = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qt = (double *)malloc(sizeof(double) * (size_t)dk);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !a || !kt || !qt || !u) {
#pragma omp atomic write
            failed = 1;
        } else {
            const int64_t sbase = p * dk * dv;
            for (int64_t e = 0; e < (int64_t)dk * dv; ++e)
                S[e] = S0 ? S0[sbase + e] : 0.0;
            for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
                const int64_t kbase = (t * H + h) * dk;
                const int64_t vbase = (t * H + h) * dv;
                const double b = widen(beta, dtype, t * H + h);
                /* 1. per-channel forget factors */
                for (int c = 0; c < dk; ++c) {
                    double gc = per_head_gate ? widen(g, dtype, t * H + h)
                                              : widen(g, dtype, kbase + c);
                    a[c] = exp(gc);
                    kt[c] = widen(k, dtype, kbase + c);
                    qt[c] = widen(q, dtype, kbase + c);
                }
                /* 2. forget: S <- Diag(a) S */
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j)
                        S[c * dv + j] *= a[c];
                /* 3. read r = S^T k  and  4. u = beta (v - r) */
                for (int j = 0; j < dv; ++j)
                    u[j] = 0.0;
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j)
                        u[j] += S[c * dv + j] * kt[c];
                for (int j = 0; j < dv; ++j)
                    u[j] = b * (widen(v, dtype, vbase + j) - u[j]);
                /* 5. write the delta: S <- S + k u^T */
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j)
                        S[c * dv + j] += kt[c] * u[j];
                /* 6. output o_t = S^T q */
                int64_t row = o_slot ? o_slot[t] : t;
                if (o && row >= 0) {
                    double *orow = o + (row * H + h) * dv;
                    for (int j = 0; j < dv; ++j)
                        orow[j] = 0.0;
                    for (int c = 0; c < dk; ++c)
                        for (int j = 0; j < dv; ++j)
                            orow[j] += S[c * dv + j] * qt[c];
                }
            }
            if (S_T)
                memcpy(S_T + sbase, S, sizeof(double) * (size_t)dk * dv);
        }
        free(S);
        free(a);
        free(kt);
        free(qt);
        free(u);
    }
    return failed ? -2 : 0;
}
