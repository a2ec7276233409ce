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

/*
 * Gradients of the recurrence: for cotangents dO [T,H,dv] (bf16 bits, fp32
 * or fp64: dO_dtype) and dS_T [N,H,dk,dv] (fp64; NULL = zeros), the
 * vector-Jacobian product
 *
 *   L = sum_t <dO_t, o_t> + sum_{n,h} <dS_T[n,h], S_T[n,h]>
 *   -> dq, dk, dv, dg, dbeta (per token) and dS0 (per sequence and head),
 *
 * by reverse-mode differentiation of the six steps above, one token at a
 * time from the last to the first, in fp64.  With S the state before the
 * token, S1 = Diag(a) S, r = S1^T k, u = beta (v - r), S2 = S1 + k u^T and
 * o = S2^T q, and G the cotangent of S2 coming from later tokens:
 *
 *   G  += q dO^T                      (o = S2^T q)
 *   dq  = S2 dO
 *   du  = G^T k,   dk += G u          (S2 = S1 + k u^T; dS1 = G so far)
 *   dbeta = du . (v - r),  dv = beta du,  dr = -beta du
 *   dS1 = G + k dr^T,  dk += S1 dr    (r = S1^T k)
 *   da  = rowsum(dS1 * S),  G <- Diag(a) dS1   (S1 = Diag(a) S)
 *   dg  = da * a                      (a = exp(g); summed over the channels
 *                                      for a per-head gate)
 *
 * and after the first token of a sequence G is dS0.  The state before each
 * token is recomputed: a first forward pass stores S every K tokens (K about
 * the square root of the sequence length) and every token's read r; every
 * stretch of K tokens is then replayed forward from its stored state (with
 * the stored r, one sweep per token) before it is walked backwards.
 *
 *   dq, dk, dv, dg, dbeta   fp64 outputs with one row per token of q, v, g
 *                           and beta, or, if row_slot != NULL, row
 *                           row_slot[t] (-1 = not recorded)
 *   dS0                     fp64 [N,H,dk,dv] (always written)
 *
 * Returns 0, or -1 on a bad argument, -2 on allocation failure.
 */
struct adj_args {
    const void *q, *k, *v, *g, *beta;
    int dtype;
    const double *S0, *dS_T;
    const void *dO;
    int dO_dtype;
    int32_t H, dk, dv;
    int per_head_gate;
    const int64_t *row_slot;
    double *dq, *dk_out, *dv_out, *dg, *dbeta, *dS0;
};

/* this token's inputs, widened */
static void adj_load(const struct adj_args *A, int64_t t, int64_t h, double *a,
                     double *kt, double *qt, double *vt, double *bt)
{
    const int64_t kb = (t * A->H + h) * A->dk, vb = (t * A->H + h) * A->dv;
    *bt = widen(A->beta, A->dtype, t * A->H + h);
    for (int c = 0; c < A->dk; ++c) {
        const double gc = A->per_head_gate ? widen(A->g, A->dtype, t * A->H + h)
                                           : widen(A->g, A->dtype, kb + c);
        a[c] = exp(gc);
        kt[c] = widen(A->k, A->dtype, kb + c);
        qt[c] = widen(A->q, A->dtype, kb + c);
    }
    for (int j = 0; j < A->dv; ++j)
        vt[j] = widen(A->v, A->dtype, vb + j);
}

/* One (sequence, head) pair: tokens t0 .. t0 + len - 1, state slot p.
   Returns 0 or -2.  Built twice, for AVX2 and for plain x86-64, and the
   faster one that the host supports is picked when the library loads. */
__attribute__((target_clones("avx2", "default")))
static int adj_pair(const struct adj_args *A, int64_t p, int64_t h, int64_t t0,
                    int64_t len)
{
    const int dk = A->dk, dv = A->dv, H = A->H;
    const int64_t DD = (int64_t)dk * dv;
    int64_t K = 16;
    while (K * K < len)
        ++K;
    const int64_t nseg = (len + K - 1) / K;
    double *ck = (double *)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * DD));
    double *seg = (double *)malloc(sizeof(double) * (size_t)(K * DD));
    double *rs = (double *)malloc(sizeof(double) * (size_t)((len > 0 ? len : 1) * dv));
    double *G = (double *)malloc(sizeof(double) * (size_t)DD);
    double *a = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kt = (double *)malloc(sizeof(double) * (size_t)dk);
    double *qt = (double *)malloc(sizeof(double) * (size_t)dk);
    double *gq = (double *)malloc(sizeof(double) * (size_t)dk);
    double *gk = (double *)malloc(sizeof(double) * (size_t)dk);
    double *da = (double *)malloc(sizeof(double) * (size_t)dk);
    double *vt = (double *)malloc(sizeof(double) * (size_t)dv);
    double *restrict u = (double *)malloc(sizeof(double) * (size_t)dv);
    double *restrict du = (double *)malloc(sizeof(double) * (size_t)dv);
    double *restrict dr = (double *)malloc(sizeof(double) * (size_t)dv);
    double *restrict dOt = (double *)malloc(sizeof(double) * (size_t)dv);
    int rc = 0;
    if (!ck || !seg || !rs || !G || !a || !kt || !qt || !gq || !gk || !da ||
        !vt || !u || !du || !dr || !dOt) {
        rc = -2;
        goto done;
    }
    double bt;
    /* forward pass: the state at the start of every stretch of K tokens and
       every token's read r = (Diag(a) S)^T k */
    double *S = seg;
    for (int64_t e = 0; e < DD; ++e)
        S[e] = A->S0 ? A->S0[p * DD + e] : 0.0;
    for (int64_t i = 0; i < len; ++i) {
        if (i % K == 0)
            memcpy(ck + (i / K) * DD, S, sizeof(double) * (size_t)DD);
        adj_load(A, t0 + i, h, a, kt, qt, vt, &bt);
        double *restrict r = rs + i * dv;
        for (int j = 0; j < dv; ++j)
            r[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
            const double w = a[c] * kt[c];
            const double *restrict row = S + (int64_t)c * dv;
            for (int j = 0; j < dv; ++j)
                r[j] += row[j] * w;
        }
        for (int j = 0; j < dv; ++j)
            u[j] = bt * (vt[j] - r[j]);
        for (int c = 0; c < dk; ++c) {
            double *restrict row = S + (int64_t)c * dv;
            const double ac = a[c], kc = kt[c];
            for (int j = 0; j < dv; ++j)
                row[j] = ac * row[j] + kc * u[j];
        }
    }
    for (int64_t e = 0; e < DD; ++e)
        G[e] = A->dS_T ? A->dS_T[p * DD + e] : 0.0;
    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t i0 = s * K, m = (len - i0 < K) ? len - i0 : K;
        /* replay the stretch: seg + i DD = state before token i0 + i */
        memcpy(seg, ck + s * DD, sizeof(double) * (size_t)DD);
        for (int64_t i = 0; i + 1 < m; ++i) {
            adj_load(A, t0 + i0 + i, h, a, kt, qt, vt, &bt);
            const double *r = rs + (i0 + i) * dv;
            for (int j = 0; j < dv; ++j)
                u[j] = bt * (vt[j] - r[j]);
            const double *restrict Sp = seg + i * DD;
            double *restrict Sn = seg + (i + 1) * DD;
            for (int c = 0; c < dk; ++c) {
                const double ac = a[c], kc = kt[c];
                for (int j = 0; j < dv; ++j)
                    Sn[(int64_t)c * dv + j] = ac * Sp[(int64_t)c * dv + j] + kc * u[j];
            }
        }
        for (int64_t i = m - 1; i >= 0; --i) {
            const int64_t t = t0 + i0 + i;
            const double *Sb = seg + i * DD; /* state before token t */
            for (int j = 0; j < dv; ++j)
                dOt[j] = widen(A->dO, A->dO_dtype, (t * H + h) * dv + j);
            const double *r = rs + (i0 + i) * dv;
            adj_load(A, t, h, a, kt, qt, vt, &bt);
            for (int j = 0; j < dv; ++j)
                u[j] = bt * (vt[j] - r[j]);
            /* G += q dO^T; dq = S2 dO; du = G^T k; dk = G u */
            for (int j = 0; j < dv; ++j)
                du[j] = 0.0;
            for (int c = 0; c < dk; ++c) {
                double sq = 0.0, sk = 0.0;
                const double *restrict Sr = Sb + (int64_t)c * dv;
                double *restrict Gr = G + (int64_t)c * dv;
                const double ac = a[c], kc = kt[c], qc = qt[c];
                /* the sums over j in SIMD lanes: a fixed, different order of
                   the same fp64 additions */
#pragma omp simd reduction(+ : sq, sk)
                for (int j = 0; j < dv; ++j) {
                    const double s2 = ac * Sr[j] + kc * u[j];
                    sq += s2 * dOt[j];
                    Gr[j] += qc * dOt[j];
                    du[j] += Gr[j] * kc;
                    sk += Gr[j] * u[j];
                }
                gq[c] = sq;
                gk[c] = sk;
            }
            double db = 0.0;
            for (int j = 0; j < dv; ++j) {
                db += du[j] * (vt[j] - r[j]);
                dr[j] = -bt * du[j];
            }
            /* dS1 = G + k dr^T; dk += S1 dr; da = rowsum(dS1 * S);
               G <- Diag(a) dS1 */
            for (int c = 0; c < dk; ++c) {
                double sk = 0.0, sa = 0.0;
                const double *restrict Sr = Sb + (int64_t)c * dv;
                double *restrict Gr = G + (int64_t)c * dv;
                const double ac = a[c], kc = kt[c];
#pragma omp simd reduction(+ : sk, sa)
                for (int j = 0; j < dv; ++j) {
                    const double d1 = Gr[j] + kc * dr[j];
                    sk += ac * Sr[j] * dr[j];
                    sa += d1 * Sr[j];
                    Gr[j] = ac * d1;
                }
                gk[c] += sk;
                da[c] = sa * a[c];
            }
            const int64_t row = A->row_slot ? A->row_slot[t] : t;
            if (row >= 0) {
                for (int c = 0; c < dk; ++c) {
                    A->dq[(row * H + h) * dk + c] = gq[c];
                    A->dk_out[(row * H + h) * dk + c] = gk[c];
                }
                for (int j = 0; j < dv; ++j)
                    A->dv_out[(row * H + h) * dv + j] = bt * du[j];
                if (A->per_head_gate) {
                    double sg = 0.0;
                    for (int c = 0; c < dk; ++c)
                        sg += da[c];
                    A->dg[row * H + h] = sg;
                } else {
                    for (int c = 0; c < dk; ++c)
                        A->dg[(row * H + h) * dk + c] = da[c];
                }
                A->dbeta[row * H + h] = db;
            }
        }
    }
    memcpy(A->dS0 + p * DD, G, sizeof(double) * (size_t)DD);
done:
    free(ck);
    free(seg);
    free(rs);
    free(G);
    free(a);
    free(kt);
    free(qt);
    free(gq);
    free(gk);
    free(da);
    free(vt);
    free(u);
    free(du);
    free(dr);
    free(dOt);
    return rc;
}

int kda_oracle_adjoint(const void *q, const void *k, const void *v,
                       const void *g, const void *beta, int dtype,
                       const double *S0, const void *dO, int dO_dtype,
                       const double *dS_T,
                       const int64_t *cu_seqlens, int32_t N, int32_t H,
                       int32_t dk, int32_t dv, int per_head_gate,
                       const int64_t *row_slot, double *dq, double *dkk,
                       double *dvv, double *dg, double *dbeta, double *dS0,
                       int threads)
{
    if (!q || !k || !v || !g || !beta || !dO || !cu_seqlens || N < 0 ||
        H <= 0 || dk <= 0 || dv <= 0 || dtype < 0 || dtype > 2 ||
        dO_dtype < 0 || dO_dtype > 2 || !dq ||
        !dkk || !dvv || !dg || !dbeta || !dS0)
        return -1;
    const struct adj_args A = {q, k, v, g, beta, dtype, S0, dS_T, dO, dO_dtype, H, dk, dv,
                               per_head_gate, row_slot, dq, dkk, dvv, dg, dbeta, dS0};
    const int64_t pairs = (int64_t)N * H;
    int failed = 0;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / H, h = p % H;
        if (adj_pair(&A, p, h, cu_seqlens[n], cu_seqlens[n + 1] - cu_seqlens[n]) != 0) {
#pragma omp atomic write
            failed = 1;
        }
    }
    return failed ? -2 : 0;
}
