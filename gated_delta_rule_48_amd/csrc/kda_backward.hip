// Chunked backward pass of KDA on gfx950: the vector-Jacobian product of
// (q, k, v, g, beta, S0) -> (o, S_T) with cotangents (dO, dS_T).
//
// "From GPT-2 to Kimi K3" (molayo1419.me), section on the parallelisation
// trick: the chunked form (masked attention inside a chunk, the state and one
// matrix product between chunks, all deltas of a chunk from one triangular
// solve) is what makes training parallel; "Kimi Linear architecture"
// (ttj.ttj.kr), section on linear attention: the chunkwise form serves
// training and prefill.  The backward pass below differentiates exactly the
// chunk algebra of the forward kernels.
//
// Forward algebra of one chunk (start state S, local rows t < n <= C):
//   b_t  = g_0 + ... + g_t (per key channel),  r = b at the middle row
//   QG = Q e^b, KG = K e^b, Kd = K e^{b_last - b}, Gn = e^{b_last}
//   Qr = Q e^{b - r}, Kr = K e^{b - r}, Ki = K e^{r - b}
//   M  = strict_tril(Kr Ki^T),  A = diag(beta) M,  T = (I + A)^{-1}
//   P  = tril(Qr Ki^T),  W = T diag(beta) KG,  U' = T diag(beta) V
//   U  = U' - W S,  O = QG S + P U,  S_next = Diag(Gn) S + Kd^T U
// (Qr Ki^T and Kr Ki^T equal the decayed products Q K^T and K K^T: the
// reference r cancels; it only keeps the factors in range.)
//
// Backward, per chunk in reverse order (reverse state walk):
//   dU = P^T dO + Kd dS_next
//   dS = Diag(Gn) dS_next + QG^T dO - W^T dU
// then, independently per chunk (local kernel):
//   dW = -dU S^T, dQG = dO S^T, dKd = U dS_next^T, dGn = rowsum(S * dS_next),
//   dP = tril(dO U^T)
//   dT = strict_tril(dW Xw^T + dU Xu^T) with Xw = diag(beta) KG, Xu = diag(beta) V
//   dXw = T^T dW, dXu = T^T dU,  dA = strict_tril(-T^T dT T^T)
//   dbeta = rowsum(dA * M) + rowsum(dXw * KG) + rowsum(dXu * V)
//   dKr = diag(beta) dA Ki, dKi = (diag(beta) dA)^T Kr + dP^T Qr, dQr = dP Ki
//   dq = dQG e^b + dQr e^{b-r},  dk = beta dXw e^b + dKr e^{b-r} + dKi e^{r-b} + dKd e^{b_last-b}
//   db = dQG QG + dQr Qr + beta dXw KG + dKr Kr - dKi Ki - dKd Kd
//        (+ sum_t dKd_t Kd_t + dGn Gn on the last row),  dv = beta dXu
//   dg = reverse cumulative sum of db over the chunk (summed over channels
//        for a per-head gate).
//
// This first version computes in fp32 on the vector units and keeps every
// intermediate of a chunk in the workspace; loops are arranged so that the
// 64 lanes of a wave read contiguous or identical addresses.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBwdThreads = 256;
constexpr int C = kChunk;

// Per-(chunk, head) arrays, fp32; slot = chunk * H + head.
struct BwdWs {
    WsHeader* header;
    int32_t* cu;
    int32_t* chunk_off;
    int2* chunk_tab;
    // [C][DK]
    float *B, *QG, *KG, *Kd, *Qr, *Kr, *Ki, *W, *dW, *dQG, *dKd, *dXw;
    // [DK][C]
    float *KiT, *XwT;
    // [C][DV] (UT and XuT are stored [DV][C])
    float *Up, *UT, *dU, *dXu, *XuT;
    // [C][C]
    float *M, *P, *T, *TT, *dP, *dT, *Y, *dA;
    // [DK]
    float *Gn, *dGn;
    // [DV][DK]: chunk start state and the state cotangent after the chunk, transposed
    float *ST, *dSnT;
};

template <typename E>
__device__ __forceinline__ float ld(const E* p, int64_t i) {
    return Elt<E>::load(p + i);
}

// ---------------------------------------------------------------------------
// Per (chunk, head): prefix sums, decayed operands, M, P, T = (I + A)^{-1},
// W and U'.
template <typename E, int DK, int DV, bool HG>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                               const E* __restrict__ v, const E* __restrict__ g,
                                                               const E* __restrict__ beta, int32_t H, BwdWs w) {
    __shared__ float sA[C][C + 1];
    __shared__ float sT[C][C + 1];
    __shared__ float sbeta[C];
    const int64_t slot = blockIdx.x;
    const int64_t chunk = slot / H;
    const int h = (int)(slot % H);
    if (w.header->bad_seqlens || chunk >= w.header->total_chunks) return;
    const int2 ct = w.chunk_tab[chunk];
    const int64_t t0 = ct.x;
    const int n = ct.y;
    const int tid = threadIdx.x;
    const size_t oCK = (size_t)slot * C * DK, oCV = (size_t)slot * C * DV, oCC = (size_t)slot * C * C;
    if (tid < C) sbeta[tid] = tid < n ? ld(beta, (t0 + tid) * H + h) : 0.f;
    __syncthreads();
    if (tid < DK) {
        const int c = tid;
        const int m = (n - 1) / 2;
        auto gate = [&](int t) -> float {
            return HG ? ld(g, (t0 + t) * H + h) : ld(g, ((t0 + t) * H + h) * DK + c);
        };
        // pass 1: the reference (middle row) and the last prefix sum
        float b = 0.f, r = 0.f;
        for (int t = 0; t < n; ++t) {
            b += gate(t);
            if (t == m) r = b;
        }
        const float bl = b;
        w.Gn[(size_t)slot * DK + c] = expf(bl);
        // pass 2: the same sums again, and every decayed operand
        b = 0.f;
        for (int t = 0; t < C; ++t) {
            float qv = 0.f, kv = 0.f;
            if (t < n) {
                b += gate(t);
                qv = ld(q, ((t0 + t) * H + h) * DK + c);
                kv = ld(k, ((t0 + t) * H + h) * DK + c);
            }
            const float e = expf(b), er = expf(b - r), eir = expf(r - b), ed = expf(bl - b);
            const size_t i = oCK + (size_t)t * DK + c;
            w.B[i] = b;
            w.QG[i] = qv * e;
            w.KG[i] = kv * e;
            w.Kd[i] = kv * ed;
            w.Qr[i] = qv * er;
            w.Kr[i] = kv * er;
            w.Ki[i] = kv * eir;
            w.KiT[oCK + (size_t)c * C + t] = kv * eir;
            w.XwT[oCK + (size_t)c * C + t] = sbeta[t] * kv * e;
        }
    }
    for (int idx = tid; idx < C * DV; idx += kBwdThreads) {
        const int t = idx / DV, c = idx % DV;
        const float vv = t < n ? ld(v, ((t0 + t) * H + h) * DV + c) : 0.f;
        w.XuT[oCV + (size_t)c * C + t] = sbeta[t] * vv;
    }
    __syncthreads();
    // M (strictly lower) and P (lower, diagonal included)
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, i = idx % C;
        float sm = 0.f, sp = 0.f;
        if (t < n && i <= t) {
            const float* kr = w.Kr + oCK + (size_t)t * DK;
            const float* qr = w.Qr + oCK + (size_t)t * DK;
            const float* kit = w.KiT + oCK + i;
            for (int c = 0; c < DK; ++c) {
                const float x = kit[(size_t)c * C];
                sm += kr[c] * x;
                sp += qr[c] * x;
            }
        }
        const float mv = i < t ? sm : 0.f;
        w.M[oCC + idx] = mv;
        w.P[oCC + idx] = sp;
        sA[t][i] = sbeta[t] * mv;
    }
    __syncthreads();
    // T = (I + A)^{-1}: column j by forward substitution (one thread per column)
    if (tid < C) {
        const int j = tid;
        for (int t = 0; t < C; ++t) {
            float val;
            if (t < j) {
                val = 0.f;
            } else if (t == j) {
                val = 1.f;
            } else {
                float s = 0.f;
                for (int i = j; i < t; ++i) s += sA[t][i] * sT[i][j];
                val = -s;
            }
            sT[t][j] = val;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, i = idx % C;
        w.T[oCC + idx] = sT[t][i];
        w.TT[oCC + idx] = sT[i][t];
    }
    // W = T diag(beta) KG,  U' = T diag(beta) V
    for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
        const int t = idx / DK, c = idx % DK;
        float s = 0.f;
        for (int i = 0; i <= t; ++i) s += sT[t][i] * sbeta[i] * w.KG[oCK + (size_t)i * DK + c];
        w.W[oCK + idx] = s;
    }
    for (int idx = tid; idx < C * DV; idx += kBwdThreads) {
        const int t = idx / DV, c = idx % DV;
        float s = 0.f;
        for (int i = 0; i <= t && i < n; ++i) s += sT[t][i] * sbeta[i] * ld(v, ((t0 + i) * H + h) * DV + c);
        w.Up[oCV + idx] = s;
    }
}

// ---------------------------------------------------------------------------
// Forward state walk per (sequence, head, 16-column slice): saves the start
// state of every chunk (transposed) and U = U' - W S (transposed).
template <int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void bwd_state_walk_kernel(int32_t H, const float* __restrict__ S0,
                                                                     BwdWs w) {
    constexpr int NS = DV / 16;
    __shared__ float sS[DK][16];
    __shared__ float sU[C][16];
    const int bid = blockIdx.x;
    const int sl = bid % NS;
    const int nh = bid / NS;
    const int h = nh % H;
    const int seq = nh / H;
    if (w.header->bad_seqlens) return;
    const int tid = threadIdx.x;
    const int col0 = sl * 16;
    for (int idx = tid; idx < DK * 16; idx += kBwdThreads) {
        const int c = idx / 16, vv = idx % 16;
        sS[c][vv] = S0 ? S0[(((size_t)seq * H + h) * DK + c) * DV + col0 + vv] : 0.f;
    }
    __syncthreads();
    const int c0 = w.chunk_off[seq], c1 = w.chunk_off[seq + 1];
    for (int ch = c0; ch < c1; ++ch) {
        const size_t slot = (size_t)ch * H + h;
        const size_t oCK = slot * C * DK, oCV = slot * C * DV, oKV = slot * DK * DV;
        for (int idx = tid; idx < DK * 16; idx += kBwdThreads) {
            const int c = idx / 16, vv = idx % 16;
            w.ST[oKV + (size_t)(col0 + vv) * DK + c] = sS[c][vv];
        }
        for (int idx = tid; idx < C * 16; idx += kBwdThreads) {
            const int t = idx / 16, vv = idx % 16;
            const float* wr = w.W + oCK + (size_t)t * DK;
            float s = w.Up[oCV + (size_t)t * DV + col0 + vv];
            for (int c = 0; c < DK; ++c) s -= wr[c] * sS[c][vv];
            sU[t][vv] = s;
            w.UT[oCV + (size_t)(col0 + vv) * C + t] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * 16; idx += kBwdThreads) {
            const int c = idx / 16, vv = idx % 16;
            float s = w.Gn[slot * DK + c] * sS[c][vv];
            for (int t = 0; t < C; ++t) s += w.Kd[oCK + (size_t)t * DK + c] * sU[t][vv];
            sS[c][vv] = s;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Reverse state walk per (sequence, head, 16-column slice): dU of every chunk
// and the state cotangent after it (transposed); dS0 at the end.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void bwd_dstate_walk_kernel(int32_t H, const E* __restrict__ dO,
                                                                      const float* __restrict__ dST,
                                                                      float* __restrict__ dS0, BwdWs w) {
    constexpr int NS = DV / 16;
    __shared__ float sdS[DK][16];
    __shared__ float sdU[C][16];
    __shared__ float sdO[C][16];
    const int bid = blockIdx.x;
    const int sl = bid % NS;
    const int nh = bid / NS;
    const int h = nh % H;
    const int seq = nh / H;
    if (w.header->bad_seqlens) return;
    const int tid = threadIdx.x;
    const int col0 = sl * 16;
    for (int idx = tid; idx < DK * 16; idx += kBwdThreads) {
        const int c = idx / 16, vv = idx % 16;
        sdS[c][vv] = dST ? dST[(((size_t)seq * H + h) * DK + c) * DV + col0 + vv] : 0.f;
    }
    __syncthreads();
    const int c0 = w.chunk_off[seq], c1 = w.chunk_off[seq + 1];
    for (int ch = c1 - 1; ch >= c0; --ch) {
        const size_t slot = (size_t)ch * H + h;
        const size_t oCK = slot * C * DK, oCV = slot * C * DV, oCC = slot * C * C, oKV = slot * DK * DV;
        const int2 ct = w.chunk_tab[ch];
        const int64_t t0 = ct.x;
        const int n = ct.y;
        for (int idx = tid; idx < DK * 16; idx += kBwdThreads) {
            const int c = idx / 16, vv = idx % 16;
            w.dSnT[oKV + (size_t)(col0 + vv) * DK + c] = sdS[c][vv];
        }
        for (int idx = tid; idx < C * 16; idx += kBwdThreads) {
            const int t = idx / 16, vv = idx % 16;
            sdO[t][vv] = t < n ? ld(dO, ((t0 + t) * H + h) * DV + col0 + vv) : 0.f;
        }
        __syncthreads();
        for (int idx = tid; idx < C * 16; idx += kBwdThreads) {
            const int t = idx / 16, vv = idx % 16;
            float s = 0.f;
            for (int i = t; i < C; ++i) s += w.P[oCC + (size_t)i * C + t] * sdO[i][vv];
            for (int c = 0; c < DK; ++c) s += w.Kd[oCK + (size_t)t * DK + c] * sdS[c][vv];
            sdU[t][vv] = s;
            w.dU[oCV + (size_t)t * DV + col0 + vv] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * 16; idx += kBwdThreads) {
            const int c = idx / 16, vv = idx % 16;
            float s = w.Gn[slot * DK + c] * sdS[c][vv];
            for (int t = 0; t < C; ++t) {
                const size_t i = oCK + (size_t)t * DK + c;
                s += w.QG[i] * sdO[t][vv] - w.W[i] * sdU[t][vv];
            }
            sdS[c][vv] = s;
        }
        __syncthreads();
    }
    if (dS0) {
        for (int idx = tid; idx < DK * 16; idx += kBwdThreads) {
            const int c = idx / 16, vv = idx % 16;
            dS0[(((size_t)seq * H + h) * DK + c) * DV + col0 + vv] = sdS[c][vv];
        }
    }
}

// ---------------------------------------------------------------------------
// Per (chunk, head): gradients of the chunk's inputs from dU, dS_next, S, U.
template <typename E, int DK, int DV, bool HG>
__global__ __launch_bounds__(kBwdThreads) void bwd_local_kernel(const E* __restrict__ v, const E* __restrict__ beta,
                                                                const E* __restrict__ dO, int32_t H, BwdWs w,
                                                                E* __restrict__ dq, E* __restrict__ dk,
                                                                E* __restrict__ dv, E* __restrict__ dg,
                                                                E* __restrict__ dbeta) {
    __shared__ float sbeta[C];
    __shared__ float sr[DK];
    __shared__ float sbl[DK];
    const int64_t slot = blockIdx.x;
    const int64_t chunk = slot / H;
    const int h = (int)(slot % H);
    if (w.header->bad_seqlens || chunk >= w.header->total_chunks) return;
    const int2 ct = w.chunk_tab[chunk];
    const int64_t t0 = ct.x;
    const int n = ct.y;
    const int tid = threadIdx.x;
    const size_t oCK = (size_t)slot * C * DK, oCV = (size_t)slot * C * DV, oCC = (size_t)slot * C * C;
    const size_t oK = (size_t)slot * DK, oKV = (size_t)slot * DK * DV;
    if (tid < C) sbeta[tid] = tid < n ? ld(beta, (t0 + tid) * H + h) : 0.f;
    if (tid < DK) {
        sr[tid] = w.B[oCK + (size_t)((n - 1) / 2) * DK + tid];
        sbl[tid] = w.B[oCK + (size_t)(n - 1) * DK + tid];
    }
    auto dOat = [&](int t, int c) -> float { return ld(dO, ((t0 + t) * H + h) * DV + c); };
    auto vat = [&](int t, int c) -> float { return ld(v, ((t0 + t) * H + h) * DV + c); };

    // phase 1: dW, dQG, dKd, dGn, dP
    for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
        const int t = idx / DK, c = idx % DK;
        float a1 = 0.f, a2 = 0.f, a3 = 0.f;
        if (t < n) {
            for (int x = 0; x < DV; ++x) {
                const float s = w.ST[oKV + (size_t)x * DK + c];
                a1 += w.dU[oCV + (size_t)t * DV + x] * s;
                a2 += dOat(t, x) * s;
                a3 += w.UT[oCV + (size_t)x * C + t] * w.dSnT[oKV + (size_t)x * DK + c];
            }
        }
        w.dW[oCK + idx] = -a1;
        w.dQG[oCK + idx] = a2;
        w.dKd[oCK + idx] = a3;
    }
    for (int c = tid; c < DK; c += kBwdThreads) {
        float s = 0.f;
        for (int x = 0; x < DV; ++x) s += w.ST[oKV + (size_t)x * DK + c] * w.dSnT[oKV + (size_t)x * DK + c];
        w.dGn[oK + c] = s;
    }
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, i = idx % C;
        float s = 0.f;
        if (i <= t && t < n)
            for (int x = 0; x < DV; ++x) s += dOat(t, x) * w.UT[oCV + (size_t)x * C + i];
        w.dP[oCC + idx] = s;
    }
    __syncthreads();

    // phase 2: dT (strictly lower), dXw = T^T dW, dXu = T^T dU
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, i = idx % C;
        float s = 0.f;
        if (i < t && t < n) {
            for (int c = 0; c < DK; ++c) s += w.dW[oCK + (size_t)t * DK + c] * w.XwT[oCK + (size_t)c * C + i];
            for (int x = 0; x < DV; ++x) s += w.dU[oCV + (size_t)t * DV + x] * w.XuT[oCV + (size_t)x * C + i];
        }
        w.dT[oCC + idx] = s;
    }
    for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
        const int t = idx / DK, c = idx % DK;
        float s = 0.f;
        for (int a = t; a < n; ++a) s += w.T[oCC + (size_t)a * C + t] * w.dW[oCK + (size_t)a * DK + c];
        w.dXw[oCK + idx] = s;
    }
    for (int idx = tid; idx < C * DV; idx += kBwdThreads) {
        const int t = idx / DV, x = idx % DV;
        float s = 0.f;
        for (int a = t; a < n; ++a) s += w.T[oCC + (size_t)a * C + t] * w.dU[oCV + (size_t)a * DV + x];
        w.dXu[oCV + idx] = s;
    }
    __syncthreads();

    // phase 3: Y = dT T^T (needed where column < row)
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int a = idx / C, i = idx % C;
        float s = 0.f;
        if (i < a && a < n)
            for (int b = 0; b <= i; ++b) s += w.dT[oCC + (size_t)a * C + b] * w.TT[oCC + (size_t)b * C + i];
        w.Y[oCC + idx] = s;
    }
    __syncthreads();

    // phase 4: dA = strict_tril(-T^T Y)
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, i = idx % C;
        float s = 0.f;
        if (i < t && t < n)
            for (int a = t; a < n; ++a) s += w.T[oCC + (size_t)a * C + t] * w.Y[oCC + (size_t)a * C + i];
        w.dA[oCC + idx] = -s;
    }
    __syncthreads();

    // phase 5: dq, dk, db (kept in dW's slot), dbeta, dv
    for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
        const int t = idx / DK, c = idx % DK;
        if (t >= n) continue;
        float dKr = 0.f, dKi = 0.f, dQr = 0.f;
        for (int i = 0; i < t; ++i) dKr += w.dA[oCC + (size_t)t * C + i] * w.Ki[oCK + (size_t)i * DK + c];
        dKr *= sbeta[t];
        for (int a = t + 1; a < n; ++a)
            dKi += sbeta[a] * w.dA[oCC + (size_t)a * C + t] * w.Kr[oCK + (size_t)a * DK + c];
        for (int a = t; a < n; ++a) dKi += w.dP[oCC + (size_t)a * C + t] * w.Qr[oCK + (size_t)a * DK + c];
        for (int i = 0; i <= t; ++i) dQr += w.dP[oCC + (size_t)t * C + i] * w.Ki[oCK + (size_t)i * DK + c];
        const size_t j = oCK + idx;
        const float dKG = sbeta[t] * w.dXw[j];
        const float dQG = w.dQG[j], dKd = w.dKd[j];
        const float b = w.B[j], r = sr[c], bl = sbl[c];
        const float e = expf(b), er = expf(b - r), eir = expf(r - b), ed = expf(bl - b);
        const int64_t o = ((t0 + t) * H + h) * DK + c;
        dq[o] = Elt<E>::from(dQG * e + dQr * er);
        dk[o] = Elt<E>::from(dKG * e + dKr * er + dKi * eir + dKd * ed);
        w.dW[j] = dQG * w.QG[j] + dQr * w.Qr[j] + dKG * w.KG[j] + dKr * w.Kr[j] - dKi * w.Ki[j] - dKd * w.Kd[j];
    }
    for (int t = tid; t < n; t += kBwdThreads) {
        float s = 0.f;
        for (int i = 0; i < t; ++i) s += w.dA[oCC + (size_t)t * C + i] * w.M[oCC + (size_t)t * C + i];
        for (int c = 0; c < DK; ++c) s += w.dXw[oCK + (size_t)t * DK + c] * w.KG[oCK + (size_t)t * DK + c];
        for (int x = 0; x < DV; ++x) s += w.dXu[oCV + (size_t)t * DV + x] * vat(t, x);
        dbeta[(t0 + t) * H + h] = Elt<E>::from(s);
    }
    for (int idx = tid; idx < C * DV; idx += kBwdThreads) {
        const int t = idx / DV, x = idx % DV;
        if (t < n) dv[((t0 + t) * H + h) * DV + x] = Elt<E>::from(sbeta[t] * w.dXu[oCV + idx]);
    }
    __syncthreads();

    // phase 6: dg = reverse cumulative sum of db; the last row's prefix sum
    // also carries e^{b_last} (Gn) and the e^{b_last} factor of Kd
    for (int c = tid; c < DK; c += kBwdThreads) {
        float acc = w.dGn[oK + c] * w.Gn[oK + c];
        for (int t = 0; t < n; ++t) acc += w.dKd[oCK + (size_t)t * DK + c] * w.Kd[oCK + (size_t)t * DK + c];
        for (int t = n - 1; t >= 0; --t) {
            acc += w.dW[oCK + (size_t)t * DK + c];
            if (HG)
                w.dQG[oCK + (size_t)t * DK + c] = acc;
            else
                dg[((t0 + t) * H + h) * DK + c] = Elt<E>::from(acc);
        }
    }
    if (HG) {
        __syncthreads();
        for (int t = tid; t < n; t += kBwdThreads) {
            float s = 0.f;
            for (int c = 0; c < DK; ++c) s += w.dQG[oCK + (size_t)t * DK + c];
            dg[(t0 + t) * H + h] = Elt<E>::from(s);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdSizes {
    size_t head, ck, cv, cc, k, kv, total;
};

BwdSizes bwd_sizes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv) {
    const size_t slots = (size_t)max_chunks_for(T, N) * H;
    BwdSizes s;
    s.head = 256 + 2 * al256((size_t)(N + 1) * 4) + al256((size_t)max_chunks_for(T, N) * sizeof(int2));
    s.ck = al256(slots * C * dk * 4);
    s.cv = al256(slots * C * dv * 4);
    s.cc = al256(slots * C * C * 4);
    s.k = al256(slots * dk * 4);
    s.kv = al256(slots * dk * dv * 4);
    s.total = s.head + 14 * s.ck + 5 * s.cv + 8 * s.cc + 2 * s.k + 2 * s.kv;
    return s;
}

BwdWs carve_bwd(void* base, int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv) {
    const BwdSizes s = bwd_sizes(T, N, H, dk, dv);
    char* p = static_cast<char*>(base);
    BwdWs w;
    w.header = reinterpret_cast<WsHeader*>(p); p += 256;
    w.cu = reinterpret_cast<int32_t*>(p); p += al256((size_t)(N + 1) * 4);
    w.chunk_off = reinterpret_cast<int32_t*>(p); p += al256((size_t)(N + 1) * 4);
    w.chunk_tab = reinterpret_cast<int2*>(p); p += al256((size_t)max_chunks_for(T, N) * sizeof(int2));
    auto take = [&](size_t bytes) { float* f = reinterpret_cast<float*>(p); p += bytes; return f; };
    float** ck[] = {&w.B, &w.QG, &w.KG, &w.Kd, &w.Qr, &w.Kr, &w.Ki, &w.W, &w.dW, &w.dQG, &w.dKd, &w.dXw,
                    &w.KiT, &w.XwT};
    for (float** f : ck) *f = take(s.ck);
    float** cv[] = {&w.Up, &w.UT, &w.dU, &w.dXu, &w.XuT};
    for (float** f : cv) *f = take(s.cv);
    float** cc[] = {&w.M, &w.P, &w.T, &w.TT, &w.dP, &w.dT, &w.Y, &w.dA};
    for (float** f : cc) *f = take(s.cc);
    w.Gn = take(s.k);
    w.dGn = take(s.k);
    w.ST = take(s.kv);
    w.dSnT = take(s.kv);
    return w;
}

template <typename E, int DK, int DV, bool HG>
hipError_t launch_bwd_t(const BwdArgs& a, const BwdWs& w, hipStream_t stream) {
    const unsigned slots = (unsigned)(a.max_chunks * a.H);
    const unsigned walks = (unsigned)((int64_t)a.N * a.H * (DV / 16));
    if (a.T > 0) {
        hipLaunchKernelGGL((bwd_prep_kernel<E, DK, DV, HG>), dim3(slots), dim3(kBwdThreads), 0, stream,
                           (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.g, (const E*)a.beta, a.H, w);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_state_walk_kernel<DK, DV>), dim3(walks), dim3(kBwdThreads), 0, stream, a.H, a.S0,
                           w);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_dstate_walk_kernel<E, DK, DV>), dim3(walks), dim3(kBwdThreads), 0, stream, a.H,
                       (const E*)a.dO, a.dS_T, a.dS0, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.T == 0) return e;
    hipLaunchKernelGGL((bwd_local_kernel<E, DK, DV, HG>), dim3(slots), dim3(kBwdThreads), 0, stream,
                       (const E*)a.v, (const E*)a.beta, (const E*)a.dO, a.H, w, (E*)a.dq, (E*)a.dk, (E*)a.dv,
                       (E*)a.dg, (E*)a.dbeta);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_bwd_g(const BwdArgs& a, const BwdWs& w, hipStream_t s) {
    return a.head_gate ? launch_bwd_t<E, DK, DV, true>(a, w, s) : launch_bwd_t<E, DK, DV, false>(a, w, s);
}

template <typename E>
hipError_t launch_bwd_e(const BwdArgs& a, const BwdWs& w, hipStream_t s) {
    if (a.dk_ == 64 && a.dv_ == 64) return launch_bwd_g<E, 64, 64>(a, w, s);
    if (a.dk_ == 64 && a.dv_ == 128) return launch_bwd_g<E, 64, 128>(a, w, s);
    if (a.dk_ == 128 && a.dv_ == 64) return launch_bwd_g<E, 128, 64>(a, w, s);
    return launch_bwd_g<E, 128, 128>(a, w, s);
}

}  // namespace

size_t bwd_workspace_bytes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv) {
    return bwd_sizes(T, N, H, dk, dv).total;
}

hipError_t launch_chunk_bwd(const BwdArgs& a, void* workspace, hipStream_t stream) {
    const BwdWs w = carve_bwd(workspace, a.T, a.N, a.H, a.dk_, a.dv_);
    hipError_t e = launch_chunk_map(a.cu_seqlens, a.N, a.T, w.header, w.cu, w.chunk_off, w.chunk_tab, stream);
    if (e != hipSuccess) return e;
    return a.bf16 ? launch_bwd_e<bf16_t>(a, w, stream) : launch_bwd_e<float>(a, w, stream);
}

}  // namespace kda
