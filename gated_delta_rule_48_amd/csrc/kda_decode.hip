// One recurrent (decode) step of KDA: a single token per sequence updates the
// fp32 state in place.  "Kimi Linear architecture" (ttj.ttj.kr), section on
// linear attention: generation updates a fixed-size state once per token.
// "From GPT-2 to Kimi K3", section on the KV cache: decoding streams memory,
// so this step is bound by HBM bandwidth (one read and one write of S).
//
// Per (sequence n, head h), with a = exp(g):
//   r = S^T (a*k),  s = S^T (a*q),  u = beta (v - r),
//   o = s + (q.k) u,  S <- Diag(a) S + k u^T
// which equals one token of S_t = (I - beta k k^T) Diag(a) S_{t-1} + beta k v^T,
// o_t = S_t^T q_t.
//
// RAW: q and k arrive unnormalised and g, beta as raw projections; the step
// then also applies q <- q/||q||, k <- k/||k||, a = exp(-softplus(g)) =
// 1 / (1 + e^g), beta <- sigmoid(beta) (the transforms of kda_prepare_inputs).
// The norms are per (n, h) scalars, so they are reduced next to q.k and
// applied to the reduced reads: r, s and q.k scale by 1/||k||, 1/||q|| and
// both, and the write uses k/||k||.
//
// Layout: one workgroup of 256 threads per (n, h).  Thread (rg, cg) owns the
// four columns 4cg..4cg+3 of the rows rg*RPT .. rg*RPT+RPT-1 of S, which it
// loads once as float4s (a row of d_v floats is read by DV/4 consecutive
// lanes: fully coalesced), keeps in registers, and writes back once.
#include "kda_internal.h"

namespace kda {

template <typename E, int DK, int DV, bool HEAD_GATE, bool RAW = false>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ g, const E* __restrict__ beta, float* __restrict__ S,
    E* __restrict__ o, int32_t H) {
    constexpr int TPR = DV / 4;          // threads per row of S
    constexpr int NRG = 256 / TPR;       // row groups
    constexpr int RPT = DK / NRG;        // rows per thread
    static_assert(RPT >= 1 && DK % NRG == 0, "tiling");

    const int tid = threadIdx.x;
    const int cg = tid % TPR;
    const int rg = tid / TPR;
    const int64_t pair = blockIdx.x;  // n * H + h
    const int64_t kbase = pair * DK;
    const int64_t vbase = pair * DV;

    __shared__ float red_r[NRG][DV];
    __shared__ float red_s[NRG][DV];
    __shared__ float red_qk[NRG];
    __shared__ float red_n[RAW ? 2 : 1][NRG];

    // State block: issue every load first so they are all in flight.
    float4* Sp = reinterpret_cast<float4*>(S + pair * (int64_t)DK * DV);
    float4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) st[i] = Sp[(rg * RPT + i) * TPR + cg];

    float a[RPT], kk[RPT], qq[RPT];
    const float gh = HEAD_GATE ? Elt<E>::load(g + pair) : 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg * RPT + i;
        const float gi = HEAD_GATE ? gh : Elt<E>::load(g + kbase + c);
        a[i] = RAW ? recip<E>(1.f + gate_exp<E>(gi)) : gate_exp<E>(gi);
        kk[i] = Elt<E>::load(k + kbase + c);
        qq[i] = Elt<E>::load(q + kbase + c);
    }
    const float b = RAW ? sigmoid<E>(Elt<E>::load(beta + pair)) : Elt<E>::load(beta + pair);

    // Partial reads over this thread's rows: r = S^T (a*k), s = S^T (a*q).
    float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), ps = pr;
    float pqk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float ak = a[i] * kk[i], aq = a[i] * qq[i];
        pr.x += st[i].x * ak; pr.y += st[i].y * ak; pr.z += st[i].z * ak; pr.w += st[i].w * ak;
        ps.x += st[i].x * aq; ps.y += st[i].y * aq; ps.z += st[i].z * aq; ps.w += st[i].w * aq;
        pqk += qq[i] * kk[i];
    }
    *reinterpret_cast<float4*>(&red_r[rg][4 * cg]) = pr;
    *reinterpret_cast<float4*>(&red_s[rg][4 * cg]) = ps;
    if (cg == 0) red_qk[rg] = pqk;
    if (RAW && cg == 0) {
        float nq = 0.f, nk = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            nq += qq[i] * qq[i];
            nk += kk[i] * kk[i];
        }
        red_n[0][rg] = nq;
        red_n[RAW ? 1 : 0][rg] = nk;
    }
    lds_barrier();

    float4 r = make_float4(0.f, 0.f, 0.f, 0.f), s = r;
    float qk = 0.f;
#pragma unroll
    for (int j = 0; j < NRG; ++j) {
        const float4 x = *reinterpret_cast<const float4*>(&red_r[j][4 * cg]);
        const float4 y = *reinterpret_cast<const float4*>(&red_s[j][4 * cg]);
        r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
        s.x += y.x; s.y += y.y; s.z += y.z; s.w += y.w;
        qk += red_qk[j];
    }
    if (RAW) {
        float nq = 0.f, nk = 0.f;
#pragma unroll
        for (int j = 0; j < NRG; ++j) {
            nq += red_n[0][j];
            nk += red_n[RAW ? 1 : 0][j];
        }
        const float iq = nq > 0.f ? 1.f / sqrtf(nq) : 0.f;
        const float ik = nk > 0.f ? 1.f / sqrtf(nk) : 0.f;
        r.x *= ik; r.y *= ik; r.z *= ik; r.w *= ik;
        s.x *= iq; s.y *= iq; s.z *= iq; s.w *= iq;
        qk *= iq * ik;
#pragma unroll
        for (int i = 0; i < RPT; ++i) kk[i] *= ik;
    }
    const int c0 = 4 * cg;
    float4 u;
    u.x = b * (Elt<E>::load(v + vbase + c0 + 0) - r.x);
    u.y = b * (Elt<E>::load(v + vbase + c0 + 1) - r.y);
    u.z = b * (Elt<E>::load(v + vbase + c0 + 2) - r.z);
    u.w = b * (Elt<E>::load(v + vbase + c0 + 3) - r.w);
    if (rg == 0) {
        o[vbase + c0 + 0] = Elt<E>::from(s.x + qk * u.x);
        o[vbase + c0 + 1] = Elt<E>::from(s.y + qk * u.y);
        o[vbase + c0 + 2] = Elt<E>::from(s.z + qk * u.z);
        o[vbase + c0 + 3] = Elt<E>::from(s.w + qk * u.w);
    }
    // S <- Diag(a) S + k u^T, written back once, as non-temporal stores: the
    // state is not read again within this step, and streaming it past the
    // caches keeps them for the next step's (or another kernel's) reads.
    // Measured on back-to-back steps over one state: 169 us against 215 us.
    typedef float nf4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float4 x = st[i];
        const nf4 y = {a[i] * x.x + kk[i] * u.x, a[i] * x.y + kk[i] * u.y, a[i] * x.z + kk[i] * u.z,
                       a[i] * x.w + kk[i] * u.w};
        __builtin_nontemporal_store(y, reinterpret_cast<nf4*>(&Sp[(rg * RPT + i) * TPR + cg]));
    }
}

template <typename E, int DK, int DV, bool HG>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const int64_t pairs = (int64_t)a.N * a.H;
    if (a.raw)
        hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, HG, true>), dim3((unsigned)pairs), dim3(256), 0, stream,
                           (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.g, (const E*)a.beta, a.S,
                           (E*)a.o, a.H);
    else
        hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, HG>), dim3((unsigned)pairs), dim3(256), 0, stream,
                           (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.g, (const E*)a.beta, a.S,
                           (E*)a.o, a.H);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
    return a.head_gate ? launch_decode_t<E, DK, DV, true>(a, s) : launch_decode_t<E, DK, DV, false>(a, s);
}

template <typename E>
static hipError_t launch_decode_e(const DecodeArgs& a, hipStream_t s) {
    if (a.dk == 64 && a.dv == 64) return launch_decode_g<E, 64, 64>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch_decode_g<E, 64, 128>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch_decode_g<E, 128, 64>(a, s);
    return launch_decode_g<E, 128, 128>(a, s);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    return a.bf16 ? launch_decode_e<bf16_t>(a, stream) : launch_decode_e<float>(a, stream);
}

}  // namespace kda
