// The steps just before the KDA recurrence, from raw projections, in one pass:
//   q <- q / ||q||,  k <- k / ||k||   (per token and head, over d_k)
//   g <- -softplus(g)                 (so that alpha = exp(g) = 1 / (1 + e^x))
//   beta <- sigmoid(beta)
// "Kimi Linear architecture" (ttj.ttj.kr), section "KDA: a memo that erases
// and rewrites": one forget rate per channel in (0, 1); "From GPT-2 to Kimi
// K3", section "Gated DeltaNet: now it can forget": alpha in [0, 1].  The
// pages do not print the parametrisation; this is the one the benchmark
// inputs are drawn with.  An all-zero q or k row stays zero.
//
// Each lane moves 16 bytes of a (token, head) row; the two squared norms are
// reduced across the row's lanes with shuffles.  HBM-bound.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kPrepThreads = 256;

// 16 bytes of E as fp32 values, and back (bf16: round to nearest even).
template <typename E> struct Vec16;
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void load(const bf16_t* p, float (&x)[8]) {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float (&x)[8]) {
        uint4 w;
        w.x = f32x2_to_bf16x2(x[0], x[1]);
        w.y = f32x2_to_bf16x2(x[2], x[3]);
        w.z = f32x2_to_bf16x2(x[4], x[5]);
        w.w = f32x2_to_bf16x2(x[6], x[7]);
        *reinterpret_cast<uint4*>(p) = w;
    }
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void load(const float* p, float (&x)[4]) {
        const float4 w = *reinterpret_cast<const float4*>(p);
        x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    }
    __device__ __forceinline__ static void store(float* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
};

// Each lane moves 16 bytes of a row; LPR lanes cover a row of d_k and a wave
// holds 64 / LPR rows.  Every lane takes part in the shuffles (rows past the
// end only skip their loads and stores).
template <typename E, int DK, bool HG>
__global__ __launch_bounds__(kPrepThreads) void prepare_kernel(const E* __restrict__ q_raw,
                                                               const E* __restrict__ k_raw,
                                                               const E* __restrict__ g_raw,
                                                               const E* __restrict__ b_raw, int64_t rows,
                                                               E* __restrict__ q, E* __restrict__ k,
                                                               E* __restrict__ g, E* __restrict__ beta) {
    using V = Vec16<E>;
    constexpr int EPL = V::N, LPR = DK / EPL, RPW = 64 / LPR, RPB = RPW * (kPrepThreads / 64);
    const int lane = threadIdx.x % 64;
    const int sub = lane % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + (threadIdx.x / 64) * RPW + lane / LPR;
    const bool valid = row < rows;
    const int64_t base = row * DK + (int64_t)sub * EPL;
    float xq[EPL], xk[EPL], xg[EPL];
    float sq = 0.f, sk = 0.f;
    if (valid) {
        V::load(q_raw + base, xq);
        V::load(k_raw + base, xk);
        if (!HG) V::load(g_raw + base, xg);
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            sq += xq[j] * xq[j];
            sk += xk[j] * xk[j];
        }
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) {
        sq += __shfl_xor(sq, off, 64);
        sk += __shfl_xor(sk, off, 64);
    }
    if (!valid) return;
    const float iq = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
    const float ik = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        xq[j] *= iq;
        xk[j] *= ik;
    }
    V::store(q + base, xq);
    V::store(k + base, xk);
    if (!HG) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) xg[j] = neg_softplus<E>(xg[j]);
        V::store(g + base, xg);
    }
    if (sub == 0) {
        if (HG) g[row] = Elt<E>::from(neg_softplus<E>(Elt<E>::load(g_raw + row)));
        beta[row] = Elt<E>::from(sigmoid<E>(Elt<E>::load(b_raw + row)));
    }
}

template <typename E, int DK, bool HG>
hipError_t launch_prepare_t(const PrepArgs& a, hipStream_t stream) {
    constexpr int RPB = 64 / (DK / Vec16<E>::N) * (kPrepThreads / 64);
    const int64_t rows = a.T * a.H;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((prepare_kernel<E, DK, HG>), dim3((unsigned)blocks), dim3(kPrepThreads), 0, stream,
                       (const E*)a.q_raw, (const E*)a.k_raw, (const E*)a.g_raw, (const E*)a.b_raw, rows, (E*)a.q,
                       (E*)a.k, (E*)a.g, (E*)a.beta);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_prepare_e(const PrepArgs& a, hipStream_t s) {
    if (a.dk == 64) return a.head_gate ? launch_prepare_t<E, 64, true>(a, s) : launch_prepare_t<E, 64, false>(a, s);
    return a.head_gate ? launch_prepare_t<E, 128, true>(a, s) : launch_prepare_t<E, 128, false>(a, s);
}

}  // namespace

hipError_t launch_prepare(const PrepArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    return a.bf16 ? launch_prepare_e<bf16_t>(a, stream) : launch_prepare_e<float>(a, stream);
}

}  // namespace kda
