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
// One wave per (token, head) row: each lane holds d_k / 64 channels, the two
// squared norms are reduced across the wave with shuffles.  HBM-bound.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kPrepThreads = 256;  // four rows per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <typename E, int DK, bool HG>
__global__ __launch_bounds__(kPrepThreads) void prepare_kernel(const E* __restrict__ q_raw,
                                                               const E* __restrict__ k_raw,
                                                               const E* __restrict__ g_raw,
                                                               const E* __restrict__ b_raw, int64_t rows,
                                                               E* __restrict__ q, E* __restrict__ k,
                                                               E* __restrict__ g, E* __restrict__ beta) {
    constexpr int EPL = DK / 64;  // channels per lane
    const int64_t row = (int64_t)blockIdx.x * (kPrepThreads / 64) + threadIdx.x / 64;
    if (row >= rows) return;
    const int lane = threadIdx.x % 64;
    const int64_t base = row * DK + (int64_t)lane * EPL;
    float xq[EPL], xk[EPL];
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        xq[j] = Elt<E>::load(q_raw + base + j);
        xk[j] = Elt<E>::load(k_raw + base + j);
        sq += xq[j] * xq[j];
        sk += xk[j] * xk[j];
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    const float iq = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
    const float ik = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        q[base + j] = Elt<E>::from(xq[j] * iq);
        k[base + j] = Elt<E>::from(xk[j] * ik);
    }
    if (!HG) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) g[base + j] = Elt<E>::from(neg_softplus(Elt<E>::load(g_raw + base + j)));
    }
    if (lane == 0) {
        if (HG) g[row] = Elt<E>::from(neg_softplus(Elt<E>::load(g_raw + row)));
        beta[row] = Elt<E>::from(sigmoid(Elt<E>::load(b_raw + row)));
    }
}

template <typename E, int DK, bool HG>
hipError_t launch_prepare_t(const PrepArgs& a, hipStream_t stream) {
    const int64_t rows = a.T * a.H;
    const int64_t blocks = (rows + kPrepThreads / 64 - 1) / (kPrepThreads / 64);
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
