// C ABI of the KDA hot path: argument validation, workspace carving and
// kernel dispatch.  The operation each entry point performs is documented in
// include/kda.h.  Nothing here allocates memory or synchronises the host,
// except kda_chunk_fwd_check, which exists to do exactly that.
#include "../../include/kda.h"
#include "kda_internal.h"

#include <limits.h>

namespace {

bool supported_d(int32_t d) { return d == 64 || d == 128; }

bool aligned(const void* p, size_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

kda_status check_common(int32_t H, int32_t dk, int32_t dv, kda_dtype dt, kda_gate gk) {
    if (H <= 0) return KDA_ERR_INVALID_ARG;
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (gk != KDA_GATE_PER_CHANNEL && gk != KDA_GATE_PER_HEAD) return KDA_ERR_UNSUPPORTED;
    if (!supported_d(dk) || !supported_d(dv)) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: null, misaligned or inconsistent argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head dimension, dtype or gate mode not supported";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP runtime call or kernel launch failed";
        case KDA_ERR_BAD_SEQLENS: return "KDA_ERR_BAD_SEQLENS: device cu_seqlens rejected";
        case KDA_ERR_TIMEOUT: return "KDA_ERR_TIMEOUT: an internal wait between waves gave up; results unspecified";
        case KDA_ERR_TOO_LARGE:
            return "KDA_ERR_TOO_LARGE: the problem needs more than the static scratch of kda_chunk_fwd_noalloc "
                   "(KDA_NOALLOC_SCRATCH_BYTES); use kda_chunk_fwd with a workspace";
    }
    return "KDA_ERR_UNKNOWN";
}

int32_t kda_version(void) { return (1 << 16) | 0; }

size_t kda_chunk_fwd_workspace_size(int64_t T_total, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                    kda_dtype dt, kda_gate gk) {
    if (check_common(H, d_k, d_v, dt, gk) != KDA_OK) return 0;
    if (N <= 0 || T_total < 0 || T_total > INT32_MAX) return 0;
    return kda::chunk_workspace_bytes(T_total, N, H, d_k, d_v, dt == KDA_BF16);
}

size_t kda_chunk_fwd_c128_workspace_size(int64_t T_total, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                         kda_dtype dt, kda_gate gk) {
    if (check_common(H, d_k, d_v, dt, gk) != KDA_OK) return 0;
    if (!kda::chunk128_supported(d_k, d_v, dt == KDA_BF16)) return 0;
    if (N <= 0 || T_total < 0 || T_total > INT32_MAX) return 0;
    return kda::chunk_workspace_bytes(T_total, N, H, d_k, d_v, dt == KDA_BF16, 128);
}

namespace {
kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const float* S0, const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                          int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk, void* o, float* S_T,
                          void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                          bool raw = false, int32_t chunk = kda::kChunk) {
    const kda_status st = check_common(H, d_k, d_v, dt, gk);
    if (st != KDA_OK) return st;
    if (chunk == 128 && !kda::chunk128_supported(d_k, d_v, dt == KDA_BF16)) return KDA_ERR_UNSUPPORTED;
    if (N <= 0 || T_total < 0 || T_total > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (!cu_seqlens && T_total % N != 0) return KDA_ERR_INVALID_ARG;
    if (!kda::chunk_grid_fits(kda::max_chunks_for(T_total, N, chunk), H, chunk)) return KDA_ERR_UNSUPPORTED;
    if (T_total > 0) {
        if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID_ARG;
        // q, k, v and a per-channel g are read two elements at a time
        const size_t esz = dt == KDA_BF16 ? 2 : 4;
        if (!aligned(q, 2 * esz) || !aligned(k, 2 * esz) || !aligned(v, 2 * esz) ||
            !aligned(g, gk == KDA_GATE_PER_HEAD ? esz : 2 * esz) || !aligned(beta, esz) || !aligned(o, esz))
            return KDA_ERR_INVALID_ARG;
    }
    if ((S0 && !aligned(S0, 4)) || (S_T && !aligned(S_T, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return KDA_ERR_INVALID_ARG;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_WORKSPACE;
    const size_t need = kda::chunk_workspace_bytes(T_total, N, H, d_k, d_v, dt == KDA_BF16, chunk);
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;

    kda::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.S0 = S0; a.cu_seqlens = cu_seqlens; a.o = o; a.S_T = S_T;
    a.N = N; a.H = H; a.dk = d_k; a.dv = d_v; a.T = T_total;
    a.max_chunks = kda::max_chunks_for(T_total, N, chunk);
    a.bf16 = dt == KDA_BF16;
    a.head_gate = gk == KDA_GATE_PER_HEAD;
    a.raw = raw;
    a.chunk = chunk;
    const kda::ChunkWorkspace ws = kda::carve_chunk_workspace(workspace, T_total, N, H, d_k, d_v, a.bf16, chunk);
    return kda::launch_chunk_fwd(a, ws, stream, events) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
}  // namespace

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* S0, const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                         int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk, void* o, float* S_T,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, g, beta, S0, cu_seqlens, N, T_total, H, d_k, d_v, dt, gk, o, S_T, workspace,
                          workspace_bytes, stream, nullptr);
}

kda_status kda_chunk_fwd_raw(const void* q_raw, const void* k_raw, const void* v, const void* g_raw,
                             const void* beta_raw, const float* S0, const int32_t* cu_seqlens, int32_t N,
                             int64_t T_total, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk,
                             void* o, float* S_T, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q_raw, k_raw, v, g_raw, beta_raw, S0, cu_seqlens, N, T_total, H, d_k, d_v, dt, gk, o, S_T,
                          workspace, workspace_bytes, stream, nullptr, true);
}

kda_status kda_chunk_fwd_c128(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              const float* S0, const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                              int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk, void* o, float* S_T,
                              void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
    return chunk_fwd_impl(q, k, v, g, beta, S0, cu_seqlens, N, T_total, H, d_k, d_v, dt, gk, o, S_T, workspace,
                          workspace_bytes, stream, events, false, 128);
}

kda_status kda_chunk_fwd_instrumented(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                      const float* S0, const int32_t* cu_seqlens, int32_t N, int64_t T_total,
                                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk, void* o,
                                      float* S_T, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                      hipEvent_t* events) {
    if (!events) return KDA_ERR_INVALID_ARG;
    return chunk_fwd_impl(q, k, v, g, beta, S0, cu_seqlens, N, T_total, H, d_k, d_v, dt, gk, o, S_T, workspace,
                          workspace_bytes, stream, events);
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                 const float* S0, const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                                 int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk, void* o, float* S_T,
                                 hipStream_t stream) {
    const kda_status st = check_common(H, d_k, d_v, dt, gk);
    if (st != KDA_OK) return st;
    if (N <= 0 || T_total < 0 || T_total > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (kda::chunk_workspace_bytes(T_total, N, H, d_k, d_v, dt == KDA_BF16) > KDA_NOALLOC_SCRATCH_BYTES)
        return KDA_ERR_TOO_LARGE;
    void* scratch = nullptr;
    if (kda::noalloc_scratch(&scratch) != hipSuccess) return KDA_ERR_HIP;
    return chunk_fwd_impl(q, k, v, g, beta, S0, cu_seqlens, N, T_total, H, d_k, d_v, dt, gk, o, S_T, scratch,
                          KDA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

kda_status kda_chunk_fwd_check(const void* workspace, hipStream_t stream) {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_WORKSPACE;
    if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
    kda::WsHeader h;
    if (hipMemcpy(&h, workspace, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return KDA_ERR_HIP;
    if (h.bad_seqlens) return KDA_ERR_BAD_SEQLENS;
    return h.wait_timeout ? KDA_ERR_TIMEOUT : KDA_OK;
}

size_t kda_chunk_bwd_workspace_size(int64_t T_total, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                    kda_dtype dt, kda_gate gk) {
    if (check_common(H, d_k, d_v, dt, gk) != KDA_OK) return 0;
    if (N <= 0 || T_total < 0 || T_total > INT32_MAX) return 0;
    return kda::bwd_workspace_bytes(T_total, N, H, d_k, d_v, dt == KDA_BF16);
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* S0, const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                         int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk, const void* dO, const float* dS_T,
                         void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dS0, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    const kda_status st = check_common(H, d_k, d_v, dt, gk);
    if (st != KDA_OK) return st;
    if (N <= 0 || T_total < 0 || T_total > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (!cu_seqlens && T_total % N != 0) return KDA_ERR_INVALID_ARG;
    if (!kda::chunk_grid_fits(kda::max_chunks_for(T_total, N), H)) return KDA_ERR_UNSUPPORTED;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    if (T_total > 0) {
        const void* need[] = {q, k, v, g, beta, dO, dq, dk, dv, dg, dbeta};
        for (const void* p : need)
            if (!p || !aligned(p, esz)) return KDA_ERR_INVALID_ARG;
    }
    if ((S0 && !aligned(S0, 4)) || (dS_T && !aligned(dS_T, 4)) || (dS0 && !aligned(dS0, 4)) ||
        (cu_seqlens && !aligned(cu_seqlens, 4)))
        return KDA_ERR_INVALID_ARG;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_WORKSPACE;
    if (kda::bwd_head_group(T_total, N, H, d_k, d_v, dt == KDA_BF16, workspace_bytes) < 1) return KDA_ERR_WORKSPACE;

    kda::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.S0 = S0; a.cu_seqlens = cu_seqlens; a.dO = dO; a.dS_T = dS_T;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dS0 = dS0;
    a.N = N; a.H = H; a.dk_ = d_k; a.dv_ = d_v; a.T = T_total;
    a.max_chunks = kda::max_chunks_for(T_total, N);
    a.bf16 = dt == KDA_BF16;
    a.head_gate = gk == KDA_GATE_PER_HEAD;
    return kda::launch_chunk_bwd(a, workspace, workspace_bytes, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

namespace {
kda_status recurrent_step_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               float* S, int32_t N, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dt,
                               kda_gate gk, void* o, hipStream_t stream, bool raw) {
    const kda_status st = check_common(H, d_k, d_v, dt, gk);
    if (st != KDA_OK) return st;
    if (N < 0 || (int64_t)N * H > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    if (!aligned(q, esz) || !aligned(k, esz) || !aligned(v, esz) || !aligned(g, esz) || !aligned(beta, esz) ||
        !aligned(o, esz) || !aligned(S, 16))
        return KDA_ERR_INVALID_ARG;
    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S = S; a.o = o;
    a.N = N; a.H = H; a.dk = d_k; a.dv = d_v;
    a.bf16 = dt == KDA_BF16;
    a.head_gate = gk == KDA_GATE_PER_HEAD;
    a.raw = raw;
    return kda::launch_decode(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
}  // namespace

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              float* S, int32_t N, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dt, kda_gate gk,
                              void* o, hipStream_t stream) {
    return recurrent_step_impl(q, k, v, g, beta, S, N, H, d_k, d_v, dt, gk, o, stream, false);
}

kda_status kda_recurrent_step_raw(const void* q_raw, const void* k_raw, const void* v, const void* g_raw,
                                  const void* beta_raw, float* S, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                  kda_dtype dt, kda_gate gk, void* o, hipStream_t stream) {
    return recurrent_step_impl(q_raw, k_raw, v, g_raw, beta_raw, S, N, H, d_k, d_v, dt, gk, o, stream, true);
}

kda_status kda_prepare_inputs(const void* q_raw, const void* k_raw, const void* g_raw, const void* beta_raw,
                              int64_t T_total, int32_t H, int32_t d_k, kda_dtype dt, kda_gate gk, void* q, void* k,
                              void* g, void* beta, hipStream_t stream) {
    if (H <= 0 || T_total < 0) return KDA_ERR_INVALID_ARG;
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (gk != KDA_GATE_PER_CHANNEL && gk != KDA_GATE_PER_HEAD) return KDA_ERR_UNSUPPORTED;
    if (!supported_d(d_k)) return KDA_ERR_UNSUPPORTED;
    if (T_total * H > (int64_t)UINT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (T_total == 0) return KDA_OK;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const void* ptrs[] = {q_raw, k_raw, g_raw, beta_raw, q, k, g, beta};
    for (const void* p : ptrs)
        if (!p || !aligned(p, esz)) return KDA_ERR_INVALID_ARG;
    // q, k and a per-channel g move in 16-byte pieces
    const void* rows[] = {q_raw, k_raw, q, k};
    for (const void* p : rows)
        if (!aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    if (gk == KDA_GATE_PER_CHANNEL && (!aligned(g_raw, 16) || !aligned(g, 16))) return KDA_ERR_INVALID_ARG;
    kda::PrepArgs a;
    a.q_raw = q_raw; a.k_raw = k_raw; a.g_raw = g_raw; a.b_raw = beta_raw;
    a.q = q; a.k = k; a.g = g; a.beta = beta;
    a.T = T_total; a.H = H; a.dk = d_k;
    a.bf16 = dt == KDA_BF16;
    a.head_gate = gk == KDA_GATE_PER_HEAD;
    return kda::launch_prepare(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
