// Chunkwise-parallel KDA forward on gfx950.
//
// "From GPT-2 to Kimi K3" (molayo1419.me), section on the parallelisation
// trick: split each sequence into chunks of C tokens, treat the inside of a
// chunk as masked attention, carry the state across chunks with one matrix
// product, and use a Householder-type reparametrisation so that all deltas of
// a chunk come out of one triangular solve.  "Kimi Linear architecture"
// (ttj.ttj.kr), section "KDA: a memo that erases and rewrites": the transition
// is diagonal plus a low-rank term built from the key itself, which is what
// lets the decay be folded into the key operands below.
//
// Chunk algebra (start state S, chunk-local tokens t = 0..n-1, C = 64):
//   b_t   = g_0 + ... + g_t              (per key channel, chunk-local)
//   A_ti  = beta_t sum_c k_tc k_ic e^{b_tc - b_ic}           i < t
//   T     = (I + A)^{-1}                 (unit lower triangular)
//   W     = T diag(beta) (K * e^b),   U' = T diag(beta) V
//   U     = U' - W S                     (the true per-token deltas)
//   O     = (Q * e^b) S + P U,   P_ti = sum_c q_tc k_ic e^{b_tc - b_ic}, i <= t
//   S    <- Diag(e^{b_last}) S + (K * e^{b_last - b})^T U
// The decay e^{b_t - b_i} inside A and P is split per 16-token tile: for a
// tile pair below the diagonal the reference rows lie between the two tiles,
// so every factor is <= 1 and nothing can overflow; inside a diagonal tile
// the reference is the tile's middle row, so a factor spans at most eight
// tokens of decay.  W, Q e^b, K e^{b_last - b} and e^{b_last} only involve
// factors <= 1.  Masks are applied by selection, never by multiplication.
//
// Kernels (one stream, in order):
//   chunk_map_kernel   validate cu_seqlens, first chunk of every sequence,
//                      first token and length of every chunk
//   intra_chunk_kernel one workgroup per (chunk, head): prefix sum of the
//                      gate, decayed operands, A and P on MFMA, (I+A)^{-1} by
//                      blocked forward substitution in LDS (fp32), W and U'
//                      on MFMA; writes W, Q*e^b, (K*e^{b_last-b})^T, U', P,
//                      e^{b_last} to the workspace
//   chunk_walk_kernel  one workgroup per (sequence, head, 16-column slice of
//                      d_v): walks the chunks in order with its fp32 slice of
//                      S in registers; U = U' - W S, O = QG S + P U,
//                      S <- Diag(Gn) S + KdT U, all on MFMA
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kda_chunk_util.h"

namespace kda {

// ----------------------------------------------------------------------------
// Chunk map (chunks of C tokens): copy (or synthesise) the sequence offsets,
// validate them, exclusive-scan the per-sequence chunk counts, and write
// every chunk's first token and length, so that a chunk's workgroup finds its tokens with a single
// load that does not depend on another.
template <int C>
__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ cu_in, int32_t N,
                                                        int64_t T, WsHeader* __restrict__ hdr,
                                                        int32_t* __restrict__ cu,
                                                        int32_t* __restrict__ chunk_off,
                                                        int2* __restrict__ chunk_tab,
                                                        int32_t* __restrict__ seg_flags, int64_t n_flags) {
    __shared__ int bad;
    __shared__ int carry;
    __shared__ int scan[256];
    const int tid = threadIdx.x;
    if (tid == 0) {
        bad = 0;
        carry = 0;
    }
    __syncthreads();
    const int64_t L = cu_in ? 0 : T / N;
    for (int i = tid; i <= N; i += 256) {
        const int64_t c = cu_in ? (int64_t)cu_in[i] : (int64_t)i * L;
        const int64_t cn = (i < N) ? (cu_in ? (int64_t)cu_in[i + 1] : (int64_t)(i + 1) * L) : T;
        cu[i] = (int32_t)c;
        if ((i == 0 && c != 0) || (i == N && c != T) || c < 0 || c > T || cn < c) bad = 1;
    }
    __syncthreads();
    const int isbad = bad;
    for (int base = 0; base < N; base += 256) {
        const int i = base + tid;
        int cnt = 0;
        if (i < N && !isbad) cnt = (cu[i + 1] - cu[i] + C - 1) / C;
        scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int x = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += x;
            __syncthreads();
        }
        if (i < N) chunk_off[i] = carry + scan[tid] - cnt;
        __syncthreads();
        if (tid == 255) carry += scan[255];
        __syncthreads();
    }
    if (tid == 0) {
        chunk_off[N] = carry;
        hdr->total_chunks = isbad ? 0 : carry;
        hdr->bad_seqlens = isbad;
        hdr->wait_timeout = 0;
        hdr->seg_ticket = 0;
    }
    for (int64_t i = tid; i < n_flags; i += 256) seg_flags[i] = 0;
    __syncthreads();  // chunk_off of every sequence is written
    const int total = isbad ? 0 : carry;
    for (int cid = tid; cid < total; cid += 256) {
        int lo = 0, hi = N;  // largest n with chunk_off[n] <= cid
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (chunk_off[mid] <= cid) lo = mid; else hi = mid;
        }
        const int t0 = cu[lo] + (cid - chunk_off[lo]) * C;
        chunk_tab[cid] = make_int2(t0, min(C, cu[lo + 1] - t0));
    }
}

// ----------------------------------------------------------------------------
// Intra-chunk transform.

template <typename E, int DK, int DV>
struct IntraLayout {
    static constexpr int C = kChunk;
    static constexpr int PAD = 16 / (int)sizeof(E);
    static constexpr int LDK = DK + PAD;  // [token][channel] row stride
    static constexpr int LDT = C + PAD;   // [channel][token] row stride
    static constexpr int LDA = C + 4;     // fp32 A / T row stride
    // threads hold two adjacent channels (values) of RPT (RPTV) consecutive rows
    static constexpr int NPART = kIntraThreads / (DK / 2);
    static constexpr int RPT = C / NPART;
    static constexpr int NPARTV = kIntraThreads / (DV / 2);
    static constexpr int RPTV = C / NPARTV;
    static_assert(RPT % 4 == 0 && RPTV % 4 == 0, "row runs of four");
    static constexpr int NBND = 12;       // b at rows 16i, 16i+8, 16i+15 of the four 16-row tiles
    static constexpr int NCS = 12;        // tile-pair decay factors (see the intra-chunk kernel)
    // Region R1: [Kr | Qr | Kt] ([token][channel], E) while A and P are
    // formed; afterwards [Kbt | Vt] ([channel][token], E) followed by the P
    // staging tile [C][C+PAD]; at the very end the W staging tile [C][DK+PAD]
    // for coalesced stores.
    static constexpr int LDP = C + PAD;
    static constexpr int LDV = DV + PAD;
    static constexpr size_t rhs_bytes = (size_t)(DK + DV) * LDT * sizeof(E);
    static constexpr size_t off_Pst = (rhs_bytes + 15) / 16 * 16;
    static constexpr size_t r1_a = (size_t)3 * C * LDK * sizeof(E);
    static constexpr size_t r1_b = off_Pst + (size_t)C * LDP * sizeof(E);
    static constexpr size_t r1_c = ((size_t)C * LDK + (size_t)DV * LDT) * sizeof(E);
    static constexpr size_t r1_max = r1_a > r1_b ? (r1_a > r1_c ? r1_a : r1_c) : (r1_b > r1_c ? r1_b : r1_c);
    static constexpr size_t off_A = (r1_max + 15) / 16 * 16;  // sA; sBnd before A
    static constexpr size_t off_beta = off_A + (size_t)C * LDA * 4;
    static constexpr size_t off_scale = off_beta + C * 4;  // sTileF; sPart before it
    static constexpr size_t scale_bytes = (size_t)NCS * DK * 4;
    static constexpr size_t part_bytes = (size_t)NPART * DK * 4;
    static constexpr size_t bytes = off_scale + (scale_bytes > part_bytes ? scale_bytes : part_bytes);
    static_assert((size_t)NBND * DK * 4 <= (size_t)C * LDA * 4, "sBnd fits in sA");
};

// RAW: q, k, g and beta are raw projections; the pre-path transforms
// (q, k scaled to unit L2 norm over d_k per token and head, g <- -softplus(g),
// beta <- sigmoid(beta); "Kimi Linear architecture", section "KDA: a memo that
// erases and rewrites": one forget rate in (0, 1) per channel) are applied
// here in fp32 as the values are loaded, each result rounded once to E.
// bf16: two workgroups per compute unit fit the LDS, so the registers are
// held to what two of them can have (the raw pre-path would otherwise take a
// few more and halve the occupancy); fp32 fits one workgroup per unit.
template <typename E, int DK, int DV, bool HG, bool RAW>
__global__ __launch_bounds__(kIntraThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 4 : 1)))
void intra_chunk_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ g,
    const E* __restrict__ beta, const WsHeader* __restrict__ hdr, const int2* __restrict__ chunk_tab,
    int32_t H, E* __restrict__ Wo, E* __restrict__ QGo,
    E* __restrict__ KdTo, E* __restrict__ Upo, E* __restrict__ Po, float* __restrict__ Gno) {
    using L = IntraLayout<E, DK, DV>;
    constexpr int C = L::C, LDK = L::LDK, LDT = L::LDT, LDA = L::LDA;
    constexpr int NPART = L::NPART, RPT = L::RPT, RPTV = L::RPTV;

    extern __shared__ __align__(16) unsigned char smem[];
    E* sKr = reinterpret_cast<E*>(smem);   // k_t e^{b_t - b_m(t)}, m(t) = middle row of t's tile
    E* sQr = sKr + C * LDK;                // q_t e^{b_t - b_m(t)}
    E* sKt = sQr + C * LDK;                // k_i e^{b_m(i) - b_i}
    E* sKbt = reinterpret_cast<E*>(smem);  // reuses R1 once A and P are done
    E* sVt = sKbt + DK * LDT;
    float* sA = reinterpret_cast<float*>(smem + L::off_A);
    float* sBnd = sA;  // [12][DK] tile-boundary prefix sums, dead before A is written
    float* sBeta = reinterpret_cast<float*>(smem + L::off_beta);
    float* sTileF = reinterpret_cast<float*>(smem + L::off_scale);  // [12][DK] tile-pair factors
    float* sPart = sTileF;  // [NPART][DK], dead before the tile factors are written

    // One workgroup per (chunk, head), heads fastest over the grid, so that the
    // workgroups resident at any time cover a few consecutive chunks of every
    // head: one contiguous span of the token-major inputs and of the workspace.
    const int cid = (int)(blockIdx.x / (unsigned)H);
    const int h = (int)(blockIdx.x - (unsigned)cid * (unsigned)H);
    // Both loads are issued together: the table entry (within the grid, set
    // for every chunk below the total) is only trusted once the total admits
    // it.  The length test never fires for a valid chunk; it is there so that
    // the compiler cannot defer the table load past the branch.
    const int total = hdr->total_chunks;  // zero when the sequence offsets were rejected
    const int2 tab = chunk_tab[cid];
    if ((cid >= total) | (tab.y <= 0)) return;
    const int64_t t0 = tab.x;
    const int len = tab.y;
    const int64_t ch = (int64_t)cid * H + h;  // chunk-head index into the workspace

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // ---- 0. every global load of the chunk, issued up front ----------------
    // In the order of first use (g for step 1, k and q for step 2, v and beta
    // by the end of step 2); loads complete in order, so each step waits only
    // for its own inputs.  Rows past the chunk's end load the last valid row
    // and are zeroed where they are first used: a load under a condition
    // would make the compiler wait for it right at the branch.
    const int cp = tid % (DK / 2), part = tid / (DK / 2);
    const int c0 = 2 * cp;
    const int jp = tid % (DV / 2), vpart = tid / (DV / 2);
    const int j0 = 2 * jp;
    auto clamp_row = [&](int row) { return min(row, len - 1); };
    Pair2<E> graw[RPT], kraw[RPT], qraw[RPT], vraw[RPTV];
    float gh[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int64_t tr = t0 + clamp_row(part * RPT + r);
        if (HG) gh[r] = Elt<E>::load(g + tr * H + h);
        else graw[r].load(g + (tr * H + h) * DK + c0);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int64_t off = ((t0 + clamp_row(part * RPT + r)) * H + h) * DK + c0;
        kraw[r].load(k + off);
        qraw[r].load(q + off);
    }
#pragma unroll
    for (int r = 0; r < RPTV; ++r) vraw[r].load(v + ((t0 + clamp_row(vpart * RPTV + r)) * H + h) * DV + j0);
    // beta of token `lane`, loaded by every wave (same 64 values) so that its
    // store into LDS needs no branch for the compiler to sink the load into
    float beta_raw = Elt<E>::load(beta + (t0 + clamp_row(lane)) * H + h);
    auto row_ok = [&](int r) { return part * RPT + r < len; };

    // ---- 0b. raw projections: the pre-path transforms, in fp32, each result
    // rounded once to E in place of the loaded value (the values
    // kda_prepare_inputs writes, up to the order of the norm's sum):
    // g <- -softplus(g) and beta <- sigmoid(beta) here, where only g's loads
    // are waited for; q and k are scaled to unit L2 norm where step 2 first
    // reads them, so that their loads stay in flight through step 1.
    if constexpr (RAW) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            if (HG) gh[r] = Elt<E>::to(Elt<E>::from(neg_softplus<E>(gh[r])));
            else graw[r].set(neg_softplus<E>(graw[r].lo()), neg_softplus<E>(graw[r].hi()));
        }
    }
    // the log-gate of row r, channel c0 + i (per head: the row's value)
    auto gate_of = [&](int r, int i) -> float { return HG ? gh[r] : (i ? graw[r].hi() : graw[r].lo()); };

    // ---- 1. chunk-local inclusive prefix sum of the log-gate ----------------
    // in base-2 units (b log2(e)), so that every decay factor below is a bare
    // exp2
    float bb[RPT][2];
    {
        float run0 = 0.f, run1 = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            run0 = fmaf(row_ok(r) ? gate_of(r, 0) : 0.f, kLog2e, run0);
            run1 = fmaf(row_ok(r) ? gate_of(r, 1) : 0.f, kLog2e, run1);
            bb[r][0] = run0;
            bb[r][1] = run1;
        }
        sPart[part * DK + c0] = run0;
        sPart[part * DK + c0 + 1] = run1;
    }
    lds_barrier();
    {
        // every partial read at once (one wait), then summed in order
        float2 pv[NPART - 1];
#pragma unroll
        for (int p = 0; p < NPART - 1; ++p) pv[p] = *reinterpret_cast<const float2*>(sPart + p * DK + c0);
        float off0 = 0.f, off1 = 0.f;
#pragma unroll
        for (int p = 0; p < NPART - 1; ++p) {
            if (p < part) {
                off0 += pv[p].x;
                off1 += pv[p].y;
            }
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            bb[r][0] += off0;
            bb[r][1] += off1;
            const int row = part * RPT + r, tr = row & 15;
            const int slot = (tr == 0) ? 0 : (tr == 8) ? 1 : (tr == 15) ? 2 : -1;
            if (slot >= 0) {
                sBnd[(3 * (row >> 4) + slot) * DK + c0] = bb[r][0];
                sBnd[(3 * (row >> 4) + slot) * DK + c0 + 1] = bb[r][1];
            }
        }
    }
    lds_barrier();
    const float last0 = sBnd[11 * DK + c0], last1 = sBnd[11 * DK + c0 + 1];

    // ---- 2. decayed operands and tile-pair scales ---------------------------
    // All three operands of A and P are referred to the middle row m of
    // their 16-row tile: Kr = k e^{b - b_m}, Qr = q e^{b - b_m},
    // Kt = k e^{b_m - b}.  Each factor spans at most eight tokens of decay,
    // so it stays a normal fp32 / bf16 number whenever the decay over eight
    // tokens is above e^-80 (exponents are capped at 80 beyond that).
    // e^{b} and e^{b_last - b} are <= 1.  (b is held in base-2 units: e^{x} is
    // computed as 2^{x log2(e)}.)
    // Over a thread's consecutive rows each of the four factors changes by
    // the row's own gate factor e^{g_t}: e^{b - b_m} and e^{b} shrink along
    // the rows, e^{b_m - b} and e^{b_last - b} grow.  So each is taken
    // directly at its largest row only and follows from there by products
    // with the gate factors (all <= 1): 24 exponentials per thread instead of
    // 64, and no intermediate value exceeds the first.
    constexpr float kCap2 = 80.f * kLog2e;
    static_assert(16 % RPT == 0, "a thread's rows lie in one tile");
    float kx[RPT][2];  // k e^b; times beta it is the W right-hand side
    E kd0[RPT], kd1[RPT];
    const float* bm = sBnd + (3 * ((part * RPT) >> 4) + 1) * DK;  // tile middle
    float eg[RPT][2];  // e^{g} of rows 1..RPT-1 (1 past the end of the chunk)
#pragma unroll
    for (int r = 1; r < RPT; ++r) {
        const bool ok = row_ok(r);
        if (HG) {
            eg[r][0] = eg[r][1] = gate_exp2<E>(ok ? gate_of(r, 0) * kLog2e : 0.f);
        } else {
            eg[r][0] = gate_exp2<E>(ok ? gate_of(r, 0) * kLog2e : 0.f);
            eg[r][1] = gate_exp2<E>(ok ? gate_of(r, 1) * kLog2e : 0.f);
        }
    }
    // e^{b_m - b} and e^{b_last - b}: from the last row back.  min(b_m - b, cap)
    // is written as -max(b - b_m, -cap), the same value.
    float ff[RPT][2], dd[RPT][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        ff[RPT - 1][j] = gate_exp2<E>(-fmaxf(bb[RPT - 1][j] - bm[c0 + j], -kCap2));
        dd[RPT - 1][j] = gate_exp2<E>((j ? last1 : last0) - bb[RPT - 1][j]);
    }
#pragma unroll
    for (int r = RPT - 2; r >= 0; --r)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            ff[r][j] = ff[r + 1][j] * eg[r + 1][j];
            dd[r][j] = dd[r + 1][j] * eg[r + 1][j];
        }
    // e^{b - b_m} and e^{b}: from the first row on
    float e0 = gate_exp2<E>(fminf(bb[0][0] - bm[c0], kCap2)), e1 = gate_exp2<E>(fminf(bb[0][1] - bm[c0 + 1], kCap2));
    float x0 = gate_exp2<E>(bb[0][0]), x1 = gate_exp2<E>(bb[0][1]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = part * RPT + r;
        const bool ok = row_ok(r);
        if constexpr (RAW) {
            // q and k of this row to unit L2 norm over d_k: the row's
            // channels lie in DK / 2 consecutive lanes of one wave (two per
            // lane; every lane takes part, rows past the end hold a copy of
            // the last row); an all-zero row stays zero
            const float rq0 = qraw[r].lo(), rq1 = qraw[r].hi(), rk0 = kraw[r].lo(), rk1 = kraw[r].hi();
            const float iq = inv_norm<E>(lane_group_sum<DK / 2>(rq0 * rq0 + rq1 * rq1));
            const float ik = inv_norm<E>(lane_group_sum<DK / 2>(rk0 * rk0 + rk1 * rk1));
            qraw[r].set(rq0 * iq, rq1 * iq);
            kraw[r].set(rk0 * ik, rk1 * ik);
        }
        const float k0 = ok ? kraw[r].lo() : 0.f, k1 = ok ? kraw[r].hi() : 0.f;
        const float q0 = ok ? qraw[r].lo() : 0.f, q1 = ok ? qraw[r].hi() : 0.f;
        if (r > 0) {
            e0 *= eg[r][0];
            e1 *= eg[r][1];
            x0 *= eg[r][0];
            x1 *= eg[r][1];
        }
        store2<E>(sKr + row * LDK + c0, k0 * e0, k1 * e1);
        store2<E>(sQr + row * LDK + c0, q0 * e0, q1 * e1);
        store2<E>(sKt + row * LDK + c0, k0 * ff[r][0], k1 * ff[r][1]);
        store2<E>(QGo + ch * C * DK + fm_off<DK>(row, frag_pos(c0)), q0 * x0, q1 * x1);
        kx[r][0] = k0 * x0;
        kx[r][1] = k1 * x1;
        kd0[r] = Elt<E>::from(k0 * dd[r][0]);
        kd1[r] = Elt<E>::from(k1 * dd[r][1]);
    }
    {
        E* p0 = KdTo + ch * DK * C;
#pragma unroll
        for (int r4 = 0; r4 < RPT / 4; ++r4) {
            const int pos = frag_pos(part * RPT + 4 * r4);  // 4 consecutive tokens stay contiguous
            store_run4<E>(p0 + fm_off<C>(c0, pos), kd0 + 4 * r4);
            store_run4<E>(p0 + fm_off<C>(c0 + 1, pos), kd1 + 4 * r4);
        }
        if (part == 0) {
            Gno[ch * DK + c0] = gate_exp2<E>(last0);
            Gno[ch * DK + c0 + 1] = gate_exp2<E>(last1);
        }
    }
    // Tile pairs.  Diagonal (ti, ti): e^{b_t - b_i} = Kr-side e^{b_t - b_m} times
    // Kt-side e^{b_m - b_i}, no further factor.  Below the diagonal (tj < ti)
    // the row operands are taken to the tile start s(ti), and the column
    // operand (shared by A and P) to the end e(tj) of its tile and then on to
    // s(ti):
    //   e^{b_t - b_i} = (e^{b_t - b_m(ti)} e^{b_m(ti) - b_s(ti)})
    //                   * ((e^{b_m(tj) - b_i} e^{b_e(tj) - b_m(tj)}) e^{b_s(ti) - b_e(tj)}),
    // factors <= 1 applied one after another, so no intermediate value drops
    // below the final product (anything that underflows is negligible).
    //   sTileF[ti - 1]     e^{b_m(ti) - b_s(ti)}, ti = 1..3
    //   sTileF[3 + tj]     e^{b_e(tj) - b_m(tj)}, tj = 0..2
    //   sTileF[6 + p]      e^{b_s(ti) - b_e(tj)}, p = ti (ti - 1) / 2 + tj
    for (int e = tid; e < L::NCS * DK; e += kIntraThreads) {
        const int v = e / DK, c = e % DK;
        float x;
        if (v < 3) {
            x = sBnd[(3 * (v + 1) + 1) * DK + c] - sBnd[(3 * (v + 1)) * DK + c];
        } else if (v < 6) {
            x = sBnd[(3 * (v - 3) + 2) * DK + c] - sBnd[(3 * (v - 3) + 1) * DK + c];
        } else {
            const int p = v - 6;
            const int ti = (p >= 3) ? 3 : (p >= 1) ? 2 : 1;
            const int tj = p - ti * (ti - 1) / 2;
            x = sBnd[(3 * ti) * DK + c] - sBnd[(3 * tj + 2) * DK + c];
        }
        sTileF[v * DK + c] = gate_exp2<E>(x);
    }
    if constexpr (RAW) beta_raw = Elt<E>::to(Elt<E>::from(sigmoid<E>(beta_raw)));
    sBeta[lane] = lane < len ? beta_raw : 0.f;  // every wave writes the same values
    lds_barrier();

    // ---- 3. A = K K^T with decay (strictly lower, row-scaled by beta) -> LDS
    //         (fp32);  P = Q K^T with decay (lower incl. diagonal) -> workspace
    // The ten lower tile pairs (ti, tj) over the eight waves.  An off-diagonal
    // pair rescales its fragments before every product, a diagonal pair does
    // not, so each of waves 2-7 takes one off-diagonal pair, (1,0) (2,0) (2,1)
    // (3,0) (3,1) (3,2), and waves 0 and 1 two diagonal pairs each plus the
    // zero tiles above the diagonal: no wave has two rescaled pairs in a row.
    int npair, pti0, ptj0, pti1 = 0, ptj1 = 0;
    if (wave < 2) {
        npair = 2;
        pti0 = ptj0 = 2 * wave;
        pti1 = ptj1 = 2 * wave + 1;
    } else {
        npair = 1;
        const int p = wave - 2;
        pti0 = p < 1 ? 1 : (p < 3 ? 2 : 3);
        ptj0 = p - pti0 * (pti0 - 1) / 2;
    }
    f32x4 accPt[2];
#pragma unroll
    for (int pq = 0; pq < 2; ++pq) {
        if (pq < npair) {
            const int ti = pq ? pti1 : pti0, tj = pq ? ptj1 : ptj0;
            f32x4 accA = zero4(), accP = zero4();
            const bool diag = tj == ti;
            // the factors are read for diagonal pairs too (and not used), so
            // that every read of a step goes out together; the rows are
            // clamped into the table
            const float* rowf = sTileF + max(ti - 1, 0) * DK;
            const float* colf = sTileF + min(3 + tj, 5) * DK;
            const float* midf = sTileF + min(6 + ti * (ti - 1) / 2 + tj, L::NCS - 1) * DK;
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const int cb = 32 * ks + 8 * lg;
                Frag<E> fb = ld_frag(sKt + (16 * tj + lr) * LDK + cb);
                Frag<E> fa = ld_frag(sKr + (16 * ti + lr) * LDK + cb);
                Frag<E> fq = ld_frag(sQr + (16 * ti + lr) * LDK + cb);
                float fr[8], fc[8], fm[8];
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4) {
                    *reinterpret_cast<f32x4*>(fr + 4 * h4) = *reinterpret_cast<const f32x4*>(rowf + cb + 4 * h4);
                    *reinterpret_cast<f32x4*>(fc + 4 * h4) = *reinterpret_cast<const f32x4*>(colf + cb + 4 * h4);
                    *reinterpret_cast<f32x4*>(fm + 4 * h4) = *reinterpret_cast<const f32x4*>(midf + cb + 4 * h4);
                }
                if (!diag) {
                    fb = scale_frag(fb, fc, fm);
                    fa = scale_frag(fa, fr);
                    fq = scale_frag(fq, fr);
                }
                accA = mma(fa, fb, accA);
                accP = mma(fq, fb, accP);
            }
            // beta of the lane's four rows, one 16-byte read
            const f32x4 bt4 = *reinterpret_cast<const f32x4*>(sBeta + 16 * ti + 4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + 4 * lg + i, col = 16 * tj + lr;
                lds_put(&sA[row * LDA + col], (row > col) ? accA[i] * bt4[i] : 0.f);
                accPt[pq][i] = (row >= col) ? accP[i] : 0.f;
            }
        }
    }
    // zero tiles of A above the diagonal: (0,1) (0,2) (0,3) by wave 0,
    // (1,2) (1,3) (2,3) by wave 1
    auto upper_tile = [&](int z, int& ti, int& tj) {
        const int zz = (wave == 0) ? z : z + 3;  // 0..5 over (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        ti = zz < 3 ? 0 : (zz < 5 ? 1 : 2);
        tj = zz < 3 ? zz + 1 : (zz < 5 ? zz - 1 : 3);
    };
    if (wave < 2) {
#pragma unroll
        for (int z = 0; z < 3; ++z) {
            int ti, tj;
            upper_tile(z, ti, tj);
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_put(&sA[(16 * ti + 4 * lg + i) * LDA + 16 * tj + lr], 0.f);
        }
    }
    lds_barrier();
    {
        E* sPst = reinterpret_cast<E*>(smem + L::off_Pst);
#pragma unroll
        for (int pq = 0; pq < 2; ++pq) {
            if (pq < npair) {
                const int ti = pq ? pti1 : pti0, tj = pq ? ptj1 : ptj0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_put(&sPst[(16 * ti + 4 * lg + i) * L::LDP + frag_pos(16 * tj + lr)], Elt<E>::from(accPt[pq][i]));
            }
        }
        if (wave < 2) {
#pragma unroll
            for (int z = 0; z < 3; ++z) {
                int ti, tj;
                upper_tile(z, ti, tj);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_put(&sPst[(16 * ti + 4 * lg + i) * L::LDP + frag_pos(16 * tj + lr)], Elt<E>::from(0.f));
            }
        }
    }

    // ---- 4. right-hand sides into the freed region; T = (I + A)^{-1} ---------
    {
        E r0[RPT], r1[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float bt = sBeta[part * RPT + r];
            r0[r] = Elt<E>::from(bt * kx[r][0]);
            r1[r] = Elt<E>::from(bt * kx[r][1]);
        }
        store_seq<E, RPT>(sKbt + c0 * LDT + part * RPT, r0);
        store_seq<E, RPT>(sKbt + (c0 + 1) * LDT + part * RPT, r1);
    }
    {
        E r0[RPTV], r1[RPTV];
#pragma unroll
        for (int r = 0; r < RPTV; ++r) {
            const bool ok = vpart * RPTV + r < len;
            const float bt = sBeta[vpart * RPTV + r];
            r0[r] = Elt<E>::from(ok ? bt * vraw[r].lo() : 0.f);
            r1[r] = Elt<E>::from(ok ? bt * vraw[r].hi() : 0.f);
        }
        store_seq<E, RPTV>(sVt + j0 * LDT + vpart * RPTV, r0);
        store_seq<E, RPTV>(sVt + (j0 + 1) * LDT + vpart * RPTV, r1);
    }
    // (a) the four 16x16 diagonal blocks, one column per thread of wave 0
    float x[16];
    if (tid < 64) {
        const int blk = tid >> 4, jc = tid & 15;
        const float* Ab = sA + (16 * blk) * LDA + 16 * blk;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < t; ++i) acc -= Ab[t * LDA + i] * x[i];
            x[t] = (t < jc) ? 0.f : ((t == jc) ? 1.f : acc);
        }
    }
    lds_barrier();
    copy_tile_out_frag<E, C, C, true>(Po + ch * C * C, reinterpret_cast<const E*>(smem + L::off_Pst), L::LDP, tid);
    if (tid < 64) {
        const int blk = tid >> 4, jc = tid & 15;
        float* Tb = sA + (16 * blk) * LDA + 16 * blk;
#pragma unroll
        for (int t = 0; t < 16; ++t) Tb[t * LDA + jc] = x[t];
    }
    lds_barrier();
    // (b) off-diagonal blocks in two levels, on the matrix cores in fp32
    //     (16x16x4).  With T_a and T_b the inverses of the leading and the
    //     trailing 32 x 32 diagonal blocks of I + A (T of a block-triangular
    //     [[M_a, 0], [A_ba, M_b]] is [[T_a, 0], [-T_b A_ba T_a, T_b]]):
    //       level 1  T10 = -T11 A10 T00 (wave 0),  T32 = -T33 A32 T22 (wave 1);
    //       level 2  Z = A_ba T_a:  Z20 = A20 T00 + A21 T10,  Z21 = A21 T11,
    //                Z30 = A30 T00 + A31 T10,  Z31 = A31 T11   (waves 0-3),
    //                then T_ba = -T_b Z:  T20 = -T22 Z20,  T21 = -T22 Z21,
    //                T30 = -(T32 Z20 + T33 Z30),  T31 = -(T32 Z21 + T33 Z31).
    //     With k = 4g + s for lane group g and step s, the accumulators of a
    //     product are exactly the B operand of the next one.  Z goes through
    //     the P staging tile, free once P has been copied out.
    {
        constexpr int LDZ = 36;  // [32][LDZ] fp32: rows of block rows 2 and 3, columns of block columns 0 and 1
        float* sZ = reinterpret_cast<float*>(smem + L::off_Pst);
        static_assert((size_t)32 * LDZ * 4 <= (size_t)C * L::LDP * sizeof(E), "Z fits in the P staging tile");
        // X += A[bi][m] T[m][bj]
        auto mul_AT = [&](int bi, int m, int bj, f32x4 X) {
            const f32x4 am = *reinterpret_cast<const f32x4*>(sA + (16 * bi + lr) * LDA + 16 * m + 4 * lg);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                X = __builtin_amdgcn_mfma_f32_16x16x4f32(am[jj], sA[(16 * m + 4 * lg + jj) * LDA + 16 * bj + lr], X, 0,
                                                         0, 0);
            return X;
        };
        // Y += T[bi][m] X, X in accumulator layout
        auto mul_TX = [&](int bi, int m, f32x4 X, f32x4 Y) {
            const f32x4 tm = *reinterpret_cast<const f32x4*>(sA + (16 * bi + lr) * LDA + 16 * m + 4 * lg);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tm[jj], X[jj], Y, 0, 0, 0);
            return Y;
        };
        auto put_block = [&](int bi, int bj, f32x4 Y) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) lds_put(&sA[(16 * bi + 4 * lg + ii) * LDA + 16 * bj + lr], -Y[ii]);
        };
        if (wave < 2) {  // level 1: block (i0 + 1, i0), i0 = 0 or 2
            const int i0 = 2 * wave;
            const f32x4 X = mul_AT(i0 + 1, i0, i0, zero4());
            put_block(i0 + 1, i0, mul_TX(i0 + 1, i0 + 1, X, zero4()));
        }
        lds_barrier();
        const int zi = 2 + (wave >> 1), zj = wave & 1;  // block (zi, zj) of level 2, waves 0-3
        if (wave < 4) {
            f32x4 Z = zero4();
            for (int m = zj; m < 2; ++m) Z = mul_AT(zi, m, zj, Z);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) lds_put(&sZ[(16 * (zi - 2) + 4 * lg + ii) * LDZ + 16 * zj + lr], Z[ii]);
        }
        lds_barrier();
        if (wave < 4) {
            f32x4 Y = zero4();
            for (int m = 2; m <= zi; ++m) {
                f32x4 Zm;  // Z[m][zj] in accumulator layout
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) Zm[jj] = sZ[(16 * (m - 2) + 4 * lg + jj) * LDZ + 16 * zj + lr];
                Y = mul_TX(zi, m, Zm, Y);
            }
            put_block(zi, zj, Y);
        }
        lds_barrier();
    }

    // ---- 5. W = T (beta K e^b),  U' = T (beta V), staged for 16-byte stores --
    {
        // wave w: token tile ti = w % 4, half (w / 4) of the W and U' columns
        const int ti = wave & 3, half = wave >> 2;
        constexpr int TNW = DK / 32, TNU = DV / 32;  // 16-column tiles per half
        const Frag<E> ft0 = ld_frag_from_f32<E>(sA + (16 * ti + lr) * LDA + 8 * lg);
        const Frag<E> ft1 = ld_frag_from_f32<E>(sA + (16 * ti + lr) * LDA + 32 + 8 * lg);
        // (rows 0..31 of T are exactly zero beyond token 31, so for ti < 2 the
        // second product adds exact zeros; it is issued anyway to keep the
        // accumulation unconditional)
        f32x4 accW[TNW], accU[TNU];
#pragma unroll
        for (int u = 0; u < TNW; ++u) {
            const int tn = half * TNW + u;
            accW[u] = mma(ft0, ld_frag(sKbt + (16 * tn + lr) * LDT + 8 * lg), zero4());
            accW[u] = mma(ft1, ld_frag(sKbt + (16 * tn + lr) * LDT + 32 + 8 * lg), accW[u]);
        }
#pragma unroll
        for (int u = 0; u < TNU; ++u) {
            const int tn = half * TNU + u;
            accU[u] = mma(ft0, ld_frag(sVt + (16 * tn + lr) * LDT + 8 * lg), zero4());
            accU[u] = mma(ft1, ld_frag(sVt + (16 * tn + lr) * LDT + 32 + 8 * lg), accU[u]);
        }
        // U' for the walk: per 16-column slice tn and lane, the 16 values the
        // lane holds in the walk's accumulator layout (token tiles ti = 0..3,
        // rows 4 lg + i), contiguous: [tn][lane][ti][i].
        {
            E* up = Upo + ch * C * DV;
#pragma unroll
            for (int u = 0; u < TNU; ++u) {
                const int tn = half * TNU + u;
                E vals[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) vals[i] = Elt<E>::from(accU[u][i]);
                store_run4<E>(up + (tn * 64 + lane) * 16 + 4 * ti, vals);
            }
        }
        lds_barrier();  // every wave is done with sKbt / sVt / sA
        E* sWst = reinterpret_cast<E*>(smem);  // [C][DK], channel columns in fragment order
#pragma unroll
        for (int u = 0; u < TNW; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds_put(&sWst[(16 * ti + 4 * lg + i) * LDK + frag_pos(16 * (half * TNW + u) + lr)],
                        Elt<E>::from(accW[u][i]));
        lds_barrier();
        copy_tile_out_frag<E, C, DK>(Wo + ch * C * DK, sWst, LDK, tid);
    }
}

// ----------------------------------------------------------------------------
// State walk + output.  One workgroup per (sequence n, head h, 16-column slice
// of d_v), four waves that never meet at a barrier:
//   wave 0 (chain)   keeps the fp32 d_k x 16 slice of S in accumulator
//                    registers and walks the chunks: U = U' - W S, then
//                    S <- Diag(Gn) S + KdT U.  The bf16 (or fp32) fragments of
//                    S and U it builds for its own products are also handed to
//                    wave 1 through a ring of kRing slots in LDS.
//   wave 1 (output)  O = QG S + P U for each chunk from those fragments; QG
//                    and P come straight from global memory.
//   wave 2 (stager)  copies the chain's operands of each chunk (W, KdT, this
//                    slice of U', Gn) into a ring of R operand slots in LDS
//                    with 16-byte LDS-DMA loads, so that the chain wave issues
//                    no global loads at all and reads its fragments from LDS.
//                    When R slots do not fit in LDS (fp32 at d = 128) the
//                    chain loads its operands from global memory itself and
//                    this wave has nothing to do.
//   wave 3 (prefetch) touches the cache lines of the chunks up to
//                    kWalkPrefetch ahead of wave 0 (LDS-DMA loads into a sink:
//                    no registers), so that waves 1 and 2 find them in L2.
// Hand-over is by LDS progress counters (absolute chunk indices):
//   ready  chunks whose operand slot the stager has filled,
//   freed  chunks whose operand slot the chain has finished reading,
//   progA  chunks whose S and U fragments the chain has published,
//   doneB  chunks whose S and U slot the output wave has finished reading.
// Every wait is bounded by kSpinLimit sleeps, past which the wave records a
// timeout in the workspace header and proceeds (results are then
// unspecified).
// Operands W, QG (channel columns) and KdT, P (token columns) are stored in
// fragment order (frag_pos), so accumulator registers serve directly as the B
// fragment of the next product, and fragment-major (fm_off), so every
// fragment is one contiguous 1 KB block, copied into LDS unchanged; U' is
// stored per slice in the accumulator layout of the walk's lanes.
#ifndef KDA_WALK_RING
#define KDA_WALK_RING 2
#endif
#ifndef KDA_WALK_SLOTS
#define KDA_WALK_SLOTS 4
#endif
constexpr int kRing = KDA_WALK_RING;          // S/U hand-over slots
constexpr int kMaxSlots = KDA_WALK_SLOTS;     // most operand slots staged ahead
#ifndef KDA_WALK_PREFETCH
#define KDA_WALK_PREFETCH 5
#endif
constexpr int kWalkPrefetch = KDA_WALK_PREFETCH;
constexpr int kWalkThreads = 256;
constexpr int kSpinLimit = 1 << 22;

// LDS layout of the walk workgroup (dynamic shared memory).
template <typename E, int DK, int DV>
struct WalkLayout {
    static constexpr int C = kChunk;
    static constexpr int KS = DK / 32, KB = C / 32;
    static constexpr int ESZ = (int)sizeof(E);
    static constexpr int LDO = 16 + 16 / ESZ;  // padded row of the O staging tile
    // one operand slot: W | KdT | U' (this slice) | Gn
    static constexpr int W_B = C * DK * ESZ, K_B = DK * C * ESZ, U_B = 64 * 16 * ESZ, G_B = DK * 4;
    static constexpr int SLOT = W_B + K_B + U_B + G_B;
    static constexpr int RING_S = kRing * KS * 64 * (int)sizeof(Frag<E>);
    static constexpr int RING_U = kRing * KB * 64 * (int)sizeof(Frag<E>);
    static constexpr int O_B = (C * LDO * ESZ + 15) / 16 * 16;
    static constexpr int SINK_B = 256, CNT_B = 64;
    static constexpr int FIXED = RING_S + RING_U + 2 * O_B + SINK_B + CNT_B;
    static constexpr int RFIT = (kLdsBytes - FIXED) / SLOT;
    static constexpr int R = RFIT > kMaxSlots ? kMaxSlots : RFIT;  // operand slots
    static constexpr bool STAGED = R >= 2;
    static constexpr int OPS_B = STAGED ? R * SLOT : 0;
    static constexpr int off_ringS = OPS_B, off_ringU = off_ringS + RING_S, off_O = off_ringU + RING_U;
    static constexpr int off_sink = off_O + 2 * O_B, off_cnt = off_sink + SINK_B;
    static constexpr int bytes = off_cnt + CNT_B;
    // LDS-DMA loads per chunk: 1 KB blocks of W, KdT and U', one load for Gn
    static constexpr int LPC = W_B / 1024 + K_B / 1024 + U_B / 1024 + 1;
    static_assert(W_B % 1024 == 0 && K_B % 1024 == 0 && U_B % 1024 == 0 && G_B <= 1024 && G_B % 16 == 0, "blocks");
    static_assert(!STAGED || LPC <= 63, "one chunk of loads within the vector-memory counter");
    static_assert(bytes <= kLdsBytes, "LDS budget");
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kWalkThreads) void chunk_walk_kernel(
    WsHeader* __restrict__ hdr, const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int32_t N,
    int32_t H, const E* __restrict__ Wi, const E* __restrict__ QGi, const E* __restrict__ KdTi,
    const E* __restrict__ UpTi, const E* __restrict__ Pi, const float* __restrict__ Gni,
    const float* __restrict__ S0, float* __restrict__ S_T, E* __restrict__ o) {
    using L = WalkLayout<E, DK, DV>;
    constexpr int C = kChunk;
    constexpr int NS = DV / 16;  // slices per (n, h)
    constexpr int MT = DK / 16;  // 16-row tiles of the state slice
    constexpr int KS = L::KS;    // 32-blocks over channels
    constexpr int TT = C / 16;   // 16-row tiles of tokens
    constexpr int KB = L::KB;    // 32-blocks over tokens
    constexpr int LDO = L::LDO;
    constexpr int R = L::R;
    extern __shared__ __align__(16) char walk_smem[];
    char* const ops = walk_smem;
    Frag<E>* const ringS = reinterpret_cast<Frag<E>*>(walk_smem + L::off_ringS);  // [kRing][KS][64]
    Frag<E>* const ringU = reinterpret_cast<Frag<E>*>(walk_smem + L::off_ringU);  // [kRing][KB][64]
    E* const sO = reinterpret_cast<E*>(walk_smem + L::off_O);                     // [2][O_B / ESZ]
    float* const sSink = reinterpret_cast<float*>(walk_smem + L::off_sink);
    int* const cnt = reinterpret_cast<int*>(walk_smem + L::off_cnt);
    int* const progA = cnt;      // chunks published by the chain wave
    int* const doneB = cnt + 1;  // chunks consumed by the output wave
    int* const ready = cnt + 2;  // chunks staged by the stager wave
    int* const freed = cnt + 3;  // chunks whose operand slot the chain released
    int* const oready = cnt + 4;   // chunks whose O tile the output wave has staged
    int* const ostored = cnt + 5;  // chunks whose O tile the store wave has read

    if (hdr->bad_seqlens) return;
    const int64_t NH = (int64_t)N * H;
    const int64_t bid = blockIdx.x;
    int64_t pair;
    int slice;
    if (NH % 8 == 0) {  // keep the NS slices of one (n, h) on one XCD (shared L2)
        const int xcd = (int)(bid & 7);
        const int64_t idx = bid >> 3;
        pair = (idx / NS) * 8 + xcd;
        slice = (int)(idx % NS);
    } else {
        pair = bid / NS;
        slice = (int)(bid % NS);
    }
    const int n = (int)(pair / H), h = (int)(pair % H);
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int col0 = slice * 16;
    const int cbeg = chunk_off[n], cend = chunk_off[n + 1];
    const int64_t seq0 = cu[n], seqend = cu[n + 1];
    if (tid < 6) cnt[tid] = cbeg;
    lds_barrier();  // the only barrier: counters initialised before any wave reads them

    // A wait that gives up only sets timed_out; each wave reports it once, on
    // exit, so that no global store sits inside a loop (a store among this
    // wave's loads would make the compiler wait for all of them at once).
    bool timed_out = false;
    auto report = [&]() {
        if (timed_out) hdr->wait_timeout = 1;
    };
    auto wait_until = [&](const int* counter, int target) {
        for (int spins = 0; lds_read_int(counter) < target; ++spins) {
            if (spins >= kSpinLimit) {
                timed_out = true;
                return;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    };
    auto put_counter = [&](int* counter, int value) {
        if (lane == 0) *(volatile __attribute__((address_space(3))) int*)(counter) = value;
    };
    auto chunk_base = [&](int c) { return (int64_t)c * H + h; };
    auto slot_of = [&](int c) { return ops + ((c - cbeg) % (R > 0 ? R : 1)) * L::SLOT; };

    if (w == 3) {
        // ---------------- prefetch + store wave ----------------
        constexpr int LW = C * DK * (int)sizeof(E) / 128;  // lines of W, of QG, of KdT
        constexpr int LP = C * C * (int)sizeof(E) / 128;
        constexpr int LG = DK * 4 / 128;
        constexpr int NL = 3 * LW + LP + LG;
        constexpr int LU = 64 * 16 * (int)sizeof(E) / 128;  // this slice's part of U'
        static_assert(LU <= 64, "one load per lane");
        auto sink = (__attribute__((address_space(3))) void*)sSink;
        auto prefetch = [&](int c) {
            const int64_t ch = chunk_base(c);
            for (int j = slice + NS * lane; j < NL; j += NS * 64) {
                const char* base;
                int off;
                if (j < LW) { base = (const char*)(Wi + ch * C * DK); off = j; }
                else if (j < 2 * LW) { base = (const char*)(QGi + ch * C * DK); off = j - LW; }
                else if (j < 3 * LW) { base = (const char*)(KdTi + ch * DK * C); off = j - 2 * LW; }
                else if (j < 3 * LW + LP) {
                    base = (const char*)(Pi + ch * C * C);
                    off = j - 3 * LW;
                    constexpr int LB = 64 * 8 * (int)sizeof(E) / 128;  // lines per fragment block
                    if (p_block_zero(off / LB / KB, off / LB % KB)) continue;
                } else { base = (const char*)(Gni + ch * DK); off = j - 3 * LW - LP; }
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base + 128 * off),
                                                 sink, 4, 0, 0);
            }
            if (lane < LU) {
                const char* up = (const char*)(UpTi + ch * DV * C + slice * 64 * 16);
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(up + 128 * lane),
                                                 sink, 4, 0, 0);
            }
        };
        // prefetch every chunk fewer than kWalkPrefetch ahead of the chain
        int pcur = cbeg;
        auto pump = [&]() {
            const int lim = min(cend, lds_read_int(progA) + kWalkPrefetch);
            for (; pcur < lim; ++pcur) prefetch(pcur);
        };
        for (int c = cbeg; c < cend; ++c) {
            // wait for the O tile of chunk c, prefetching meanwhile
            for (int spins = 0;; ++spins) {
                pump();
                if (lds_read_int(oready) > c) break;
                if (spins >= kSpinLimit) {
                    timed_out = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            lds_acquire();
            // each lane stores one token row of the slice (16 outputs); the
            // LDS reads are issued before the counter write, so the output
            // wave cannot overwrite the tile before they are performed
            const E* tile = sO + (c & 1) * (L::O_B / (int)sizeof(E));
            const uint32_t srow = lds_addr(tile + lane * LDO);
            constexpr int NB = 16 * (int)sizeof(E) / 16;  // 16-byte pieces of a row
            uint4 r0, r1, r2, r3;
            // in asm: the compiler would otherwise wait for this wave's
            // prefetch loads (it cannot tell that they write elsewhere in LDS)
            if constexpr (NB == 2) {
                asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(r0), "=v"(r1)
                             : "v"(srow)
                             : "memory");
            } else {
                asm volatile(
                    "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:16\n\t"
                    "ds_read_b128 %2, %4 offset:32\n\tds_read_b128 %3, %4 offset:48\n\ts_waitcnt lgkmcnt(0)"
                    : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3)
                    : "v"(srow)
                    : "memory");
            }
            put_counter(ostored, c + 1);
            const int64_t tok = seq0 + (int64_t)(c - cbeg) * C + lane;
            if (tok < seqend) {
                uint4* drow = reinterpret_cast<uint4*>(o + (tok * H + h) * DV + col0);
                drow[0] = r0;
                drow[1] = r1;
                if constexpr (NB == 4) {
                    drow[2] = r2;
                    drow[3] = r3;
                }
            }
        }
        // No LDS-DMA load may still be in flight when the workgroup's LDS is
        // released.
        wait_vmcnt<0>();
        report();
        return;
    }

    if (w == 2) {
        // ---------------- stager wave ----------------
        if constexpr (L::STAGED) {
            for (int c = cbeg; c < cend; ++c) {
                if (lds_read_int(freed) < c - R + 1) {
                    // about to block on a slot: first finish and announce
                    // every chunk already in flight
                    wait_vmcnt<0>();
                    put_counter(ready, c);
                    wait_until(freed, c - R + 1);
                    lds_acquire();
                }
                const int64_t ch = chunk_base(c);
                char* s = slot_of(c);
                const char* gw = (const char*)(Wi + ch * C * DK) + 16 * lane;
                const char* gk = (const char*)(KdTi + ch * DK * C) + 16 * lane;
                const char* gu = (const char*)(UpTi + ch * DV * C + slice * 64 * 16) + 16 * lane;
#pragma unroll
                for (int i = 0; i < L::W_B / 1024; ++i) lds_dma16(gw + 1024 * i, s + 1024 * i);
#pragma unroll
                for (int i = 0; i < L::K_B / 1024; ++i) lds_dma16(gk + 1024 * i, s + L::W_B + 1024 * i);
#pragma unroll
                for (int i = 0; i < L::U_B / 1024; ++i) lds_dma16(gu + 1024 * i, s + L::W_B + L::K_B + 1024 * i);
                if (lane < L::G_B / 16)
                    lds_dma16((const char*)(Gni + ch * DK) + 16 * lane, s + L::W_B + L::K_B + L::U_B);
                // every load before this chunk's has landed in LDS
                wait_vmcnt<L::LPC>();
                put_counter(ready, c);
            }
            wait_vmcnt<0>();
            put_counter(ready, cend);
        }
        report();
        return;
    }

    if (w == 0) {
        // ---------------- chain wave ----------------
        f32x4 Sreg[MT];
        if (S0) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) Sreg[m][i] = S0[(pair * DK + 16 * m + 4 * lg + i) * DV + col0 + lr];
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m) Sreg[m] = zero4();
        }
        Frag<E> fW[TT][KS], fK[MT][KB];
        typename Raw4<E>::T up[TT];  // U' kept in its stored form until used
        f32x4 gn[MT];
        // operand c is in LDS once `ready` has passed it (staged), else in
        // global memory; `seen` is a value of `ready` read earlier
        auto acquire_ops = [&](int c, int seen) {
            if constexpr (L::STAGED) {
                if (seen < c + 1) wait_until(ready, c + 1);
                lds_acquire();
            }
        };
        auto load_w = [&](int c) {
            const E* Wp;
            if constexpr (L::STAGED) Wp = reinterpret_cast<const E*>(slot_of(c));
            else Wp = Wi + chunk_base(c) * C * DK;
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) fW[t][ks] = ld_frag(Wp + ((t * KS + ks) * 64 + lane) * 8);
        };
        auto load_rest = [&](int c) {
            const E *Kp, *Up;
            const float* Gp;
            if constexpr (L::STAGED) {
                const char* s = slot_of(c);
                Kp = reinterpret_cast<const E*>(s + L::W_B);
                Up = reinterpret_cast<const E*>(s + L::W_B + L::K_B) + lane * 16;
                Gp = reinterpret_cast<const float*>(s + L::W_B + L::K_B + L::U_B);
            } else {
                const int64_t ch = chunk_base(c);
                Kp = KdTi + ch * DK * C;
                Up = UpTi + ch * DV * C + (slice * 64 + lane) * 16;
                Gp = Gni + ch * DK;
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) fK[m][kb] = ld_frag(Kp + ((m * KB + kb) * 64 + lane) * 8);
#pragma unroll
            for (int t = 0; t < TT; ++t) up[t] = Raw4<E>::load(Up + 4 * t);
#pragma unroll
            for (int m = 0; m < MT; ++m) gn[m] = *reinterpret_cast<const f32x4*>(Gp + 16 * m + 4 * lg);
        };
        if (cbeg < cend) {
            acquire_ops(cbeg, cbeg);
            load_w(cbeg);
            load_rest(cbeg);
        }
        for (int c = cbeg; c < cend; ++c) {
            const int slot = (c - cbeg) % kRing;
            const int nxt = min(c + 1, cend - 1);
            // counters read early, checked after the products
            const int freeB = lds_read_int(doneB);
            const int seen = L::STAGED ? lds_read_int(ready) : 0;
            Frag<E> sf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sf[ks] = acc_to_frag(E{}, Sreg[2 * ks], Sreg[2 * ks + 1]);
            // Diag(Gn) S now (S itself is needed again only as the
            // accumulator of KdT U below), overlapping the products
#pragma unroll
            for (int m = 0; m < MT; ++m) Sreg[m] = gn[m] * Sreg[m];
            // U = U' - W S
            f32x4 X[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) X[t] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < TT; ++t) X[t] = mma(fW[t][ks], sf[ks], X[t]);
            // every product is issued before the wave can stall on a counter
            // or an LDS read below: the matrix cores work through the wait
            __builtin_amdgcn_sched_barrier(0);
            acquire_ops(nxt, seen);
            load_w(nxt);
            Frag<E> uf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                uf[kb] = acc_to_frag(E{}, Raw4<E>::widen(up[2 * kb]) - X[2 * kb],
                                     Raw4<E>::widen(up[2 * kb + 1]) - X[2 * kb + 1]);
            // hand S and U to the output wave once its slot is free
            if (freeB < c - kRing + 1) wait_until(doneB, c - kRing + 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ringS[(slot * KS + ks) * 64 + lane] = sf[ks];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) ringU[(slot * KB + kb) * 64 + lane] = uf[kb];
            // S <- Diag(Gn) S + KdT U  (the ring writes drain meanwhile)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int m = 0; m < MT; ++m) Sreg[m] = mma(fK[m][kb], uf[kb], Sreg[m]);
            __builtin_amdgcn_sched_barrier(0);
            // every operand of chunk c has been read (its registers are in
            // use above), and S, U of chunk c are in the ring
            lds_release();
            put_counter(progA, c + 1);
            if constexpr (L::STAGED) put_counter(freed, c + 1);
            load_rest(nxt);
        }
        if (S_T) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) S_T[(pair * DK + 16 * m + 4 * lg + i) * DV + col0 + lr] = Sreg[m][i];
        }
        report();
        return;
    }

    // ---------------- output wave (w == 1) ----------------
    // QG and P of chunk c + 2 are loaded while chunk c is computed (two
    // register sets).  The O tile goes to LDS and wave 3 stores it, so that
    // this wave issues loads only and can wait for exactly the ones it needs.
    struct QP {
        Frag<E> q[TT][KS], p[TT][KB];
    };
    QP opA, opB;
    auto load_qp = [&](QP& x, int c) {
        const int64_t ch = chunk_base(min(c, cend - 1));
        const E* Qp = QGi + ch * C * DK;
        const E* Pp = Pi + ch * C * C;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) x.q[t][ks] = ld_frag(Qp + ((t * KS + ks) * 64 + lane) * 8);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                if (!p_block_zero(t, kb)) x.p[t][kb] = ld_frag(Pp + ((t * KB + kb) * 64 + lane) * 8);
        }
    };
    auto out_chunk = [&](QP& x, int c) {
        const int slot = (c - cbeg) % kRing;
        wait_until(progA, c + 1);
        lds_acquire();
        Frag<E> sf[KS], uf[KB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sf[ks] = ringS[(slot * KS + ks) * 64 + lane];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) uf[kb] = ringU[(slot * KB + kb) * 64 + lane];
        lds_release();  // the reads above have completed
        put_counter(doneB, c + 1);
        f32x4 O[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) O[t] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < TT; ++t) O[t] = mma(x.q[t][ks], sf[ks], O[t]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < TT; ++t)
                if (!p_block_zero(t, kb)) O[t] = mma(x.p[t][kb], uf[kb], O[t]);
        load_qp(x, c + 2);
        // O tile slot c & 1 is free once wave 3 has read chunk c - 2 from it
        wait_until(ostored, c - 1);
        lds_acquire();
        E* tile = sO + (c & 1) * (L::O_B / (int)sizeof(E));
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_put(&tile[(16 * t + 4 * lg + i) * LDO + lr], Elt<E>::from(O[t][i]));
        lds_release();
        put_counter(oready, c + 1);
    };
    if (cbeg < cend) {
        load_qp(opA, cbeg);
        lds_acquire();  // compiler barrier: keep every load of opA ahead of opB's
        load_qp(opB, cbeg + 1);
    }
    for (int c = cbeg; c < cend;) {
        out_chunk(opA, c);
        if (++c >= cend) break;
        out_chunk(opB, c);
        ++c;
    }
    report();
}

// ----------------------------------------------------------------------------
// Segmented walk (bf16 operands, d_k = d_v = 128): the two-level form of the
// chunk chain, for prefills with few (sequence, head) pairs.  The chunks of
// every pair are cut into G segments of consecutive chunks, one workgroup per
// segment, each owning all d_v columns of the state (eight waves, one
// 16-column slice each), so that a chunk's operands are fetched once per head
// rather than once per slice.  The chunk step S <- A_c S + KdT U' with
// A_c = Diag(Gn) - KdT W is affine in S, so a segment maps its start state to
// its end state by S_end = M S_start + B, M the product of its A_c ("Kimi
// Linear architecture", section on the chunkwise form).  Per segment j:
//   pass 1  walk the segment without outputs: B from S = 0 with the inputs,
//           M from the identity without them (U' taken as 0), both with the
//           same W, KdT and Gn.  Segment 0 knows its start state and walks S
//           from S0 instead (B is then its end state; no M).
//   chain   once S_start(j) is published by segment j - 1:
//           S_start(j + 1) = M S_start(j) + B (one 128 x 128 x 128 product,
//           each operand split into two bf16 parts so that the product keeps
//           about 16 bits), published in turn.
//   pass 3  walk the segment again from S_start(j), with outputs; the last
//           segment writes S_T and has no pass 1.
// Workgroups take (segment, pair) from an atomic ticket in segment-major
// order, so a workgroup only ever waits for a segment with a lower ticket,
// which was taken by a workgroup that is resident or done and that itself
// waits only for lower tickets.  Every wait is bounded: on timeout the
// header's wait_timeout is set and the results are unspecified.
// Per chunk, the operands go to LDS by 16-byte LDS-DMA loads spread over the
// eight waves, double-buffered (the next chunk's while this one is
// computed), with two workgroup barriers per chunk; the O tile of a chunk is
// staged in LDS and stored by all waves during the next chunk.  The two
// operand slots are distinct LDS objects and the loops are unrolled by two,
// so that the compiler can tell that the matrix-core operand reads of one
// slot do not depend on the loads in flight into the other.
constexpr int kSegWaves = 8;
constexpr int kSegThreads = 64 * kSegWaves;
constexpr int kSegTarget = 256;          // workgroups wanted: one per compute unit
constexpr int kSegMaxGroups = 64;        // most segments per pair
constexpr int kSegMinChunks = 8;         // fewest chunks per segment (on average)
constexpr int kSegSpinLimit = 1 << 24;   // polls of about 128 clocks: several seconds

struct SegLayout {
    static constexpr int C = kChunk, DK = 128, DV = 128, KS = DK / 32, KB = C / 32;
    static constexpr int W_B = C * DK * 2, K_B = DK * C * 2, U_B = C * DV * 2, Q_B = C * DK * 2;
    static constexpr int P_B = 6 * 1024, G_B = DK * 4;  // P: its 6 nonzero 1 KB fragment blocks
    static constexpr int off_W = 0, off_K = W_B, off_U = off_K + K_B, off_G = off_U + U_B, off_Q = off_G + G_B,
                         off_P = off_Q + Q_B;
    static constexpr int SLOT = off_P + P_B;  // 72,192 B
    static constexpr int LDO = DV + 8;        // O tile row (bf16), padded
    static constexpr int LDM = DK + 8;        // M tile row (bf16), padded; two tiles in the second slot
    static constexpr int M_B = DK * LDM * 2;
    // 1 KB LDS-DMA pieces per chunk: W, KdT, U', Gn (half a piece) in pass 1;
    // then QG and the P blocks in pass 3
    static constexpr int PIECES1 = W_B / 1024 + K_B / 1024 + U_B / 1024 + 1;
    static constexpr int PIECES3 = PIECES1 + Q_B / 1024 + P_B / 1024;
    static constexpr int bytes = 2 * SLOT + C * LDO * 2 + 16;
    static_assert(bytes <= kLdsBytes, "LDS budget");
    static_assert(2 * M_B <= SLOT, "both M tiles fit in the second slot");
};

__global__ __launch_bounds__(kSegThreads) void seg_walk_kernel(
    WsHeader* __restrict__ hdr, int* __restrict__ seg_flags, float* __restrict__ seg_state,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int32_t N, int32_t H, int32_t G,
    const bf16_t* __restrict__ Wi, const bf16_t* __restrict__ QGi, const bf16_t* __restrict__ KdTi,
    const bf16_t* __restrict__ UpTi, const bf16_t* __restrict__ Pi, const float* __restrict__ Gni,
    const float* __restrict__ S0, float* __restrict__ S_T, bf16_t* __restrict__ o) {
    using L = SegLayout;
    using E = bf16_t;
    constexpr int C = kChunk, DK = L::DK, DV = L::DV, KS = L::KS, KB = L::KB;
    constexpr int MT = DK / 16, TT = C / 16;
    __shared__ __align__(16) char slotA[L::SLOT];
    __shared__ __align__(16) char slotB[L::SLOT];
    __shared__ __align__(16) E sO[C * L::LDO];
    __shared__ int sticket;

    if (hdr->bad_seqlens) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
    const int lr = lane & 15, lg = lane >> 4;
    if (tid == 0) sticket = atomicAdd(&hdr->seg_ticket, 1);
    __syncthreads();
    const int64_t NP = (int64_t)N * H;
    const int64_t ticket = __builtin_amdgcn_readfirstlane(sticket);  // uniform: scalar addressing below
    const int j = (int)(ticket / NP);
    const int64_t pair = ticket % NP;
    const int n = (int)(pair / H), h = (int)(pair % H);
    const int cbeg = chunk_off[n], cend = chunk_off[n + 1];
    const int64_t seq0 = cu[n], seqend = cu[n + 1];
    const int seglen = (cend - cbeg + G - 1) / G;
    const int s0 = min(cend, cbeg + j * seglen), s1 = min(cend, s0 + seglen);
    const int col0 = 16 * w;  // this wave's value columns
    const bool first = j == 0, last = j == G - 1;
    // S_start(i) for 1 <= i < G lives at seg_state[pair][i - 1]; its flag is
    // seg_flags[pair][i]
    auto start_state = [&](int i) { return seg_state + (pair * (G - 1) + i - 1) * DK * DV; };

    // this wave's share of the LDS-DMA pieces of chunk c into slot sb
    auto dma_chunk = [&](int c, char* sb, bool pass3) __attribute__((always_inline)) {
        // (chunk, head) index through readfirstlane: opaque to the loop
        // optimiser, which would otherwise keep every piece's address as a
        // 64-bit induction variable in vector registers
        const int64_t ch = (int64_t)__builtin_amdgcn_readfirstlane(c) * H + h;
        const int np = pass3 ? L::PIECES3 : L::PIECES1;
#pragma unroll
        for (int k = 0; k < (L::PIECES3 + kSegWaves - 1) / kSegWaves; ++k) {
            const int p = w + kSegWaves * k;
            if (p >= np) break;
            const char* src;
            int dst;
            if (p < 16) {
                src = (const char*)(Wi + ch * C * DK) + 1024 * p;
                dst = L::off_W + 1024 * p;
            } else if (p < 32) {
                src = (const char*)(KdTi + ch * DK * C) + 1024 * (p - 16);
                dst = L::off_K + 1024 * (p - 16);
            } else if (p < 48) {
                src = (const char*)(UpTi + ch * DV * C) + 1024 * (p - 32);
                dst = L::off_U + 1024 * (p - 32);
            } else if (p == 48) {
                if (lane < L::G_B / 16) lds_dma16((const char*)(Gni + ch * DK) + 16 * lane, sb + L::off_G);
                continue;
            } else if (p < 49 + 16) {
                src = (const char*)(QGi + ch * C * DK) + 1024 * (p - 49);
                dst = L::off_Q + 1024 * (p - 49);
            } else {
                const int b = p - 65;  // b-th kept block of P, (t, kb) in p_block_index order
                const int t = b < 2 ? b : 2 + (b - 2) / 2, kb = b < 2 ? 0 : (b - 2) % 2;
                src = (const char*)(Pi + ch * C * C) + 1024 * (t * KB + kb);
                dst = L::off_P + 1024 * b;
            }
            lds_dma16(src + 16 * lane, sb + dst);
        }
    };
    auto frag_at = [&](const char* sb, int off, int blk) __attribute__((always_inline)) {
        return ld_frag(reinterpret_cast<const E*>(sb + off) + (blk * 64 + lane) * 8);
    };
    // state slices in accumulator layout: lane holds rows 16 m + 4 lg + i of
    // column col0 + lr
    auto load_state = [&](f32x4 (&S)[MT], const float* src) {
        if (src) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[m][i] = src[(16 * m + 4 * lg + i) * DV + col0 + lr];
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m) S[m] = zero4();
        }
    };
    auto store_state = [&](const f32x4 (&S)[MT], float* dst) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * m + 4 * lg + i) * DV + col0 + lr] = S[m][i];
    };
    // The start states pass between workgroups on any of the chip's L2
    // caches, so they are written and read with device-scope accesses, which
    // are coherent at the device level by themselves; a release/acquire pair
    // around plain accesses would instead write back and invalidate a whole
    // L2 at every hand-over.  Ordering: every lane waits for its stores'
    // completion before the barrier that precedes the flag store, and the
    // loads are issued after the flag was seen.
    auto publish_state = [&](const f32x4 (&S)[MT], float* dst) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __hip_atomic_store(&dst[(16 * m + 4 * lg + i) * DV + col0 + lr], S[m][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    };
    auto fetch_state = [&](f32x4 (&S)[MT], const float* src) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[m][i] = __hip_atomic_load(&src[(16 * m + 4 * lg + i) * DV + col0 + lr], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    };
    // one chunk step of Y (accumulator layout) with the operands in sb:
    // X = W Y;  Y <- Diag(Gn) Y + KdT (in - X), in = U' (with_u) or 0.
    // yf, uf: the fragments of Y before the step and of in - X.
    auto chain_step = [&](f32x4 (&Y)[MT], const char* sb, bool with_u, Frag<E> (&yf)[KS], Frag<E> (&uf)[KB])
                          __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) yf[ks] = acc_to_frag(E{}, Y[2 * ks], Y[2 * ks + 1]);
        f32x4 X[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) X[t] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < TT; ++t) X[t] = mma(frag_at(sb, L::off_W, t * KS + ks), yf[ks], X[t]);
        const float* gn = reinterpret_cast<const float*>(sb + L::off_G);
#pragma unroll
        for (int m = 0; m < MT; ++m) Y[m] = *reinterpret_cast<const f32x4*>(gn + 16 * m + 4 * lg) * Y[m];
        f32x4 up[TT];
        if (with_u) {
            const E* Up = reinterpret_cast<const E*>(sb + L::off_U) + (w * 64 + lane) * 16;
#pragma unroll
            for (int t = 0; t < TT; ++t) up[t] = Raw4<E>::widen(Raw4<E>::load(Up + 4 * t));
        } else {
#pragma unroll
            for (int t = 0; t < TT; ++t) up[t] = zero4();
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            uf[kb] = acc_to_frag(E{}, up[2 * kb] - X[2 * kb], up[2 * kb + 1] - X[2 * kb + 1]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int m = 0; m < MT; ++m) Y[m] = mma(frag_at(sb, L::off_K, m * KB + kb), uf[kb], Y[m]);
    };
    // the chunk steps of B (with U') and of M (without) at once: each W and
    // KdT fragment is read from LDS once and feeds both products (each
    // accumulates in the order chain_step uses).  Each product's operand
    // fragments are read together, ahead of its matrix-core instructions,
    // with a scheduling barrier between the two groups: left to itself the
    // compiler interleaves every read with the instruction that uses it and
    // waits for each read in turn.
    auto chain_step2 = [&](f32x4 (&Y1)[MT], f32x4 (&Y2)[MT], const char* sb) __attribute__((always_inline)) {
        Frag<E> wf[TT * KS];
#pragma unroll
        for (int i = 0; i < TT * KS; ++i) wf[i] = frag_at(sb, L::off_W, i);
        Frag<E> yf1[KS], yf2[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            yf1[ks] = acc_to_frag(E{}, Y1[2 * ks], Y1[2 * ks + 1]);
            yf2[ks] = acc_to_frag(E{}, Y2[2 * ks], Y2[2 * ks + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 X1[TT], X2[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) X1[t] = X2[t] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                X1[t] = mma(wf[t * KS + ks], yf1[ks], X1[t]);
                X2[t] = mma(wf[t * KS + ks], yf2[ks], X2[t]);
            }
        __builtin_amdgcn_sched_barrier(0);
        Frag<E> kf[MT * KB];
#pragma unroll
        for (int i = 0; i < MT * KB; ++i) kf[i] = frag_at(sb, L::off_K, i);
        const float* gn = reinterpret_cast<const float*>(sb + L::off_G);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(gn + 16 * m + 4 * lg);
            Y1[m] = gm * Y1[m];
            Y2[m] = gm * Y2[m];
        }
        const E* Up = reinterpret_cast<const E*>(sb + L::off_U) + (w * 64 + lane) * 16;
        Frag<E> uf1[KB], uf2[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            uf1[kb] = acc_to_frag(E{}, Raw4<E>::widen(Raw4<E>::load(Up + 8 * kb)) - X1[2 * kb],
                                  Raw4<E>::widen(Raw4<E>::load(Up + 8 * kb + 4)) - X1[2 * kb + 1]);
            uf2[kb] = acc_to_frag(E{}, zero4() - X2[2 * kb], zero4() - X2[2 * kb + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                Y1[m] = mma(kf[m * KB + kb], uf1[kb], Y1[m]);
                Y2[m] = mma(kf[m * KB + kb], uf2[kb], Y2[m]);
            }
    };
    // wait until S_start(i) is published (one lane polls; the others wait at
    // the barrier)
    auto wait_start = [&](int i) {
        if (tid == 0) {
            for (int spins = 0;
                 __hip_atomic_load(&seg_flags[pair * G + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
                 ++spins) {
                if (spins >= kSegSpinLimit) {
                    hdr->wait_timeout = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
    };

    // ------------------------------------------------------------ pass 1
    if (!last) {
        f32x4 B[MT], M[MT];
        load_state(B, first ? (S0 ? S0 + pair * DK * DV : nullptr) : nullptr);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) M[m][i] = (16 * m + 4 * lg + i == col0 + lr) ? 1.f : 0.f;
        // chunk c from slot cur, the next chunk's operands loading into nxt
        auto step1 = [&](int c, const char* cur, char* nxt) __attribute__((always_inline)) {
            if (c + 1 < s1) dma_chunk(c + 1, nxt, false);
            if (first) {
                Frag<E> yf[KS], uf[KB];
                chain_step(B, cur, true, yf, uf);
            } else {
                chain_step2(B, M, cur);
            }
            wait_vmcnt<0>();
            lds_barrier();
        };
        if (s0 < s1) {
            dma_chunk(s0, slotA, false);
            wait_vmcnt<0>();
            lds_barrier();
        }
        for (int c = s0; c < s1; c += 2) {
            step1(c, slotA, slotB);
            if (c + 1 < s1) step1(c + 1, slotB, slotA);
        }
        // ---- chain: S_start(j + 1) = M S_start(j) + B (segment 0: B itself)
        if (!first) {
            // M to LDS as two bf16 tiles (row-major, columns in fragment
            // order) for the A operand, in the second slot (free: the walk
            // ended at a barrier)
            E* sMh = reinterpret_cast<E*>(slotB);
            E* sMl = sMh + DK * L::LDM;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int at = (16 * m + 4 * lg + i) * L::LDM + frag_pos(col0 + lr);
                    const E hi = Elt<E>::from(M[m][i]);
                    lds_put(&sMh[at], hi);
                    lds_put(&sMl[at], Elt<E>::from(M[m][i] - Elt<E>::to(hi)));
                }
            wait_start(j);
            f32x4 Sj[MT];
            fetch_state(Sj, start_state(j));
            if (s0 < s1) {
                Frag<E> sh[KS], sl[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) split_frag(Sj[2 * ks], Sj[2 * ks + 1], sh[ks], sl[ks]);
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int at = (16 * m + lr) * L::LDM + 32 * ks + 8 * lg;
                        const Frag<E> mh = ld_frag(sMh + at), ml = ld_frag(sMl + at);
                        B[m] = mma(mh, sh[ks], B[m]);
                        B[m] = mma(mh, sl[ks], B[m]);
                        B[m] = mma(ml, sh[ks], B[m]);
                    }
            } else {
                // empty segment: the map is the identity
#pragma unroll
                for (int m = 0; m < MT; ++m) B[m] = Sj[m];
            }
        }
        publish_state(B, start_state(j + 1));
        wait_vmcnt<0>();  // this lane's part has reached the device level
        __syncthreads();  // every wave's part (and the M tiles are read)
        if (tid == 0) __hip_atomic_store(&seg_flags[pair * G + j + 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ------------------------------------------------------------ pass 3
    if (s0 < s1) dma_chunk(s0, slotA, true);  // in flight during the wait below
    f32x4 S[MT];
    if (first) {
        load_state(S, S0 ? S0 + pair * DK * DV : nullptr);
    } else {
        if (last) wait_start(j);
        fetch_state(S, start_state(j));
    }
    // store the O rows of chunk c from the O tile: 16 KB as 1 KB pieces of
    // four token rows, two pieces per wave
    auto store_o = [&](int c) __attribute__((always_inline)) {
        const int64_t t0 = seq0 + (int64_t)(c - cbeg) * C;
#pragma unroll
        for (int k = 0; k < C * DV * 2 / 1024 / kSegWaves; ++k) {
            const int piece = w + kSegWaves * k;
            const int row = 4 * piece + (lane >> 4), c8 = 8 * (lane & 15);
            const uint4 v = *reinterpret_cast<const uint4*>(sO + row * L::LDO + c8);
            const int64_t tok = t0 + row;
            if (tok < seqend) *reinterpret_cast<uint4*>(o + (tok * H + h) * DV + c8) = v;
        }
    };
    auto step3 = [&](int c, const char* cur, char* nxt) __attribute__((always_inline)) {
        if (c > s0) store_o(c - 1);
        if (c + 1 < s1) dma_chunk(c + 1, nxt, true);
        // one group of fragment reads per product, as in chain_step:
        // X = W S, then O = QG S, then S <- Diag(Gn) S + KdT U and O += P U
        Frag<E> sf[KS], uf[KB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sf[ks] = acc_to_frag(E{}, S[2 * ks], S[2 * ks + 1]);
        f32x4 X[TT], O[TT];
        {
            Frag<E> wf[TT * KS];
#pragma unroll
            for (int i = 0; i < TT * KS; ++i) wf[i] = frag_at(cur, L::off_W, i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < TT; ++t) X[t] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < TT; ++t) X[t] = mma(wf[t * KS + ks], sf[ks], X[t]);
            __builtin_amdgcn_sched_barrier(0);
        }
        {
            Frag<E> qf[TT * KS];
#pragma unroll
            for (int i = 0; i < TT * KS; ++i) qf[i] = frag_at(cur, L::off_Q, i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < TT; ++t) O[t] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < TT; ++t) O[t] = mma(qf[t * KS + ks], sf[ks], O[t]);
            __builtin_amdgcn_sched_barrier(0);
        }
        {
            Frag<E> kf[MT * KB], pf[6];
#pragma unroll
            for (int i = 0; i < MT * KB; ++i) kf[i] = frag_at(cur, L::off_K, i);
#pragma unroll
            for (int i = 0; i < 6; ++i) pf[i] = frag_at(cur, L::off_P, i);
            const float* gn = reinterpret_cast<const float*>(cur + L::off_G);
#pragma unroll
            for (int m = 0; m < MT; ++m) S[m] = *reinterpret_cast<const f32x4*>(gn + 16 * m + 4 * lg) * S[m];
            const E* Up = reinterpret_cast<const E*>(cur + L::off_U) + (w * 64 + lane) * 16;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                uf[kb] = acc_to_frag(E{}, Raw4<E>::widen(Raw4<E>::load(Up + 8 * kb)) - X[2 * kb],
                                     Raw4<E>::widen(Raw4<E>::load(Up + 8 * kb + 4)) - X[2 * kb + 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int m = 0; m < MT; ++m) S[m] = mma(kf[m * KB + kb], uf[kb], S[m]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t = 0; t < TT; ++t)
                    if (!p_block_zero(t, kb)) O[t] = mma(pf[p_block_index(t, kb)], uf[kb], O[t]);
        }
        // every wave has read the previous chunk's rows out of the O tile
        // (the reads were waited for here; no fence, which would also wait
        // for the loads in flight into the other slot)
        lds_release();
        __builtin_amdgcn_s_barrier();
        lds_acquire();
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds_put(&sO[(16 * t + 4 * lg + i) * L::LDO + col0 + lr], Elt<E>::from(O[t][i]));
        wait_vmcnt<0>();
        lds_barrier();
    };
    if (s0 < s1) {
        wait_vmcnt<0>();
        lds_barrier();
    }
    for (int c = s0; c < s1; c += 2) {
        step3(c, slotA, slotB);
        if (c + 1 < s1) step3(c + 1, slotB, slotA);
    }
    if (s0 < s1) store_o(s1 - 1);
    if (last && S_T) store_state(S, S_T + pair * DK * DV);
}

// ----------------------------------------------------------------------------
// Host side.
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t max_chunks_for(int64_t T, int32_t N, int32_t chunk) { return (T + chunk - 1) / chunk + N; }

// Segments per (sequence, head) of the segmented walk, or 0 where the
// per-slice walk runs (fp32 operands, other head sizes).  Enough segments
// for about one workgroup per compute unit, but on average at least
// kSegMinChunks chunks per segment (shorter ones spend more on the extra
// pass and the chain than they gain).
int32_t seg_groups_for(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16, int32_t chunk) {
    if (!bf16 || dk != 128 || dv != 128 || N <= 0 || H <= 0) return 0;
    const int64_t np = (int64_t)N * H;
    int64_t g = np >= kSegTarget ? 1 : kSegTarget / np;
    const int64_t per_seq = (T + (int64_t)N * chunk - 1) / ((int64_t)N * chunk);  // mean chunks per sequence
    g = std::min<int64_t>(g, std::max<int64_t>(1, per_seq / kSegMinChunks));
    return (int32_t)std::min<int64_t>(g, kSegMaxGroups);
}

// The intra-chunk grid (one workgroup per chunk and head, in one dimension)
// must stay within the 2^32 work-items a grid dimension can hold.
bool chunk_grid_fits(int64_t max_chunks, int32_t H, int32_t chunk) {
    const int64_t threads = chunk == 128 ? 1024 : kIntraThreads;
    return max_chunks * H * threads <= (int64_t)UINT32_MAX;
}

namespace {
struct WsSizes {
    size_t header, cu, chunk_off, chunk_tab, W, QG, KdT, Up, P, Gn, seg_state, seg_flags;
    int32_t seg_groups;
};
WsSizes ws_sizes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16, int32_t chunk) {
    const size_t esz = bf16 ? 2 : 4;
    const size_t mc = (size_t)max_chunks_for(T, N, chunk);
    const size_t C = (size_t)chunk;
    WsSizes s;
    s.header = 256;
    s.cu = align256((size_t)(N + 1) * 4);
    s.chunk_off = align256((size_t)(N + 1) * 4);
    s.chunk_tab = align256(mc * sizeof(int2));
    s.W = align256(mc * H * C * dk * esz);
    s.QG = s.W;
    s.KdT = s.W;
    s.Up = align256(mc * H * C * dv * esz);
    s.P = align256(mc * H * C * C * esz);
    s.Gn = align256(mc * H * dk * 4);
    s.seg_groups = seg_groups_for(T, N, H, dk, dv, bf16, chunk);
    const size_t np = (size_t)N * H, G = (size_t)s.seg_groups;
    s.seg_state = G > 1 ? align256(np * (G - 1) * dk * dv * 4) : 0;
    s.seg_flags = G > 1 ? align256(np * G * 4) : 0;
    return s;
}
}  // namespace

size_t chunk_workspace_bytes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16, int32_t chunk) {
    const WsSizes s = ws_sizes(T, N, H, dk, dv, bf16, chunk);
    return s.header + s.cu + s.chunk_off + s.chunk_tab + s.W + s.QG + s.KdT + s.Up + s.P + s.Gn + s.seg_state +
           s.seg_flags;
}

ChunkWorkspace carve_chunk_workspace(void* base, int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                                     bool bf16, int32_t chunk) {
    const WsSizes s = ws_sizes(T, N, H, dk, dv, bf16, chunk);
    char* p = static_cast<char*>(base);
    ChunkWorkspace w;
    w.header = reinterpret_cast<WsHeader*>(p); p += s.header;
    w.cu = reinterpret_cast<int32_t*>(p); p += s.cu;
    w.chunk_off = reinterpret_cast<int32_t*>(p); p += s.chunk_off;
    w.chunk_tab = reinterpret_cast<int2*>(p); p += s.chunk_tab;
    w.W = p; p += s.W;
    w.QG = p; p += s.QG;
    w.KdT = p; p += s.KdT;
    w.Up = p; p += s.Up;
    w.P = p; p += s.P;
    w.Gn = reinterpret_cast<float*>(p); p += s.Gn;
    w.seg_groups = s.seg_groups;
    w.seg_state = s.seg_state ? reinterpret_cast<float*>(p) : nullptr; p += s.seg_state;
    w.seg_flags = s.seg_flags ? reinterpret_cast<int32_t*>(p) : nullptr;
    return w;
}


template <typename E, int DK, int DV, bool HG, bool RAW>
static hipError_t launch_intra(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream) {
    using L = IntraLayout<E, DK, DV>;
    auto kern = intra_chunk_kernel<E, DK, DV, HG, RAW>;
    static std::atomic<uint64_t> attr_done{0};
    if (hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), (int)L::bytes, attr_done);
        e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.max_chunks * a.H)), dim3(kIntraThreads), L::bytes, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.g, (const E*)a.beta, ws.header,
                       ws.chunk_tab, a.H, (E*)ws.W, (E*)ws.QG, (E*)ws.KdT, (E*)ws.Up, (E*)ws.P, ws.Gn);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
static hipError_t launch_walk(const ChunkArgs& a, const ChunkWorkspace& ws, int64_t blocks, hipStream_t stream) {
    using L = WalkLayout<E, DK, DV>;
    auto kern = chunk_walk_kernel<E, DK, DV>;
    static std::atomic<uint64_t> attr_done{0};
    if (hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), (int)L::bytes, attr_done);
        e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kWalkThreads), L::bytes, stream, ws.header, ws.cu,
                       ws.chunk_off, a.N, a.H, (const E*)ws.W, (const E*)ws.QG, (const E*)ws.KdT, (const E*)ws.Up,
                       (const E*)ws.P, (const float*)ws.Gn, a.S0, a.S_T, (E*)a.o);
    return hipGetLastError();
}

static inline hipError_t mark(hipEvent_t* ev, int i, hipStream_t stream) {
    return ev ? hipEventRecord(ev[i], stream) : hipSuccess;
}

static hipError_t launch_seg_walk(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.N * a.H * ws.seg_groups;
    hipLaunchKernelGGL(seg_walk_kernel, dim3((unsigned)blocks), dim3(kSegThreads), 0, stream, ws.header,
                       ws.seg_flags, ws.seg_state, ws.cu, ws.chunk_off, a.N, a.H, ws.seg_groups,
                       (const bf16_t*)ws.W, (const bf16_t*)ws.QG, (const bf16_t*)ws.KdT, (const bf16_t*)ws.Up,
                       (const bf16_t*)ws.P, (const float*)ws.Gn, a.S0, a.S_T, (bf16_t*)a.o);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
static hipError_t launch_chunk_t(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream,
                                 hipEvent_t* ev) {
    hipError_t e = mark(ev, 1, stream);
    if (e != hipSuccess) return e;
    if (a.T > 0) {
        if (a.raw)
            e = a.head_gate ? launch_intra<E, DK, DV, true, true>(a, ws, stream)
                            : launch_intra<E, DK, DV, false, true>(a, ws, stream);
        else
            e = a.head_gate ? launch_intra<E, DK, DV, true, false>(a, ws, stream)
                            : launch_intra<E, DK, DV, false, false>(a, ws, stream);
        if (e != hipSuccess) return e;
    }
    if ((e = mark(ev, 2, stream)) != hipSuccess) return e;
    if constexpr (std::is_same<E, bf16_t>::value && DK == SegLayout::DK && DV == SegLayout::DV) {
        if (ws.seg_groups > 0) e = launch_seg_walk(a, ws, stream);
        else e = launch_walk<E, DK, DV>(a, ws, (int64_t)a.N * a.H * (DV / 16), stream);
    } else {
        e = launch_walk<E, DK, DV>(a, ws, (int64_t)a.N * a.H * (DV / 16), stream);
    }
    if (e != hipSuccess) return e;
    return mark(ev, 3, stream);
}

template <typename E>
static hipError_t launch_chunk_e(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t s, hipEvent_t* ev) {
    if (a.dk == 64 && a.dv == 64) return launch_chunk_t<E, 64, 64>(a, ws, s, ev);
    if (a.dk == 64 && a.dv == 128) return launch_chunk_t<E, 64, 128>(a, ws, s, ev);
    if (a.dk == 128 && a.dv == 64) return launch_chunk_t<E, 128, 64>(a, ws, s, ev);
    return launch_chunk_t<E, 128, 128>(a, ws, s, ev);
}

hipError_t launch_chunk_map(const int32_t* cu_seqlens, int32_t N, int64_t T, WsHeader* header, int32_t* cu,
                            int32_t* chunk_off, int2* chunk_tab, int32_t* seg_flags, int64_t n_flags,
                            hipStream_t stream, int32_t chunk) {
    if (chunk == 128)
        hipLaunchKernelGGL(chunk_map_kernel<128>, dim3(1), dim3(256), 0, stream, cu_seqlens, N, T, header, cu,
                           chunk_off, chunk_tab, seg_flags, n_flags);
    else
        hipLaunchKernelGGL(chunk_map_kernel<kChunk>, dim3(1), dim3(256), 0, stream, cu_seqlens, N, T, header, cu,
                           chunk_off, chunk_tab, seg_flags, n_flags);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream, hipEvent_t* ev) {
    hipError_t e = mark(ev, 0, stream);
    if (e != hipSuccess) return e;
    const int64_t n_flags = ws.seg_groups > 1 ? (int64_t)a.N * a.H * ws.seg_groups : 0;
    e = launch_chunk_map(a.cu_seqlens, a.N, a.T, ws.header, ws.cu, ws.chunk_off, ws.chunk_tab, ws.seg_flags, n_flags,
                         stream, a.chunk);
    if (e != hipSuccess) return e;
    if (a.chunk == 128) return launch_chunk128_kernels(a, ws, stream, ev);
    return a.bf16 ? launch_chunk_e<bf16_t>(a, ws, stream, ev) : launch_chunk_e<float>(a, ws, stream, ev);
}

}  // namespace kda
