// Chunkwise KDA forward with chunks of 128 tokens on gfx950.
//
// "From GPT-2 to Kimi K3" (molayo1419.me), section on the parallelisation
// trick, names chunks of 64 or of 128 tokens as the sizes that work best.
// This file holds the 128-token variant of the two chunk kernels; the
// 64-token kernels are in kda_chunk.hip.  The chunk algebra is the same, with
// C = 128 (chunk-local tokens t = 0..n-1, start state S):
//   b_t   = g_0 + ... + g_t                       (per key channel)
//   A_ti  = beta_t sum_c k_tc k_ic e^{b_tc - b_ic}   (i < t),  T = (I + A)^{-1}
//   W     = T diag(beta) (K e^b),   U' = T diag(beta) V,   U = U' - W S
//   O     = (Q e^b) S + P U,        P_ti = sum_c q_tc k_ic e^{b_tc - b_ic}  (i <= t)
//   S    <- Diag(e^{b_last}) S + (K e^{b_last - b})^T U
// What the size changes on this chip:
//   intra128_kernel  one workgroup of sixteen waves per (chunk, head).  The
//                    128 x 128 triangle has 36 tile pairs of 16 x 16 (28 below
//                    the diagonal, each with its own decay factors, as in the
//                    64-token kernel).  (I + A)^{-1} is built on three levels of
//                    the block-triangular inverse (32, 64 and 128 rows) above
//                    the 16 x 16 diagonal blocks.  The operand tiles of the A
//                    and P products and A itself do not fit in LDS together,
//                    so A is written over the operand tiles once the products
//                    are in registers; one workgroup per compute unit.
//   walk128_kernel   one workgroup per (segment, sequence, head), one wave per
//                    16 columns of d_v, each keeping its slice of S in
//                    registers.  A chunk's shared operands (W, QG, KdT, Gn and
//                    the twenty kept blocks of P) take 116.5 KB in bf16, so
//                    only one set fits next to the O tile: it is refilled in
//                    two halves, W and QG once the products that read them
//                    are done, KdT, Gn and P once the rest of the chunk is,
//                    so that each half loads while the other half computes.
//                    U' is read by each wave straight into registers.  fp32
//                    operands are read from memory by every wave instead (no
//                    staging).  The segmented form of the chain (bf16,
//                    d_k = d_v) is the one of the 64-token walk.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kda_chunk_util.h"

namespace kda {

constexpr int kChunk128 = 128;
constexpr int kIntra128Threads = 1024;  // sixteen waves per (chunk, head)

// ----------------------------------------------------------------------------
// Intra-chunk transform, 128-token chunks.
template <typename E, int DK, int DV>
struct Intra128Layout {
    static constexpr int C = kChunk128, NT = kIntra128Threads, TILES = C / 16;
    static constexpr int PAD = 16 / (int)sizeof(E);
    static constexpr int LDK = DK + PAD;  // [token][channel] row stride
    static constexpr int LDT = C + PAD;   // [channel][token] row stride
    static constexpr int LDA = C + 4;     // fp32 A / T row stride
    static constexpr int LDP = C + PAD;   // P staging row stride
    static constexpr int LDZ = 64 + 4;    // fp32 Z of the two outer levels, [64][LDZ]
    // threads hold two adjacent channels (values) of RPT (RPTV) consecutive rows
    static constexpr int NPART = NT / (DK / 2), RPT = C / NPART;
    static constexpr int NPARTV = NT / (DV / 2), RPTV = C / NPARTV;
    static_assert(RPT % 4 == 0 && RPTV % 4 == 0 && 16 % RPT == 0, "row runs of four within one tile");
    static constexpr int NBND = 3 * TILES;                // b at rows 16i, 16i + 8, 16i + 15 of every tile
    static constexpr int NOFF = TILES * (TILES - 1) / 2;  // tile pairs below the diagonal
    // factor rows: e^{b_m(ti) - b_s(ti)} (ti = 1..7), e^{b_e(tj) - b_m(tj)}
    // (tj = 0..6), e^{b_s(ti) - b_e(tj)} (the 28 pairs tj < ti)
    static constexpr int ROWF = 0, COLF = TILES - 1, MIDF = 2 * (TILES - 1), NCS = MIDF + NOFF;
    // While A and P are formed: [Kr | Qr | Kt] | boundary sums | factor rows
    // (the prefix-sum partials before them).
    static constexpr size_t off_bnd = (size_t)3 * C * LDK * sizeof(E);
    static constexpr size_t off_tf = off_bnd + (size_t)NBND * DK * 4;
    static constexpr size_t end1 = off_tf + (size_t)(NCS > NPART ? NCS : NPART) * DK * 4;
    // Afterwards: A, then T in place, fp32 [C][LDA] | region X: the P staging
    // tile, then [Kbt | Vt], then the W staging tile | Z.
    static constexpr size_t off_X = (size_t)C * LDA * 4;
    static constexpr size_t pst_b = (size_t)C * LDP * sizeof(E);
    static constexpr size_t rhs_b = (size_t)(DK + DV) * LDT * sizeof(E);
    static constexpr size_t wst_b = (size_t)C * LDK * sizeof(E);
    static constexpr size_t x_b = pst_b > rhs_b ? (pst_b > wst_b ? pst_b : wst_b) : (rhs_b > wst_b ? rhs_b : wst_b);
    static constexpr size_t off_Z = off_X + (x_b + 15) / 16 * 16;
    static constexpr size_t end2 = off_Z + (size_t)64 * LDZ * 4;
    static constexpr size_t off_beta = ((end1 > end2 ? end1 : end2) + 15) / 16 * 16;
    static constexpr size_t bytes = off_beta + C * 4;
    static_assert(bytes <= (size_t)kLdsBytes, "LDS budget");
};

template <typename E, int DK, int DV, bool HG>
__global__ __launch_bounds__(kIntra128Threads) void intra128_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ g,
    const E* __restrict__ beta, const WsHeader* __restrict__ hdr, const int2* __restrict__ chunk_tab,
    int32_t H, E* __restrict__ Wo, E* __restrict__ QGo, E* __restrict__ KdTo, E* __restrict__ Upo,
    E* __restrict__ Po, float* __restrict__ Gno) {
    using L = Intra128Layout<E, DK, DV>;
    constexpr int C = L::C, NT = L::NT, TILES = L::TILES, LDK = L::LDK, LDT = L::LDT, LDA = L::LDA;
    constexpr int LDZ = L::LDZ, NPART = L::NPART, RPT = L::RPT, RPTV = L::RPTV;

    extern __shared__ __align__(16) unsigned char smem[];
    E* sKr = reinterpret_cast<E*>(smem);  // k_t e^{b_t - b_m(t)}, m(t) = middle row of t's tile
    E* sQr = sKr + C * LDK;               // q_t e^{b_t - b_m(t)}
    E* sKt = sQr + C * LDK;               // k_i e^{b_m(i) - b_i}
    float* sBnd = reinterpret_cast<float*>(smem + L::off_bnd);
    float* sTileF = reinterpret_cast<float*>(smem + L::off_tf);
    float* sPart = sTileF;                           // dead before the factor rows are written
    float* sA = reinterpret_cast<float*>(smem);     // once the A and P products are in registers
    E* sX = reinterpret_cast<E*>(smem + L::off_X);  // P staging, then [Kbt | Vt], then W staging
    E* sKbt = sX;
    E* sVt = sX + DK * LDT;
    float* sZ = reinterpret_cast<float*>(smem + L::off_Z);
    float* sBeta = reinterpret_cast<float*>(smem + L::off_beta);

    // one workgroup per (chunk, head), heads fastest over the grid
    const int cid = (int)(blockIdx.x / (unsigned)H);
    const int h = (int)(blockIdx.x - (unsigned)cid * (unsigned)H);
    const int total = hdr->total_chunks;  // zero when the sequence offsets were rejected
    const int2 tab = chunk_tab[cid];
    if ((cid >= total) | (tab.y <= 0)) return;
    const int64_t t0 = tab.x;
    const int len = tab.y;
    const int64_t ch = (int64_t)cid * H + h;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // ---- 0. every global load of the chunk, issued up front (rows past the
    // chunk's end load the last valid row and are zeroed where first used)
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
    const int brow = tid & (C - 1);  // beta of token brow, loaded by eight threads each
    const float beta_raw = Elt<E>::load(beta + (t0 + clamp_row(brow)) * H + h);
    auto row_ok = [&](int r) { return part * RPT + r < len; };
    auto gate_of = [&](int r, int i) -> float { return HG ? gh[r] : (i ? graw[r].hi() : graw[r].lo()); };

    // ---- 1. chunk-local inclusive prefix sum of the log-gate, in base-2 units
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
    const float last0 = sBnd[(L::NBND - 1) * DK + c0], last1 = sBnd[(L::NBND - 1) * DK + c0 + 1];

    // ---- 2. decayed operands (the scheme of the 64-token kernel: each factor
    // spans at most eight tokens of decay, or is <= 1; exponents capped at 80)
    constexpr float kCap2 = 80.f * kLog2e;
    float kx[RPT][2];  // k e^b; times beta it is the W right-hand side
    E kd0[RPT], kd1[RPT];
    const float* bm = sBnd + (3 * ((part * RPT) >> 4) + 1) * DK;  // tile middle
    float eg[RPT][2];
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
    float e0 = gate_exp2<E>(fminf(bb[0][0] - bm[c0], kCap2)), e1 = gate_exp2<E>(fminf(bb[0][1] - bm[c0 + 1], kCap2));
    float x0 = gate_exp2<E>(bb[0][0]), x1 = gate_exp2<E>(bb[0][1]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = part * RPT + r;
        const bool ok = row_ok(r);
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
            const int pos = frag_pos(part * RPT + 4 * r4);
            store_run4<E>(p0 + fm_off<C>(c0, pos), kd0 + 4 * r4);
            store_run4<E>(p0 + fm_off<C>(c0 + 1, pos), kd1 + 4 * r4);
        }
        if (part == 0) {
            Gno[ch * DK + c0] = gate_exp2<E>(last0);
            Gno[ch * DK + c0 + 1] = gate_exp2<E>(last1);
        }
    }
    // tile-pair factors (the pair (ti, tj), tj < ti, has index ti (ti - 1) / 2 + tj)
    for (int e = tid; e < L::NCS * DK; e += NT) {
        const int vrow = e / DK, c = e % DK;
        float x;
        if (vrow < L::COLF) {
            const int ti = vrow + 1;
            x = sBnd[(3 * ti + 1) * DK + c] - sBnd[(3 * ti) * DK + c];
        } else if (vrow < L::MIDF) {
            const int tj = vrow - L::COLF;
            x = sBnd[(3 * tj + 2) * DK + c] - sBnd[(3 * tj + 1) * DK + c];
        } else {
            const int p = vrow - L::MIDF;
            int ti = 1;
            while ((ti + 1) * ti / 2 <= p) ++ti;
            const int tj = p - ti * (ti - 1) / 2;
            x = sBnd[(3 * ti) * DK + c] - sBnd[(3 * tj + 2) * DK + c];
        }
        sTileF[vrow * DK + c] = gate_exp2<E>(x);
    }
    sBeta[brow] = brow < len ? beta_raw : 0.f;  // eight threads write the same value
    lds_barrier();

    // ---- 3. the A and P tiles of the 36 tile pairs, in registers: wave w
    // takes pairs w, w + 16 and w + 32 of the list (28 below the diagonal
    // first, then the 8 diagonal ones), so no wave has more than two
    // rescaled pairs
    constexpr int NPAIRS = L::NOFF + TILES;
    constexpr int NWAVES = NT / 64;
    constexpr int PPW = (NPAIRS + NWAVES - 1) / NWAVES;
    f32x4 accA[PPW], accP[PPW];
    int pti[PPW], ptj[PPW];
#pragma unroll
    for (int s = 0; s < PPW; ++s) {
        const int p = wave + NWAVES * s;
        int ti, tj;
        if (p < L::NOFF) {
            ti = 1;
            while ((ti + 1) * ti / 2 <= p) ++ti;
            tj = p - ti * (ti - 1) / 2;
        } else {
            ti = tj = min(p - L::NOFF, TILES - 1);
        }
        pti[s] = ti;
        ptj[s] = tj;
        accA[s] = zero4();
        accP[s] = zero4();
        if (p < NPAIRS) {
            const bool diag = tj == ti;
            const float* rowf = sTileF + (L::ROWF + max(ti - 1, 0)) * DK;
            const float* colf = sTileF + (L::COLF + min(tj, TILES - 2)) * DK;
            const float* midf = sTileF + (L::MIDF + (diag ? 0 : ti * (ti - 1) / 2 + tj)) * DK;
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const int cb = 32 * ks + 8 * lg;
                Frag<E> fb = ld_frag(sKt + (16 * tj + lr) * LDK + cb);
                Frag<E> fa = ld_frag(sKr + (16 * ti + lr) * LDK + cb);
                Frag<E> fq = ld_frag(sQr + (16 * ti + lr) * LDK + cb);
                if (!diag) {
                    float fr[8], fc[8], fm[8];
#pragma unroll
                    for (int h4 = 0; h4 < 2; ++h4) {
                        *reinterpret_cast<f32x4*>(fr + 4 * h4) = *reinterpret_cast<const f32x4*>(rowf + cb + 4 * h4);
                        *reinterpret_cast<f32x4*>(fc + 4 * h4) = *reinterpret_cast<const f32x4*>(colf + cb + 4 * h4);
                        *reinterpret_cast<f32x4*>(fm + 4 * h4) = *reinterpret_cast<const f32x4*>(midf + cb + 4 * h4);
                    }
                    fb = scale_frag(fb, fc, fm);
                    fa = scale_frag(fa, fr);
                    fq = scale_frag(fq, fr);
                }
                accA[s] = mma(fa, fb, accA[s]);
                accP[s] = mma(fq, fb, accP[s]);
            }
        }
    }
    lds_barrier();  // every wave is done with the operand tiles and factors

    // A (strictly lower, rows scaled by beta) and the P staging tile (lower
    // including the diagonal, columns in fragment order) over the operand
    // tiles; the tiles (2u, 2u + 1) above the diagonal are read by the
    // 32-wide products below and are zeroed
    E* sPst = sX;
#pragma unroll
    for (int s = 0; s < PPW; ++s) {
        if (wave + NWAVES * s < NPAIRS) {
            const int ti = pti[s], tj = ptj[s];
            const f32x4 bt4 = *reinterpret_cast<const f32x4*>(sBeta + 16 * ti + 4 * lg);  // the lane's four rows
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + 4 * lg + i, col = 16 * tj + lr;
                lds_put(&sA[row * LDA + col], (row > col) ? accA[s][i] * bt4[i] : 0.f);
                lds_put(&sPst[row * L::LDP + frag_pos(col)], Elt<E>::from((row >= col) ? accP[s][i] : 0.f));
            }
        }
    }
    if (wave < TILES / 2) {
        const int ti = 2 * wave, tj = ti + 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * ti + 4 * lg + i, col = 16 * tj + lr;
            lds_put(&sA[row * LDA + col], 0.f);
            lds_put(&sPst[row * L::LDP + frag_pos(col)], Elt<E>::from(0.f));
        }
    }
    lds_barrier();

    // ---- 4. T = (I + A)^{-1}
    // (a) the eight 16 x 16 diagonal blocks, one column per thread of waves
    //     0 and 1; meanwhile P goes out
    float x[16];
    if (tid < 16 * TILES) {
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
    copy_tile_out_frag<E, C, C, true, NT>(Po + ch * C * C, sPst, L::LDP, tid);
    lds_barrier();  // P staging read out; diagonal blocks of A read
    if (tid < 16 * TILES) {
        const int blk = tid >> 4, jc = tid & 15;
        float* Tb = sA + (16 * blk) * LDA + 16 * blk;
#pragma unroll
        for (int t = 0; t < 16; ++t) Tb[t * LDA + jc] = x[t];
    }
    // right-hand sides beta K e^b and beta V, [channel][token], over the P staging tile
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
    lds_barrier();
    // (b) off-diagonal blocks on the matrix cores in fp32 (16x16x4), level by
    //     level: T of [[M_a, 0], [A_ba, M_b]] is [[T_a, 0], [-T_b A_ba T_a, T_b]]
    //     with Z = A_ba T_a formed first, for blocks of 32, 64 and 128 rows.
    //     With k = 4g + s for lane group g and step s, the accumulators of a
    //     product are exactly the B operand of the next one.
    {
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
        // Z block (zr, zc) of the Z buffer, in accumulator layout
        auto put_z = [&](int zr, int zc, f32x4 Z) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) lds_put(&sZ[(16 * zr + 4 * lg + ii) * LDZ + 16 * zc + lr], Z[ii]);
        };
        auto get_z = [&](int zr, int zc) {
            f32x4 Z;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Z[jj] = sZ[(16 * zr + 4 * lg + jj) * LDZ + 16 * zc + lr];
            return Z;
        };
        // level 1 (32 rows): block (i0 + 1, i0), i0 = 0, 2, 4, 6, waves 0-3
        if (wave < TILES / 2) {
            const int i0 = 2 * wave;
            const f32x4 X = mul_AT(i0 + 1, i0, i0, zero4());
            put_block(i0 + 1, i0, mul_TX(i0 + 1, i0 + 1, X, zero4()));
        }
        lds_barrier();
        // level 2 (64 rows): in half hh (tiles 4hh..4hh+3), blocks (zi, zj) with
        // zi in {4hh + 2, 4hh + 3}, zj in {4hh, 4hh + 1}, waves 0-7
        const int hh = wave >> 2;
        const int zi = 4 * hh + 2 + ((wave >> 1) & 1), zj = 4 * hh + (wave & 1);
        if (wave < 8) {
            f32x4 Z = zero4();
            for (int m = zj; m <= 4 * hh + 1; ++m) Z = mul_AT(zi, m, zj, Z);
            put_z(2 * hh + (zi - 4 * hh - 2), zj - 4 * hh, Z);
        }
        lds_barrier();
        if (wave < 8) {
            f32x4 Y = zero4();
            for (int m = 4 * hh + 2; m <= zi; ++m) Y = mul_TX(zi, m, get_z(2 * hh + (m - 4 * hh - 2), zj - 4 * hh), Y);
            put_block(zi, zj, Y);
        }
        lds_barrier();
        // level 3 (128 rows): blocks (bi, bj), bi = 4..7, bj = 0..3, one per wave
        const int bi = 4 + (wave >> 2), bj = wave & 3;
        {
            f32x4 Z = zero4();
            for (int m = bj; m < 4; ++m) Z = mul_AT(bi, m, bj, Z);
            put_z(bi - 4, bj, Z);
        }
        lds_barrier();
        {
            f32x4 Y = zero4();
            for (int m = 4; m <= bi; ++m) Y = mul_TX(bi, m, get_z(m - 4, bj), Y);
            put_block(bi, bj, Y);
        }
        lds_barrier();
    }

    // ---- 5. W = T (beta K e^b),  U' = T (beta V)
    {
        // wave w: token tile ti = w % 8, half (w / 8) of the W and U' columns;
        // T's row tile ti is zero beyond column 16 ti + 15, so only its first
        // ti / 2 + 1 blocks of 32 columns enter
        const int ti = wave & (TILES - 1), half = wave >> 3;
        const int kmax = ti >> 1;
        constexpr int TNW = DK / 32, TNU = DV / 32;  // 16-column tiles per half
        constexpr int KBT = C / 32;
        Frag<E> ft[KBT];
#pragma unroll
        for (int kb = 0; kb < KBT; ++kb)
            if (kb <= kmax) ft[kb] = ld_frag_from_f32<E>(sA + (16 * ti + lr) * LDA + 32 * kb + 8 * lg);
        f32x4 accW[TNW], accU[TNU];
#pragma unroll
        for (int u = 0; u < TNW; ++u) {
            const int tn = half * TNW + u;
            accW[u] = zero4();
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
                if (kb <= kmax) accW[u] = mma(ft[kb], ld_frag(sKbt + (16 * tn + lr) * LDT + 32 * kb + 8 * lg), accW[u]);
        }
#pragma unroll
        for (int u = 0; u < TNU; ++u) {
            const int tn = half * TNU + u;
            accU[u] = zero4();
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
                if (kb <= kmax) accU[u] = mma(ft[kb], ld_frag(sVt + (16 * tn + lr) * LDT + 32 * kb + 8 * lg), accU[u]);
        }
        // U' for the walk: per 16-column slice tn and lane, the 32 values the
        // lane holds in the walk's accumulator layout (token tiles 0..7, rows
        // 4 lg + i), contiguous: [tn][lane][ti][i]
        {
            E* up = Upo + ch * C * DV;
#pragma unroll
            for (int u = 0; u < TNU; ++u) {
                const int tn = half * TNU + u;
                E vals[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) vals[i] = Elt<E>::from(accU[u][i]);
                store_run4<E>(up + (tn * 64 + lane) * (C / 4) + 4 * ti, vals);
            }
        }
        lds_barrier();  // every wave is done with Kbt / Vt / T
        E* sWst = sX;   // [C][DK], channel columns in fragment order
#pragma unroll
        for (int u = 0; u < TNW; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds_put(&sWst[(16 * ti + 4 * lg + i) * LDK + frag_pos(16 * (half * TNW + u) + lr)],
                        Elt<E>::from(accW[u][i]));
        lds_barrier();
        copy_tile_out_frag<E, C, DK, false, NT>(Wo + ch * C * DK, sWst, LDK, tid);
    }
}

// ----------------------------------------------------------------------------
// State walk + output, 128-token chunks.  One workgroup per (segment j,
// sequence, head), DV / 16 waves, wave w owning columns 16w..16w+15 of S
// (fp32, accumulator layout) and of the outputs.  Per chunk:
//   phase a   U = U' - W S, O = QG S                 (reads W, QG)
//   phase b   O += P U, S <- Diag(Gn) S + KdT U      (reads P, KdT, Gn)
// bf16 operands: W and QG of the next chunk are loaded into LDS (16-byte
// LDS-DMA, spread over the waves) during phase b, KdT, Gn and P during the
// next chunk's phase a; a barrier after each phase, each preceded by the
// wait for the loads issued before the phase.  The O tile is staged in LDS
// and stored by all waves during the next chunk's phase a.  fp32 operands
// are read by every wave from memory.
// Segmented form (bf16, d_k = d_v): as in the 64-token walk, pass 1 maps each
// segment's start state to its end state, S_end = M S_start + B, the chain
// hands S_start(j + 1) = M S_start(j) + B from segment to segment through
// device-scope accesses (tickets in segment-major order, bounded waits), and
// pass 3 walks the segment again with outputs.
constexpr int kWalk128SpinLimit = 1 << 24;  // polls of about 128 clocks: several seconds

template <typename E, int DK, int DV>
struct Walk128Layout {
    static constexpr int C = kChunk128, KS = DK / 32, KB = C / 32, TT = C / 16, MT = DK / 16, NW = DV / 16;
    static constexpr bool STAGED = sizeof(E) == 2;  // bf16: operands through LDS
    static constexpr bool SEG = STAGED && DK == DV;  // the segmented form (square map M)
    static constexpr int NPB = p_block_index(TT - 1, (TT - 1) / 2) + 1;  // kept blocks of P
    // 1 KB LDS-DMA pieces (bf16): W, QG; KdT, one for Gn, the kept P blocks
    static constexpr int PW = C * DK * 2 / 1024, PK = DK * C * 2 / 1024;
    static constexpr int LDO = DV + 16 / (int)sizeof(E);  // O tile row, padded
    static_assert(NPB == 20, "twenty kept blocks of P");
    static_assert(!SEG || DK <= C, "the map M fits in the W and QG tiles");
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 16)) void walk128_kernel(
    WsHeader* __restrict__ hdr, int* __restrict__ seg_flags, float* __restrict__ seg_state,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int32_t N, int32_t H, int32_t G,
    const E* __restrict__ Wi, const E* __restrict__ QGi, const E* __restrict__ KdTi, const E* __restrict__ UpTi,
    const E* __restrict__ Pi, const float* __restrict__ Gni, const float* __restrict__ S0,
    float* __restrict__ S_T, E* __restrict__ o) {
    using L = Walk128Layout<E, DK, DV>;
    constexpr int C = L::C, KS = L::KS, KB = L::KB, TT = L::TT, MT = L::MT, NW = L::NW, NT = 64 * NW;
    constexpr bool STAGED = L::STAGED, SEG = L::SEG;
    constexpr int LDO = L::LDO;
    // distinct LDS objects, so that the compiler can tell the operand reads
    // of one half from the loads in flight into the other
    __shared__ __align__(16) E sW[STAGED ? C * DK : 8];
    __shared__ __align__(16) E sQ[STAGED ? C * DK : 8];
    __shared__ __align__(16) E sK[STAGED ? DK * C : 8];
    __shared__ __align__(16) float sG[STAGED ? DK : 4];
    __shared__ __align__(16) E sP[STAGED ? L::NPB * 512 : 8];
    __shared__ __align__(16) E sO[C * LDO];
    __shared__ int sticket;

    if (hdr->bad_seqlens) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    if (tid == 0) sticket = atomicAdd(&hdr->seg_ticket, 1);
    __syncthreads();
    const int64_t NP = (int64_t)N * H;
    const int64_t ticket = __builtin_amdgcn_readfirstlane(sticket);
    const int j = (int)(ticket / NP);
    const int64_t pair = ticket % NP;
    const int n = (int)(pair / H), h = (int)(pair % H);
    const int cbeg = chunk_off[n], cend = chunk_off[n + 1];
    const int64_t seq0 = cu[n], seqend = cu[n + 1];
    const int seglen = (cend - cbeg + G - 1) / G;
    const int s0 = min(cend, cbeg + j * seglen), s1 = min(cend, s0 + seglen);
    const int col0 = 16 * w;
    const bool first = j == 0, last = j == G - 1;
    auto start_state = [&](int i) { return seg_state + (pair * (G - 1) + i - 1) * DK * DV; };
    auto chunk_ch = [&](int c) { return (int64_t)__builtin_amdgcn_readfirstlane(c) * H + h; };

    // ---- operands of chunk c (LDS when staged, else memory)
    auto frag = [&](const E* base, int blk) __attribute__((always_inline)) {
        return ld_frag(base + (blk * 64 + lane) * 8);
    };
    auto baseW = [&](int64_t ch) __attribute__((always_inline)) -> const E* {
        if constexpr (STAGED) return sW; else return Wi + ch * C * DK;
    };
    auto baseQ = [&](int64_t ch) __attribute__((always_inline)) -> const E* {
        if constexpr (STAGED) return sQ; else return QGi + ch * C * DK;
    };
    auto baseK = [&](int64_t ch) __attribute__((always_inline)) -> const E* {
        if constexpr (STAGED) return sK; else return KdTi + ch * DK * C;
    };
    auto baseG = [&](int64_t ch) __attribute__((always_inline)) -> const float* {
        if constexpr (STAGED) return sG; else return Gni + ch * DK;
    };
    auto p_frag = [&](int64_t ch, int t, int kb) __attribute__((always_inline)) {
        if constexpr (STAGED) return frag(sP, p_block_index(t, kb));
        else return frag(Pi + ch * C * C, t * KB + kb);
    };
    // this wave's share of the LDS-DMA pieces: phase-a operands (W; QG too
    // with outputs) and phase-b operands (KdT, Gn; the P blocks with outputs).
    // The lane's byte offset is made opaque at every call, so that the loop
    // optimiser cannot keep a 64-bit address per piece and lane live across
    // the chunk loop (uniform base plus a 32-bit lane offset instead).
    auto lane_off = [&]() __attribute__((always_inline)) {
        int off = 16 * lane;
        asm volatile("" : "+v"(off));
        return off;
    };
    auto dma_a = [&](int c, bool out) __attribute__((always_inline)) {
        if constexpr (STAGED) {
            const int64_t ch = chunk_ch(c);
            const int lo = lane_off();
            const int np = out ? 2 * L::PW : L::PW;
#pragma unroll
            for (int kk = 0; kk < (2 * L::PW + NW - 1) / NW; ++kk) {
                const int p = w + NW * kk;
                if (p >= np) break;
                if (p < L::PW)
                    lds_dma16((const char*)(Wi + ch * C * DK) + 1024 * p + lo, (char*)sW + 1024 * p);
                else
                    lds_dma16((const char*)(QGi + ch * C * DK) + 1024 * (p - L::PW) + lo,
                              (char*)sQ + 1024 * (p - L::PW));
            }
        }
    };
    auto dma_b = [&](int c, bool out) __attribute__((always_inline)) {
        if constexpr (STAGED) {
            const int64_t ch = chunk_ch(c);
            const int lo = lane_off();
            const int np = out ? L::PK + 1 + L::NPB : L::PK + 1;
#pragma unroll
            for (int kk = 0; kk < (L::PK + 1 + L::NPB + NW - 1) / NW; ++kk) {
                const int p = w + NW * kk;
                if (p >= np) break;
                if (p < L::PK) {
                    lds_dma16((const char*)(KdTi + ch * DK * C) + 1024 * p + lo, (char*)sK + 1024 * p);
                } else if (p == L::PK) {
                    if (lane < DK * 4 / 16) lds_dma16((const char*)(Gni + ch * DK) + lo, sG);
                } else {
                    const int b = p - L::PK - 1;  // b-th kept block of P: (t, kb) in p_block_index order
                    int t = 0;
                    while (t + 1 < TT && p_block_index(t + 1, 0) <= b) ++t;
                    const int kb = b - p_block_index(t, 0);
                    lds_dma16((const char*)(Pi + ch * C * C) + 1024 * (t * KB + kb) + lo, (char*)sP + 1024 * b);
                }
            }
        }
    };
    // this wave's slice of U' of chunk c, in its stored form
    typename Raw4<E>::T up[TT];
    auto load_u = [&](int c) __attribute__((always_inline)) {
        const E* Up = UpTi + chunk_ch(c) * DV * C + (w * 64 + lane) * (C / 4);
#pragma unroll
        for (int t = 0; t < TT; ++t) up[t] = Raw4<E>::load(Up + 4 * t);
    };

    // ---- state slices: lane holds rows 16 m + 4 lg + i of column col0 + lr
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
    // device-scope accesses for the start states that pass between
    // workgroups (coherent at the device level without a whole-L2 write-back
    // or invalidate)
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
    auto wait_start = [&](int i) {
        if (tid == 0) {
            for (int spins = 0;
                 __hip_atomic_load(&seg_flags[pair * G + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
                 ++spins) {
                if (spins >= kWalk128SpinLimit) {
                    hdr->wait_timeout = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
    };

    // ---- the two phases of a chunk step of Y
    // phase a: yf = fragments of Y, X = W Y, uf = fragments of in - X with
    // in = U' (with_u) or 0 (only uf is kept across the barrier)
    auto phase_a = [&](int64_t ch, const f32x4 (&Y)[MT], bool with_u, Frag<E> (&yf)[KS], Frag<E> (&uf)[KB])
                       __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) yf[ks] = acc_to_frag(E{}, Y[2 * ks], Y[2 * ks + 1]);
        const E* Wp = baseW(ch);
        f32x4 X[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) X[t] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < TT; ++t) X[t] = mma(frag(Wp, t * KS + ks), yf[ks], X[t]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const f32x4 a = with_u ? Raw4<E>::widen(up[2 * kb]) - X[2 * kb] : -X[2 * kb];
            const f32x4 b = with_u ? Raw4<E>::widen(up[2 * kb + 1]) - X[2 * kb + 1] : -X[2 * kb + 1];
            uf[kb] = acc_to_frag(E{}, a, b);
        }
    };
    // phase b: Y <- Diag(Gn) Y + KdT (in - X)
    auto phase_b = [&](int64_t ch, f32x4 (&Y)[MT], const Frag<E> (&uf)[KB]) __attribute__((always_inline)) {
        const float* gn = baseG(ch);
#pragma unroll
        for (int m = 0; m < MT; ++m) Y[m] = *reinterpret_cast<const f32x4*>(gn + 16 * m + 4 * lg) * Y[m];
        const E* Kp = baseK(ch);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int m = 0; m < MT; ++m) Y[m] = mma(frag(Kp, m * KB + kb), uf[kb], Y[m]);
    };

    // ------------------------------------------------------------ pass 1
    if constexpr (SEG) {
        if (!last) {
            f32x4 B[MT], M[MT];
            load_state(B, first ? (S0 ? S0 + pair * DK * DV : nullptr) : nullptr);
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) M[m][i] = (16 * m + 4 * lg + i == col0 + lr) ? 1.f : 0.f;
            if (s0 < s1) {
                dma_a(s0, false);
                dma_b(s0, false);
                load_u(s0);
                wait_vmcnt<0>();
                lds_barrier();
            }
            for (int c = s0; c < s1; ++c) {
                const int64_t ch = chunk_ch(c);
                Frag<E> yf[KS], ufB[KB], ufM[KB];
                phase_a(ch, B, true, yf, ufB);
                // one product at a time: interleaving the two would keep both
                // fp32 results and two sets of operand fragments live
                __builtin_amdgcn_sched_barrier(0);
                if (!first) phase_a(ch, M, false, yf, ufM);
                wait_vmcnt<0>();
                lds_barrier();  // W read by every wave; KdT, Gn of c in LDS
                if (c + 1 < s1) dma_a(c + 1, false);
                phase_b(ch, B, ufB);
                if (!first) phase_b(ch, M, ufM);
                if (c + 1 < s1) load_u(c + 1);
                wait_vmcnt<0>();
                lds_barrier();  // KdT, Gn read by every wave; W of c + 1 in LDS
                if (c + 1 < s1) dma_b(c + 1, false);
            }
            // ---- chain: S_start(j + 1) = M S_start(j) + B (segment 0: B itself)
            if (!first) {
                // M to LDS as two bf16 parts, fragment-major with its columns
                // in fragment order (the A operand of M S), over W and QG
                // (free: the walk ended at a barrier with no loads in flight)
                E* sMh = sW;
                E* sMl = sQ;
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t at = fm_off<DK>(16 * m + 4 * lg + i, frag_pos(col0 + lr));
                        const E hi = Elt<E>::from(M[m][i]);
                        lds_put(&sMh[at], hi);
                        lds_put(&sMl[at], Elt<E>::from(M[m][i] - Elt<E>::to(hi)));
                    }
                wait_start(j);  // its barrier also orders the M tiles before their reads
                f32x4 Sj[MT];
                fetch_state(Sj, start_state(j));
                if (s0 < s1) {
                    Frag<bf16_t> sh[KS], sl[KS];
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) split_frag(Sj[2 * ks], Sj[2 * ks + 1], sh[ks], sl[ks]);
#pragma unroll
                    for (int m = 0; m < MT; ++m)
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            const Frag<E> mh = frag(sMh, m * KS + ks), ml = frag(sMl, m * KS + ks);
                            B[m] = mma(mh, sh[ks], B[m]);
                            B[m] = mma(mh, sl[ks], B[m]);
                            B[m] = mma(ml, sh[ks], B[m]);
                        }
                } else {
#pragma unroll
                    for (int m = 0; m < MT; ++m) B[m] = Sj[m];  // empty segment: the identity map
                }
            }
            publish_state(B, start_state(j + 1));
            wait_vmcnt<0>();  // this lane's part has reached the device level
            __syncthreads();  // every wave's part (and the M tiles are read)
            if (tid == 0)
                __hip_atomic_store(&seg_flags[pair * G + j + 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ------------------------------------------------------------ pass 3
    if (s0 < s1) {
        dma_a(s0, true);  // in flight during the wait below
        dma_b(s0, true);
        load_u(s0);
    }
    f32x4 S[MT];
    if (first) {
        load_state(S, S0 ? S0 + pair * DK * DV : nullptr);
    } else {
        if (last) wait_start(j);
        fetch_state(S, start_state(j));
    }
    // the O rows of chunk c from the O tile, 16-byte pieces over all waves
    auto store_o = [&](int c) __attribute__((always_inline)) {
        const int64_t t0 = seq0 + (int64_t)(c - cbeg) * C;
        constexpr int PR = DV * (int)sizeof(E) / 16;  // pieces per row
        constexpr int PE = 16 / (int)sizeof(E);       // elements per piece
#pragma unroll
        for (int kk = 0; kk < C * PR / NT; ++kk) {
            const int i = tid + NT * kk;
            const int row = i / PR, c8 = (i % PR) * PE;
            const uint4 val = *reinterpret_cast<const uint4*>(sO + row * LDO + c8);
            const int64_t tok = t0 + row;
            if (tok < seqend) *reinterpret_cast<uint4*>(o + (tok * H + h) * DV + c8) = val;
        }
    };
    if (s0 < s1) {
        wait_vmcnt<0>();
        lds_barrier();
    }
    for (int c = s0; c < s1; ++c) {
        const int64_t ch = chunk_ch(c);
        Frag<E> sf[KS], uf[KB];
        f32x4 O[TT];
        phase_a(ch, S, true, sf, uf);
        const E* Qp = baseQ(ch);
#pragma unroll
        for (int t = 0; t < TT; ++t) O[t] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < TT; ++t) O[t] = mma(frag(Qp, t * KS + ks), sf[ks], O[t]);
        if (c > s0) store_o(c - 1);
        wait_vmcnt<0>();
        lds_barrier();  // W, QG and the O tile read by every wave; KdT, Gn, P of c in LDS
        if (c + 1 < s1) dma_a(c + 1, true);
        phase_b(ch, S, uf);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < TT; ++t)
                if (!p_block_zero(t, kb)) O[t] = mma(p_frag(ch, t, kb), uf[kb], O[t]);
        if (c + 1 < s1) load_u(c + 1);
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_put(&sO[(16 * t + 4 * lg + i) * LDO + col0 + lr], Elt<E>::from(O[t][i]));
        wait_vmcnt<0>();
        lds_barrier();  // KdT, Gn, P read; the O tile written; W, QG of c + 1 in LDS
        if (c + 1 < s1) dma_b(c + 1, true);
    }
    if (s0 < s1) store_o(s1 - 1);
    if (last && S_T) store_state(S, S_T + pair * DK * DV);
}

// ----------------------------------------------------------------------------
// Host side.
template <typename E, int DK, int DV, bool HG>
static hipError_t launch_intra128(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream) {
    using L = Intra128Layout<E, DK, DV>;
    auto kern = intra128_kernel<E, DK, DV, HG>;
    static std::atomic<uint64_t> attr_done{0};
    if (hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), (int)L::bytes, attr_done);
        e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.max_chunks * a.H)), dim3(kIntra128Threads), L::bytes, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.g, (const E*)a.beta, ws.header,
                       ws.chunk_tab, a.H, (E*)ws.W, (E*)ws.QG, (E*)ws.KdT, (E*)ws.Up, (E*)ws.P, ws.Gn);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
static hipError_t launch_walk128(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream) {
    const int32_t G = ws.seg_groups > 1 ? ws.seg_groups : 1;
    const int64_t blocks = (int64_t)a.N * a.H * G;
    hipLaunchKernelGGL((walk128_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(64 * (DV / 16)), 0, stream,
                       ws.header, ws.seg_flags, ws.seg_state, ws.cu, ws.chunk_off, a.N, a.H, G, (const E*)ws.W,
                       (const E*)ws.QG, (const E*)ws.KdT, (const E*)ws.Up, (const E*)ws.P, (const float*)ws.Gn,
                       a.S0, a.S_T, (E*)a.o);
    return hipGetLastError();
}

static inline hipError_t mark128(hipEvent_t* ev, int i, hipStream_t stream) {
    return ev ? hipEventRecord(ev[i], stream) : hipSuccess;
}

template <typename E, int DK, int DV>
static hipError_t launch_chunk128_t(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream,
                                    hipEvent_t* ev) {
    hipError_t e = mark128(ev, 1, stream);
    if (e != hipSuccess) return e;
    if (a.T > 0) {
        e = a.head_gate ? launch_intra128<E, DK, DV, true>(a, ws, stream)
                        : launch_intra128<E, DK, DV, false>(a, ws, stream);
        if (e != hipSuccess) return e;
    }
    if ((e = mark128(ev, 2, stream)) != hipSuccess) return e;
    if ((e = launch_walk128<E, DK, DV>(a, ws, stream)) != hipSuccess) return e;
    return mark128(ev, 3, stream);
}

bool chunk128_supported(int32_t dk, int32_t dv, bool bf16) {
    const bool d_ok = (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
    return d_ok && (bf16 || (dk == 64 && dv == 64));
}

hipError_t launch_chunk128_kernels(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t s, hipEvent_t* ev) {
    if (!chunk128_supported(a.dk, a.dv, a.bf16)) return hipErrorInvalidValue;
    if (!a.bf16) return launch_chunk128_t<float, 64, 64>(a, ws, s, ev);
    if (a.dk == 64 && a.dv == 64) return launch_chunk128_t<bf16_t, 64, 64>(a, ws, s, ev);
    if (a.dk == 64 && a.dv == 128) return launch_chunk128_t<bf16_t, 64, 128>(a, ws, s, ev);
    if (a.dk == 128 && a.dv == 64) return launch_chunk128_t<bf16_t, 128, 64>(a, ws, s, ev);
    return launch_chunk128_t<bf16_t, 128, 128>(a, ws, s, ev);
}

}  // namespace kda
