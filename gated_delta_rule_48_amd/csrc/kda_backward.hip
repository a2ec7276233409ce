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
//   b_t  = g_0 + ... + g_t (per key channel),  r_t = b at the middle row of
//          t's 16-row tile
//   QG = Q e^b, KG = K e^b, Kd = K e^{b_last - b}, Gn = e^{b_last}
//   Qr = Q e^{b - r}, Kr = K e^{b - r}, Ki = K e^{r - b}
//   M  = strict_tril(K K^T with decay),  A = diag(beta) M,  T = (I + A)^{-1}
//   P  = tril(Q K^T with decay),  W = T diag(beta) KG,  U' = T diag(beta) V
//   U  = U' - W S,  O = QG S + P U,  S_next = Diag(Gn) S + Kd^T U
// (Inside one tile the decayed products are Qr Ki^T and Kr Ki^T; between two
// tiles the decay is rebuilt from factors <= 1, see the tile factors below.
// The references only keep the factors in range: the exact values do not
// depend on them.)
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
//        (tile by tile, with the same factors between tiles as M and P)
//   dq = dQG e^b + dQr e^{b-r},  dk = beta dXw e^b + dKr e^{b-r} + dKi e^{r-b} + dKd e^{b_last-b}
//   db = dQG QG + dQr Qr + beta dXw KG + dKr Kr - dKi Ki - dKd Kd
//        (+ sum_t dKd_t Kd_t + dGn Gn on the last row),  dv = beta dXu
//   dg = reverse cumulative sum of db over the chunk (summed over channels
//        for a per-head gate).
//
// All arithmetic is fp32; every matrix product runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32), except, for bf16 inputs, those of the two walks and
// of the first local launch, which run on the bf16 matrix cores with fp32
// accumulation (the walks' operands are stored in bf16; an fp32 operand enters
// as two bf16 parts, see the bf16 walks below).  Every intermediate of a chunk
// is kept in the workspace, except Qr, Kr and Ki (the two launches that
// multiply them form them again from q, k and b as they stage them) and dXu
// (used only inside the middle local launch).  The two walks run one
// workgroup per (sequence, head, 16-column slice) with register tiles and the
// next chunk's operands in flight; the other products of the per-chunk
// kernels run as 64 x N block products tiled through LDS with 4 x N/16
// register tiles.
#include "kda_internal.h"

#include <type_traits>

namespace kda {

namespace {

constexpr int kBwdThreads = 256;
constexpr int C = kChunk;

// Per-(chunk, head) arrays, fp32 except the walks' operands, which are kept
// in the input type; slot = chunk * H + head, where H counts the heads of the
// group being processed.  Token and state tensors are indexed with the full
// head count Hs (their row stride); the host offsets their pointers to the
// group's first head.
//
// The walks' operands.  fp32 inputs: QG, Kd, W [C][DK] and P [C][C],
// row-major.  bf16 inputs: the A operands of the walks' products in fragment
// order (frag_at), QG^T, Kd, W^T and P^T for the reverse walk, W (in Wr) and
// Kd^T (in KdT) for the state walk; Wr and KdT are empty for fp32 inputs.
struct BwdWs {
    WsHeader* header;
    int32_t* cu;
    int32_t* chunk_off;
    int2* chunk_tab;
    // [C][DK]
    float *B, *QG, *KG, *Kd, *W, *dW, *dQG, *dKd, *dXw, *Wr, *KdT;
    // [C][DV]
    float *Up, *U, *dU;
    // [C]: dbeta's row sums of dA * M and dXu * V
    float* dBr;
    // [C][C]
    float *M, *P, *T, *dP, *dA;
    // [DK]
    float *Gn, *dGn;
    // [DK][DV]: chunk start state and the state cotangent after the chunk
    float *S, *dSn;
};

template <typename E>
__device__ __forceinline__ float ld(const E* p, int64_t i) {
    return Elt<E>::load(p + i);
}

// Fragment order of an R x K matrix-core A operand (bf16, R rows, K the
// length of the contraction, a multiple of 32): blocks of 16 rows by 32 k
// (1 KB), block (r / 16, k / 32) at index (r / 16) (K / 32) + k / 32; inside
// it, lane 16 ((k % 32) / 8) + r % 16 holds k % 8 = 0..7 in 16 contiguous
// bytes (the A fragment of v_mfma_f32_16x16x32_bf16, which is also the B
// fragment of the transposed matrix).  A wave reads one block with one
// coalesced 16-byte load per lane.
template <int K>
__host__ __device__ constexpr int frag_at(int r, int k) {
    return (((r >> 4) * (K / 32) + (k >> 5)) * 64 + 16 * ((k & 31) >> 3) + (r & 15)) * 8 + (k & 7);
}

// ---------------------------------------------------------------------------
// 64 x N block product on the 256 threads of a workgroup:
//   acc(m, n) += sum_k a(m, k) b(k, n),   m < 64, n < N, k < K.
// a and b are element loaders; A_KFAST / B_NFAST say which index is the
// contiguous one in memory, so that the staging loads are coalesced.  Tiles
// of 16 k-steps pass through LDS (k-major) and are multiplied on the fp32
// matrix cores (16 x 16 x 4 per instruction): wave w owns rows 16w..16w+15,
// and lane (g, r) = (lane / 16, lane % 16) holds rows 16w + 4g + i (i < 4) of
// column 16j + r of every 16-column tile j.  The next tile is fetched into
// registers while the current one is multiplied.  Every thread of the workgroup must call it (it contains
// barriers); whatever the loaders read must be complete before the call.
constexpr int kGemmLds = 16 * (64 + 4) + 16 * (128 + 4);  // floats

template <int N>
struct Acc {
    f32x4 t[N / 16];  // t[j][i]: row row(i), column col(j)
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int j = 0; j < N / 16; ++j) t[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __device__ __forceinline__ static int row(int i) {
        return 16 * (threadIdx.x / 64) + 4 * ((threadIdx.x % 64) / 16) + i;
    }
    __device__ __forceinline__ static int col(int j) { return 16 * j + threadIdx.x % 16; }
};

template <int N, int K, bool A_KFAST, bool B_NFAST, typename LA, typename LB>
__device__ __forceinline__ void gemm64(Acc<N>& acc, LA la, LB lb, float* lds) {
    constexpr int KT = 16, M = 64, SA = M + 4, SB = N + 4, NT = N / 16;
    constexpr int RA = M * KT / kBwdThreads, RB = N * KT / kBwdThreads;
    float* sA = lds;
    float* sB = lds + KT * SA;
    const int tid = threadIdx.x, wv = tid / 64, lg = (tid % 64) / 16, lr = tid % 16;
    // element r of this thread's share of a tile
    auto a_mk = [&](int r, int& m, int& kk) {
        const int idx = tid + r * kBwdThreads;
        m = A_KFAST ? idx / KT : idx % M;
        kk = A_KFAST ? idx % KT : idx / M;
    };
    auto b_kn = [&](int r, int& kk, int& n) {
        const int idx = tid + r * kBwdThreads;
        n = B_NFAST ? idx % N : idx / KT;
        kk = B_NFAST ? idx / N : idx % KT;
    };
    // two tiles in flight: buffer 0 holds even tiles, buffer 1 odd ones
    static_assert(K % (2 * KT) == 0, "tiles in pairs");
    float ra0[RA], rb0[RB], ra1[RA], rb1[RB];
    auto fetch = [&](float (&ra)[RA], float (&rb)[RB], int k0) {
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            int m, kk;
            a_mk(r, m, kk);
            ra[r] = la(m, k0 + kk);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            int kk, n;
            b_kn(r, kk, n);
            rb[r] = lb(k0 + kk, n);
        }
    };
    auto tile = [&](float (&ra)[RA], float (&rb)[RB], int k0) {
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            int m, kk;
            a_mk(r, m, kk);
            sA[kk * SA + m] = ra[r];
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            int kk, n;
            b_kn(r, kk, n);
            sB[kk * SB + n] = rb[r];
        }
        // the tiles are shared through LDS only: the later tiles' global loads
        // stay in flight across these barriers
        lds_barrier();
        if (k0 + 2 * KT < K) fetch(ra, rb, k0 + 2 * KT);
#pragma unroll
        for (int ks = 0; ks < KT; ks += 4) {
            const float a = sA[(ks + lg) * SA + 16 * wv + lr];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const float b = sB[(ks + lg) * SB + 16 * j + lr];
                acc.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc.t[j], 0, 0, 0);
            }
        }
        lds_barrier();
    };
    fetch(ra0, rb0, 0);
    fetch(ra1, rb1, KT);
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 2 * KT) {
        tile(ra0, rb0, k0);
        tile(ra1, rb1, k0 + KT);
    }
}

// gemm64 for a B operand whose values are already in registers: lb(kt, r, k)
// gives element r of this thread's share of k-tile kt (row k of B, column
// (tid + r * threads) % N), so the tiles are staged without waiting for
// memory; A is read through la as in gemm64.  Every thread must call it.
template <int N, int K, bool A_KFAST, typename LA, typename LB>
__device__ __forceinline__ void gemm64_regb(Acc<N>& acc, LA la, LB lb, float* lds) {
    constexpr int KT = 16, M = 64, SA = M + 4, SB = N + 4, NT = N / 16;
    constexpr int RA = M * KT / kBwdThreads, RB = N * KT / kBwdThreads;
    float* sA = lds;
    float* sB = lds + KT * SA;
    const int tid = threadIdx.x, wv = tid / 64, lg = (tid % 64) / 16, lr = tid % 16;
#pragma unroll
    for (int kt = 0; kt < K / KT; ++kt) {
        const int k0 = kt * KT;
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            const int idx = tid + r * kBwdThreads;
            const int m = A_KFAST ? idx / KT : idx % M, kk = A_KFAST ? idx % KT : idx / M;
            sA[kk * SA + m] = la(m, k0 + kk);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int idx = tid + r * kBwdThreads;
            sB[(idx / N) * SB + idx % N] = lb(kt, r, k0 + idx / N);
        }
        lds_barrier();
#pragma unroll
        for (int ks = 0; ks < KT; ks += 4) {
            const float a = sA[(ks + lg) * SA + 16 * wv + lr];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const float b = sB[(ks + lg) * SB + 16 * j + lr];
                acc.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc.t[j], 0, 0, 0);
            }
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// Decay references of the four 16-row tiles of a chunk.  Tile a covers rows
// 16a..16a+15, with start row s(a) = 16a, middle row m(a) = 16a + 8 and end
// row e(a) = 16a + 15.  Every stored decayed operand of row t is referred to
// the middle row of t's own tile (Qr = Q e^{b - b_m}, Kr = K e^{b - b_m},
// Ki = K e^{b_m - b}), so each of its factors spans at most eight tokens of
// decay.  The decay between rows of two different tiles a > bb is rebuilt
// from factors that are each <= 1 (the prefix sums do not increase along the
// rows), applied one after another, so that no large intermediate value ever
// meets a small later factor:
//   fs[a]      e^{b_m(a) - b_s(a)}   takes a row operand of tile a to s(a)
//   fe[bb]     e^{b_e(bb) - b_m(bb)} takes a column operand of tile bb to e(bb)
//   fx[a,bb]   e^{b_s(a) - b_e(bb)}  from e(bb) on to s(a)   (M and P)
//   f1[a,bb]   e^{b_m(a) - b_e(bb)}  from e(bb) on to m(a)   (row-side gradients)
//   f2[a,bb]   e^{b_s(a) - b_m(bb)}  from s(a) on to m(bb)   (column-side gradients)
// for the six pairs a > bb, pair index a (a - 1) / 2 + bb.  Every exponent is
// capped at 80 nats, so that a gate outside the supported range still gives
// finite values.  f1 spans up to nine tokens, so inside the supported range
// it can fall below the smallest normal float (e^-87); the row-side results
// later multiply it by a row factor of up to e^80.  The table is therefore
// computed with the library expf, which returns subnormal results, for
// either input type (the hardware exp of the bf16 path flushes them to
// zero); the products with it keep subnormals as well.
constexpr int kTiles = C / 16;
constexpr int kPairs = kTiles * (kTiles - 1) / 2;
constexpr float kCapNats = 80.f;
__device__ __forceinline__ int pair_of(int a, int bb) { return a * (a - 1) / 2 + bb; }
__device__ __forceinline__ int tile_mid_row(int a) { return 16 * a + 8; }

template <typename E>
__device__ __forceinline__ float capped_exp(float x) { return gate_exp<E>(fminf(x, kCapNats)); }

// Rows of the factor table (each DK floats).  Prep uses rows [0, kTfPrepRows)
// and the last local launch rows [kTfLocalRow0, kTfRows), so each keeps only
// its own part in LDS (prep then fits three workgroups per compute unit).
constexpr int kTfFx = 0;                    // fx[a,bb]
constexpr int kTfFs = kTfFx + kPairs;       // fs[a]
constexpr int kTfFe = kTfFs + kTiles;       // fe[bb]
constexpr int kTfBm = kTfFe + kTiles;       // b_m(a), the reference of tile a
constexpr int kTfF1 = kTfBm + kTiles;       // f1[a,bb]
constexpr int kTfF2 = kTfF1 + kPairs;       // f2[a,bb]
constexpr int kTfRows = kTfF2 + kPairs;
constexpr int kTfPrepRows = kTfBm;          // fx, fs, fe
constexpr int kTfLocalRow0 = kTfFs;         // fs, fe, b_m, f1, f2

// Fill rows [row0, row1) of the factor table from the chunk's prefix sums
// into tf (row r at tf + (r - row0) DK); b(row, c) reads the prefix sum of
// row `row` (rows past the chunk's end hold the last sum).  Every thread of
// the workgroup calls it; the caller publishes the table with a barrier.
__device__ __forceinline__ float table_exp(float x) { return expf(fminf(x, kCapNats)); }

template <typename E, int DK, int ROW0, int ROW1, typename BF>
__device__ __forceinline__ void fill_tile_factors(float* tf, BF b) {
    for (int idx = threadIdx.x; idx < (ROW1 - ROW0) * DK; idx += kBwdThreads) {
        const int row = ROW0 + idx / DK, c = idx % DK;
        float v;
        if (row >= kTfBm && row < kTfF1) {
            v = b(tile_mid_row(row - kTfBm), c);
        } else if (row >= kTfFs && row < kTfFe) {
            const int a = row - kTfFs;
            v = table_exp(b(tile_mid_row(a), c) - b(16 * a, c));
        } else if (row >= kTfFe && row < kTfBm) {
            const int bb = row - kTfFe;
            v = table_exp(b(16 * bb + 15, c) - b(tile_mid_row(bb), c));
        } else {
            // fx (kind 0), f1 (kind 1), f2 (kind 2)
            const int kind = row < kTfFs ? 0 : (row < kTfF2 ? 1 : 2);
            const int p = row - (kind == 0 ? kTfFx : kind == 1 ? kTfF1 : kTfF2);
            const int a = p >= 3 ? 3 : (p >= 1 ? 2 : 1), bb = p - pair_of(a, 0);
            const int ra = kind == 1 ? tile_mid_row(a) : 16 * a;           // fx, f2: s(a); f1: m(a)
            const int rb = kind == 2 ? tile_mid_row(bb) : 16 * bb + 15;     // fx, f1: e(bb); f2: m(bb)
            v = table_exp(b(ra, c) - b(rb, c));
        }
        tf[idx] = v;
    }
}

// M = strict_tril(K K^T with decay) and P = tril(Q K^T with decay) of one
// chunk, by 16 x 16 tiles: wave a computes the tiles (a, bb), bb <= a, of its
// row tile.  The decayed operands are formed from q, k and the chunk's prefix
// sums b ([C][DK] in LDS) as each tile is staged: Kr = k e^{b - r},
// Qr = q e^{b - r}, Ki = k e^{r - b}, with r the b of the middle row of the
// row's own 16-row tile (rows past the chunk's end are zero).  A diagonal
// tile multiplies them as they are (both referred to m(a)); below the
// diagonal the row operand is taken to s(a) (times fs[a]) and the column
// operand to e(bb) (times fe[bb]) and on to s(a) (times fx[a,bb]).  Channels
// pass through LDS in tiles of 16; the q and k of the next two tiles are in
// flight in registers while the current one is multiplied.
// acc[bb][i] holds row 16a + 4 (lane / 16) + i, column 16bb + lane % 16.
template <typename E, int DK>
__device__ __forceinline__ void decayed_mp(const E* q, const E* k, int64_t t0, int n, int32_t Hs, int h,
                                           const float* sB, const float* tf, float* lds, f32x4 (&accM)[kTiles],
                                           f32x4 (&accP)[kTiles]) {
    constexpr int KT = 16, SA = C + 4, R = C * KT / kBwdThreads;
    float* tKr = lds;
    float* tQr = tKr + KT * SA;
    float* tKi = tQr + KT * SA;
    const int tid = threadIdx.x, lg = (tid % 64) / 16, lr = tid % 16;
    const int a = __builtin_amdgcn_readfirstlane(tid / 64);
#pragma unroll
    for (int bb = 0; bb < kTiles; ++bb) accM[bb] = accP[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // raw values in flight (converted when staged, so that nothing waits for
    // the loads before the products), two tiles ahead in three buffers; rows
    // past the end load the last row
    constexpr int NKT = DK / KT;
    E rq[3][R], rk[3][R];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int idx = tid + r * kBwdThreads;
            const int64_t o = ((t0 + min(idx / KT, n - 1)) * Hs + h) * DK + kt * KT + idx % KT;
            rq[kt][r] = q[o];
            rk[kt][r] = k[o];
        }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
        const int k0 = kt * KT, b = kt % 3;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int idx = tid + r * kBwdThreads, t = idx / KT, c = k0 + idx % KT, j = (idx % KT) * SA + t;
            const float bt = sB[t * DK + c], rm = sB[tile_mid_row(t / 16) * DK + c];
            const float er = capped_exp<E>(bt - rm), eir = capped_exp<E>(rm - bt);
            const float qv = t < n ? Elt<E>::to(rq[b][r]) : 0.f, kv = t < n ? Elt<E>::to(rk[b][r]) : 0.f;
            tKr[j] = kv * er;
            tQr[j] = qv * er;
            tKi[j] = kv * eir;
        }
        lds_barrier();
        if (kt + 2 < NKT) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int idx = tid + r * kBwdThreads;
                const int64_t o = ((t0 + min(idx / KT, n - 1)) * Hs + h) * DK + k0 + 2 * KT + idx % KT;
                rq[(kt + 2) % 3][r] = q[o];
                rk[(kt + 2) % 3][r] = k[o];
            }
        }
#pragma unroll
        for (int ks = 0; ks < KT; ks += 4) {
            const int kr = ks + lg, c = k0 + kr;
            const float ar = tKr[kr * SA + 16 * a + lr], aq = tQr[kr * SA + 16 * a + lr];
            const float fsa = tf[(kTfFs + a) * DK + c];
            const float ars = ar * fsa, aqs = aq * fsa;
#pragma unroll
            for (int bb = 0; bb < kTiles; ++bb) {
                if (bb > a) continue;
                float bi = tKi[kr * SA + 16 * bb + lr];
                const bool off = bb < a;
                if (off) bi = (bi * tf[(kTfFe + bb) * DK + c]) * tf[(kTfFx + pair_of(a, bb)) * DK + c];
                accM[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(off ? ars : ar, bi, accM[bb], 0, 0, 0);
                accP[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(off ? aqs : aq, bi, accP[bb], 0, 0, 0);
            }
        }
        lds_barrier();
    }
}

// Four stored operand values as loaded (fp32, or four bf16 in 8 bytes) and
// their widening to fp32.
template <typename ST> struct Op4;
template <> struct Op4<float> {
    typedef f32x4 T;
    __device__ __forceinline__ static f32x4 widen(T w) { return w; }
    __device__ __forceinline__ static T neg(T w) { return -w; }
};
template <> struct Op4<bf16_t> {
    typedef uint2 T;
    __device__ __forceinline__ static f32x4 widen(T w) {
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xffff0000u)};
    }
    __device__ __forceinline__ static T neg(T w) { return uint2{w.x ^ 0x80008000u, w.y ^ 0x80008000u}; }
};

// Four consecutive operand values stored in the walks' storage type (the
// arrays are laid out for fp32; a bf16 array uses the first half of its slot
// region, element i at (bf16*)base + i).
template <typename ST>
__device__ __forceinline__ void store_op4(float* base, size_t i, f32x4 v) {
    if constexpr (std::is_same<ST, float>::value) {
        *reinterpret_cast<f32x4*>(base + i) = v;
    } else {
        *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(base) + i) =
            uint2{f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])};
    }
}

// ---------------------------------------------------------------------------
// Per (chunk, head): prefix sums, decayed operands, M, P, T = (I + A)^{-1},
// W and U'.
// Three workgroups per compute unit: the registers are held to what three
// can have (one over it otherwise), the LDS fits.
template <typename E, int DK, int DV, bool HG>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_prep_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                               const E* __restrict__ v, const E* __restrict__ g,
                                                               const E* __restrict__ beta, int32_t H, int32_t Hs, BwdWs w) {
    // sA | sT for the solve; before that, the chunk's prefix sums b [C][DK]
    __shared__ __align__(16) float sAT[2 * C * (C + 1)];
    __shared__ float sbeta[C];
    __shared__ float sTf[kTfPrepRows * DK];  // tile decay factors fx, fs, fe
    constexpr int kLdsFloats = kGemmLds > 3 * 16 * (C + 4) ? kGemmLds : 3 * 16 * (C + 4);
    __shared__ __align__(16) float lds[kLdsFloats];
    static_assert(C * DK <= 2 * C * (C + 1), "prefix sums fit in the solve's LDS");
    float (*sA)[C + 1] = reinterpret_cast<float (*)[C + 1]>(sAT);
    float (*sT)[C + 1] = reinterpret_cast<float (*)[C + 1]>(sAT + C * (C + 1));
    float* sB = sAT;
    const int64_t slot = blockIdx.x;
    const int64_t chunk = slot / H;
    const int h = (int)(slot % H);
    if (w.header->bad_seqlens || chunk >= w.header->total_chunks) return;
    const int2 ct = w.chunk_tab[chunk];
    const int64_t t0 = ct.x;
    const int n = ct.y;
    const int tid = threadIdx.x;
    const size_t oCK = (size_t)slot * C * DK, oCV = (size_t)slot * C * DV, oCC = (size_t)slot * C * C;
    if (tid < C) sbeta[tid] = tid < n ? ld(beta, (t0 + tid) * Hs + h) : 0.f;
    // the chunk's gate, loaded first (rows past the end re-read the last row)
    constexpr int NG = C * DK / kBwdThreads;
    E rg[NG];
#pragma unroll
    for (int r = 0; r < NG; ++r) {
        const int idx = tid + r * kBwdThreads, t = idx / DK, c = idx % DK;
        const int64_t tr = t0 + min(t, n - 1);
        rg[r] = HG ? g[tr * Hs + h] : g[(tr * Hs + h) * DK + c];
    }
    asm volatile("" ::: "memory");  // the gate's loads go out before those of q and k
    // q and k of this thread's elements of the decayed-operand pass below,
    // issued next so that they arrive while the gate is staged and summed
    // (rows past the end re-read the last row); waiting for the gate does not
    // wait for them.  The thread takes four consecutive channels qc.. of NQ
    // consecutive rows qt0.., one load per row.
    using QK4 = typename std::conditional<std::is_same<E, float>::value, f32x4, uint2>::type;
    constexpr int NQ = C * DK / (4 * kBwdThreads);
    const int qc = 4 * (tid % (DK / 4)), qt0 = NQ * (tid / (DK / 4));
    QK4 rq4[NQ], rk4[NQ];
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int t = qt0 + it, c = qc;
        const int64_t o = ((t0 + min(t, n - 1)) * Hs + h) * DK + c;
        rq4[it] = *reinterpret_cast<const QK4*>(q + o);
        rk4[it] = *reinterpret_cast<const QK4*>(k + o);
    }
    auto elem4 = [](QK4 x, int j) -> float {
        if constexpr (std::is_same<E, float>::value) {
            return x[j];
        } else {
            const uint32_t u = j < 2 ? x.x : x.y;
            return __uint_as_float((j & 1) ? (u & 0xffff0000u) : (u << 16));
        }
    };
    // the gate into LDS (rows past the end as 0)
#pragma unroll
    for (int r = 0; r < NG; ++r) {
        const int idx = tid + r * kBwdThreads;
        sB[idx] = idx / DK < n ? Elt<E>::to(rg[r]) : 0.f;
    }
    __syncthreads();
    // prefix sums per channel, in place (rows past the end keep the last sum)
    for (int c = tid; c < DK; c += kBwdThreads) {
        float b = 0.f;
#pragma unroll
        for (int t = 0; t < C; ++t) {
            b += sB[t * DK + c];
            sB[t * DK + c] = b;
        }
        w.Gn[(size_t)slot * DK + c] = gate_exp<E>(b);
    }
    __syncthreads();
    fill_tile_factors<E, DK, 0, kTfPrepRows>(sTf, [&](int row, int c) { return sB[row * DK + c]; });
    // the prefix sums and the decayed operands the later launches read (QG,
    // KG, Kd; the tile-referred Kr, Qr, Ki are formed again from q, k and b
    // wherever they are used).  Four consecutive channels per thread, so each
    // row-major array is written with 16-byte stores; for bf16 inputs the
    // walks' fragment-ordered QG^T and Kd^T take the thread's NQ consecutive
    // rows of one channel in one store.
    constexpr bool kFrag = std::is_same<E, bf16_t>::value;
    uint32_t pq[4][NQ / 2], pk[4][NQ / 2];  // bf16 pairs of QG and Kd over rows (kFrag)
    f32x4 evQ, evK;                         // the even row's values, until its pair is packed
    const f32x4 bl4 = *reinterpret_cast<const f32x4*>(sB + (n - 1) * DK + qc);
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int t = qt0 + it, c = qc, idx = t * DK + c;
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(sB + idx);
        f32x4 oQG, oKG, oKd;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float qr = elem4(rq4[it], j), kr = elem4(rk4[it], j);
            const float qv = t < n ? qr : 0.f, kv = t < n ? kr : 0.f;
            const float b = b4[j], bl = bl4[j];
            const float e = gate_exp<E>(b), ed = gate_exp<E>(bl - b);
            oQG[j] = qv * e;
            oKG[j] = kv * e;
            oKd[j] = kv * ed;
        }
        const size_t i = oCK + idx;
        *reinterpret_cast<f32x4*>(w.B + i) = b4;
        *reinterpret_cast<f32x4*>(w.KG + i) = oKG;
        if constexpr (kFrag) {
            // Kd as the reverse walk's A operand (rows t, k = channel)
            *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(w.Kd) + oCK + frag_at<DK>(t, c)) =
                uint2{f32x2_to_bf16x2(oKd[0], oKd[1]), f32x2_to_bf16x2(oKd[2], oKd[3])};
            if (it % 2 == 0) {
                evQ = oQG;
                evK = oKd;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pq[j][it / 2] = f32x2_to_bf16x2(evQ[j], oQG[j]);
                    pk[j][it / 2] = f32x2_to_bf16x2(evK[j], oKd[j]);
                }
            }
        } else {
            store_op4<E>(w.QG, i, oQG);
            store_op4<E>(w.Kd, i, oKd);
        }
    }
    if constexpr (kFrag) {
        // QG^T (reverse walk) and Kd^T (state walk) as A operands: rows =
        // channels, k = the thread's NQ consecutive rows (NQ | 8)
        static_assert(NQ == 4 || NQ == 8, "one store per channel");
        using PK = typename std::conditional<NQ == 8, uint4, uint2>::type;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t o = oCK + frag_at<C>(qc + j, qt0);
            if constexpr (NQ == 8) {
                *reinterpret_cast<PK*>(reinterpret_cast<bf16_t*>(w.QG) + o) = PK{pq[j][0], pq[j][1], pq[j][2], pq[j][3]};
                *reinterpret_cast<PK*>(reinterpret_cast<bf16_t*>(w.KdT) + o) = PK{pk[j][0], pk[j][1], pk[j][2], pk[j][3]};
            } else {
                *reinterpret_cast<PK*>(reinterpret_cast<bf16_t*>(w.QG) + o) = PK{pq[j][0], pq[j][1]};
                *reinterpret_cast<PK*>(reinterpret_cast<bf16_t*>(w.KdT) + o) = PK{pk[j][0], pk[j][1]};
            }
        }
    }
    __syncthreads();
    // M = strict_tril(K K^T with decay) and P = tril(Q K^T with decay), by
    // tiles with the decay rebuilt from factors <= 1 below the diagonal
    {
        f32x4 am[kTiles], ap[kTiles];
        decayed_mp<E, DK>(q, k, t0, n, Hs, h, sB, sTf, lds, am, ap);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < C / 16; ++b) {
                const int t = Acc<C>::row(a), i = Acc<C>::col(b);
                const float mv = (i < t && t < n) ? am[b][a] : 0.f;
                w.M[oCC + (size_t)t * C + i] = mv;
                if constexpr (!kFrag) w.P[oCC + (size_t)t * C + i] = (i <= t && t < n) ? ap[b][a] : 0.f;
                lds_put(&sA[t][i], sbeta[t] * mv);
            }
        if constexpr (kFrag) {
            // P^T as the reverse walk's A operand (rows i, k = t): the lane's
            // four consecutive rows t are four consecutive elements
#pragma unroll
            for (int b = 0; b < C / 16; ++b) {
                const int t = Acc<C>::row(0), i = Acc<C>::col(b);
                float pv[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) pv[a] = (i <= t + a && t + a < n) ? ap[b][a] : 0.f;
                *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(w.P) + oCC + frag_at<C>(i, t)) =
                    uint2{f32x2_to_bf16x2(pv[0], pv[1]), f32x2_to_bf16x2(pv[2], pv[3])};
            }
        }
    }
    __syncthreads();
    // T = (I + A)^{-1} by 16 x 16 blocks.  The four diagonal blocks by
    // forward substitution (one column per thread of wave 0, sixteen rows);
    // the blocks below the diagonal on the fp32 matrix cores in two levels,
    // with T_a, T_b the inverses of the leading and trailing halves (the
    // inverse of [[M_a, 0], [A_ba, M_b]] is [[T_a, 0], [-T_b A_ba T_a, T_b]]):
    //   level 1  T10 = -T11 A10 T00 (wave 0),  T32 = -T33 A32 T22 (wave 1);
    //   level 2  Z = A_ba T_a:  Z20 = A20 T00 + A21 T10,  Z21 = A21 T11,
    //            Z30 = A30 T00 + A31 T10,  Z31 = A31 T11  (waves 0-3),
    //            then T20 = -T22 Z20,  T21 = -T22 Z21,
    //            T30 = -(T32 Z20 + T33 Z30),  T31 = -(T32 Z21 + T33 Z31).
    // The blocks above the diagonal are zero.  (One column per thread over
    // all 64 rows had taken about 2,000 dependent steps on one wave.)
    {
        static_assert(C == 64, "four 16-row blocks");
        const int wv = tid / 64, lg = (tid % 64) / 16, lr = tid % 16;
        if (tid < 64) {
            const int blk = tid >> 4, jc = tid & 15, b0 = 16 * blk;
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < t; ++i) acc -= sA[b0 + t][b0 + i] * x[i];
                x[t] = (t < jc) ? 0.f : ((t == jc) ? 1.f : acc);
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) sT[b0 + t][b0 + jc] = x[t];
        }
        // the six blocks above the diagonal: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        for (int idx = tid; idx < 6 * 256; idx += kBwdThreads) {
            const int pz = idx / 256, e = idx % 256;
            const int bi = pz < 3 ? 0 : (pz < 5 ? 1 : 2), bj = pz < 3 ? pz + 1 : (pz < 5 ? pz - 1 : 3);
            sT[16 * bi + e / 16][16 * bj + e % 16] = 0.f;
        }
        __syncthreads();
        // X += A[bi][m] T[m][bj]: instruction s takes k = 4 lg + s of the block
        auto mul_AT = [&](int bi, int m, int bj, f32x4 X) {
            float av[4], bv[4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                av[s4] = sA[16 * bi + lr][16 * m + 4 * lg + s4];
                bv[s4] = sT[16 * m + 4 * lg + s4][16 * bj + lr];
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) X = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s4], bv[s4], X, 0, 0, 0);
            return X;
        };
        // Y += T[bi][m] X, X in accumulator layout (which is the B operand of
        // this product: row 4 lg + s, column lr)
        auto mul_TX = [&](int bi, int m, f32x4 X, f32x4 Y) {
            float tv[4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) tv[s4] = sT[16 * bi + lr][16 * m + 4 * lg + s4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[s4], X[s4], Y, 0, 0, 0);
            return Y;
        };
        auto put_block = [&](int bi, int bj, f32x4 Y) {
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_put(&sT[16 * bi + 4 * lg + i][16 * bj + lr], -Y[i]);
        };
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        if (wv < 2) {  // level 1: block (i0 + 1, i0), i0 = 0 or 2
            const int i0 = 2 * wv;
            put_block(i0 + 1, i0, mul_TX(i0 + 1, i0 + 1, mul_AT(i0 + 1, i0, i0, z4), z4));
        }
        __syncthreads();
        constexpr int LDZ = 33;  // [32][LDZ]: rows of block rows 2 and 3, columns of block columns 0 and 1
        float* sZ = lds;
        static_assert(32 * LDZ <= kGemmLds, "Z fits in the block products' staging");
        const int zi = 2 + (wv >> 1), zj = wv & 1;  // block (zi, zj) of level 2, one per wave
        {
            f32x4 Z = z4;
            for (int m = zj; m < 2; ++m) Z = mul_AT(zi, m, zj, Z);
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_put(&sZ[(16 * (zi - 2) + 4 * lg + i) * LDZ + 16 * zj + lr], Z[i]);
        }
        __syncthreads();
        {
            f32x4 Y = z4;
            for (int m = 2; m <= zi; ++m) {
                f32x4 Zm;  // Z[m][zj] in accumulator layout
#pragma unroll
                for (int i = 0; i < 4; ++i) Zm[i] = sZ[(16 * (m - 2) + 4 * lg + i) * LDZ + 16 * zj + lr];
                Y = mul_TX(zi, m, Zm, Y);
            }
            put_block(zi, zj, Y);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, i = idx % C;
        w.T[oCC + idx] = sT[t][i];
    }
    // W = T Xw (Xw = diag(beta) KG),  U' = T Xu (Xu = diag(beta) V)
    {
        const float* KG = w.KG + oCK;
        Acc<DK> aw;
        aw.zero();
        gemm64<DK, C, true, true>(aw, [&](int t, int i) { return sT[t][i]; },
                                  [&](int i, int c) { return sbeta[i] * KG[(size_t)i * DK + c]; }, lds);
        if constexpr (kFrag) {
            // W^T for the reverse walk (rows = channels, k = t: the lane's four
            // rows t are consecutive elements) and W for the state walk (rows
            // t, k = channel: one element each)
            bf16_t* WT = reinterpret_cast<bf16_t*>(w.W) + oCK;
            bf16_t* Wr = reinterpret_cast<bf16_t*>(w.Wr) + oCK;
            const int t = Acc<DK>::row(0);
#pragma unroll
            for (int b = 0; b < DK / 16; ++b) {
                const int c = Acc<DK>::col(b);
                const f32x4 x = aw.t[b];
                *reinterpret_cast<uint2*>(WT + frag_at<C>(c, t)) =
                    uint2{f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3])};
#pragma unroll
                for (int a = 0; a < 4; ++a) Wr[frag_at<DK>(t + a, c)] = f32_to_bf16(x[a]);
            }
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < DK / 16; ++b)
                    w.W[oCK + (size_t)Acc<DK>::row(a) * DK + Acc<DK>::col(b)] = aw.t[b][a];
        }
        Acc<DV> au;
        au.zero();
        // beta_i is zero past the chunk's end, so the rows there (which re-read
        // the last row of v) give zero; a select here would be turned into a
        // branch around the load, which then waits where it is issued
        gemm64<DV, C, true, true>(au, [&](int t, int i) { return sT[t][i]; },
                                  [&](int i, int x) {
                                      return sbeta[i] * ld(v, ((t0 + min(i, n - 1)) * Hs + h) * DV + x);
                                  }, lds);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < DV / 16; ++b)
                w.Up[oCV + (size_t)Acc<DV>::row(a) * DV + Acc<DV>::col(b)] = au.t[b][a];
    }
}

// ---------------------------------------------------------------------------
// The two walks run one workgroup per (sequence, head, 16-column slice of
// d_v); their products run on the fp32 matrix cores (layout at mfma_tile).
// A chunk's operands sit in LDS (rows padded by 4 floats); the next ones are
// loaded into registers while the current chunk is computed and written to
// LDS afterwards.  The waves share only LDS, so the barriers order LDS alone
// and leave those loads in flight.

// Load a C x WIDTH fp32 block (row-major, 16-byte aligned) into registers:
// this thread's share, C * WIDTH / 1024 float4; then write it to LDS rows of
// `stride` floats.
template <int WIDTH>
constexpr int block_regs() { return C * WIDTH / 4 / kBwdThreads; }

template <int WIDTH, typename ST>
__device__ __forceinline__ void block_load(typename Op4<ST>::T (&r)[block_regs<WIDTH>()], const ST* src) {
    const typename Op4<ST>::T* s4 = reinterpret_cast<const typename Op4<ST>::T*>(src) + threadIdx.x;
#pragma unroll
    for (int i = 0; i < block_regs<WIDTH>(); ++i) r[i] = s4[i * kBwdThreads];
}

// block_load with the loads issued in index order wherever it is inlined, so
// that a wait for one register of r is computed alike on every path.
template <int WIDTH, typename ST>
__device__ __forceinline__ void block_load_ordered(typename Op4<ST>::T (&r)[block_regs<WIDTH>()], const ST* src) {
    const typename Op4<ST>::T* s4 = reinterpret_cast<const typename Op4<ST>::T*>(src) + threadIdx.x;
#pragma unroll
    for (int i = 0; i < block_regs<WIDTH>(); ++i) {
        r[i] = s4[i * kBwdThreads];
        asm volatile("" ::: "memory");
    }
}

template <int WIDTH, typename ST>
__device__ __forceinline__ void block_store(const typename Op4<ST>::T (&r)[block_regs<WIDTH>()], float* dst, int stride) {
#pragma unroll
    for (int i = 0; i < block_regs<WIDTH>(); ++i) {
        const int idx = threadIdx.x + i * kBwdThreads;
        *reinterpret_cast<f32x4*>(dst + (idx / (WIDTH / 4)) * stride + 4 * (idx % (WIDTH / 4))) = Op4<ST>::widen(r[i]);
    }
}

// Matrix-core layout of the walks (v_mfma_f32_16x16x4f32): wave wv owns
// 16-row tiles and lane (lg, lr) = (lane / 16, lane % 16) holds rows 4 lg + i
// (i < 4) of a tile in column lr.  acc += sum over k < K of A(r, k) B(k, lr),
// where a(k) reads A at the lane's row r = lr of the tile and b(k) reads
// B(k, lr); each instruction takes k = k0 + lg.  Even and odd steps of four
// accumulate separately, so two independent instructions are in flight.
// Every operand of the tile is read first and the instructions follow (a
// scheduling barrier keeps the two groups apart): left to itself the compiler
// placed each pair of reads right before its instruction, behind a wait of
// its own, so that every step paid a whole LDS round trip.
template <int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mfma_tile(f32x4 acc, FA a, FB b, int lg) {
    static_assert(K % 8 == 0, "two accumulators");
    float av[K / 4], bv[K / 4];
#pragma unroll
    for (int s = 0; s < K / 4; ++s) {
        av[s] = a(4 * s + lg);
        bv[s] = b(4 * s + lg);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 odd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K / 4; s += 2) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
        odd = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s + 1], bv[s + 1], odd, 0, 0, 0);
    }
    return acc + odd;
}

// mfma_tile for two row tiles that share the B operand: both tiles' A values
// and the common B values are read first, then the instructions of the two
// tiles interleave (four independent accumulations).  Each tile's result is
// computed exactly as mfma_tile computes it.
template <int K, typename FA0, typename FA1, typename FB>
__device__ __forceinline__ void mfma_tile2(f32x4& acc0, f32x4& acc1, FA0 a0, FA1 a1, FB b, int lg) {
    static_assert(K % 8 == 0, "two accumulators");
    float av0[K / 4], av1[K / 4], bv[K / 4];
#pragma unroll
    for (int s = 0; s < K / 4; ++s) {
        av0[s] = a0(4 * s + lg);
        av1[s] = a1(4 * s + lg);
        bv[s] = b(4 * s + lg);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 odd0 = {0.f, 0.f, 0.f, 0.f}, odd1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K / 4; s += 2) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[s], bv[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[s], bv[s], acc1, 0, 0, 0);
        odd0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[s + 1], bv[s + 1], odd0, 0, 0, 0);
        odd1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[s + 1], bv[s + 1], odd1, 0, 0, 0);
    }
    acc0 = acc0 + odd0;
    acc1 = acc1 + odd1;
}

// The (sequence, head) pair and 16-column slice of a walk workgroup.  Blocks
// are dispatched to the eight XCDs in turn (block b to XCD b mod 8); when the
// pairs fill whole rounds of eight, the NS slices of a pair are all placed on
// one XCD, so its L2 fetches the pair's per-chunk operands once instead of
// once per slice.
__device__ __forceinline__ void walk_item(int NS, int& slice, int& pair) {
    const int64_t NH = (int64_t)(gridDim.x / NS);
    const int64_t bid = blockIdx.x;
    if (NH % 8 == 0) {
        const int64_t idx = bid >> 3;
        pair = (int)((idx / NS) * 8 + (bid & 7));
        slice = (int)(idx % NS);
    } else {
        pair = (int)(bid / NS);
        slice = (int)(bid % NS);
    }
}

// ---------------------------------------------------------------------------
// Forward state walk: saves the start state S of every chunk and
// U = U' - W S, then S <- Diag(Gn) S + Kd^T U.
template <int DK, int DV>
struct StateWalkLds {
    static constexpr int SK = DK + 4;
    static constexpr int W = 0, Kd = W + C * SK, S = Kd + C * SK, U = S + DK * 16, floats = U + C * 16;
    static constexpr size_t bytes = (size_t)floats * 4;
};

// One workgroup of four waves per CU at most (LDS), so a wave may use the
// whole register file: the next two chunks' operands are held in registers.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_state_walk_kernel(int32_t H, int32_t Hs, const float* __restrict__ S0,
                                                                     BwdWs w) {
    using L = StateWalkLds<DK, DV>;
    constexpr int NS = DV / 16, SK = L::SK, TPW = DK / 64, RS = 4 * TPW;  // 16-row tiles of S per wave
    extern __shared__ __align__(16) float smem[];
    float* sW = smem + L::W;    // [C][SK]
    float* sKd = smem + L::Kd;  // [C][SK]
    float* sS = smem + L::S;    // [DK][16]
    float* sU = smem + L::U;    // [C][16]
    int sl, nh;
    walk_item(NS, sl, nh);
    const int h = nh % H;
    const int seq = nh / H;
    if (w.header->bad_seqlens) return;
    const int tid = threadIdx.x, wv = tid / 64, lg = (tid % 64) / 16, lr = tid % 16;
    const int col = sl * 16 + lr;
    const int t0 = 16 * wv + 4 * lg;  // this lane's rows of U: t0 .. t0 + 3
    auto srow = [&](int i) { return 16 * (wv * TPW + i / 4) + 4 * lg + i % 4; };  // rows of S
    const int c0 = w.chunk_off[seq], c1 = w.chunk_off[seq + 1];
    // this lane's rows of S stay in registers; sS mirrors them for the U step
    float S[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i) S[i] = S0 ? S0[(((size_t)seq * Hs + h) * DK + srow(i)) * DV + col] : 0.f;
    // Two chunks' operands in flight: buffer a holds even steps, b odd ones.
    // A wait for a load also waits for every load issued before it, so no
    // load needed sooner is issued after one needed later: a step fetches
    // W and Kd two chunks ahead once they are in LDS, and that chunk's Gn
    // and U' at its end, after their last use.  Past the sequence's last
    // chunk the fetches re-read that chunk (unused), so that every path
    // issues the same loads and the compiler's waits stay exact.
    constexpr int NR = block_regs<DK>();
    using OT = typename Op4<E>::T;  // W and Kd as stored (in the input type)
    OT rWa[NR], rKa[NR], rWb[NR], rKb[NR];
    float gna[RS], upa[4], gnb[RS], upb[4];
    auto fetch_wk = [&](int ch, OT (&rW)[NR], OT (&rK)[NR]) {
        const size_t slot = (size_t)ch * H + h;
        block_load_ordered<DK, E>(rW, reinterpret_cast<const E*>(w.W) + slot * C * DK);
        block_load_ordered<DK, E>(rK, reinterpret_cast<const E*>(w.Kd) + slot * C * DK);
    };
    auto fetch_gu = [&](int ch, float (&gn)[RS], float (&up)[4]) {
        const size_t slot = (size_t)ch * H + h;
#pragma unroll
        for (int i = 0; i < RS; ++i) gn[i] = w.Gn[slot * DK + srow(i)];
#pragma unroll
        for (int i = 0; i < 4; ++i) up[i] = w.Up[slot * C * DV + (size_t)(t0 + i) * DV + col];
    };
    auto step = [&](int ch, OT (&rW)[NR], OT (&rK)[NR], float (&gn)[RS], float (&up)[4]) {
        const size_t slot = (size_t)ch * H + h;
        const size_t oCV = slot * C * DV, oKV = slot * DK * DV;
        block_store<DK, E>(rW, sW, SK);
        block_store<DK, E>(rK, sKd, SK);
#pragma unroll
        for (int i = 0; i < RS; ++i) sS[srow(i) * 16 + lr] = S[i];
        lds_barrier();
        // operands two chunks ahead, in flight during this and the next chunk
        fetch_wk(min(ch + 2, c1 - 1), rW, rK);
        // the saved S as 16-byte stores from its LDS copy (four lanes per row)
#pragma unroll
        for (int i = tid; i < DK * 4; i += kBwdThreads)
            *reinterpret_cast<f32x4*>(w.S + oKV + (size_t)(i / 4) * DV + sl * 16 + 4 * (i % 4)) =
                *reinterpret_cast<const f32x4*>(sS + 4 * i);
        // U = U' - W S (this wave's 16 rows)
        const f32x4 ws = mfma_tile<DK>(f32x4{0.f, 0.f, 0.f, 0.f},
                                       [&](int k) { return sW[(16 * wv + lr) * SK + k]; },
                                       [&](int k) { return sS[k * 16 + lr]; }, lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) sU[(t0 + i) * 16 + lr] = up[i] - ws[i];
        lds_barrier();
        // U as 16-byte stores from its LDS copy: one per thread
        *reinterpret_cast<f32x4*>(w.U + oCV + (size_t)(tid / 4) * DV + sl * 16 + 4 * (tid % 4)) =
            *reinterpret_cast<const f32x4*>(sU + 4 * tid);
        // S <- Diag(Gn) S + Kd^T U (this wave's TPW tiles of rows; with two
        // tiles both are computed together, sharing U)
        if constexpr (TPW == 2) {
            const int m0 = 16 * (wv * TPW), m1 = m0 + 16;
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
            mfma_tile2<C>(a0, a1, [&](int k) { return sKd[k * SK + m0 + lr]; },
                          [&](int k) { return sKd[k * SK + m1 + lr]; }, [&](int k) { return sU[k * 16 + lr]; }, lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S[i] = gn[i] * S[i] + a0[i];
                S[4 + i] = gn[4 + i] * S[4 + i] + a1[i];
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int m0 = 16 * (wv * TPW + tt);
                const f32x4 a = mfma_tile<C>(f32x4{0.f, 0.f, 0.f, 0.f},
                                             [&](int k) { return sKd[k * SK + m0 + lr]; },
                                             [&](int k) { return sU[k * 16 + lr]; }, lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[4 * tt + i] = gn[4 * tt + i] * S[4 * tt + i] + a[i];
            }
        }
        fetch_gu(min(ch + 2, c1 - 1), gn, up);
        lds_barrier();
    };
    if (c0 >= c1) return;
    fetch_wk(c0, rWa, rKa);
    fetch_gu(c0, gna, upa);
    asm volatile("" ::: "memory");  // buffer a's loads all issue before buffer b's
    fetch_wk(min(c0 + 1, c1 - 1), rWb, rKb);
    fetch_gu(min(c0 + 1, c1 - 1), gnb, upb);
    for (int ch = c0; ch < c1; ch += 2) {
        step(ch, rWa, rKa, gna, upa);
        if (ch + 1 < c1) step(ch + 1, rWb, rKb, gnb, upb);
    }
}

// ---------------------------------------------------------------------------
// Reverse state walk: saves dS_next and dU = P^T dO + Kd dS_next of every
// chunk, then dS = Diag(Gn) dS_next + QG^T dO - W^T dU; dS0 at the end.
template <int DK, int DV>
struct DStateWalkLds {
    static constexpr int SK = DK + 4, SC = C + 4;
    static constexpr int P = 0, Kd = P + C * SC, QG = Kd + C * SK, W = QG + C * SK, dS = W + C * SK,
                         dU = dS + DK * 16, dO = dU + C * 16, floats = dO + 2 * C * 16;
    static constexpr size_t bytes = (size_t)floats * 4;
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dstate_walk_kernel(int32_t H, int32_t Hs, const E* __restrict__ dO,
                                                                      const float* __restrict__ dST,
                                                                      float* __restrict__ dS0, BwdWs w) {
    using L = DStateWalkLds<DK, DV>;
    constexpr int NS = DV / 16, SK = L::SK, SC = L::SC, TPW = DK / 64, RS = 4 * TPW;
    extern __shared__ __align__(16) float smem[];
    float* sP = smem + L::P;    // [C][SC]
    float* sKd = smem + L::Kd;  // [C][SK]
    float* sQG = smem + L::QG;  // [C][SK]
    float* sW = smem + L::W;    // [C][SK]
    float* sdS = smem + L::dS;  // [DK][16]
    float* sdU = smem + L::dU;  // [C][16]
    float* sdO = smem + L::dO;  // two [C][16] buffers
    int sl, nh;
    walk_item(NS, sl, nh);
    const int h = nh % H;
    const int seq = nh / H;
    if (w.header->bad_seqlens) return;
    const int tid = threadIdx.x, wv = tid / 64, lg = (tid % 64) / 16, lr = tid % 16;
    const int col = sl * 16 + lr;
    const int t0 = 16 * wv + 4 * lg;  // this lane's rows of dU (and of dO it loads)
    auto srow = [&](int i) { return 16 * (wv * TPW + i / 4) + 4 * lg + i % 4; };  // rows of dS
    const int c0 = w.chunk_off[seq], c1 = w.chunk_off[seq + 1];
    float dS[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i) dS[i] = dST ? dST[(((size_t)seq * Hs + h) * DK + srow(i)) * DV + col] : 0.f;
    if (c0 >= c1) {
        if (dS0) {
#pragma unroll
            for (int i = 0; i < RS; ++i) dS0[(((size_t)seq * Hs + h) * DK + srow(i)) * DV + col] = dS[i];
        }
        return;
    }
    // A wait for a load also waits for every load issued before it.  So no
    // load's address depends on another load inside the loop (a chunk's
    // tokens follow from the sequence's offsets), no load sits in a branch,
    // and each chunk's loads are issued in the order they are needed: a
    // step starts by fetching the previous chunk's dO, P, Kd (staged at its
    // end) and, after its second barrier, that chunk's Gn, QG, W (Gn for its
    // end, QG and W for the middle of the next step).
    const int tok0 = w.cu[seq], tok1 = w.cu[seq + 1];
    // dO of a chunk for this lane's 4 rows of column `col`, as stored; rows
    // past the chunk's end re-read its last row and are zeroed when staged
    auto rows_of = [&](int ch) { return min(C, tok1 - (tok0 + (ch - c0) * C)); };
    auto load_dO = [&](int ch, E (&r)[4]) {
        const int first = tok0 + (ch - c0) * C, n = rows_of(ch);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = dO[(((int64_t)first + min(t0 + i, n - 1)) * Hs + h) * DV + col];
    };
    auto stage_dO = [&](int ch, const E (&r)[4], float* dst) {
        const int n = rows_of(ch);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(t0 + i) * 16 + lr] = t0 + i < n ? Elt<E>::to(r[i]) : 0.f;
    };
    constexpr int NP = block_regs<C>(), NK = block_regs<DK>();
    using OT = typename Op4<E>::T;  // P, Kd, QG and W as stored (in the input type)
    OT rP[NP], rK[NK], rQ[NK], rW[NK];
    E rO[4];
    float gn[RS], gnn[RS];
    auto fetch_far = [&](int ch) {  // P, Kd, dO: staged at the end of the step that fetches them
        const size_t slot = (size_t)ch * H + h;
        load_dO(ch, rO);
        block_load_ordered<C, E>(rP, reinterpret_cast<const E*>(w.P) + slot * C * C);
        block_load_ordered<DK, E>(rK, reinterpret_cast<const E*>(w.Kd) + slot * C * DK);
        asm volatile("" ::: "memory");
    };
    auto fetch_near = [&](int ch) {  // Gn, QG, W: used at the end of this step and in the next one
        const size_t slot = (size_t)ch * H + h;
#pragma unroll
        for (int i = 0; i < RS; ++i) gnn[i] = w.Gn[slot * DK + srow(i)];
        asm volatile("" ::: "memory");
        block_load_ordered<DK, E>(rQ, reinterpret_cast<const E*>(w.QG) + slot * C * DK);
        block_load_ordered<DK, E>(rW, reinterpret_cast<const E*>(w.W) + slot * C * DK);
    };
    int buf = 0;
    fetch_far(c1 - 1);
    fetch_near(c1 - 1);
    block_store<C, E>(rP, sP, SC);
    block_store<DK, E>(rK, sKd, SK);
    stage_dO(c1 - 1, rO, sdO);
#pragma unroll
    for (int i = 0; i < RS; ++i) gn[i] = gnn[i];
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int ch = c1 - 1; ch >= c0; --ch) {
        const size_t slot = (size_t)ch * H + h;
        const size_t oCV = slot * C * DV, oKV = slot * DK * DV;
        float* dOc = sdO + buf * C * 16;
        // this chunk's P and Kd are in LDS already: the previous chunk's are
        // fetched now, in flight during both product phases (past the first
        // chunk this re-reads it, unused)
        fetch_far(max(ch - 1, c0));
#pragma unroll
        for (int i = 0; i < RS; ++i) sdS[srow(i) * 16 + lr] = dS[i];
        lds_barrier();
        // the saved dS_next as 16-byte stores from its LDS copy (four lanes per row)
#pragma unroll
        for (int i = tid; i < DK * 4; i += kBwdThreads)
            *reinterpret_cast<f32x4*>(w.dSn + oKV + (size_t)(i / 4) * DV + sl * 16 + 4 * (i % 4)) =
                *reinterpret_cast<const f32x4*>(sdS + 4 * i);
        // dU = P^T dO + Kd dS_next (this wave's 16 rows)
        f32x4 du = mfma_tile<C>(zero, [&](int k) { return sP[k * SC + 16 * wv + lr]; },
                                [&](int k) { return dOc[k * 16 + lr]; }, lg);
        du = mfma_tile<DK>(du, [&](int k) { return sKd[(16 * wv + lr) * SK + k]; },
                           [&](int k) { return sdS[k * 16 + lr]; }, lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) sdU[(t0 + i) * 16 + lr] = du[i];
        // no work that waits for the loads in flight is scheduled into the products
        __builtin_amdgcn_sched_barrier(0);
        block_store<DK, E>(rQ, sQG, SK);
#pragma unroll
        for (int i = 0; i < NK; ++i) rW[i] = Op4<E>::neg(rW[i]);
        block_store<DK, E>(rW, sW, SK);  // sW holds -W
        lds_barrier();
        *reinterpret_cast<f32x4*>(w.dU + oCV + (size_t)(tid / 4) * DV + sl * 16 + 4 * (tid % 4)) =
            *reinterpret_cast<const f32x4*>(sdU + 4 * tid);
        fetch_near(max(ch - 1, c0));
        // dS = Diag(Gn) dS_next + QG^T dO - W^T dU (this wave's TPW tiles of
        // rows; with two tiles both are computed together, sharing dO and dU)
        if constexpr (TPW == 2) {
            const int m0 = 16 * (wv * TPW), m1 = m0 + 16;
            f32x4 a0 = zero, a1 = zero;
            mfma_tile2<C>(a0, a1, [&](int k) { return sQG[k * SK + m0 + lr]; },
                          [&](int k) { return sQG[k * SK + m1 + lr]; }, [&](int k) { return dOc[k * 16 + lr]; }, lg);
            mfma_tile2<C>(a0, a1, [&](int k) { return sW[k * SK + m0 + lr]; },
                          [&](int k) { return sW[k * SK + m1 + lr]; }, [&](int k) { return sdU[k * 16 + lr]; }, lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dS[i] = gn[i] * dS[i] + a0[i];
                dS[4 + i] = gn[4 + i] * dS[4 + i] + a1[i];
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int m0 = 16 * (wv * TPW + tt);
                f32x4 a = mfma_tile<C>(zero, [&](int k) { return sQG[k * SK + m0 + lr]; },
                                       [&](int k) { return dOc[k * 16 + lr]; }, lg);
                a = mfma_tile<C>(a, [&](int k) { return sW[k * SK + m0 + lr]; },
                                 [&](int k) { return sdU[k * 16 + lr]; }, lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) dS[4 * tt + i] = gn[4 * tt + i] * dS[4 * tt + i] + a[i];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // the staging below stays after the products
        // sP and sKd were last read before the second barrier, the other dO
        // buffer a step ago; the next step's first barrier publishes these
        block_store<C, E>(rP, sP, SC);
        block_store<DK, E>(rK, sKd, SK);
        stage_dO(max(ch - 1, c0), rO, sdO + (buf ^ 1) * C * 16);
#pragma unroll
        for (int i = 0; i < RS; ++i) gn[i] = gnn[i];
        buf ^= 1;
    }
    if (dS0) {
#pragma unroll
        for (int i = 0; i < RS; ++i) dS0[(((size_t)seq * Hs + h) * DK + srow(i)) * DV + col] = dS[i];
    }
}

// ---------------------------------------------------------------------------
// The two walks for bf16 inputs, on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16).  Their operands were rounded to bf16 when prep
// stored them, in fragment order (frag_at), so each wave loads the fragments
// of its own tiles straight into registers, one chunk ahead, and no operand
// passes through LDS.  The fp32 state (S, or dS) and U (or dU) enter a product
// as two bf16 parts, x = hi + lo with hi = bf16(x) and lo = bf16(x - hi),
// which carry about 16 significant bits; dO is bf16 already.  LDS holds only
// what the waves exchange: those parts and dO, transposed (16 rows, one per
// column of the slice) as the products' B fragments, and fp32 copies of the
// state and of U (dU) for the 16-byte stores of the saved values.
// Same work item per workgroup and the same results in the workspace as the
// fp32 walks above.

// Eight bytes to LDS as one store that is never paired with another
// (lds_put; matrix-core results reach LDS only this way)
__device__ __forceinline__ void lds_put8(bf16_t* p, uint2 v) {
    lds_put(reinterpret_cast<unsigned long long*>(p), (static_cast<unsigned long long>(v.y) << 32) | v.x);
}

// x = hi + lo for four values, each part as four packed bf16
__device__ __forceinline__ void split4(f32x4 x, uint2& hi, uint2& lo) {
    const uint32_t h01 = f32x2_to_bf16x2(x[0], x[1]), h23 = f32x2_to_bf16x2(x[2], x[3]);
    hi = uint2{h01, h23};
    lo = uint2{f32x2_to_bf16x2(x[0] - __uint_as_float(h01 << 16), x[1] - __uint_as_float(h01 & 0xffff0000u)),
               f32x2_to_bf16x2(x[2] - __uint_as_float(h23 << 16), x[3] - __uint_as_float(h23 & 0xffff0000u))};
}

// fragment f of a fragment-ordered operand (one coalesced 16-byte load per lane)
__device__ __forceinline__ Frag<bf16_t> load_frag(const bf16_t* base, int f, int lane) {
    Frag<bf16_t> r;
    r.v = *reinterpret_cast<const u16x8*>(base + f * 512 + lane * 8);
    return r;
}

// LDS of the bf16 walks, in floats: fp32 copies [rows][16], then the bf16
// transposed parts [16][rows + 8] (the pad spreads a fragment read's rows
// over the banks)
template <int DK>
struct WalkLdsB {
    static constexpr int SK = DK + 8, SC = C + 8;  // bf16 row strides
    static constexpr int X = 0, Y = X + DK * 16, Xh = Y + C * 16, Xl = Xh + 8 * SK, Yh = Xl + 8 * SK,
                         Yl = Yh + 8 * SC, O = Yl + 8 * SC, floats = O + 8 * SC;
};

// Forward state walk (bf16 inputs): saves S and U = U' - W S of every chunk,
// then S <- Diag(Gn) S + Kd^T U.
template <int DK>
struct StateOpsB {
    Frag<bf16_t> w[DK / 32];          // W: the wave's 16 rows t, k over the channels
    float up[4];                      // U' of the lane's rows t0 .. t0 + 3 in column col
    Frag<bf16_t> kt[DK / 64 * C / 32];  // Kd^T: the wave's channel tiles, k over the rows
    f32x4 gn[DK / 64];                // Gn of the lane's rows of S
};

template <int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_state_walk_bf16_kernel(
    int32_t H, int32_t Hs, const float* __restrict__ S0, BwdWs w) {
    using L = WalkLdsB<DK>;
    constexpr int NS = DV / 16, SK = L::SK, SC = L::SC, TPW = DK / 64, RS = 4 * TPW, KBD = DK / 32, KBC = C / 32;
    __shared__ __align__(16) float smem[L::floats];
    float* sS = smem + L::X;                                // [DK][16]
    float* sU = smem + L::Y;                                // [C][16]
    bf16_t* sSh = reinterpret_cast<bf16_t*>(smem + L::Xh);  // [16][SK]: S^T, both parts
    bf16_t* sSl = reinterpret_cast<bf16_t*>(smem + L::Xl);
    bf16_t* sUh = reinterpret_cast<bf16_t*>(smem + L::Yh);  // [16][SC]: U^T, both parts
    bf16_t* sUl = reinterpret_cast<bf16_t*>(smem + L::Yl);
    int sl, nh;
    walk_item(NS, sl, nh);
    const int h = nh % H;
    const int seq = nh / H;
    if (w.header->bad_seqlens) return;
    const int tid = threadIdx.x, wv = tid / 64, lane = tid % 64, lg = lane / 16, lr = lane % 16;
    const int col = sl * 16 + lr;
    const int t0 = 16 * wv + 4 * lg;  // this lane's rows of U
    const int c0 = w.chunk_off[seq], c1 = w.chunk_off[seq + 1];
    // this lane's rows of S (16 (wv TPW + tt) + 4 lg + i) stay in registers
    float S[RS];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[4 * tt + i] =
                S0 ? S0[(((size_t)seq * Hs + h) * DK + 16 * (wv * TPW + tt) + 4 * lg + i) * DV + col] : 0.f;
    if (c0 >= c1) return;
    // Loads in the order of use; past the sequence's last chunk the fetches
    // re-read that chunk (unused), so that every path issues the same loads.
    auto fetch = [&](int ch, StateOpsB<DK>& X) {
        const size_t slot = (size_t)ch * H + h;
        const bf16_t* Wr = reinterpret_cast<const bf16_t*>(w.Wr) + slot * C * DK;
        const bf16_t* KT = reinterpret_cast<const bf16_t*>(w.KdT) + slot * C * DK;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) X.w[kb] = load_frag(Wr, wv * KBD + kb, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) X.up[i] = w.Up[slot * C * DV + (size_t)(t0 + i) * DV + col];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) X.kt[tt * KBC + kb] = load_frag(KT, (wv * TPW + tt) * KBC + kb, lane);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
            X.gn[tt] = *reinterpret_cast<const f32x4*>(w.Gn + slot * DK + 16 * (wv * TPW + tt) + 4 * lg);
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // X holds chunk ch; the next chunk's operands are fetched into Y first,
    // so they are in flight during the whole step
    auto step = [&](int ch, StateOpsB<DK>& X, StateOpsB<DK>& Y) {
        const size_t slot = (size_t)ch * H + h;
        const size_t oCV = slot * C * DV, oKV = slot * DK * DV;
        fetch(min(ch + 1, c1 - 1), Y);
        // S: the fp32 copy for the saved state, the two parts for the product
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int r0 = 16 * (wv * TPW + tt) + 4 * lg;
            const f32x4 x = {S[4 * tt], S[4 * tt + 1], S[4 * tt + 2], S[4 * tt + 3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_put(&sS[(r0 + i) * 16 + lr], x[i]);
            uint2 hi, lo;
            split4(x, hi, lo);
            lds_put8(sSh + lr * SK + r0, hi);
            lds_put8(sSl + lr * SK + r0, lo);
        }
        lds_barrier();
        // the saved S as 16-byte stores from its fp32 copy (four lanes per row)
#pragma unroll
        for (int i = tid; i < DK * 4; i += kBwdThreads)
            *reinterpret_cast<f32x4*>(w.S + oKV + (size_t)(i / 4) * DV + sl * 16 + 4 * (i % 4)) =
                *reinterpret_cast<const f32x4*>(sS + 4 * i);
        // U = U' - W S (this wave's 16 rows)
        Frag<bf16_t> bh[KBD], bl[KBD];
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            bh[kb] = ld_frag(sSh + lr * SK + 32 * kb + 8 * lg);
            bl[kb] = ld_frag(sSl + lr * SK + 32 * kb + 8 * lg);
        }
        f32x4 wh = zero, wl = zero;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            wh = mma(X.w[kb], bh[kb], wh);
            wl = mma(X.w[kb], bl[kb], wl);
        }
        f32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = X.up[i] - (wh[i] + wl[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_put(&sU[(t0 + i) * 16 + lr], u[i]);
        {
            uint2 hi, lo;
            split4(u, hi, lo);
            lds_put8(sUh + lr * SC + t0, hi);
            lds_put8(sUl + lr * SC + t0, lo);
        }
        lds_barrier();
        // U as 16-byte stores from its fp32 copy: one per thread
        *reinterpret_cast<f32x4*>(w.U + oCV + (size_t)(tid / 4) * DV + sl * 16 + 4 * (tid % 4)) =
            *reinterpret_cast<const f32x4*>(sU + 4 * tid);
        // S <- Diag(Gn) S + Kd^T U (this wave's TPW tiles of rows)
        Frag<bf16_t> uh[KBC], ul[KBC];
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) {
            uh[kb] = ld_frag(sUh + lr * SC + 32 * kb + 8 * lg);
            ul[kb] = ld_frag(sUl + lr * SC + 32 * kb + 8 * lg);
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            f32x4 ah = zero, al = zero;
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                ah = mma(X.kt[tt * KBC + kb], uh[kb], ah);
                al = mma(X.kt[tt * KBC + kb], ul[kb], al);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) S[4 * tt + i] = X.gn[tt][i] * S[4 * tt + i] + (ah[i] + al[i]);
        }
    };
    StateOpsB<DK> A, B;
    fetch(c0, A);
    // whole rounds of two steps (A, then B), then the chunk left (in A)
    int ch = c0;
    for (; ch + 1 < c1; ch += 2) {
        step(ch, A, B);
        step(ch + 1, B, A);
    }
    if (ch < c1) step(ch, A, B);
}

// Reverse state walk (bf16 inputs): saves dS_next and dU = P^T dO + Kd dS_next
// of every chunk, then dS = Diag(Gn) dS_next + QG^T dO - W^T dU; dS0 at the end.
template <int DK>
struct RevOpsB {
    uint2 o;                            // dO: row tid / 4, columns 4 (tid % 4) .. + 3 of the slice
    Frag<bf16_t> pt[C / 32];            // P^T: the wave's 16 rows, k over the chunk's rows
    Frag<bf16_t> kd[DK / 32];           // Kd: the wave's 16 rows t, k over the channels
    Frag<bf16_t> qt[DK / 64 * C / 32];  // QG^T: the wave's channel tiles, k over the rows
    Frag<bf16_t> wt[DK / 64 * C / 32];  // W^T: likewise
    f32x4 gn[DK / 64];                  // Gn of the lane's rows of dS
};

template <int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dstate_walk_bf16_kernel(
    int32_t H, int32_t Hs, const bf16_t* __restrict__ dO, const float* __restrict__ dST, float* __restrict__ dS0,
    BwdWs w) {
    using L = WalkLdsB<DK>;
    constexpr int NS = DV / 16, SK = L::SK, SC = L::SC, TPW = DK / 64, RS = 4 * TPW, KBD = DK / 32, KBC = C / 32;
    __shared__ __align__(16) float smem[L::floats];
    float* sdS = smem + L::X;                               // [DK][16]
    float* sdU = smem + L::Y;                               // [C][16]
    bf16_t* sDh = reinterpret_cast<bf16_t*>(smem + L::Xh);  // [16][SK]: dS_next^T, both parts
    bf16_t* sDl = reinterpret_cast<bf16_t*>(smem + L::Xl);
    bf16_t* sUh = reinterpret_cast<bf16_t*>(smem + L::Yh);  // [16][SC]: dU^T, both parts
    bf16_t* sUl = reinterpret_cast<bf16_t*>(smem + L::Yl);
    bf16_t* sO = reinterpret_cast<bf16_t*>(smem + L::O);    // [16][SC]: dO^T
    int sl, nh;
    walk_item(NS, sl, nh);
    const int h = nh % H;
    const int seq = nh / H;
    if (w.header->bad_seqlens) return;
    const int tid = threadIdx.x, wv = tid / 64, lane = tid % 64, lg = lane / 16, lr = lane % 16;
    const int col = sl * 16 + lr;
    const int t0 = 16 * wv + 4 * lg;  // this lane's rows of dU (and of dO it loads)
    const int c0 = w.chunk_off[seq], c1 = w.chunk_off[seq + 1];
    auto srow = [&](int i) { return 16 * (wv * TPW + i / 4) + 4 * lg + i % 4; };  // rows of dS
    float dS[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i) dS[i] = dST ? dST[(((size_t)seq * Hs + h) * DK + srow(i)) * DV + col] : 0.f;
    if (c0 < c1) {
        const int tok0 = w.cu[seq], tok1 = w.cu[seq + 1];
        // rows past a chunk's end re-read its last row and are zeroed when staged
        auto rows_of = [&](int ch) { return min(C, tok1 - (tok0 + (ch - c0) * C)); };
        auto fetch = [&](int ch, RevOpsB<DK>& X) {
            const size_t slot = (size_t)ch * H + h;
            const int first = tok0 + (ch - c0) * C, n = rows_of(ch);
            X.o = *reinterpret_cast<const uint2*>(dO + (((int64_t)first + min(tid / 4, n - 1)) * Hs + h) * DV + sl * 16 +
                                                  4 * (tid % 4));
            const bf16_t* P = reinterpret_cast<const bf16_t*>(w.P) + slot * C * C;
            const bf16_t* Kd = reinterpret_cast<const bf16_t*>(w.Kd) + slot * C * DK;
            const bf16_t* QT = reinterpret_cast<const bf16_t*>(w.QG) + slot * C * DK;
            const bf16_t* WT = reinterpret_cast<const bf16_t*>(w.W) + slot * C * DK;
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) X.pt[kb] = load_frag(P, wv * KBC + kb, lane);
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) X.kd[kb] = load_frag(Kd, wv * KBD + kb, lane);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) X.qt[tt * KBC + kb] = load_frag(QT, (wv * TPW + tt) * KBC + kb, lane);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) X.wt[tt * KBC + kb] = load_frag(WT, (wv * TPW + tt) * KBC + kb, lane);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
                X.gn[tt] = *reinterpret_cast<const f32x4*>(w.Gn + slot * DK + 16 * (wv * TPW + tt) + 4 * lg);
        };
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        // Every LDS array is written before the step's first barrier or
        // between its two, and read between the two or after the second; so
        // one copy of each suffices.
        // X holds chunk ch; the previous chunk's operands are fetched into Y
        // first, so they are in flight during the whole step
        auto step = [&](int ch, RevOpsB<DK>& X, RevOpsB<DK>& Y) {
            const size_t slot = (size_t)ch * H + h;
            const size_t oCV = slot * C * DV, oKV = slot * DK * DV;
            fetch(max(ch - 1, c0), Y);
            {
                // dO transposed, zero past the chunk's end
                const int t = tid / 4, c = 4 * (tid % 4);
                const uint2 o = t < rows_of(ch) ? X.o : uint2{0u, 0u};
                sO[(c + 0) * SC + t] = (bf16_t)(o.x & 0xffffu);
                sO[(c + 1) * SC + t] = (bf16_t)(o.x >> 16);
                sO[(c + 2) * SC + t] = (bf16_t)(o.y & 0xffffu);
                sO[(c + 3) * SC + t] = (bf16_t)(o.y >> 16);
            }
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int r0 = 16 * (wv * TPW + tt) + 4 * lg;
                const f32x4 x = {dS[4 * tt], dS[4 * tt + 1], dS[4 * tt + 2], dS[4 * tt + 3]};
#pragma unroll
                for (int i = 0; i < 4; ++i) lds_put(&sdS[(r0 + i) * 16 + lr], x[i]);
                uint2 hi, lo;
                split4(x, hi, lo);
                lds_put8(sDh + lr * SK + r0, hi);
                lds_put8(sDl + lr * SK + r0, lo);
            }
            lds_barrier();
            // the saved dS_next as 16-byte stores from its fp32 copy (four lanes per row)
#pragma unroll
            for (int i = tid; i < DK * 4; i += kBwdThreads)
                *reinterpret_cast<f32x4*>(w.dSn + oKV + (size_t)(i / 4) * DV + sl * 16 + 4 * (i % 4)) =
                    *reinterpret_cast<const f32x4*>(sdS + 4 * i);
            // dU = P^T dO + Kd dS_next (this wave's 16 rows)
            Frag<bf16_t> of[KBC], dh[KBD], dl[KBD];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) of[kb] = ld_frag(sO + lr * SC + 32 * kb + 8 * lg);
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                dh[kb] = ld_frag(sDh + lr * SK + 32 * kb + 8 * lg);
                dl[kb] = ld_frag(sDl + lr * SK + 32 * kb + 8 * lg);
            }
            f32x4 uo = zero, uh = zero, ul = zero;
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) uo = mma(X.pt[kb], of[kb], uo);
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                uh = mma(X.kd[kb], dh[kb], uh);
                ul = mma(X.kd[kb], dl[kb], ul);
            }
            f32x4 du;
#pragma unroll
            for (int i = 0; i < 4; ++i) du[i] = uo[i] + (uh[i] + ul[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_put(&sdU[(t0 + i) * 16 + lr], du[i]);
            {
                uint2 hi, lo;
                split4(du, hi, lo);
                lds_put8(sUh + lr * SC + t0, hi);
                lds_put8(sUl + lr * SC + t0, lo);
            }
            lds_barrier();
            // dU as 16-byte stores from its fp32 copy: one per thread
            *reinterpret_cast<f32x4*>(w.dU + oCV + (size_t)(tid / 4) * DV + sl * 16 + 4 * (tid % 4)) =
                *reinterpret_cast<const f32x4*>(sdU + 4 * tid);
            // dS = Diag(Gn) dS_next + QG^T dO - W^T dU (this wave's TPW tiles of rows)
            Frag<bf16_t> eh[KBC], el[KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                eh[kb] = ld_frag(sUh + lr * SC + 32 * kb + 8 * lg);
                el[kb] = ld_frag(sUl + lr * SC + 32 * kb + 8 * lg);
            }
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                f32x4 aq = zero, ah = zero, al = zero;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) {
                    aq = mma(X.qt[tt * KBC + kb], of[kb], aq);
                    ah = mma(X.wt[tt * KBC + kb], eh[kb], ah);
                    al = mma(X.wt[tt * KBC + kb], el[kb], al);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) dS[4 * tt + i] = X.gn[tt][i] * dS[4 * tt + i] + (aq[i] - (ah[i] + al[i]));
            }
        };
        RevOpsB<DK> A, B;
        fetch(c1 - 1, A);
        // whole rounds of two steps (A, then B), then the chunk left (in A)
        int ch = c1 - 1;
        for (; ch - 1 >= c0; ch -= 2) {
            step(ch, A, B);
            step(ch - 1, B, A);
        }
        if (ch >= c0) step(ch, A, B);
    }
    if (dS0) {
#pragma unroll
        for (int i = 0; i < RS; ++i) dS0[(((size_t)seq * Hs + h) * DK + srow(i)) * DV + col] = dS[i];
    }
}

// ---------------------------------------------------------------------------
// Per (chunk, head): gradients of the chunk's inputs from dU, dS_next, S, U.
// Three launches, PH = 0, 1, 2: phase 1; phases 2-4; phases 5-6.  The
// phases exchange everything through the workspace, so the split only moves
// barriers to kernel boundaries; each launch holds far fewer registers.
template <typename E, int DK, int DV, bool HG, int PH>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(PH == 1 ? 3 : 2))) void bwd_local_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                                const E* __restrict__ v, const E* __restrict__ beta,
                                                                const E* __restrict__ dO, int32_t H, int32_t Hs, BwdWs w,
                                                                E* __restrict__ dq, E* __restrict__ dk,
                                                                E* __restrict__ dv, E* __restrict__ dg,
                                                                E* __restrict__ dbeta) {
    __shared__ float sbeta[C];
    __shared__ float sbl[DK];
    __shared__ float sRowKG[C];       // sum_c dXw[t][c] KG[t][c], per row
    __shared__ float sColKd[4 * DK];  // sum_t dKd[t][c] Kd[t][c], per wave and column
    // phases 1 and 5 stage five and seven operand tiles at once (phase 1 for
    // bf16 inputs: the two bf16 parts of S, dS_next and U for 32 value
    // columns, rows padded to 40); phases 2-4 use gemm64's two
    constexpr bool kBf = std::is_same<E, bf16_t>::value;
    constexpr int kLdsFloats = PH == 0   ? (kBf ? (4 * DK + 2 * C) * 20 : 16 * (3 * (C + 4) + 2 * (DK + 4)))
                               : PH == 2 ? (16 * 3 * (DK + 4) > C * (DK + 1) ? 16 * 3 * (DK + 4) : C * (DK + 1))
                                         : kGemmLds;
    __shared__ __align__(16) float lds[kLdsFloats];
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
    if (tid < C) sbeta[tid] = tid < n ? ld(beta, (t0 + tid) * Hs + h) : 0.f;
    if (tid < DK) sbl[tid] = w.B[oCK + (size_t)(n - 1) * DK + tid];
    __syncthreads();  // sbeta, sbl are read by every thread (also inside block-product loaders)
    const float* Sm = w.S + oKV;
    const float* dSn = w.dSn + oKV;
    const float* Um = w.U + oCV;
    const float* dUm = w.dU + oCV;
    const float* Tm = w.T + oCC;  // T[a][i] at Tm[a * C + i]
    // dO of row t (zero past the chunk's end; the load itself is
    // unconditional, so that the prefetch is not waited for where it is issued)
    auto dOat = [&](int t, int x) -> float {
        const float d = ld(dO, ((t0 + min(t, n - 1)) * Hs + h) * DV + x);
        return t < n ? d : 0.f;
    };
    // store a 64 x N accumulator tile (times s) to dst (row stride N), rows >= n as zero
    auto put = [&](auto& acc, float* dst, int N, float s) {
        constexpr int NT = sizeof(acc.t) / sizeof(acc.t[0]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < NT; ++b) {
                const int t = 16 * (tid / 64) + 4 * ((tid % 64) / 16) + a, c = 16 * b + tid % 16;
                dst[(size_t)t * N + c] = t < n ? s * acc.t[b][a] : 0.f;
            }
    };

    if constexpr (PH == 0 && kBf) {
    // phase 1 for bf16 inputs, on the bf16 matrix cores: dW = -dU S^T,
    // dQG = dO S^T, dKd = U dS_next^T, dP = tril(dO U^T) and dGn[c] = sum_x
    // S[c][x] dS_next[c][x].  Every product contracts over the value index x,
    // which is contiguous in every operand, so a fragment (frag_at) is eight
    // consecutive x of one row.  Per block of 32 x, S, dS_next and U (the B
    // sides, all their rows) are staged in LDS as two bf16 parts,
    // x = hi + lo; the wave's rows of dU and dO (the A sides) are loaded into
    // registers, dU split likewise and dO exact; U as an A side is read from
    // its staged parts.  A product of two split operands is hi hi + hi lo +
    // lo hi (the dropped lo lo is below 2^-16 of it); one with dO is dO hi +
    // dO lo.  dGn is summed in fp32 from the values as loaded.
    {
        constexpr int XB = 32, SP = XB + 8, NT = DK / 16;
        bf16_t* sSh = reinterpret_cast<bf16_t*>(lds);  // [DK][SP]
        bf16_t* sSl = sSh + DK * SP;
        bf16_t* sDh = sSl + DK * SP;                   // dS_next, [DK][SP]
        bf16_t* sDl = sDh + DK * SP;
        bf16_t* sUh = sDl + DK * SP;                   // [C][SP]
        bf16_t* sUl = sUh + C * SP;
        static_assert((4 * DK + 2 * C) * SP <= 2 * kLdsFloats, "phase-1 parts fit");
        const int wv = tid / 64, lg = (tid % 64) / 16, lr = tid % 16;
        const int ta = 16 * wv + lr;  // the lane's row of the A sides
        // staging shares: rows cs of S and dS_next (TS threads a row, XS
        // values each), rows cu of U (TU threads a row, XU values each)
        constexpr int TS = kBwdThreads / DK, XS = XB / TS, TU = kBwdThreads / C, XU = XB / TU;
        const int cs = tid / TS, xs = XS * (tid % TS), cu = tid / TU, xu = XU * (tid % TU);
        Acc<DK> aW, aQ, aK;
        Acc<C> aP;
        aW.zero();
        aQ.zero();
        aK.zero();
        aP.zero();
        f32x4 rS[XS / 4], rD[XS / 4], rU[XU / 4], rdU[2];
        uint4 rdO;
        auto fetch = [&](int x0) {
#pragma unroll
            for (int i = 0; i < XS / 4; ++i) {
                rS[i] = *reinterpret_cast<const f32x4*>(Sm + (size_t)cs * DV + x0 + xs + 4 * i);
                rD[i] = *reinterpret_cast<const f32x4*>(dSn + (size_t)cs * DV + x0 + xs + 4 * i);
            }
#pragma unroll
            for (int i = 0; i < XU / 4; ++i)
                rU[i] = *reinterpret_cast<const f32x4*>(Um + (size_t)cu * DV + x0 + xu + 4 * i);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                rdU[i] = *reinterpret_cast<const f32x4*>(dUm + (size_t)ta * DV + x0 + 8 * lg + 4 * i);
            rdO = *reinterpret_cast<const uint4*>(dO + ((t0 + min(ta, n - 1)) * Hs + h) * DV + x0 + 8 * lg);
        };
        auto put2 = [&](bf16_t* hi, bf16_t* lo, int at, f32x4 v) {
            uint2 ph, pl;
            split4(v, ph, pl);
            *reinterpret_cast<uint2*>(hi + at) = ph;
            *reinterpret_cast<uint2*>(lo + at) = pl;
        };
        float gn = 0.f;
        fetch(0);
        for (int x0 = 0; x0 < DV; x0 += XB) {
#pragma unroll
            for (int i = 0; i < XS / 4; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) gn += rS[i][j] * rD[i][j];
                put2(sSh, sSl, cs * SP + xs + 4 * i, rS[i]);
                put2(sDh, sDl, cs * SP + xs + 4 * i, rD[i]);
            }
#pragma unroll
            for (int i = 0; i < XU / 4; ++i) put2(sUh, sUl, cu * SP + xu + 4 * i, rU[i]);
            // the A sides of this block: dU in two parts, dO (zero past the chunk's end)
            Frag<bf16_t> dUh, dUl, dOf;
            {
                uint2 h0, l0, h1, l1;
                split4(rdU[0], h0, l0);
                split4(rdU[1], h1, l1);
                dUh.v = __builtin_bit_cast(u16x8, uint4{h0.x, h0.y, h1.x, h1.y});
                dUl.v = __builtin_bit_cast(u16x8, uint4{l0.x, l0.y, l1.x, l1.y});
                dOf.v = __builtin_bit_cast(u16x8, ta < n ? rdO : uint4{0u, 0u, 0u, 0u});
            }
            lds_barrier();
            if (x0 + XB < DV) fetch(x0 + XB);
            const Frag<bf16_t> uhA = ld_frag(sUh + ta * SP + 8 * lg), ulA = ld_frag(sUl + ta * SP + 8 * lg);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int at = (16 * j + lr) * SP + 8 * lg;
                const Frag<bf16_t> sh = ld_frag(sSh + at), sl = ld_frag(sSl + at);
                const Frag<bf16_t> dh = ld_frag(sDh + at), dl = ld_frag(sDl + at);
                aW.t[j] = mma(dUh, sh, aW.t[j]);
                aQ.t[j] = mma(dOf, sh, aQ.t[j]);
                aK.t[j] = mma(uhA, dh, aK.t[j]);
                aW.t[j] = mma(dUh, sl, aW.t[j]);
                aQ.t[j] = mma(dOf, sl, aQ.t[j]);
                aK.t[j] = mma(uhA, dl, aK.t[j]);
                aW.t[j] = mma(dUl, sh, aW.t[j]);
                aK.t[j] = mma(ulA, dh, aK.t[j]);
            }
#pragma unroll
            for (int j = 0; j < C / 16; ++j) {
                const int at = (16 * j + lr) * SP + 8 * lg;
                aP.t[j] = mma(dOf, ld_frag(sUh + at), aP.t[j]);
                aP.t[j] = mma(dOf, ld_frag(sUl + at), aP.t[j]);
            }
            lds_barrier();
        }
        // the TS threads of a row of S hold partial sums of dGn
#pragma unroll
        for (int o = 1; o < TS; o <<= 1) gn += __shfl_xor(gn, o);
        put(aW, w.dW + oCK, DK, -1.f);
        put(aQ, w.dQG + oCK, DK, 1.f);
        put(aK, w.dKd + oCK, DK, 1.f);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < C / 16; ++b) {
                const int t = Acc<C>::row(a), i = Acc<C>::col(b);
                w.dP[oCC + (size_t)t * C + i] = (i <= t && t < n) ? aP.t[b][a] : 0.f;
            }
        if (tid % TS == 0) w.dGn[oK + cs] = gn;
    }
    }  // PH == 0, bf16

    if constexpr (PH == 0 && !kBf) {
    // phase 1 as one pass over the value index x in tiles of 16: dW = -dU S^T,
    // dQG = dO S^T, dKd = U dS_next^T, dP = tril(dO U^T) and dGn[c] = sum_x
    // S[c][x] dS_next[c][x].  Each operand tile is read from memory once and
    // serves every product that uses it (U is the left operand of dKd and the
    // right one of dP, with the same LDS layout).
    {
        constexpr int KT = 16, SA = C + 4, SB = DK + 4, NT = DK / 16;
        constexpr int RA = C * KT / kBwdThreads, RB = DK * KT / kBwdThreads;
        static_assert(KT * (3 * SA + 2 * SB) <= kLdsFloats, "phase-1 tiles fit");
        float* tdU = lds;
        float* tdO = tdU + KT * SA;
        float* tU = tdO + KT * SA;
        float* tS = tU + KT * SA;
        float* tD = tS + KT * SB;
        const int wv = tid / 64, lg = (tid % 64) / 16, lr = tid % 16;
        Acc<DK> aW, aQ, aK;
        Acc<C> aP;
        aW.zero();
        aQ.zero();
        aK.zero();
        aP.zero();
        float gn = 0.f;
        float rdU[RA], rdO[RA], rU[RA], rS[RB], rD[RB];
        // thread's share of a tile: element idx = tid + r * threads at row idx / KT, x0 + idx % KT
        auto fetch = [&](int x0) {
#pragma unroll
            for (int r = 0; r < RA; ++r) {
                const int idx = tid + r * kBwdThreads, m = idx / KT, x = x0 + idx % KT;
                rdU[r] = dUm[(size_t)m * DV + x];
                rdO[r] = dOat(m, x);
                rU[r] = Um[(size_t)m * DV + x];
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int idx = tid + r * kBwdThreads, c = idx / KT, x = x0 + idx % KT;
                rS[r] = Sm[(size_t)c * DV + x];
                rD[r] = dSn[(size_t)c * DV + x];
            }
        };
        fetch(0);
        for (int x0 = 0; x0 < DV; x0 += KT) {
#pragma unroll
            for (int r = 0; r < RA; ++r) {
                const int idx = tid + r * kBwdThreads, m = idx / KT, kk = idx % KT;
                tdU[kk * SA + m] = rdU[r];
                tdO[kk * SA + m] = rdO[r];
                tU[kk * SA + m] = rU[r];
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int idx = tid + r * kBwdThreads, c = idx / KT, kk = idx % KT;
                tS[kk * SB + c] = rS[r];
                tD[kk * SB + c] = rD[r];
            }
            lds_barrier();
            if (x0 + KT < DV) fetch(x0 + KT);
            if (tid < DK) {
#pragma unroll
                for (int kk = 0; kk < KT; ++kk) gn += tS[kk * SB + tid] * tD[kk * SB + tid];
            }
#pragma unroll
            for (int ks = 0; ks < KT; ks += 4) {
                const int kr = ks + lg;
                const float a_dU = tdU[kr * SA + 16 * wv + lr], a_dO = tdO[kr * SA + 16 * wv + lr],
                            a_U = tU[kr * SA + 16 * wv + lr];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const float bS = tS[kr * SB + 16 * j + lr], bD = tD[kr * SB + 16 * j + lr];
                    aW.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_dU, bS, aW.t[j], 0, 0, 0);
                    aQ.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_dO, bS, aQ.t[j], 0, 0, 0);
                    aK.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_U, bD, aK.t[j], 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < C / 16; ++j) {
                    const float bU = tU[kr * SA + 16 * j + lr];
                    aP.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_dO, bU, aP.t[j], 0, 0, 0);
                }
            }
            lds_barrier();
        }
        put(aW, w.dW + oCK, DK, -1.f);
        put(aQ, w.dQG + oCK, DK, 1.f);
        put(aK, w.dKd + oCK, DK, 1.f);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < C / 16; ++b) {
                const int t = Acc<C>::row(a), i = Acc<C>::col(b);
                w.dP[oCC + (size_t)t * C + i] = (i <= t && t < n) ? aP.t[b][a] : 0.f;
            }
        if (tid < DK) w.dGn[oK + tid] = gn;
    }
    }  // PH == 0

    if constexpr (PH == 1) {
    // dT and Y are used only inside this launch: they stay in LDS
    __shared__ float sdT[C][C + 1];
    __shared__ float sY[C][C + 1];
    __shared__ float sRsu[C];  // row sums of dXu * V (for dbeta)
    // phase 2: dT = strict_tril(dW Xw^T + dU Xu^T), dXw = T^T dW, dXu = T^T dU
    {
        const float* dW = w.dW + oCK;
        const float* KG = w.KG + oCK;
        Acc<C> at;
        at.zero();
        gemm64<C, DK, true, false>(at, [&](int t, int c) { return dW[(size_t)t * DK + c]; },
                                   [&](int c, int i) { return sbeta[i] * KG[(size_t)i * DK + c]; }, lds);
        gemm64<C, DV, true, false>(at, [&](int t, int x) { return dUm[(size_t)t * DV + x]; },
                                   [&](int x, int i) {  // beta_i is zero past the end (no select: see prep)
                                       return sbeta[i] * ld(v, ((t0 + min(i, n - 1)) * Hs + h) * DV + x);
                                   },
                                   lds);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < C / 16; ++b) {
                const int t = Acc<C>::row(a), i = Acc<C>::col(b);
                lds_put(&sdT[t][i], (i < t && t < n) ? at.t[b][a] : 0.f);
            }
        Acc<DK> ax;
        ax.zero();
        gemm64<DK, C, false, true>(ax, [&](int t, int a) { return Tm[(size_t)a * C + t]; },
                                  [&](int a, int c) { return dW[(size_t)a * DK + c]; }, lds);
        put(ax, w.dXw + oCK, DK, 1.f);
        Acc<DV> au;
        au.zero();
        gemm64<DV, C, false, true>(au, [&](int t, int a) { return Tm[(size_t)a * C + t]; },
                                  [&](int a, int x) { return dUm[(size_t)a * DV + x]; }, lds);
        // dXu is used only here: dv = diag(beta) dXu, and the row sums of
        // dXu * V for dbeta (in a fixed order: the lane's columns, then the
        // 16 lanes of its group).  A row's v is loaded before any of its
        // stores, and loads are never under a condition (rows past the end
        // re-read the last row): either would make every load wait in turn.
        E vx[4][DV / 16];  // raw, all loaded before the first store
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < DV / 16; ++b)
                vx[a][b] = v[((t0 + min(Acc<DV>::row(a), n - 1)) * Hs + h) * DV + Acc<DV>::col(b)];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int t = Acc<DV>::row(a);
            const int64_t o0 = ((t0 + min(t, n - 1)) * Hs + h) * DV;
            float rs = 0.f;
#pragma unroll
            for (int b = 0; b < DV / 16; ++b) {
                if (t < n) {
                    dv[o0 + Acc<DV>::col(b)] = Elt<E>::from(sbeta[t] * au.t[b][a]);
                    rs += au.t[b][a] * Elt<E>::to(vx[a][b]);
                }
            }
            rs += __shfl_xor(rs, 1, 64);
            rs += __shfl_xor(rs, 2, 64);
            rs += __shfl_xor(rs, 4, 64);
            rs += __shfl_xor(rs, 8, 64);
            if (tid % 16 == 0) sRsu[t] = rs;
        }
    }
    __syncthreads();

    // phase 3: Y = dT T^T (kept where column < row)
    {
        Acc<C> ay;
        ay.zero();
        gemm64<C, C, true, false>(ay, [&](int a, int b) { return sdT[a][b]; },
                                  [&](int b, int i) { return Tm[(size_t)i * C + b]; }, lds);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < C / 16; ++b) {
                const int r = Acc<C>::row(a), i = Acc<C>::col(b);
                lds_put(&sY[r][i], (i < r && r < n) ? ay.t[b][a] : 0.f);
            }
    }
    __syncthreads();

    // phase 4: dA = strict_tril(-T^T Y)
    {
        Acc<C> aa;
        aa.zero();
        gemm64<C, C, false, true>(aa, [&](int t, int a) { return Tm[(size_t)a * C + t]; },
                                 [&](int a, int i) { return sY[a][i]; }, lds);
        // dA, and the row sums of dA * M plus those of dXu * V: dbeta less
        // its dXw * KG part, which the last launch adds
        float mv[4][C / 16];  // all loaded before the dA stores, which might alias M for the compiler
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < C / 16; ++b) mv[a][b] = w.M[oCC + (size_t)Acc<C>::row(a) * C + Acc<C>::col(b)];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int t = Acc<C>::row(a);
            float rs = 0.f;
#pragma unroll
            for (int b = 0; b < C / 16; ++b) {
                const int i = Acc<C>::col(b);
                const float da = (i < t && t < n) ? -aa.t[b][a] : 0.f;
                w.dA[oCC + (size_t)t * C + i] = da;
                rs += da * mv[a][b];  // M is zero where dA is masked
            }
            rs += __shfl_xor(rs, 1, 64);
            rs += __shfl_xor(rs, 2, 64);
            rs += __shfl_xor(rs, 4, 64);
            rs += __shfl_xor(rs, 8, 64);
            if (tid % 16 == 0 && t < n) w.dBr[(size_t)slot * C + t] = rs + sRsu[t];
        }
    }
    }  // PH == 1

    if constexpr (PH == 2) {
    __shared__ float sTf[(kTfRows - kTfLocalRow0) * DK];  // tile decay factors and references fs, fe, b_m, f1, f2
    // dA and dP of the chunk, read as column blocks and as row blocks by the
    // pass below: loaded once, all at the start
    __shared__ float sdA[C][C + 1], sdP[C][C + 1];
    {
        constexpr int NA = C * C / 4 / kBwdThreads;
        f32x4 ra[NA], rp[NA];
        const f32x4* a4 = reinterpret_cast<const f32x4*>(w.dA + oCC) + tid;
        const f32x4* p4 = reinterpret_cast<const f32x4*>(w.dP + oCC) + tid;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            ra[i] = a4[i * kBwdThreads];
            rp[i] = p4[i * kBwdThreads];
        }
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int e = 4 * (tid + i * kBwdThreads), t = e / C, c = e % C;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sdA[t][c + j] = ra[i][j];
                sdP[t][c + j] = rp[i][j];
            }
        }
    }
    // db = the gate's gradient per row before its reverse prefix sum, [C][DK + 1],
    // in the operand tiles' LDS once the pass over the chunk rows is done
    float* sDb = lds;
    static_assert(C * (DK + 1) <= kLdsFloats, "db fits in the operand tiles");
    // the table needs the prefix sums of twelve rows (the start, middle and
    // end row of each 16-row tile): loaded at once into the operand tiles'
    // LDS, rather than one round trip per table entry
    {
        float* sBr = lds;  // [12][DK]: row 3 a + {0, 1, 2} = s(a), m(a), e(a)
        static_assert(12 * DK % kBwdThreads == 0 && 12 * DK <= kLdsFloats, "table rows");
#pragma unroll
        for (int r = 0; r < 12 * DK / kBwdThreads; ++r) {
            const int idx = tid + r * kBwdThreads, q3 = idx / DK, c = idx % DK;
            const int row = 16 * (q3 / 3) + (q3 % 3 == 0 ? 0 : q3 % 3 == 1 ? 8 : 15);
            sBr[idx] = w.B[oCK + (size_t)row * DK + c];
        }
        __syncthreads();
        fill_tile_factors<E, DK, kTfLocalRow0, kTfRows>(sTf, [&](int row, int c) {
            const int o = row % 16;
            return sBr[(3 * (row / 16) + (o == 0 ? 0 : o == 8 ? 1 : 2)) * DK + c];
        });
    }
    auto tf_row = [&](int row) { return sTf + (row - kTfLocalRow0) * DK; };
    __syncthreads();

    // phase 5: dKr = diag(beta) dA Ki, dKi = (diag(beta) dA)^T Kr + dP^T Qr,
    // dQr = dP Ki; then dq, dk, db (in LDS) and dbeta (dv comes from the
    // middle launch).  Tile by tile: row-side results (dKr, dQr) of row tile
    // a are referred to m(a), column-side ones (dKi) of column tile bb to
    // m(bb), i.e. every result of a row is referred to the middle row of its
    // own tile, like the decayed operands.  Between two tiles the operand is
    // first taken to its own tile's end (fe) or start (fs) and then on to the
    // other tile's middle (f1, f2), factors <= 1 one after another.
    {
        const float* Bm = w.B + oCK;
        // One pass over the chunk-row index in tiles of 16, all three results
        // in registers: dKr and dQr take dA's and dP's column blocks against
        // Ki's rows; dKi takes dA's and dP's row blocks (transposed use)
        // against Kr's and Qr's rows.  Kr, Qr and Ki are formed from q, k
        // and b as their rows are staged (the same values prep multiplied),
        // nothing is parked.
        constexpr int KT = 16, SB = DK + 4, NT = DK / 16;
        constexpr int RB = DK * KT / kBwdThreads;
        static_assert(KT * 3 * SB <= kLdsFloats, "phase-5 tiles fit");
        float* tKi = lds;            // [kk][c] = Ki[k0 + kk][c]
        float* tKr = tKi + KT * SB;
        float* tQr = tKr + KT * SB;
        const int wv = __builtin_amdgcn_readfirstlane(tid / 64), lg = (tid % 64) / 16, lr = tid % 16;
        Acc<DK> aKr, aQr, acc;  // acc: dKi
        aKr.zero();
        aQr.zero();
        acc.zero();
        // q, k and b two adjacent channels at a time: raw values, converted
        // when staged (rows past the end load the last row)
        using E2 = typename std::conditional<std::is_same<E, float>::value, float2, uint32_t>::type;
        constexpr int RB2 = RB / 2, DK2 = DK / 2;
        float2 rb[RB2];
        E2 rq[RB2], rk[RB2];
        auto lo_hi = [](E2 x, float& lo, float& hi) {
            if constexpr (std::is_same<E, float>::value) {
                lo = x.x;
                hi = x.y;
            } else {
                lo = __uint_as_float(x << 16);
                hi = __uint_as_float(x & 0xffff0000u);
            }
        };
        auto fetch = [&](int k0) {
#pragma unroll
            for (int r = 0; r < RB2; ++r) {
                const int idx = tid + r * kBwdThreads;
                const int t = k0 + idx / DK2, c = 2 * (idx % DK2);
                const int64_t o = ((t0 + min(t, n - 1)) * Hs + h) * DK + c;
                rq[r] = *reinterpret_cast<const E2*>(q + o);
                rk[r] = *reinterpret_cast<const E2*>(k + o);
                rb[r] = *reinterpret_cast<const float2*>(Bm + (size_t)t * DK + c);
            }
        };
        fetch(0);
        for (int k0 = 0; k0 < C; k0 += KT) {
            // Kr = k e^{b - r}, Qr = q e^{b - r}, Ki = k e^{r - b}, r the b
            // of the middle row of this row tile
            const float* rmid = tf_row(kTfBm + k0 / KT);
#pragma unroll
            for (int r = 0; r < RB2; ++r) {
                const int idx = tid + r * kBwdThreads;
                const int t = k0 + idx / DK2, c = 2 * (idx % DK2), j = (idx / DK2) * SB + c;
                const float2 rm = *reinterpret_cast<const float2*>(rmid + c);
                float q0, q1, k0v, k1v;
                lo_hi(rq[r], q0, q1);
                lo_hi(rk[r], k0v, k1v);
                if (t >= n) q0 = q1 = k0v = k1v = 0.f;
                const float er0 = capped_exp<E>(rb[r].x - rm.x), eir0 = capped_exp<E>(rm.x - rb[r].x);
                const float er1 = capped_exp<E>(rb[r].y - rm.y), eir1 = capped_exp<E>(rm.y - rb[r].y);
                *reinterpret_cast<float2*>(tKi + j) = float2{k0v * eir0, k1v * eir1};
                *reinterpret_cast<float2*>(tKr + j) = float2{k0v * er0, k1v * er1};
                *reinterpret_cast<float2*>(tQr + j) = float2{q0 * er0, q1 * er1};
            }
            lds_barrier();
            if (k0 + KT < C) fetch(k0 + KT);
            // kt: the tile of the summed token index.  Row side: dA and dP
            // are zero above the diagonal (kt > wv); below it Ki goes to
            // e(kt), then to m(wv).  Column side: nothing for kt < wv; for
            // kt > wv, Kr and Qr go to s(kt), then to m(wv).
            const int kt = k0 / KT;
            const bool below = kt < wv, above = kt > wv;
            // No branch inside the loop (tested there, every column tile had
            // been a branch of its own around a few reads and instructions):
            // both sides' instructions run for every tile pair, and the side
            // that does not apply multiplies exact zeros, since dA and dP are
            // zero above the diagonal (row side, kt > wv) and their
            // transposes below it (column side, kt < wv); its right operand
            // is then left unscaled, finite.
            const float* fu = tf_row(kt < wv ? kTfFe + kt : kTfFs + kt);
            const float* fv = tf_row(kt < wv ? kTfF1 + pair_of(wv, kt) : kTfF2 + pair_of(kt > wv ? kt : 1, kt > wv ? wv : 0));
#pragma unroll
            for (int ks = 0; ks < KT; ks += 4) {
                // dA and dP as column blocks (row 16 wv + lr, column k0 + kr)
                // and as row blocks (row k0 + kr, column 16 wv + lr); P's
                // diagonal enters dq and dk in the epilogue instead
                const int kr = ks + lg, m = 16 * wv + lr, kc = k0 + kr;
                const float a_Ac = sdA[m][kc], a_Pc = m == kc ? 0.f : sdP[m][kc];
                const float a_Ar = sbeta[kc] * sdA[kc][m], a_Pr = kc == m ? 0.f : sdP[kc][m];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int br = kr * SB + 16 * j + lr;
                    const float bKi = tKi[br], bKr = tKr[br], bQr = tQr[br];
                    const float u = fu[16 * j + lr], x = fv[16 * j + lr];
                    const float sKi = below ? (bKi * u) * x : bKi;
                    const float sKr = above ? (bKr * u) * x : bKr, sQr = above ? (bQr * u) * x : bQr;
                    aKr.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_Ac, sKi, aKr.t[j], 0, 0, 0);
                    aQr.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_Pc, sKi, aQr.t[j], 0, 0, 0);
                    acc.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_Ar, sKr, acc.t[j], 0, 0, 0);
                    acc.t[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_Pr, sQr, acc.t[j], 0, 0, 0);
                }
            }
            lds_barrier();
        }
        // dKr, dQr and dKi share the accumulator layout: same (t, c) positions.
        // The same pass forms the row sums of dXw * KG (for dbeta) and the
        // column sums of dKd * Kd (for the last row of the gate's prefix sum),
        // with KG = k e^b and Kd = k e^{b_last - b} from factors at hand.
        // Two pairs of terms cancel exactly in the gate's gradient and are
        // left out of it, so that their rounding does not swamp a gradient
        // that strong decay makes small: P's diagonal (P_tt = q_t . k_t
        // carries no decay; it was left out of the products above and enters
        // dq and dk here directly), and the last row's own Kd term against
        // its share of the last-row column sum (Kd = k there).
        float rowp[4] = {0.f, 0.f, 0.f, 0.f};
        float colp[DK / 16];
#pragma unroll
        for (int b = 0; b < DK / 16; ++b) colp[b] = 0.f;
        // Row by row (eight elements per lane): every load of a row is issued
        // before its first store, since a load is not moved above a store
        // that might alias it and each would otherwise wait in turn; no load
        // is under a condition (a load under a condition is waited for where
        // it is issued); the row's dq and dk are stored together after all
        // its elements are computed (a store under a condition between two
        // elements made the next element wait for it).  Rows past the
        // chunk's end are computed from what the workspace holds there (q
        // and k re-read the last row) and are neither stored nor summed.
        constexpr int NB = DK / 16;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int t = Acc<DK>::row(a);
            const bool live = t < n;
            const size_t j0 = oCK + (size_t)t * DK;
            const int64_t o0 = ((t0 + min(t, n - 1)) * Hs + h) * DK;
            float xw[NB], xq[NB], xd[NB], xb[NB];
            E rk[NB], rq[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int c = Acc<DK>::col(b);
                xw[b] = w.dXw[j0 + c];
                xq[b] = w.dQG[j0 + c];
                xd[b] = w.dKd[j0 + c];
                xb[b] = w.B[j0 + c];
                rk[b] = k[o0 + c];
                rq[b] = q[o0 + c];
            }
            const float dPd = sdP[t][t];
            const float bt = sbeta[t];
            float oq[NB], ok[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int c = Acc<DK>::col(b);
                const float dKr = bt * aKr.t[b][a], dKi = acc.t[b][a], dQr = aQr.t[b][a];
                const float dXw = xw[b];
                const float dKG = bt * dXw;
                const float dQG = xq[b], dKd = xd[b];
                const float bb = xb[b], r = tf_row(kTfBm + wv)[c], bl = sbl[c];
                const float e = gate_exp<E>(bb), er = capped_exp<E>(bb - r), eir = capped_exp<E>(r - bb),
                            ed = gate_exp<E>(bl - bb);
                // the decayed operands are q or k times these factors, so the
                // gate's gradient needs q and k themselves, not the six arrays
                const float gq = dQG * e + dQr * er;    // dq without P's diagonal
                const float gk_up = dKG * e + dKr * er;  // factors that grow with b
                const float gk_dd = dKi * eir, gk_kd = t == n - 1 ? 0.f : dKd * ed;
                const float kv = Elt<E>::to(rk[b]), qv = Elt<E>::to(rq[b]);
                oq[b] = gq + dPd * kv;
                ok[b] = gk_up + gk_dd + dKd * ed + dPd * qv;
                lds_put(&sDb[t * (DK + 1) + c], qv * gq + kv * (gk_up - (gk_dd + gk_kd)));
                rowp[a] += live ? dXw * kv * e : 0.f;
                colp[b] += live ? gk_kd * kv : 0.f;
            }
            if (live) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    dq[o0 + Acc<DK>::col(b)] = Elt<E>::from(oq[b]);
                    dk[o0 + Acc<DK>::col(b)] = Elt<E>::from(ok[b]);
                }
            }
        }
        // rows: the 16 lanes of a lane group; columns: the four lane groups of a
        // wave, then the four waves in a fixed order (no atomics: deterministic)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            float x = rowp[a];
            x += __shfl_xor(x, 1, 64);
            x += __shfl_xor(x, 2, 64);
            x += __shfl_xor(x, 4, 64);
            x += __shfl_xor(x, 8, 64);
            if ((tid & 15) == 0) sRowKG[Acc<DK>::row(a)] = x;
        }
#pragma unroll
        for (int b = 0; b < DK / 16; ++b) {
            float x = colp[b];
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            if ((tid & 63) < 16) sColKd[(tid / 64) * DK + Acc<DK>::col(b)] = x;
        }
    }
    __syncthreads();
    // dbeta: the middle launch's row sums of dA * M and dXu * V, plus those of
    // dXw * KG
    for (int t = tid; t < n; t += kBwdThreads)
        dbeta[(t0 + t) * Hs + h] = Elt<E>::from(w.dBr[(size_t)slot * C + t] + sRowKG[t]);

    // phase 6: dg = reverse cumulative sum of db (in LDS); the last row's
    // prefix sum also carries e^{b_last} (Gn) and the e^{b_last} factor of Kd
    for (int c = tid; c < DK; c += kBwdThreads) {
        float acc = w.dGn[oK + c] * w.Gn[oK + c] + ((sColKd[c] + sColKd[DK + c]) + (sColKd[2 * DK + c] + sColKd[3 * DK + c]));
#pragma unroll 8
        for (int t = n - 1; t >= 0; --t) {
            acc += sDb[t * (DK + 1) + c];
            if (HG)
                sDb[t * (DK + 1) + c] = acc;
            else
                dg[((t0 + t) * Hs + h) * DK + c] = Elt<E>::from(acc);
        }
    }
    if (HG) {
        __syncthreads();
        for (int t = tid; t < n; t += kBwdThreads) {
            float s = 0.f;
#pragma unroll 8
            for (int c = 0; c < DK; ++c) s += sDb[t * (DK + 1) + c];
            dg[(t0 + t) * Hs + h] = Elt<E>::from(s);
        }
    }
    }  // PH == 2
}

// ---------------------------------------------------------------------------
// Host side.
inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdSizes {
    size_t head, ck, ckw, ckb, cv, cc, ccw, c, k, kv, total;
};

// The walks' operands (QG, Kd, W: C x DK; P: C x C) are kept in the input
// type (bf16 for bf16 inputs), every other array in fp32; bf16 inputs keep W
// and Kd twice (Wr, KdT: one layout per walk).
BwdSizes bwd_sizes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16) {
    const size_t slots = (size_t)max_chunks_for(T, N) * H;
    const size_t ew = bf16 ? 2 : 4;
    BwdSizes s;
    s.head = 256 + 2 * al256((size_t)(N + 1) * 4) + al256((size_t)max_chunks_for(T, N) * sizeof(int2));
    s.ck = al256(slots * C * dk * 4);
    s.ckw = al256(slots * C * dk * ew);
    s.ckb = bf16 ? s.ckw : 0;
    s.cv = al256(slots * C * dv * 4);
    s.cc = al256(slots * C * C * 4);
    s.ccw = al256(slots * C * C * ew);
    s.c = al256(slots * C * 4);
    s.k = al256(slots * dk * 4);
    s.kv = al256(slots * dk * dv * 4);
    s.total = s.head + 6 * s.ck + 3 * s.ckw + 2 * s.ckb + 3 * s.cv + 4 * s.cc + s.ccw + s.c + 2 * s.k + 2 * s.kv;
    return s;
}

BwdWs carve_bwd(void* base, int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16) {
    const BwdSizes s = bwd_sizes(T, N, H, dk, dv, bf16);
    char* p = static_cast<char*>(base);
    BwdWs w;
    w.header = reinterpret_cast<WsHeader*>(p); p += 256;
    w.cu = reinterpret_cast<int32_t*>(p); p += al256((size_t)(N + 1) * 4);
    w.chunk_off = reinterpret_cast<int32_t*>(p); p += al256((size_t)(N + 1) * 4);
    w.chunk_tab = reinterpret_cast<int2*>(p); p += al256((size_t)max_chunks_for(T, N) * sizeof(int2));
    auto take = [&](size_t bytes) { float* f = reinterpret_cast<float*>(p); p += bytes; return f; };
    float** ck[] = {&w.B, &w.KG, &w.dW, &w.dQG, &w.dKd, &w.dXw};
    for (float** f : ck) *f = take(s.ck);
    float** ckw[] = {&w.QG, &w.Kd, &w.W};
    for (float** f : ckw) *f = take(s.ckw);
    float** ckb[] = {&w.Wr, &w.KdT};
    for (float** f : ckb) *f = s.ckb ? take(s.ckb) : nullptr;
    float** cv[] = {&w.Up, &w.U, &w.dU};
    for (float** f : cv) *f = take(s.cv);
    float** cc[] = {&w.M, &w.T, &w.dP, &w.dA};
    for (float** f : cc) *f = take(s.cc);
    w.P = take(s.ccw);
    w.dBr = take(s.c);
    w.Gn = take(s.k);
    w.dGn = take(s.k);
    w.S = take(s.kv);
    w.dSn = take(s.kv);
    return w;
}

// Allow a kernel more than the default 64 KB of dynamic LDS.
hipError_t lds_attr(const void* kern, size_t bytes) {
    return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// One head group: a.H heads starting at the pointers given (already offset),
// token and state tensors with a row stride of Hs heads.
template <typename E, int DK, int DV, bool HG>
hipError_t launch_bwd_t(const BwdArgs& a, int32_t Hs, const BwdWs& w, hipStream_t stream) {
    const unsigned slots = (unsigned)(a.max_chunks * a.H);
    const unsigned walks = (unsigned)((int64_t)a.N * a.H * (DV / 16));
    hipError_t e = hipSuccess;
    if (a.T > 0) {
        hipLaunchKernelGGL((bwd_prep_kernel<E, DK, DV, HG>), dim3(slots), dim3(kBwdThreads), 0, stream,
                           (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.g, (const E*)a.beta, a.H, Hs,
                           w);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if constexpr (std::is_same<E, bf16_t>::value) {
            hipLaunchKernelGGL((bwd_state_walk_bf16_kernel<DK, DV>), dim3(walks), dim3(kBwdThreads), 0, stream, a.H,
                               Hs, a.S0, w);
        } else {
            auto sw = bwd_state_walk_kernel<E, DK, DV>;
            constexpr size_t sw_lds = StateWalkLds<DK, DV>::bytes;
            if ((e = lds_attr(reinterpret_cast<const void*>(sw), sw_lds)) != hipSuccess) return e;
            hipLaunchKernelGGL(sw, dim3(walks), dim3(kBwdThreads), sw_lds, stream, a.H, Hs, a.S0, w);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (std::is_same<E, bf16_t>::value) {
        hipLaunchKernelGGL((bwd_dstate_walk_bf16_kernel<DK, DV>), dim3(walks), dim3(kBwdThreads), 0, stream, a.H, Hs,
                           (const bf16_t*)a.dO, a.dS_T, a.dS0, w);
    } else {
        auto dw = bwd_dstate_walk_kernel<E, DK, DV>;
        constexpr size_t dw_lds = DStateWalkLds<DK, DV>::bytes;
        if ((e = lds_attr(reinterpret_cast<const void*>(dw), dw_lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(dw, dim3(walks), dim3(kBwdThreads), dw_lds, stream, a.H, Hs, (const E*)a.dO, a.dS_T,
                           a.dS0, w);
    }
    e = hipGetLastError();
    if (e != hipSuccess || a.T == 0) return e;
    hipLaunchKernelGGL((bwd_local_kernel<E, DK, DV, HG, 0>), dim3(slots), dim3(kBwdThreads), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const E*)a.dO, a.H, Hs, w,
                       (E*)a.dq, (E*)a.dk, (E*)a.dv,
                       (E*)a.dg, (E*)a.dbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_local_kernel<E, DK, DV, HG, 1>), dim3(slots), dim3(kBwdThreads), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const E*)a.dO, a.H, Hs, w,
                       (E*)a.dq, (E*)a.dk, (E*)a.dv,
                       (E*)a.dg, (E*)a.dbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_local_kernel<E, DK, DV, HG, 2>), dim3(slots), dim3(kBwdThreads), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const E*)a.dO, a.H, Hs, w,
                       (E*)a.dq, (E*)a.dk, (E*)a.dv,
                       (E*)a.dg, (E*)a.dbeta);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_bwd_g(const BwdArgs& a, int32_t Hs, const BwdWs& w, hipStream_t s) {
    return a.head_gate ? launch_bwd_t<E, DK, DV, true>(a, Hs, w, s) : launch_bwd_t<E, DK, DV, false>(a, Hs, w, s);
}

template <typename E>
hipError_t launch_bwd_e(const BwdArgs& a, int32_t Hs, const BwdWs& w, hipStream_t s) {
    if (a.dk_ == 64 && a.dv_ == 64) return launch_bwd_g<E, 64, 64>(a, Hs, w, s);
    if (a.dk_ == 64 && a.dv_ == 128) return launch_bwd_g<E, 64, 128>(a, Hs, w, s);
    if (a.dk_ == 128 && a.dv_ == 64) return launch_bwd_g<E, 128, 64>(a, Hs, w, s);
    return launch_bwd_g<E, 128, 128>(a, Hs, w, s);
}

// p advanced by `elems` elements of `esz` bytes (null stays null)
template <typename P>
P* at(P* p, size_t elems, size_t esz) {
    using B = typename std::conditional<std::is_const<P>::value, const char, char>::type;
    return p ? reinterpret_cast<P*>(reinterpret_cast<B*>(p) + elems * esz) : nullptr;
}

}  // namespace

size_t bwd_workspace_bytes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16) {
    return bwd_sizes(T, N, H, dk, dv, bf16).total;
}

int32_t bwd_head_group(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16, size_t workspace_bytes) {
    int32_t g = H;
    while (g > 0 && bwd_sizes(T, N, g, dk, dv, bf16).total > workspace_bytes) --g;
    return g;
}

hipError_t launch_chunk_bwd(const BwdArgs& a, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    // heads are independent: process them in the largest groups whose
    // intermediates fit the workspace, one group after another on the stream
    const int32_t G = bwd_head_group(a.T, a.N, a.H, a.dk_, a.dv_, a.bf16, workspace_bytes);
    const BwdWs w = carve_bwd(workspace, a.T, a.N, G, a.dk_, a.dv_, a.bf16);
    hipError_t e = launch_chunk_map(a.cu_seqlens, a.N, a.T, w.header, w.cu, w.chunk_off, w.chunk_tab, nullptr, 0,
                                    stream);
    if (e != hipSuccess) return e;
    const size_t esz = a.bf16 ? 2 : 4;
    for (int32_t h0 = 0; h0 < a.H; h0 += G) {
        BwdArgs b = a;
        b.H = a.H - h0 < G ? a.H - h0 : G;
        const size_t hk = (size_t)h0 * a.dk_, hv = (size_t)h0 * a.dv_, hs = (size_t)h0 * a.dk_ * a.dv_;
        const size_t hgk = a.head_gate ? (size_t)h0 : hk;
        b.q = at(a.q, hk, esz); b.k = at(a.k, hk, esz); b.v = at(a.v, hv, esz); b.g = at(a.g, hgk, esz);
        b.beta = at(a.beta, h0, esz); b.dO = at(a.dO, hv, esz);
        b.dq = at(a.dq, hk, esz); b.dk = at(a.dk, hk, esz); b.dv = at(a.dv, hv, esz); b.dg = at(a.dg, hgk, esz);
        b.dbeta = at(a.dbeta, h0, esz);
        b.S0 = at(a.S0, hs, 4); b.dS_T = at(a.dS_T, hs, 4); b.dS0 = at(a.dS0, hs, 4);
        e = a.bf16 ? launch_bwd_e<bf16_t>(b, a.H, w, stream) : launch_bwd_e<float>(b, a.H, w, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
