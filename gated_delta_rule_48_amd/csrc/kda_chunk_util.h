// Device helpers shared by the chunked-forward kernels (chunks of 64 and
// of 128 tokens): element pairs, lane-group sums, tile stores, the
// fragment-major operand layout, LDS hand-over and LDS-DMA primitives.
#pragma once

#include <atomic>

#include "kda_internal.h"

namespace kda {

constexpr int kIntraThreads = 512;  // eight waves per (chunk, head)
constexpr int kLdsBytes = 160 * 1024;  // LDS of one gfx950 compute unit

// Two adjacent elements as one register-sized value (raw, not yet widened).
template <typename E> struct Pair2;
template <> struct Pair2<bf16_t> {
    uint32_t w;
    __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const uint32_t*>(p); }
    __device__ __forceinline__ float lo() const { return __uint_as_float(w << 16); }
    __device__ __forceinline__ float hi() const { return __uint_as_float(w & 0xffff0000u); }
    __device__ __forceinline__ void set(float a, float b) { w = f32x2_to_bf16x2(a, b); }  // rounded
};
template <> struct Pair2<float> {
    float2 w;
    __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const float2*>(p); }
    __device__ __forceinline__ float lo() const { return w.x; }
    __device__ __forceinline__ float hi() const { return w.y; }
    __device__ __forceinline__ void set(float a, float b) { w = make_float2(a, b); }
};

// Sum of x over aligned groups of LANES (32 or 64) lanes, in every lane of
// the group, in one fixed order: within each 16-lane row by DPP (swap
// neighbours, swap pairs, mirror halves, mirror the row), then the four row
// sums read as scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int LANES>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(LANES == 32 || LANES == 64, "half or whole wave");
    x += dpp_f32<0xb1>(x);   // quad_perm(1, 0, 3, 2)
    x += dpp_f32<0x4e>(x);   // quad_perm(2, 3, 0, 1)
    x += dpp_f32<0x141>(x);  // row_half_mirror
    x += dpp_f32<0x140>(x);  // row_mirror
    auto row = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l)); };
    const float r0 = row(0), r1 = row(16), r2 = row(32), r3 = row(48);
    if constexpr (LANES == 64) return (r0 + r1) + (r2 + r3);
    else return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
}

// 1 / sqrt(x), 0 for x = 0: exact division of the rounded square root for
// fp32 inputs, the hardware reciprocal square root (about one ulp) for bf16.
template <typename E> __device__ __forceinline__ float inv_norm(float x);
template <> __device__ __forceinline__ float inv_norm<float>(float x) { return x > 0.f ? 1.f / sqrtf(x) : 0.f; }
template <> __device__ __forceinline__ float inv_norm<bf16_t>(float x) {
    return x > 0.f ? __builtin_amdgcn_rsqf(x) : 0.f;
}

template <typename E> __device__ __forceinline__ void load2(const E* p, float& a, float& b);
template <> __device__ __forceinline__ void load2<bf16_t>(const bf16_t* p, float& a, float& b) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xffff0000u);
}
template <> __device__ __forceinline__ void load2<float>(const float* p, float& a, float& b) {
    const float2 w = *reinterpret_cast<const float2*>(p);
    a = w.x;
    b = w.y;
}
template <typename E> __device__ __forceinline__ void store2(E* p, float a, float b);
template <> __device__ __forceinline__ void store2<bf16_t>(bf16_t* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = f32x2_to_bf16x2(a, b);
}
template <> __device__ __forceinline__ void store2<float>(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

// Store N contiguous elements held in registers with 16-byte stores
// (dst 16-byte aligned, N * sizeof(E) a multiple of 16).
template <typename E, int N>
__device__ __forceinline__ void store_run(E* dst, const E (&vals)[N]) {
    constexpr int PER = 16 / (int)sizeof(E);
    static_assert(N % PER == 0, "run length");
#pragma unroll
    for (int i = 0; i < N / PER; ++i) {
        uint4 w;
        __builtin_memcpy(&w, &vals[i * PER], 16);
        *reinterpret_cast<uint4*>(dst + i * PER) = w;
    }
}

// Store 4 contiguous elements (8 bytes for bf16, 16 for fp32).
template <typename E> __device__ __forceinline__ void store_run4(E* dst, const E* vals);
template <> __device__ __forceinline__ void store_run4<bf16_t>(bf16_t* dst, const bf16_t* v) {
    *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                                                (uint32_t)v[2] | ((uint32_t)v[3] << 16));
}
template <> __device__ __forceinline__ void store_run4<float>(float* dst, const float* v) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
}

// Store N contiguous elements (N a multiple of 4; dst aligned to the store
// width): 16-byte stores where the run allows, else 4-element stores.
template <typename E, int N>
__device__ __forceinline__ void store_seq(E* dst, const E (&vals)[N]) {
    if constexpr (N * sizeof(E) % 16 == 0) {
        store_run<E, N>(dst, vals);
    } else {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) store_run4<E>(dst + 4 * i, vals + 4 * i);
    }
}

// Copy a ROWS x COLS tile from LDS (row stride lds_ld elements) to a dense
// global tile with 16-byte loads and stores spread over the workgroup.
template <typename E, int ROWS, int COLS, int NT = kIntraThreads>
__device__ __forceinline__ void copy_tile_out(E* __restrict__ dst, const E* src, int lds_ld, int tid) {
    constexpr int VPR = COLS * (int)sizeof(E) / 16;
    constexpr int PER = 16 / (int)sizeof(E);
#pragma unroll
    for (int i = tid; i < ROWS * VPR; i += NT) {
        const int r = i / VPR, c = (i % VPR) * PER;
        *reinterpret_cast<uint4*>(dst + r * COLS + c) = *reinterpret_cast<const uint4*>(src + r * lds_ld + c);
    }
}

// Position at which index x of a reduction dimension is stored so that the
// chunk walk can feed accumulator registers straight back into the matrix
// cores.  Within each block of 32, x = 16h + 4a + b is stored at 8a + 4h + b:
// an A fragment read as 8 contiguous elements at 8g then holds indices
// {4g..4g+3, 16+4g..16+4g+3}, which are exactly the rows a lane holds in the
// accumulators of the two 16-row tiles of that block.
__device__ __forceinline__ int frag_pos(int x) {
    return (x & ~31) | ((x & 12) << 1) | ((x & 16) >> 2) | (x & 3);
}

// Fragment-major storage of an R x K operand whose K index is already in
// fragment order: each 16 x 32 block is stored as 64 lanes x 8 contiguous
// elements, lane = (row % 16) + 16 * ((col % 32) / 8), so that one fragment
// load of a wave reads 1 KB (bf16) of contiguous memory.
template <int K>
__device__ __forceinline__ int64_t fm_off(int row, int colpos) {
    const int lane = (row & 15) | (((colpos >> 3) & 3) << 4);
    return ((int64_t)((row >> 4) * (K / 32) + (colpos >> 5)) * 64 + lane) * 8 + (colpos & 7);
}

// The 16 x 32 fragment blocks of the C x C matrix P (rows: query tokens of
// 16-row tile t; columns: key tokens of 32-block kb) that lie wholly above the
// diagonal.  P is lower triangular, so they are zero: the intra-chunk kernel
// does not store them and the walk neither loads nor multiplies them.
__host__ __device__ constexpr bool p_block_zero(int t, int kb) { return 16 * t + 15 < 32 * kb; }

// Copy an R x K tile held row-major in LDS (K already in fragment order) to
// fragment-major global memory: thread i writes the i-th 16-byte piece.  With
// LOWER the blocks p_block_zero names are skipped (R = K = C only).  A wave
// writes whole cache lines here, so the stores are non-temporal: the tile is
// read back only by the next kernel (measured: both kernels ~1.5 % faster).
template <typename E, int R, int K, bool LOWER = false, int NT = kIntraThreads>
__device__ __forceinline__ void copy_tile_out_frag(E* __restrict__ dst, const E* src, int lds_ld, int tid) {
    constexpr int PER = 16 / (int)sizeof(E);  // elements per 16-byte piece
    constexpr int PIECES = R * K / PER;
#pragma unroll
    for (int i = tid; i < PIECES; i += NT) {
        // piece i covers lane-part (i % (8 / PER)) of lane (i / (8 / PER)) % 64 of block i / (64 * 8 / PER)
        const int sub = i % (8 / PER);
        const int lane = (i / (8 / PER)) % 64;
        const int blk = i / (64 * 8 / PER);
        if (LOWER && p_block_zero(blk / (K / 32), blk % (K / 32))) continue;
        const int row = 16 * (blk / (K / 32)) + (lane & 15);
        const int col = 32 * (blk % (K / 32)) + 8 * (lane >> 4) + sub * PER;
        typedef unsigned int nu4 __attribute__((ext_vector_type(4)));
        const uint4 v = *reinterpret_cast<const uint4*>(src + row * lds_ld + col);
        __builtin_nontemporal_store(nu4{v.x, v.y, v.z, v.w}, reinterpret_cast<nu4*>(dst + (int64_t)i * PER));
    }
}

// f[j] <- (f[j] * s[j]) * t[j], j = 0..7, the two products in this order.
__device__ __forceinline__ Frag<bf16_t> scale_frag(Frag<bf16_t> f, const float* s, const float* t) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(s), b = *reinterpret_cast<const f32x4*>(s + 4);
    const f32x4 c = *reinterpret_cast<const f32x4*>(t), d = *reinterpret_cast<const f32x4*>(t + 4);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {f32x2_to_bf16x2(bf16_to_f32(f.v[0]) * a[0] * c[0], bf16_to_f32(f.v[1]) * a[1] * c[1]),
                     f32x2_to_bf16x2(bf16_to_f32(f.v[2]) * a[2] * c[2], bf16_to_f32(f.v[3]) * a[3] * c[3]),
                     f32x2_to_bf16x2(bf16_to_f32(f.v[4]) * b[0] * d[0], bf16_to_f32(f.v[5]) * b[1] * d[1]),
                     f32x2_to_bf16x2(bf16_to_f32(f.v[6]) * b[2] * d[2], bf16_to_f32(f.v[7]) * b[3] * d[3])};
    f.v = __builtin_bit_cast(u16x8, w);
    return f;
}
__device__ __forceinline__ Frag<float> scale_frag(Frag<float> f, const float* s, const float* t) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(s), b = *reinterpret_cast<const f32x4*>(s + 4);
    const f32x4 c = *reinterpret_cast<const f32x4*>(t), d = *reinterpret_cast<const f32x4*>(t + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f.v[j] = f.v[j] * a[j] * c[j];
        f.v[j + 4] = f.v[j + 4] * b[j] * d[j];
    }
    return f;
}

// f[j] <- f[j] * s[j], j = 0..7 (s: 8 contiguous fp32 in LDS).
__device__ __forceinline__ Frag<bf16_t> scale_frag(Frag<bf16_t> f, const float* s) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(s);
    const f32x4 b = *reinterpret_cast<const f32x4*>(s + 4);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {f32x2_to_bf16x2(bf16_to_f32(f.v[0]) * a[0], bf16_to_f32(f.v[1]) * a[1]),
                     f32x2_to_bf16x2(bf16_to_f32(f.v[2]) * a[2], bf16_to_f32(f.v[3]) * a[3]),
                     f32x2_to_bf16x2(bf16_to_f32(f.v[4]) * b[0], bf16_to_f32(f.v[5]) * b[1]),
                     f32x2_to_bf16x2(bf16_to_f32(f.v[6]) * b[2], bf16_to_f32(f.v[7]) * b[3])};
    f.v = __builtin_bit_cast(u16x8, w);
    return f;
}
__device__ __forceinline__ Frag<float> scale_frag(Frag<float> f, const float* s) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(s);
    const f32x4 b = *reinterpret_cast<const f32x4*>(s + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f.v[j] *= a[j];
        f.v[j + 4] *= b[j];
    }
    return f;
}

__device__ __forceinline__ int lds_read_int(const int* p) {
    return *(volatile const __attribute__((address_space(3))) int*)(p);
}

// Hand-over between waves of one workgroup through LDS.  The LDS performs the
// accesses of a wave in the order it issues them, so a counter written after
// a wave's data accesses is seen after them by every other wave.  Release
// additionally waits until this wave's LDS accesses are done (lgkmcnt only:
// the compiler's own fences would also wait for outstanding global loads,
// which the walk keeps in flight on purpose); acquire only keeps the compiler
// from hoisting later LDS reads above the counter read.
// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ void lds_release() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_acquire() { asm volatile("" ::: "memory"); }

// Accumulator tiles a (rows 0..15 of a 32-block) and b (rows 16..31) of one
// lane -> the B fragment of that 32-block (see frag_pos).
__device__ __forceinline__ Frag<bf16_t> acc_to_frag(bf16_t, f32x4 a, f32x4 b) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {f32x2_to_bf16x2(a[0], a[1]), f32x2_to_bf16x2(a[2], a[3]), f32x2_to_bf16x2(b[0], b[1]),
                     f32x2_to_bf16x2(b[2], b[3])};
    Frag<bf16_t> f;
    f.v = __builtin_bit_cast(u16x8, w);
    return f;
}
__device__ __forceinline__ Frag<float> acc_to_frag(float, f32x4 a, f32x4 b) {
    Frag<float> f;
    f.v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

// Four consecutive elements in their stored form (8 bytes of bf16 or 16 bytes
// of fp32), widened to fp32 only where they are used.
template <typename E> struct Raw4;
template <> struct Raw4<bf16_t> {
    typedef uint2 T;
    __device__ __forceinline__ static T load(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ static f32x4 widen(T w) {
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xffff0000u)};
    }
};
template <> struct Raw4<float> {
    typedef f32x4 T;
    __device__ __forceinline__ static T load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ static f32x4 widen(T w) { return w; }
};

// One 16-byte LDS-DMA load per active lane: lane i copies 16 bytes from its
// own global address to lds + 16 i (lds must be uniform over the wave).
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are outstanding (they
// complete in order).  Also a compiler barrier for memory accesses.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Index of the nonzero fragment block (t, kb) of P among those kept, in
// row-tile order: row tile t keeps blocks kb = 0..t/2, so the tiles before
// 2a keep a (a + 1) blocks and those before 2a + 1 keep (a + 1)^2 (six blocks
// for 64-token chunks, twenty for 128-token chunks).
__host__ __device__ constexpr int p_block_index(int t, int kb) {
    return ((t & 1) ? (t / 2 + 1) * (t / 2 + 1) : (t / 2) * (t / 2 + 1)) + kb;
}

// x split into a bf16 part and the bf16 of the remainder: hi + lo carries
// about 16 significant bits.
__device__ __forceinline__ void split_frag(f32x4 a, f32x4 b, Frag<bf16_t>& hi, Frag<bf16_t>& lo) {
    hi = acc_to_frag(bf16_t{}, a, b);
    const u16x8 hv = hi.v;
    f32x4 ra, rb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = a[i] - bf16_to_f32(hv[i]);
        rb[i] = b[i] - bf16_to_f32(hv[4 + i]);
    }
    lo = acc_to_frag(bf16_t{}, ra, rb);
}

// Allow a kernel more than the default dynamic LDS, once per (kernel, device):
// `done` holds one bit per device, set once the call has succeeded there.
// Setting the attribute twice (two threads racing on a first call) is
// harmless.
static inline hipError_t ensure_lds_attr(const void* kern, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

}  // namespace kda
