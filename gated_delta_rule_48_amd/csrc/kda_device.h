// Internal device helpers for the KDA kernels (gfx950 / CDNA4).
//
// Element types: bf16 is carried as raw uint16_t bit patterns (widened to fp32
// by a shift, narrowed with round-to-nearest-even); fp32 is plain float.
//
// Matrix-core fragments.  Every product in the chunked path is built from
// 16x16 output tiles with a K-block of 32.  One K-block is one
// v_mfma_f32_16x16x32_bf16 for bf16 operands, or eight
// v_mfma_f32_16x16x4_f32 for fp32 operands.  Both use the same per-lane view,
// with lane = 16*g + r (r = lane % 16, g = lane / 16):
//   A fragment : A[r][8g + j],  j = 0..7   (row r of a 16 x 32 A block)
//   B fragment : B[8g + j][r],  j = 0..7   (column r of a 32 x 16 B block)
//   accumulator: C[4g + i][r],  i = 0..3
// For fp32 the j-th single MFMA consumes element j of every lane, i.e. the
// k-index 8g + j is fed to the 4-wide instruction's k-slot g; the sum over k
// is the same.  A B fragment is therefore read exactly like an A fragment
// from the TRANSPOSED matrix (8 contiguous elements of row r), which is how
// every operand is laid out in LDS and in the workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

typedef uint16_t bf16_t;  // raw bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
// Two values at once, packed low | high << 16.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), b2));
}

template <typename E> struct Elt;
template <> struct Elt<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static bf16_t from(float f) { return f32_to_bf16(f); }
    __device__ __forceinline__ static float to(bf16_t h) { return bf16_to_f32(h); }
};
template <> struct Elt<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static float from(float f) { return f; }
    __device__ __forceinline__ static float to(float f) { return f; }
};

// One operand fragment: 8 elements per lane.
template <typename E> struct Frag;
template <> struct Frag<bf16_t> { u16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ f32x4 mma(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                   __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
}

// Read 8 contiguous elements (one fragment) from p (16-byte aligned for bf16,
// 32-byte for fp32).
__device__ __forceinline__ Frag<bf16_t> ld_frag(const bf16_t* p) {
    Frag<bf16_t> f;
    f.v = *reinterpret_cast<const u16x8*>(p);
    return f;
}
__device__ __forceinline__ Frag<float> ld_frag(const float* p) {
    Frag<float> f;
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 a = q[0], b = q[1];
    f.v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}
// Read 8 contiguous fp32 values and narrow them to an E fragment.
template <typename E> __device__ __forceinline__ Frag<E> ld_frag_from_f32(const float* p);
template <> __device__ __forceinline__ Frag<float> ld_frag_from_f32<float>(const float* p) { return ld_frag(p); }
template <> __device__ __forceinline__ Frag<bf16_t> ld_frag_from_f32<bf16_t>(const float* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 a = q[0], b = q[1];
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {f32x2_to_bf16x2(a[0], a[1]), f32x2_to_bf16x2(a[2], a[3]), f32x2_to_bf16x2(b[0], b[1]),
                     f32x2_to_bf16x2(b[2], b[3])};
    Frag<bf16_t> f;
    f.v = __builtin_bit_cast(u16x8, w);
    return f;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Scalar LDS store that the backend keeps as a single ds_write.  Used for
// every store of matrix-core accumulator values into LDS: the gfx950 backend
// of ROCm 7.2 can give a wrong offset to a ds_write2 pair it forms from such
// values (seen with conditionally accumulated tiles), silently misplacing one
// element.  A volatile access is never paired.
// The pointer is cast to the LDS address space so that the volatile access
// stays a plain ds_write (a generic volatile store becomes a flat store with
// a full memory wait).
template <typename T>
__device__ __forceinline__ void lds_put(T* p, T v) {
    *(volatile __attribute__((address_space(3))) T*)(p) = v;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also releases
// global memory, which on gfx9 means waiting for every outstanding global
// load (one counter covers loads and stores) and so would drain any loads
// issued ahead of their use.  Kernels whose waves communicate only through
// LDS use this instead.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// exp(x) for the gate factors.  bf16 inputs use the hardware exp2 path; fp32
// inputs use the correctly-rounded-ish library expf.
template <typename E> __device__ __forceinline__ float gate_exp(float x);
template <> __device__ __forceinline__ float gate_exp<bf16_t>(float x) { return __expf(x); }
template <> __device__ __forceinline__ float gate_exp<float>(float x) { return expf(x); }

// 2^x for decay exponents already in base-2 units (the chunk kernels keep the
// gate's prefix sums scaled by log2(e)).  bf16 inputs use the hardware exp2;
// fp32 inputs the library exp2f.
constexpr float kLog2e = 1.44269504088896340736f;
template <typename E> __device__ __forceinline__ float gate_exp2(float x);
template <> __device__ __forceinline__ float gate_exp2<bf16_t>(float x) { return __builtin_amdgcn_exp2f(x); }
template <> __device__ __forceinline__ float gate_exp2<float>(float x) { return exp2f(x); }

// -softplus(x) = -(max(x, 0) + log(1 + e^-|x|)) and the logistic function
// 1 / (1 + e^-x), without overflow for large |x|.  fp32 inputs use the
// library expf / log1pf; bf16 inputs the hardware exp and log, with
// log(1 + t) = t - t^2/2 + t^3/3 - t^4/4 below t = 1/16, where rounding 1 + t
// would lose the small result (series error < 3e-6 relative).
template <typename E> __device__ __forceinline__ float softplus_tail(float t);
template <> __device__ __forceinline__ float softplus_tail<float>(float t) { return log1pf(t); }
template <> __device__ __forceinline__ float softplus_tail<bf16_t>(float t) {
    return t < 0.0625f ? t * (1.f - t * (0.5f - t * (1.f / 3.f - t * 0.25f))) : __logf(1.f + t);
}
template <typename E>
__device__ __forceinline__ float neg_softplus(float x) {
    return -(fmaxf(x, 0.f) + softplus_tail<E>(gate_exp<E>(-fabsf(x))));
}
// 1 / x: exact division for fp32 inputs, the hardware reciprocal (about one
// ulp) for bf16 inputs.
template <typename E> __device__ __forceinline__ float recip(float x);
template <> __device__ __forceinline__ float recip<float>(float x) { return 1.f / x; }
template <> __device__ __forceinline__ float recip<bf16_t>(float x) { return __builtin_amdgcn_rcpf(x); }

template <typename E>
__device__ __forceinline__ float sigmoid(float x) {
    const float e = gate_exp<E>(-fabsf(x));
    return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// Workspace header written by the chunk-map kernel.
struct WsHeader {
    int32_t bad_seqlens;   // nonzero: cu_seqlens rejected, every later kernel exits
    int32_t total_chunks;  // number of chunks over all sequences
    int32_t wait_timeout;  // nonzero: a bounded wait gave up
    int32_t seg_ticket;    // next (segment, pair) ticket of the segmented walk
};

}  // namespace kda
