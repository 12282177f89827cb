// gr_device.h -- device helpers shared by the HIP kernels of the GR library.
//
// gfx950 (CDNA4) only: wave64, bf16 stored as raw 16-bit words and widened to
// fp32 by shifts, rounded back with the hardware round-to-nearest-even
// conversion, sigmoid built from the hardware exp2 and reciprocal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grk {

typedef uint16_t bf16_t;  // bf16 storage word
typedef uint8_t fp8_t;    // OCP e4m3 (e4m3fn) storage byte
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> fp32 --------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 v = {a, b};
    bf16x2 h = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float a) {
    return __builtin_bit_cast(bf16_t, (__bf16)a);
}

// ---- fp8 (OCP e4m3) <-> fp32 --------------------------------------------
// gfx950's conversions are OCP e4m3fn with round to nearest even; values that
// round beyond 448 would become NaN, so stores clamp to +-448 first
// (saturating, v_med3).  Every e4m3 value is exact in bf16 and fp32.
constexpr float kFp8Max = 448.0f;
__device__ __forceinline__ float fp8_sat(float x) { return __builtin_amdgcn_fmed3f(x, -kFp8Max, kFp8Max); }
// four floats -> e4m3 bytes 0..3 of a word (byte 0 = a)
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_sat(a), fp8_sat(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_sat(c), fp8_sat(d), w, true);
    return (uint32_t)w;
}
// bytes (0,1) or (2,3) of a word -> two floats
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 fp8x2_lo(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false); }
__device__ __forceinline__ f32x2 fp8x2_hi(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true); }

// eq:write for eight bf16 elements: packed y and r words (low half = even
// channel) -> packed words of r + s y, formed by one fp32 FMA and rounded to
// bf16 (nearest even).
__device__ __forceinline__ u32x4 write8_bf16(float s, u32x4 y, u32x4 r) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(fmaf(s, bf16_lo(y[e]), bf16_lo(r[e])), fmaf(s, bf16_hi(y[e]), bf16_hi(r[e])));
    return o;
}

// eq:write for eight e4m3 elements: r holds bytes 0..7 (channel order), y four
// packed bf16 words -> the stored bytes of r + s y (one fp32 FMA, saturated,
// rounded to e4m3, nearest even).
__device__ __forceinline__ u32x2 write8_fp8(float s, u32x4 y, u32x2 r) {
    u32x2 o;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const f32x2 a = fp8x2_lo(r[k]), b = fp8x2_hi(r[k]);
        o[k] = pack_fp8x4(fmaf(s, bf16_lo(y[2 * k]), a.x), fmaf(s, bf16_hi(y[2 * k]), a.y),
                          fmaf(s, bf16_lo(y[2 * k + 1]), b.x), fmaf(s, bf16_hi(y[2 * k + 1]), b.y));
    }
    return o;
}
// Eight e4m3 bytes -> four packed bf16 words of the same values (exact).
__device__ __forceinline__ u32x4 widen8_fp8_bf16(u32x2 r) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const f32x2 a = fp8x2_lo(r[k]), b = fp8x2_hi(r[k]);
        w[2 * k] = pack_bf16x2(a.x, a.y);
        w[2 * k + 1] = pack_bf16x2(b.x, b.y);
    }
    return w;
}

// Storage-type adapters for the generic kernels.
template <typename T> struct Store;
template <> struct Store<float> {
    __device__ static __forceinline__ float load(const float *p) { return *p; }
    __device__ static __forceinline__ float round(float v) { return v; }
    // eq:write: one fp32 fused multiply-add
    __device__ static __forceinline__ float write(float s, float y, float r) { return fmaf(s, y, r); }
    __device__ static __forceinline__ void store(float *p, float v) { *p = v; }
};
template <> struct Store<bf16_t> {
    __device__ static __forceinline__ float load(const bf16_t *p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
    // eq:write: one fp32 fused multiply-add, rounded to bf16 (stored value, widened)
    __device__ static __forceinline__ float write(float s, float y, float r) { return round(fmaf(s, y, r)); }
    __device__ static __forceinline__ void store(bf16_t *p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Store<fp8_t> {
    __device__ static __forceinline__ float load(const fp8_t *p) { return __builtin_amdgcn_cvt_f32_fp8((int)*p, 0); }
    __device__ static __forceinline__ uint32_t enc(float v) {
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fp8_sat(v), 0.f, 0, false) & 0xffu;
    }
    __device__ static __forceinline__ float round(float v) { return __builtin_amdgcn_cvt_f32_fp8((int)enc(v), 0); }
    __device__ static __forceinline__ void store(fp8_t *p, float v) { *p = (fp8_t)enc(v); }
    // eq:write: one fp32 fused multiply-add, rounded to e4m3 (stored value, widened)
    __device__ static __forceinline__ float write(float s, float y, float r) { return round(fmaf(s, y, r)); }
};

// ---- activations ----------------------------------------------------------
// sigmoid(x) = 1 / (1 + e^-x) with e^-x = 2^(-x log2 e): hardware v_exp_f32 and
// v_rcp_f32.  Saturates cleanly: e^-x -> inf gives 0, e^-x -> 0 gives 1.
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// tanh(x) = sign(x) (1 - e^{-2|x|}) / (1 + e^{-2|x|}), from the hardware exp2.
__device__ __forceinline__ float tanh_f(float x) {
    float e = __builtin_amdgcn_exp2f(-2.0f * kLog2e * fabsf(x));
    float t = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    return copysignf(t, x);
}

// ---- wave64 / workgroup reductions ----------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Sum over the whole workgroup (blockDim.x a multiple of 64, at most 1024).
// `scratch` holds at least blockDim.x / 64 floats.  Every thread gets the sum.
__device__ __forceinline__ float block_sum(float v, float *scratch) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < nw; ++w) t += scratch[w];
    return t;
}
// K sums over the whole workgroup with one exchange: v[q] becomes the sum of
// every thread's v[q] (each the same as block_sum(v[q]) would give).
// `scratch` holds at least K * blockDim.x / 64 floats.
template <int K>
__device__ __forceinline__ void block_sum_many(float (&v)[K], float *scratch) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nw = blockDim.x >> 6;
#pragma unroll
    for (int q = 0; q < K; ++q) v[q] = wave_sum(v[q]);
    __syncthreads();
    if (lane == 0) {
#pragma unroll
        for (int q = 0; q < K; ++q) scratch[q * nw + wave] = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < K; ++q) {
        float t = 0.f;
        for (int w = 0; w < nw; ++w) t += scratch[q * nw + w];
        v[q] = t;
    }
}

}  // namespace grk
