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

// eq:write for a bf16 state element: r + s y rounded ONCE to bf16 (nearest
// even).  fmaf gives r + s y correctly rounded to fp32; rounding that again to
// bf16 can only go wrong where the fp32 value lies exactly on a bf16 rounding
// midpoint (low 16 bits 0x8000) while the exact sum does not -- common when s
// saturates near 0 or 2.  There the sign of the fp32 rounding error decides:
// s y - v is exact in fp64 (when v is such a midpoint both terms lie within
// 2^42 of each other), one more fp64 add of r rounds once and keeps the sign.
// The fp32 value is moved one unit off the midpoint towards the exact sum, and
// the final bf16 conversion then rounds the right way.  Returns that fp32 value.
// s_pow2: s is 0 or +-2^k (no mantissa bits).  Then s y is exact with at most
// 8 significant bits, and r + s y is either exact in fp32 or within 2^-16 of
// its larger term -- never on a midpoint -- so the check is skipped (s == 1
// without a write projection; there midpoints are frequent and all exact).
__device__ __forceinline__ bool write_scale_pow2(float s) {
    return (__float_as_uint(s) & 0x7fffffu) == 0u;
}
__device__ __forceinline__ float write_sum_bf16(float s, float y, float r, bool s_pow2) {
    float v = fmaf(s, y, r);
    uint32_t b = __float_as_uint(v);
    if (__builtin_expect((b & 0xffffu) == 0x8000u && !s_pow2, 0)) {
        const double e = fma((double)s, (double)y, -(double)v) + (double)r;
        if (e != 0.0) b += ((e > 0.0) == (v > 0.0)) ? 1u : 0xffffffffu;
        v = __uint_as_float(b);
    }
    return v;
}

// Eight eq:write elements of a bf16 state: packed y and r words (low half =
// even channel) -> packed stored words, each the exact r + s y rounded once.
// The midpoint test runs on all eight sums; the fp64 tie-break (rare) is one
// branch for the group.
__device__ __forceinline__ u32x4 write8_bf16(float s, bool s_pow2, u32x4 y, u32x4 r) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = fmaf(s, bf16_lo(y[e]), bf16_lo(r[e]));
        v[2 * e + 1] = fmaf(s, bf16_hi(y[e]), bf16_hi(r[e]));
    }
    bool mid = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) mid |= (__float_as_uint(v[k]) & 0xffffu) == 0x8000u;
    if (__builtin_expect(mid && !s_pow2, 0)) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float yk = (k & 1) ? bf16_hi(y[k >> 1]) : bf16_lo(y[k >> 1]);
            const float rk = (k & 1) ? bf16_hi(r[k >> 1]) : bf16_lo(r[k >> 1]);
            v[k] = write_sum_bf16(s, yk, rk, false);
        }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    return o;
}

// Storage-type adapters for the generic kernels.
template <typename T> struct Store;
template <> struct Store<float> {
    __device__ static __forceinline__ float load(const float *p) { return *p; }
    __device__ static __forceinline__ float round(float v) { return v; }
    // eq:write, one rounding (fmaf)
    __device__ static __forceinline__ float write(float s, float y, float r) { return fmaf(s, y, r); }
    __device__ static __forceinline__ void store(float *p, float v) { *p = v; }
};
template <> struct Store<bf16_t> {
    __device__ static __forceinline__ float load(const bf16_t *p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
    // eq:write, one rounding to bf16 (stored value, widened)
    __device__ static __forceinline__ float write(float s, float y, float r) {
        return round(write_sum_bf16(s, y, r, write_scale_pow2(s)));
    }
    __device__ static __forceinline__ void store(bf16_t *p, float v) { *p = f32_to_bf16(v); }
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

}  // namespace grk
