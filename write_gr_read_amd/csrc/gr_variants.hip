// gr_variants.hip -- streaming kernels of the variants on the widened state:
// expand, the AltUp-style static read and round-robin write, the per-channel
// write, and the collapse.
//
//   expand             "Paper reading: Qwen3.8 Flash Next", part 2 (Residual),
//                      sec. 6, eq:rcv: every branch starts at the embedding.
//   static read,       the same page, sec. 1, eq:input (u = sum_i h_i R_i) and
//   round-robin write  eq:output (y added to branch layer mod n only).
//   per-channel write  "Qwen3.8-Flash-Next architecture notes, 06 Residual",
//                      sec. 3: per-channel write strengths, here a learned
//                      [n][d] parameter.
//   collapse           read-out after the last block: RMSNorm of the sum of
//                      the branches.
//
// Each lane moves 16 bytes of the state per vector (4 fp32, 8 bf16 or 16 e4m3
// values) with the matching span of the d-wide tensors; arithmetic in fp32,
// stores rounded to nearest even (e4m3 saturating at +-448).  Streams that
// are only read (static read, collapse) or only written (expand) use
// non-temporal accesses (static read 123 -> 104 us, collapse 125 -> 109 us,
// expand 123 -> 117 us at N = 16384, d = 4096, n = 4 bf16); the in-place
// writes keep ordinary ones (non-temporal there: 58 -> 65 and 235 -> 271 us).
#include "gr_device.h"
#include "gr_internal.h"

namespace grk {
namespace {

constexpr int kVarThreads = 256;

// 16 bytes of T <-> floats
template <typename T> struct V16;
// 16-byte accesses; NT: non-temporal (a stream read or written once)
template <bool NT, typename V> __device__ __forceinline__ V ld16(const V *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, typename V> __device__ __forceinline__ void st16(V *p, V x) {
    if constexpr (NT) __builtin_nontemporal_store(x, p);
    else *p = x;
}
template <> struct V16<float> {
    static constexpr int E = 4;
    template <bool NT = false> __device__ static void load(const float *p, float *v) {
        const f32x4 x = ld16<NT>(reinterpret_cast<const f32x4 *>(p));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = x[e];
    }
    template <bool NT = false> __device__ static void store(float *p, const float *v) {
        st16<NT>(reinterpret_cast<f32x4 *>(p), f32x4{v[0], v[1], v[2], v[3]});
    }
};
template <> struct V16<bf16_t> {
    static constexpr int E = 8;
    template <bool NT = false> __device__ static void load(const bf16_t *p, float *v) {
        const u32x4 x = ld16<NT>(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[2 * e] = bf16_lo(x[e]); v[2 * e + 1] = bf16_hi(x[e]); }
    }
    template <bool NT = false> __device__ static void store(bf16_t *p, const float *v) {
        u32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        st16<NT>(reinterpret_cast<u32x4 *>(p), x);
    }
};
template <> struct V16<fp8_t> {
    static constexpr int E = 16;
    template <bool NT = false> __device__ static void load(const fp8_t *p, float *v) {
        const u32x4 x = ld16<NT>(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x2 a = fp8x2_lo(x[e]), b = fp8x2_hi(x[e]);
            v[4 * e] = a.x; v[4 * e + 1] = a.y; v[4 * e + 2] = b.x; v[4 * e + 3] = b.y;
        }
    }
    template <bool NT = false> __device__ static void store(fp8_t *p, const float *v) {
        u32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = pack_fp8x4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]);
        st16<NT>(reinterpret_cast<u32x4 *>(p), x);
    }
};
// E consecutive values of type W (E a multiple of V16<W>::E)
template <typename W, int E, bool NT = false> __device__ __forceinline__ void loadE(const W *p, float *v) {
#pragma unroll
    for (int k = 0; k < E / V16<W>::E; ++k) V16<W>::template load<NT>(p + k * V16<W>::E, v + k * V16<W>::E);
}
template <typename W, int E> __device__ __forceinline__ void storeE(W *p, const float *v) {
#pragma unroll
    for (int k = 0; k < E / V16<W>::E; ++k) V16<W>::store(p + k * V16<W>::E, v + k * V16<W>::E);
}

// R[t][i] = e[t] for every branch i
template <typename T, typename W>
__global__ void __launch_bounds__(kVarThreads)
k_expand(const W *__restrict__ emb, T *__restrict__ state, int64_t N, int n, int d) {
    constexpr int E = V16<T>::E;
    const int dv = d / E;
    const int64_t total = N * dv;
    for (int64_t q = (int64_t)blockIdx.x * kVarThreads + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * kVarThreads) {
        const int64_t t = q / dv;
        const int cv = (int)(q % dv);
        float v[E];
        loadE<W, E, true>(emb + t * d + cv * E, v);
        for (int i = 0; i < n; ++i) V16<T>::template store<true>(state + (t * n + i) * (int64_t)d + cv * E, v);
    }
}

// u[t] = sum_i h_i R[t][i]  (h: n floats on the device)
template <typename T, typename W>
__global__ void __launch_bounds__(kVarThreads)
k_static_read(const T *__restrict__ state, const float *__restrict__ h, W *__restrict__ u,
              int64_t N, int n, int d) {
    constexpr int E = V16<T>::E;
    const int dv = d / E;
    const int64_t total = N * dv;
    for (int64_t q = (int64_t)blockIdx.x * kVarThreads + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * kVarThreads) {
        const int64_t t = q / dv;
        const int cv = (int)(q % dv);
        float acc[E], v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;
        for (int i = 0; i < n; ++i) {
            V16<T>::template load<true>(state + (t * n + i) * (int64_t)d + cv * E, v);
            const float hi = h[i];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(hi, v[e], acc[e]);
        }
        storeE<W, E>(u + t * d + cv * E, acc);
    }
}

// R[t][k] += y[t] for the one branch k = layer mod n (one fp32 add, then the store)
template <typename T, typename W>
__global__ void __launch_bounds__(kVarThreads)
k_round_robin_write(T *__restrict__ state, const W *__restrict__ y, int64_t N, int n, int d, int k) {
    constexpr int E = V16<T>::E;
    const int dv = d / E;
    const int64_t total = N * dv;
    for (int64_t q = (int64_t)blockIdx.x * kVarThreads + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * kVarThreads) {
        const int64_t t = q / dv;
        const int cv = (int)(q % dv);
        float v[E], yv[E];
        T *p = state + (t * n + k) * (int64_t)d + cv * E;
        V16<T>::load(p, v);
        loadE<W, E>(y + t * d + cv * E, yv);
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = v[e] + yv[e];
        V16<T>::store(p, v);
    }
}

// R[t][i][c] += s[i][c] y[t][c]  (s: [n][d] floats; one fp32 FMA, then the store);
// a lane takes one (token, vector) and walks the branches, so y is read once
template <typename T, typename W>
__global__ void __launch_bounds__(kVarThreads)
k_write_per_channel(T *__restrict__ state, const W *__restrict__ y, const float *__restrict__ s,
                    int64_t N, int n, int d) {
    constexpr int E = V16<T>::E;
    const int dv = d / E;
    const int64_t total = N * dv;
    for (int64_t q = (int64_t)blockIdx.x * kVarThreads + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * kVarThreads) {
        const int64_t t = q / dv;
        const int cv = (int)(q % dv);
        float yv[E];
        loadE<W, E>(y + t * d + cv * E, yv);
        for (int i = 0; i < n; ++i) {
            float v[E], sv[E];
            T *p = state + (t * n + i) * (int64_t)d + cv * E;
            V16<T>::load(p, v);
            loadE<float, E>(s + (int64_t)i * d + cv * E, sv);
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = fmaf(sv[e], yv[e], v[e]);
            V16<T>::store(p, v);
        }
    }
}

// out[t] = w . h / sqrt(mean(h^2) + eps), h = sum_i R[t][i] in fp32 (not stored);
// one workgroup per token.  STAGE (d <= 8192): h is kept in LDS (d floats of
// dynamic shared memory) between the two passes; otherwise it is formed again
// from the row, which the first pass left in cache.
template <typename T, typename W, bool STAGE>
__global__ void __launch_bounds__(kVarThreads)
k_collapse(const T *__restrict__ state, const W *__restrict__ w, float eps, W *__restrict__ out,
           int n, int d) {
    constexpr int E = V16<T>::E;
    __shared__ float red[kVarThreads / 64];
    extern __shared__ float hbuf[];
    const int64_t t = blockIdx.x;
    const int dv = d / E;
    const T *row = state + t * n * (int64_t)d;
    auto branch_sum = [&](int cv, float *hsum) {
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) hsum[e] = 0.f;
        for (int i = 0; i < n; ++i) {
            V16<T>::template load<true>(row + (int64_t)i * d + cv * E, v);
#pragma unroll
            for (int e = 0; e < E; ++e) hsum[e] += v[e];
        }
    };
    float ss = 0.f;
    for (int cv = threadIdx.x; cv < dv; cv += kVarThreads) {
        float hsum[E];
        branch_sum(cv, hsum);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            ss = fmaf(hsum[e], hsum[e], ss);
            if (STAGE) hbuf[cv * E + e] = hsum[e];
        }
    }
    ss = block_sum(ss, red);   // (its barriers also order the LDS writes above)
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    for (int cv = threadIdx.x; cv < dv; cv += kVarThreads) {
        float hsum[E], wv[E];
        if (STAGE) {
#pragma unroll
            for (int e = 0; e < E; ++e) hsum[e] = hbuf[cv * E + e];
        } else {
            branch_sum(cv, hsum);
        }
        loadE<W, E>(w + cv * E, wv);
#pragma unroll
        for (int e = 0; e < E; ++e) hsum[e] = wv[e] * (hsum[e] * inv);
        storeE<W, E>(out + t * d + cv * E, hsum);
    }
}

// widest row whose branch sum is staged in LDS (32 KB of dynamic shared memory)
constexpr int kCollapseStageMax = 8192;

unsigned grid_for(int64_t vectors) {
    const int64_t b = (vectors + kVarThreads - 1) / kVarThreads;
    return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

}  // namespace

// dt: 0 fp32, 1 bf16, 2 e4m3 state with bf16 activations

#define GR_VAR_DISPATCH(DT, CALL_F32, CALL_BF16, CALL_FP8) \
    switch (DT) {                                          \
    case 0: CALL_F32; break;                               \
    case 1: CALL_BF16; break;                              \
    case 2: CALL_FP8; break;                               \
    default: return hipErrorInvalidValue;                  \
    }                                                      \
    return hipGetLastError();

hipError_t launch_expand(const void *e, void *state, int dt, int64_t N, int n, int d, hipStream_t st) {
    const int E = dt == 0 ? 4 : dt == 1 ? 8 : 16;
    const dim3 g(grid_for(N * (d / E))), b(kVarThreads);
    GR_VAR_DISPATCH(dt,
        hipLaunchKernelGGL((k_expand<float, float>), g, b, 0, st, (const float *)e, (float *)state, N, n, d),
        hipLaunchKernelGGL((k_expand<bf16_t, bf16_t>), g, b, 0, st, (const bf16_t *)e, (bf16_t *)state, N, n, d),
        hipLaunchKernelGGL((k_expand<fp8_t, bf16_t>), g, b, 0, st, (const bf16_t *)e, (fp8_t *)state, N, n, d))
}

hipError_t launch_static_read(const void *state, const float *h, void *u, int dt, int64_t N, int n, int d,
                              hipStream_t st) {
    const int E = dt == 0 ? 4 : dt == 1 ? 8 : 16;
    const dim3 g(grid_for(N * (d / E))), b(kVarThreads);
    GR_VAR_DISPATCH(dt,
        hipLaunchKernelGGL((k_static_read<float, float>), g, b, 0, st, (const float *)state, h, (float *)u, N, n, d),
        hipLaunchKernelGGL((k_static_read<bf16_t, bf16_t>), g, b, 0, st, (const bf16_t *)state, h, (bf16_t *)u, N, n, d),
        hipLaunchKernelGGL((k_static_read<fp8_t, bf16_t>), g, b, 0, st, (const fp8_t *)state, h, (bf16_t *)u, N, n, d))
}

hipError_t launch_round_robin_write(void *state, const void *y, int dt, int64_t N, int n, int d, int layer,
                                    hipStream_t st) {
    const int E = dt == 0 ? 4 : dt == 1 ? 8 : 16;
    const int k = layer % n;
    const dim3 g(grid_for(N * (d / E))), b(kVarThreads);
    GR_VAR_DISPATCH(dt,
        hipLaunchKernelGGL((k_round_robin_write<float, float>), g, b, 0, st, (float *)state, (const float *)y, N, n, d, k),
        hipLaunchKernelGGL((k_round_robin_write<bf16_t, bf16_t>), g, b, 0, st, (bf16_t *)state, (const bf16_t *)y, N, n, d, k),
        hipLaunchKernelGGL((k_round_robin_write<fp8_t, bf16_t>), g, b, 0, st, (fp8_t *)state, (const bf16_t *)y, N, n, d, k))
}

hipError_t launch_write_per_channel(void *state, const void *y, const float *s, int dt, int64_t N, int n, int d,
                                    hipStream_t st) {
    const int E = dt == 0 ? 4 : dt == 1 ? 8 : 16;
    const dim3 g(grid_for(N * (d / E))), b(kVarThreads);
    GR_VAR_DISPATCH(dt,
        hipLaunchKernelGGL((k_write_per_channel<float, float>), g, b, 0, st, (float *)state, (const float *)y, s, N, n, d),
        hipLaunchKernelGGL((k_write_per_channel<bf16_t, bf16_t>), g, b, 0, st, (bf16_t *)state, (const bf16_t *)y, s, N, n, d),
        hipLaunchKernelGGL((k_write_per_channel<fp8_t, bf16_t>), g, b, 0, st, (fp8_t *)state, (const bf16_t *)y, s, N, n, d))
}

hipError_t launch_collapse(const void *state, const void *w, float eps, void *out, int dt, int64_t N, int n,
                           int d, hipStream_t st) {
    const dim3 g((unsigned)N), b(kVarThreads);
    if (d <= kCollapseStageMax) {
        const size_t lds = sizeof(float) * (size_t)d;
        GR_VAR_DISPATCH(dt,
            hipLaunchKernelGGL((k_collapse<float, float, true>), g, b, lds, st, (const float *)state, (const float *)w, eps, (float *)out, n, d),
            hipLaunchKernelGGL((k_collapse<bf16_t, bf16_t, true>), g, b, lds, st, (const bf16_t *)state, (const bf16_t *)w, eps, (bf16_t *)out, n, d),
            hipLaunchKernelGGL((k_collapse<fp8_t, bf16_t, true>), g, b, lds, st, (const fp8_t *)state, (const bf16_t *)w, eps, (bf16_t *)out, n, d))
    }
    GR_VAR_DISPATCH(dt,
        hipLaunchKernelGGL((k_collapse<float, float, false>), g, b, 0, st, (const float *)state, (const float *)w, eps, (float *)out, n, d),
        hipLaunchKernelGGL((k_collapse<bf16_t, bf16_t, false>), g, b, 0, st, (const bf16_t *)state, (const bf16_t *)w, eps, (bf16_t *)out, n, d),
        hipLaunchKernelGGL((k_collapse<fp8_t, bf16_t, false>), g, b, 0, st, (const fp8_t *)state, (const bf16_t *)w, eps, (bf16_t *)out, n, d))
}

#undef GR_VAR_DISPATCH

}  // namespace grk
