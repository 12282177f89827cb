// gr_generic.hip -- shape-generic kernels of the GR library.
//
// These cover every shape the C ABI accepts (1 <= n <= 8, any d with the
// vector alignment, 0 <= r <= 512, fp32, bf16 or an fp8 state with bf16
// activations and weights) with plain VALU code: one workgroup per token,
// fp32 arithmetic.  The MFMA fast path of the widened
// bf16 state lives in gr_fast.hip; these are the fallback and the fp32 path.
//
// Method: "Paper reading: Qwen3.8 Flash Next", part 2 (Residual), sec. 4
// (Gated Residual), eq:rms, eq:gate, eq:use_gate, eq:s, eq:write; the n = 1
// fused add + RMSNorm of "Residual" (LLM inference), sec. 3.3.
#include "gr_device.h"
#include "gr_internal.h"

namespace grk {

constexpr int kGenThreads = 256;
constexpr int kRowsPerPass = 16;  // projection rows accumulated per sweep (one reduction each)

// ---------------------------------------------------------------------------
// GR read (optionally preceded by the write of the previous sublayer), one
// workgroup per token.  Every pass walks the row in the same (branch, channel)
// order with the same thread mapping, so each thread only re-reads elements it
// wrote itself.
//   FUSED: R' = R + s_in y is computed (one fp32 FMA), rounded to the state
//   dtype, stored, and the read then uses the stored R'.
// T: state storage type; W: storage type of y, u, gamma and the weights.
template <typename T, typename W, bool FUSED>
__global__ void __launch_bounds__(kGenThreads)
k_read_generic(T *__restrict__ state, const W *__restrict__ y, const float *__restrict__ s_in,
               int n, int d, int r, float eps, const W *__restrict__ gamma,
               const W *__restrict__ wd, const W *__restrict__ wu, const W *__restrict__ ww,
               W *__restrict__ u, float *__restrict__ s_out) {
    __shared__ float red[kRowsPerPass * (kGenThreads / 64)];
    __shared__ float rho[8];
    __shared__ float proj[512 + 8];  // z (then SiLU) for k < r, write logits after
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nd = (int64_t)n * d;
    T *Rt = state + t * nd;

    // eq:write (FUSED) and the per-branch sum of squares of eq:rms (n <= 8),
    // reduced together.
    float ss[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ss[i] = 0.f;
        if (i < n) {
            const float si = FUSED ? s_in[t * n + i] : 0.f;
            for (int c = tid; c < d; c += kGenThreads) {
                float v = Store<T>::load(Rt + (int64_t)i * d + c);
                if (FUSED) {
                    v = Store<T>::write(si, Store<W>::load(y + t * d + c), v);
                    Store<T>::store(Rt + (int64_t)i * d + c, v);
                }
                ss[i] = fmaf(v, v, ss[i]);
            }
        }
    }
    block_sum_many(ss, red);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (tid == i && i < n) rho[i] = 1.0f / sqrtf(ss[i] / (float)d + eps);
    __syncthreads();

    // eq:gate down projection and eq:s logits: rows k < r of W_down, then the
    // n rows of W_write, against v = vec(R-hat).
    const int rows = r + (ww ? n : 0);
    for (int k0 = 0; k0 < rows; k0 += kRowsPerPass) {
        float acc[kRowsPerPass];
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q) acc[q] = 0.f;
        for (int i = 0; i < n; ++i) {
            const float ri = rho[i];
            for (int c = tid; c < d; c += kGenThreads) {
                const int64_t j = (int64_t)i * d + c;
                const float v = Store<W>::load(gamma + j) * Store<T>::load(Rt + j) * ri;
#pragma unroll
                for (int q = 0; q < kRowsPerPass; ++q) {
                    const int k = k0 + q;
                    if (k < rows) {
                        const W *wrow = k < r ? wd + (int64_t)k * nd : ww + (int64_t)(k - r) * nd;
                        acc[q] = fmaf(Store<W>::load(wrow + j), v, acc[q]);
                    }
                }
            }
        }
        block_sum_many(acc, red);
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q)
            if (tid == q && k0 + q < rows) proj[k0 + q] = acc[q] / (float)n;
    }
    __syncthreads();
    for (int k = tid; k < r; k += kGenThreads) proj[k] = silu_f(proj[k]);
    __syncthreads();

    // eq:gate up projection + sigmoid, eq:use_gate combine.
    for (int c = tid; c < d; c += kGenThreads) {
        float acc_u = 0.f;
        for (int i = 0; i < n; ++i) {
            const int64_t j = (int64_t)i * d + c;
            float g = 1.0f;
            if (r > 0) {
                // sixteen weights per batch: independent loads, one round trip
                float l = 0.f;
                const W *wrow = wu + j * r;
                for (int k0 = 0; k0 < r; k0 += 16) {
                    float wv[16];
#pragma unroll
                    for (int q = 0; q < 16; ++q) wv[q] = k0 + q < r ? Store<W>::load(wrow + k0 + q) : 0.f;
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        if (k0 + q < r) l = fmaf(wv[q], proj[k0 + q], l);
                }
                g = sigmoid_f(l);
            }
            const float v = Store<W>::load(gamma + j) * Store<T>::load(Rt + j) * rho[i];
            acc_u = fmaf(g, v, acc_u);
        }
        Store<W>::store(u + t * d + c, acc_u / (float)n);
    }
    if (s_out && tid < n) s_out[t * n + tid] = ww ? 2.0f * sigmoid_f(proj[r + tid]) : 1.0f;
}

// ---------------------------------------------------------------------------
// The same read (and fused write + read) for small fp32 rows: n = 4,
// d = 256 EPT, r = 16 RB (RB = 1, 2, 4).  With every trip count known at
// compile time each phase is straight-line code, so a thread's loads of all
// four branches (and of all projection rows) go out together instead of one
// loop iteration's round trip after another; every reduction hands all its
// sums to every thread (z, SiLU(z) and the write logits stay in registers).
// ONE (the weights a thread needs fit in registers: d = 256 with r = 16): the
// W_down / W_write rows and the W_up rows are loaded with the state, so the
// whole call is one memory round trip followed by two block reductions;
// otherwise the projection rows come 16 at a time, one round trip per pass.
// Same arithmetic and order of operations per element as k_read_generic.
template <bool FUSED, int EPT, int RB>
__global__ void __launch_bounds__(kGenThreads)
k_read_small(float *__restrict__ state, const float *__restrict__ y, const float *__restrict__ s_in,
             float eps, const float *__restrict__ gamma, const float *__restrict__ wd,
             const float *__restrict__ wu, const float *__restrict__ ww, float *__restrict__ u,
             float *__restrict__ s_out) {
    constexpr int NB = 4, D = kGenThreads * EPT, ND = NB * D, R = 16 * RB;
    constexpr int PASSES = RB + 1;                   // 16 projection rows each; the last one the write rows
    constexpr int ROWS = R + NB;                     // down rows, then the write rows
    constexpr bool ONE = NB * EPT * ROWS <= 96 && NB * EPT * R <= 64;
    constexpr int KR = ONE ? ROWS : 16;              // sums per projection reduction
    __shared__ float red[(KR > NB ? KR : NB) * (kGenThreads / 64)];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    float *Rt = state + t * ND;
    const bool haw = ww != nullptr;

    // ONE: every weight this thread uses, issued before the state is touched
    // (a missing W_write reads W_down's rows instead; their sums are unused)
    float wv[ONE ? ROWS : 1][NB][EPT];
    float wuv[ONE ? NB : 1][EPT][ONE ? R : 1];
    if constexpr (ONE) {
#pragma unroll
        for (int k = 0; k < ROWS; ++k) {
            const float *wrow = k < R ? wd + (int64_t)k * ND : (haw ? ww + (int64_t)(k - R) * ND : wd);
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int q = 0; q < EPT; ++q) wv[k][i][q] = wrow[i * D + tid + kGenThreads * q];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int q = 0; q < EPT; ++q) {
                const float4 *wrow = reinterpret_cast<const float4 *>(wu + (int64_t)(i * D + tid + kGenThreads * q) * R);
#pragma unroll
                for (int k4 = 0; k4 < R / 4; ++k4) {
                    const float4 w4 = wrow[k4];
                    wuv[i][q][4 * k4] = w4.x;
                    wuv[i][q][4 * k4 + 1] = w4.y;
                    wuv[i][q][4 * k4 + 2] = w4.z;
                    wuv[i][q][4 * k4 + 3] = w4.w;
                }
            }
    }

    // eq:write (FUSED) and the sums of squares of eq:rms
    float rv[NB][EPT], gv[NB][EPT], ss[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const float si = FUSED ? s_in[t * NB + i] : 0.f;
        ss[i] = 0.f;
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const int c = tid + kGenThreads * q;
            float v = Rt[i * D + c];
            if (FUSED) {
                v = fmaf(si, y[t * D + c], v);
                Rt[i * D + c] = v;
            }
            rv[i][q] = v;
            gv[i][q] = gamma[i * D + c];
            ss[i] = fmaf(v, v, ss[i]);
        }
    }
    block_sum_many(ss, red);
    float rho[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) rho[i] = 1.0f / sqrtf(ss[i] / (float)D + eps);
    // v = vec(R-hat) for this thread's elements
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int q = 0; q < EPT; ++q) gv[i][q] = gv[i][q] * rv[i][q] * rho[i];

    // eq:gate down projection (rows k < R) and eq:s logits (the n rows of W_write)
    float proj[16 * PASSES];
    if constexpr (ONE) {
        float acc[ROWS];
#pragma unroll
        for (int k = 0; k < ROWS; ++k) {
            acc[k] = 0.f;
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int q = 0; q < EPT; ++q) acc[k] = fmaf(wv[k][i][q], gv[i][q], acc[k]);
        }
        block_sum_many(acc, red);
#pragma unroll
        for (int k = 0; k < ROWS; ++k) proj[k] = acc[k] / (float)NB;
    } else {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            float acc[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                acc[k] = 0.f;
                const int row = 16 * p + k;
                const bool on = p < RB || (haw && k < NB);
                if (on) {
                    const float *wrow = p < RB ? wd + (int64_t)row * ND : ww + (int64_t)k * ND;
#pragma unroll
                    for (int i = 0; i < NB; ++i)
#pragma unroll
                        for (int q = 0; q < EPT; ++q)
                            acc[k] = fmaf(wrow[i * D + tid + kGenThreads * q], gv[i][q], acc[k]);
                }
            }
            block_sum_many(acc, red);
#pragma unroll
            for (int k = 0; k < 16; ++k) proj[16 * p + k] = acc[k] / (float)NB;
        }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) proj[k] = silu_f(proj[k]);

    // eq:gate up projection + sigmoid, eq:use_gate combine
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int c = tid + kGenThreads * q;
        float acc_u = 0.f;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            float l = 0.f;
            if constexpr (ONE) {
#pragma unroll
                for (int k = 0; k < R; ++k) l = fmaf(wuv[i][q][k], proj[k], l);
            } else {
                const float *wrow = wu + (int64_t)(i * D + c) * R;
#pragma unroll
                for (int k = 0; k < R; ++k) l = fmaf(wrow[k], proj[k], l);
            }
            acc_u = fmaf(sigmoid_f(l), gv[i][q], acc_u);
        }
        u[t * D + c] = acc_u / (float)NB;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (s_out && tid == i) s_out[t * NB + i] = haw ? 2.0f * sigmoid_f(proj[16 * RB + i]) : 1.0f;
}

// ---------------------------------------------------------------------------
// GR write, eq:write: streaming, 16-byte vectors (8 bf16 or 4 fp32 channels).
template <typename T>
__global__ void __launch_bounds__(256)
k_write(T *__restrict__ state, const T *__restrict__ y, const float *__restrict__ s,
        int64_t chunks, int n, int dv /* d / VEC */) {
    constexpr int VEC = 16 / sizeof(T);
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < chunks;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t cv = q % dv;
        const int64_t ti = q / dv;  // t * n + i
        const int64_t t = ti / n;
        const float si = s[ti];
        u32x4 rv = *reinterpret_cast<const u32x4 *>(state + q * VEC);
        const u32x4 yv = *reinterpret_cast<const u32x4 *>(y + (t * dv + cv) * VEC);
        if constexpr (sizeof(T) == 2) {
            rv = write8_bf16(si, yv, rv);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rv[e] = __float_as_uint(fmaf(si, __uint_as_float(yv[e]), __uint_as_float(rv[e])));
        }
        *reinterpret_cast<u32x4 *>(state + q * VEC) = rv;
    }
}

// The same for an fp8 state and bf16 y: 16 channels (16 state bytes, 32 y
// bytes) per item; eq:write in fp32, stored as e4m3 (saturating).
__global__ void __launch_bounds__(256)
k_write_fp8(fp8_t *__restrict__ state, const bf16_t *__restrict__ y, const float *__restrict__ s,
            int64_t chunks, int n, int dv /* d / 16 */) {
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < chunks;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t cv = q % dv;
        const int64_t ti = q / dv;  // t * n + i
        const int64_t t = ti / n;
        const float si = s[ti];
        u32x4 rv = *reinterpret_cast<const u32x4 *>(state + q * 16);
        const u32x4 *yp = reinterpret_cast<const u32x4 *>(y + (t * dv + cv) * 16);
        const u32x4 y0 = yp[0], y1 = yp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const u32x4 &yv = e < 2 ? y0 : y1;
            const uint32_t ya = yv[(2 * e) & 3], yb = yv[(2 * e + 1) & 3];  // channels 4e .. 4e+3
            const f32x2 r01 = fp8x2_lo(rv[e]), r23 = fp8x2_hi(rv[e]);
            rv[e] = pack_fp8x4(fmaf(si, bf16_lo(ya), r01[0]), fmaf(si, bf16_hi(ya), r01[1]),
                               fmaf(si, bf16_lo(yb), r23[0]), fmaf(si, bf16_hi(yb), r23[1]));
        }
        *reinterpret_cast<u32x4 *>(state + q * 16) = rv;
    }
}

// ---------------------------------------------------------------------------
// n = 1 fused residual add + RMSNorm ("Residual", sec. 3.3), one workgroup
// per token.  KPT > 0: each thread keeps KPT 16-byte chunks of h in registers;
// KPT == 0: any width, h is re-read (each thread only its own chunks).
template <typename T, int KPT>
__global__ void __launch_bounds__(256)
k_add_rmsnorm(T *__restrict__ x, const T *y, const T *__restrict__ w, float eps,
              T *out, int d) {
    constexpr int VEC = 16 / sizeof(T);
    __shared__ float red[4];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int dv = d / VEC;
    T *xt = x + t * d;
    const T *yt = y + t * d;
    T *ot = out + t * d;
    auto add_chunk = [&](int cv, u32x4 &hv, float &ss) {
        u32x4 xv = *reinterpret_cast<const u32x4 *>(xt + cv * VEC);
        const u32x4 yv = *reinterpret_cast<const u32x4 *>(yt + cv * VEC);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[e] = pack_bf16x2(bf16_lo(xv[e]) + bf16_lo(yv[e]), bf16_hi(xv[e]) + bf16_hi(yv[e]));
                const float a = bf16_lo(xv[e]), b = bf16_hi(xv[e]);
                ss = fmaf(a, a, ss);
                ss = fmaf(b, b, ss);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float h = __uint_as_float(xv[e]) + __uint_as_float(yv[e]);
                xv[e] = __float_as_uint(h);
                ss = fmaf(h, h, ss);
            }
        }
        *reinterpret_cast<u32x4 *>(xt + cv * VEC) = xv;
        hv = xv;
    };
    auto norm_chunk = [&](int cv, const u32x4 &hv, float inv) {
        const u32x4 wv = *reinterpret_cast<const u32x4 *>(w + cv * VEC);
        u32x4 ov;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ov[e] = pack_bf16x2(bf16_lo(wv[e]) * bf16_lo(hv[e]) * inv,
                                    bf16_hi(wv[e]) * bf16_hi(hv[e]) * inv);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ov[e] = __float_as_uint(__uint_as_float(wv[e]) * __uint_as_float(hv[e]) * inv);
        }
        *reinterpret_cast<u32x4 *>(ot + cv * VEC) = ov;
    };

    float ss = 0.f;
    if constexpr (KPT > 0) {
        u32x4 h[KPT];
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int cv = tid + k * 256;
            if (cv < dv) add_chunk(cv, h[k], ss);
        }
        const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)d + eps);
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int cv = tid + k * 256;
            if (cv < dv) norm_chunk(cv, h[k], inv);
        }
    } else {
        u32x4 h;
        for (int cv = tid; cv < dv; cv += 256) add_chunk(cv, h, ss);
        const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)d + eps);
        for (int cv = tid; cv < dv; cv += 256) {
            h = *reinterpret_cast<const u32x4 *>(xt + cv * VEC);
            norm_chunk(cv, h, inv);
        }
    }
}

// Persistent form for rows of at most 2048 vectors (d <= 16384 bf16): four
// workgroups per CU walk the tokens t = blockIdx, blockIdx + grid, ..., so the
// grid sweeps memory as one narrow front; w stays in registers, and the next
// token's x and y are loaded while the current token's sum of squares is
// reduced.  x and y are read and h written with non-temporal hints (streamed
// once; h is used again only after the sublayer), out with ordinary stores (the
// sublayer reads it next): 51 -> 43.5 us at N = 8192, d = 4096 bf16, where all
// non-temporal gives 45.7 us and none 51 us.  Same arithmetic, in the same
// order, as k_add_rmsnorm.  y is not restrict-qualified in either form:
// the call allows out == y.
template <typename T, int KPT>
__global__ void __launch_bounds__(256)
k_add_rmsnorm_walk(T *__restrict__ x, const T *y, const T *__restrict__ w, float eps,
                   T *out, int d, int64_t N) {
    constexpr int VEC = 16 / sizeof(T);
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int dv = d / VEC;
    u32x4 wv[KPT], xv[KPT], yv[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const int cv = tid + k * 256;
        wv[k] = cv < dv ? *reinterpret_cast<const u32x4 *>(w + cv * VEC) : u32x4{0u, 0u, 0u, 0u};
    }
    auto load = [&](int64_t t) {
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int cv = tid + k * 256;
            if (t < N && cv < dv) {
                xv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + t * d + cv * VEC));
                yv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(y + t * d + cv * VEC));
            }
        }
    };
    int64_t t = blockIdx.x;
    load(t);
    for (; t < N; t += gridDim.x) {
        u32x4 h[KPT];
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int cv = tid + k * 256;
            if (cv >= dv) continue;
            u32x4 hv;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hv[e] = pack_bf16x2(bf16_lo(xv[k][e]) + bf16_lo(yv[k][e]), bf16_hi(xv[k][e]) + bf16_hi(yv[k][e]));
                    const float a = bf16_lo(hv[e]), b = bf16_hi(hv[e]);
                    ss = fmaf(a, a, ss);
                    ss = fmaf(b, b, ss);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float hf = __uint_as_float(xv[k][e]) + __uint_as_float(yv[k][e]);
                    hv[e] = __float_as_uint(hf);
                    ss = fmaf(hf, hf, ss);
                }
            }
            __builtin_nontemporal_store(hv, reinterpret_cast<u32x4 *>(x + t * d + cv * VEC));
            h[k] = hv;
        }
        load(t + gridDim.x);   // the next token's rows fly during the reduction
        const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)d + eps);
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int cv = tid + k * 256;
            if (cv >= dv) continue;
            u32x4 ov;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ov[e] = pack_bf16x2(bf16_lo(wv[k][e]) * bf16_lo(h[k][e]) * inv,
                                        bf16_hi(wv[k][e]) * bf16_hi(h[k][e]) * inv);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ov[e] = __float_as_uint(__uint_as_float(wv[k][e]) * __uint_as_float(h[k][e]) * inv);
            }
            *reinterpret_cast<u32x4 *>(out + t * d + cv * VEC) = ov;
        }
    }
}

// ---------------------------------------------------------------------------
// Measurement support: y = 0.1 tanh(u) elementwise; plain 16-byte copy.
template <typename T>
__global__ void __launch_bounds__(256)
k_tanh_standin(const T *__restrict__ u, T *__restrict__ y, int64_t count) {
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < count;
         q += (int64_t)gridDim.x * blockDim.x)
        Store<T>::store(y + q, 0.1f * tanh_f(Store<T>::load(u + q)));
}
// the same over 16-byte vectors (u and y are 16-byte aligned, as the ABI
// requires); elements past the last whole vector are left to k_tanh_standin
template <typename T>
__global__ void __launch_bounds__(256)
k_tanh_standin_vec(const T *__restrict__ u, T *__restrict__ y, int64_t vecs) {
    constexpr int VEC = 16 / sizeof(T);
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < vecs;
         q += (int64_t)gridDim.x * blockDim.x) {
        T in[VEC], out[VEC];
        *reinterpret_cast<u32x4 *>(in) = *reinterpret_cast<const u32x4 *>(u + q * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) Store<T>::store(out + e, 0.1f * tanh_f(Store<T>::load(in + e)));
        *reinterpret_cast<u32x4 *>(y + q * VEC) = *reinterpret_cast<const u32x4 *>(out);
    }
}

__global__ void __launch_bounds__(256)
k_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t vecs) {
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < vecs;
         q += (int64_t)gridDim.x * blockDim.x)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + q), dst + q);
}

// ---------------------------------------------------------------------------
// Host launchers.
static unsigned grid_for(int64_t items, int64_t per_block, int64_t cap = 1 << 16) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (unsigned)g;
}

template <bool FUSED, int EPT>
static void read_small_rb(const ReadArgs &a, hipStream_t st) {
    const int rb = a.r / 16;
#define GR_SMALL(RB)                                                                                   \
    hipLaunchKernelGGL((k_read_small<FUSED, EPT, RB>), dim3((unsigned)a.N), dim3(kGenThreads), 0, st, \
                       (float *)a.state, (const float *)a.y, a.s_in, a.eps, (const float *)a.gamma,    \
                       (const float *)a.wd, (const float *)a.wu, (const float *)a.ww, (float *)a.u,     \
                       a.s_out)
    if (rb == 1) GR_SMALL(1);
    else if (rb == 2) GR_SMALL(2);
    else GR_SMALL(4);
#undef GR_SMALL
}

// fp32, n = 4, d in {256, 512, 1024}, r in {16, 32, 64}: k_read_small
static bool small_shape(const ReadArgs &a) {
    return !a.bf16 && !a.fp8 && a.n == 4 && (a.d == 256 || a.d == 512 || a.d == 1024) &&
           (a.r == 16 || a.r == 32 || a.r == 64);
}

template <bool FUSED>
static void read_small(const ReadArgs &a, hipStream_t st) {
    if (a.d == 256) read_small_rb<FUSED, 1>(a, st);
    else if (a.d == 512) read_small_rb<FUSED, 2>(a, st);
    else read_small_rb<FUSED, 4>(a, st);
}

template <typename T, typename W>
static hipError_t read_generic_t(const ReadArgs &a, hipStream_t st) {
    T *state = (T *)a.state;
    if (small_shape(a)) {
        if (a.fused) read_small<true>(a, st);
        else read_small<false>(a, st);
        return hipGetLastError();
    }
    if (a.fused)
        hipLaunchKernelGGL((k_read_generic<T, W, true>), dim3((unsigned)a.N), dim3(kGenThreads), 0,
                           st, state, (const W *)a.y, a.s_in, a.n, a.d, a.r, a.eps,
                           (const W *)a.gamma, (const W *)a.wd, (const W *)a.wu,
                           (const W *)a.ww, (W *)a.u, a.s_out);
    else
        hipLaunchKernelGGL((k_read_generic<T, W, false>), dim3((unsigned)a.N), dim3(kGenThreads), 0,
                           st, state, (const W *)nullptr, (const float *)nullptr, a.n, a.d, a.r,
                           a.eps, (const W *)a.gamma, (const W *)a.wd, (const W *)a.wu,
                           (const W *)a.ww, (W *)a.u, a.s_out);
    return hipGetLastError();
}

hipError_t launch_read_generic(const ReadArgs &a, hipStream_t st) {
    if (a.fp8) return read_generic_t<fp8_t, bf16_t>(a, st);
    return a.bf16 ? read_generic_t<bf16_t, bf16_t>(a, st) : read_generic_t<float, float>(a, st);
}

hipError_t launch_write(void *state, const void *y, const float *s, bool bf16, bool fp8, int64_t N,
                        int n, int d, hipStream_t st) {
    if (fp8) {
        const int64_t chunks = N * n * (int64_t)(d / 16);
        const unsigned g = grid_for(chunks, 256, 256 * 64);
        hipLaunchKernelGGL(k_write_fp8, dim3(g), dim3(256), 0, st, (fp8_t *)state, (const bf16_t *)y, s,
                           chunks, n, d / 16);
        return hipGetLastError();
    }
    const int vec = bf16 ? 8 : 4;
    const int64_t chunks = N * n * (int64_t)(d / vec);
    const unsigned g = grid_for(chunks, 256, 256 * 64);
    if (bf16)
        hipLaunchKernelGGL(k_write<bf16_t>, dim3(g), dim3(256), 0, st, (bf16_t *)state,
                           (const bf16_t *)y, s, chunks, n, d / vec);
    else
        hipLaunchKernelGGL(k_write<float>, dim3(g), dim3(256), 0, st, (float *)state,
                           (const float *)y, s, chunks, n, d / vec);
    return hipGetLastError();
}

template <typename T, int KPT>
static void add_rmsnorm_k(void *x, const void *y, const void *w, float eps, void *out,
                          int64_t N, int d, hipStream_t st) {
    if constexpr (KPT > 0) {
        if (N > 1024) {
            hipLaunchKernelGGL((k_add_rmsnorm_walk<T, KPT>), dim3(1024), dim3(256), 0, st, (T *)x,
                               (const T *)y, (const T *)w, eps, (T *)out, d, N);
            return;
        }
    }
    hipLaunchKernelGGL((k_add_rmsnorm<T, KPT>), dim3((unsigned)N), dim3(256), 0, st, (T *)x,
                       (const T *)y, (const T *)w, eps, (T *)out, d);
}

template <typename T>
static void add_rmsnorm_t(void *x, const void *y, const void *w, float eps, void *out, int64_t N,
                          int d, hipStream_t st) {
    const int dv = d / (16 / (int)sizeof(T));
    if (dv <= 256) add_rmsnorm_k<T, 1>(x, y, w, eps, out, N, d, st);
    else if (dv <= 512) add_rmsnorm_k<T, 2>(x, y, w, eps, out, N, d, st);
    else if (dv <= 1024) add_rmsnorm_k<T, 4>(x, y, w, eps, out, N, d, st);
    else if (dv <= 2048) add_rmsnorm_k<T, 8>(x, y, w, eps, out, N, d, st);
    else add_rmsnorm_k<T, 0>(x, y, w, eps, out, N, d, st);
}

hipError_t launch_add_rmsnorm(void *x, const void *y, const void *w, float eps, void *out,
                              bool bf16, int64_t N, int d, hipStream_t st) {
    if (bf16) add_rmsnorm_t<bf16_t>(x, y, w, eps, out, N, d, st);
    else add_rmsnorm_t<float>(x, y, w, eps, out, N, d, st);
    return hipGetLastError();
}

template <typename T>
static void tanh_standin_t(const T *u, T *y, int64_t count, hipStream_t st) {
    constexpr int VEC = 16 / sizeof(T);
    const int64_t vecs = count / VEC, done = vecs * VEC;
    if (vecs > 0)
        hipLaunchKernelGGL(k_tanh_standin_vec<T>, dim3(grid_for(vecs, 256, 256 * 64)), dim3(256), 0, st, u, y, vecs);
    if (done < count)
        hipLaunchKernelGGL(k_tanh_standin<T>, dim3(grid_for(count - done, 256, 256 * 64)), dim3(256), 0, st,
                           u + done, y + done, count - done);
}

hipError_t launch_tanh_standin(const void *u, void *y, bool bf16, int64_t count, hipStream_t st) {
    if (bf16) tanh_standin_t((const bf16_t *)u, (bf16_t *)y, count, st);
    else tanh_standin_t((const float *)u, (float *)y, count, st);
    return hipGetLastError();
}

hipError_t launch_copy(const void *src, void *dst, size_t bytes, hipStream_t st) {
    // four workgroups per CU, each thread striding over the whole range: the
    // grid sweeps memory as one narrow front (faster here than many short
    // workgroups or several loads in flight per thread)
    const int64_t vecs = (int64_t)(bytes / 16);
    const unsigned g = grid_for(vecs, 256 * 4, 1024);
    hipLaunchKernelGGL(k_copy, dim3(g), dim3(256), 0, st, (const u32x4 *)src, (u32x4 *)dst, vecs);
    return hipGetLastError();
}

}  // namespace grk
