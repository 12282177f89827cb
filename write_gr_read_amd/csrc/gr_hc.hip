// gr_hc.hip -- Hyper-Connections (HC) and manifold-constrained HC (mHC) on the
// widened state [N][n][d]: read, write, and the fused write + read.
//
// Definitions ("Paper reading: Qwen3.8 Flash Next", part 2 (Residual), sec. 2
// Hyper-Connections: eq:block, eq:mix, eq:combine; "DepthBench", sec. 2.5,
// Block AttnRes and mHC):
//   Rbar_i  = g_i . R_i / rms(R_i)                     per-branch RMSNorm
//   a_ik    = Rbar_i . P_k   (k < n+2; P rows: W_mix, W_comb, then the columns of W_res)
//   HC : H_mix_i = hm_i + lm tanh(a_i0),  H_comb_i = hc_i + lc tanh(a_i1),
//        H_res_ij = hr_ij + lr tanh(a_i,2+j)
//   mHC: H_mix_i = sig(hm_i + lm a_i0),  H_comb_i = 2 sig(hc_i + lc a_i1),
//        H_res = Sinkhorn-Knopp^iters(exp(hr_ij + lr a_i,2+j)) (rows, then columns)
//   x = sum_i H_mix_i R_i,  u = w . x / rms(x)        the block's pre-norm
//   write: R'_i = sum_j H_res_ij R_j + H_comb_i y
// The read hands [H_comb | H_res] (n + n*n fp32 per token) to the write.
//
// Fast kernel (bf16 state, n in {1, 2, 4}, d <= 4096, d % 8 == 0): a team of
// 256 threads per token (two teams per workgroup, one workgroup per CU,
// persistent over tokens), the next token's loads in flight while the current
// one computes.  Thread t of a team holds the 8-channel chunks t + 256 k of
// every branch, so a token's state stays in registers, the gains and the n + 2
// projection rows in LDS, and one pass over the state gives everything:
//   - per-thread fp32 sums over its channels of R_i^2, R_i R_j (the branch Gram
//     matrix) and (g_i R_i) P_k; one cross-lane reduction (lane swaps and DPP
//     row sums), one LDS exchange between the four waves;
//   - rms(x)^2 = sum_ij H_mix_i H_mix_j Gram_ij / d: the sum of x_c^2
//     regrouped, so x needs no second reduction;
//   - Sinkhorn on lanes 0..n*n-1 of one wave (which wave rotates by token),
//     row and column sums by DPP, exp taken after subtracting the row maximum
//     (the first row scaling cancels any per-row factor).
// Everything else (fp32 state, n = 3 or 5..8, d > 4096) runs the generic kernel:
// a workgroup per token, three passes over its channels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gr_device.h"
#include "gr_internal.h"

namespace grk {
namespace {

constexpr int kHcThreads = 256;
enum { kModeHC = 0, kModeMHC = 1 };

// ---- cross-lane helpers (gfx950, wave64) -----------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Sum over the 16 lanes of a row; every lane of the row gets it.
__device__ __forceinline__ float row_total(float v) {
    v += dpp<kRowRor8>(v);
    v += dpp<kRowRor4>(v);
    v += dpp<kRowRor2>(v);
    v += dpp<kRowRor1>(v);
    return v;
}

// a, b -> (a summed over lanes l, l^32) in lanes 0..31, (b summed) in 32..63.
__device__ __forceinline__ float fold32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// a, b -> (a summed over lanes l, l^16) in rows 0 and 2, (b summed) in rows 1 and 3.
__device__ __forceinline__ float fold16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reduce V values (V % 4 == 0) over the 64 lanes of a wave.  On return, every
// lane of row q (lanes 16q..16q+15) holds in out[m] the total of value
// 4 m + 2 (q & 1) + (q >> 1).
template <int V>
__device__ __forceinline__ void wave_reduce_rows(const float (&v)[V], float (&out)[V / 4]) {
    float w[V / 2];
#pragma unroll
    for (int m = 0; m < V / 2; ++m) w[m] = fold32(v[2 * m], v[2 * m + 1]);
#pragma unroll
    for (int m = 0; m < V / 4; ++m) out[m] = row_total(fold16(w[2 * m], w[2 * m + 1]));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                          false);
}

__device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// Row sum / column sum of an n x n matrix held one entry per lane (lane = n i + j)
// in lanes 0..n*n-1 (n = 4: row 0 of the wave; n = 2: quad 0).
template <int NB>
__device__ __forceinline__ float mat_row_sum(float v) {
    if constexpr (NB == 4) {
        v += dpp<kQuadXor1>(v);
        return v + dpp<kQuadXor2>(v);
    } else if constexpr (NB == 2) {
        return v + dpp<kQuadXor1>(v);
    } else {
        return v;
    }
}
template <int NB>
__device__ __forceinline__ float mat_row_max(float v) {
    if constexpr (NB == 4) {
        v = fmaxf(v, dpp<kQuadXor1>(v));
        return fmaxf(v, dpp<kQuadXor2>(v));
    } else if constexpr (NB == 2) {
        return fmaxf(v, dpp<kQuadXor1>(v));
    } else {
        return v;
    }
}
template <int NB>
__device__ __forceinline__ float mat_col_sum(float v) {
    if constexpr (NB == 4) {
        v += dpp<kRowRor8>(v);
        return v + dpp<kRowRor4>(v);
    } else if constexpr (NB == 2) {
        return v + dpp<kQuadXor2>(v);
    } else {
        return v;
    }
}

// ---- fast kernel ----------------------------------------------------------
// A workgroup of 512 threads is two teams of 256; each team takes its own
// token per step (tokens 2p and 2p+1 of pair p), and both teams share the
// read's parameters in LDS (gains, pre-norm gain, projection rows: 88 KiB at
// n = 4, d = 4096), one copy per CU.
constexpr int kHcTeams = 2;
constexpr int kHcFastThreads = kHcTeams * kHcThreads;

template <int NB, int K>
struct HcTok {
    u32x4 R[NB][K];   // state chunks (bf16)
    u32x4 Y[K];       // y chunks (write)
    float C;          // coefficient record, lane l < n + n*n holding entry l (write)
};

// Loads of one token, all unconditional (so the compiler's wait counting stays
// exact across the ping-pong below): a chunk past d/8 loads the last chunk
// and is zeroed after arrival (hc_mask).
template <int NB, int K, bool WRITE>
__device__ __forceinline__ void hc_load(HcTok<NB, K> &t, const bf16_t *__restrict__ S,
                                        const bf16_t *__restrict__ Yp, const float *__restrict__ cin,
                                        int64_t tok, int d, int D8, int ttid) {
    constexpr int NC = NB + NB * NB;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int q = min(ttid + kHcThreads * k, D8 - 1);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            t.R[i][k] = *reinterpret_cast<const u32x4 *>(S + (tok * NB + i) * d + 8 * q);
        if (WRITE) t.Y[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(Yp + tok * d + 8 * q));
    }
    if (WRITE) t.C = cin[tok * NC + min(ttid & 63, NC - 1)];
}

template <int NB, int K>
__device__ __forceinline__ void hc_mask(HcTok<NB, K> &t, int D8, int ttid) {
    if (D8 >= K * kHcThreads) return;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t m = ttid + kHcThreads * k < D8 ? 0xffffffffu : 0u;
#pragma unroll
        for (int i = 0; i < NB; ++i) t.R[i][k] &= m;
        t.Y[k] &= m;
    }
}

__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int NB, int K, int MODE, bool WRITE, bool READ>
__global__ void __launch_bounds__(kHcFastThreads, 1) k_hc_fast(HcArgs a) {
    constexpr int NC = NB + NB * NB;          // coefficient record [H_comb | H_res]
    constexpr int NP = NB + 2;                // projection rows
    constexpr int NG = NB * (NB - 1) / 2;     // off-diagonal Gram entries
    constexpr int V0 = NB + NG + NB * NP;     // values summed per token
    constexpr int V = (V0 + 3) & ~3;
    constexpr int OFF_G = NB, OFF_P = NB + NG;
    constexpr int KC = K * kHcThreads;        // 8-channel chunks covered by a team
    __shared__ f32x4 red[kHcTeams][2][V];     // [team][buffer][value] -> the team's four waves
    __shared__ u32x4 lds_p[READ ? NP : 1][READ ? KC : 1];   // projection rows
    __shared__ u32x4 lds_g[READ ? NB : 1][READ ? KC : 1];   // per-branch gains
    __shared__ u32x4 lds_w[READ ? KC : 1];                  // pre-norm gain

    const int tid = threadIdx.x, team = tid / kHcThreads, ttid = tid % kHcThreads;
    const int lane = tid & 63, wave = ttid >> 6;
    const int d = a.d, D8 = d >> 3;
    const float inv_d = 1.0f / (float)d;
    bf16_t *__restrict__ S = static_cast<bf16_t *>(a.state);
    const bf16_t *__restrict__ Yp = static_cast<const bf16_t *>(a.y);
    const float *__restrict__ cin = a.coeff_in;

    // This lane's coefficient (H_res entry on lanes 0..n*n-1, H_comb entry on
    // lanes 16..16+n-1): its branch, its projection value, its static term and
    // lambda, all fixed for the launch.
    const bool res_lane = lane < NB * NB, comb_lane = lane >= 16 && lane < 16 + NB;
    const int bi = res_lane ? lane / NB : comb_lane ? lane - 16 : 0;
    const int pv = OFF_P + bi * NP + (res_lane ? 2 + lane % NB : 1);
    float hs_lane = 0.f, lam_lane = a.lam_r, hm_s[NB];
    if (comb_lane) lam_lane = a.lam_c;
    if constexpr (READ) {
        const bf16_t *g = static_cast<const bf16_t *>(a.gamma);
        const bf16_t *p = static_cast<const bf16_t *>(a.w_proj);
        const bf16_t *wn = static_cast<const bf16_t *>(a.w_norm);
        for (int q = tid; q < KC; q += kHcFastThreads) {
            const bool ok = q < D8;
#pragma unroll
            for (int i = 0; i < NB; ++i)
                lds_g[i][q] = ok ? *reinterpret_cast<const u32x4 *>(g + i * d + 8 * q) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NP; ++m)
                lds_p[m][q] = ok ? *reinterpret_cast<const u32x4 *>(p + m * d + 8 * q) : u32x4{0, 0, 0, 0};
            lds_w[q] = ok ? *reinterpret_cast<const u32x4 *>(wn + 8 * q) : u32x4{0, 0, 0, 0};
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NB; ++i) hm_s[i] = a.h_static[i];
        if (res_lane) hs_lane = a.h_static[2 * NB + lane];
        else if (comb_lane) hs_lane = a.h_static[NB + lane - 16];
    }

    const int64_t N = a.N;
    auto process = [&](HcTok<NB, K> &cur, const int64_t tok, const bool live, const int it)
                       __attribute__((always_inline)) {
        hc_mask<NB, K>(cur, D8, ttid);
        // ---- write: R'_i = sum_j H_res_ij R_j + H_comb_i y (fp32, one rounding to bf16)
        if constexpr (WRITE) {
            float hc[NB], hr[NB][NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) hc[i] = lane_value(cur.C, i);
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) hr[i][j] = lane_value(cur.C, NB + i * NB + j);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                u32x4 o[NB];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float yl = bf16_lo(cur.Y[k][e]), yh = bf16_hi(cur.Y[k][e]);
                    float rl[NB], rh[NB];
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        rl[j] = bf16_lo(cur.R[j][k][e]);
                        rh[j] = bf16_hi(cur.R[j][k][e]);
                    }
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        float ol = hc[i] * yl, oh = hc[i] * yh;
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            ol = fmaf(hr[i][j], rl[j], ol);
                            oh = fmaf(hr[i][j], rh[j], oh);
                        }
                        o[i][e] = pack_bf16x2(ol, oh);
                    }
                }
                const int q = ttid + kHcThreads * k;
                if (live && q < D8) {
#pragma unroll
                    for (int i = 0; i < NB; ++i)
                        *reinterpret_cast<u32x4 *>(S + (tok * NB + i) * d + 8 * q) = o[i];
                }
#pragma unroll
                for (int i = 0; i < NB; ++i) cur.R[i][k] = o[i];
            }
        }

        if constexpr (READ) {
            // ---- per-thread sums: ss_i, Gram_ij (i < j), (g_i R_i) . P_m
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int q = ttid + kHcThreads * k;
                u32x4 Pw[NP], Gm[NB];
#pragma unroll
                for (int m = 0; m < NP; ++m) Pw[m] = lds_p[m][q];
#pragma unroll
                for (int i = 0; i < NB; ++i) Gm[i] = lds_g[i][q];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
#pragma unroll
                    for (int i = 0; i < NB; ++i) acc[i] = dot2(cur.R[i][k][e], cur.R[i][k][e], acc[i]);
                    {
                        int gidx = OFF_G;
#pragma unroll
                        for (int i = 0; i < NB; ++i)
#pragma unroll
                            for (int j = i + 1; j < NB; ++j, ++gidx)
                                acc[gidx] = dot2(cur.R[i][k][e], cur.R[j][k][e], acc[gidx]);
                    }
                    float pl[NP], ph[NP];
#pragma unroll
                    for (int m = 0; m < NP; ++m) {
                        pl[m] = bf16_lo(Pw[m][e]);
                        ph[m] = bf16_hi(Pw[m][e]);
                    }
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        const float gl = bf16_lo(Gm[i][e]) * bf16_lo(cur.R[i][k][e]);
                        const float gh = bf16_hi(Gm[i][e]) * bf16_hi(cur.R[i][k][e]);
#pragma unroll
                        for (int m = 0; m < NP; ++m) {
                            float &s = acc[OFF_P + i * NP + m];
                            s = fmaf(gl, pl[m], s);
                            s = fmaf(gh, ph[m], s);
                        }
                    }
                }
            }
            // ---- team totals: wave reduction, then the team's four waves through LDS
            float part[V / 4];
            wave_reduce_rows<V>(acc, part);
            const int buf = it & 1, q = lane >> 4;
            if ((lane & 15) == 0) {
#pragma unroll
                for (int m = 0; m < V / 4; ++m)
                    reinterpret_cast<float *>(&red[team][buf][4 * m + 2 * (q & 1) + (q >> 1)])[wave] = part[m];
            }
            __syncthreads();
            auto total = [&](int v) {
                const f32x4 t = red[team][buf][v];
                return (t[0] + t[1]) + (t[2] + t[3]);
            };

            // ---- H_mix and rms(x) (uniform over the team)
            float hm[NB], ss[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                ss[i] = total(i);
                const float am = rsq(ss[i] * inv_d + a.eps) * total(OFF_P + i * NP);
                if constexpr (MODE == kModeHC) hm[i] = hm_s[i] + a.lam_m * tanh_f(am);
                else hm[i] = sigmoid_f(hm_s[i] + a.lam_m * am);
            }
            float xx = 0.f;
#pragma unroll
            for (int i = 0; i < NB; ++i) xx = fmaf(hm[i] * hm[i], ss[i], xx);
            {
                int gidx = OFF_G;
#pragma unroll
                for (int i = 0; i < NB; ++i)
#pragma unroll
                    for (int j = i + 1; j < NB; ++j, ++gidx) xx = fmaf(2.f * hm[i] * hm[j], total(gidx), xx);
            }
            const float rx = rsq(fmaxf(xx, 0.f) * inv_d + a.eps);

            // ---- u = w . x / rms(x)
            bf16_t *U = static_cast<bf16_t *>(a.u);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int qq = ttid + kHcThreads * k;
                const u32x4 wn = lds_w[qq];
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float xl = 0.f, xh = 0.f;
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        xl = fmaf(hm[i], bf16_lo(cur.R[i][k][e]), xl);
                        xh = fmaf(hm[i], bf16_hi(cur.R[i][k][e]), xh);
                    }
                    o[e] = pack_bf16x2(bf16_lo(wn[e]) * (xl * rx), bf16_hi(wn[e]) * (xh * rx));
                }
                if (live && qq < D8) __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(U + tok * d + 8 * qq));
            }

            // ---- H_comb and H_res: one wave of the team, one coefficient per lane
            if (live && wave == (it & 3)) {
                const float arg = rsq(total(bi) * inv_d + a.eps) * total(pv);
                float h;
                if constexpr (MODE == kModeHC) {
                    h = hs_lane + lam_lane * tanh_f(arg);
                } else {
                    if (comb_lane) {
                        h = 2.f * sigmoid_f(hs_lane + lam_lane * arg);
                    } else {
                        float L = res_lane ? hs_lane + lam_lane * arg : 0.f;
                        if (a.iters > 0) L -= mat_row_max<NB>(L);
                        float m = __builtin_amdgcn_exp2f(L * kLog2e);
                        for (int s = 0; s < a.iters; ++s) {
                            m *= __builtin_amdgcn_rcpf(mat_row_sum<NB>(m));
                            m *= __builtin_amdgcn_rcpf(mat_col_sum<NB>(m));
                        }
                        h = m;
                    }
                }
                float *co = a.coeff_out + tok * NC;
                if (res_lane) co[NB + lane] = h;
                else if (comb_lane) co[lane - 16] = h;
            }
        }
    };

    // Pairs of tokens (2p, 2p+1), one per team; both teams take the same number
    // of steps (a team without a token computes on a clamped copy and stores
    // nothing), so every barrier is reached by all eight waves.  Two token
    // buffers, no copies between them: the next pair's loads are in flight while
    // the current one is processed.
    const int64_t pairs = (N + 1) / 2, G = gridDim.x;
    int64_t pr = blockIdx.x;
    auto token_of = [&](int64_t p) { return min(2 * p + team, N - 1); };
    HcTok<NB, K> A, B;
    hc_load<NB, K, WRITE>(A, S, Yp, cin, token_of(pr), d, D8, ttid);
    for (int it = 0;; it += 2) {
        hc_load<NB, K, WRITE>(B, S, Yp, cin, token_of(min(pr + G, pairs - 1)), d, D8, ttid);
        process(A, token_of(pr), 2 * pr + team < N, it);
        if ((pr += G) >= pairs) break;
        hc_load<NB, K, WRITE>(A, S, Yp, cin, token_of(min(pr + G, pairs - 1)), d, D8, ttid);
        process(B, token_of(pr), 2 * pr + team < N, it + 1);
        if ((pr += G) >= pairs) break;
    }
}

// ---- generic kernel: any n <= 8, fp32 or bf16, any d ------------------------
template <typename T, int MODE, bool WRITE, bool READ>
__global__ void __launch_bounds__(kHcThreads) k_hc_generic(HcArgs a) {
    constexpr int MAXN = 8, MAXV = MAXN + MAXN * (MAXN + 2);
    __shared__ float part[kHcThreads / 64][MAXV];
    __shared__ float tot[MAXV + 1];
    __shared__ float coef[MAXN + MAXN + MAXN * MAXN];   // H_mix | H_comb | H_res
    const int n = a.n, d = a.d, np = n + 2, nv = n + n * np, nc = n + n * n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    T *S = static_cast<T *>(a.state);
    const T *Yp = static_cast<const T *>(a.y);
    const T *g = static_cast<const T *>(a.gamma);
    const T *P = static_cast<const T *>(a.w_proj);
    const T *wn = static_cast<const T *>(a.w_norm);
    T *U = static_cast<T *>(a.u);
    for (int64_t tok = blockIdx.x; tok < a.N; tok += gridDim.x) {
        T *Rt = S + tok * n * (int64_t)d;
        if (WRITE) {
            const float *c = a.coeff_in + tok * nc;
            for (int ch = tid; ch < d; ch += kHcThreads) {
                float old[MAXN];
                for (int j = 0; j < n; ++j) old[j] = Store<T>::load(Rt + j * (int64_t)d + ch);
                const float yv = Store<T>::load(Yp + tok * d + ch);
                for (int i = 0; i < n; ++i) {
                    float acc = c[i] * yv;
                    for (int j = 0; j < n; ++j) acc = fmaf(c[n + i * n + j], old[j], acc);
                    Store<T>::store(Rt + i * (int64_t)d + ch, acc);
                }
            }
        }
        if (!READ) continue;
        // sums over channels: ss_i and (g_i R_i) . P_m (each thread reads back what it wrote)
        float acc[MAXV];
        for (int v = 0; v < nv; ++v) acc[v] = 0.f;
        for (int ch = tid; ch < d; ch += kHcThreads) {
            for (int i = 0; i < n; ++i) {
                const float r = Store<T>::load(Rt + i * (int64_t)d + ch);
                acc[i] = fmaf(r, r, acc[i]);
                const float gr = Store<T>::load(g + i * (int64_t)d + ch) * r;
                for (int m = 0; m < np; ++m)
                    acc[n + i * np + m] = fmaf(gr, Store<T>::load(P + m * (int64_t)d + ch), acc[n + i * np + m]);
            }
        }
        for (int v = 0; v < nv; ++v) {
            const float w = wave_sum(acc[v]);
            if (lane == 0) part[wave][v] = w;
        }
        __syncthreads();
        if (tid < nv) {
            float t = 0.f;
            for (int w = 0; w < kHcThreads / 64; ++w) t += part[w][tid];
            tot[tid] = t;
        }
        __syncthreads();
        if (tid == 0) {
            const float *hs = a.h_static;
            float rho[MAXN];
            for (int i = 0; i < n; ++i) rho[i] = rsq(tot[i] / (float)d + a.eps);
            for (int i = 0; i < n; ++i) {
                const float am = rho[i] * tot[n + i * np], ac = rho[i] * tot[n + i * np + 1];
                if (MODE == kModeHC) {
                    coef[i] = hs[i] + a.lam_m * tanh_f(am);
                    coef[n + i] = hs[n + i] + a.lam_c * tanh_f(ac);
                } else {
                    coef[i] = sigmoid_f(hs[i] + a.lam_m * am);
                    coef[n + i] = 2.f * sigmoid_f(hs[n + i] + a.lam_c * ac);
                }
                for (int j = 0; j < n; ++j) {
                    const float ar = rho[i] * tot[n + i * np + 2 + j];
                    coef[2 * n + i * n + j] = MODE == kModeHC ? hs[2 * n + i * n + j] + a.lam_r * tanh_f(ar)
                                                              : hs[2 * n + i * n + j] + a.lam_r * ar;
                }
            }
            if (MODE == kModeMHC) {
                float *M = coef + 2 * n;
                for (int i = 0; i < n; ++i) {
                    float mx = -INFINITY;
                    for (int j = 0; j < n; ++j) mx = fmaxf(mx, M[i * n + j]);
                    for (int j = 0; j < n; ++j)
                        M[i * n + j] = __builtin_amdgcn_exp2f((M[i * n + j] - (a.iters > 0 ? mx : 0.f)) * kLog2e);
                }
                for (int s = 0; s < a.iters; ++s) {
                    for (int i = 0; i < n; ++i) {
                        float r = 0.f;
                        for (int j = 0; j < n; ++j) r += M[i * n + j];
                        r = __builtin_amdgcn_rcpf(r);
                        for (int j = 0; j < n; ++j) M[i * n + j] *= r;
                    }
                    for (int j = 0; j < n; ++j) {
                        float c = 0.f;
                        for (int i = 0; i < n; ++i) c += M[i * n + j];
                        c = __builtin_amdgcn_rcpf(c);
                        for (int i = 0; i < n; ++i) M[i * n + j] *= c;
                    }
                }
            }
        }
        __syncthreads();
        if (tid < nc) a.coeff_out[tok * nc + tid] = coef[n + tid];
        // x = sum_i H_mix_i R_i, its mean square, then u
        float xs = 0.f;
        for (int ch = tid; ch < d; ch += kHcThreads) {
            float x = 0.f;
            for (int i = 0; i < n; ++i) x = fmaf(coef[i], Store<T>::load(Rt + i * (int64_t)d + ch), x);
            xs = fmaf(x, x, xs);
        }
        xs = wave_sum(xs);
        if (lane == 0) part[wave][0] = xs;
        __syncthreads();
        if (tid == 0) {
            float t = 0.f;
            for (int w = 0; w < kHcThreads / 64; ++w) t += part[w][0];
            tot[MAXV] = rsq(t / (float)d + a.eps);
        }
        __syncthreads();
        const float rx = tot[MAXV];
        for (int ch = tid; ch < d; ch += kHcThreads) {
            float x = 0.f;
            for (int i = 0; i < n; ++i) x = fmaf(coef[i], Store<T>::load(Rt + i * (int64_t)d + ch), x);
            Store<T>::store(U + tok * d + ch, Store<T>::load(wn + ch) * (x * rx));
        }
        __syncthreads();   // part / tot / coef are reused by the next token
    }
}

int hc_grid(int64_t N, int per_cu) {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
    }
    const int64_t g = (int64_t)cus * per_cu;
    return (int)(N < g ? N : g);
}

template <int NB, int K, int MODE>
hipError_t launch_fast_mode(const HcArgs &a, hipStream_t st) {
    const dim3 grid(hc_grid((a.N + 1) / 2, 1)), block(kHcFastThreads);
    if (a.do_write && a.do_read) hipLaunchKernelGGL((k_hc_fast<NB, K, MODE, true, true>), grid, block, 0, st, a);
    else if (a.do_read) hipLaunchKernelGGL((k_hc_fast<NB, K, MODE, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_hc_fast<NB, K, kModeHC, true, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int NB, int K>
hipError_t launch_fast_k(const HcArgs &a, hipStream_t st) {
    return a.mode == kModeMHC ? launch_fast_mode<NB, K, kModeMHC>(a, st) : launch_fast_mode<NB, K, kModeHC>(a, st);
}

template <int NB>
hipError_t launch_fast_nb(const HcArgs &a, hipStream_t st) {
    return a.d <= 8 * kHcThreads ? launch_fast_k<NB, 1>(a, st) : launch_fast_k<NB, 2>(a, st);
}

template <typename T, int MODE>
hipError_t launch_generic_mode(const HcArgs &a, hipStream_t st) {
    const dim3 grid(hc_grid(a.N, 4)), block(kHcThreads);
    if (a.do_write && a.do_read) hipLaunchKernelGGL((k_hc_generic<T, MODE, true, true>), grid, block, 0, st, a);
    else if (a.do_read) hipLaunchKernelGGL((k_hc_generic<T, MODE, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_hc_generic<T, kModeHC, true, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_generic_t(const HcArgs &a, hipStream_t st) {
    return a.mode == kModeMHC ? launch_generic_mode<T, kModeMHC>(a, st) : launch_generic_mode<T, kModeHC>(a, st);
}

}  // namespace

bool hc_fast_ok(const HcArgs &a) {
    return a.bf16 && (a.n == 1 || a.n == 2 || a.n == 4) && a.d % 8 == 0 && a.d <= 2 * 8 * kHcThreads;
}

hipError_t launch_hc(const HcArgs &a, hipStream_t st, bool force_generic) {
    if (a.N <= 0) return hipSuccess;
    if (!force_generic && hc_fast_ok(a)) {
        switch (a.n) {
        case 1: return launch_fast_nb<1>(a, st);
        case 2: return launch_fast_nb<2>(a, st);
        default: return launch_fast_nb<4>(a, st);
        }
    }
    return a.bf16 ? launch_generic_t<bf16_t>(a, st) : launch_generic_t<float>(a, st);
}

}  // namespace grk
