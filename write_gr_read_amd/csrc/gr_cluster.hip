// gr_cluster.hip -- single-pass GR read and fused write+read for a bf16 or
// e4m3 widened state with n = 4 ("Paper reading: Qwen3.8 Flash Next", part 2
// Residual, sec. 4: eq:write, eq:rms, eq:gate, eq:use_gate, eq:s; sec. 7: the
// read and the write each one traversal of the state).
//
// The gate couples every channel of a token (z contracts all n*d values of
// vec(R-hat), and each u_c needs z), so a kernel that owns whole tokens must
// either hold 32 KB of R' per token on chip or read R' twice.  Here the
// channels are split instead: the 32 workgroups on one XCD (a "cluster", one
// workgroup per CU, blockIdx % 8 = XCD under round-robin dispatch) each own
// CW = d/32 channels of all n = 4 branches, keep the weight slices of those
// channels in registers for the whole launch, and walk the cluster's token
// tiles (TOK tokens each) together.  Per tile a workgroup
//   S  streams its slice once: R' = R + s y (one fp32 FMA, rounded to the
//      state dtype, stored), R' kept in LDS, partial sums of squares;
//   M  projects its slice: P_i = W^(i) (gamma_i . R'_i) for the W_down rows
//      and the W_write rows (MFMA, gamma . R' split into bf16 hi + lo; with
//      eight waves, two waves share a branch, each taking half its channels);
//   Q  gathers every member's sums of squares -> rho_i, and publishes
//      Q = sum_i rho_i P_i (one row per W_down / W_write row);
//   R  reduces, for the token(s) it owns, the members' Q rows ->
//      z = Q/n, a = SiLU(z) (published), s = 2 sigmoid(Q_write / n) (stored);
//   C  gathers a for the tile, forms its channels' gate logits (MFMA up
//      projection from resident W_up rows), G = sigmoid, and
//      u_c = (1/n) sum_i G_ic gamma_ic rho_i R'_ic from the R' still in LDS.
// The stages of consecutive tiles are software-pipelined over three tiles,
// iteration k running R(k-2), S(k), M(k-1), Q(k-1), C(k-2), so every wait on
// the other members comes at least a stage, mostly a whole iteration, after
// the values it waits for were published (the walk below).
//
// Exchange.  Values cross workgroups as 8-byte records (value bits, tag) in a
// library-owned device array (`exchange`); a record is valid when its tag is
// the one expected for that tile of this call, so no flag, fence or memory
// count wait orders the data: each aligned 8-byte record is written and read
// whole.  Writers use ordinary stores (written through the CU's L1 into the
// XCD's L2); readers poll with device-scope (L1-bypassing) loads.  A
// workgroup that finds itself on another XCD than blockIdx % 8 writes its
// records with device-scope stores instead, so the protocol stays correct
// whatever the placement.  Tags are epoch + tile + 1, the epoch of a cluster
// advanced on the device by the last member to finish a call (so replays of
// a captured graph get fresh tags too).  Every wait is bounded: on time-out a
// device error word is set and the call's results are not to be trusted.
//
// The launch must have all 32 workgroups of every cluster resident at once:
// 256 workgroups (512 threads for 128-channel slices, 256 for 64-channel
// ones) with ~150 KB / ~100 KB of LDS, one per CU, on a GPU with 8 XCDs of 32
// CUs; the host checks this before choosing the path, and calls of this path
// on one GPU are serialised by the host (they share the array).
#include "gr_device.h"
#include "gr_internal.h"

#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <type_traits>

namespace grk {
namespace cluster {

constexpr int kMembers = 32;     // workgroups per cluster (CUs per XCD)
// workgroup size: 8 waves (two per SIMD, 256 registers each) for 128-channel
// slices, 4 waves (one per SIMD) for 64-channel slices
constexpr int waves_of(int cw) { return cw == 128 ? 8 : 4; }
constexpr int threads_of(int cw) { return 64 * waves_of(cw); }
constexpr int kMaxClusters = 8;
constexpr int kMaxNRB = 5;       // projection rows r + nw <= 80 (16-row MFMA blocks)
constexpr int kMaxRKS = 2;       // gate rank r <= 64 (32-wide MFMA k-steps)

// exchange layout: control words, then per cluster the ss / Q / act rings
// (two slots each) of 8-byte records, sized for TOK * rows <= 2304 and
// TOK * 32*rks <= 2048.
constexpr size_t kCtlBytes = 256;                                   // epoch[8], done[8], err
constexpr size_t kSsBytes = 2ull * 64 * kMembers * 4 * 8;           // [slot][t][member][4]
constexpr size_t kQBytes = 2ull * 2304 * kMembers * 8;              // [slot][t][member][rows]
constexpr size_t kActBytes = 2ull * 2048 * 8;                       // [slot][t][rk]
constexpr size_t kClusterBytes = kSsBytes + kQBytes + kActBytes;
constexpr size_t kExchangeBytes = kCtlBytes + kMaxClusters * kClusterBytes;

// The exchange array: one copy per GPU, zero at load (tag 0 is never valid).
static __device__ __align__(256) unsigned char exchange[kExchangeBytes];

struct KArgs {
    void *state;
    const bf16_t *y;
    const float *s_in;
    const bf16_t *gamma, *wd, *ww, *wu;
    bf16_t *u;
    float *s_out;
    unsigned char *xs;       // the device's `exchange` (from hipGetSymbolAddress)
    int64_t N;
    int d, r, nw, rows, nrb, rks, tiles, ncl;
    float eps;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t xrsrc(unsigned char *p) {
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)kExchangeBytes, 0x00020000);
}
// device-scope (L1-bypassing) 16- and 8-byte loads of the exchange
__device__ __forceinline__ u32x4 xload16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 16));
}
__device__ __forceinline__ u32x2 xload8(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 16));
}
// record stores: ordinary (same-XCD L2) or device scope
__device__ __forceinline__ void xstore16(__amdgpu_buffer_rsrc_t rs, unsigned char *base, uint32_t off, u32x4 v,
                                         bool dev) {
    if (dev) __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, 16);
    else *reinterpret_cast<u32x4 *>(base + off) = v;
}
__device__ __forceinline__ void xstore8(__amdgpu_buffer_rsrc_t rs, unsigned char *base, uint32_t off, u32x2 v,
                                        bool dev) {
    if (dev) __builtin_amdgcn_raw_buffer_store_b64(v, rs, (int)off, 0, 16);
    else *reinterpret_cast<u32x2 *>(base + off) = v;
}

constexpr int kSpinLimit = 1 << 20;   // polls per wait (about a second) before giving up
__device__ __forceinline__ void report_timeout(unsigned char *xs) {
    __hip_atomic_fetch_or(reinterpret_cast<uint32_t *>(xs + 128), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bf16x8 as_b8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
// c + lo^2 + hi^2 of a packed bf16 pair (v_dot2 with fp32 accumulation)
__device__ __forceinline__ float sq2(uint32_t w, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 h = __builtin_bit_cast(bf16x2, w);
    return __builtin_amdgcn_fdot2_f32_bf16(h, h, c, false);
}

// s_waitcnt immediate waiting until at most n vector memory operations are
// outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14; exp and lgkm counts
// left at their maxima)
constexpr unsigned vmcnt_imm(unsigned n) { return (n & 15u) | ((n >> 4) & 3u) << 14 | 7u << 4 | 15u << 8; }
static_assert(vmcnt_imm(0) == 0x0F70 && vmcnt_imm(16) == 0x4F70, "s_waitcnt vmcnt encoding");

template <bool F8> struct St { using T = bf16_t; using V = u32x4; };
template <> struct St<true> { using T = fp8_t; using V = u32x2; };

template <int CW, bool FUSED>
__global__ void __launch_bounds__(threads_of(CW), 1) k_cluster(KArgs a) {
    constexpr bool F8 = false;
    constexpr int WAVES = waves_of(CW);
    constexpr int kThreads = threads_of(CW);
    constexpr int WPB = WAVES / 4;         // waves per branch in the down projection
    constexpr int PCS = CW / 8;            // 8-channel pieces per (token, branch) of a slice
    constexpr int TOK = 32;                // tokens per tile
    constexpr int SJ = TOK * PCS / kThreads;  // (token, piece) pairs per thread in stage S (1 or 2)
    constexpr int KS = CW / 32;            // MFMA k-steps per branch slice
    constexpr int KSW = KS / WPB;          // ... per wave (the wave's part of its branch's channels)
    constexpr int CWW = CW / WAVES;        // channels per wave in the up projection and combine
    constexpr int NTG = TOK / 16;          // 16-token MFMA column groups per tile
    constexpr int NB2 = CWW / 4;           // up-projection row blocks per wave (4 branches x CWW channels)
    constexpr int PR = 4 * CW * 2 + 16;    // LDS bytes per token of an R' tile (padded: conflict-free MFMA reads)
    constexpr int RKM = 64;                // act columns per token (gate rank <= 64)
    constexpr int AP = RKM * 2 + 16;       // LDS bytes per token of an act plane
    constexpr int SPX = 72;                // staging floats per (branch, token): rows (<= 68) + padding
    constexpr int QI = kThreads / 128;     // reduction items per projection row (QI rows <= kThreads)
    constexpr int QM = kMembers / QI;      // members summed per reduction item
    constexpr int TPT = kThreads / TOK;    // threads per token when publishing the projections
    constexpr int NSS = TOK * kMembers / kThreads;  // (token, member) sum-of-squares records per thread
    constexpr int NAI = TOK * (RKM / 2) / kThreads; // act record pairs per thread
    static_assert(SJ >= 1 && NSS >= 1 && NAI >= 1 && KSW >= 1 && NB2 >= 1 && QI * QM == kMembers, "tile shape");
    using T = typename St<F8>::T;
    using SV = typename St<F8>::V;

    // ---- LDS
    constexpr int kRBytes = 3 * TOK * PR;          // three R' tiles (written, projected, combined)
    constexpr int kRhoBytes = 3 * TOK * 16;
    constexpr int kStgBytes = 4 * TOK * SPX * 4;
    constexpr int kRedBytes = QI * SPX * 4;
    constexpr int kActL = 2 * TOK * AP;
    static_assert(kStgBytes >= TOK * kMembers * 16, "the sums-of-squares gather shares the staging area");
    __shared__ __attribute__((aligned(16))) unsigned char
        lds[kRBytes + kRhoBytes + kStgBytes + kRedBytes + kActL + 4 * CW * 2];
    unsigned char *const Rl = lds;
    float *const rhol = reinterpret_cast<float *>(lds + kRBytes);
    float *const stg = reinterpret_cast<float *>(lds + kRBytes + kRhoBytes);
    float *const red = reinterpret_cast<float *>(lds + kRBytes + kRhoBytes + kStgBytes);
    unsigned char *const actl = lds + kRBytes + kRhoBytes + kStgBytes + kRedBytes;
    bf16_t *const gml = reinterpret_cast<bf16_t *>(actl + kActL);
    __shared__ int aborted_;   // a wait of this workgroup timed out: later waits give up at once
    volatile int *const aborted = &aborted_;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int ncl = a.ncl;
    const int x = (int)(blockIdx.x % ncl), member = (int)(blockIdx.x / ncl);
    const int d = a.d, r = a.r, rows = a.rows, nrb = a.nrb, rks = a.rks;
    const int64_t nd = 4 * (int64_t)d;
    const int c0 = member * CW;
    unsigned char *const xs = a.xs;
    const __amdgpu_buffer_rsrc_t rs = xrsrc(xs);
    const bool devw = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15) != x || ncl != 8;
    const uint32_t xbase = (uint32_t)(kCtlBytes + (size_t)x * kClusterBytes);
    const uint32_t ss_off = xbase, q_off = xbase + (uint32_t)kSsBytes, act_off = q_off + (uint32_t)kQBytes;
    const int K = x < a.tiles ? (a.tiles - x + ncl - 1) / ncl : 0;   // this cluster's tiles
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(reinterpret_cast<uint32_t *>(xs) + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    auto tag_of = [&](int k) __attribute__((always_inline)) { return epoch + (uint32_t)k + 1u; };
    auto tok0_of = [&](int k) __attribute__((always_inline)) { return (int64_t)(x + (int64_t)k * ncl) * TOK; };
    const float inv_n = 0.25f;
    const int64_t Nm1 = a.N - 1;

    // ---- resident operands
    // gains of the slice (LDS, bf16), for the down projection's B side and the combine
    for (int e = tid; e < 4 * CW / 8; e += kThreads) {
        const int i = e / PCS, q = e % PCS;
        *reinterpret_cast<u32x4 *>(gml + i * CW + 8 * q) =
            *reinterpret_cast<const u32x4 *>(a.gamma + (int64_t)i * d + c0 + 8 * q);
    }
    // down projection A fragments: wave = (branch bi, part kp of its channels);
    // row j = 16 blk + l16 of (W_down ; W_write ; 0), k = channels
    // c0 + 32 (KSW kp + ks) + 8 g .. + 7 of branch bi
    const int bi = wave / WPB, kp = wave % WPB;
    u32x4 af[kMaxNRB][KSW];
#pragma unroll
    for (int blk = 0; blk < kMaxNRB; ++blk) {
        const int j = 16 * blk + l16;
        const bf16_t *src = j < r ? a.wd + (int64_t)j * nd : (j < rows ? a.ww + (int64_t)(j - r) * nd : nullptr);
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
            af[blk][ks] = u32x4{0u, 0u, 0u, 0u};
            if (src && blk < nrb)
                af[blk][ks] = *reinterpret_cast<const u32x4 *>(src + (int64_t)bi * d + c0 + 32 * (KSW * kp + ks) + 8 * g);
        }
    }
    // up projection A fragments: wave w owns local channels w*CWW .. + CWW - 1; block b,
    // row 4 g' + m (g' = l16 / 4, m = l16 % 4) is (branch m, channel NB2 g' + b of the
    // wave), k = 32 ks + 8 g .. + 7 (zero at k >= r)
    u32x4 au[NB2][kMaxRKS];
    {
        const int gp = l16 >> 2, m = l16 & 3;
#pragma unroll
        for (int b = 0; b < NB2; ++b) {
            const int ch = c0 + wave * CWW + NB2 * gp + b;
            const bf16_t *src = a.wu + ((int64_t)m * d + ch) * r;
#pragma unroll
            for (int ks = 0; ks < kMaxRKS; ++ks) {
                u32x4 v = {0u, 0u, 0u, 0u};
                const int k0 = 32 * ks + 8 * g;
                if (ks < rks && k0 < r) v = *reinterpret_cast<const u32x4 *>(src + k0);
                au[b][ks] = v;
            }
        }
    }

    // ---- loads of tile k into registers: this thread's (token, piece) pairs
    // p = tid + kThreads j (tokens past the end read the last token; unused)
    u32x4 pr[SJ][4], py[SJ];
    f32x4 psv[SJ];
    auto prefetch = [&](int k) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < SJ; ++j) {
            const int p = tid + kThreads * j, t = p / PCS, q = p % PCS;
            int64_t tok = tok0_of(k) + t;
            tok = tok < Nm1 ? tok : Nm1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pr[j][i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const T *>(a.state) + (tok * 4 + i) * (int64_t)d + c0 + 8 * q);
            if (FUSED) {
                py[j] = *reinterpret_cast<const u32x4 *>(a.y + tok * d + c0 + 8 * q);
                psv[j] = *reinterpret_cast<const f32x4 *>(a.s_in + tok * 4);
            }
        }
    };
    // ---- stage S: R' = R + s y (stored), into the tile's LDS slot; sums of squares
    auto stage_S = [&](int k) __attribute__((always_inline)) {
        const uint32_t tg = tag_of(k);
#pragma unroll
        for (int j = 0; j < SJ; ++j) {
            const int p = tid + kThreads * j, t = p / PCS, q = p % PCS;
            const int64_t tok = tok0_of(k) + t;
            const bool v = tok < a.N;
            unsigned char *slot = Rl + (k % 3) * TOK * PR + t * PR;
            float ss[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 w = pr[j][i];
                if (FUSED) {
                    w = write8_bf16(psv[j][i], py[j], pr[j][i]);
                    if (v) *reinterpret_cast<u32x4 *>(reinterpret_cast<T *>(a.state) + (tok * 4 + i) * (int64_t)d + c0 + 8 * q) = w;
                }
                if (!v) w = u32x4{0u, 0u, 0u, 0u};   // a token past the end contributes zeros
                *reinterpret_cast<u32x4 *>(slot + i * CW * 2 + 16 * q) = w;
                float s_ = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) s_ = sq2(w[e], s_);
                ss[i] = s_;
            }
            // sum over the PCS lanes of the token (fixed butterfly)
#pragma unroll
            for (int msk = 1; msk < PCS; msk <<= 1)
#pragma unroll
                for (int i = 0; i < 4; ++i) ss[i] += __shfl_xor(ss[i], msk, 64);
            if (q == 0) {
                const uint32_t off = ss_off + (uint32_t)((((k & 1) * TOK + t) * kMembers + member) * 32);
                xstore16(rs, xs, off, u32x4{__float_as_uint(ss[0]), tg, __float_as_uint(ss[1]), tg}, devw);
                xstore16(rs, xs, off + 16, u32x4{__float_as_uint(ss[2]), tg, __float_as_uint(ss[3]), tg}, devw);
            }
        }
    };

    // ---- stage M: down projection of the wave's channels of branch bi for every
    // token group of tile k
    f32x4 pacc[NTG][kMaxNRB];
    auto stage_M = [&](int k) __attribute__((always_inline)) {
        const unsigned char *slot = Rl + (k % 3) * TOK * PR;
#pragma unroll
        for (int tgp = 0; tgp < NTG; ++tgp) {
#pragma unroll
            for (int blk = 0; blk < kMaxNRB; ++blk) pacc[tgp][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int t = 16 * tgp + l16;
#pragma unroll
            for (int ks = 0; ks < KSW; ++ks) {
                const int kg = KSW * kp + ks;
                const u32x4 rv = *reinterpret_cast<const u32x4 *>(slot + t * PR + bi * CW * 2 + (32 * kg + 8 * g) * 2);
                const u32x4 gv = *reinterpret_cast<const u32x4 *>(gml + bi * CW + 32 * kg + 8 * g);
                u32x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = bf16_lo(rv[e]) * bf16_lo(gv[e]);
                    const float x1 = bf16_hi(rv[e]) * bf16_hi(gv[e]);
                    hi[e] = pack_bf16x2(x0, x1);
                    lo[e] = pack_bf16x2(x0 - bf16_lo(hi[e]), x1 - bf16_hi(hi[e]));
                }
#pragma unroll
                for (int blk = 0; blk < kMaxNRB; ++blk) {
                    if (blk < nrb) {
                        pacc[tgp][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(af[blk][ks]), as_b8(hi), pacc[tgp][blk], 0, 0, 0);
                        pacc[tgp][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(af[blk][ks]), as_b8(lo), pacc[tgp][blk], 0, 0, 0);
                    }
                }
            }
        }
    };

    // re-poll a record pair until both tags are `tg` (v holds the first read)
    auto settle16 = [&](u32x4 &v, uint32_t off, uint32_t tg) __attribute__((always_inline)) {
        int spins = 0;
        while (!(v.y == tg && v.w == tg)) {
            if (++spins > kSpinLimit || *aborted) {
                *aborted = 1;
                report_timeout(xs);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            v = xload16(rs, off);
        }
    };

    // ---- stage Q, first half: loads of every member's sums of squares [t][member][4]
    u32x4 ssv[NSS][2];
    auto ss_off_of = [&](int k, int p) __attribute__((always_inline)) {
        const int t = p / kMembers, m = p % kMembers;
        return ss_off + (uint32_t)((((k & 1) * TOK + t) * kMembers + m) * 32);
    };
    auto issue_ss = [&](int k) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NSS; ++j) {
            const uint32_t off = ss_off_of(k, tid + kThreads * j);
            ssv[j][0] = xload16(rs, off);
            ssv[j][1] = xload16(rs, off + 16);
        }
    };
    // ---- stage Q: rho of the tile, then this member's rows Q = sum_i rho_i P_i
    auto stage_Q = [&](int k) __attribute__((always_inline)) {
        const uint32_t tg = tag_of(k);
#pragma unroll
        for (int j = 0; j < NSS; ++j) {
            const int p = tid + kThreads * j;
            settle16(ssv[j][0], ss_off_of(k, p), tg);
            settle16(ssv[j][1], ss_off_of(k, p) + 16, tg);
            *reinterpret_cast<u32x4 *>(stg + p * 4) = u32x4{ssv[j][0].x, ssv[j][0].z, ssv[j][1].x, ssv[j][1].z};
        }
        __syncthreads();
        for (int e = tid; e < TOK * 4; e += kThreads) {
            const int t = e >> 2, i = e & 3;
            float ss = 0.f;
            // members in a rotated order (fixed per token): the lanes of a wave then
            // read different LDS banks
            for (int m = 0; m < kMembers; ++m) ss += stg[(t * kMembers + ((m + t) & (kMembers - 1))) * 4 + i];
            rhol[(k % 3) * TOK * 4 + e] = 1.0f / sqrtf(ss / (float)d + a.eps);
        }
        __syncthreads();
        // scaled partials to the staging area [branch][t][row]; where two waves
        // share a branch, the second writes and the first adds its own after a
        // barrier (a + b: the same value in either order)
        auto stage_partials = [&](bool add) __attribute__((always_inline)) {
#pragma unroll
            for (int tgp = 0; tgp < NTG; ++tgp) {
                const int t = 16 * tgp + l16;
                const float rho = rhol[(k % 3) * TOK * 4 + t * 4 + bi];
#pragma unroll
                for (int blk = 0; blk < kMaxNRB; ++blk) {
                    const int row = 16 * blk + 4 * g;
                    if (blk < nrb && row < rows) {
                        f32x4 *dst = reinterpret_cast<f32x4 *>(stg + (bi * TOK + t) * SPX + row);
                        const f32x4 v = pacc[tgp][blk] * rho;
                        *dst = add ? *dst + v : v;
                    }
                }
            }
        };
        if constexpr (WPB == 1) {
            stage_partials(false);
        } else {
            static_assert(WPB == 2, "two waves per branch");
            if (kp == 1) stage_partials(false);
            __syncthreads();
            if (kp == 0) stage_partials(true);
        }
        __syncthreads();
        // sum over branches (in order), publish as records [slot][t][member][rows]
        static_assert(TOK * TPT == kThreads, "publish mapping: TPT threads per token");
        const int t = tid / TPT;
        for (int v = 2 * (tid % TPT); v < rows; v += 2 * TPT) {
            float q0 = 0.f, q1 = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                q0 += stg[(i * TOK + t) * SPX + v];
                q1 += stg[(i * TOK + t) * SPX + v + 1];
            }
            const uint32_t off = q_off + (uint32_t)(((((k & 1) * TOK + t) * kMembers + member) * rows + v) * 8);
            xstore16(rs, xs, off, u32x4{__float_as_uint(q0), tg, __float_as_uint(q1), tg}, devw);
        }
    };

    // ---- stage R, first half: loads of the members' Q rows for this member's token;
    // item tid = (part h, row v) sums members QM h .. QM h + QM - 1 (QI rows items <= kThreads)
    u32x2 qv[QM];
    const int nqi = QI * rows;
    const int qi_v = tid < nqi ? tid % rows : 0, qi_h = tid < nqi ? tid / rows : 0;   // once per launch
    const uint32_t qi_base = (uint32_t)(((member * kMembers + QM * qi_h) * rows + qi_v) * 8);
    const uint32_t qi_mstride = (uint32_t)(rows * 8);
    auto q_off_of = [&](int k, int m) __attribute__((always_inline)) {
        return q_off + (uint32_t)(((k & 1) * TOK * kMembers * rows) * 8) + qi_base + (uint32_t)m * qi_mstride;
    };
    auto issue_q = [&](int k) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < QM; ++m) qv[m] = xload8(rs, q_off_of(k, m));
    };
    // ---- stage R: this member's token of tile k: z, a = SiLU(z), s
    auto stage_R = [&](int k) __attribute__((always_inline)) {
        const uint32_t tg = tag_of(k);
        if (tid < nqi) {
            float sum = 0.f;
#pragma unroll
            for (int m = 0; m < QM; ++m) {
                int spins = 0;
                while (qv[m].y != tg) {
                    if (++spins > kSpinLimit || *aborted) { *aborted = 1; report_timeout(xs); break; }
                    __builtin_amdgcn_s_sleep(1);
                    qv[m] = xload8(rs, q_off_of(k, m));
                }
                sum += __uint_as_float(qv[m].x);
            }
            red[qi_h * SPX + qi_v] = sum;
        }
        __syncthreads();
        const int64_t tok = tok0_of(k) + member;
        if (tid < rows) {
            const int v = tid;
            float q = red[v];
#pragma unroll
            for (int h = 1; h < QI; ++h) q += red[h * SPX + v];
            if (v < r) {
                const float av = -kLog2e * silu_f(q * inv_n);
                const uint32_t off = act_off + (uint32_t)((((k & 1) * TOK + member) * RKM + v) * 8);
                xstore8(rs, xs, off, u32x2{__float_as_uint(av), tg}, devw);
            } else if (tok < a.N) {
                a.s_out[tok * 4 + (v - r)] = 2.0f * sigmoid_f(q * inv_n);
            }
        }
        if (a.nw == 0 && tid < 4 && tok < a.N) a.s_out[tok * 4 + tid] = 1.0f;
    };

    // ---- stage C, first half: loads of a for the tile ([t][v] record pairs)
    u32x4 av_[NAI];
    auto act_off_of = [&](int k, int e) __attribute__((always_inline)) {
        const int t = e / (RKM / 2);
        int v = 2 * (e % (RKM / 2));
        v = v < r ? v : 0;   // columns past the gate rank read a valid record, unused
        return act_off + (uint32_t)((((k & 1) * TOK + t) * RKM + v) * 8);
    };
    auto issue_act = [&](int k) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NAI; ++j) av_[j] = xload16(rs, act_off_of(k, tid + kThreads * j));
    };
    // ---- stage C: up projection, gate and combine of tile k
    auto stage_C = [&](int k) __attribute__((always_inline)) {
        const uint32_t tg = tag_of(k);
#pragma unroll
        for (int j = 0; j < NAI; ++j) {
            const int e = tid + kThreads * j;
            const int t = e / (RKM / 2), v = 2 * (e % (RKM / 2));
            float a0 = 0.f, a1 = 0.f;
            if (v < r) {
                settle16(av_[j], act_off_of(k, e), tg);
                a0 = __uint_as_float(av_[j].x);
                a1 = __uint_as_float(av_[j].z);
            }
            const uint32_t h = pack_bf16x2(a0, a1);
            const uint32_t l = pack_bf16x2(a0 - bf16_lo(h), a1 - bf16_hi(h));
            *reinterpret_cast<uint32_t *>(actl + t * AP + v * 2) = h;
            *reinterpret_cast<uint32_t *>(actl + TOK * AP + t * AP + v * 2) = l;
        }
        __syncthreads();
        const unsigned char *slot = Rl + (k % 3) * TOK * PR;
        const int64_t tok0 = tok0_of(k);
        const int cl = wave * CWW + NB2 * g;          // this lane's first local channel
#pragma unroll
        for (int tgp = 0; tgp < NTG; ++tgp) {
            const int t = 16 * tgp + l16;
            u32x4 bh[kMaxRKS], bl[kMaxRKS];
#pragma unroll
            for (int ks = 0; ks < kMaxRKS; ++ks) {
                bh[ks] = bl[ks] = u32x4{0u, 0u, 0u, 0u};
                if (ks < rks) {
                    bh[ks] = *reinterpret_cast<const u32x4 *>(actl + t * AP + (32 * ks + 8 * g) * 2);
                    bl[ks] = *reinterpret_cast<const u32x4 *>(actl + TOK * AP + t * AP + (32 * ks + 8 * g) * 2);
                }
            }
            f32x4 tl[NB2];
#pragma unroll
            for (int b = 0; b < NB2; ++b) {
                tl[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < kMaxRKS; ++ks)
                    if (ks < rks) {
                        tl[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(au[b][ks]), as_b8(bh[ks]), tl[b], 0, 0, 0);
                        tl[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(au[b][ks]), as_b8(bl[ks]), tl[b], 0, 0, 0);
                    }
            }
            const f32x4 rho = *reinterpret_cast<const f32x4 *>(rhol + (k % 3) * TOK * 4 + t * 4);
            float uo[NB2];
#pragma unroll
            for (int b = 0; b < NB2; ++b) uo[b] = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // R' and gains of branch m at channels cl .. cl + NB2 - 1
                float rv[NB2], gv[NB2];
                if constexpr (NB2 == 8) {
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(slot + t * PR + (m * CW + cl) * 2);
                    const u32x4 gw = *reinterpret_cast<const u32x4 *>(gml + m * CW + cl);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        rv[2 * e] = bf16_lo(w[e]); rv[2 * e + 1] = bf16_hi(w[e]);
                        gv[2 * e] = bf16_lo(gw[e]); gv[2 * e + 1] = bf16_hi(gw[e]);
                    }
                } else {
                    const u32x2 w = *reinterpret_cast<const u32x2 *>(slot + t * PR + (m * CW + cl) * 2);
                    const u32x2 gw = *reinterpret_cast<const u32x2 *>(gml + m * CW + cl);
                    rv[0] = bf16_lo(w.x); rv[1] = bf16_hi(w.x); rv[2] = bf16_lo(w.y); rv[3] = bf16_hi(w.y);
                    gv[0] = bf16_lo(gw.x); gv[1] = bf16_hi(gw.x); gv[2] = bf16_lo(gw.y); gv[3] = bf16_hi(gw.y);
                }
                const float rm = rho[m] * inv_n;
#pragma unroll
                for (int b = 0; b < NB2; ++b) {
                    // G = sigmoid(l) = 1 / (1 + 2^t) with t = -log2(e) l (the MFMA result)
                    const float den = 1.0f + __builtin_amdgcn_exp2f(tl[b][m]);
                    uo[b] = fmaf(gv[b] * rv[b] * rm, __builtin_amdgcn_rcpf(den), uo[b]);
                }
            }
            if (tok0 + t < a.N) {
                bf16_t *dst = a.u + (tok0 + t) * d + c0 + cl;
                if constexpr (NB2 == 8) {
                    *reinterpret_cast<u32x4 *>(dst) = u32x4{pack_bf16x2(uo[0], uo[1]), pack_bf16x2(uo[2], uo[3]),
                                                            pack_bf16x2(uo[4], uo[5]), pack_bf16x2(uo[6], uo[7])};
                } else {
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(uo[0], uo[1]), pack_bf16x2(uo[2], uo[3])};
                }
            }
        }
    };

    // ---- the walk: a three-tile software pipeline.  Iteration k: the loads of
    // ss(k-1) go out, R(k-2), S(k), M(k-1) and Q(k-1), the loads of a(k-2), the
    // loads of tile k+1, C(k-2), then the loads of Q(k-1)'s records.  Every
    // exchange is read at least a stage after it was written, most of them an
    // iteration after: ss(k) is published in iteration k and gathered in k+1,
    // Q(k) in k+1 and reduced at the start of k+2, a(k) at the start of k+2 and
    // gathered at its end.  A wave's memory-count waits complete in issue
    // order, so each wait on exchange loads covers only what was issued before
    // them (the loads of tile k+1 come after those of a(k-2)); the stage flags
    // are compile-time constants, so the counts are exact.
    auto iterate = [&](int k, auto doS, auto doMQ, auto doRC) __attribute__((always_inline)) {
        if constexpr (doMQ.value) issue_ss(k - 1);
        if constexpr (doRC.value) stage_R(k - 2);
        if constexpr (doS.value) stage_S(k);
        if constexpr (doMQ.value) {
            stage_M(k - 1);
            stage_Q(k - 1);
        }
        if constexpr (doRC.value) issue_act(k - 2);
        if constexpr (doS.value) prefetch(k + 1 < K ? k + 1 : k);
        if constexpr (doRC.value) stage_C(k - 2);
        __syncthreads();
        if constexpr (doMQ.value) issue_q(k - 1);
    };
    using T1 = std::integral_constant<bool, true>;
    using F0 = std::integral_constant<bool, false>;
    if (tid == 0) *aborted = 0;
    __syncthreads();
    if (K > 0) {
        prefetch(0);
        iterate(0, T1{}, F0{}, F0{});
        if (K >= 2) iterate(1, T1{}, T1{}, F0{});
        else iterate(1, F0{}, T1{}, F0{});
        for (int k = 2; k < K; ++k) iterate(k, T1{}, T1{}, T1{});   // steady state
        if (K >= 2) iterate(K, F0{}, T1{}, T1{});
        iterate(K + 1, F0{}, F0{}, T1{});
    }
    // the last member of the cluster to finish advances its epoch
    if (tid == 0) {
        uint32_t *ctl = reinterpret_cast<uint32_t *>(xs);
        const uint32_t old = __hip_atomic_fetch_add(ctl + 8 + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old % kMembers == kMembers - 1)
            __hip_atomic_store(ctl + x, epoch + (uint32_t)K + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace cluster
}  // namespace grk

// ---------------------------------------------------------------------------
// Host side.
namespace grk {
namespace cluster {
namespace {

// Per-GPU state: whether the path can run there, the device address of that
// GPU's `exchange`, and the last launch (calls from different streams are
// ordered one after the other: they share the array and each needs the whole
// GPU resident at once).
struct DevState {
    std::once_flag once;
    bool ok = false;
    unsigned char *xs = nullptr;
    int ncl = 0;
    std::mutex mu;
    hipEvent_t last{};
    hipStream_t last_stream{};
    bool have_last = false;
};
constexpr int kMaxDevices = 64;
DevState g_dev[kMaxDevices];

template <int CW, bool FUSED> void *kernel_ptr() { return reinterpret_cast<void *>(&k_cluster<CW, FUSED>); }

bool occupancy_ok(void *fn, int threads) {
    int nb = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, 0) == hipSuccess && nb >= 1;
}

void init_device(int dev, DevState &s) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return;
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0) return;
    if (p.multiProcessorCount != kMembers * kMaxClusters) return;   // 8 XCDs of 32 CUs
    if (!occupancy_ok(kernel_ptr<128, true>(), threads_of(128)) || !occupancy_ok(kernel_ptr<128, false>(), threads_of(128)) ||
        !occupancy_ok(kernel_ptr<64, true>(), threads_of(64)) || !occupancy_ok(kernel_ptr<64, false>(), threads_of(64)))
        return;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(exchange)) != hipSuccess || !ptr) return;
    if (hipEventCreateWithFlags(&s.last, hipEventDisableTiming) != hipSuccess) return;
    s.xs = static_cast<unsigned char *>(ptr);
    s.ncl = p.multiProcessorCount / kMembers;
    s.ok = true;
}

DevState *device_state() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DevState &s = g_dev[dev];
    std::call_once(s.once, [&] { init_device(dev, s); });
    (void)hipGetLastError();
    return s.ok ? &s : nullptr;
}

// channels per workgroup for this shape (0: not a cluster shape)
int slice_width(const ReadArgs &a) {
    if (!a.bf16 || a.fp8 || a.n != 4 || a.r < 16 || a.r % 16 || a.r > 64) return 0;
    if (a.d == 32 * 128) return 128;
    if (a.d == 32 * 64) return 64;
    return 0;
}

template <int CW, bool FUSED>
hipError_t launch_t(const KArgs &k, int ncl, hipStream_t st) {
    hipLaunchKernelGGL((k_cluster<CW, FUSED>), dim3(kMembers * ncl), dim3(threads_of(CW)), 0, st, k);
    return hipGetLastError();
}

}  // namespace
}  // namespace cluster

bool cluster_path_ok(const ReadArgs &a) {
    // opt-in (GR_KERNEL_VARIANT=single): slower than the two-pass fast path
    // at every measured shape, kept for its single traversal of the state
    const char *v = getenv("GR_KERNEL_VARIANT");
    if (!v || strcmp(v, "single") != 0) return false;
    if (!cluster::slice_width(a)) return false;
    return cluster::device_state() != nullptr;
}

hipError_t launch_cluster(const ReadArgs &a, hipStream_t st) {
    using namespace cluster;
    DevState *s = device_state();
    const int cw = slice_width(a);
    if (!s || !cw) return hipErrorInvalidValue;
    const int tok = 32;
    KArgs k{};
    k.state = a.state; k.y = static_cast<const bf16_t *>(a.y); k.s_in = a.s_in;
    k.gamma = static_cast<const bf16_t *>(a.gamma);
    k.wd = static_cast<const bf16_t *>(a.wd);
    k.ww = static_cast<const bf16_t *>(a.ww);
    k.wu = static_cast<const bf16_t *>(a.wu);
    k.u = static_cast<bf16_t *>(a.u); k.s_out = a.s_out;
    k.xs = s->xs;
    k.N = a.N; k.d = a.d; k.r = a.r; k.nw = a.ww ? 4 : 0;
    k.rows = k.r + k.nw;
    k.nrb = (k.rows + 15) / 16;
    k.rks = (k.r + 31) / 32;
    k.tiles = (int)((a.N + tok - 1) / tok);
    k.ncl = s->ncl;
    k.eps = a.eps;
    std::lock_guard<std::mutex> lk(s->mu);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) cs = hipStreamCaptureStatusNone;
    const bool capturing = cs != hipStreamCaptureStatusNone;
    if (!capturing && s->have_last && s->last_stream != st) {
        hipError_t e = hipStreamWaitEvent(st, s->last, 0);
        if (e != hipSuccess) return e;
    }
    hipError_t e;
    if (cw == 128) e = a.fused ? launch_t<128, true>(k, s->ncl, st) : launch_t<128, false>(k, s->ncl, st);
    else e = a.fused ? launch_t<64, true>(k, s->ncl, st) : launch_t<64, false>(k, s->ncl, st);
    if (e != hipSuccess) return e;
    if (!capturing) {
        if ((e = hipEventRecord(s->last, st)) != hipSuccess) return e;
        s->last_stream = st;
        s->have_last = true;
    }
    return hipSuccess;
}

// Device error word of the cluster path on the current GPU (1 if a wait timed
// out since the last reset); reset clears it.
hipError_t cluster_error_word(uint32_t *word, bool reset) {
    using namespace cluster;
    *word = 0;
    DevState *s = device_state();
    if (!s) return hipSuccess;
    hipError_t e = hipMemcpy(word, s->xs + 128, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess && reset) e = hipMemset(s->xs + 128, 0, sizeof(uint32_t));
    return e;
}

}  // namespace grk
