// gr_fast_k2.hip -- the rest of the fast path's call (see gr_fast.hip): the
// reduction of kernel 1's records (rho of eq:rms, the SiLU activations of
// eq:gate, the write strengths of eq:s) and the forms of kernel 2 (up
// projection on MFMA, sigmoid gate of eq:gate, gated combine of eq:use_gate;
// "Paper reading: Qwen3.8 Flash Next", part 2 Residual, sec. 4): staged (few
// tokens), resident (many tokens), resident for an e4m3 state, and the XCD
// walk of a wide gate; and which form a call takes.
#include "gr_fast_common.h"

#include <atomic>

namespace grk {
namespace fast {
namespace {

// Kernel 1b: combine the partial records written by kernel 1.  One wave per
// token, RW tokens per workgroup: lanes 0..NB-1 sum the squares over the
// splits (rho_i, rms_i; shared by shuffles), and each lane owns outputs
// j = lane, lane + 64, ...: the split sums of P_i[j] for every branch (lanes
// read consecutive j: coalesced), rho applied, summed over branches in order.
// The loads of the sums of squares and of the first JO outputs per lane go
// out together (JO = 2, or 6 for a wide gate's up to 384 outputs with at most
// two splits), so a wave waits for memory once.
//   j < r        z = (1/n) sum_i rho_i P_i[j]  ->  -log2(e) SiLU(z) as (hi, lo)
//   r <= j < rk  zero padding of the up projection's k-steps
//   rk + i       s_i = 2 sigmoid((1/n) sum_i' rho_i' P_i'[r + i])  (1 without W_write)
// RW waves (tokens) per workgroup: four, or one for few tokens, whose
// workgroups then spread over all CUs.
template <int NB, int S, int JO, int RW>
__global__ void __launch_bounds__(64 * RW)
k_reduce_records(float *__restrict__ s_out, Workspace ws, FastShape sh, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * RW + (threadIdx.x >> 6);
    if (t >= sh.N) return;  // whole wave
    const int ps = sh.pstride;
    const float inv_n = 1.0f / (float)NB;
    const float *rec = ws.partial + t * NB * S * (int64_t)ps;  // (i, k) at (i*S + k)*pstride
    // sum over the S splits of record word `off` of branch i (pairwise, fixed order)
    auto split_sum = [&](int i, int off) {
        const float *q = rec + (int64_t)i * S * ps + off;
        float v[S];
#pragma unroll
        for (int k = 0; k < S; ++k) v[k] = q[k * ps];
#pragma unroll
        for (int w = 1; w < S; w *= 2)
#pragma unroll
            for (int k = 0; k + w < S; k += 2 * w) v[k] += v[k + w];
        return v[0];
    };
    // P row feeding output j (below), or -1 for a zero pad / no W_write
    const int outs = sh.rk + NB;
    auto prow = [&](int j) {
        if (j < sh.rk) return j < sh.r ? j : -1;
        return sh.nw ? sh.r + (j - sh.rk) : -1;
    };
    // (no row: output j is past the end, a zero pad, or s = 1 without W_write,
    // none of which uses the sums, so row 0, present in every record, is read;
    // loads without a condition all go out before the first wait)
    auto gather = [&](int j, float (&p)[NB]) {
        const int row = j < outs ? prow(j) : -1;
        const int rr = row >= 0 ? row : 0;
#pragma unroll
        for (int i = 0; i < NB; ++i) p[i] = split_sum(i, 4 + rr);
    };
    // one round of loads: the sums of squares with the rows of the lane's
    // first JO outputs (none of them waits for rho)
    const float ss_l = split_sum(lane < NB ? lane : 0, 0);   // used by lanes < NB
    float pj[JO][NB];
#pragma unroll
    for (int q = 0; q < JO; ++q) gather(lane + 64 * q, pj[q]);
    float rho_l = 0.f;
    if (lane < NB) {
        const float rms = sqrtf(ss_l / (float)sh.d + eps);
        rho_l = 1.0f / rms;
        ws.rms[t * NB + lane] = rms;
    }
    float rho[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) rho[i] = __shfl(rho_l, i, 64);
    // output j from p[i] = sum over splits of P_i[row(j)]: sum_i rho_i p_i, i in order
    auto emit = [&](int j, const float (&p)[NB]) {
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < NB; ++i) z = fmaf(rho[i], p[i], z);
        if (j < sh.rk) {
            const float v = j < sh.r ? -kLog2e * silu_f(z * inv_n) : 0.f;
            const bf16_t h = f32_to_bf16(v);
            ws.act[(t * 2) * sh.rk + j] = h;
            ws.act[(t * 2 + 1) * sh.rk + j] = f32_to_bf16(v - bf16_to_f32(h));
        } else {
            const int i = j - sh.rk;
            s_out[t * NB + i] = sh.nw ? 2.0f * sigmoid_f(z * inv_n) : 1.0f;
        }
    };
#pragma unroll
    for (int q = 0; q < JO; ++q)
        if (lane + 64 * q < outs) emit(lane + 64 * q, pj[q]);
    for (int j = lane + 64 * JO; j < outs; j += 64) {
        float p[NB];
        gather(j, p);
        emit(j, p);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2.  blockIdx -> (tile, channel range); NB = n (compile time).
// Staged per 32-channel chunk: W_up rows of the NB branches (as stored), placed
// in LDS in MFMA row order -- LDS row i*32 + 16h + m holds channel
// 8(m/4) + 4h + m%4 -- so that the result of block h lands on channels
// 8g + 4h + m' of lane group g (the layout the state is loaded in) and each
// fragment read covers 16 consecutive LDS rows (no bank conflicts at a pitch of
// an odd number of 16-byte units).  Also staged: gamma/n of the chunk as bf16
// words (exact for n = 4) masked to one half, so v_dot2 forms (gamma/n) R'
// straight from the packed state.  Pipeline: the state of the chunk two ahead
// and the W_up rows of the chunk after it are in flight while a chunk is
// combined.  ONE: every range is one chunk (decode-sized calls): all loads go
// out at once, with no prefetch and no loop.
template <int NB, int RKS, bool F8, bool ONE>
__global__ void __launch_bounds__(kK2Threads, kK2WavesPerSimd)
k_gate_combine(const typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ gamma,
               const bf16_t *__restrict__ wu, bf16_t *__restrict__ u, Workspace ws, FastShape sh,
               int ranges) {
    constexpr int KC = kChunk;                         // channels per iteration
    constexpr int RK = RKS * 32;
    constexpr int kPitch = RK + 8;                     // bf16 per staged W_up row
    constexpr int NV = NB * KC * (RK / 8);             // 16-byte vectors of W_up per iteration
    constexpr int WV = (NV + kK2Threads - 1) / kK2Threads;
    constexpr int NG = (NB * KC + kK2Threads - 1) / kK2Threads;
    __shared__ __attribute__((aligned(16))) bf16_t lds_u[2][NB * KC * kPitch];
    __shared__ uint32_t lds_g[2][NB * KC];  // (gamma/n) of channel cc in the half cc%2 of a word

    const int d = sh.d, r = sh.r;
    const int64_t b = blockIdx.x;
    const int64_t tile = b / ranges;
    const int range = (int)(b % ranges);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4;
    const int64_t t = tile * kK2Tile + wave * 16 + (lane & 15);
    const bool valid = t < sh.N;
    const int c_begin = range * sh.k2_chan;
    const int c_end = (c_begin + sh.k2_chan) < d ? (c_begin + sh.k2_chan) : d;
    const int nit = (c_end - c_begin) / kChunk;        // 32-channel chunks of this range (>= 1)
    const float inv_n = 1.0f / (float)NB;
    // Loads are issued without conditions (with conditions the compiler waits
    // for every load in flight before the first use, which at one or two chunks
    // per workgroup is the whole kernel): a token past the end of a ragged tile
    // reads the last token (its u is never stored), a prefetch past the last
    // chunk re-reads that chunk (never used), and W_up / gamma entries outside
    // the range or past r read the start of their tensor and are zeroed.
    const int64_t tl_ = valid ? t : sh.N - 1;          // token whose data this lane loads
    constexpr u32x4 z4 = {0u, 0u, 0u, 0u};

    // W_up rows (branch i, channel c) of one iteration; row index i * KC + cc
    u32x4 wreg[WV];
    uint32_t greg[NG];
    auto load_w = [&](int it) {
        const int c0 = c_begin + (it < nit ? it : nit - 1) * KC;
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * kK2Threads;
            const int row = v / (RK / 8), kv = v % (RK / 8);
            const int i = row / KC, cc = row % KC;
            const bool ok = v < NV && c0 + cc < c_end && kv * 8 < r;
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(ok ? wu + ((int64_t)i * d + c0 + cc) * r + kv * 8 : wu);
            wreg[q] = ok ? wv : z4;
        }
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int v = tid + q * kK2Threads;
            const bool ok = v < NB * KC && c0 + v % KC < c_end;
            const bf16_t gr = gamma[ok ? (int64_t)(v / KC) * d + c0 + v % KC : 0];
            const bf16_t gk = f32_to_bf16(bf16_to_f32(gr) * inv_n);
            const uint32_t gw = (v & 1) ? ((uint32_t)gk << 16) : (uint32_t)gk;
            greg[q] = ok ? gw : 0u;
        }
    };
    // LDS row of (branch i, channel cc of the chunk): MFMA row order
    auto store_w = [&](int buf) {
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * kK2Threads;
            if (v < NV) {
                const int row = v / (RK / 8), kv = v % (RK / 8);
                const int i = row / KC, cc = row % KC;
                const int pos = i * kChunk + 16 * ((cc >> 2) & 1) + 4 * (cc >> 3) + (cc & 3);
                *reinterpret_cast<u32x4 *>(&lds_u[buf][pos * kPitch + kv * 8]) = wreg[q];
            }
        }
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int v = tid + q * kK2Threads;
            if (v < NB * KC) lds_g[buf][v] = greg[q];
        }
    };

    // B operand: -log2(e) SiLU(z) of this lane's token as (hi, lo), k-steps of 32
    bf16x8 bop[RKS], bopl[RKS];
    float rms[NB];
#pragma unroll
    for (int ks = 0; ks < RKS; ++ks) {
        bop[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(ws.act + (tl_ * 2) * RK + ks * 32 + 8 * g));
        bopl[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(ws.act + (tl_ * 2 + 1) * RK + ks * 32 + 8 * g));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) rms[i] = ws.rms[tl_ * NB + i];

    const typename StateT<F8>::type *srow = state + tl_ * (int64_t)NB * d + 8 * g;
    bf16_t *urow = u + t * (int64_t)d + 8 * g;
    const int m16 = lane & 15;  // A row this lane feeds

    u32x4 s0[NB], s1[NB];
    auto load_state = [&](int it, u32x4 (&sv)[NB]) {
        const int c0 = c_begin + (it < nit ? it : nit - 1) * KC;
#pragma unroll
        for (int i = 0; i < NB; ++i) sv[i] = load8_as_bf16<F8>(srow + (int64_t)i * d + c0);
    };

    // gate and combine chunk `it` (W_up in LDS buffer it & 1, its state in s0)
    auto combine = [&](int it) {
        const int cur = it & 1;
        {
            const int c0 = c_begin + it * KC;
            float uacc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) uacc[e] = 0.f;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4 tl = {0.f, 0.f, 0.f, 0.f};
                    const bf16_t *ap = &lds_u[cur][(i * kChunk + 16 * h + m16) * kPitch + 8 * g];
#pragma unroll
                    for (int ks = 0; ks < RKS; ++ks) {
                        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(ap + ks * 32));
                        tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[ks], tl, 0, 0, 0);
                        tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bopl[ks], tl, 0, 0, 0);
                    }
                    // tl[m] = -log2(e) * l for channel 8g + 4h + m of branch i
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int e = 4 * h + m;
                        const float bterm = dot2_bf16(s0[i][e >> 1], lds_g[cur][i * KC + 8 * g + e], 0.f);
                        const float den = fmaf(__builtin_amdgcn_exp2f(tl[m]), rms[i], rms[i]);
                        uacc[e] = fmaf(bterm, __builtin_amdgcn_rcpf(den), uacc[e]);
                    }
                }
                // materialise per branch (else the element work sinks into the store's branch)
#pragma unroll
                for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(uacc[e]));
            }
            if (valid && c0 < c_end) {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(uacc[2 * e], uacc[2 * e + 1]);
                *reinterpret_cast<u32x4 *>(urow + c0) = o;
            }
        }
    };

    if constexpr (ONE) {
        load_state(0, s0);
        load_w(0);
        store_w(0);
        __syncthreads();
        combine(0);
        return;
    }
    load_w(0);
    store_w(0);
    load_w(1);
    load_state(0, s0);
    __syncthreads();
    for (int it = 0; it < nit; ++it) {
        load_state(it + 1, s1);
        combine(it);
        if (it + 1 < nit) store_w((it & 1) ^ 1);
        load_w(it + 2);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NB; ++i) s0[i] = s1[i];
    }
}

// The up projection's B operand for token t (-log2(e) a as bf16 hi and lo
// words, lane group g's eight of each k-step) and 1/rho of its branches.  A
// token past the end of a ragged last tile reads the last token's values
// instead: its u is never stored, and loads without a condition let the
// compiler keep them in flight (a conditional load with a default value was
// merged at once, a wait for every load in flight at each tile change).
template <int NB, int RKS>
__device__ __forceinline__ void load_act_rms(const Workspace &ws, const FastShape &sh, int64_t t, int g,
                                             bf16x8 (&hi)[RKS], bf16x8 (&lo)[RKS], float (&rm)[NB]) {
    constexpr int RK = RKS * 32;
    if (t >= sh.N) t = sh.N - 1;
#pragma unroll
    for (int ks = 0; ks < RKS; ++ks) {
        hi[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(ws.act + (t * 2) * RK + ks * 32 + 8 * g));
        lo[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(ws.act + (t * 2 + 1) * RK + ks * 32 + 8 * g));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) rm[i] = ws.rms[t * NB + i];
}

// ---------------------------------------------------------------------------
// Kernel 2, resident form (many tokens).  One workgroup per (channel range of
// CH channels, residue class p of the token tiles modulo P).  The W_up rows of
// the range (every branch, MFMA row order as above) and gamma/n are staged in
// LDS once; the workgroup then walks the tiles p, p + P, ... (those kernel 1
// wrote last first, see TileWalk) in steps of 64 channels.  A step reads, per
// token and branch, one whole 128-byte line of the state (its two 64-byte
// halves back to back) and writes one whole line of u, so no line is fetched
// or written in halves.  The next step's state is
// loaded branch by branch, each as soon as the current step has finished with
// that branch: the prefetch costs no registers beyond one step's state.  The
// activations and rms of the next tile are loaded before the state of its
// first step, so waiting for them never waits for that state.
// Stage the W_up rows of a channel range (every branch, NC 32-channel chunks,
// MFMA row order: LDS row (i NC + chunk) 32 + 16h + m holds channel
// 8(m/4) + 4h + m%4 of the chunk) and gamma/n of the range (bf16 in the half word
// of the channel's parity).  A thread's loads go out BATCH at a time before
// their LDS stores, one round trip per batch (as a loop of load-then-store,
// one per vector).  Channels past nchan and k past r stage zeros.
template <int NB, int CH, int RK, int THREADS, int BATCH>
__device__ __forceinline__ void stage_wup(bf16_t *lds_u, uint32_t *lds_g, const bf16_t *__restrict__ wu,
                                          const bf16_t *__restrict__ gamma, int d, int r, int c_begin,
                                          int nchan, float inv_n, int tid) {
    constexpr int NC = CH / kChunk;
    constexpr int kPitch = RK + 8;
    constexpr int NVEC = NB * CH * (RK / 8);
    constexpr int PER = (NVEC + THREADS - 1) / THREADS;
    constexpr int GPER = (NB * CH + THREADS - 1) / THREADS;
    constexpr u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b0 = 0; b0 < PER; b0 += BATCH) {
        u32x4 w[BATCH];
        uint32_t gw[GPER];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int v = tid + (b0 + j) * THREADS;
            const int row = v / (RK / 8), kv = v % (RK / 8);
            const int i = row / CH, cc = row % CH;
            const bool ok = b0 + j < PER && v < NVEC && cc < nchan && kv * 8 < r;
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(ok ? wu + ((int64_t)i * d + c_begin + cc) * r + kv * 8 : wu);
            w[j] = ok ? wv : z4;
        }
        if (b0 == 0) {
#pragma unroll
            for (int j = 0; j < GPER; ++j) {
                const int v = tid + j * THREADS;
                const int i = v / CH, cc = v % CH;
                const bool ok = v < NB * CH && cc < nchan;
                const bf16_t gr = gamma[ok ? (int64_t)i * d + c_begin + cc : 0];
                const bf16_t gk = f32_to_bf16(bf16_to_f32(gr) * inv_n);
                const uint32_t gv = (cc & 1) ? ((uint32_t)gk << 16) : (uint32_t)gk;
                gw[j] = ok ? gv : 0u;
            }
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int v = tid + (b0 + j) * THREADS;
            if (b0 + j < PER && v < NVEC) {
                const int row = v / (RK / 8), kv = v % (RK / 8);
                const int i = row / CH, cc = row % CH, c32 = cc % kChunk;
                const int pos = (i * NC + cc / kChunk) * kChunk + 16 * ((c32 >> 2) & 1) + 4 * (c32 >> 3) + (c32 & 3);
                *reinterpret_cast<u32x4 *>(&lds_u[pos * kPitch + kv * 8]) = w[j];
            }
        }
        if (b0 == 0) {
#pragma unroll
            for (int j = 0; j < GPER; ++j) {
                const int v = tid + j * THREADS;
                if (v < NB * CH) lds_g[v] = gw[j];
            }
        }
    }
}

template <int RKS> struct ResidentCfg {
    // channels per workgroup: keeps the staged W_up near 72 KiB (two per CU);
    // a wide gate (RKS > 4) gets 32 channels, ~84 KiB (one per CU)
    static constexpr int CH = RKS <= 2 ? 128 : (RKS <= 4 ? 64 : 32);
    // 32-channel chunks per step: two (one 128-byte line of bf16) when the range allows
    static constexpr int SC = CH >= 64 ? 2 : 1;
};

constexpr int kResWaves = 8;
constexpr int kResWavesPerSimd = 4;              // occupancy target (narrow gate)
constexpr int kResThreads = 64 * kResWaves;
constexpr int kResTile = 16 * kResWaves;         // tokens per tile
constexpr int kResWgsTarget = 512;               // workgroups wanted (two per CU)

template <int NB, int RKS, int CH, int SC>
__global__ void __launch_bounds__(kResThreads, RKS <= 2 ? kResWavesPerSimd : 2)
k_gate_combine_resident(const bf16_t *__restrict__ state, const bf16_t *__restrict__ gamma,
                        const bf16_t *__restrict__ wu, bf16_t *__restrict__ u, Workspace ws,
                        FastShape sh, int ranges, int P) {
    constexpr int NC = CH / kChunk;                    // 32-channel chunks per range
    constexpr int RK = RKS * 32;
    constexpr int kPitch = RK + 8;                     // bf16 per staged W_up row
    __shared__ __attribute__((aligned(16))) bf16_t lds_u[NB * CH * kPitch];
    __shared__ __attribute__((aligned(16))) uint32_t lds_g[NB * CH];

    const int d = sh.d, r = sh.r;
    const int range = (int)(blockIdx.x % ranges);
    const int64_t p = blockIdx.x / ranges;
    const int64_t tiles = (sh.N + kResTile - 1) / kResTile;
    if (p >= tiles) return;                            // whole workgroup
    const int c_begin = range * CH;
    constexpr int kResStep = SC * kChunk;             // channels per step
    const int nchan = (d - c_begin) < CH ? (d - c_begin) : CH;
    const int nsteps = nchan / kResStep;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, m16 = lane & 15;
    const float inv_n = 1.0f / (float)NB;

    auto token = [&](int64_t T) { return T * kResTile + wave * 16 + m16; };
    auto load_act = [&](int64_t T, bf16x8 (&hi)[RKS], bf16x8 (&lo)[RKS], float (&rm)[NB]) {
        load_act_rms<NB, RKS>(ws, sh, token(T), g, hi, lo, rm);
    };
    // state of branch i, step st of tile T: SC 16-byte words per lane
    auto load_state = [&](int64_t T, int st, int i, u32x4 (&sv)[SC]) {
        const int64_t t = token(T);
        const bf16_t *q = state + t * (int64_t)NB * d + (int64_t)i * d + c_begin + st * kResStep + 8 * g;
        const bool ok = t < sh.N;
#pragma unroll
        for (int sc = 0; sc < SC; ++sc)
            sv[sc] = ok ? *reinterpret_cast<const u32x4 *>(q + sc * kChunk) : u32x4{0u, 0u, 0u, 0u};
    };

    bf16x8 bop[RKS], bopl[RKS], nbop[RKS], nbopl[RKS];
    float rms[NB], nrms[NB];
    u32x4 sv[NB][SC];
    const TileWalk walk = tile_walk(sh, p, P, tiles, c_begin);
    int pass = 0;
    int64_t T = walk.next(p, pass);                    // >= 0: p < tiles
    int st = 0;
    load_act(T, bop, bopl, rms);
#pragma unroll
    for (int i = 0; i < NB; ++i) load_state(T, 0, i, sv[i]);

    // stage W_up rows (branch i, channel cc of the range) and gamma/n
    stage_wup<NB, CH, RK, kResThreads, 8>(lds_u, lds_g, wu, gamma, d, r, c_begin, nchan, inv_n, tid);
    __syncthreads();

    for (;;) {
        int64_t Tn = T;
        int sn = st + 1, pn = pass;
        if (sn == nsteps) { sn = 0; Tn = walk.next(T + P, pn); }
        const bool more = Tn >= 0;
        if (sn == 0 && more) load_act(Tn, nbop, nbopl, nrms);

        float uacc[SC][8];
#pragma unroll
        for (int sc = 0; sc < SC; ++sc)
#pragma unroll
            for (int e = 0; e < 8; ++e) uacc[sc][e] = 0.f;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
            for (int sc = 0; sc < SC; ++sc) {
                const int chunk = i * NC + st * SC + sc;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4 tl = {0.f, 0.f, 0.f, 0.f};
                    const bf16_t *ap = &lds_u[(chunk * kChunk + 16 * h + m16) * kPitch + 8 * g];
#pragma unroll
                    for (int ks = 0; ks < RKS; ++ks) {
                        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(ap + ks * 32));
                        tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[ks], tl, 0, 0, 0);
                        tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bopl[ks], tl, 0, 0, 0);
                    }
                    // tl[m] = -log2(e) * l for channel 8g + 4h + m of the chunk, branch i
                    const uint32_t *gp = &lds_g[i * CH + (st * SC + sc) * kChunk + 8 * g + 4 * h];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int e = 4 * h + m;
                        const float bterm = dot2_bf16(sv[i][sc][e >> 1], gp[m], 0.f);
                        const float den = fmaf(__builtin_amdgcn_exp2f(tl[m]), rms[i], rms[i]);
                        uacc[sc][e] = fmaf(bterm, __builtin_amdgcn_rcpf(den), uacc[sc][e]);
                    }
                }
            }
            // Materialise the sums here: otherwise the compiler sinks all of the
            // step's element work into the (token < N) store below and keeps
            // every MFMA result live at once.
#pragma unroll
            for (int sc = 0; sc < SC; ++sc)
#pragma unroll
                for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(uacc[sc][e]));
            // branch i of this step is consumed: fetch it for the next step
            if (more) load_state(Tn, sn, i, sv[i]);
        }
        const int64_t t = token(T);
        if (t < sh.N) {
            bf16_t *q = u + t * (int64_t)d + c_begin + st * kResStep + 8 * g;
#pragma unroll
            for (int sc = 0; sc < SC; ++sc) {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(uacc[sc][2 * e], uacc[sc][2 * e + 1]);
                *reinterpret_cast<u32x4 *>(q + sc * kChunk) = o;
            }
        }
        if (!more) break;
        if (sn == 0) {
#pragma unroll
            for (int ks = 0; ks < RKS; ++ks) { bop[ks] = nbop[ks]; bopl[ks] = nbopl[ks]; }
#pragma unroll
            for (int i = 0; i < NB; ++i) rms[i] = nrms[i];
        }
        T = Tn;
        st = sn;
        pass = pn;
    }
}

// ---------------------------------------------------------------------------
// Kernel 2, wide gate (more than four k-steps, r > 128), many tokens.  The
// up projection's B operand -- -log2(e) a as hi / lo words, RKS * 8 VGPRs per
// lane -- is the largest input of a (channel range, token tile) unit once r is
// large, and every range reads it again.  So the walk is made XCD-aware: one
// workgroup per CU, blockIdx % 8 taken as the XCD (round-robin dispatch), XCD
// x taking the token tiles T = x, x + 8, ... and its workgroups splitting the
// (range, tile) units of those tiles range by range.  The activations of an
// XCD's tiles (a few MB) then stay in its L2 while all ranges pass over them.
// A unit is one step of kernel 2's resident form at 32 channels per range,
// i.e. half of each 128-byte line of a state row; so workgroups come in
// pairs, 2m and 2m + 1 of an XCD taking ranges 2p and 2p + 1 of the same
// tiles in the same order, and each line's second half is an L2 hit.  The
// W_up rows of a range (NB * 32 rows, MFMA row order) are restaged in LDS
// whenever a workgroup moves on to its next range.
template <int NB, int RKS, bool F8>
__global__ void __launch_bounds__(kResThreads, 2)
k_gate_combine_wide(const typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ gamma,
                    const bf16_t *__restrict__ wu, bf16_t *__restrict__ u, Workspace ws,
                    FastShape sh, int ranges, int wgs_per_xcd) {
    constexpr int CH = kChunk;                         // channels per range
    constexpr int RK = RKS * 32;
    constexpr int kPitch = RK + 8;                     // bf16 per staged W_up row
    __shared__ __attribute__((aligned(16))) bf16_t lds_u[NB * CH * kPitch];
    __shared__ __attribute__((aligned(16))) uint32_t lds_g[NB * CH];

    const int d = sh.d, r = sh.r;
    const int xcd = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
    // GS workgroups in lockstep cover one 128-byte line of the state rows
    constexpr int GS = F8 ? 4 : 2;
    using SV = typename StateT<F8>::vec8;              // 8 channels of the state
    const int grp = j / GS, side = j % GS, groups = wgs_per_xcd / GS;
    const int64_t tiles = (sh.N + kResTile - 1) / kResTile;
    const int rgs = ranges / GS;                       // range groups (GS ranges each)
    // XCD x takes the tiles x, x + 8, ... and every range group; with fewer
    // than 8 tiles, XCD x takes tile x % tiles and every reps-th range group
    // from x / tiles, so that all XCDs work (reps = 8 / tiles)
    int64_t ntx, tile0;
    int rg0 = 0, rgstep = 1, nrg = rgs;
    if (tiles >= 8) {
        ntx = tiles > xcd ? (tiles - xcd + 7) / 8 : 0;
        tile0 = xcd;
    } else {
        const int reps = 8 / (int)tiles;
        ntx = xcd < tiles * reps ? 1 : 0;
        tile0 = xcd % tiles;
        rg0 = xcd / (int)tiles;
        rgstep = reps;
        nrg = rg0 < rgs ? (rgs - rg0 + reps - 1) / reps : 0;
    }
    const int64_t units = (int64_t)nrg * ntx;         // (range group, tile) units
    if (grp >= groups) return;                         // whole workgroup (the count's remainder idles)
    const int64_t u0 = units * grp / groups, u1 = units * (grp + 1) / groups;
    if (u0 >= u1) return;                              // whole workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, m16 = lane & 15;
    const float inv_n = 1.0f / (float)NB;

    auto unit_tile = [&](int64_t q) { return tile0 + 8 * (q % ntx); };
    auto unit_range = [&](int64_t q) { return GS * (rg0 + rgstep * (int)(q / ntx)) + side; };
    auto token = [&](int64_t T) { return T * kResTile + wave * 16 + m16; };
    // state of branch i, range rg of tile T: 8 channels per lane
    auto load_state = [&](int64_t T, int rg, int i) {
        const int64_t t = token(T);
        if (t >= sh.N) return SV{};
        return *reinterpret_cast<const SV *>(state + t * (int64_t)NB * d + (int64_t)i * d + rg * CH + 8 * g);
    };
    // W_up rows (branch i, channel cc of range rg) in MFMA row order, and gamma/n
    // (a loop of load-then-store; issuing a batch of loads before the stores, as
    // the resident forms do, made this kernel slower: 312 -> 343 us at r = 320)
    auto stage = [&](int rg) {
        const int c_begin = rg * CH;
        for (int v = tid; v < NB * CH * (RK / 8); v += kResThreads) {
            const int row = v / (RK / 8), kv = v % (RK / 8);
            const int i = row / CH, cc = row % CH;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (kv * 8 < r)
                w = *reinterpret_cast<const u32x4 *>(wu + ((int64_t)i * d + c_begin + cc) * r + kv * 8);
            const int pos = i * CH + 16 * ((cc >> 2) & 1) + 4 * (cc >> 3) + (cc & 3);
            *reinterpret_cast<u32x4 *>(&lds_u[pos * kPitch + kv * 8]) = w;
        }
        for (int v = tid; v < NB * CH; v += kResThreads) {
            const int i = v / CH, cc = v % CH;
            const bf16_t gk = f32_to_bf16(bf16_to_f32(gamma[(int64_t)i * d + c_begin + cc]) * inv_n);
            lds_g[v] = (cc & 1) ? ((uint32_t)gk << 16) : (uint32_t)gk;
        }
    };

    // The activations (B operand) of a unit come in two halves of the k-steps,
    // K0 and RKS - K0: the second half of the current unit is loaded while the
    // first half's MFMAs run, and the next unit's first half into the registers
    // the first half frees -- 80 instead of 160 VGPRs of activations in flight,
    // which leaves the compiler room to keep more W_up fragment reads ahead of
    // the MFMAs.  Each gate still accumulates its k-steps 0 .. RKS-1 in order.
    constexpr int K0 = (RKS + 1) / 2, K1 = RKS - K0;
    constexpr int RK_ = RKS * 32;
    auto load_half = [&](int64_t T, int kb, int kn, bf16x8 *hi, bf16x8 *lo) {
        int64_t t = token(T);
        if (t >= sh.N) t = sh.N - 1;
#pragma unroll
        for (int k = 0; k < K0; ++k) {
            if (k < kn) {
                hi[k] = as_bf16x8(*reinterpret_cast<const u32x4 *>(ws.act + (t * 2) * RK_ + (kb + k) * 32 + 8 * g));
                lo[k] = as_bf16x8(*reinterpret_cast<const u32x4 *>(ws.act + (t * 2 + 1) * RK_ + (kb + k) * 32 + 8 * g));
            }
        }
    };
    auto load_rms = [&](int64_t T, float (&rm)[NB]) {
        int64_t t = token(T);
        if (t >= sh.N) t = sh.N - 1;
#pragma unroll
        for (int i = 0; i < NB; ++i) rm[i] = ws.rms[t * NB + i];
    };
    bf16x8 bA[K0], bAl[K0], bB[K0], bBl[K0];
    float rms[NB], nrms[NB];
    SV sv[NB];
    int64_t q = u0;
    int64_t T = unit_tile(q);
    int rg = unit_range(q);
    load_half(T, 0, K0, bA, bAl);
    load_rms(T, rms);
#pragma unroll
    for (int i = 0; i < NB; ++i) sv[i] = load_state(T, rg, i);
    stage(rg);
    __syncthreads();

    for (;;) {
        const bool more = q + 1 < u1;
        const int64_t Tn = more ? unit_tile(q + 1) : T;
        const int rn = more ? unit_range(q + 1) : rg;
        load_half(T, K0, K1, bB, bBl);                // this unit's second half

        f32x4 tl[NB][2];
        // W_up fragments of chain c = (i, h), k-steps kb .. kb + K0 - 1, read one
        // chain ahead of the MFMAs that use them
        bf16x8 fa[2][K0];
        auto read_frags = [&](int c, int kb, int kn, bf16x8 (&f)[K0]) {
            const bf16_t *ap = &lds_u[((c >> 1) * CH + 16 * (c & 1) + m16) * kPitch + 8 * g];
#pragma unroll
            for (int k = 0; k < K0; ++k)
                if (k < kn) f[k] = as_bf16x8(*reinterpret_cast<const u32x4 *>(ap + (kb + k) * 32));
        };
        read_frags(0, 0, K0, fa[0]);
#pragma unroll
        for (int c = 0; c < 2 * NB; ++c) {
            if (c + 1 < 2 * NB) read_frags(c + 1, 0, K0, fa[(c + 1) & 1]);
            else read_frags(0, K0, K1, fa[(c + 1) & 1]);   // the second half's first chain
            __builtin_amdgcn_sched_barrier(0);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < K0; ++ks) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[c & 1][ks], bA[ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[c & 1][ks], bAl[ks], acc, 0, 0, 0);
            }
            tl[c >> 1][c & 1] = acc;
        }
        if (more) {                                    // the next unit's first half, into the freed registers
            load_half(Tn, 0, K0, bA, bAl);
            load_rms(Tn, nrms);
        }

        float uacc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) uacc[e] = 0.f;
        constexpr int F0 = (2 * NB) & 1;                // buffer holding the second half's chain 0
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 2 * i + h;
                const int cur = (F0 + c) & 1;
                if (c + 1 < 2 * NB) read_frags(c + 1, K0, K1, fa[cur ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < K1; ++ks) {
                    tl[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][ks], bB[ks], tl[i][h], 0, 0, 0);
                    tl[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][ks], bBl[ks], tl[i][h], 0, 0, 0);
                }
                const f32x4 tv = tl[i][h];
                // tv[m] = -log2(e) * l for channel 8g + 4h + m of the range, branch i
                const uint32_t *gp = &lds_g[i * CH + 8 * g + 4 * h];
                float xe[4];                              // e4m3: elements 4h .. 4h+3 of the lane's 8
                if constexpr (F8) {
                    const f32x2 a01 = fp8x2_lo(sv[i][h]), a23 = fp8x2_hi(sv[i][h]);
                    xe[0] = a01.x; xe[1] = a01.y; xe[2] = a23.x; xe[3] = a23.y;
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = 4 * h + m;
                    float bterm;
                    if constexpr (F8)   // (gamma/n) in the half word of this channel's parity
                        bterm = xe[m] * ((m & 1) ? bf16_hi(gp[m]) : bf16_lo(gp[m]));
                    else
                        bterm = dot2_bf16(sv[i][e >> 1], gp[m], 0.f);
                    const float den = fmaf(__builtin_amdgcn_exp2f(tv[m]), rms[i], rms[i]);
                    uacc[e] = fmaf(bterm, __builtin_amdgcn_rcpf(den), uacc[e]);
                }
            }
            // materialise per branch (else the element work sinks into the store's branch)
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(uacc[e]));
            // branch i of this unit is consumed: fetch it for the next unit
            if (more) sv[i] = load_state(Tn, rn, i);
        }
        const int64_t t = token(T);
        if (t < sh.N) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(uacc[2 * e], uacc[2 * e + 1]);
            *reinterpret_cast<u32x4 *>(u + t * (int64_t)d + rg * CH + 8 * g) = o;
        }
        if (!more) break;
        if (rn != rg) {  // next range: every wave is done with this one's rows
            __syncthreads();
            stage(rn);
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) rms[i] = nrms[i];
        T = Tn;
        rg = rn;
        ++q;
    }
}

// ---------------------------------------------------------------------------
// Kernel 2 for an e4m3 state, resident form.  Same walk as above, but a step
// is one 64-channel unit: a 64-byte half line of the state per token and
// branch, of which lane group g owns channels 16g .. 16g + 15 (one 16-byte
// word of e4m3).  The W_up rows of a unit sit in LDS so that block h
// (h = 0..3) of the up projection lands there: LDS row 16h + 4g + m of a unit
// holds channel 16g + 4h + m, and tl[m] of block h is element 4h + m of the
// lane's word.  Each branch's word of the next step is fetched as soon as the
// current step has used it.  (Two units per step, one whole 128-byte line,
// needs 16 more VGPRs than the two-workgroups-per-CU budget allows and
// measured slower.)
constexpr int kF8Unit = 64;

template <int NB, int RKS, int CH>
__global__ void __launch_bounds__(kResThreads, RKS <= 2 ? kResWavesPerSimd : 2)
k_gate_combine_resident_fp8(const fp8_t *__restrict__ state, const bf16_t *__restrict__ gamma,
                            const bf16_t *__restrict__ wu, bf16_t *__restrict__ u, Workspace ws,
                            FastShape sh, int ranges, int P) {
    constexpr int NU = CH / kF8Unit;                   // units per range
    constexpr int RK = RKS * 32;
    constexpr int kPitch = RK + 8;                     // bf16 per staged W_up row
    __shared__ __attribute__((aligned(16))) bf16_t lds_u[NB * CH * kPitch];
    __shared__ __attribute__((aligned(16))) float lds_g[NB * CH];

    const int d = sh.d, r = sh.r;
    const int range = (int)(blockIdx.x % ranges);
    const int64_t p = blockIdx.x / ranges;
    const int64_t tiles = (sh.N + kResTile - 1) / kResTile;
    if (p >= tiles) return;                            // whole workgroup
    const int c_begin = range * CH;
    const int nchan = (d - c_begin) < CH ? (d - c_begin) : CH;   // a multiple of kF8Unit
    const int nsteps = nchan / kF8Unit;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, m16 = lane & 15;
    const float inv_n = 1.0f / (float)NB;

    auto token = [&](int64_t T) { return T * kResTile + wave * 16 + m16; };
    auto load_act = [&](int64_t T, bf16x8 (&hi)[RKS], bf16x8 (&lo)[RKS], float (&rm)[NB]) {
        load_act_rms<NB, RKS>(ws, sh, token(T), g, hi, lo, rm);
    };
    // e4m3 word of branch i, step st of tile T
    auto load_state = [&](int64_t T, int st, int i) {
        const int64_t t = token(T);
        if (t >= sh.N) return u32x4{0u, 0u, 0u, 0u};
        return *reinterpret_cast<const u32x4 *>(state + t * (int64_t)NB * d + (int64_t)i * d + c_begin +
                                                st * kF8Unit + 16 * g);
    };

    bf16x8 bop[RKS], bopl[RKS], nbop[RKS], nbopl[RKS];
    float rms[NB], nrms[NB];
    u32x4 sv[NB];
    const TileWalk walk = tile_walk(sh, p, P, tiles, c_begin);
    int pass = 0;
    int64_t T = walk.next(p, pass);                    // >= 0: p < tiles
    int st = 0;
    load_act(T, bop, bopl, rms);
#pragma unroll
    for (int i = 0; i < NB; ++i) sv[i] = load_state(T, 0, i);

    // stage W_up rows (branch i, channel cc of the range) and gamma/n: a thread's
    // loads all go out before its LDS stores (one round trip, not one per vector)
    {
        constexpr int NVEC = NB * CH * (RK / 8);
        constexpr int PER = (NVEC + kResThreads - 1) / kResThreads;
        constexpr int GPER = (NB * CH + kResThreads - 1) / kResThreads;
        u32x4 w[PER];
        float gq[GPER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int v = tid + j * kResThreads;
            const int row = v / (RK / 8), kv = v % (RK / 8);
            const int i = row / CH, cc = row % CH;
            const bool ok = v < NVEC && cc < nchan && kv * 8 < r;
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(ok ? wu + ((int64_t)i * d + c_begin + cc) * r + kv * 8 : wu);
            w[j] = ok ? wv : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < GPER; ++j) {
            const int v = tid + j * kResThreads;
            const int i = v / CH, cc = v % CH;
            const bool ok = v < NB * CH && cc < nchan;
            const bf16_t gr = gamma[ok ? (int64_t)i * d + c_begin + cc : 0];
            const float gv = bf16_to_f32(f32_to_bf16(bf16_to_f32(gr) * inv_n));
            gq[j] = ok ? gv : 0.f;
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int v = tid + j * kResThreads;
            if (v < NVEC) {
                const int row = v / (RK / 8), kv = v % (RK / 8);
                const int i = row / CH, cc = row % CH, c64 = cc % kF8Unit;
                const int pos = (i * NU + cc / kF8Unit) * kF8Unit + 16 * ((c64 >> 2) & 3) + 4 * (c64 >> 4) + (c64 & 3);
                *reinterpret_cast<u32x4 *>(&lds_u[pos * kPitch + kv * 8]) = w[j];
            }
        }
#pragma unroll
        for (int j = 0; j < GPER; ++j) {
            const int v = tid + j * kResThreads;
            if (v < NB * CH) lds_g[v] = gq[j];
        }
    }
    __syncthreads();

    for (;;) {
        int64_t Tn = T;
        int sn = st + 1, pn = pass;
        if (sn == nsteps) { sn = 0; Tn = walk.next(T + P, pn); }
        const bool more = Tn >= 0;
        if (sn == 0 && more) load_act(Tn, nbop, nbopl, nrms);

        float uacc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) uacc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                f32x4 tl = {0.f, 0.f, 0.f, 0.f};
                const bf16_t *ap = &lds_u[((i * NU + st) * kF8Unit + 16 * h + m16) * kPitch + 8 * g];
#pragma unroll
                for (int ks = 0; ks < RKS; ++ks) {
                    const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(ap + ks * 32));
                    tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[ks], tl, 0, 0, 0);
                    tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bopl[ks], tl, 0, 0, 0);
                }
                // tl[m] = -log2(e) * l for channel 16g + 4h + m of the unit, branch i
                const f32x2 x01 = fp8x2_lo(sv[i][h]), x23 = fp8x2_hi(sv[i][h]);
                const float x[4] = {x01.x, x01.y, x23.x, x23.y};
                const float *gp = &lds_g[i * CH + st * kF8Unit + 16 * g + 4 * h];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = 4 * h + m;
                    const float den = fmaf(__builtin_amdgcn_exp2f(tl[m]), rms[i], rms[i]);
                    uacc[e] = fmaf(x[m] * gp[m], __builtin_amdgcn_rcpf(den), uacc[e]);
                }
            }
            // materialise per branch (else the element work sinks into the store's branch)
#pragma unroll
            for (int e = 0; e < 16; ++e) asm volatile("" : "+v"(uacc[e]));
            // branch i of this step is consumed: fetch it for the next step
            if (more) sv[i] = load_state(Tn, sn, i);
        }
        const int64_t t = token(T);
        if (t < sh.N) {
            bf16_t *q = u + t * (int64_t)d + c_begin + st * kF8Unit + 16 * g;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(uacc[8 * k + 2 * e], uacc[8 * k + 2 * e + 1]);
                *reinterpret_cast<u32x4 *>(q + 8 * k) = o;
            }
        }
        if (!more) break;
        if (sn == 0) {
#pragma unroll
            for (int ks = 0; ks < RKS; ++ks) { bop[ks] = nbop[ks]; bopl[ks] = nbopl[ks]; }
#pragma unroll
            for (int i = 0; i < NB; ++i) rms[i] = nrms[i];
        }
        T = Tn;
        st = sn;
        pass = pn;
    }
}

template <int NB, bool F8>
hipError_t launch_k2(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    const int ranges = (sh.d + sh.k2_chan - 1) / sh.k2_chan;
    const unsigned grid = (unsigned)(((sh.N + kK2Tile - 1) / kK2Tile) * ranges);
#define GR_K2(RKS)                                                                          \
    case RKS:                                                                               \
        if (sh.k2_chan == kChunk)                                                           \
            hipLaunchKernelGGL((k_gate_combine<NB, RKS, F8, true>), dim3(grid), dim3(kK2Threads), 0, st, \
                               (const typename StateT<F8>::type *)a.state, (const bf16_t *)a.gamma, \
                               (const bf16_t *)a.wu, (bf16_t *)a.u, w, sh, ranges);         \
        else                                                                                \
            hipLaunchKernelGGL((k_gate_combine<NB, RKS, F8, false>), dim3(grid), dim3(kK2Threads), 0, st, \
                               (const typename StateT<F8>::type *)a.state, (const bf16_t *)a.gamma, \
                               (const bf16_t *)a.wu, (bf16_t *)a.u, w, sh, ranges);         \
        break;
    switch (sh.rk / 32) {
        GR_K2(1) GR_K2(2) GR_K2(3) GR_K2(4)
    default: return hipErrorInvalidValue;
    }
#undef GR_K2
    return hipGetLastError();
}

template <int NB, int RKS>
hipError_t launch_k2_resident_rks(const ReadArgs &a, const FastShape &sh, const Workspace &w,
                                  hipStream_t st) {
    constexpr int CH = ResidentCfg<RKS>::CH;
    const int ranges = (sh.d + CH - 1) / CH;
    const int64_t tiles = (sh.N + kResTile - 1) / kResTile;
    int64_t P = (kResWgsTarget + ranges / 2) / ranges;
    if (P > tiles) P = tiles;
    if (P < 1) P = 1;
    hipLaunchKernelGGL((k_gate_combine_resident<NB, RKS, CH, ResidentCfg<RKS>::SC>), dim3((unsigned)(ranges * P)),
                       dim3(kResThreads), 0, st, (const bf16_t *)a.state, (const bf16_t *)a.gamma,
                       (const bf16_t *)a.wu, (bf16_t *)a.u, w, sh, ranges, (int)P);
    return hipGetLastError();
}

template <int NB, int RKS>
hipError_t launch_k2_resident_fp8_rks(const ReadArgs &a, const FastShape &sh, const Workspace &w,
                                      hipStream_t st) {
    constexpr int CH = ResidentCfg<RKS>::CH;
    const int ranges = (sh.d + CH - 1) / CH;
    const int64_t tiles = (sh.N + kResTile - 1) / kResTile;
    int64_t P = (kResWgsTarget + ranges / 2) / ranges;
    if (P > tiles) P = tiles;
    if (P < 1) P = 1;
    hipLaunchKernelGGL((k_gate_combine_resident_fp8<NB, RKS, CH>), dim3((unsigned)(ranges * P)),
                       dim3(kResThreads), 0, st, (const fp8_t *)a.state, (const bf16_t *)a.gamma,
                       (const bf16_t *)a.wu, (bf16_t *)a.u, w, sh, ranges, (int)P);
    return hipGetLastError();
}

template <int NB>
hipError_t launch_k2_resident_fp8(const ReadArgs &a, const FastShape &sh, const Workspace &w,
                                  hipStream_t st) {
    switch (sh.rk / 32) {
    case 1: return launch_k2_resident_fp8_rks<NB, 1>(a, sh, w, st);
    case 2: return launch_k2_resident_fp8_rks<NB, 2>(a, sh, w, st);
    case 3: return launch_k2_resident_fp8_rks<NB, 3>(a, sh, w, st);
    case 4: return launch_k2_resident_fp8_rks<NB, 4>(a, sh, w, st);
    default: return hipErrorInvalidValue;
    }
}

// Compute units of the current device (cached per device; calls may come from
// several threads, so the cache entries are atomics: a race only repeats the query).
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int NB, int RKS, bool F8>
hipError_t launch_k2_wide_rks(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    // ranges: d / 32, a multiple of the lockstep group (2 bf16, 4 e4m3): d is a
    // multiple of 64 (bf16) or 128 (e4m3 wide gate)
    const int ranges = sh.d / kChunk;
    const int per_xcd = (cu_count() + 7) / 8;
    hipLaunchKernelGGL((k_gate_combine_wide<NB, RKS, F8>), dim3((unsigned)(8 * per_xcd)), dim3(kResThreads), 0, st,
                       (const typename StateT<F8>::type *)a.state, (const bf16_t *)a.gamma, (const bf16_t *)a.wu,
                       (bf16_t *)a.u, w, sh, ranges, per_xcd);
    return hipGetLastError();
}

template <int NB, bool F8>
hipError_t launch_k2_wide(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    switch (sh.rk / 32) {
    case 5: return launch_k2_wide_rks<NB, 5, F8>(a, sh, w, st);
    case 6: return launch_k2_wide_rks<NB, 6, F8>(a, sh, w, st);
    case 7: return launch_k2_wide_rks<NB, 7, F8>(a, sh, w, st);
    case 8: return launch_k2_wide_rks<NB, 8, F8>(a, sh, w, st);
    case 9: return launch_k2_wide_rks<NB, 9, F8>(a, sh, w, st);
    case 10: return launch_k2_wide_rks<NB, 10, F8>(a, sh, w, st);
    default: return hipErrorInvalidValue;
    }
}

template <int NB>
hipError_t launch_k2_resident(const ReadArgs &a, const FastShape &sh, const Workspace &w,
                              hipStream_t st) {
    switch (sh.rk / 32) {
    case 1: return launch_k2_resident_rks<NB, 1>(a, sh, w, st);
    case 2: return launch_k2_resident_rks<NB, 2>(a, sh, w, st);
    case 3: return launch_k2_resident_rks<NB, 3>(a, sh, w, st);
    case 4: return launch_k2_resident_rks<NB, 4>(a, sh, w, st);
    case 5: return launch_k2_resident_rks<NB, 5>(a, sh, w, st);
    case 6: return launch_k2_resident_rks<NB, 6>(a, sh, w, st);
    case 7: return launch_k2_resident_rks<NB, 7>(a, sh, w, st);
    case 8: return launch_k2_resident_rks<NB, 8>(a, sh, w, st);
    case 9: return launch_k2_resident_rks<NB, 9>(a, sh, w, st);
    case 10: return launch_k2_resident_rks<NB, 10>(a, sh, w, st);
    default: return hipErrorInvalidValue;
    }
}

// The resident kernel 2 pays a one-off W_up staging per workgroup; it wins
// once every workgroup walks a few token tiles.
constexpr int64_t kResidentMinTokens = 4096;
constexpr int64_t kResidentMinTokensFp8 = 1024;  // (e4m3: the staged form loses from ~1-2k tokens)
// The XCD-aware walk of a wide gate's kernel 2 wants several tiles per XCD.
constexpr int64_t kWideXcdMinTokens = 8 * 4 * kResTile;

}  // namespace

// one wave per workgroup up to this many tokens (the grid then reaches every CU)
constexpr int64_t kRedOneWaveBelow = 512;

template <int RW>
hipError_t launch_reduce_rw(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st, bool wide) {
    const dim3 rgrid((unsigned)((sh.N + RW - 1) / RW)), rblock(64 * RW);
    switch (sh.ksplit) {
    case 1:
        if (wide) hipLaunchKernelGGL((k_reduce_records<4, 1, 6, RW>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps);
        else hipLaunchKernelGGL((k_reduce_records<4, 1, 2, RW>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps);
        break;
    case 2:
        if (wide) hipLaunchKernelGGL((k_reduce_records<4, 2, 6, RW>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps);
        else hipLaunchKernelGGL((k_reduce_records<4, 2, 2, RW>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps);
        break;
    case 4: hipLaunchKernelGGL((k_reduce_records<4, 4, 2, RW>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    case 8: hipLaunchKernelGGL((k_reduce_records<4, 8, 2, RW>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    case 16: hipLaunchKernelGGL((k_reduce_records<4, 16, 2, RW>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_reduce(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    // a wide gate's records (more than 128 outputs) with one or two splits: all
    // of a lane's outputs in one round of loads
    const bool wide = sh.rk + 4 > 128;
    if (sh.N <= kRedOneWaveBelow) return launch_reduce_rw<1>(a, sh, w, st, wide);
    return launch_reduce_rw<4>(a, sh, w, st, wide);
}

hipError_t launch_kernel2(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    // an e4m3 state: the staged form (few tokens) or the resident form (narrow
    // gate), or the XCD walk (wide gate)
    if (a.fp8) {
        if (sh.rk > 128) return launch_k2_wide<4, true>(a, sh, w, st);
        const bool res8 = a.k2_variant == 2 || (a.k2_variant == 0 && sh.N >= kResidentMinTokensFp8);
        return res8 ? launch_k2_resident_fp8<4>(a, sh, w, st) : launch_k2<4, true>(a, sh, w, st);
    }
    // a wide gate (more than four k-steps) has the resident form only, walked
    // XCD by XCD once every XCD has several token tiles
    if (sh.rk > 128 && sh.N >= kWideXcdMinTokens && a.k2_variant != 2) return launch_k2_wide<4, false>(a, sh, w, st);
    const bool resident = sh.rk > 128 || a.k2_variant == 2 || (a.k2_variant == 0 && sh.N >= kResidentMinTokens);
    return resident ? launch_k2_resident<4>(a, sh, w, st) : launch_k2<4, false>(a, sh, w, st);
}

}  // namespace fast
}  // namespace grk
