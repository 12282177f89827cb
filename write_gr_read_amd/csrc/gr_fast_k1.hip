// gr_fast_k1.hip -- kernel 1 of the fast path (see gr_fast.hip for the whole
// call): the W' preparation and the three forms of kernel 1 -- the tile walk
// (k_stream_proj), the few-token form (k_stream_proj_small) and the wide-gate
// form (k_stream_proj_wide).  Each streams the state once: eq:write when fused,
// the sums of squares of eq:rms, and the down and write projections of eq:gate
// and eq:s on MFMA, ending in per-(token, branch, split) records ("Paper
// reading: Qwen3.8 Flash Next", part 2 Residual, sec. 4; one traversal per
// direction as in its sec. 7).
#include "gr_fast_common.h"

namespace grk {
namespace fast {
namespace {

// W' of every branch for the whole call: rows j < r of W_down, r..r+nw-1 of
// W_write, zero up to 16*row_blocks; times gamma; bf16 hi and lo planes,
// [n][2][rows][d].  The same arithmetic as kernel 1's own split.
__global__ void __launch_bounds__(256)
k_prep_wprime(const bf16_t *__restrict__ gamma, const bf16_t *__restrict__ wd,
              const bf16_t *__restrict__ ww, Workspace ws, FastShape sh) {
    const int d8 = sh.d / 8, rows_p = 16 * sh.row_blocks;
    const int64_t total = (int64_t)sh.n * rows_p * d8;
    const int64_t nd = (int64_t)sh.n * sh.d;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
        const int cv = (int)(q % d8);
        const int64_t rest = q / d8;
        const int j = (int)(rest % rows_p), i = (int)(rest / rows_p);
        const int64_t col = (int64_t)i * sh.d + cv * 8;
        const bf16_t *src = j < sh.r ? wd + (int64_t)j * nd
                          : (j < sh.rows ? ww + (int64_t)(j - sh.r) * nd : nullptr);
        u32x4 w = {0u, 0u, 0u, 0u}, gm = {0u, 0u, 0u, 0u};
        if (src) {
            w = *reinterpret_cast<const u32x4 *>(src + col);
            gm = *reinterpret_cast<const u32x4 *>(gamma + col);
        }
        u32x4 hi, lo;
        split_product(w, gm, hi, lo);
        *reinterpret_cast<u32x4 *>(ws.wprime + ((int64_t)(i * 2) * rows_p + j) * sh.d + cv * 8) = hi;
        *reinterpret_cast<u32x4 *>(ws.wprime + ((int64_t)(i * 2 + 1) * rows_p + j) * sh.d + cv * 8) = lo;
    }
}

// ---------------------------------------------------------------------------
// Kernel 1.  blockIdx -> (tile, branch, split), XCD-aware (blockIdx % 8 is the
// XCD under round-robin dispatch): the workgroups of a tile that share an XCD
// share y in its L2, and with four branches an XCD streams the W' of two of
// them (the mapping is spelled out in the kernel).
//
// Memory side: a round covers RC = 128 channels of the wave's 16 tokens.  One
// load instruction takes 4 tokens x 256 contiguous bytes (16 lanes per token
// row, adjacent lanes on adjacent 16-byte pieces), which HBM serves much
// better than 16 rows x 64 bytes; eq:write, its store and the sum of squares
// run in that layout.  The stored R' is also written to a wave-private LDS
// tile (16 tokens x 16 pieces at a pitch of 17 pieces, so both the row-wise
// writes and the column-wise MFMA reads are free of bank conflicts), from
// which the MFMA B operand (token = lane % 16, 8 channels of lane group
// lane / 16) is read.
//
// W' (W_down / W_write rows of the branch times gamma, as bf16 hi and lo
// planes) is read ready-made from the workspace, where k_prep_wprime wrote it
// once for the call (every token tile would otherwise redo the same split).
// It is staged in a double-buffered LDS slot per chunk: the chunk after next
// is loaded into registers while a chunk is used, with one barrier per chunk.
// The next round's state loads are issued as soon as the element phase has
// freed their registers, so they fly during the MFMA phase at no register
// cost; y (mostly an L2 hit: the n workgroups of a tile share it) is loaded at
// the start of its round.
template <bool FUSED, int NRB, bool F8>
__global__ void __launch_bounds__(kThreads, NRB <= 5 ? kK1WavesPerSimd : 2)
k_stream_proj(typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ y,
              const float *__restrict__ s_in, const bf16_t *__restrict__ gamma,
              const bf16_t *__restrict__ wd, const bf16_t *__restrict__ ww, Workspace ws,
              FastShape sh) {
    constexpr int WAVES = kWaves;                      // each wave carries 16 tokens
    constexpr int THREADS = 64 * WAVES;
    constexpr int NQ = 4;                              // load instructions per round (4 tokens each)
    constexpr int RC = 2 * kIter;                      // channels per round
    constexpr int PCS = RC / 8;                        // 16-byte pieces per token row and round
    constexpr int KS = kIter / kChunk;                 // MFMA k-steps per W' chunk
    // A staged W' row is kIter bf16 = eight 16-byte pieces, with piece p of row
    // `row` stored at p ^ ((row >> 1) & 7): the MFMA A reads (16 rows, one
    // piece each per lane group) then hit distinct banks, where a padded pitch
    // of 144 bytes still conflicted (~2e7 conflict cycles per call).  Rows
    // m16 and m16 + 16 k share the swizzle.
    constexpr int kPitch = kIter;                      // bf16 per staged W' row
    auto swz = [](int row) { return (row >> 1) & 7; };
    static_assert(kIter / 8 == 8, "the W' swizzle permutes eight 16-byte pieces per row");
    constexpr int NV = NRB * 16 * (kIter / 8);         // 16-byte vectors of W' per chunk (per plane)
    constexpr int WV = (2 * NV + THREADS - 1) / THREADS;  // hi and lo planes
    using T = typename StateT<F8>::type;
    using SV = typename StateT<F8>::vec8;              // 8 channels of the state
    static_assert(PCS == 16, "a round is 16 pieces of 8 channels per token");
    // [buffer][hi/lo][row][k]
    __shared__ __attribute__((aligned(16))) bf16_t lds_w[2][2][NRB * 16 * kPitch];
    constexpr int RP = PCS + 1;                        // LDS tile pitch in pieces (odd: no bank conflicts)
    __shared__ __attribute__((aligned(16))) u32x4 lds_r[WAVES][16 * RP];

    const int n = sh.n, d = sh.d, S = sh.ksplit;
    const int64_t b = blockIdx.x;
    // blockIdx % 8 is the XCD (round-robin dispatch).  With four branches, XCD
    // x takes branches 2 (x / 4) and 2 (x / 4) + 1 of the tiles T = x mod 4
    // (mod 4): an XCD then streams the W' of two branches (2.5 MB at the
    // prefill shape, within its 4 MB L2) instead of all four, and the two
    // workgroups of a tile on it (consecutive slots) still share y in L2.
    // Otherwise the n workgroups of a tile share an XCD.
    int64_t tile;
    int br, split;
    if (n == 4) {
        const int x = (int)(b % 8);
        const int64_t j = b / 8;
        split = (int)(j % S);
        br = 2 * (x / 4) + (int)((j / S) % 2);
        tile = (j / (2 * S)) * 4 + (x % 4);
    } else {
        tile = (b / 8 / (n * S)) * 8 + (b % 8);
        br = (int)((b / 8) % (n * S)) / S;
        split = (int)((b / 8) % S);
    }
    if (tile >= sh.tiles) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, m16 = lane & 15;
    const int64_t t0 = tile * kTile + wave * 16;        // first token of this wave
    const int64_t nd = (int64_t)n * d;
    const int chan = sh.ksplit_chan;                    // channels of this split (multiple of kIter)
    const int nit = chan / kIter;                       // W' chunks
    const int nround = (chan + RC - 1) / RC;
    const int c_base = split * chan;                    // first channel of this split
    const int rows_p = NRB * 16;
    // The rounds start at a rotation per tile (the n workgroups of a tile share
    // it, and with it their y reads from L2): the tiles running at one time then
    // stream four columns of their rows, a quarter of the row apart, instead of
    // all the same one, which HBM serves better; four offsets, not one per tile,
    // keep the W' chunks in use few enough to stay in L2.  Round s of the walk
    // is round rnd(s) of the split; the W' chunks follow, chunk i of the walk
    // being (c0 + i) mod nit.
    const int rot = k1_round_rotation(tile, nround);
    const int c0 = rot * (RC / kIter);
    auto rnd = [&](int s_) { return (s_ + rot) % nround; };   // s_ < nround

    // W' staging: vector v < NV of the hi plane, NV + v of the lo plane
    u32x4 wreg[WV];
    auto chunk_of = [&](int it) { const int c_ = c0 + it; return c_ >= nit ? c_ - nit : c_; };  // it < nit
    auto load_w = [&](int it) {
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * THREADS;
            const int plane = v / NV, rem = v % NV;
            const int row = rem / (kIter / 8), cv = rem % (kIter / 8);
            wreg[q] = u32x4{0u, 0u, 0u, 0u};
            if (v < 2 * NV && it < nit)
                wreg[q] = *reinterpret_cast<const u32x4 *>(
                    ws.wprime + ((int64_t)(br * 2 + plane) * rows_p + row) * d + c_base + chunk_of(it) * kIter + cv * 8);
        }
    };
    auto store_w = [&](int buf) {
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * THREADS;
            if (v < 2 * NV) {
                const int plane = v / NV, rem = v % NV;
                const int row = rem / (kIter / 8), cv = rem % (kIter / 8);
                *reinterpret_cast<u32x4 *>(&lds_w[buf][plane][row * kPitch + (cv ^ swz(row)) * 8]) = wreg[q];
            }
        }
    };

    // load instruction q: token t0 + 4q + g, piece m16 (channels 8*m16 .. +7 of the round)
    bool vq[NQ];
    float sq[NQ];
    float ss[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t t = t0 + 4 * q + g;
        vq[q] = t < sh.N;
        sq[q] = (FUSED && vq[q]) ? s_in[t * n + br] : 0.f;
        ss[q] = 0.f;
    }
    // addresses: a wave-uniform base (token t0, this branch and split) plus a
    // 32-bit lane offset; instruction q adds 4q tokens, round rd adds rd*RC
    T *const sbase = state + (t0 * n + br) * (int64_t)d + c_base;
    const bf16_t *const ybase = FUSED ? y + t0 * (int64_t)d + c_base : nullptr;
    const uint32_t soff = (uint32_t)(g * nd + 8 * m16), yoff = (uint32_t)(g * d + 8 * m16);
    const int64_t qstride = 4 * nd, qystride = 4 * (int64_t)d;

    SV rr[NQ];
    u32x4 yy[NQ];
    // load round `ar` of the split (valid: the walk has such a step): its
    // state (ds) and / or its y (dy)
    auto load_round = [&](int ar, bool valid, bool ds, bool dy) {
        const bool in = valid && ar * RC + 8 * m16 < chan;
        const T *const rs = sbase + ar * RC;                   // wave-uniform
        const bf16_t *const ry = FUSED ? ybase + ar * RC : nullptr;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (ds) rr[q] = SV{};
            if (dy) yy[q] = u32x4{0u, 0u, 0u, 0u};
            if (vq[q] && in) {
                if (ds) rr[q] = *reinterpret_cast<const SV *>(rs + q * qstride + soff);
                if (FUSED && dy) yy[q] = *reinterpret_cast<const u32x4 *>(ry + q * qystride + yoff);
            }
        }
    };

    f32x4 acc[NRB];
#pragma unroll
    for (int k = 0; k < NRB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 *my_r = lds_r[wave];

    load_w(0);
    store_w(0);
    load_w(1);
    load_round(rot, true, true, false);
    __syncthreads();
    int it = 0;                                         // W' chunks of the walk used so far
    int ar = rot;                                       // round of the split at walk step rd
    for (int rd = 0; rd < nround; ++rd) {
        const int an = ar + 1 == nround ? 0 : ar + 1;   // ... at step rd + 1
        load_round(ar, true, false, true);
        // eq:write in the load layout: store, sum of squares, LDS tile
        const bool in = ar * RC + 8 * m16 < chan;
        T *const ws_ = sbase + ar * RC;                          // wave-uniform
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            u32x4 w;  // the 8 stored values as bf16 (exact for an e4m3 state)
            if constexpr (F8) {
                u32x2 o = rr[q];
                if (FUSED) {
                    o = write8_fp8(sq[q], yy[q], rr[q]);
                    if (vq[q] && in) *reinterpret_cast<u32x2 *>(ws_ + q * qstride + soff) = o;
                }
                w = widen8_fp8_bf16(o);
            } else {
                w = rr[q];
                if (FUSED) {
                    w = write8_bf16(sq[q], yy[q], rr[q]);
                    if (vq[q] && in) *reinterpret_cast<u32x4 *>(ws_ + q * qstride + soff) = w;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ss[q] = dot2_bf16(w[e], w[e], ss[q]);
            my_r[(4 * q + g) * RP + m16] = w;
        }
        // the wave's LDS writes above complete before its reads below (LDS
        // instructions of a wave execute in order); keep the phases apart so
        // the element work and the MFMA operands are not live together
        __builtin_amdgcn_sched_barrier(0);
        load_round(an, rd + 1 < nround, true, false);
#pragma unroll
        for (int h = 0; h < RC / kIter; ++h) {
            if (ar * (RC / kIter) + h < nit) {               // chunk h of this round exists
                const int cur = it & 1;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int pc = (h * kIter + ks * kChunk) / 8 + g;   // piece of this lane group
                    const bf16x8 bop = as_bf16x8(my_r[m16 * RP + pc]);
                    const int pw = ((ks * kChunk / 8 + g) ^ swz(m16)) * 8;   // swizzled piece
                    const bf16_t *wh = &lds_w[cur][0][m16 * kPitch + pw];
                    const bf16_t *wl = &lds_w[cur][1][m16 * kPitch + pw];
#pragma unroll
                    for (int k = 0; k < NRB; ++k) {
                        const u32x4 ah = *reinterpret_cast<const u32x4 *>(wh + k * 16 * kPitch);
                        const u32x4 al = *reinterpret_cast<const u32x4 *>(wl + k * 16 * kPitch);
                        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), bop, acc[k], 0, 0, 0);
                        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), bop, acc[k], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (it + 1 < nit) store_w(cur ^ 1);
                load_w(it + 2);
                __syncthreads();
                ++it;
            }
        }
        ar = an;
    }

    // The record (ss, P) of this (token, branch, split); k_reduce_records,
    // launched next on the same stream, combines them.  ss of token 4q + g is
    // spread over the 16 lanes of lane group g.
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) ss[q] += __shfl_xor(ss[q], m, 64);
        if (m16 == 0 && vq[q])
            ws.partial[((t0 + 4 * q + g) * n + br) * S * (int64_t)sh.pstride + split * (int64_t)sh.pstride] = ss[q];
    }
    {
        const int64_t t = t0 + m16;  // MFMA column of this lane
        if (t < sh.N) {
            float *rec = ws.partial + ((t * n + br) * S + split) * (int64_t)sh.pstride;
#pragma unroll
            for (int k = 0; k < NRB; ++k) *reinterpret_cast<f32x4 *>(rec + 4 + 16 * k + 4 * g) = acc[k];
        }
    }
}

// Kernel 1, few-token form.  With few tokens the tile walk above has too few
// (tile, branch) units to fill the GPU, and each unit is a chain of rounds.
// Here a workgroup takes 16 TG tokens of one branch and a split of the
// channels, one slice of kpw k-steps (32 channels each) per wave, so a wave
// makes one short pass.  With TG = 2 (two 16-token groups) every W fragment a
// wave loads feeds the MFMAs of both groups: half the W reads per token, at
// twice the splits for the same number of workgroups.  A lane loads its state words straight in the MFMA B layout
// (token = lane % 16, 8 channels of lane group lane / 16): eq:write, its store
// and the sum of squares run there, with no LDS tile.  As in the wide form the
// contraction is P_i = W^{(i)} (gamma_i . R'_i): the raw W_down / W_write rows
// are the A operand, loaded straight from memory (row lane % 16 of each 16-row
// block, the same 8 channels), and gamma . R' -- exact in fp32 -- is split into
// bf16 hi + lo once per k-step as the B operand.  The waves' partial
// projections and sums of squares are added in LDS in wave order and written as
// the (token, branch, split) record that k_reduce_records expects.
// k-steps loaded together (one batch): four, or one for a wide gate (its
// NRB W fragments per k-step take 4 NRB VGPRs)
template <int NRB> constexpr int small_kb() { return NRB <= kMaxRowBlocks ? 4 : 1; }
// ... in the batch loop, where the loop's state takes registers too: two
// from 7 row blocks and with two token groups, so that nothing spills
template <int NRB, int TG> constexpr int small_loop_kb() {
    return NRB > kMaxRowBlocks ? 1 : (NRB >= 7 || TG > 1 ? 2 : 4);
}
constexpr int kSmallPass = kMaxRowBlocks;  // row blocks per pass of the LDS reduction
// ONEKB > 0: the wave's slice is one batch of at most ONEKB k-steps
// (decode-sized calls; ONEKB = 1, 2 or 4 as the slice needs, so that no
// k-step is loaded for nothing): straight-line code, so the compiler counts the
// loads in flight instead of waiting for all of them before the first element,
// and does not wait for the stores before the reduction (a loop, or a join
// with one, makes it do both).  ONEKB = 0: the slice in batches of small_loop_kb.
template <bool FUSED, int NRB, bool F8, int ONEKB, int TG>
__global__ void __launch_bounds__(64 * kSmallWaves, 2)
k_stream_proj_small(typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ y,
                    const float *__restrict__ s_in, const bf16_t *__restrict__ gamma,
                    const bf16_t *__restrict__ wd, const bf16_t *__restrict__ ww, Workspace ws,
                    FastShape sh) {
    using T = typename StateT<F8>::type;
    using SV = typename StateT<F8>::vec8;
    constexpr int kSmallKB = ONEKB > 0 ? ONEKB : small_loop_kb<NRB, TG>();
    constexpr int PB = NRB < kSmallPass ? NRB : kSmallPass;   // row blocks per reduction pass
    constexpr int NPASS = (NRB + PB - 1) / PB;
    constexpr int ACC = 4 * PB;                                // words per lane, group and pass
    constexpr int TOKW = 16 * TG;                              // tokens of a workgroup (and of each wave)
    // per wave: a pass's accumulators of each token group, then the groups' ss
    __shared__ float lds_p[kSmallWaves][TG * ACC + TG][64];
    const int n = sh.n, d = sh.d, S = sh.ksplit, kpw = sh.small_kpw;
    // blockIdx -> (token group, branch, split) with (branch, split) fastest, so
    // the workgroups reading one slice of W sit on one XCD when n S % 8 == 0
    const int64_t b = blockIdx.x;
    const int bs = (int)(b % (n * S));
    const int64_t tg = b / (n * S);
    const int br = bs / S, split = bs % S;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, m16 = lane & 15;
    const int64_t nd = (int64_t)n * d;
    const int c_wave = (split * kSmallWaves + wave) * kpw * kChunk;
    // token group j of the wave: this lane's token (MFMA column) tg TOKW + 16 j + m16
    bool valid[TG];
    float sv[TG];
    T *srow[TG];
    const bf16_t *yrow[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) {
        const int64_t t = tg * TOKW + 16 * j + m16;
        valid[j] = t < sh.N;
        sv[j] = (FUSED && valid[j]) ? s_in[t * n + br] : 0.f;
        // rows of a token past the end are never read or written: point at token 0
        const int64_t tv = valid[j] ? t : 0;
        srow[j] = state + (tv * n + br) * (int64_t)d;
        yrow[j] = FUSED ? y + tv * (int64_t)d : nullptr;
    }

    f32x4 acc[TG][NRB];
    float ss[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) {
        ss[j] = 0.f;
#pragma unroll
        for (int k = 0; k < NRB; ++k) acc[j][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // one batch of kSmallKB k-steps starting at k-step kb of the wave's slice
    auto batch = [&](int kb) {
        SV rr[TG][kSmallKB];
        u32x4 yy[TG][kSmallKB], gm[kSmallKB], wv[kSmallKB][NRB];
        bool kin[kSmallKB];
        // Every load is issued unconditionally (a masked one reads the start of
        // its tensor) and its value zeroed after: with the loads under
        // branches the compiler waits for all of them before the first use.
        constexpr u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ks = 0; ks < kSmallKB; ++ks) {
            const int c0 = c_wave + (kb + ks) * kChunk;   // whole 32-channel chunk in or out (d % 32 == 0)
            kin[ks] = kb + ks < kpw && c0 < d;
            const int c = c0 + 8 * g;
#pragma unroll
            for (int j = 0; j < TG; ++j) {
                const bool okr = kin[ks] && valid[j];
                const SV rv = *reinterpret_cast<const SV *>(okr ? srow[j] + c : state);
                rr[j][ks] = okr ? rv : SV{};
                if (FUSED) {
                    const u32x4 yv = *reinterpret_cast<const u32x4 *>(okr ? yrow[j] + c : y);
                    yy[j][ks] = okr ? yv : z4;
                } else {
                    yy[j][ks] = z4;
                }
            }
            const u32x4 gv = *reinterpret_cast<const u32x4 *>(kin[ks] ? gamma + (int64_t)br * d + c : gamma);
            gm[ks] = kin[ks] ? gv : z4;
#pragma unroll
            for (int k = 0; k < NRB; ++k) {
                const int row = 16 * k + m16;
                const bool okw = kin[ks] && row < sh.rows;
                const bf16_t *src = row < sh.r ? wd + (int64_t)row * nd
                                  : (okw ? ww + (int64_t)(row - sh.r) * nd : wd);
                const u32x4 wvv = *reinterpret_cast<const u32x4 *>(okw ? src + (int64_t)br * d + c : wd);
                wv[ks][k] = okw ? wvv : z4;
            }
        }
#pragma unroll
        for (int ks = 0; ks < kSmallKB; ++ks) {
            const int c = c_wave + (kb + ks) * kChunk + 8 * g;
#pragma unroll
            for (int j = 0; j < TG; ++j) {
                u32x4 w;  // the 8 stored values as bf16 (exact for an e4m3 state)
                if constexpr (F8) {
                    u32x2 o = rr[j][ks];
                    if (FUSED) {
                        o = write8_fp8(sv[j], yy[j][ks], rr[j][ks]);
                        if (valid[j] && kin[ks]) *reinterpret_cast<u32x2 *>(srow[j] + c) = o;
                    }
                    w = widen8_fp8_bf16(o);
                } else {
                    w = rr[j][ks];
                    if (FUSED) {
                        w = write8_bf16(sv[j], yy[j][ks], rr[j][ks]);
                        if (valid[j] && kin[ks]) *reinterpret_cast<u32x4 *>(srow[j] + c) = w;
                    }
                }
                // masked lanes and chunks hold zeros: they add nothing below
#pragma unroll
                for (int e = 0; e < 4; ++e) ss[j] = dot2_bf16(w[e], w[e], ss[j]);
                // B = gamma . R' as bf16 hi + lo (exact fp32 product split once per
                // k-step); A = the raw W rows, shared by the TG token groups
                u32x4 bh, bl;
                split_product(w, gm[ks], bh, bl);
#pragma unroll
                for (int k = 0; k < NRB; ++k) {
                    acc[j][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[ks][k]), as_bf16x8(bh), acc[j][k], 0, 0, 0);
                    acc[j][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[ks][k]), as_bf16x8(bl), acc[j][k], 0, 0, 0);
                }
            }
        }
    };
    if constexpr (ONEKB > 0) {
        batch(0);
    } else {
        for (int kb = 0; kb < kpw; kb += kSmallKB) batch(kb);
    }
    // this wave's share of ss per token: the four lane groups hold its channels
#pragma unroll
    for (int j = 0; j < TG; ++j) {
        ss[j] += __shfl_xor(ss[j], 16, 64);
        ss[j] += __shfl_xor(ss[j], 32, 64);
    }
    // add the waves' accumulators in LDS, PB row blocks per pass (ss with the first)
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        if (ps > 0) __syncthreads();                      // the previous pass is read
#pragma unroll
        for (int j = 0; j < TG; ++j) {
#pragma unroll
            for (int k = 0; k < PB; ++k)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (ps * PB + k < NRB) lds_p[wave][j * ACC + 4 * k + m][lane] = acc[j][ps * PB + k][m];
            if (ps == 0) lds_p[wave][TG * ACC + j][lane] = ss[j];
        }
        __syncthreads();
        // words j ACC + 4 k + m (m < 4) of lane l: P rows 16(ps PB + k) + 4(l/16) + m
        // of token 16 j + l%16, consecutive in its record, so a thread sums the
        // four (waves in order) and stores them as one 16-byte vector; word
        // TG ACC + j: ss of token 16 j + l%16 (first pass)
        const int blocks = ps * PB + PB <= NRB ? PB : NRB - ps * PB;   // row blocks of this pass
        for (int v = tid; v < TG * PB * 64; v += 64 * kSmallWaves) {
            const int qi = v >> 6, l = v & 63;
            const int jg = qi / PB, k = qi - jg * PB;
            const int64_t tt = tg * TOKW + 16 * jg + (l & 15);
            if (tt >= sh.N || k >= blocks) continue;
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kSmallWaves; ++w)
#pragma unroll
                for (int m = 0; m < 4; ++m) sum[m] += lds_p[w][jg * ACC + 4 * k + m][l];
            float *rec = ws.partial + ((tt * n + br) * S + split) * (int64_t)sh.pstride;
            *reinterpret_cast<f32x4 *>(rec + 4 + 16 * (ps * PB + k) + 4 * (l >> 4)) = sum;
        }
        if (ps == 0 && tid < 16 * TG) {
            const int jg = tid >> 4, l = tid & 15;
            const int64_t tt = tg * TOKW + 16 * jg + l;
            if (tt < sh.N) {
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < kSmallWaves; ++w) sum += lds_p[w][TG * ACC + jg][l];
                ws.partial[((tt * n + br) * S + split) * (int64_t)sh.pstride] = sum;
            }
        }
    }
}

// Kernel 1, wide form (r + n > 128; bf16 or e4m3 state, loaded and written as
// in k_stream_proj).  Same walk, load layout,
// eq:write and records as k_stream_proj, but the contraction is arranged so
// that the weights cost one LDS plane instead of two:
//   P_i = W^{(i)} (gamma_i . R'_i),
// with W^{(i)} the raw W_down / W_write columns of branch i (exact bf16, the
// MFMA A operand, staged 32 channels at a time, double-buffered) and
// gamma_i . R'_i -- exact in fp32, 16 significant bits -- carried as two bf16
// words hi + lo in two wave-private LDS tiles (the B operand; the same split as
// W' above, applied on the state side).  Every A fragment read from LDS then
// feeds two MFMAs.  One workgroup per CU (the W chunks and B tiles take
// ~123 KB of LDS); NRB * 4 accumulators per lane, so two waves per SIMD: the
// state / y words of the next two rounds are kept in flight (two register
// slots, each refilled as soon as its round's element phase is done).
template <bool FUSED, int NRB, bool F8>
__global__ void __launch_bounds__(kThreads, 2)
k_stream_proj_wide(typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ y,
                   const float *__restrict__ s_in, const bf16_t *__restrict__ gamma,
                   const bf16_t *__restrict__ wd, const bf16_t *__restrict__ ww, Workspace ws,
                   FastShape sh) {
    constexpr int NQ = 4;                              // load instructions per round (4 tokens each)
    constexpr int RC = 128;                            // channels per round
    constexpr int PCS = RC / 8;                        // 16-byte pieces per token row and round
    constexpr int KW = kChunk;                         // channels per W chunk (one MFMA k-step)
    constexpr int CPR = RC / KW;                       // W chunks per round
    constexpr int kPitch = KW + 8;                     // bf16 per staged W row (odd number of 16-byte units)
    constexpr int NV = NRB * 16 * (KW / 8);            // 16-byte vectors of W per chunk
    constexpr int WV = (NV + kThreads - 1) / kThreads;
    constexpr int RP = PCS + 1;                        // B tile pitch in pieces (odd: no bank conflicts)
    using T = typename StateT<F8>::type;
    using SV = typename StateT<F8>::vec8;              // 8 channels of the state
    __shared__ __attribute__((aligned(16))) bf16_t lds_w[2][NRB * 16 * kPitch];
    __shared__ __attribute__((aligned(16))) u32x4 lds_b[kWaves][2][16 * RP];   // hi, lo

    const int n = sh.n, d = sh.d, S = sh.ksplit;
    const int64_t b = blockIdx.x;
    // blockIdx % 8 is the XCD (round-robin dispatch).  With four branches, XCD
    // x takes branches 2 (x / 4) and 2 (x / 4) + 1 of the tiles T = x mod 4
    // (mod 4), as kernel 1's narrow walk does: an XCD streams the W rows of two
    // branches instead of four, and the two workgroups of a tile on it
    // (consecutive slots) share y in L2.  Otherwise the n workgroups of a tile
    // share an XCD.
    int64_t tile;
    int br, split;
    if (n == 4) {
        const int x = (int)(b % 8);
        const int64_t j = b / 8;
        split = (int)(j % S);
        br = 2 * (x / 4) + (int)((j / S) % 2);
        tile = (j / (2 * S)) * 4 + (x % 4);
    } else {
        tile = (b / 8 / (n * S)) * 8 + (b % 8);
        br = (int)((b / 8) % (n * S)) / S;
        split = (int)((b / 8) % S);
    }
    if (tile >= sh.tiles) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, m16 = lane & 15;
    const int64_t t0 = tile * kTile + wave * 16;        // first token of this wave
    const int64_t nd = (int64_t)n * d;
    const int chan = sh.ksplit_chan;                    // channels of this split (multiple of 64)
    const int nit = chan / KW;                          // W chunks
    const int nround = (chan + RC - 1) / RC;
    const int c_base = split * chan;

    // W staging: row j < r from W_down, r .. r+nw-1 from W_write, the rest zero
    u32x4 wreg[WV];
    auto load_w = [&](int it) {
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * kThreads;
            const int row = v / (KW / 8), cv = v % (KW / 8);
            const bf16_t *src = nullptr;
            if (v < NV && it < nit) {
                if (row < sh.r) src = wd + (int64_t)row * nd;
                else if (row < sh.rows) src = ww + (int64_t)(row - sh.r) * nd;
            }
            wreg[q] = src ? *reinterpret_cast<const u32x4 *>(src + (int64_t)br * d + c_base + it * KW + cv * 8)
                          : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_w = [&](int buf) {
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * kThreads;
            if (v < NV) {
                const int row = v / (KW / 8), cv = v % (KW / 8);
                *reinterpret_cast<u32x4 *>(&lds_w[buf][row * kPitch + cv * 8]) = wreg[q];
            }
        }
    };

    // load instruction q: token t0 + 4q + g, piece m16 (channels 8*m16 .. +7 of the round)
    bool vq[NQ];
    float sq[NQ], ss[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t t = t0 + 4 * q + g;
        vq[q] = t < sh.N;
        sq[q] = (FUSED && vq[q]) ? s_in[t * n + br] : 0.f;
        ss[q] = 0.f;
    }
    T *const sbase = state + (t0 * n + br) * (int64_t)d + c_base;
    const bf16_t *const ybase = FUSED ? y + t0 * (int64_t)d + c_base : nullptr;
    const bf16_t *const gbase = gamma + (int64_t)br * d + c_base + 8 * m16;
    const uint32_t soff = (uint32_t)(g * nd + 8 * m16), yoff = (uint32_t)(g * d + 8 * m16);
    const int64_t qstride = 4 * nd, qystride = 4 * (int64_t)d;

    // two slots of state / y words: round rd uses slot rd % 2, and the loads
    // of round rd + 2 go into that slot as soon as its element phase is done
    SV rrA[NQ], rrB[NQ];
    u32x4 yyA[NQ], yyB[NQ];
    auto load_round = [&](int rd, SV (&rr)[NQ], u32x4 (&yy)[NQ]) {
        const bool in = rd < nround && rd * RC + 8 * m16 < chan;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            rr[q] = (vq[q] && in) ? *reinterpret_cast<const SV *>(sbase + q * qstride + rd * RC + soff) : SV{};
            yy[q] = (FUSED && vq[q] && in) ? *reinterpret_cast<const u32x4 *>(ybase + q * qystride + rd * RC + yoff)
                                           : u32x4{0u, 0u, 0u, 0u};
        }
    };

    f32x4 acc[NRB];
#pragma unroll
    for (int k = 0; k < NRB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 *my_hi = lds_b[wave][0], *my_lo = lds_b[wave][1];

    auto do_round = [&](int rd, SV (&rr)[NQ], u32x4 (&yy)[NQ]) {
        const bool in = rd * RC + 8 * m16 < chan;
        const u32x4 gm = in ? *reinterpret_cast<const u32x4 *>(gbase + rd * RC) : u32x4{0u, 0u, 0u, 0u};
        // eq:write in the load layout: store, sum of squares, gamma . R' as hi / lo tiles
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            u32x4 w;  // the 8 stored values as bf16 (exact for an e4m3 state)
            if constexpr (F8) {
                u32x2 o = rr[q];
                if (FUSED) {
                    o = write8_fp8(sq[q], yy[q], rr[q]);
                    if (vq[q] && in) *reinterpret_cast<u32x2 *>(sbase + q * qstride + rd * RC + soff) = o;
                }
                w = widen8_fp8_bf16(o);
            } else {
                w = rr[q];
                if (FUSED) {
                    w = write8_bf16(sq[q], yy[q], rr[q]);
                    if (vq[q] && in) *reinterpret_cast<u32x4 *>(sbase + q * qstride + rd * RC + soff) = w;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ss[q] = dot2_bf16(w[e], w[e], ss[q]);
            u32x4 hi, lo;
            split_product(w, gm, hi, lo);
            my_hi[(4 * q + g) * RP + m16] = hi;
            my_lo[(4 * q + g) * RP + m16] = lo;
        }
        __builtin_amdgcn_sched_barrier(0);
        load_round(rd + 2, rr, yy);
#pragma unroll
        for (int h = 0; h < CPR; ++h) {
            const int it = rd * CPR + h;
            if (it < nit) {
                const int cur = it & 1;
                const int pc = h * (KW / 8) + g;             // piece of this lane group
                const bf16x8 bh = as_bf16x8(my_hi[m16 * RP + pc]);
                const bf16x8 bl = as_bf16x8(my_lo[m16 * RP + pc]);
                const bf16_t *wp = &lds_w[cur][m16 * kPitch + 8 * g];
#pragma unroll
                for (int k = 0; k < NRB; ++k) {
                    const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(wp + k * 16 * kPitch));
                    acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[k], 0, 0, 0);
                    acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[k], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (it + 1 < nit) store_w(cur ^ 1);
                load_w(it + 2);
                __syncthreads();
            }
        }
    };

    load_w(0);
    store_w(0);
    load_w(1);
    load_round(0, rrA, yyA);
    load_round(1, rrB, yyB);
    __syncthreads();
    for (int rd = 0; rd < nround; rd += 2) {
        do_round(rd, rrA, yyA);
        if (rd + 1 < nround) do_round(rd + 1, rrB, yyB);
    }

    // the record (ss, P) of this (token, branch, split)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) ss[q] += __shfl_xor(ss[q], m, 64);
        if (m16 == 0 && vq[q])
            ws.partial[((t0 + 4 * q + g) * n + br) * S * (int64_t)sh.pstride + split * (int64_t)sh.pstride] = ss[q];
    }
    const int64_t t = t0 + m16;  // MFMA column of this lane
    if (t < sh.N) {
        float *rec = ws.partial + ((t * n + br) * S + split) * (int64_t)sh.pstride;
#pragma unroll
        for (int k = 0; k < NRB; ++k) *reinterpret_cast<f32x4 *>(rec + 4 + 16 * k + 4 * g) = acc[k];
    }
}

// The few-token kernel 1 at the batch size its slice needs and the token
// groups per wave the shape asks for (see k_stream_proj_small).
template <bool FUSED, int NRB, bool F8, int TG>
void launch_small_tg(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    using T = typename StateT<F8>::type;
    constexpr int KB = small_kb<NRB>();
    const unsigned sgrid = (unsigned)(((sh.N + 16 * TG - 1) / (16 * TG)) * sh.n * sh.ksplit);
    const dim3 block(64 * kSmallWaves);
    const bf16_t *y = (const bf16_t *)a.y, *gm = (const bf16_t *)a.gamma;
    const bf16_t *wd = (const bf16_t *)a.wd, *ww = (const bf16_t *)a.ww;
    if (sh.small_kpw <= 1) {
        hipLaunchKernelGGL((k_stream_proj_small<FUSED, NRB, F8, 1, TG>), dim3(sgrid), block, 0, st,
                           (T *)a.state, y, a.s_in, gm, wd, ww, w, sh);
        return;
    }
    if constexpr (KB >= 4) {
        if (sh.small_kpw <= 2)
            hipLaunchKernelGGL((k_stream_proj_small<FUSED, NRB, F8, 2, TG>), dim3(sgrid), block, 0, st,
                               (T *)a.state, y, a.s_in, gm, wd, ww, w, sh);
        else if (sh.small_kpw <= 4)
            hipLaunchKernelGGL((k_stream_proj_small<FUSED, NRB, F8, 4, TG>), dim3(sgrid), block, 0, st,
                               (T *)a.state, y, a.s_in, gm, wd, ww, w, sh);
        else
            hipLaunchKernelGGL((k_stream_proj_small<FUSED, NRB, F8, 0, TG>), dim3(sgrid), block, 0, st,
                               (T *)a.state, y, a.s_in, gm, wd, ww, w, sh);
    } else {
        hipLaunchKernelGGL((k_stream_proj_small<FUSED, NRB, F8, 0, TG>), dim3(sgrid), block, 0, st,
                           (T *)a.state, y, a.s_in, gm, wd, ww, w, sh);
    }
}

template <bool FUSED, int NRB, bool F8>
void launch_small(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    if constexpr (NRB <= kSmallTg2MaxRB) {
        if (sh.small_tg == 2) {
            launch_small_tg<FUSED, NRB, F8, 2>(a, sh, w, st);
            return;
        }
    }
    launch_small_tg<FUSED, NRB, F8, 1>(a, sh, w, st);
}

template <bool FUSED, bool F8>
hipError_t launch_k1(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    using T = typename StateT<F8>::type;
    const int64_t tiles8 = (sh.tiles + 7) / 8 * 8;
    const unsigned grid = (unsigned)(tiles8 * sh.n * sh.ksplit);
    const bf16_t *y = (const bf16_t *)a.y;
    if (sh.prep) {
        const int64_t total = (int64_t)sh.n * 16 * sh.row_blocks * (sh.d / 8);
        const int64_t blocks = (total + 255) / 256;
        hipLaunchKernelGGL(k_prep_wprime, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st,
                           (const bf16_t *)a.gamma, (const bf16_t *)a.wd, (const bf16_t *)a.ww, w, sh);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
#define GR_K1(NRB)                                                                          \
    case NRB:                                                                               \
        hipLaunchKernelGGL((k_stream_proj<FUSED, NRB, F8>), dim3(grid), dim3(kThreads), 0, st, \
                           (T *)a.state, y, a.s_in, (const bf16_t *)a.gamma,                \
                           (const bf16_t *)a.wd, (const bf16_t *)a.ww, w, sh);              \
        break;
    if (sh.small) {
#define GR_K1S(NRB)                                                                         \
    case NRB:                                                                               \
        launch_small<FUSED, NRB, F8>(a, sh, w, st);                                         \
        break;
        switch (sh.row_blocks) {
            GR_K1S(1) GR_K1S(2) GR_K1S(3) GR_K1S(4) GR_K1S(5) GR_K1S(6) GR_K1S(7) GR_K1S(8)
            GR_K1S(9) GR_K1S(10) GR_K1S(11) GR_K1S(12) GR_K1S(13) GR_K1S(14) GR_K1S(15)
            GR_K1S(16) GR_K1S(17) GR_K1S(18) GR_K1S(19) GR_K1S(20) GR_K1S(21)
        default: return hipErrorInvalidValue;
        }
#undef GR_K1S
        return hipGetLastError();
    }
    if (sh.wide) {
#define GR_K1W(NRB)                                                                         \
    case NRB:                                                                               \
        hipLaunchKernelGGL((k_stream_proj_wide<FUSED, NRB, F8>), dim3(grid), dim3(kThreads), 0, st, \
                           (T *)a.state, y, a.s_in, (const bf16_t *)a.gamma,                \
                           (const bf16_t *)a.wd, (const bf16_t *)a.ww, w, sh);              \
        break;
        switch (sh.row_blocks) {
            GR_K1W(9) GR_K1W(10) GR_K1W(11) GR_K1W(12) GR_K1W(13) GR_K1W(14) GR_K1W(15)
            GR_K1W(16) GR_K1W(17) GR_K1W(18) GR_K1W(19) GR_K1W(20) GR_K1W(21)
        default: return hipErrorInvalidValue;
        }
#undef GR_K1W
        return hipGetLastError();
    }
    switch (sh.row_blocks) {
        GR_K1(1) GR_K1(2) GR_K1(3) GR_K1(4) GR_K1(5) GR_K1(6) GR_K1(7) GR_K1(8)
    default: return hipErrorInvalidValue;
    }
#undef GR_K1
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kernel1(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    return a.fp8 ? (a.fused ? launch_k1<true, true>(a, sh, w, st) : launch_k1<false, true>(a, sh, w, st))
                 : (a.fused ? launch_k1<true, false>(a, sh, w, st) : launch_k1<false, false>(a, sh, w, st));
}

}  // namespace fast
}  // namespace grk
