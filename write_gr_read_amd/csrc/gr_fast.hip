// gr_fast.hip -- MFMA fast path of the GR read / fused write+read for a bf16
// or e4m3 widened state ("Paper reading: Qwen3.8 Flash Next", part 2
// Residual, sec. 4 Gated Residual: eq:rms, eq:gate, eq:use_gate, eq:s;
// eq:write first when fused; sec. 7: read fused into one traversal with Group
// RMSNorm, and the FP8 state).
//
// Up to four kernels in stream order, no inter-workgroup waiting (so no
// co-residency assumption).  Below, the narrow-gate (r + n <= 128) forms at
// many tokens; an e4m3 state uses the same kernel 1 template and its own
// resident kernel 2 (k_gate_combine_resident_fp8), a wide gate (r up to 320,
// the pages' r = d/8 at d = 2560) has its own kernel 1 and 2
// (k_stream_proj_wide, k_gate_combine_wide), and below 1024 tokens (512 for a
// wide gate) kernel 1 is k_stream_proj_small; each is described where it is
// defined.
//
// k_prep_wprime   (tile walk) W' = (W_down ; W_write) . gamma per branch,
//                 split once into bf16 hi / lo planes for the whole call.
// k_stream_proj   one workgroup per (token tile of 16*WAVES tokens, branch i).
//                 Streams branch i of the tile once: (fused) R' = R + s_i y in
//                 fp32, rounded to bf16 and stored; sum of squares of the stored
//                 values (v_dot2_f32_bf16); and the down projection
//                 P_i = W'^{(i)} R'_i on MFMA (v_mfma_f32_16x16x32_bf16), where
//                 W' stacks W_down's and W_write's columns of branch i with the
//                 gain gamma_i folded in.  Because
//                     W_down vec(R-hat) = sum_i rho_i W_down^{(i)} (gamma_i . R_i)
//                 the projections need no second sweep: rho_i is applied after.
//                 Each workgroup writes a record (ss_i, P_i) per token.
// k_reduce_records  one wave per token: rho_i = (ss_i/d + eps)^-1/2,
//                 z = (1/n) sum_i rho_i P_i, a = SiLU(z),
//                 s = 2 sigmoid((1/n) sum_i rho_i P_i[r + .]).
// k_gate_combine  one workgroup per (token tile, channel range) -- or, for
//                 many tokens, per (channel range, tile residue), walking
//                 tiles with the range's W_up resident.  Up projection
//                 t = W_up (-log2(e) a) on MFMA, then per element
//                 G_i rho_i = 1 / ((1 + 2^t) rms_i) and
//                 u_c = sum_i (gamma_ic / n) R'_ic / ((1 + 2^t_ic) rms_i).
//
// Precision: an fp32 operand x of a contraction is carried as two bf16 words,
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (16 significant bits), and
// multiplied in two MFMAs with fp32 accumulation.  This is done for W'
// (W_down / W_write with gamma folded in) and for -log2(e) a; the state and
// W_up enter as stored (exact bf16).
//
// MFMA operand convention (16x16x32 bf16): lane l holds A[l%16][8(l/16)+e] and
// B[8(l/16)+e][l%16], e = 0..7; the result D[4(l/16)+m][l%16], m = 0..3.
// A and B use the same k assignment, so the contraction is independent of how
// the hardware orders k inside a lane group.
#include "gr_device.h"
#include "gr_internal.h"

namespace grk {

namespace {

constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16 * kWaves;        // tokens per workgroup
constexpr int kChunk = 32;                // channels per MFMA k-step

#ifndef GR_K1_DEPTH
#define GR_K1_DEPTH 0
#endif
constexpr int kIter = 64;                 // channels per W' chunk of kernel 1 (a round is two)
constexpr int kDepth = GR_K1_DEPTH;       // kernel 1: rounds of state / y loads in flight ahead
#ifndef GR_K1_TG
#define GR_K1_TG 1
#endif
constexpr int kTG = GR_K1_TG;             // 16-token MFMA column groups per kernel-1 wave
#ifndef GR_K2_WAVES_PER_SIMD
#define GR_K2_WAVES_PER_SIMD 3
#endif
#ifndef GR_K2_WAVES
#define GR_K2_WAVES 4
#endif
constexpr int kK2WavesPerSimd = GR_K2_WAVES_PER_SIMD;  // occupancy target of kernel 2
constexpr int kK2Waves = GR_K2_WAVES;                  // waves per kernel-2 workgroup
constexpr int kK2Threads = 64 * kK2Waves;
constexpr int kK2Tile = 16 * kK2Waves;                 // tokens per kernel-2 workgroup
#ifndef GR_K2_SUB
#define GR_K2_SUB 1
#endif
constexpr int kK2Sub = GR_K2_SUB;  // 32-channel chunks per kernel-2 iteration (whole 128-byte lines)
constexpr int kMaxRowBlocks = 8;          // (r + n) padded to 16, at most 128 (narrow gate)
constexpr int kMaxWideRowBlocks = 21;     // wide gate (kernel 1 wide form): r + n up to 336
constexpr int kMaxWideRKS = 10;           // wide gate: r up to 320 (k-steps of 32 of the up projection)
constexpr int kChanPerWg = 256;           // channels per k_gate_combine workgroup
#ifndef GR_SPLIT_TARGET
#define GR_SPLIT_TARGET 256
#endif
constexpr int kSplitTarget = GR_SPLIT_TARGET;  // kernel-1 workgroups wanted before splitting channels
constexpr int kMaxSplit = 16;             // channel splits of kernel 1 (a power of two)
#ifndef GR_SMALL_BELOW
#define GR_SMALL_BELOW 32
#endif
constexpr int kSmallBelow = GR_SMALL_BELOW;  // ... used while (token tiles) x n is below this
constexpr int kSmallBelowWide = 16;          // ... for a wide gate
#ifndef GR_SMALL_TARGET
#define GR_SMALL_TARGET 256
#endif
constexpr int kSmallTarget = GR_SMALL_TARGET;  // few-token kernel 1: workgroups wanted before splitting
constexpr int kSmallWaves = 8;            // waves per few-token kernel-1 workgroup


struct FastShape {
    int n, d, r, nw;     // nw = n if W_write given, else 0
    int rows;            // r + nw
    int row_blocks;      // ceil(rows / 16)
    int pstride;         // floats per (token, branch, split) partial record
    int ksplit;          // channel splits of kernel 1 (workgroups per (tile, branch))
    int ksplit_chan;     // channels per split (multiple of kIter)
    int k2_chan;         // channels per kernel-2 workgroup (multiple of kChunk)
    int rk;              // r padded to a multiple of 32 (k-steps of the up projection)
    bool prep;           // W' split once per call by k_prep_wprime (enough token tiles)
    bool wide;           // r + n beyond 128: kernel 1's wide form (gamma on the state side, no W')
    bool small;          // few tokens: kernel 1's few-token form (k_stream_proj_small)
    int small_kpw;       // ... its k-steps (32 channels) per wave
    int64_t N, tiles;
};

FastShape shape_of(const ReadArgs &a) {
    FastShape s;
    s.n = a.n; s.d = a.d; s.r = a.r;
    s.nw = a.ww ? a.n : 0;
    s.rows = s.r + s.nw;
    s.row_blocks = (s.rows + 15) / 16;
    s.pstride = 4 + 16 * s.row_blocks;
    s.rk = (s.r + 31) / 32 * 32;
    s.N = a.N;
    s.tiles = (a.N + kTile - 1) / kTile;
    // Enough workgroups to fill the GPU below ~16k tokens: split the channels
    // of kernel 1's tile walk (partial records are summed in the tile
    // reduction) and narrow the channel range of the staged kernel 2.
    int ks = 1;
    while (s.tiles * s.n * ks < kSplitTarget && ks < kMaxSplit && (s.d / (ks * 2)) % kIter == 0 &&
           s.d / (ks * 2) >= 2 * kIter)
        ks *= 2;
    s.ksplit = ks;
    s.ksplit_chan = s.d / ks;
    int c2 = kChanPerWg;
    const int64_t tiles2 = (a.N + kK2Tile - 1) / kK2Tile;
    while (tiles2 * ((s.d + c2 - 1) / c2) < 1024 && c2 > kChunk && (c2 / 2) % kChunk == 0) c2 /= 2;
    s.k2_chan = c2;
    s.wide = s.row_blocks > kMaxRowBlocks;
    // Few tokens: kernel 1's few-token form (narrow or wide gate), whose workgroups are
    // (16 tokens, branch, split); splits (a power of two, at most kMaxSplit)
    // until the grid has kSmallTarget workgroups or a wave's slice is one k-step.
    s.small = false;
    s.small_kpw = 0;
    if (s.tiles * s.n < (s.wide ? kSmallBelowWide : kSmallBelow)) {
        const int64_t groups = (s.N + 15) / 16;
        int sp = 1;
        while (groups * s.n * sp < kSmallTarget && sp < kMaxSplit && s.d / (2 * sp) >= kSmallWaves * kChunk) sp *= 2;
        const int per = kSmallWaves * kChunk * sp;   // channels covered per k-step of every wave
        s.small = true;
        s.ksplit = sp;
        s.ksplit_chan = 0;
        s.small_kpw = (s.d + per - 1) / per;
    }
    // the tile walk of a narrow gate (at least 8 tiles) reads W' split once per call
    s.prep = !s.wide && !s.small;
    return s;
}

// Workspace layout (all offsets 256-byte aligned; every region is written
// before it is read within a call, so no initialisation is needed):
//   partial   [N][n][ksplit][pstride] f32: ss at [0], projection rows at [4 ..]
//   act       [N][2][rk] bf16     -log2(e) SiLU(z) as hi, lo words, zero-padded
//   rms       [N][n] f32          1/rho
//   wprime    [n][2][16*row_blocks][d] bf16   W' hi and lo planes (narrow gate only)
struct Workspace {
    float *partial;
    bf16_t *act;
    float *rms;
    bf16_t *wprime;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_layout(const FastShape &s, char *base, Workspace *w) {
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    size_t o_par = take(sizeof(float) * s.N * s.n * s.ksplit * s.pstride);
    size_t o_act = take(sizeof(bf16_t) * s.N * 2 * s.rk);
    size_t o_rms = take(sizeof(float) * s.N * s.n);
    size_t o_wp = take(s.wide ? 0 : sizeof(bf16_t) * (size_t)s.n * 2 * 16 * s.row_blocks * s.d);
    if (w) {
        w->partial = (float *)(base + o_par);
        w->act = (bf16_t *)(base + o_act);
        w->rms = (float *)(base + o_rms);
        w->wprime = (bf16_t *)(base + o_wp);
    }
    return off;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                          __builtin_bit_cast(bf16x2, b), c, false);
}

// x = a (.) b for 8 bf16 channels (one 16-byte vector of each) -- W' = W . gamma,
// or gamma . R' -- as bf16 hi and lo words: hi = bf16(x), lo = bf16(x - hi);
// the product of two bf16 values is exact in fp32.
__device__ __forceinline__ void split_product(u32x4 w, u32x4 gm, u32x4 &hi, u32x4 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(w[e]) * bf16_lo(gm[e]);
        const float x1 = bf16_hi(w[e]) * bf16_hi(gm[e]);
        hi[e] = pack_bf16x2(x0, x1);
        lo[e] = pack_bf16x2(x0 - bf16_lo(hi[e]), x1 - bf16_hi(hi[e]));
    }
}

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

// Kernel 1's walk over the rounds (128 channels each) of token tile T starts at
// this round of its nround: one of four offsets a quarter of a row apart, the
// same for the tile's n workgroups (see k_stream_proj).  Kernel 2 uses it to
// read first what kernel 1 wrote last.
constexpr int kK1Round = 2 * kIter;       // channels per kernel-1 round
__device__ __forceinline__ int k1_round_rotation(int64_t tile, int nround) {
    return (int)(((tile >> 3) & 3) * ((nround + 3) / 4) % nround);
}

// The token tiles p, p + P, ... of a resident kernel-2 workgroup, in two
// passes: first the tiles whose channels of this range kernel 1 wrote in the
// second half of its walk over the tile (the likeliest to be still in the
// 256 MB Infinity Cache when kernel 2 starts), then the others.  nround1 = 0
// (kernel 1 did not rotate) gives the plain order.
struct TileWalk {
    int64_t p, P, tiles;
    int nround1, kround;   // kernel 1's rounds per split, and this range's round
    __device__ bool first_pass(int64_t X) const {
        if (nround1 == 0) return true;
        int s_ = kround - k1_round_rotation(X, nround1);
        if (s_ < 0) s_ += nround1;
        return s_ >= nround1 / 2;
    }
    // next tile at or after `from` in pass `pass` (0 or 1), moving on to pass 1
    // when pass 0 is exhausted; -1 at the end of the walk
    __device__ int64_t next(int64_t from, int &pass) const {
        for (int64_t X = from; X < tiles; X += P)
            if (first_pass(X) == (pass == 0)) return X;
        if (pass == 0) {
            pass = 1;
            for (int64_t X = p; X < tiles; X += P)
                if (!first_pass(X)) return X;
        }
        return -1;
    }
};
__device__ __forceinline__ TileWalk tile_walk(const FastShape &sh, int64_t p, int64_t P, int64_t tiles, int c_begin) {
    TileWalk w{p, P, tiles, 0, 0};
    if (!sh.wide && !sh.small && sh.ksplit_chan > 0) {
        w.nround1 = (sh.ksplit_chan + kK1Round - 1) / kK1Round;
        w.kround = (c_begin % sh.ksplit_chan) / kK1Round;
    }
    return w;
}

// State element type of the fast path: bf16 words or e4m3 bytes.
template <bool F8> struct StateT { using type = bf16_t; using vec8 = u32x4; };
template <> struct StateT<true> { using type = fp8_t; using vec8 = u32x2; };

// Eight state values at p as four packed bf16 words (exact for e4m3).
template <bool F8>
__device__ __forceinline__ u32x4 load8_as_bf16(const typename StateT<F8>::type *p) {
    if constexpr (F8) return widen8_fp8_bf16(*reinterpret_cast<const u32x2 *>(p));
    else return *reinterpret_cast<const u32x4 *>(p);
}

// ---------------------------------------------------------------------------
#ifndef GR_K1_WAVES_PER_SIMD
#define GR_K1_WAVES_PER_SIMD 4
#endif
// Kernel 1.  blockIdx -> (tile, branch) so that the n workgroups of a tile get
// the same blockIdx % 8 (same XCD under round-robin dispatch: y is shared in
// that XCD's L2) and consecutive dispatch slots.
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
// DEPTH > 0: DEPTH rounds of state / y loads are in flight ahead of the round
// in use.  DEPTH = 0: the next round's state loads are issued as soon as the
// element phase has freed their registers, so they fly during the MFMA phase
// at no register cost; y (mostly an L2 hit: the n workgroups of a tile share
// it) is loaded at the start of its round.
template <bool FUSED, int NRB, int DEPTH, int TG, bool F8>
__global__ void __launch_bounds__(64 * (kWaves / TG), (NRB <= 5 && TG == 1) ? GR_K1_WAVES_PER_SIMD : 2)
k_stream_proj(typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ y,
              const float *__restrict__ s_in, const bf16_t *__restrict__ gamma,
              const bf16_t *__restrict__ wd, const bf16_t *__restrict__ ww, Workspace ws,
              FastShape sh) {
    constexpr int WAVES = kWaves / TG;                 // each wave carries TG groups of 16 tokens
    constexpr int THREADS = 64 * WAVES;
    constexpr int NQ = 4 * TG;                         // load instructions per round (4 tokens each)
    constexpr int RC = 2 * kIter;                      // channels per round
    constexpr int PCS = RC / 8;                        // 16-byte pieces per token row and round
    constexpr int KS = kIter / kChunk;                 // MFMA k-steps per W' chunk
    constexpr int kPitch = kIter + 8;                  // bf16 per staged W' row
    constexpr int NV = NRB * 16 * (kIter / 8);         // 16-byte vectors of W' per chunk (per plane)
    constexpr int WV = (2 * NV + THREADS - 1) / THREADS;  // hi and lo planes
    constexpr int NSLOT = DEPTH + 1;
    using T = typename StateT<F8>::type;
    using SV = typename StateT<F8>::vec8;              // 8 channels of the state
    static_assert(PCS == 16, "a round is 16 pieces of 8 channels per token");
    // [buffer][hi/lo][row][k]
    __shared__ __attribute__((aligned(16))) bf16_t lds_w[2][2][NRB * 16 * kPitch];
    constexpr int RP = PCS + 1;                        // LDS tile pitch in pieces (odd: no bank conflicts)
    __shared__ __attribute__((aligned(16))) u32x4 lds_r[WAVES][16 * TG * RP];

    const int n = sh.n, d = sh.d, S = sh.ksplit;
    const int64_t b = blockIdx.x;
    const int64_t tile = (b / 8 / (n * S)) * 8 + (b % 8);
    const int br = (int)((b / 8) % (n * S)) / S;
    const int split = (int)((b / 8) % S);
    if (tile >= sh.tiles) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, m16 = lane & 15;
    const int64_t t0 = tile * kTile + wave * 16 * TG;   // first token of this wave
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
                *reinterpret_cast<u32x4 *>(&lds_w[buf][plane][row * kPitch + cv * 8]) = wreg[q];
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

    SV rr[NSLOT][NQ];
    u32x4 yy[NSLOT][NQ];
    // load round `ar` of the split (valid: the walk has such a step)
    auto load_round = [&](int ar, bool valid, int slot, bool ds = true, bool dy = true) {
        const bool in = valid && ar * RC + 8 * m16 < chan;
        const T *const rs = sbase + ar * RC;                   // wave-uniform
        const bf16_t *const ry = FUSED ? ybase + ar * RC : nullptr;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (ds) rr[slot][q] = SV{};
            if (dy) yy[slot][q] = u32x4{0u, 0u, 0u, 0u};
            if (vq[q] && in) {
                if (ds) rr[slot][q] = *reinterpret_cast<const SV *>(rs + q * qstride + soff);
                if (FUSED && dy) yy[slot][q] = *reinterpret_cast<const u32x4 *>(ry + q * qystride + yoff);
            }
        }
    };

    f32x4 acc[TG][NRB];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int k = 0; k < NRB; ++k) acc[tg][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 *my_r = lds_r[wave];

    load_w(0);
    store_w(0);
    load_w(1);
#pragma unroll
    for (int q = 0; q < DEPTH; ++q) load_round(q < nround ? rnd(q) : 0, q < nround, q);
    if (DEPTH == 0) load_round(rot, true, 0, true, false);
    __syncthreads();
    int it = 0;                                         // W' chunks of the walk used so far
    int ar = rot;                                       // round of the split at walk step rd
    for (int rd = 0; rd < nround; ++rd) {
        const int an = ar + 1 == nround ? 0 : ar + 1;   // ... at step rd + 1
        if (DEPTH > 0) load_round(rd + DEPTH < nround ? rnd(rd + DEPTH) : 0, rd + DEPTH < nround, DEPTH);
        else load_round(ar, true, 0, false, true);
        // eq:write in the load layout: store, sum of squares, LDS tile
        const bool in = ar * RC + 8 * m16 < chan;
        T *const ws_ = sbase + ar * RC;                          // wave-uniform
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            u32x4 w;  // the 8 stored values as bf16 (exact for an e4m3 state)
            if constexpr (F8) {
                u32x2 o = rr[0][q];
                if (FUSED) {
                    o = write8_fp8(sq[q], yy[0][q], rr[0][q]);
                    if (vq[q] && in) *reinterpret_cast<u32x2 *>(ws_ + q * qstride + soff) = o;
                }
                w = widen8_fp8_bf16(o);
            } else {
                w = rr[0][q];
                if (FUSED) {
                    w = write8_bf16(sq[q], yy[0][q], rr[0][q]);
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
        if (DEPTH == 0) load_round(an, rd + 1 < nround, 0, true, false);
#pragma unroll
        for (int h = 0; h < RC / kIter; ++h) {
            if (ar * (RC / kIter) + h < nit) {               // chunk h of this round exists
                const int cur = it & 1;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int pc = (h * kIter + ks * kChunk) / 8 + g;   // piece of this lane group
                    bf16x8 bop[TG];
#pragma unroll
                    for (int tg = 0; tg < TG; ++tg)
                        bop[tg] = as_bf16x8(my_r[(16 * tg + m16) * RP + pc]);
                    const bf16_t *wh = &lds_w[cur][0][m16 * kPitch + ks * kChunk + 8 * g];
                    const bf16_t *wl = &lds_w[cur][1][m16 * kPitch + ks * kChunk + 8 * g];
#pragma unroll
                    for (int k = 0; k < NRB; ++k) {
                        const u32x4 ah = *reinterpret_cast<const u32x4 *>(wh + k * 16 * kPitch);
                        const u32x4 al = *reinterpret_cast<const u32x4 *>(wl + k * 16 * kPitch);
#pragma unroll
                        for (int tg = 0; tg < TG; ++tg) {
                            acc[tg][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), bop[tg], acc[tg][k], 0, 0, 0);
                            acc[tg][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), bop[tg], acc[tg][k], 0, 0, 0);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (it + 1 < nit) store_w(cur ^ 1);
                load_w(it + 2);
                __syncthreads();
                ++it;
            }
        }
#pragma unroll
        for (int q = 0; q < DEPTH; ++q)
#pragma unroll
            for (int e = 0; e < NQ; ++e) {
                rr[q][e] = rr[q + 1][e];
                yy[q][e] = yy[q + 1][e];
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
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
        const int64_t t = t0 + 16 * tg + m16;  // MFMA column of this lane
        if (t < sh.N) {
            float *rec = ws.partial + ((t * n + br) * S + split) * (int64_t)sh.pstride;
#pragma unroll
            for (int k = 0; k < NRB; ++k) *reinterpret_cast<f32x4 *>(rec + 4 + 16 * k + 4 * g) = acc[tg][k];
        }
    }
}

// Kernel 1, few-token form.  With few tokens the tile walk above has too few
// (tile, branch) units to fill the GPU, and each unit is a chain of rounds.
// Here a workgroup takes 16 tokens of one branch and a split of the channels,
// one slice of kpw k-steps (32 channels each) per wave, so a wave makes one
// short pass.  A lane loads its state words straight in the MFMA B layout
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
constexpr int kSmallPass = kMaxRowBlocks;  // row blocks per pass of the LDS reduction
template <bool FUSED, int NRB, bool F8>
__global__ void __launch_bounds__(64 * kSmallWaves, 2)
k_stream_proj_small(typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ y,
                    const float *__restrict__ s_in, const bf16_t *__restrict__ gamma,
                    const bf16_t *__restrict__ wd, const bf16_t *__restrict__ ww, Workspace ws,
                    FastShape sh) {
    using T = typename StateT<F8>::type;
    using SV = typename StateT<F8>::vec8;
    constexpr int kSmallKB = small_kb<NRB>();
    constexpr int PB = NRB < kSmallPass ? NRB : kSmallPass;   // row blocks per reduction pass
    constexpr int NPASS = (NRB + PB - 1) / PB;
    __shared__ float lds_p[kSmallWaves][4 * PB + 1][64];  // per wave: a pass's accumulators, then ss
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
    const int64_t t = tg * 16 + m16;                      // this lane's token (MFMA column)
    const bool valid = t < sh.N;
    const int64_t nd = (int64_t)n * d;
    const int c_wave = (split * kSmallWaves + wave) * kpw * kChunk;
    const float sv = (FUSED && valid) ? s_in[t * n + br] : 0.f;
    T *const srow = state + (t * n + br) * (int64_t)d;
    const bf16_t *const yrow = FUSED ? y + t * (int64_t)d : nullptr;

    f32x4 acc[NRB];
#pragma unroll
    for (int k = 0; k < NRB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    for (int kb = 0; kb < kpw; kb += kSmallKB) {
        SV rr[kSmallKB];
        u32x4 yy[kSmallKB], gm[kSmallKB], wv[kSmallKB][NRB];
        bool kin[kSmallKB];
#pragma unroll
        for (int ks = 0; ks < kSmallKB; ++ks) {
            const int c0 = c_wave + (kb + ks) * kChunk;   // whole 32-channel chunk in or out (d % 32 == 0)
            kin[ks] = kb + ks < kpw && c0 < d;
            const int c = c0 + 8 * g;
            rr[ks] = SV{};
            yy[ks] = gm[ks] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < NRB; ++k) wv[ks][k] = u32x4{0u, 0u, 0u, 0u};
            if (kin[ks]) {
                if (valid) {
                    rr[ks] = *reinterpret_cast<const SV *>(srow + c);
                    if (FUSED) yy[ks] = *reinterpret_cast<const u32x4 *>(yrow + c);
                }
                gm[ks] = *reinterpret_cast<const u32x4 *>(gamma + (int64_t)br * d + c);
#pragma unroll
                for (int k = 0; k < NRB; ++k) {
                    const int row = 16 * k + m16;
                    const bf16_t *src = row < sh.r ? wd + (int64_t)row * nd
                                      : (row < sh.rows ? ww + (int64_t)(row - sh.r) * nd : nullptr);
                    if (src) wv[ks][k] = *reinterpret_cast<const u32x4 *>(src + (int64_t)br * d + c);
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < kSmallKB; ++ks) {
            const int c = c_wave + (kb + ks) * kChunk + 8 * g;
            u32x4 w;  // the 8 stored values as bf16 (exact for an e4m3 state)
            if constexpr (F8) {
                u32x2 o = rr[ks];
                if (FUSED) {
                    o = write8_fp8(sv, yy[ks], rr[ks]);
                    if (valid && kin[ks]) *reinterpret_cast<u32x2 *>(srow + c) = o;
                }
                w = widen8_fp8_bf16(o);
            } else {
                w = rr[ks];
                if (FUSED) {
                    w = write8_bf16(sv, yy[ks], rr[ks]);
                    if (valid && kin[ks]) *reinterpret_cast<u32x4 *>(srow + c) = w;
                }
            }
            // masked lanes and chunks hold zeros: they add nothing below
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = dot2_bf16(w[e], w[e], ss);
            // B = gamma . R' as bf16 hi + lo (exact fp32 product split once per
            // k-step); A = the raw W rows
            u32x4 bh, bl;
            split_product(w, gm[ks], bh, bl);
#pragma unroll
            for (int k = 0; k < NRB; ++k) {
                acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[ks][k]), as_bf16x8(bh), acc[k], 0, 0, 0);
                acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[ks][k]), as_bf16x8(bl), acc[k], 0, 0, 0);
            }
        }
    }
    // this wave's share of ss per token: the four lane groups hold its channels
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    // add the waves' accumulators in LDS, PB row blocks per pass (ss with the first)
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        constexpr int ACC = 4 * PB;                       // words per lane and pass
        if (ps > 0) __syncthreads();                      // the previous pass is read
#pragma unroll
        for (int k = 0; k < PB; ++k)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (ps * PB + k < NRB) lds_p[wave][4 * k + m][lane] = acc[ps * PB + k][m];
        if (ps == 0) lds_p[wave][ACC][lane] = ss;
        __syncthreads();
        // word j of lane l: P row 16(ps PB + j/4) + 4(l/16) + j%4 of token l%16
        // (j < ACC), ss (j = ACC, first pass)
        const int words = 4 * (ps * PB + PB <= NRB ? PB : NRB - ps * PB);   // P words of this pass
        for (int v = tid; v < (ACC + 1) * 64; v += 64 * kSmallWaves) {
            const int j = v >> 6, l = v & 63;
            const int64_t tt = tg * 16 + (l & 15);
            const bool is_ss = j == ACC;
            if (tt >= sh.N || (is_ss ? (ps != 0 || l >= 16) : j >= words)) continue;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < kSmallWaves; ++w) sum += lds_p[w][j][l];
            float *rec = ws.partial + ((tt * n + br) * S + split) * (int64_t)sh.pstride;
            rec[is_ss ? 0 : 4 + 16 * (ps * PB + (j >> 2)) + 4 * (l >> 4) + (j & 3)] = sum;
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
    const int64_t tile = (b / 8 / (n * S)) * 8 + (b % 8);
    const int br = (int)((b / 8) % (n * S)) / S;
    const int split = (int)((b / 8) % S);
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

// Kernel 1b: combine the partial records written by kernel 1.  One wave per
// token, four tokens per workgroup: lanes 0..NB-1 sum the squares over the
// splits (rho_i, rms_i; shared by shuffles), and each lane owns outputs
// j = lane, lane + 64, ...: the split sums of P_i[j] for every branch (lanes
// read consecutive j: coalesced), rho applied, summed over branches in order.
// The loads of the sums of squares and of the first two outputs per lane go
// out together, so a call of few tokens waits for memory once.
//   j < r        z = (1/n) sum_i rho_i P_i[j]  ->  -log2(e) SiLU(z) as (hi, lo)
//   r <= j < rk  zero padding of the up projection's k-steps
//   rk + i       s_i = 2 sigmoid((1/n) sum_i' rho_i' P_i'[r + i])  (1 without W_write)
constexpr int kRedWaves = 4;
template <int NB, int S>
__global__ void __launch_bounds__(64 * kRedWaves)
k_reduce_records(float *__restrict__ s_out, Workspace ws, FastShape sh, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRedWaves + (threadIdx.x >> 6);
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
    auto gather = [&](int j, float (&p)[NB]) {
        const int row = j < outs ? prow(j) : -1;
#pragma unroll
        for (int i = 0; i < NB; ++i) p[i] = row >= 0 ? split_sum(i, 4 + row) : 0.f;
    };
    // one round of loads: the sums of squares with the rows of the lane's
    // first two outputs (none of them waits for rho)
    const float ss_l = lane < NB ? split_sum(lane, 0) : 0.f;
    float pa[NB], pb[NB];
    gather(lane, pa);
    gather(lane + 64, pb);
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
    if (lane < outs) emit(lane, pa);
    if (lane + 64 < outs) emit(lane + 64, pb);
    for (int j = lane + 128; j < outs; j += 64) {
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
// combined.
template <int NB, int RKS, bool F8>
__global__ void __launch_bounds__(kK2Threads, kK2WavesPerSimd)
k_gate_combine(const typename StateT<F8>::type *__restrict__ state, const bf16_t *__restrict__ gamma,
               const bf16_t *__restrict__ wu, bf16_t *__restrict__ u, Workspace ws, FastShape sh,
               int ranges) {
    constexpr int SUB = kK2Sub;                        // 32-channel chunks per iteration
    constexpr int KC = SUB * kChunk;                   // channels per iteration
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
    const int nch = (c_end - c_begin) / kChunk;        // 32-channel chunks of this range
    const int nit = (nch + SUB - 1) / SUB;
    const float inv_n = 1.0f / (float)NB;

    // W_up rows (branch i, channel c) of one iteration; row index i * KC + cc
    u32x4 wreg[WV];
    uint32_t greg[NG];
    auto load_w = [&](int it) {
        const int c0 = c_begin + it * KC;
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * kK2Threads;
            const int row = v / (RK / 8), kv = v % (RK / 8);
            const int i = row / KC, cc = row % KC;
            wreg[q] = u32x4{0u, 0u, 0u, 0u};
            if (v < NV && it < nit && c0 + cc < c_end && kv * 8 < r)
                wreg[q] = *reinterpret_cast<const u32x4 *>(wu + ((int64_t)i * d + c0 + cc) * r + kv * 8);
        }
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int v = tid + q * kK2Threads;
            greg[q] = 0u;
            if (v < NB * KC && it < nit && c0 + v % KC < c_end) {
                const bf16_t gk = f32_to_bf16(bf16_to_f32(gamma[(int64_t)(v / KC) * d + c0 + v % KC]) * inv_n);
                greg[q] = (v & 1) ? ((uint32_t)gk << 16) : (uint32_t)gk;
            }
        }
    };
    // LDS row of (branch i, channel cc): chunk cc/32, then MFMA row order within it
    auto store_w = [&](int buf) {
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int v = tid + q * kK2Threads;
            if (v < NV) {
                const int row = v / (RK / 8), kv = v % (RK / 8);
                const int i = row / KC, cc = row % KC, c32 = cc % kChunk;
                const int pos = (i * SUB + cc / kChunk) * kChunk + 16 * ((c32 >> 2) & 1) + 4 * (c32 >> 3) + (c32 & 3);
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
        u32x4 v = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
        if (valid) {
            v = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2) * RK + ks * 32 + 8 * g);
            vl = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2 + 1) * RK + ks * 32 + 8 * g);
        }
        bop[ks] = as_bf16x8(v);
        bopl[ks] = as_bf16x8(vl);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) rms[i] = valid ? ws.rms[t * NB + i] : 1.0f;

    const typename StateT<F8>::type *srow = state + t * (int64_t)NB * d + 8 * g;
    bf16_t *urow = u + t * (int64_t)d + 8 * g;
    const int m16 = lane & 15;  // A row this lane feeds

    u32x4 s0[SUB][NB], s1[SUB][NB];
    auto load_state = [&](int it, u32x4 (&sv)[SUB][NB]) {
#pragma unroll
        for (int sc = 0; sc < SUB; ++sc)
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int c0 = c_begin + it * KC + sc * kChunk;
                sv[sc][i] = u32x4{0u, 0u, 0u, 0u};
                if (valid && it < nit && c0 < c_end)
                    sv[sc][i] = load8_as_bf16<F8>(srow + (int64_t)i * d + c0);
            }
    };

    load_w(0);
    store_w(0);
    load_w(1);
    load_state(0, s0);
    __syncthreads();
    for (int it = 0; it < nit; ++it) {
        const int cur = it & 1;
        load_state(it + 1, s1);
#pragma unroll
        for (int sc = 0; sc < SUB; ++sc) {
            const int c0 = c_begin + it * KC + sc * kChunk;
            float uacc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) uacc[e] = 0.f;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4 tl = {0.f, 0.f, 0.f, 0.f};
                    const bf16_t *ap = &lds_u[cur][((i * SUB + sc) * kChunk + 16 * h + m16) * kPitch + 8 * g];
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
                        const float bterm = dot2_bf16(s0[sc][i][e >> 1],
                                                      lds_g[cur][i * KC + sc * kChunk + 8 * g + e], 0.f);
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
        if (it + 1 < nit) store_w(cur ^ 1);
        load_w(it + 2);
        __syncthreads();
#pragma unroll
        for (int sc = 0; sc < SUB; ++sc)
#pragma unroll
            for (int i = 0; i < NB; ++i) s0[sc][i] = s1[sc][i];
    }
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
template <int RKS> struct ResidentCfg {
    // channels per workgroup: keeps the staged W_up near 72 KiB (two per CU);
    // a wide gate (RKS > 4) gets 32 channels, ~84 KiB (one per CU)
    static constexpr int CH = RKS <= 2 ? 128 : (RKS <= 4 ? 64 : 32);
    // 32-channel chunks per step: two (one 128-byte line of bf16) when the range allows
    static constexpr int SC = CH >= 64 ? 2 : 1;
};

#ifndef GR_K2R_WAVES
#define GR_K2R_WAVES 8
#endif
#ifndef GR_K2R_WAVES_PER_SIMD
#define GR_K2R_WAVES_PER_SIMD 4
#endif
constexpr int kResWaves = GR_K2R_WAVES;
constexpr int kResThreads = 64 * kResWaves;
constexpr int kResTile = 16 * kResWaves;         // tokens per tile
constexpr int kResWgsTarget = 512;               // workgroups wanted (two per CU)

template <int NB, int RKS, int CH, int SC>
__global__ void __launch_bounds__(kResThreads, RKS <= 2 ? GR_K2R_WAVES_PER_SIMD : 2)
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
        const int64_t t = token(T);
        const bool ok = t < sh.N;
#pragma unroll
        for (int ks = 0; ks < RKS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
            if (ok) {
                v = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2) * RK + ks * 32 + 8 * g);
                vl = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2 + 1) * RK + ks * 32 + 8 * g);
            }
            hi[ks] = as_bf16x8(v);
            lo[ks] = as_bf16x8(vl);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) rm[i] = ok ? ws.rms[t * NB + i] : 1.0f;
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
    for (int v = tid; v < NB * CH * (RK / 8); v += kResThreads) {
        const int row = v / (RK / 8), kv = v % (RK / 8);
        const int i = row / CH, cc = row % CH, c32 = cc % kChunk;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (cc < nchan && kv * 8 < r)
            w = *reinterpret_cast<const u32x4 *>(wu + ((int64_t)i * d + c_begin + cc) * r + kv * 8);
        const int pos = (i * NC + cc / kChunk) * kChunk + 16 * ((c32 >> 2) & 1) + 4 * (c32 >> 3) + (c32 & 3);
        *reinterpret_cast<u32x4 *>(&lds_u[pos * kPitch + kv * 8]) = w;
    }
    for (int v = tid; v < NB * CH; v += kResThreads) {
        const int i = v / CH, cc = v % CH;
        uint32_t gw = 0u;
        if (cc < nchan) {
            const bf16_t gk = f32_to_bf16(bf16_to_f32(gamma[(int64_t)i * d + c_begin + cc]) * inv_n);
            gw = (cc & 1) ? ((uint32_t)gk << 16) : (uint32_t)gk;
        }
        lds_g[v] = gw;
    }
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
    auto load_act = [&](int64_t T, bf16x8 (&hi)[RKS], bf16x8 (&lo)[RKS], float (&rm)[NB]) {
        const int64_t t = token(T);
        const bool ok = t < sh.N;
#pragma unroll
        for (int ks = 0; ks < RKS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
            if (ok) {
                v = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2) * RK + ks * 32 + 8 * g);
                vl = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2 + 1) * RK + ks * 32 + 8 * g);
            }
            hi[ks] = as_bf16x8(v);
            lo[ks] = as_bf16x8(vl);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) rm[i] = ok ? ws.rms[t * NB + i] : 1.0f;
    };
    // state of branch i, range rg of tile T: 8 channels per lane
    auto load_state = [&](int64_t T, int rg, int i) {
        const int64_t t = token(T);
        if (t >= sh.N) return SV{};
        return *reinterpret_cast<const SV *>(state + t * (int64_t)NB * d + (int64_t)i * d + rg * CH + 8 * g);
    };
    // W_up rows (branch i, channel cc of range rg) in MFMA row order, and gamma/n
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

    bf16x8 bop[RKS], bopl[RKS], nbop[RKS], nbopl[RKS];
    float rms[NB], nrms[NB];
    SV sv[NB];
    int64_t q = u0;
    int64_t T = unit_tile(q);
    int rg = unit_range(q);
    load_act(T, bop, bopl, rms);
#pragma unroll
    for (int i = 0; i < NB; ++i) sv[i] = load_state(T, rg, i);
    stage(rg);
    __syncthreads();

    for (;;) {
        const bool more = q + 1 < u1;
        const int64_t Tn = more ? unit_tile(q + 1) : T;
        const int rn = more ? unit_range(q + 1) : rg;
        if (more) load_act(Tn, nbop, nbopl, nrms);

        float uacc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) uacc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 tl = {0.f, 0.f, 0.f, 0.f};
                const bf16_t *ap = &lds_u[(i * CH + 16 * h + m16) * kPitch + 8 * g];
#pragma unroll
                for (int ks = 0; ks < RKS; ++ks) {
                    const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(ap + ks * 32));
                    tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[ks], tl, 0, 0, 0);
                    tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bopl[ks], tl, 0, 0, 0);
                }
                // tl[m] = -log2(e) * l for channel 8g + 4h + m of the range, branch i
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
                    const float den = fmaf(__builtin_amdgcn_exp2f(tl[m]), rms[i], rms[i]);
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
        for (int ks = 0; ks < RKS; ++ks) { bop[ks] = nbop[ks]; bopl[ks] = nbopl[ks]; }
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
__global__ void __launch_bounds__(kResThreads, RKS <= 2 ? GR_K2R_WAVES_PER_SIMD : 2)
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
        const int64_t t = token(T);
        const bool ok = t < sh.N;
#pragma unroll
        for (int ks = 0; ks < RKS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
            if (ok) {
                v = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2) * RK + ks * 32 + 8 * g);
                vl = *reinterpret_cast<const u32x4 *>(ws.act + (t * 2 + 1) * RK + ks * 32 + 8 * g);
            }
            hi[ks] = as_bf16x8(v);
            lo[ks] = as_bf16x8(vl);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) rm[i] = ok ? ws.rms[t * NB + i] : 1.0f;
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

    // stage W_up rows (branch i, channel cc of the range) and gamma/n
    for (int v = tid; v < NB * CH * (RK / 8); v += kResThreads) {
        const int row = v / (RK / 8), kv = v % (RK / 8);
        const int i = row / CH, cc = row % CH, c64 = cc % kF8Unit;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (cc < nchan && kv * 8 < r)
            w = *reinterpret_cast<const u32x4 *>(wu + ((int64_t)i * d + c_begin + cc) * r + kv * 8);
        const int pos = (i * NU + cc / kF8Unit) * kF8Unit + 16 * ((c64 >> 2) & 3) + 4 * (c64 >> 4) + (c64 & 3);
        *reinterpret_cast<u32x4 *>(&lds_u[pos * kPitch + kv * 8]) = w;
    }
    for (int v = tid; v < NB * CH; v += kResThreads) {
        const int i = v / CH, cc = v % CH;
        lds_g[v] = cc < nchan ? bf16_to_f32(f32_to_bf16(bf16_to_f32(gamma[(int64_t)i * d + c_begin + cc]) * inv_n))
                              : 0.f;
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
        hipLaunchKernelGGL((k_stream_proj<FUSED, NRB, kDepth, kTG, F8>), dim3(grid), dim3(64 * (kWaves / kTG)), 0, st, \
                           (T *)a.state, y, a.s_in, (const bf16_t *)a.gamma,                \
                           (const bf16_t *)a.wd, (const bf16_t *)a.ww, w, sh);              \
        break;
    if (sh.small) {
        const unsigned sgrid = (unsigned)(((sh.N + 15) / 16) * sh.n * sh.ksplit);
#define GR_K1S(NRB)                                                                         \
    case NRB:                                                                               \
        hipLaunchKernelGGL((k_stream_proj_small<FUSED, NRB, F8>), dim3(sgrid), dim3(64 * kSmallWaves), 0, st, \
                           (T *)a.state, y, a.s_in, (const bf16_t *)a.gamma,                \
                           (const bf16_t *)a.wd, (const bf16_t *)a.ww, w, sh);              \
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

template <int NB, bool F8>
hipError_t launch_k2(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st) {
    const int ranges = (sh.d + sh.k2_chan - 1) / sh.k2_chan;
    const unsigned grid = (unsigned)(((sh.N + kK2Tile - 1) / kK2Tile) * ranges);
#define GR_K2(RKS)                                                                          \
    case RKS:                                                                               \
        hipLaunchKernelGGL((k_gate_combine<NB, RKS, F8>), dim3(grid), dim3(kK2Threads), 0, st, \
                           (const typename StateT<F8>::type *)a.state, (const bf16_t *)a.gamma, \
                           (const bf16_t *)a.wu, (bf16_t *)a.u, w, sh, ranges);             \
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

// Compute units of the current device (cached per device).
int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev] = v;
    }
    return cached[dev];
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

bool fast_path_ok(const ReadArgs &a) {
    if (!a.bf16 || a.n != 4) return false;
    if (a.r < 16 || a.r % 16 || a.r > 32 * kMaxWideRKS) return false;
    if (a.d % kIter) return false;
    const int rows = a.r + (a.ww ? a.n : 0);
    const int nrb = (rows + 15) / 16;
    if (nrb <= kMaxRowBlocks && a.r <= 128) return true;
    // wide gate; an e4m3 state also needs d % 128 (kernel 2 covers whole
    // 128-byte state lines with four 32-channel ranges in lockstep)
    return nrb <= kMaxWideRowBlocks && (!a.fp8 || a.d % 128 == 0);
}

size_t fast_workspace_bytes(const ReadArgs &a) {
    // the layout of exactly this call: with or without W_write the record
    // stride, the gate form (narrow / wide) and so the W' planes differ
    return workspace_layout(shape_of(a), nullptr, nullptr);
}

hipError_t launch_read_fast(const ReadArgs &a, hipStream_t st) {
    const FastShape sh = shape_of(a);
    Workspace w;
    workspace_layout(sh, (char *)a.ws, &w);
    hipError_t e = a.fp8 ? (a.fused ? launch_k1<true, true>(a, sh, w, st) : launch_k1<false, true>(a, sh, w, st))
                         : (a.fused ? launch_k1<true, false>(a, sh, w, st) : launch_k1<false, false>(a, sh, w, st));
    if (e != hipSuccess) return e;
    const dim3 rgrid((unsigned)((sh.N + kRedWaves - 1) / kRedWaves)), rblock(64 * kRedWaves);
    switch (sh.ksplit) {
    case 1: hipLaunchKernelGGL((k_reduce_records<4, 1>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    case 2: hipLaunchKernelGGL((k_reduce_records<4, 2>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    case 4: hipLaunchKernelGGL((k_reduce_records<4, 4>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    case 8: hipLaunchKernelGGL((k_reduce_records<4, 8>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    case 16: hipLaunchKernelGGL((k_reduce_records<4, 16>), rgrid, rblock, 0, st, a.s_out, w, sh, a.eps); break;
    default: return hipErrorInvalidValue;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
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

}  // namespace grk
