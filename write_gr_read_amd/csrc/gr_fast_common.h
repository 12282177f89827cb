// gr_fast_common.h -- what the fast path's translation units share: tuning
// constants, the call's shape (FastShape) and workspace layout, device helpers,
// and the launchers one file offers another.  gr_fast.hip holds the overview
// of the kernels and the entry points; gr_fast_k1.hip the W' preparation and
// the three forms of kernel 1; gr_fast_k2.hip the record reduction and the
// forms of kernel 2.
#pragma once

#include "gr_device.h"
#include "gr_internal.h"

namespace grk {
namespace fast {

constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16 * kWaves;        // tokens per workgroup
constexpr int kChunk = 32;                // channels per MFMA k-step

constexpr int kIter = 64;                 // channels per W' chunk of kernel 1 (a round is two)
constexpr int kK1WavesPerSimd = 4;        // occupancy target of kernel 1 (narrow gate)
constexpr int kK2WavesPerSimd = 3;        // occupancy target of the few-token kernel 2
constexpr int kK2Waves = 4;               // waves per few-token kernel-2 workgroup
constexpr int kK2Threads = 64 * kK2Waves;
constexpr int kK2Tile = 16 * kK2Waves;    // tokens per few-token kernel-2 workgroup
constexpr int kMaxRowBlocks = 8;          // (r + n) padded to 16, at most 128 (narrow gate)
constexpr int kMaxWideRowBlocks = 21;     // wide gate (kernel 1 wide form): r + n up to 336
constexpr int kMaxWideRKS = 10;           // wide gate: r up to 320 (k-steps of 32 of the up projection)
constexpr int kChanPerWg = 256;           // channels per k_gate_combine workgroup
constexpr int kSplitTarget = 256;         // kernel-1 workgroups wanted before splitting channels
constexpr int kMaxSplit = 16;             // channel splits of kernel 1 (a power of two)
constexpr int kSmallBelow = 36;           // few-token kernel 1 while (token tiles) x n is below this (n = 4: N <= 1024)
constexpr int kSmallBelowWide = 16;          // ... for a wide gate
constexpr int kSmallTarget = 256;         // few-token kernel 1: workgroups wanted before splitting
constexpr int kSmallWaves = 8;            // waves per few-token kernel-1 workgroup
constexpr int kSmallTg2From = 256;        // few-token kernel 1: two 16-token groups per wave from this many tokens
constexpr int kSmallTg2MaxRB = 5;         // ... for gates of at most this many 16-row blocks

struct FastShape {
    int n, d, r, nw;     // nw = n if W_write given, else 0
    int rows;            // r + nw
    int row_blocks;      // ceil(rows / 16)
    int pstride;         // floats per (token, branch, split) partial record
    int ksplit;          // channel splits of kernel 1 (workgroups per (tile, branch))
    int ksplit_chan;     // channels per split (multiple of kIter)
    int k2_chan;         // channels per kernel-2 workgroup (multiple of kChunk)
    int rk;              // r padded to a multiple of 32 (k-steps of the up projection)
    // flags as 32-bit ints: every field of the struct, a kernel argument, is
    // then dword-aligned and read through the scalar cache (a bool pair at an
    // odd offset took a vector load and a wait at kernel start)
    int prep;            // W' split once per call by k_prep_wprime (enough token tiles)
    int wide;            // r + n beyond 128: kernel 1's wide form (gamma on the state side, no W')
    int small;           // few tokens: kernel 1's few-token form (k_stream_proj_small)
    int small_kpw;       // ... its k-steps (32 channels) per wave
    int small_tg;        // ... its 16-token groups per wave (1 or 2; they share each W fragment)
    int64_t N, tiles;
};

// The call's shape and kernel forms (gr_fast.hip).
FastShape shape_of(const ReadArgs &a);

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

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline size_t workspace_layout(const FastShape &s, char *base, Workspace *w) {
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

// Launchers of one translation unit used by another.
hipError_t launch_kernel1(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st);  // gr_fast_k1.hip
hipError_t launch_reduce(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st);   // gr_fast_k2.hip
hipError_t launch_kernel2(const ReadArgs &a, const FastShape &sh, const Workspace &w, hipStream_t st);  // gr_fast_k2.hip

}  // namespace fast
}  // namespace grk
