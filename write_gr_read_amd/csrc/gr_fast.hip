// gr_fast.hip -- MFMA fast path of the GR read / fused write+read for a bf16
// or e4m3 widened state ("Paper reading: Qwen3.8 Flash Next", part 2 Residual,
// sec. 4 Gated Residual: eq:rms, eq:gate, eq:use_gate, eq:s; eq:write first
// when fused; sec. 7: read fused into one traversal with Group RMSNorm, and the
// FP8 state).  This file: the overview below, the choice of kernel forms for a
// call (shape_of) and the entry points.  The kernels are in gr_fast_k1.hip
// (kernel 1 and the W' preparation) and gr_fast_k2.hip (record reduction,
// kernel 2); what they share is in gr_fast_common.h.
//
// Up to four kernels in stream order, no inter-workgroup waiting (so no
// co-residency assumption).  Below, the narrow-gate (r + n <= 128) forms at
// many tokens; an e4m3 state uses the same kernel 1 template and its own
// resident kernel 2 (k_gate_combine_resident_fp8), a wide gate (r up to 320,
// the pages' r = d/8 at d = 2560) has its own kernel 1 and 2
// (k_stream_proj_wide, k_gate_combine_wide), and with fewer than 8 token tiles
// of 128 (N <= 896; fewer than 4, N <= 384, for a wide gate) kernel 1 is
// k_stream_proj_small; each is described where it is defined.
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
#include "gr_fast_common.h"

namespace grk {
namespace fast {

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
    // (16 or 32 tokens, branch, split); splits (a power of two, at most kMaxSplit)
    // until the grid has kSmallTarget workgroups or a wave's slice is one k-step.
    // With two token groups per wave (86 KB of LDS at 5 row blocks: one
    // workgroup per CU) the grid stays within kSmallTarget, one round of
    // workgroups: at 600-896 tokens a second, partial round cost 2-3 us.
    s.small = 0;
    s.small_kpw = 0;
    s.small_tg = 1;
    if (s.tiles * s.n < (s.wide ? kSmallBelowWide : kSmallBelow)) {
        // from kSmallTg2From tokens a wave takes two 16-token groups: each W
        // fragment it loads then serves 32 tokens (half the W reads from L2)
        s.small_tg = (s.N >= kSmallTg2From && s.row_blocks <= kSmallTg2MaxRB) ? 2 : 1;
        const int64_t groups = (s.N + 16 * s.small_tg - 1) / (16 * s.small_tg);
        int sp = 1;
        if (s.small_tg == 2) {
            while (groups * s.n * sp * 2 <= kSmallTarget && sp < kMaxSplit && s.d / (2 * sp) >= kSmallWaves * kChunk)
                sp *= 2;
        } else {
            while (groups * s.n * sp < kSmallTarget && sp < kMaxSplit && s.d / (2 * sp) >= kSmallWaves * kChunk) sp *= 2;
        }
        const int per = kSmallWaves * kChunk * sp;   // channels covered per k-step of every wave
        s.small = 1;
        s.ksplit = sp;
        s.ksplit_chan = 0;
        s.small_kpw = (s.d + per - 1) / per;
    }
    // the tile walk of a narrow gate (at least 8 tiles) reads W' split once per call
    s.prep = !s.wide && !s.small;
    return s;
}

}  // namespace fast

using namespace fast;

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
    hipError_t e = launch_kernel1(a, sh, w, st);
    if (e != hipSuccess) return e;
    if ((e = launch_reduce(a, sh, w, st)) != hipSuccess) return e;
    return launch_kernel2(a, sh, w, st);
}

}  // namespace grk
