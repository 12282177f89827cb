/*
 * gr.h -- C ABI of the MI355X (gfx950) Gated Residual read/write library.
 *
 * Gated Residual (GR) keeps n branch states per token, R in R^{n x d}.  Around
 * each sublayer F it performs
 *   read : R-hat_i = RMSNorm(R_i; gamma_i)                              eq:rms
 *          G = unvec sigmoid(W_up SiLU((1/n) W_down vec(R-hat)))        eq:gate
 *          u = (1/n) sum_i G_i (.) R-hat_i      (the sublayer input)     eq:use_gate
 *          s = 2 sigmoid((1/n) W_write vec(R-hat))  (write strengths)    eq:s
 *   F    : y = F(u), once, outside this library
 *   write: R'_i = R_i + s_i y                                             eq:write
 * ("Paper reading: Qwen3.8 Flash Next", part 2 Residual, sec. 4 Gated
 * Residual; restated in "Qwen3.8-Flash-Next architecture notes, 06 Residual",
 * sec. 2 and 3).  The pages fuse the read into one kernel and the write into
 * another (same paper reading, sec. 7).  This library computes s inside the
 * read (it depends only on R-hat, which the read holds) and hands it to the
 * write, and adds a fused write(l)+read(l+1) call, so the write's output is
 * read back without a separate call.  The n = 1 degenerate case is the fused
 * residual add + RMSNorm of "Residual" (LLM inference), sec. 3.3.
 *
 * Conventions shared by every call
 *   Memory     All tensor pointers are DEVICE pointers owned by the caller;
 *              the library keeps no reference after a call returns.  Scratch
 *              memory comes from the caller's workspace argument, except on
 *              the single-pass path (GR_KERNEL_VARIANT=single, below), which
 *              exchanges partial sums through a library-owned device array
 *              of ~11 MB per GPU and allocates nothing.
 *   Layout     Contiguous, row-major: state [N][n][d] (token, branch,
 *              channel); y, u [N][d]; s [N][n] (always fp32); gamma [n][d];
 *              W_down [r][n*d]; W_up [n*d][r]; W_write [n][n*d].  The vec()
 *              index of (branch i, channel c) is i*d + c.  Weights, gamma, y
 *              and u have the state dtype, except with GR_FP8_E4M3, where
 *              only the state is fp8 and they are bf16.
 *   Alignment  Every pointer 16-byte aligned; d a multiple of 8 (bf16), 4
 *              (fp32) or 16 (fp8 state).
 *   Sizes      1 <= n <= 8, d >= 1, 0 <= r <= 512, N >= 0.  r == 0 means a
 *              unit gate (G == 1).  W_write == NULL means s == 1 (the value
 *              of 2 sigmoid(0)).  eps is added inside the square root.
 *   N == 0     A no-op returning GR_SUCCESS (pointers are not inspected).
 *   Aliasing   No two arguments may overlap, except out == y in
 *              residual_add_rmsnorm.
 *   Streams    `stream` is a hipStream_t (NULL = the default stream).  Calls
 *              are asynchronous; a fault inside a kernel surfaces at the
 *              caller's next synchronisation.
 *   Errors     Argument errors are detected on the host before any HIP call
 *              and return GR_ERROR_INVALID_VALUE / GR_ERROR_NOT_SUPPORTED /
 *              GR_ERROR_WORKSPACE; a failed launch returns GR_ERROR_LAUNCH.
 *              gr_last_error() gives a message for the calling thread.
 *              No call aborts the process.
 *   Threads    Calls are stateless and may be made from several threads.
 */
#ifndef GR_H
#define GR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gr_dtype {
    GR_F32 = 0,       /* fp32 state and weights, fp32 arithmetic */
    GR_BF16 = 1,      /* bf16 state and weights, fp32 accumulation */
    GR_FP8_E4M3 = 2   /* fp8 branch state (OCP e4m3, values saturate at +-448;
                         "Paper reading: Qwen3.8 Flash Next", part 2 Residual,
                         sec. 7 names an FP8 state), bf16 y, u, gains and
                         weights, fp32 accumulation.  Not for
                         residual_add_rmsnorm or the tanh stand-in. */
} gr_dtype;

typedef enum gr_status {
    GR_SUCCESS = 0,
    GR_ERROR_INVALID_VALUE = 1,  /* bad pointer, size, dtype or alignment */
    GR_ERROR_NOT_SUPPORTED = 2,  /* valid but outside what the kernels handle */
    GR_ERROR_LAUNCH = 3,         /* the HIP runtime refused a launch */
    GR_ERROR_WORKSPACE = 4       /* workspace smaller than gr_workspace_size() */
} gr_status;

/* One GR module's parameters (device pointers, state dtype). */
typedef struct gr_layer {
    int32_t n;             /* branches, 1..8 */
    int32_t d;             /* width of each branch and of the sublayer */
    int32_t r;             /* gate rank, 0..512 (0 = unit gate) */
    float eps;             /* RMSNorm epsilon (>= 0, finite) */
    const void *gamma;     /* [n][d]    effective per-branch gains */
    const void *w_down;    /* [r][n*d]  NULL iff r == 0 */
    const void *w_up;      /* [n*d][r]  NULL iff r == 0 */
    const void *w_write;   /* [n][n*d]  or NULL (s == 1) */
} gr_layer;

/* Operation ids for gr_workspace_size. */
enum { GR_OP_READ = 0, GR_OP_FUSED_WRITE_READ = 1 };

/*
 * gr_read -- the GR read (eq:rms, eq:gate, eq:use_gate) plus the write
 * strengths of the same module (eq:s), which depend only on R-hat.
 *   state  in  [N][n][d]  (not modified)
 *   u      out [N][d]     sublayer input, state dtype
 *   s      out [N][n]     fp32 write strengths for the later gr_write
 *   workspace / ws_bytes  device scratch of at least
 *                         gr_workspace_size(GR_OP_READ, ...) bytes
 */
gr_status gr_read(const void *state, gr_dtype dt, int64_t N, const gr_layer *L,
                  void *u, float *s, void *workspace, size_t ws_bytes, void *stream);

/*
 * gr_write -- eq:write, in place: state[t][i][c] += s[t][i] * y[t][c],
 * computed as one fp32 fused multiply-add (the exact value rounded once to
 * fp32) and stored in the state dtype (round to nearest even; an fp8 state
 * saturates at +-448).
 *   state  in/out [N][n][d];  y in [N][d];  s in [N][n] fp32
 */
gr_status gr_write(void *state, const void *y, const float *s, gr_dtype dt, int64_t N,
                   int32_t n, int32_t d, void *stream);

/*
 * gr_fused_write_read -- gr_write of sublayer l, then gr_read of sublayer
 * l+1 with `next`, on the STORED (rounded) state.  Results equal gr_write
 * followed by gr_read (state bit for bit).  The default kernels pass over
 * the state twice: the first forms and stores R' together with its
 * projections, the second reads R' back for the gated combine (28 d bytes
 * per token with a bf16 state, where one pass would move 20 d).  With
 * GR_KERNEL_VARIANT=single (n = 4, bf16 state, d = 4096 or 2048,
 * 16 <= r <= 64, r % 16 == 0, a GPU of 8 XCDs x 32 CUs) one persistent
 * kernel keeps R' on chip between the two and reads the state once; it is
 * currently slower than the default, see gr_device_error_word for its
 * diagnostic, and calls of it on one GPU run one after the other.
 *   state  in/out [N][n][d];  y in [N][d];  s_in in [N][n] fp32
 *   u_next out [N][d];  s_next out [N][n] fp32
 *   workspace >= gr_workspace_size(GR_OP_FUSED_WRITE_READ, ...) bytes
 */
gr_status gr_fused_write_read(void *state, const void *y, const float *s_in, gr_dtype dt,
                              int64_t N, const gr_layer *next, void *u_next, float *s_next,
                              void *workspace, size_t ws_bytes, void *stream);

/*
 * gr_fused_write_read_noalloc -- gr_fused_write_read for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): same arguments without the workspace.
 * The scratch memory its kernels need comes from a library-owned device array
 * of 48 MiB per GPU (enough for 16384 tokens at d = 4096, n = 4, r = 64), set
 * up on the first call on each GPU and held until the process ends; the call
 * itself allocates nothing.  A call whose scratch would exceed 48 MiB returns
 * GR_ERROR_WORKSPACE before any launch.  Every call on one GPU shares that
 * array (the kernels write every byte they read, so nothing needs clearing),
 * so calls that overlap in time on one GPU -- on different streams without
 * ordering -- race and must not be made.
 */
gr_status gr_fused_write_read_noalloc(void *state, const void *y, const float *s_in, gr_dtype dt,
                                      int64_t N, const gr_layer *next, void *u_next, float *s_next,
                                      void *stream);

/*
 * residual_add_rmsnorm -- n = 1 fused residual add + RMSNorm ("Residual",
 * LLM inference, sec. 3.3): h = x + y stored in place of x, then
 * out = w (.) h / sqrt(mean(h^2) + eps), the mean taken over the stored h.
 * dtype GR_F32 or GR_BF16 (GR_FP8_E4M3 returns GR_ERROR_NOT_SUPPORTED).
 *   x in/out [N][d];  y in [N][d];  w in [d];  out out [N][d] (may equal y)
 */
gr_status residual_add_rmsnorm(void *x, const void *y, const void *w, float eps, void *out,
                               gr_dtype dt, int64_t N, int32_t d, void *stream);

/*
 * Variants on the same widened state.  Same conventions as above; "act dtype"
 * is the state dtype, or bf16 with GR_FP8_E4M3.  Sums and products in fp32,
 * one store rounded to nearest even (an fp8 state saturating at +-448).
 *
 * gr_expand -- the stream's start ("Paper reading: Qwen3.8 Flash Next",
 * part 2 Residual, sec. 6, eq:rcv: every branch's initial value is the token
 * embedding): state[t][i][c] = e[t][c] for every branch i.
 *   e in [N][d] (act dtype);  state out [N][n][d]
 */
gr_status gr_expand(const void *e, void *state, gr_dtype dt, int64_t N, int32_t n, int32_t d,
                    void *stream);

/*
 * gr_static_read -- the AltUp-style read of the widened stream (same page,
 * sec. 1, eq:input): u[t][c] = sum_i h[i] state[t][i][c], with n learned
 * scalars h (no normalisation).
 *   state in [N][n][d];  h in [n] fp32 (device);  u out [N][d] (act dtype)
 */
gr_status gr_static_read(const void *state, const float *h, void *u, gr_dtype dt, int64_t N,
                         int32_t n, int32_t d, void *stream);

/*
 * gr_round_robin_write -- the AltUp-style write (same page, sec. 1,
 * eq:output): the block output is added to the one branch layer mod n, in
 * place, the other branches untouched: state[t][layer % n][c] += y[t][c]
 * (one fp32 add, then the store).  layer >= 0.
 *   state in/out [N][n][d];  y in [N][d] (act dtype)
 */
gr_status gr_round_robin_write(void *state, const void *y, int32_t layer, gr_dtype dt, int64_t N,
                               int32_t n, int32_t d, void *stream);

/*
 * gr_write_per_channel -- eq:write with per-channel strengths ("Qwen3.8-
 * Flash-Next architecture notes, 06 Residual", sec. 3: a per-channel write
 * was tried in place of the per-branch scalar).  The pages give no formula
 * for predicting per-channel strengths; here they are a learned [n][d]
 * parameter: state[t][i][c] += s[i][c] * y[t][c] (one fp32 FMA, then the
 * store), in place.
 *   state in/out [N][n][d];  y in [N][d] (act dtype);  s in [n][d] fp32
 */
gr_status gr_write_per_channel(void *state, const void *y, const float *s, gr_dtype dt, int64_t N,
                               int32_t n, int32_t d, void *stream);

/*
 * gr_collapse -- read-out of the widened stream after the last block: the
 * branches summed in fp32 (h, not stored), then out = w (.) h /
 * sqrt(mean(h^2) + eps).  (The GR pages describe no read-out; the sum-then-
 * RMSNorm form is the one given for another four-stream residual.)
 *   state in [N][n][d];  w in [d] (act dtype);  out out [N][d] (act dtype)
 */
gr_status gr_collapse(const void *state, const void *w, float eps, void *out, gr_dtype dt, int64_t N,
                      int32_t n, int32_t d, void *stream);

/*
 * ---- Hyper-Connections (HC) and manifold-constrained HC (mHC) -------------
 * The branch-mixing family the GR design was cut down from ("Paper reading:
 * Qwen3.8 Flash Next", part 2 Residual, sec. 2 Hyper-Connections): a block
 * reads x = H_mix^T R, runs y = F(Norm(x)) (eq:block) and writes
 *   R'_i = sum_j H_res[i][j] R_j + H_comb[i] y,
 * each operator a static term plus a data-dependent one predicted from the
 * per-branch-normalised state Rbar_i = g_i (.) R_i / rms(R_i) (eq:mix,
 * eq:combine), with a_ik = Rbar_i . P_k:
 *   GR_HC_TANH (HC):  H_mix_i = hm_i + lm tanh(a_i0), H_comb_i = hc_i + lc tanh(a_i1),
 *                     H_res[i][j] = hr_ij + lr tanh(a_i,2+j)
 *   GR_HC_MHC  (mHC): H_mix_i = sigmoid(hm_i + lm a_i0), H_comb_i = 2 sigmoid(hc_i + lc a_i1),
 *                     H_res = `sinkhorn_iters` Sinkhorn-Knopp steps (rows scaled
 *                     to sum 1, then columns) on exp(hr_ij + lr a_i,2+j)
 * ("DepthBench", sec. 2.5: sigmoid read weights, twice-sigmoid write weights,
 * 20 Sinkhorn-Knopp iterations).  The block's Norm is an RMSNorm with gain
 * w_norm: u = w_norm (.) x / sqrt(mean(x^2) + eps).  The read predicts all
 * three operators from the same state and hands the write's coefficient
 * record coeff[t] = [H_comb (n) | H_res row-major (n*n)] (fp32).
 * dtype GR_F32 or GR_BF16 (state, y, u, gains and P share it); 1 <= n <= 8.
 * bf16 with n in {1, 2, 4} and d <= 4096 runs one workgroup per token that
 * keeps the token's state in registers: the fused call reads and writes the
 * state once.  No workspace; coeff_in and coeff_out must not overlap.
 */
typedef enum gr_hc_mode { GR_HC_TANH = 0, GR_HC_MHC = 1 } gr_hc_mode;

typedef struct gr_hc_layer {
    int32_t n, d;              /* branches (1..8) and width */
    int32_t mode;              /* gr_hc_mode */
    int32_t sinkhorn_iters;    /* GR_HC_MHC: Sinkhorn-Knopp steps (0..1000); the pages use 20 */
    float eps;                 /* both RMSNorms, inside the root (>= 0, finite) */
    float lambda_mix, lambda_comb, lambda_res;   /* scales of the dynamic terms */
    const void *gamma;         /* [n][d]   per-branch gains of Rbar */
    const void *w_norm;        /* [d]      gain of the block's RMSNorm on x */
    const void *w_proj;        /* [n+2][d] rows W_mix, W_comb, then column j of W_res as row 2+j */
    const float *h_static;     /* [2n + n*n] fp32: hm | hc | hr (row-major) */
} gr_hc_layer;

/*
 * gr_hc_read -- x, its RMSNorm u, and the write's coefficients.
 *   state in [N][n][d];  u out [N][d];  coeff out [N][n + n*n] fp32
 */
gr_status gr_hc_read(const void *state, gr_dtype dt, int64_t N, const gr_hc_layer *L, void *u,
                     float *coeff, void *stream);

/*
 * gr_hc_write -- in place: R'_i = sum_j H_res[i][j] R_j + H_comb[i] y, summed
 * in fp32 and stored in the state dtype (round to nearest even).
 *   state in/out [N][n][d];  y in [N][d];  coeff in [N][n + n*n] fp32
 */
gr_status gr_hc_write(void *state, const void *y, const float *coeff, gr_dtype dt, int64_t N,
                      int32_t n, int32_t d, void *stream);

/*
 * gr_hc_fused_write_read -- gr_hc_write of block l, then gr_hc_read of block
 * l+1 with `next` on the stored state (the state equals gr_hc_write's).
 *   state in/out [N][n][d];  y in [N][d];  coeff_in in [N][n + n*n]
 *   u_next out [N][d];  coeff_next out [N][n + n*n]
 */
gr_status gr_hc_fused_write_read(void *state, const void *y, const float *coeff_in, gr_dtype dt,
                                 int64_t N, const gr_hc_layer *next, void *u_next, float *coeff_next,
                                 void *stream);

/* Bytes of workspace `op` needs for N tokens of layer L (may be 0), for that
 * layer as given: with or without W_write the layout differs, so query with
 * the layer the call will use.
 * The workspace needs no initialisation: a call writes every byte it reads.
 * Calls that share a workspace must not run concurrently (same stream, or
 * synchronised). */
gr_status gr_workspace_size(int op, gr_dtype dt, int64_t N, const gr_layer *L, size_t *bytes);

/* Diagnostic of the single-pass path (GR_KERNEL_VARIANT=single): *word
 * receives the current GPU's device error word of that path -- bit 0 is set
 * when one of its bounded waits on another workgroup timed out, after which
 * the call's outputs are not to be trusted -- and is cleared when reset != 0.
 * Synchronous (copies one word from the device).  0 when the path is unused. */
gr_status gr_device_error_word(uint32_t *word, int reset);

/* Static description of a status code. */
const char *gr_status_string(gr_status status);

/* Message of the calling thread's last failed call ("" if none). */
const char *gr_last_error(void);

/* ---- measurement support (not part of the GR method) ------------------ */

/* The chained workload's elementwise sublayer stand-in: y = 0.1 tanh(u),
 * computed in fp32 and stored in dtype (GR_F32 or GR_BF16).  u, y [count]. */
gr_status gr_bench_tanh_standin(const void *u, void *y, gr_dtype dt, int64_t count,
                                void *stream);

/* Streaming copy probe: dst[0..bytes) = src[0..bytes), 16-byte vectors.
 * bytes must be a multiple of 16.  Measures attainable HBM bandwidth. */
gr_status gr_bench_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GR_H */
