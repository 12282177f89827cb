// gr_internal.h -- declarations shared by the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace grk {

// Arguments of a read or fused write+read, already validated by the API.
struct ReadArgs {
    bool bf16;           // y, u, gamma and weights are bf16 (else fp32)
    bool fp8;            // the state is fp8 e4m3 (then bf16 is set too)
    bool fused;          // run eq:write with (y, s_in) first, in place
    void *state;         // [N][n][d]
    const void *y;       // [N][d]   (fused only)
    const float *s_in;   // [N][n]   (fused only)
    int64_t N;
    int n, d, r;
    float eps;
    const void *gamma, *wd, *wu, *ww;
    void *u;             // [N][d]
    float *s_out;        // [N][n]
    void *ws;            // workspace (device)
    size_t ws_bytes;
    int k2_variant;      // fast path's second kernel: 0 by size, 1 staged, 2 resident
};

hipError_t launch_read_generic(const ReadArgs &a, hipStream_t st);
hipError_t launch_write(void *state, const void *y, const float *s, bool bf16, bool fp8, int64_t N,
                        int n, int d, hipStream_t st);
hipError_t launch_add_rmsnorm(void *x, const void *y, const void *w, float eps, void *out,
                              bool bf16, int64_t N, int d, hipStream_t st);
hipError_t launch_tanh_standin(const void *u, void *y, bool bf16, int64_t count, hipStream_t st);
hipError_t launch_copy(const void *src, void *dst, size_t bytes, hipStream_t st);

// Variants on the widened state (gr_variants.hip); dt: 0 fp32, 1 bf16,
// 2 e4m3 state with bf16 activations.
hipError_t launch_expand(const void *e, void *state, int dt, int64_t N, int n, int d, hipStream_t st);
hipError_t launch_static_read(const void *state, const float *h, void *u, int dt, int64_t N, int n, int d,
                              hipStream_t st);
hipError_t launch_round_robin_write(void *state, const void *y, int dt, int64_t N, int n, int d, int layer,
                                    hipStream_t st);
hipError_t launch_write_per_channel(void *state, const void *y, const float *s, int dt, int64_t N, int n, int d,
                                    hipStream_t st);
hipError_t launch_collapse(const void *state, const void *w, float eps, void *out, int dt, int64_t N, int n,
                           int d, hipStream_t st);

// Single-pass cluster path (gr_cluster.hip): n = 4, bf16 or e4m3 state,
// d = 4096 (r <= 64) or d = 2048 (r <= 32), on an 8-XCD gfx950 GPU.
bool cluster_path_ok(const ReadArgs &a);
hipError_t launch_cluster(const ReadArgs &a, hipStream_t st);
hipError_t cluster_error_word(uint32_t *word, bool reset);

// Hyper-Connections / mHC (gr_hc.hip); validated by the API.
struct HcArgs {
    bool bf16;                 // state, y, u, gains and P in bf16 (else fp32)
    bool do_write, do_read;
    void *state;               // [N][n][d]
    const void *y;             // [N][d]          (write)
    const float *coeff_in;     // [N][n + n*n]    (write)
    const void *gamma;         // [n][d]          (read)
    const void *w_norm;        // [d]
    const void *w_proj;        // [n+2][d]
    const float *h_static;     // [2n + n*n]
    void *u;                   // [N][d]
    float *coeff_out;          // [N][n + n*n]
    int64_t N;
    int n, d, mode, iters;
    float eps, lam_m, lam_c, lam_r;
};
bool hc_fast_ok(const HcArgs &a);
hipError_t launch_hc(const HcArgs &a, hipStream_t st, bool force_generic);

// MFMA fast path for the bf16 widened state (gr_fast.hip).
bool fast_path_ok(const ReadArgs &a);
size_t fast_workspace_bytes(const ReadArgs &a);   // workspace bytes of this call's fast path
hipError_t launch_read_fast(const ReadArgs &a, hipStream_t st);

}  // namespace grk
