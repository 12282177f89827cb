// gr_api.hip -- host side of the C ABI declared in include/gr.h.
//
// Validates every argument on the host (before any HIP call, so argument
// errors are testable without a GPU), picks a kernel variant and launches it
// on the caller's stream.  No allocation, no synchronisation, no global state
// except the per-thread error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/gr.h"
#include "gr_internal.h"

namespace {

thread_local char g_err[512] = "";

gr_status fail(gr_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

gr_status ok() {
    g_err[0] = '\0';
    return GR_SUCCESS;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

gr_status check_dtype(gr_dtype dt, const char *fn) {
    if (dt != GR_F32 && dt != GR_BF16 && dt != GR_FP8_E4M3)
        return fail(GR_ERROR_INVALID_VALUE, "%s: unknown dtype %d", fn, (int)dt);
    return GR_SUCCESS;
}

// Calls whose tensors all share one dtype (no fp8 state).
gr_status check_plain_dtype(gr_dtype dt, const char *fn) {
    gr_status st = check_dtype(dt, fn);
    if (st) return st;
    if (dt == GR_FP8_E4M3) return fail(GR_ERROR_NOT_SUPPORTED, "%s: fp8 is a state dtype only", fn);
    return GR_SUCCESS;
}

gr_status check_ptr(const void *p, const char *what, const char *fn) {
    if (!p) return fail(GR_ERROR_INVALID_VALUE, "%s: %s is NULL", fn, what);
    if (!aligned16(p)) return fail(GR_ERROR_INVALID_VALUE, "%s: %s is not 16-byte aligned", fn, what);
    return GR_SUCCESS;
}

gr_status check_width(gr_dtype dt, int64_t d, const char *fn) {
    if (d < 1) return fail(GR_ERROR_INVALID_VALUE, "%s: d = %lld must be >= 1", fn, (long long)d);
    const int vec = dt == GR_FP8_E4M3 ? 16 : dt == GR_BF16 ? 8 : 4;
    if (d % vec)
        return fail(GR_ERROR_NOT_SUPPORTED, "%s: d = %lld must be a multiple of %d for this dtype", fn,
                    (long long)d, vec);
    if (d > (1 << 24)) return fail(GR_ERROR_NOT_SUPPORTED, "%s: d = %lld too large", fn, (long long)d);
    return GR_SUCCESS;
}

gr_status check_tokens(int64_t N, const char *fn) {
    if (N < 0) return fail(GR_ERROR_INVALID_VALUE, "%s: N = %lld is negative", fn, (long long)N);
    if (N > 0x7fffffffLL) return fail(GR_ERROR_NOT_SUPPORTED, "%s: N = %lld exceeds 2^31-1", fn, (long long)N);
    return GR_SUCCESS;
}

gr_status check_layer(const gr_layer *L, gr_dtype dt, const char *fn) {
    if (!L) return fail(GR_ERROR_INVALID_VALUE, "%s: layer is NULL", fn);
    if (L->n < 1 || L->n > 8) return fail(GR_ERROR_INVALID_VALUE, "%s: n = %d outside 1..8", fn, L->n);
    gr_status st = check_width(dt, L->d, fn);
    if (st) return st;
    if (L->r < 0 || L->r > 512) return fail(GR_ERROR_INVALID_VALUE, "%s: r = %d outside 0..512", fn, L->r);
    if (!(L->eps >= 0.f) || !isfinite(L->eps))
        return fail(GR_ERROR_INVALID_VALUE, "%s: eps must be finite and >= 0", fn);
    if ((int64_t)L->n * L->d > (1 << 24))
        return fail(GR_ERROR_NOT_SUPPORTED, "%s: n*d too large", fn);
    if ((st = check_ptr(L->gamma, "gamma", fn))) return st;
    if (L->r > 0) {
        if ((st = check_ptr(L->w_down, "w_down", fn))) return st;
        if ((st = check_ptr(L->w_up, "w_up", fn))) return st;
    } else if (L->w_down || L->w_up) {
        return fail(GR_ERROR_INVALID_VALUE, "%s: r == 0 requires w_down == w_up == NULL", fn);
    }
    if (L->w_write && !aligned16(L->w_write))
        return fail(GR_ERROR_INVALID_VALUE, "%s: w_write is not 16-byte aligned", fn);
    return GR_SUCCESS;
}

// GR_KERNEL_VARIANT selects kernels for A/B checks: "generic" forces the
// shape-generic kernels; "staged" / "resident" force that form of the fast
// path's second kernel whatever the token count; "single" takes the
// single-pass cluster kernel where the shape allows it (n = 4, d = 4096 or
// 2048, 16 <= r <= 64 with r % 16 == 0, bf16 state).
bool force_generic() {
    const char *v = getenv("GR_KERNEL_VARIANT");
    return v && strcmp(v, "generic") == 0;
}

int k2_variant() {
    const char *v = getenv("GR_KERNEL_VARIANT");
    if (v && strcmp(v, "staged") == 0) return 1;
    if (v && strcmp(v, "resident") == 0) return 2;
    return 0;
}

size_t read_workspace(gr_dtype dt, int64_t N, const gr_layer *L) {
    grk::ReadArgs a{};
    a.bf16 = dt != GR_F32;
    a.fp8 = dt == GR_FP8_E4M3;
    a.N = N; a.n = L->n; a.d = L->d; a.r = L->r;
    a.ww = L->w_write;
    if (grk::cluster_path_ok(a)) return 0;   // single pass: exchange in the library's own device array
    return grk::fast_path_ok(a) && !force_generic() ? grk::fast_workspace_bytes(a) : 0;
}

gr_status launched(hipError_t e, const char *fn) {
    if (e != hipSuccess) return fail(GR_ERROR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

gr_status run_read(grk::ReadArgs &a, const gr_layer *L, size_t ws_bytes, hipStream_t st,
                   const char *fn) {
    const gr_dtype dt = a.fp8 ? GR_FP8_E4M3 : a.bf16 ? GR_BF16 : GR_F32;
    const size_t need = read_workspace(dt, a.N, L);
    if (need > 0) {
        if (ws_bytes < need)
            return fail(GR_ERROR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
        gr_status s = check_ptr(a.ws, "workspace", fn);
        if (s) return s;
    }
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    a.k2_variant = k2_variant();
    if (grk::cluster_path_ok(a)) return launched(grk::launch_cluster(a, st), fn);
    if (grk::fast_path_ok(a) && !force_generic()) return launched(grk::launch_read_fast(a, st), fn);
    return launched(grk::launch_read_generic(a, st), fn);
}

void fill_layer(grk::ReadArgs &a, const gr_layer *L) {
    a.n = L->n; a.d = L->d; a.r = L->r; a.eps = L->eps;
    a.gamma = L->gamma; a.wd = L->w_down; a.wu = L->w_up; a.ww = L->w_write;
}

// Shared checks of the variant calls: dtype, N, n, d; 0 fp32, 1 bf16, 2 fp8 state.
gr_status check_variant(gr_dtype dt, int64_t N, int32_t n, int32_t d, const char *fn, int *code) {
    gr_status st;
    if ((st = check_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (n < 1 || n > 8) return fail(GR_ERROR_INVALID_VALUE, "%s: n = %d outside 1..8", fn, n);
    if ((st = check_width(dt, d, fn))) return st;
    *code = dt == GR_F32 ? 0 : dt == GR_BF16 ? 1 : 2;
    return GR_SUCCESS;
}

// Scratch of gr_fused_write_read_noalloc: one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = 48ull << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ScratchPtr {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
constexpr int kMaxScratchDevices = 64;
ScratchPtr g_scratch[kMaxScratchDevices];

// Device address of the current GPU's `scratch` (set up on its first use).
hipError_t scratch_ptr(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    ScratchPtr &sp = g_scratch[dev];
    std::call_once(sp.once, [&] {
        sp.err = hipGetSymbolAddress(&sp.ptr, HIP_SYMBOL(scratch));
        if (sp.err == hipSuccess && !sp.ptr) sp.err = hipErrorInvalidSymbol;
    });
    *ptr = sp.ptr;
    return sp.err;
}

}  // namespace

extern "C" {

gr_status gr_read(const void *state, gr_dtype dt, int64_t N, const gr_layer *L, void *u, float *s,
                  void *workspace, size_t ws_bytes, void *stream) {
    const char *fn = "gr_read";
    gr_status st;
    if ((st = check_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if ((st = check_layer(L, dt, fn))) return st;
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(u, "u", fn)) ||
        (st = check_ptr(s, "s", fn)))
        return st;
    grk::ReadArgs a{};
    a.bf16 = dt != GR_F32;
    a.fp8 = dt == GR_FP8_E4M3;
    a.fused = false;
    a.state = const_cast<void *>(state);
    a.N = N;
    fill_layer(a, L);
    a.u = u; a.s_out = s; a.ws = workspace; a.ws_bytes = ws_bytes;
    return run_read(a, L, ws_bytes, (hipStream_t)stream, fn);
}

gr_status gr_fused_write_read(void *state, const void *y, const float *s_in, gr_dtype dt, int64_t N,
                              const gr_layer *next, void *u_next, float *s_next, void *workspace,
                              size_t ws_bytes, void *stream) {
    const char *fn = "gr_fused_write_read";
    gr_status st;
    if ((st = check_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if ((st = check_layer(next, dt, fn))) return st;
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(y, "y", fn)) ||
        (st = check_ptr(s_in, "s_in", fn)) || (st = check_ptr(u_next, "u_next", fn)) ||
        (st = check_ptr(s_next, "s_next", fn)))
        return st;
    grk::ReadArgs a{};
    a.bf16 = dt != GR_F32;
    a.fp8 = dt == GR_FP8_E4M3;
    a.fused = true;
    a.state = state; a.y = y; a.s_in = s_in;
    a.N = N;
    fill_layer(a, next);
    a.u = u_next; a.s_out = s_next; a.ws = workspace; a.ws_bytes = ws_bytes;
    return run_read(a, next, ws_bytes, (hipStream_t)stream, fn);
}

gr_status gr_fused_write_read_noalloc(void *state, const void *y, const float *s_in, gr_dtype dt,
                                      int64_t N, const gr_layer *next, void *u_next, float *s_next,
                                      void *stream) {
    const char *fn = "gr_fused_write_read_noalloc";
    gr_status st;
    if ((st = check_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if ((st = check_layer(next, dt, fn))) return st;
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(y, "y", fn)) ||
        (st = check_ptr(s_in, "s_in", fn)) || (st = check_ptr(u_next, "u_next", fn)) ||
        (st = check_ptr(s_next, "s_next", fn)))
        return st;
    const size_t need = read_workspace(dt, N, next);
    if (need > kNoAllocScratchBytes)
        return fail(GR_ERROR_WORKSPACE,
                    "%s: this call needs %zu bytes of scratch, more than the %zu bytes of the "
                    "library's static array (use gr_fused_write_read with a workspace, or fewer tokens)",
                    fn, need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        (void)hipGetLastError();
        hipError_t e = scratch_ptr(&ws);
        if (e != hipSuccess) return fail(GR_ERROR_LAUNCH, "%s: scratch set-up failed: %s", fn, hipGetErrorString(e));
    }
    grk::ReadArgs a{};
    a.bf16 = dt != GR_F32;
    a.fp8 = dt == GR_FP8_E4M3;
    a.fused = true;
    a.state = state; a.y = y; a.s_in = s_in;
    a.N = N;
    fill_layer(a, next);
    a.u = u_next; a.s_out = s_next; a.ws = ws; a.ws_bytes = kNoAllocScratchBytes;
    return run_read(a, next, kNoAllocScratchBytes, (hipStream_t)stream, fn);
}

}  // extern "C"

namespace {

gr_status check_hc_layer(const gr_hc_layer *L, gr_dtype dt, const char *fn) {
    if (!L) return fail(GR_ERROR_INVALID_VALUE, "%s: layer is NULL", fn);
    if (L->n < 1 || L->n > 8) return fail(GR_ERROR_INVALID_VALUE, "%s: n = %d outside 1..8", fn, L->n);
    gr_status st = check_width(dt, L->d, fn);
    if (st) return st;
    if ((int64_t)L->n * L->d > (1 << 24)) return fail(GR_ERROR_NOT_SUPPORTED, "%s: n*d too large", fn);
    if (L->mode != GR_HC_TANH && L->mode != GR_HC_MHC)
        return fail(GR_ERROR_INVALID_VALUE, "%s: unknown mode %d", fn, L->mode);
    if (L->sinkhorn_iters < 0 || L->sinkhorn_iters > 1000)
        return fail(GR_ERROR_INVALID_VALUE, "%s: sinkhorn_iters = %d outside 0..1000", fn, L->sinkhorn_iters);
    if (!(L->eps >= 0.f) || !isfinite(L->eps) || !isfinite(L->lambda_mix) || !isfinite(L->lambda_comb) ||
        !isfinite(L->lambda_res))
        return fail(GR_ERROR_INVALID_VALUE, "%s: eps must be finite and >= 0, the lambdas finite", fn);
    if ((st = check_ptr(L->gamma, "gamma", fn)) || (st = check_ptr(L->w_norm, "w_norm", fn)) ||
        (st = check_ptr(L->w_proj, "w_proj", fn)) || (st = check_ptr(L->h_static, "h_static", fn)))
        return st;
    return GR_SUCCESS;
}

gr_status check_hc_dtype(gr_dtype dt, const char *fn) {
    gr_status st = check_dtype(dt, fn);
    if (st) return st;
    if (dt == GR_FP8_E4M3) return fail(GR_ERROR_NOT_SUPPORTED, "%s: the HC calls take fp32 or bf16", fn);
    return GR_SUCCESS;
}

void fill_hc(grk::HcArgs &a, const gr_hc_layer *L) {
    a.n = L->n; a.d = L->d; a.mode = L->mode; a.iters = L->sinkhorn_iters;
    a.eps = L->eps; a.lam_m = L->lambda_mix; a.lam_c = L->lambda_comb; a.lam_r = L->lambda_res;
    a.gamma = L->gamma; a.w_norm = L->w_norm; a.w_proj = L->w_proj; a.h_static = L->h_static;
}

}  // namespace

extern "C" {

gr_status gr_hc_read(const void *state, gr_dtype dt, int64_t N, const gr_hc_layer *L, void *u,
                     float *coeff, void *stream) {
    const char *fn = "gr_hc_read";
    gr_status st;
    if ((st = check_hc_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if ((st = check_hc_layer(L, dt, fn))) return st;
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(u, "u", fn)) ||
        (st = check_ptr(coeff, "coeff", fn)))
        return st;
    grk::HcArgs a{};
    a.bf16 = dt == GR_BF16;
    a.do_read = true;
    a.state = const_cast<void *>(state);
    a.N = N;
    fill_hc(a, L);
    a.u = u; a.coeff_out = coeff;
    (void)hipGetLastError();
    return launched(grk::launch_hc(a, (hipStream_t)stream, force_generic()), fn);
}

gr_status gr_hc_write(void *state, const void *y, const float *coeff, gr_dtype dt, int64_t N,
                      int32_t n, int32_t d, void *stream) {
    const char *fn = "gr_hc_write";
    gr_status st;
    if ((st = check_hc_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if (n < 1 || n > 8) return fail(GR_ERROR_INVALID_VALUE, "%s: n = %d outside 1..8", fn, n);
    if ((st = check_width(dt, d, fn))) return st;
    if ((int64_t)n * d > (1 << 24)) return fail(GR_ERROR_NOT_SUPPORTED, "%s: n*d too large", fn);
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(y, "y", fn)) ||
        (st = check_ptr(coeff, "coeff", fn)))
        return st;
    grk::HcArgs a{};
    a.bf16 = dt == GR_BF16;
    a.do_write = true;
    a.state = state; a.y = y; a.coeff_in = coeff;
    a.N = N; a.n = n; a.d = d;
    (void)hipGetLastError();
    return launched(grk::launch_hc(a, (hipStream_t)stream, force_generic()), fn);
}

gr_status gr_hc_fused_write_read(void *state, const void *y, const float *coeff_in, gr_dtype dt,
                                 int64_t N, const gr_hc_layer *next, void *u_next, float *coeff_next,
                                 void *stream) {
    const char *fn = "gr_hc_fused_write_read";
    gr_status st;
    if ((st = check_hc_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if ((st = check_hc_layer(next, dt, fn))) return st;
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(y, "y", fn)) ||
        (st = check_ptr(coeff_in, "coeff_in", fn)) || (st = check_ptr(u_next, "u_next", fn)) ||
        (st = check_ptr(coeff_next, "coeff_next", fn)))
        return st;
    grk::HcArgs a{};
    a.bf16 = dt == GR_BF16;
    a.do_write = true; a.do_read = true;
    a.state = state; a.y = y; a.coeff_in = coeff_in;
    a.N = N;
    fill_hc(a, next);
    a.u = u_next; a.coeff_out = coeff_next;
    (void)hipGetLastError();
    return launched(grk::launch_hc(a, (hipStream_t)stream, force_generic()), fn);
}

gr_status gr_device_error_word(uint32_t *word, int reset) {
    const char *fn = "gr_device_error_word";
    if (!word) return fail(GR_ERROR_INVALID_VALUE, "%s: word is NULL", fn);
    hipError_t e = grk::cluster_error_word(word, reset != 0);
    if (e != hipSuccess) return fail(GR_ERROR_LAUNCH, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

gr_status gr_write(void *state, const void *y, const float *s, gr_dtype dt, int64_t N, int32_t n,
                   int32_t d, void *stream) {
    const char *fn = "gr_write";
    gr_status st;
    if ((st = check_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if (n < 1 || n > 8) return fail(GR_ERROR_INVALID_VALUE, "%s: n = %d outside 1..8", fn, n);
    if ((st = check_width(dt, d, fn))) return st;
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(y, "y", fn)) ||
        (st = check_ptr(s, "s", fn)))
        return st;
    (void)hipGetLastError();
    return launched(grk::launch_write(state, y, s, dt != GR_F32, dt == GR_FP8_E4M3, N, n, d,
                                      (hipStream_t)stream), fn);
}

gr_status residual_add_rmsnorm(void *x, const void *y, const void *w, float eps, void *out,
                               gr_dtype dt, int64_t N, int32_t d, void *stream) {
    const char *fn = "residual_add_rmsnorm";
    gr_status st;
    if ((st = check_plain_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if ((st = check_width(dt, d, fn))) return st;
    if (!(eps >= 0.f) || !isfinite(eps))
        return fail(GR_ERROR_INVALID_VALUE, "%s: eps must be finite and >= 0", fn);
    if ((st = check_ptr(x, "x", fn)) || (st = check_ptr(y, "y", fn)) || (st = check_ptr(w, "w", fn)) ||
        (st = check_ptr(out, "out", fn)))
        return st;
    if (out == x) return fail(GR_ERROR_INVALID_VALUE, "%s: out must not alias x", fn);
    (void)hipGetLastError();
    return launched(grk::launch_add_rmsnorm(x, y, w, eps, out, dt == GR_BF16, N, d, (hipStream_t)stream), fn);
}

gr_status gr_expand(const void *e, void *state, gr_dtype dt, int64_t N, int32_t n, int32_t d,
                    void *stream) {
    const char *fn = "gr_expand";
    gr_status st;
    int code = 0;
    if ((st = check_variant(dt, N, n, d, fn, &code))) return st;
    if (N == 0) return ok();
    if ((st = check_ptr(e, "e", fn)) || (st = check_ptr(state, "state", fn))) return st;
    (void)hipGetLastError();
    return launched(grk::launch_expand(e, state, code, N, n, d, (hipStream_t)stream), fn);
}

gr_status gr_static_read(const void *state, const float *h, void *u, gr_dtype dt, int64_t N,
                         int32_t n, int32_t d, void *stream) {
    const char *fn = "gr_static_read";
    gr_status st;
    int code = 0;
    if ((st = check_variant(dt, N, n, d, fn, &code))) return st;
    if (N == 0) return ok();
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(h, "h", fn)) || (st = check_ptr(u, "u", fn)))
        return st;
    (void)hipGetLastError();
    return launched(grk::launch_static_read(state, h, u, code, N, n, d, (hipStream_t)stream), fn);
}

gr_status gr_round_robin_write(void *state, const void *y, int32_t layer, gr_dtype dt, int64_t N,
                               int32_t n, int32_t d, void *stream) {
    const char *fn = "gr_round_robin_write";
    gr_status st;
    int code = 0;
    if ((st = check_variant(dt, N, n, d, fn, &code))) return st;
    if (layer < 0) return fail(GR_ERROR_INVALID_VALUE, "%s: layer = %d is negative", fn, layer);
    if (N == 0) return ok();
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(y, "y", fn))) return st;
    (void)hipGetLastError();
    return launched(grk::launch_round_robin_write(state, y, code, N, n, d, layer, (hipStream_t)stream), fn);
}

gr_status gr_write_per_channel(void *state, const void *y, const float *s, gr_dtype dt, int64_t N,
                               int32_t n, int32_t d, void *stream) {
    const char *fn = "gr_write_per_channel";
    gr_status st;
    int code = 0;
    if ((st = check_variant(dt, N, n, d, fn, &code))) return st;
    if (N == 0) return ok();
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(y, "y", fn)) || (st = check_ptr(s, "s", fn)))
        return st;
    (void)hipGetLastError();
    return launched(grk::launch_write_per_channel(state, y, s, code, N, n, d, (hipStream_t)stream), fn);
}

gr_status gr_collapse(const void *state, const void *w, float eps, void *out, gr_dtype dt, int64_t N,
                      int32_t n, int32_t d, void *stream) {
    const char *fn = "gr_collapse";
    gr_status st;
    int code = 0;
    if ((st = check_variant(dt, N, n, d, fn, &code))) return st;
    if (!(eps >= 0.f) || !isfinite(eps))
        return fail(GR_ERROR_INVALID_VALUE, "%s: eps must be finite and >= 0", fn);
    if (N == 0) return ok();
    if ((st = check_ptr(state, "state", fn)) || (st = check_ptr(w, "w", fn)) || (st = check_ptr(out, "out", fn)))
        return st;
    (void)hipGetLastError();
    return launched(grk::launch_collapse(state, w, eps, out, code, N, n, d, (hipStream_t)stream), fn);
}

gr_status gr_workspace_size(int op, gr_dtype dt, int64_t N, const gr_layer *L, size_t *bytes) {
    const char *fn = "gr_workspace_size";
    gr_status st;
    if (!bytes) return fail(GR_ERROR_INVALID_VALUE, "%s: bytes is NULL", fn);
    *bytes = 0;
    if (op != GR_OP_READ && op != GR_OP_FUSED_WRITE_READ)
        return fail(GR_ERROR_INVALID_VALUE, "%s: unknown op %d", fn, op);
    if ((st = check_dtype(dt, fn)) || (st = check_tokens(N, fn))) return st;
    if (N == 0) return ok();
    if (!L) return fail(GR_ERROR_INVALID_VALUE, "%s: layer is NULL", fn);
    if (L->n < 1 || L->n > 8) return fail(GR_ERROR_INVALID_VALUE, "%s: n = %d outside 1..8", fn, L->n);
    if ((st = check_width(dt, L->d, fn))) return st;
    if (L->r < 0 || L->r > 512) return fail(GR_ERROR_INVALID_VALUE, "%s: r = %d outside 0..512", fn, L->r);
    *bytes = read_workspace(dt, N, L);
    return ok();
}

const char *gr_status_string(gr_status status) {
    switch (status) {
    case GR_SUCCESS: return "success";
    case GR_ERROR_INVALID_VALUE: return "invalid value";
    case GR_ERROR_NOT_SUPPORTED: return "not supported";
    case GR_ERROR_LAUNCH: return "launch failed";
    case GR_ERROR_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

const char *gr_last_error(void) { return g_err; }

gr_status gr_bench_tanh_standin(const void *u, void *y, gr_dtype dt, int64_t count, void *stream) {
    const char *fn = "gr_bench_tanh_standin";
    gr_status st;
    if ((st = check_plain_dtype(dt, fn)) || (st = check_tokens(count, fn))) return st;
    if (count == 0) return ok();
    if ((st = check_ptr(u, "u", fn)) || (st = check_ptr(y, "y", fn))) return st;
    (void)hipGetLastError();
    return launched(grk::launch_tanh_standin(u, y, dt == GR_BF16, count, (hipStream_t)stream), fn);
}

gr_status gr_bench_copy(const void *src, void *dst, size_t bytes, void *stream) {
    const char *fn = "gr_bench_copy";
    gr_status st;
    if (bytes == 0) return ok();
    if (bytes % 16) return fail(GR_ERROR_INVALID_VALUE, "%s: bytes must be a multiple of 16", fn);
    if ((st = check_ptr(src, "src", fn)) || (st = check_ptr(dst, "dst", fn))) return st;
    (void)hipGetLastError();
    return launched(grk::launch_copy(src, dst, bytes, (hipStream_t)stream), fn);
}

}  // extern "C"
