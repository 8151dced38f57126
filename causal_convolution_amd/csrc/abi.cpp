// C ABI of libwanvae.so: argument validation, workspace planning, dispatch
// to the HIP kernels, per-kernel timing.  Every check runs on the host before
// the first launch of a call; see include/wanvae.h for the contract.
#include "wanvae.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

#define WV_CHECK(cond, code, ...)              \
    do {                                       \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+an) and [b, b+bn) intersect (empty ranges never do)
bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bn && b0 < a0 + an;
}

size_t esize(int32_t dt) { return dt == WANVAE_BF16 ? 2 : 4; }

bool valid_dtype(int32_t dt) { return dt == WANVAE_F32 || dt == WANVAE_BF16; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// number of positions n*t*h*w, with overflow / sign checks
int positions(const wanvae_dims *d, int64_t *P) {
    WV_CHECK(d != nullptr, WANVAE_ERR_NULL, "dims is NULL");
    WV_CHECK(d->n >= 0 && d->t >= 0 && d->h >= 0 && d->w >= 0, WANVAE_ERR_SHAPE,
             "negative extent [%lld,%lld,%lld,%lld]", (long long)d->n, (long long)d->t,
             (long long)d->h, (long long)d->w);
    WV_CHECK(d->h <= (1 << 30) && d->w <= (1 << 30), WANVAE_ERR_SHAPE, "h or w too large");
    int64_t p1, p2, p3;
    WV_CHECK(mul_ok(d->n, d->t, &p1) && mul_ok(p1, d->h, &p2) && mul_ok(p2, d->w, &p3) &&
                 p3 <= (INT64_MAX >> 12),
             WANVAE_ERR_SHAPE, "tensor extent overflows");
    *P = p3;
    return WANVAE_OK;
}

// ------------------------------------------------------------------ timing
struct TimingRec {
    int kind;
    hipEvent_t start, stop;
};
std::mutex g_tm_mu;
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;
// Records kept at most: past this many, launches go untimed until the next
// reset (a caller that enables timing and never resets holds bounded state).
constexpr size_t kMaxTimingRecs = 1 << 16;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launches of a call that must not allocate (the no-workspace entry point)
// are never timed: a timing event may have to be created.
thread_local bool g_untimed = false;

// Runs one launch, bracketed by timing events when timing is enabled.
template <typename F>
int timed_launch(int kind, hipStream_t s, const char *what, F &&launch) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (!g_untimed) {
        std::lock_guard<std::mutex> lk(g_tm_mu);
        if (g_timing && g_recs.size() < kMaxTimingRecs) {
            e0 = take_event();
            e1 = take_event();
        }
    }
    bool timed = e0 && e1 && hipEventRecord(e0, s) == hipSuccess;
    const hipError_t err = launch();
    timed = timed && hipEventRecord(e1, s) == hipSuccess;
    if (e0 || e1) {
        std::lock_guard<std::mutex> lk(g_tm_mu);
        if (timed) {
            g_recs.push_back({kind, e0, e1});
        } else {
            if (e0) g_pool.push_back(e0);
            if (e1) g_pool.push_back(e1);
        }
    }
    if (err != hipSuccess)
        return fail(WANVAE_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(err));
    return WANVAE_OK;
}

// ------------------------------------------------------------------ validated launchers
int run_norm(const void *x, void *y, int64_t rows, int C, const float *g, const float *b,
             float eps, int32_t dt, hipStream_t s) {
    if (rows == 0) return WANVAE_OK;
    return timed_launch(WANVAE_KERNEL_NORM, s, "rmsnorm_silu", [&] {
        return dt == WANVAE_BF16 ? wanvae::launch_rmsnorm_silu_bf16(x, y, rows, C, g, b, eps, s)
                                 : wanvae::launch_rmsnorm_silu_f32(x, y, rows, C, g, b, eps, s);
    });
}

// Norm into the conv input layout: 16-channel slices per frame for bf16 (the
// MFMA conv reads whole cache lines of them), channels-last for fp32.
int run_norm_conv_input(const void *x, void *y, int64_t rows, int C, int64_t hw, const float *g,
                        const float *b, float eps, int32_t dt, hipStream_t s) {
    if (dt != WANVAE_BF16) return run_norm(x, y, rows, C, g, b, eps, dt, s);
    if (rows == 0) return WANVAE_OK;
    return timed_launch(WANVAE_KERNEL_NORM, s, "rmsnorm_silu", [&] {
        return wanvae::launch_rmsnorm_silu_bf16_sliced(x, y, rows, C, hw, g, b, eps, s);
    });
}

int run_conv(const wanvae::ConvLaunch &c, int32_t dt, hipStream_t s) {
    if (c.n * c.t * c.h * c.w_ == 0) return WANVAE_OK;
    if (dt == WANVAE_BF16)
        return timed_launch(WANVAE_KERNEL_CONV_BF16, s, "conv3d_bf16", [&] {
            return wanvae::conv3d_narrow_supported(c) ? wanvae::launch_conv3d_narrow(c, s)
                                                      : wanvae::launch_conv3d_bf16(c, s);
        });
    return timed_launch(WANVAE_KERNEL_CONV_F32, s, "conv3d_f32",
                        [&] { return wanvae::launch_conv3d_f32(c, s); });
}

// The bf16 conv addresses one frame slab (h*w*C elements) with 32-bit byte
// offsets: a slab must stay below 2 GiB.
int check_conv_slab(const wanvae_dims *d, int32_t c, int32_t dt) {
    if (dt != WANVAE_BF16) return WANVAE_OK;
    WV_CHECK((double)d->h * (double)d->w * c * 2.0 < 2147483648.0, WANVAE_ERR_SHAPE,
             "a frame of h*w*C = %lld*%lld*%d bf16 values exceeds 2 GiB", (long long)d->h,
             (long long)d->w, c);
    return WANVAE_OK;
}

int check_conv_channels(int32_t cin, int32_t cout, int32_t dt) {
    if (dt == WANVAE_BF16) {
        WV_CHECK(wanvae::conv3d_bf16_supported(cin, cout), WANVAE_ERR_SHAPE,
                 "bf16 conv needs cin a multiple of 16 in [16, 1024] and cout in [1, 1024] "
                 "(got %d, %d)", cin, cout);
    } else {
        WV_CHECK(cin >= 1 && cin <= 1024 && cout >= 1 && cout <= 1024, WANVAE_ERR_SHAPE,
                 "fp32 conv needs cin, cout in [1, 1024] (got %d, %d)", cin, cout);
    }
    return WANVAE_OK;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_params(const wanvae_resblock_params *p) {
    WV_CHECK(p != nullptr, WANVAE_ERR_NULL, "params is NULL");
    WV_CHECK(valid_dtype(p->dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", p->dtype);
    WV_CHECK(wanvae::rmsnorm_silu_supported(p->in_dim) && wanvae::rmsnorm_silu_supported(p->out_dim),
             WANVAE_ERR_SHAPE, "in_dim and out_dim must be multiples of 32 in [32, 1024] (got %d, %d)",
             p->in_dim, p->out_dim);
    if (int r = check_conv_channels(p->in_dim, p->out_dim, p->dtype)) return r;
    WV_CHECK(std::isfinite(p->eps) && p->eps >= 0.0f, WANVAE_ERR_SHAPE, "eps must be finite and >= 0");
    WV_CHECK(p->gamma1 && p->w_a && p->gamma2 && p->w_b, WANVAE_ERR_NULL,
             "gamma1, w_a, gamma2 and w_b are required");
    WV_CHECK(p->w_sc != nullptr || p->in_dim == p->out_dim, WANVAE_ERR_SHAPE,
             "identity shortcut (w_sc NULL) needs in_dim == out_dim (got %d, %d)", p->in_dim,
             p->out_dim);
    const void *ptrs[] = {p->gamma1, p->beta1, p->w_a, p->b_a, p->gamma2,
                          p->beta2,  p->w_b,   p->b_b, p->w_sc, p->b_sc};
    for (const void *q : ptrs)
        WV_CHECK(aligned16(q), WANVAE_ERR_SHAPE, "parameter pointers must be 16-byte aligned");
    return WANVAE_OK;
}

// Workspace: [conv input region | conv A output a].  The conv input region
// holds n1 (the conv A input), then n2 (the conv B input) once conv A has
// consumed n1: P * max(in_dim, out_dim) elements.  bf16 writes n1 and n2 in
// the sliced conv input layout; fp32 normalises a in place into n2.
struct Plan {
    int64_t P = 0;
    size_t x_bytes = 0, y_bytes = 0, n_off = 0, n_bytes = 0, a_off = 0, a_bytes = 0, total = 0;
};

int plan_block(const wanvae_resblock_params *p, const wanvae_dims *d, Plan *pl) {
    if (int r = check_params(p)) return r;
    if (int r = positions(d, &pl->P)) return r;
    if (int r = check_conv_slab(d, p->in_dim > p->out_dim ? p->in_dim : p->out_dim, p->dtype))
        return r;
    const size_t es = esize(p->dtype);
    pl->x_bytes = (size_t)pl->P * p->in_dim * es;
    pl->y_bytes = (size_t)pl->P * p->out_dim * es;
    pl->n_off = 0;
    pl->n_bytes = pl->x_bytes > pl->y_bytes ? pl->x_bytes : pl->y_bytes;
    pl->a_off = round_up(pl->n_bytes);
    pl->a_bytes = pl->y_bytes;
    pl->total = pl->a_off + round_up(pl->a_bytes);
    return WANVAE_OK;
}

// The 1x1x1 shortcut as a separate projection GEMM, S = w_sc x + b_sc, into
// the conv A output region (free once norm2 has read it), added to conv B as a
// plain residual.  Taken where the GEMM kernel's tiles fit the channel counts
// (bf16; in_dim 128, 256 or 384, out_dim a multiple of 64): conv B's fused
// shortcut stages read x in 64-byte pieces and cost several times their
// FLOPs.  S is rounded to bf16 once, like the other stored intermediates.
bool shortcut_as_gemm(const wanvae_resblock_params *p) {
    return p->dtype == WANVAE_BF16 && p->w_sc != nullptr && wanvae::gemm_bf16_tiled_supported(p->in_dim, p->out_dim);
}

// conv B's residual: x itself (identity), S computed into `region`, or x with
// the fused 1x1x1 stages
int setup_residual(const wanvae_resblock_params *p, const void *x, int64_t P, void *region,
                   wanvae::ConvLaunch *cb, hipStream_t s) {
    if (shortcut_as_gemm(p)) {
        if (int r = timed_launch(WANVAE_KERNEL_GEMM, s, "shortcut projection", [&] {
                return wanvae::launch_gemm_bf16_tiled(x, p->w_sc, p->b_sc, nullptr, region, P, p->in_dim,
                                                      p->out_dim, s);
            }))
            return r;
        cb->res = region;
        cb->cres = p->out_dim;
        cb->wsc = nullptr;
        cb->bsc = nullptr;
        return WANVAE_OK;
    }
    cb->res = x;
    cb->wsc = p->w_sc;
    cb->bsc = p->b_sc;
    cb->cres = p->in_dim;
    return WANVAE_OK;
}

int check_block_buffers(const wanvae_resblock_params *p, const Plan &pl, const void *x,
                        const void *y, void *ws, size_t ws_bytes) {
    WV_CHECK(x && y, WANVAE_ERR_NULL, "x and y are required");
    WV_CHECK(aligned16(x) && aligned16(y), WANVAE_ERR_SHAPE, "x and y must be 16-byte aligned");
    WV_CHECK(!overlaps(x, pl.x_bytes, y, pl.y_bytes), WANVAE_ERR_ALIAS, "y overlaps x");
    WV_CHECK(ws != nullptr, WANVAE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", pl.total);
    WV_CHECK(ws_bytes >= pl.total, WANVAE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed",
             ws_bytes, pl.total);
    WV_CHECK(aligned16(ws), WANVAE_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    WV_CHECK(!overlaps(ws, pl.total, x, pl.x_bytes) && !overlaps(ws, pl.total, y, pl.y_bytes),
             WANVAE_ERR_ALIAS, "workspace overlaps x or y");
    (void)p;
    return WANVAE_OK;
}

int forward_planned(const wanvae_resblock_params *p, const Plan &pl, const void *x, void *y,
                    const wanvae_dims *d, void *workspace, hipStream_t s);

// Workspace of wanvae_resblock_forward_noalloc: a file-scope device array that
// each GPU the library runs on holds until the process ends.  Its device
// address is looked up once per device (the name itself is only a host-side
// stand-in) and kept; calls on one device share it.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
int scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    WV_CHECK(dev >= 0 && dev < kMaxDevices, WANVAE_ERR_HIP, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(WANVAE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return WANVAE_OK;
}
}  // namespace

extern "C" {

const char *wanvae_last_error(void) { return g_error.c_str(); }

int wanvae_rmsnorm_silu(const void *x, void *y, int64_t rows, int32_t C, const float *gamma,
                        const float *beta, float eps, int32_t dtype, void *stream) {
    g_error.clear();
    WV_CHECK(valid_dtype(dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", dtype);
    WV_CHECK(wanvae::rmsnorm_silu_supported(C), WANVAE_ERR_SHAPE,
             "C must be a multiple of 32 in [32, 1024] (got %d)", C);
    WV_CHECK(rows >= 0 && rows <= (INT64_MAX >> 12), WANVAE_ERR_SHAPE, "bad row count %lld",
             (long long)rows);
    WV_CHECK(std::isfinite(eps) && eps >= 0.0f, WANVAE_ERR_SHAPE, "eps must be finite and >= 0");
    if (rows == 0) return WANVAE_OK;
    WV_CHECK(x && y && gamma, WANVAE_ERR_NULL, "x, y and gamma are required");
    WV_CHECK(aligned16(x) && aligned16(y) && aligned16(gamma) && aligned16(beta), WANVAE_ERR_SHAPE,
             "pointers must be 16-byte aligned");
    const size_t bytes = (size_t)rows * C * esize(dtype);
    WV_CHECK(x == y || !overlaps(x, bytes, y, bytes), WANVAE_ERR_ALIAS,
             "y partially overlaps x (only y == x is allowed)");
    return run_norm(x, y, rows, C, gamma, beta, eps, dtype, static_cast<hipStream_t>(stream));
}

int wanvae_causal_conv3d(const void *x, const void *cache, const void *w, const float *bias,
                         void *y, const wanvae_dims *d, int32_t cin, int32_t cout, int32_t dtype,
                         void *stream) {
    g_error.clear();
    WV_CHECK(valid_dtype(dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", dtype);
    int64_t P = 0;
    if (int r = positions(d, &P)) return r;
    if (int r = check_conv_channels(cin, cout, dtype)) return r;
    if (int r = check_conv_slab(d, cin > cout ? cin : cout, dtype)) return r;
    if (P == 0) return WANVAE_OK;
    WV_CHECK(x && w && y, WANVAE_ERR_NULL, "x, w and y are required");
    WV_CHECK(aligned16(x) && aligned16(w) && aligned16(y) && aligned16(cache) && aligned16(bias),
             WANVAE_ERR_SHAPE, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype);
    const size_t xb = (size_t)P * cin * es, yb = (size_t)P * cout * es;
    const size_t cb = (size_t)d->n * 2 * d->h * d->w * cin * es;
    const size_t wb = (size_t)wanvae::packed_conv3d_weight_elems(cin, cout, dtype == WANVAE_BF16) * es;
    WV_CHECK(!overlaps(y, yb, x, xb) && !overlaps(y, yb, cache, cb) && !overlaps(y, yb, w, wb),
             WANVAE_ERR_ALIAS, "y overlaps x, cache or w");
    wanvae::ConvLaunch c;
    c.x = x;
    c.cache = cache;
    c.w = w;
    c.bias = bias;
    c.y = y;
    c.n = d->n;
    c.t = d->t;
    c.h = d->h;
    c.w_ = d->w;
    c.cin = cin;
    c.cout = cout;
    return run_conv(c, dtype, static_cast<hipStream_t>(stream));
}

int wanvae_rmsnorm_silu_conv_out(const void *x, const void *cache, const float *gamma, const float *beta,
                                 float eps, const void *w, const float *bias, void *y, const wanvae_dims *d,
                                 int32_t cin, int32_t cout, int32_t dtype, void *stream) {
    g_error.clear();
    WV_CHECK(dtype == WANVAE_BF16, WANVAE_ERR_DTYPE, "the fused norm + conv_out is bf16 only (got dtype %d)",
             dtype);
    WV_CHECK(cin >= 16 && cin <= 96 && cin % 16 == 0 && cout >= 1 && cout <= 3, WANVAE_ERR_SHAPE,
             "the fused norm + conv_out needs cin a multiple of 16 in [16, 96] and cout in [1, 3] "
             "(got %d, %d)", cin, cout);
    WV_CHECK(std::isfinite(eps) && eps >= 0.0f, WANVAE_ERR_SHAPE, "eps must be finite and >= 0");
    int64_t P = 0;
    if (int r = positions(d, &P)) return r;
    if (int r = check_conv_slab(d, cin, dtype)) return r;
    if (P == 0) return WANVAE_OK;
    WV_CHECK(x && w && y && gamma, WANVAE_ERR_NULL, "x, w, y and gamma are required");
    WV_CHECK(aligned16(x) && aligned16(w) && aligned16(y) && aligned16(cache) && aligned16(bias) &&
                 aligned16(gamma) && aligned16(beta),
             WANVAE_ERR_SHAPE, "pointers must be 16-byte aligned");
    const size_t xb = (size_t)P * cin * 2, yb = (size_t)P * cout * 2;
    const size_t cb = (size_t)d->n * 2 * d->h * d->w * cin * 2;
    const size_t wb = (size_t)wanvae::packed_conv3d_weight_elems(cin, cout, true) * 2;
    WV_CHECK(!overlaps(y, yb, x, xb) && !overlaps(y, yb, cache, cb) && !overlaps(y, yb, w, wb),
             WANVAE_ERR_ALIAS, "y overlaps x, cache or w");
    wanvae::ConvLaunch c;
    c.x = x;
    c.cache = cache;
    c.w = w;
    c.bias = bias;
    c.y = y;
    c.n = d->n;
    c.t = d->t;
    c.h = d->h;
    c.w_ = d->w;
    c.cin = cin;
    c.cout = cout;
    c.in_norm_gamma = gamma;
    c.in_norm_beta = beta;
    c.in_norm_eps = eps;
    return run_conv(c, dtype, static_cast<hipStream_t>(stream));
}

int wanvae_pack_conv3d_weights(const void *w, void *packed, int32_t cin, int32_t cout, int32_t dtype,
                               void *stream) {
    g_error.clear();
    WV_CHECK(valid_dtype(dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", dtype);
    if (dtype == WANVAE_BF16) {
        WV_CHECK(cin >= 16 && cin <= 1024 && cin % 16 == 0 && cout >= 1 && cout <= 1024,
                 WANVAE_ERR_SHAPE, "bf16 packing needs cin a multiple of 16 in [16, 1024] and cout in "
                 "[1, 1024] (got %d, %d)", cin, cout);
    } else {
        WV_CHECK(cin >= 1 && cin <= 1024 && cout >= 1 && cout <= 1024, WANVAE_ERR_SHAPE,
                 "fp32 packing needs cin, cout in [1, 1024] (got %d, %d)", cin, cout);
    }
    WV_CHECK(w && packed, WANVAE_ERR_NULL, "w and packed are required");
    WV_CHECK(aligned16(w) && aligned16(packed), WANVAE_ERR_SHAPE, "pointers must be 16-byte aligned");
    const size_t bytes = (size_t)27 * cin * cout * esize(dtype);
    const size_t pbytes =
        (size_t)wanvae::packed_conv3d_weight_elems(cin, cout, dtype == WANVAE_BF16) * esize(dtype);
    WV_CHECK(!overlaps(w, bytes, packed, pbytes), WANVAE_ERR_ALIAS, "packed overlaps w");
    const hipError_t e = wanvae::launch_pack_conv3d_weights(w, packed, cin, cout, dtype == WANVAE_BF16,
                                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "weight packing launch failed: %s", hipGetErrorString(e));
    return WANVAE_OK;
}

int wanvae_packed_conv3d_weight_elems(int32_t cin, int32_t cout, int32_t dtype, int64_t *elems) {
    g_error.clear();
    WV_CHECK(elems != nullptr, WANVAE_ERR_NULL, "elems is NULL");
    WV_CHECK(valid_dtype(dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", dtype);
    WV_CHECK(cin >= 1 && cin <= 1024 && cout >= 1 && cout <= 1024 &&
                 (dtype != WANVAE_BF16 || cin % 16 == 0),
             WANVAE_ERR_SHAPE, "unsupported channel counts %d -> %d", cin, cout);
    *elems = wanvae::packed_conv3d_weight_elems(cin, cout, dtype == WANVAE_BF16);
    return WANVAE_OK;
}

int wanvae_packed_conv2d_weight_elems(int32_t cin, int32_t cout, int32_t dtype, int64_t *elems) {
    g_error.clear();
    WV_CHECK(elems != nullptr, WANVAE_ERR_NULL, "elems is NULL");
    WV_CHECK(dtype == WANVAE_BF16, WANVAE_ERR_DTYPE, "2D conv weights are bf16 only (got dtype %d)", dtype);
    WV_CHECK(wanvae::conv3d_bf16_supported(cin, cout), WANVAE_ERR_SHAPE,
             "bf16 conv needs cin a multiple of 16 in [16, 1024] and cout in [1, 1024] (got %d, %d)", cin, cout);
    *elems = wanvae::packed_conv2d_weight_elems(cin, cout);
    return WANVAE_OK;
}

int wanvae_pack_conv2d_weights(const void *w, void *packed, int32_t cin, int32_t cout, int32_t dtype,
                               void *stream) {
    int64_t elems = 0;
    if (int r = wanvae_packed_conv2d_weight_elems(cin, cout, dtype, &elems)) return r;
    WV_CHECK(w && packed, WANVAE_ERR_NULL, "w and packed are required");
    WV_CHECK(aligned16(w) && aligned16(packed), WANVAE_ERR_SHAPE, "pointers must be 16-byte aligned");
    WV_CHECK(!overlaps(w, (size_t)9 * cin * cout * 2, packed, (size_t)elems * 2), WANVAE_ERR_ALIAS,
             "packed overlaps w");
    const hipError_t e = wanvae::launch_pack_conv2d_weights(w, packed, cin, cout, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "weight packing launch failed: %s", hipGetErrorString(e));
    return WANVAE_OK;
}

namespace {
// upsample2d (temporal = false) and upsample3d (temporal: 2t - 1 output frames)
int upsample_conv(const void *x, const void *w, const float *bias, void *y, const wanvae_dims *d, int32_t cin,
                  int32_t cout, int32_t dtype, bool temporal, void *stream) {
    g_error.clear();
    WV_CHECK(valid_dtype(dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", dtype);
    WV_CHECK(dtype == WANVAE_BF16, WANVAE_ERR_DTYPE, "the upsampler conv is bf16 only");
    int64_t P = 0;
    if (int r = positions(d, &P)) return r;
    if (int r = check_conv_channels(cin, cout, dtype)) return r;
    // the output frame is 2h x 2w; upsample3d makes 2t - 1 frames of t
    wanvae_dims od = *d;
    od.h = 2 * d->h;
    od.w = 2 * d->w;
    if (temporal) od.t = d->t > 0 ? 2 * d->t - 1 : 0;
    int64_t Po = 0;
    if (int r = positions(&od, &Po)) return r;
    if (int r = check_conv_slab(d, cin, dtype)) return r;
    if (int r = check_conv_slab(&od, cout, dtype)) return r;
    if (P == 0) return WANVAE_OK;
    WV_CHECK(x && w && y, WANVAE_ERR_NULL, "x, w and y are required");
    WV_CHECK(aligned16(x) && aligned16(w) && aligned16(y) && aligned16(bias), WANVAE_ERR_SHAPE,
             "pointers must be 16-byte aligned");
    const size_t xb = (size_t)P * cin * 2, yb = (size_t)Po * cout * 2;
    const size_t wb = (size_t)wanvae::packed_conv2d_weight_elems(cin, cout) * 2;
    WV_CHECK(!overlaps(y, yb, x, xb) && !overlaps(y, yb, w, wb) && !overlaps(y, yb, bias, (size_t)cout * 4),
             WANVAE_ERR_ALIAS, "y overlaps x, w or bias");
    wanvae::ConvLaunch c;
    c.x = x;
    c.w = w;
    c.bias = bias;
    c.y = y;
    c.n = od.n;
    c.t = od.t;
    c.h = od.h;
    c.w_ = od.w;
    c.cin = cin;
    c.cout = cout;
    c.up2 = true;
    c.up_t = temporal;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return timed_launch(WANVAE_KERNEL_UPSAMPLE, s, temporal ? "upsample3d conv" : "upsample2d conv",
                        [&] { return wanvae::launch_conv3d_bf16(c, s); });
}
}  // namespace

int wanvae_upsample2d_conv(const void *x, const void *w, const float *bias, void *y, const wanvae_dims *d,
                           int32_t cin, int32_t cout, int32_t dtype, void *stream) {
    return upsample_conv(x, w, bias, y, d, cin, cout, dtype, false, stream);
}

int wanvae_upsample3d_conv(const void *x, const void *w, const float *bias, void *y, const wanvae_dims *d,
                           int32_t cin, int32_t cout, int32_t dtype, void *stream) {
    return upsample_conv(x, w, bias, y, d, cin, cout, dtype, true, stream);
}

int wanvae_pointwise_conv(const void *x, const void *w, const float *bias, void *y, int64_t rows,
                          int32_t cin, int32_t cout, int32_t dtype, void *stream) {
    g_error.clear();
    WV_CHECK(valid_dtype(dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", dtype);
    WV_CHECK(cin >= 1 && cin <= 64 && cout >= 1 && cout <= 64, WANVAE_ERR_SHAPE,
             "pointwise conv needs cin, cout in [1, 64] (got %d, %d)", cin, cout);
    WV_CHECK(rows >= 0 && rows <= (INT64_MAX >> 12), WANVAE_ERR_SHAPE, "bad row count %lld",
             (long long)rows);
    if (rows == 0) return WANVAE_OK;
    WV_CHECK(x && w && y, WANVAE_ERR_NULL, "x, w and y are required");
    WV_CHECK(aligned16(x) && aligned16(w) && aligned16(y) && aligned16(bias), WANVAE_ERR_SHAPE,
             "pointers must be 16-byte aligned");
    const size_t es = esize(dtype);
    const size_t xb = (size_t)rows * cin * es, yb = (size_t)rows * cout * es;
    WV_CHECK(!overlaps(y, yb, x, xb) && !overlaps(y, yb, w, (size_t)cout * cin * es) &&
                 !overlaps(y, yb, bias, (size_t)cout * 4),
             WANVAE_ERR_ALIAS, "y overlaps x, w or bias");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return timed_launch(WANVAE_KERNEL_POINTWISE, s, "pointwise_conv", [&] {
        return wanvae::launch_pointwise_conv(x, w, bias, y, rows, cin, cout, dtype == WANVAE_BF16, s);
    });
}

int wanvae_resblock_workspace_size(const wanvae_resblock_params *p, const wanvae_dims *d,
                                   size_t *bytes) {
    g_error.clear();
    WV_CHECK(bytes != nullptr, WANVAE_ERR_NULL, "bytes is NULL");
    Plan pl;
    if (int r = plan_block(p, d, &pl)) return r;
    *bytes = pl.total;
    return WANVAE_OK;
}

int wanvae_resblock_forward(const wanvae_resblock_params *p, const void *x, void *y,
                            const wanvae_dims *d, void *workspace, size_t ws_bytes, void *stream) {
    g_error.clear();
    Plan pl;
    if (int r = plan_block(p, d, &pl)) return r;
    if (pl.P == 0) return WANVAE_OK;
    if (int r = check_block_buffers(p, pl, x, y, workspace, ws_bytes)) return r;
    return forward_planned(p, pl, x, y, d, workspace, static_cast<hipStream_t>(stream));
}

int wanvae_resblock_forward_noalloc(const wanvae_resblock_params *p, const void *x, void *y,
                                    const wanvae_dims *d, void *stream) {
    g_error.clear();
    Plan pl;
    if (int r = plan_block(p, d, &pl)) return r;
    if (pl.P == 0) return WANVAE_OK;
    WV_CHECK(pl.total <= kScratchBytes, WANVAE_ERR_WORKSPACE,
             "block of %lld positions needs %zu bytes of workspace; the library's own scratch holds "
             "%zu (use wanvae_resblock_forward with a caller workspace)",
             (long long)pl.P, pl.total, kScratchBytes);
    void *ws = nullptr;
    if (int r = scratch_address(&ws)) return r;
    if (int r = check_block_buffers(p, pl, x, y, ws, kScratchBytes)) return r;
    g_untimed = true;
    const int r = forward_planned(p, pl, x, y, d, ws, static_cast<hipStream_t>(stream));
    g_untimed = false;
    return r;
}

int wanvae_wait_giveups(uint64_t *count) {
    g_error.clear();
    WV_CHECK(count != nullptr, WANVAE_ERR_NULL, "count is NULL");
    const hipError_t e = wanvae::read_wait_giveups(count);
    if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "reading the wait give-up count: %s", hipGetErrorString(e));
    return WANVAE_OK;
}

int wanvae_wait_giveups_reset(void) {
    g_error.clear();
    const hipError_t e = wanvae::reset_wait_giveups();
    if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "resetting the wait give-up count: %s", hipGetErrorString(e));
    return WANVAE_OK;
}

int wanvae_set_wait_bound(int32_t polls) {
    g_error.clear();
    wanvae::set_wait_bound(polls);
    return WANVAE_OK;
}

}  // extern "C"

namespace {
// Where the block's intermediates live in the workspace, and whether conv A
// computes norm2 + SiLU in its epilogue (bf16 with out_dim 32 or 96: one
// tile then holds every channel of its positions).  Unfused, n1 and later n2
// take the conv input region (bf16: n2 sliced from a; fp32: a normalised in
// place) and S, a GEMM shortcut's output, takes a's region once norm2 has
// read it.  Fused, conv A writes n2 straight into a's region (n1 is still
// being read there by other tiles) and S takes the conv input region.
struct Regions {
    void *n1, *a, *n2, *s;
    bool fused;
};

Regions block_regions(const wanvae_resblock_params *p, const Plan &pl, void *workspace) {
    char *ws = static_cast<char *>(workspace);
    Regions r;
    r.n1 = ws + pl.n_off;
    r.a = ws + pl.a_off;
    r.fused = p->dtype == WANVAE_BF16 && wanvae::conv3d_bf16_norm_supported(p->out_dim);
    r.n2 = r.fused ? r.a : p->dtype == WANVAE_BF16 ? r.n1 : r.a;
    r.s = r.fused ? r.n1 : r.a;
    return r;
}

// conv A: into a, or with norm2 + SiLU in its epilogue into n2 when fused
wanvae::ConvLaunch conv_a_launch(const wanvae_resblock_params *p, const wanvae_dims *d, const Regions &g) {
    wanvae::ConvLaunch ca;
    ca.x = g.n1;
    ca.x_sliced = p->dtype == WANVAE_BF16;
    ca.w = p->w_a;
    ca.bias = p->b_a;
    ca.y = g.fused ? g.n2 : g.a;
    ca.n = d->n;
    ca.t = d->t;
    ca.h = d->h;
    ca.w_ = d->w;
    ca.cin = p->in_dim;
    ca.cout = p->out_dim;
    if (g.fused) {
        ca.norm_out = true;
        ca.norm_gamma = p->gamma2;
        ca.norm_beta = p->beta2;
        ca.norm_eps = p->eps;
    }
    return ca;
}

// The block's launches once plan and buffers are checked.
int forward_planned(const wanvae_resblock_params *p, const Plan &pl, const void *x, void *y,
                    const wanvae_dims *d, void *workspace, hipStream_t s) {
    const Regions g = block_regions(p, pl, workspace);
    const int64_t hw = d->h * d->w;

    if (int r = run_norm_conv_input(x, g.n1, pl.P, p->in_dim, hw, p->gamma1, p->beta1, p->eps, p->dtype, s))
        return r;
    wanvae::ConvLaunch ca = conv_a_launch(p, d, g);
    if (int r = run_conv(ca, p->dtype, s)) return r;
    if (!g.fused)
        if (int r = run_norm_conv_input(g.a, g.n2, pl.P, p->out_dim, hw, p->gamma2, p->beta2, p->eps, p->dtype, s))
            return r;
    wanvae::ConvLaunch cb = ca;
    cb.norm_out = false;
    cb.x = g.n2;
    cb.w = p->w_b;
    cb.bias = p->b_b;
    cb.y = y;
    cb.cin = p->out_dim;
    if (int r = setup_residual(p, x, pl.P, g.s, &cb, s)) return r;
    return run_conv(cb, p->dtype, s);
}
}  // namespace

extern "C" {

int wanvae_resblock_stream_step(const wanvae_resblock_params *p, const void *x_chunk,
                                void *y_chunk, const wanvae_dims *d, void *cache_a, void *cache_b,
                                void *workspace, size_t ws_bytes, void *stream) {
    g_error.clear();
    Plan pl;
    if (int r = plan_block(p, d, &pl)) return r;
    if (pl.P == 0) return WANVAE_OK;
    if (int r = check_block_buffers(p, pl, x_chunk, y_chunk, workspace, ws_bytes)) return r;
    WV_CHECK(cache_a && cache_b, WANVAE_ERR_NULL, "cache_a and cache_b are required");
    WV_CHECK(aligned16(cache_a) && aligned16(cache_b), WANVAE_ERR_SHAPE,
             "caches must be 16-byte aligned");
    const size_t es = esize(p->dtype);
    const size_t slab_a = (size_t)d->h * d->w * p->in_dim * es;
    const size_t slab_b = (size_t)d->h * d->w * p->out_dim * es;
    const size_t ca_bytes = (size_t)d->n * 2 * slab_a, cb_bytes = (size_t)d->n * 2 * slab_b;
    WV_CHECK(!overlaps(cache_a, ca_bytes, cache_b, cb_bytes) &&
                 !overlaps(cache_a, ca_bytes, x_chunk, pl.x_bytes) &&
                 !overlaps(cache_a, ca_bytes, y_chunk, pl.y_bytes) &&
                 !overlaps(cache_b, cb_bytes, x_chunk, pl.x_bytes) &&
                 !overlaps(cache_b, cb_bytes, y_chunk, pl.y_bytes) &&
                 !overlaps(cache_a, ca_bytes, workspace, pl.total) &&
                 !overlaps(cache_b, cb_bytes, workspace, pl.total),
             WANVAE_ERR_ALIAS, "caches overlap each other, x, y or the workspace");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Regions g = block_regions(p, pl, workspace);
    const int64_t hw = d->h * d->w;

    if (int r = run_norm_conv_input(x_chunk, g.n1, pl.P, p->in_dim, hw, p->gamma1, p->beta1, p->eps,
                                    p->dtype, s))
        return r;
    wanvae::ConvLaunch ca = conv_a_launch(p, d, g);
    ca.cache = cache_a;
    if (int r = run_conv(ca, p->dtype, s)) return r;
    if (int r = timed_launch(WANVAE_KERNEL_ROLL, s, "roll_cache", [&] {
            return wanvae::launch_roll_cache(cache_a, g.n1, d->n, d->t, (int64_t)slab_a, s);
        }))
        return r;
    // n2 (or S) may take n1's place: the roll above has been enqueued before it
    if (!g.fused)
        if (int r = run_norm_conv_input(g.a, g.n2, pl.P, p->out_dim, hw, p->gamma2, p->beta2, p->eps,
                                        p->dtype, s))
            return r;
    wanvae::ConvLaunch cb = ca;
    cb.norm_out = false;
    cb.x = g.n2;
    cb.cache = cache_b;
    cb.w = p->w_b;
    cb.bias = p->b_b;
    cb.y = y_chunk;
    cb.cin = p->out_dim;
    if (int r = setup_residual(p, x_chunk, pl.P, g.s, &cb, s)) return r;
    if (int r = run_conv(cb, p->dtype, s)) return r;
    return timed_launch(WANVAE_KERNEL_ROLL, s, "roll_cache", [&] {
        return wanvae::launch_roll_cache(cache_b, g.n2, d->n, d->t, (int64_t)slab_b, s);
    });
}

namespace {
struct AttnPlan {
    int64_t P = 0, F = 0, HW = 0, HWp = 0;
    size_t x_bytes = 0, u_off = 0, qkv_off = 0, vt_off = 0, o_off = 0, total = 0;
};

int plan_attention(const wanvae_attention_params *p, const wanvae_dims *d, AttnPlan *pl) {
    WV_CHECK(p != nullptr, WANVAE_ERR_NULL, "params is NULL");
    WV_CHECK(wanvae::attention_supported(p->dim), WANVAE_ERR_SHAPE,
             "attention dim must be 64, 128 or 384 (got %d)", p->dim);
    WV_CHECK(std::isfinite(p->eps) && p->eps >= 0.0f, WANVAE_ERR_SHAPE, "eps must be finite and >= 0");
    WV_CHECK(p->gamma && p->w_qkv && p->w_o, WANVAE_ERR_NULL, "gamma, w_qkv and w_o are required");
    const void *ptrs[] = {p->gamma, p->beta, p->w_qkv, p->b_qkv, p->w_o, p->b_o};
    for (const void *q : ptrs)
        WV_CHECK(aligned16(q), WANVAE_ERR_SHAPE, "parameter pointers must be 16-byte aligned");
    if (int r = positions(d, &pl->P)) return r;
    WV_CHECK(d->h * d->w <= (1 << 30), WANVAE_ERR_SHAPE, "h*w too large");
    if (int r = check_conv_slab(d, 3 * p->dim, WANVAE_BF16)) return r;
    const int64_t C = p->dim;
    pl->F = d->n * d->t;
    pl->HW = d->h * d->w;
    pl->HWp = wanvae::attention_keys_padded(pl->HW);
    pl->x_bytes = (size_t)pl->P * C * 2;
    pl->u_off = 0;
    pl->qkv_off = round_up(pl->x_bytes);
    pl->vt_off = pl->qkv_off + round_up((size_t)pl->P * 3 * C * 2);
    pl->o_off = pl->vt_off + round_up((size_t)pl->F * C * pl->HWp * 2);
    pl->total = pl->o_off + round_up(pl->x_bytes);
    return WANVAE_OK;
}
}  // namespace

int wanvae_attention_workspace_size(const wanvae_attention_params *p, const wanvae_dims *d, size_t *bytes) {
    g_error.clear();
    WV_CHECK(bytes != nullptr, WANVAE_ERR_NULL, "bytes is NULL");
    AttnPlan pl;
    if (int r = plan_attention(p, d, &pl)) return r;
    *bytes = pl.total;
    return WANVAE_OK;
}

int wanvae_attention_block(const wanvae_attention_params *p, const void *x, void *y, const wanvae_dims *d,
                           void *workspace, size_t ws_bytes, void *stream) {
    g_error.clear();
    AttnPlan pl;
    if (int r = plan_attention(p, d, &pl)) return r;
    if (pl.P == 0) return WANVAE_OK;
    WV_CHECK(x && y, WANVAE_ERR_NULL, "x and y are required");
    WV_CHECK(aligned16(x) && aligned16(y), WANVAE_ERR_SHAPE, "x and y must be 16-byte aligned");
    WV_CHECK(!overlaps(x, pl.x_bytes, y, pl.x_bytes), WANVAE_ERR_ALIAS, "y overlaps x");
    WV_CHECK(workspace != nullptr, WANVAE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", pl.total);
    WV_CHECK(ws_bytes >= pl.total, WANVAE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes,
             pl.total);
    WV_CHECK(aligned16(workspace), WANVAE_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    WV_CHECK(!overlaps(workspace, pl.total, x, pl.x_bytes) && !overlaps(workspace, pl.total, y, pl.x_bytes),
             WANVAE_ERR_ALIAS, "workspace overlaps x or y");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    void *u = ws + pl.u_off, *qkv = ws + pl.qkv_off, *vt = ws + pl.vt_off, *o = ws + pl.o_off;
    const int C = p->dim;

    if (int r = timed_launch(WANVAE_KERNEL_NORM, s, "rms_norm", [&] {
            return wanvae::launch_rms_norm_bf16(x, u, pl.P, C, p->gamma, p->beta, p->eps, s);
        }))
        return r;
    wanvae::ConvLaunch g;
    g.gemm = true;
    g.x = u;
    g.w = p->w_qkv;
    g.bias = p->b_qkv;
    g.y = qkv;
    g.n = d->n;
    g.t = d->t;
    g.h = d->h;
    g.w_ = d->w;
    g.cin = C;
    g.cout = 3 * C;
    // the projections: the dedicated GEMM kernel where its tiles fit the
    // channel counts, else the conv kernel's GEMM mode
    auto project = [&](const wanvae::ConvLaunch &c) {
        if (wanvae::gemm_bf16_tiled_supported(c.cin, c.cout))
            return wanvae::launch_gemm_bf16_tiled(c.x, c.w, c.bias, c.res, c.y, pl.P, c.cin, c.cout, s);
        return wanvae::launch_gemm_bf16(c, s);
    };
    if (int r = timed_launch(WANVAE_KERNEL_GEMM, s, "qkv projection", [&] { return project(g); }))
        return r;
    if (int r = timed_launch(WANVAE_KERNEL_TRANSPOSE, s, "v transpose", [&] {
            return wanvae::launch_transpose_v(qkv, vt, pl.F, (int)pl.HW, C, s);
        }))
        return r;
    if (int r = timed_launch(WANVAE_KERNEL_ATTENTION, s, "flash attention", [&] {
            return wanvae::launch_flash_attention(qkv, vt, o, pl.F, (int)pl.HW, C, s);
        }))
        return r;
    wanvae::ConvLaunch go = g;
    go.x = o;
    go.w = p->w_o;
    go.bias = p->b_o;
    go.res = x;
    go.cres = C;
    go.y = y;
    go.cout = C;
    return timed_launch(WANVAE_KERNEL_GEMM, s, "output projection", [&] { return project(go); });
}

namespace {
int cache_io(const void *src, void *dst, const wanvae_dims *d, int32_t C, int32_t dtype, bool to_sliced,
             void *stream) {
    g_error.clear();
    WV_CHECK(valid_dtype(dtype), WANVAE_ERR_DTYPE, "unknown dtype %d", dtype);
    WV_CHECK(d != nullptr, WANVAE_ERR_NULL, "dims is NULL");
    wanvae_dims fd = *d;
    fd.t = 2;   // the cache's two frames per batch item
    int64_t P = 0;
    if (int r = positions(&fd, &P)) return r;
    WV_CHECK(C >= 1 && C <= 1024 && (dtype != WANVAE_BF16 || C % 16 == 0), WANVAE_ERR_SHAPE,
             "cache channels must be in [1, 1024] (a multiple of 16 for bf16; got %d)", C);
    if (P == 0) return WANVAE_OK;
    WV_CHECK(src && dst, WANVAE_ERR_NULL, "both buffers are required");
    WV_CHECK(aligned16(src) && aligned16(dst), WANVAE_ERR_SHAPE, "pointers must be 16-byte aligned");
    const size_t bytes = (size_t)P * C * esize(dtype);
    WV_CHECK(!overlaps(src, bytes, dst, bytes), WANVAE_ERR_ALIAS, "the two buffers overlap");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == WANVAE_BF16)
        e = wanvae::launch_cache_layout(src, dst, d->n * 2, d->h * d->w, C, to_sliced, s);
    else   // fp32 caches are channels-last already
        e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "cache layout copy failed: %s", hipGetErrorString(e));
    return WANVAE_OK;
}
}  // namespace

int wanvae_stream_cache_export(const void *cache, void *out, const wanvae_dims *d, int32_t C, int32_t dtype,
                               void *stream) {
    return cache_io(cache, out, d, C, dtype, false, stream);
}

int wanvae_stream_cache_import(const void *in, void *cache, const wanvae_dims *d, int32_t C, int32_t dtype,
                               void *stream) {
    return cache_io(in, cache, d, C, dtype, true, stream);
}

int wanvae_stream_copy(const void *src, void *dst, int64_t bytes, int32_t unroll, int32_t blocks_per_cu,
                       void *stream) {
    g_error.clear();
    WV_CHECK(bytes >= 0 && bytes % 16 == 0, WANVAE_ERR_SHAPE, "bytes must be a non-negative multiple of 16");
    WV_CHECK(unroll == 1 || unroll == 2 || unroll == 4 || unroll == 8, WANVAE_ERR_SHAPE,
             "unroll must be 1, 2, 4 or 8 (got %d)", unroll);
    WV_CHECK(blocks_per_cu >= 1 && blocks_per_cu <= 64, WANVAE_ERR_SHAPE, "blocks_per_cu must be in [1, 64]");
    if (bytes == 0) return WANVAE_OK;
    WV_CHECK(src && dst, WANVAE_ERR_NULL, "src and dst are required");
    WV_CHECK(aligned16(src) && aligned16(dst), WANVAE_ERR_SHAPE, "pointers must be 16-byte aligned");
    WV_CHECK(!overlaps(src, (size_t)bytes, dst, (size_t)bytes), WANVAE_ERR_ALIAS, "dst overlaps src");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return timed_launch(WANVAE_KERNEL_COPY, s, "stream copy", [&] {
        return wanvae::launch_stream_copy(src, dst, bytes, unroll, blocks_per_cu, s);
    });
}

int wanvae_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_tm_mu);
    g_timing = on != 0;
    return WANVAE_OK;
}

int wanvae_timing_reset(void) {
    std::lock_guard<std::mutex> lk(g_tm_mu);
    for (auto &r : g_recs) {
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_recs.clear();
    return WANVAE_OK;
}

int wanvae_timing_read(int32_t kind, int64_t *launches, double *total_ms) {
    g_error.clear();
    WV_CHECK(launches && total_ms, WANVAE_ERR_NULL, "launches and total_ms are required");
    WV_CHECK(kind >= 0 && kind < WANVAE_KERNEL_KINDS, WANVAE_ERR_SHAPE, "unknown kernel kind %d",
             kind);
    std::lock_guard<std::mutex> lk(g_tm_mu);
    int64_t n = 0;
    double ms = 0.0;
    for (auto &r : g_recs) {
        if (r.kind != kind) continue;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
        float f = 0.0f;
        e = hipEventElapsedTime(&f, r.start, r.stop);
        if (e != hipSuccess) return fail(WANVAE_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
        ms += f;
        ++n;
    }
    *launches = n;
    *total_ms = ms;
    return WANVAE_OK;
}

}  // extern "C"
