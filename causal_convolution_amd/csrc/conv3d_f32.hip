// Causal 3x3x3 conv in fp32, direct form (correctness path for fp32 blocks).
//
//   y[p, co] = bias[co] + sum_{kt,kh,kw,ci} w[co][kt][kh][kw][ci] * Z[t+kt-2, h+kh-1, w+kw-1, ci]
// ("Sharding of WAN 2.2 VAE", Available Sharding Dimensions for the conv;
// "Closing the gap", section 2 for the causal T pad and the H/W zero pad).
// Frames before 0 come from the feat_cache when one is given, else are 0.
// The epilogue adds the residual: x itself (identity shortcut) or the 1x1x1
// shortcut w_sc . x + b_sc, with one final fp32 rounding chain.
//
// One thread per output element (position, output channel); the reduction
// runs over taps then input channels with fp32 fma.  The fp32 blocks are
// small, so this kernel favours clarity over speed; the bf16 blocks use the
// MFMA implicit-GEMM kernel.
#include "internal.h"

namespace wanvae {
namespace {

__global__ __launch_bounds__(256) void conv3d_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ cache, const float *__restrict__ w,
    const float *__restrict__ bias, const float *__restrict__ res, const float *__restrict__ wsc,
    const float *__restrict__ bsc, float *__restrict__ y, int64_t N, int64_t T, int64_t H,
    int64_t W, int cin, int cout, int cres) {
    const int64_t total = N * T * H * W * cout;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int co = (int)(idx % cout);
        const int64_t p = idx / cout;
        const int64_t wq = p % W;
        const int64_t hq = (p / W) % H;
        const int64_t tq = (p / (W * H)) % T;
        const int64_t nq = p / (W * H * T);
        float acc = 0.0f;
        for (int kt = 0; kt < 3; ++kt) {
            const int64_t ts = tq + kt - 2;
            for (int kh = 0; kh < 3; ++kh) {
                const int64_t hs = hq + kh - 1;
                if (hs < 0 || hs >= H) continue;
                for (int kw = 0; kw < 3; ++kw) {
                    const int64_t ws = wq + kw - 1;
                    if (ws < 0 || ws >= W) continue;
                    const float *src;
                    if (ts >= 0)
                        src = x + (((nq * T + ts) * H + hs) * W + ws) * cin;
                    else if (cache)
                        src = cache + (((nq * 2 + (ts + 2)) * H + hs) * W + ws) * cin;
                    else
                        continue;
                    const float *wr = w + ((int64_t)co * 27 + kt * 9 + kh * 3 + kw) * cin;
                    for (int ci = 0; ci < cin; ++ci) acc = fmaf(wr[ci], src[ci], acc);
                }
            }
        }
        float v = acc + (bias ? bias[co] : 0.0f);
        if (res) {
            if (wsc) {
                float s = 0.0f;
                const float *xr = res + p * cres;
                const float *wr = wsc + (int64_t)co * cres;
                for (int ci = 0; ci < cres; ++ci) s = fmaf(wr[ci], xr[ci], s);
                v += s + (bsc ? bsc[co] : 0.0f);
            } else {
                v += res[p * cres + co];
            }
        }
        y[p * cout + co] = v;
    }
}

// cache[nb][0..1] <- last two frames of [cache[nb], chunk[nb]], 4-byte units.
// With a one-frame chunk each unit moves frame 1 to frame 0 and the chunk's
// frame into frame 1; every unit is read before it is written by the same
// thread, so the in-place shift is race-free.
__global__ __launch_bounds__(256) void roll_cache_kernel(uint32_t *__restrict__ cache,
                                                         const uint32_t *__restrict__ chunk,
                                                         int64_t nbatch, int64_t tc, int64_t slab) {
    const int64_t total = nbatch * slab;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t nb = idx / slab, i = idx % slab;
        uint32_t *c = cache + nb * 2 * slab;
        const uint32_t *z = chunk + nb * tc * slab;
        if (tc >= 2) {
            c[i] = z[(tc - 2) * slab + i];
            c[slab + i] = z[(tc - 1) * slab + i];
        } else {
            const uint32_t prev = c[slab + i];
            c[i] = prev;
            c[slab + i] = z[i];
        }
    }
}

int64_t grid_for(int64_t work, int64_t threads) {
    int64_t b = (work + threads - 1) / threads;
    if (b > 65536) b = 65536;
    return b < 1 ? 1 : b;
}

}  // namespace

hipError_t launch_conv3d_f32(const ConvLaunch &a, hipStream_t s) {
    const int64_t total = a.n * a.t * a.h * a.w_ * a.cout;
    conv3d_f32_kernel<<<dim3((unsigned)grid_for(total, 256)), dim3(256), 0, s>>>(
        static_cast<const float *>(a.x), static_cast<const float *>(a.cache),
        static_cast<const float *>(a.w), a.bias, static_cast<const float *>(a.res),
        static_cast<const float *>(a.wsc), a.bsc, static_cast<float *>(a.y), a.n, a.t, a.h, a.w_,
        a.cin, a.cout, a.cres);
    return hipGetLastError();
}

hipError_t launch_roll_cache(void *cache, const void *chunk, int64_t nbatch, int64_t tc,
                             int64_t slab_bytes, hipStream_t s) {
    const int64_t slab = slab_bytes / 4;
    roll_cache_kernel<<<dim3((unsigned)grid_for(nbatch * slab, 256)), dim3(256), 0, s>>>(
        static_cast<uint32_t *>(cache), static_cast<const uint32_t *>(chunk), nbatch, tc, slab);
    return hipGetLastError();
}

}  // namespace wanvae
