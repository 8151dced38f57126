// Pointwise (1x1x1) conv over rows of channels:
//   y[r][co] = bias[co] + sum_ci w[co][ci] * x[r][ci]
// The decoder's post_quant_conv is such a CausalConv3d with kernel 1 over the
// latent channels ("Sharding of WAN 2.2 VAE", the decoder module tree); with
// kernel size 1 the causal pad is empty, so every position is independent.
//
// Small channel counts only (C_in, C_out <= 64).  C_in in {8, 16, 32, 64}
// (the latent's 16 among them) takes the row form below; any other C_in the
// general form: one thread per output element, C_out consecutive threads per
// row.  Either way the sum runs in fp32 over ascending C_in, the bias is
// added last, and bf16 outputs are rounded once to nearest even.  The work is
// bandwidth-bound: (C_in + C_out) * sizeof(T) bytes per row.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

constexpr int kThreads = 256;
constexpr int kGridCap = 8192;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ inline float load_f32(const T *p);
template <>
__device__ inline float load_f32<float>(const float *p) { return *p; }
template <>
__device__ inline float load_f32<uint16_t>(const uint16_t *p) { return bf16_bits_to_f32(*p); }

template <typename T>
__device__ inline void store_f32(T *p, float v);
template <>
__device__ inline void store_f32<float>(float *p, float v) { *p = v; }
template <>
__device__ inline void store_f32<uint16_t>(uint16_t *p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }

template <typename T>
__global__ __launch_bounds__(kThreads) void pointwise_kernel(const T *__restrict__ x, const T *__restrict__ w,
                                                             const float *__restrict__ bias, T *__restrict__ y,
                                                             int64_t rows, int cin, int cout) {
    const int64_t total = rows * cout;
    for (int64_t e = blockIdx.x * (int64_t)kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        const int64_t r = e / cout;
        const int co = (int)(e - r * cout);
        const T *xr = x + r * cin;
        const T *wr = w + (int64_t)co * cin;
        float acc = 0.0f;
        for (int ci = 0; ci < cin; ++ci) acc = fmaf(load_f32(wr + ci), load_f32(xr + ci), acc);
        if (bias) acc += bias[co];
        store_f32(y + e, acc);
    }
}

// Row form for C_in in {8, 16, 32, 64}: one thread per row holds the row's
// C_in inputs in registers (loaded as 16-byte pieces), the weights and bias
// sit in LDS as fp32 (read as broadcasts: every lane of a wave reads the same
// weight), and the outputs go out 8 at a time as 16-byte stores when C_out is
// a multiple of 8, else one value at a time.
template <typename T, int CIN>
__global__ __launch_bounds__(kThreads) void pointwise_rows_kernel(const T *__restrict__ x, const T *__restrict__ w,
                                                                  const float *__restrict__ bias,
                                                                  T *__restrict__ y, int64_t rows, int cout) {
    __shared__ float ws[64 * CIN];
    __shared__ float bs[64];
    for (int i = threadIdx.x; i < cout * CIN; i += kThreads) ws[i] = load_f32(w + i);
    for (int i = threadIdx.x; i < cout; i += kThreads) bs[i] = bias ? bias[i] : 0.0f;
    __syncthreads();
    constexpr int EPV = 16 / (int)sizeof(T);   // elements per 16-byte piece
    for (int64_t r = blockIdx.x * (int64_t)kThreads + threadIdx.x; r < rows;
         r += (int64_t)gridDim.x * kThreads) {
        float xv[CIN];
#pragma unroll
        for (int k = 0; k < CIN; k += EPV) {
            const u32x4 d = *reinterpret_cast<const u32x4 *>(x + r * CIN + k);
            const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                if constexpr (sizeof(T) == 2)
                    xv[k + e] = bf16_bits_to_f32(e % 2 ? wd[e / 2] >> 16 : wd[e / 2] & 0xffffu);
                else
                    xv[k + e] = __uint_as_float(wd[e]);
            }
        }
        if (cout % 8 == 0) {
            for (int c0 = 0; c0 < cout; c0 += 8) {
                float o[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    float acc = 0.0f;
#pragma unroll
                    for (int ci = 0; ci < CIN; ++ci) acc = fmaf(ws[(c0 + q) * CIN + ci], xv[ci], acc);
                    o[q] = acc + bs[c0 + q];
                }
                T *yp = y + r * cout + c0;
                if constexpr (sizeof(T) == 2) {
                    u32x4 d;
                    d.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
                    d.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
                    d.z = f32_to_bf16_bits(o[4]) | (f32_to_bf16_bits(o[5]) << 16);
                    d.w = f32_to_bf16_bits(o[6]) | (f32_to_bf16_bits(o[7]) << 16);
                    *reinterpret_cast<u32x4 *>(yp) = d;
                } else {
#pragma unroll
                    for (int q = 0; q < 8; q += 4)
                        *reinterpret_cast<u32x4 *>(yp + q) =
                            u32x4{__float_as_uint(o[q]), __float_as_uint(o[q + 1]),
                                  __float_as_uint(o[q + 2]), __float_as_uint(o[q + 3])};
                }
            }
        } else {
            for (int co = 0; co < cout; ++co) {
                float acc = 0.0f;
#pragma unroll
                for (int ci = 0; ci < CIN; ++ci) acc = fmaf(ws[co * CIN + ci], xv[ci], acc);
                store_f32(y + r * cout + co, acc + bs[co]);
            }
        }
    }
}

template <typename T>
hipError_t launch_rows(const T *x, const T *w, const float *bias, T *y, int64_t rows, int cin, int cout,
                       hipStream_t s) {
    int64_t blocks = (rows + kThreads - 1) / kThreads;
    if (blocks > kGridCap) blocks = kGridCap;
    const dim3 g((unsigned)blocks), b(kThreads);
    switch (cin) {
        case 8: pointwise_rows_kernel<T, 8><<<g, b, 0, s>>>(x, w, bias, y, rows, cout); break;
        case 16: pointwise_rows_kernel<T, 16><<<g, b, 0, s>>>(x, w, bias, y, rows, cout); break;
        case 32: pointwise_rows_kernel<T, 32><<<g, b, 0, s>>>(x, w, bias, y, rows, cout); break;
        case 64: pointwise_rows_kernel<T, 64><<<g, b, 0, s>>>(x, w, bias, y, rows, cout); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pointwise_conv(const void *x, const void *w, const float *bias, void *y,
                                 int64_t rows, int cin, int cout, bool bf16, hipStream_t s) {
    const int64_t total = rows * cout;
    if (total == 0) return hipSuccess;
    if (cin == 8 || cin == 16 || cin == 32 || cin == 64) {
        if (bf16)
            return launch_rows(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w), bias,
                               static_cast<uint16_t *>(y), rows, cin, cout, s);
        return launch_rows(static_cast<const float *>(x), static_cast<const float *>(w), bias,
                           static_cast<float *>(y), rows, cin, cout, s);
    }
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > kGridCap) blocks = kGridCap;
    if (bf16)
        pointwise_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
            static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w), bias,
            static_cast<uint16_t *>(y), rows, cin, cout);
    else
        pointwise_kernel<float><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
            static_cast<const float *>(x), static_cast<const float *>(w), bias,
            static_cast<float *>(y), rows, cin, cout);
    return hipGetLastError();
}

}  // namespace wanvae
