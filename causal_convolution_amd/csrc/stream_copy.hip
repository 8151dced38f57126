// A plain streaming copy: the attainable HBM rate for the library's
// bandwidth-bound kernels (the fused RMS_norm + SiLU reads x once and writes
// y once, exactly what a copy of the same size does).
//
// Each lane moves 16-byte pieces, U of them in flight per pass, with
// nontemporal loads and stores; consecutive lanes take consecutive pieces, so
// every instruction of a wave covers 1 KB of whole cache lines.  The grid
// strides over the buffer, a few workgroups per compute unit, so the launch
// does not depend on the size.
#include "internal.h"

namespace wanvae {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int U>
__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const u32x4 *__restrict__ src,
                                                               u32x4 *__restrict__ dst, int64_t n16) {
    const int64_t step = (int64_t)gridDim.x * kThreads * U;
    for (int64_t i = (int64_t)blockIdx.x * kThreads * U + threadIdx.x; i < n16; i += step) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = i + (int64_t)u * kThreads;
            v[u] = k < n16 ? __builtin_nontemporal_load(src + k) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = i + (int64_t)u * kThreads;
            if (k < n16) __builtin_nontemporal_store(v[u], dst + k);
        }
    }
}

template <int U>
hipError_t launch_u(const void *src, void *dst, int64_t n16, int blocks_per_cu, hipStream_t s) {
    int ncu = 0;
    const hipError_t e = device_cu_count(&ncu);
    if (e != hipSuccess) return e;
    int64_t blocks = (n16 + (int64_t)kThreads * U - 1) / ((int64_t)kThreads * U);
    const int64_t cap = (int64_t)ncu * blocks_per_cu;
    if (blocks > cap) blocks = cap;
    stream_copy_kernel<U><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n16);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, int unroll, int blocks_per_cu,
                              hipStream_t s) {
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    switch (unroll) {
        case 1: return launch_u<1>(src, dst, n16, blocks_per_cu, s);
        case 2: return launch_u<2>(src, dst, n16, blocks_per_cu, s);
        case 4: return launch_u<4>(src, dst, n16, blocks_per_cu, s);
        case 8: return launch_u<8>(src, dst, n16, blocks_per_cu, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wanvae
