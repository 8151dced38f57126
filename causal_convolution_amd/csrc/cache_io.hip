// The stream caches' frames between the library's conv-input layout and
// channels-last.  A bf16 cache holds each of its frames as 16-channel slices,
// [C/16][h][w][16] (the layout the MFMA conv reads); callers that seed a
// stream from real frames, or save and restore one, see them channels-last,
// [h][w][C].  A pure permutation of 16-byte pieces (8 channels): bit-exact
// either way.
#include "internal.h"

namespace wanvae {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// piece i of the channels-last tensor: frame f, position q, slice k, half h
// (i = ((f * hw + q) * (C / 16) + k) * 2 + h); TO_SLICED copies it into the
// sliced tensor, else the other way
template <bool TO_SLICED>
__global__ __launch_bounds__(256) void cache_layout_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                           int64_t frames, int64_t hw, int ks) {
    const int64_t total = frames * hw * ks * 2;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int h = (int)(i & 1);
        const int64_t r = i >> 1;
        const int k = (int)(r % ks);
        const int64_t fq = r / ks;
        const int64_t q = fq % hw, f = fq / hw;
        const int64_t sliced = ((f * ks + k) * hw + q) * 2 + h;
        if constexpr (TO_SLICED)
            dst[sliced] = src[i];
        else
            dst[i] = src[sliced];
    }
}

}  // namespace

hipError_t launch_cache_layout(const void *src, void *dst, int64_t frames, int64_t hw, int C, bool to_sliced,
                               hipStream_t s) {
    const int64_t total = frames * hw * (C / 16) * 2;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (to_sliced)
        cache_layout_kernel<true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), frames, hw, C / 16);
    else
        cache_layout_kernel<false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), frames, hw, C / 16);
    return hipGetLastError();
}

}  // namespace wanvae
