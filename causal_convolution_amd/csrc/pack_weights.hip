// Conv weight packing: from the PyTorch Conv3d layout [C_out][C_in][3][3][3]
// (the weight of "Sharding of WAN 2.2 VAE", Available Sharding Dimensions)
// into the layout each conv kernel streams.
//
//   fp32: [C_out][kt][kh][kw][C_in]        (the direct kernel walks C_in innermost)
//   bf16: [kt][C_in/16][kh][kw][C_out_p][16], C_out_p = C_out rounded up to 32
//         (the MFMA tile's channel block), zero weights in the padding
//
// A 2D 3x3 weight [C_out][C_in][3][3] (the decoder upsampler's conv) packs
// the same way with one temporal tap: [C_in/16][kh][kw][C_out_p][16].  For
// the upsampler conv by output phase (C_out a multiple of 96) it packs instead
// as [C_in/16][phase][a][b][C_out_p][16]: after nearest x2 upsampling, output
// row 2i + py reads input rows i + py - 1 + a (a = 0, 1) only, row tap a
// gathering the kernel rows dy (-1, 0, +1) that land on that input row:
// {-1} and {0, +1} for py = 0, {-1, 0} and {+1} for py = 1; columns the same.
// Each merged weight is the fp32 sum of its (up to 4) taps, rounded to bf16
// once.
//
// The bf16 layout follows the MFMA conv's K loop: one stage consumes temporal
// tap kt and a 16-channel slice of C_in for all 9 (kh, kw) taps, so a stage's
// weights for one tap are C_out x 32 bytes in one contiguous run (whole
// 128-byte cache lines) instead of 32-byte pieces C_in * 54 bytes apart.
// One thread per packed element; the gather is read once per call, at set-up.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

template <typename T>
__global__ void pack_f32_kernel(const T *__restrict__ w, T *__restrict__ out, int cin, int cout,
                                int64_t total) {
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        // o = ((co * 27) + tap) * cin + ci
        const int ci = (int)(o % cin);
        const int64_t r = o / cin;
        const int tap = (int)(r % 27);
        const int co = (int)(r / 27);
        out[o] = w[((int64_t)co * cin + ci) * 27 + tap];
    }
}

// kd: temporal taps of the source weight (3, or 1 for a 2D weight)
__global__ void pack_bf16_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ out, int cin,
                                 int cout, int cout_p, int kd, int64_t total) {
    const int slices = cin / 16;
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        // o = ((((kt * slices + cc) * 9 + khw) * cout_p + co) * 16 + c16
        const int c16 = (int)(o % 16);
        int64_t r = o / 16;
        const int co = (int)(r % cout_p);
        r /= cout_p;
        const int khw = (int)(r % 9);
        r /= 9;
        const int cc = (int)(r % slices);
        const int kt = (int)(r / slices);
        const int ci = cc * 16 + c16;
        // output channels past cout are padding: zero weights
        out[o] = co < cout ? w[(((int64_t)co * cin + ci) * kd + kt) * 9 + khw] : (uint16_t)0;
    }
}

// kernel taps (0..2 for dy = -1..+1) that output phase p's tap t gathers:
// lo .. hi
__device__ inline void phase_taps(int p, int t, int &lo, int &hi) {
    lo = p == 0 ? (t == 0 ? 0 : 1) : (t == 0 ? 0 : 2);
    hi = p == 0 ? (t == 0 ? 0 : 2) : (t == 0 ? 1 : 2);
}

__global__ void pack_phase_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ out, int cin, int cout,
                                  int cout_p, int64_t total) {
    const int slices = cin / 16;
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        // o = ((((cc * 4 + ph) * 4 + tap) * cout_p + co) * 16 + c16
        const int c16 = (int)(o % 16);
        int64_t r = o / 16;
        const int co = (int)(r % cout_p);
        r /= cout_p;
        const int tap = (int)(r % 4);
        r /= 4;
        const int ph = (int)(r % 4);
        const int cc = (int)(r / 4);
        if (cc >= slices || co >= cout) {
            out[o] = 0;
            continue;
        }
        const int ci = cc * 16 + c16;
        int y0, y1, x0, x1;
        phase_taps(ph >> 1, tap >> 1, y0, y1);
        phase_taps(ph & 1, tap & 1, x0, x1);
        float sum = 0.0f;
        for (int ky = y0; ky <= y1; ++ky)
            for (int kx = x0; kx <= x1; ++kx)
                sum += bf16_bits_to_f32(w[(((int64_t)co * cin + ci) * 3 + ky) * 3 + kx]);
        out[o] = (uint16_t)f32_to_bf16_bits(sum);
    }
}

}  // namespace

int64_t packed_conv3d_weight_elems(int cin, int cout, bool bf16) {
    return (int64_t)27 * cin * (bf16 ? (cout + 31) / 32 * 32 : cout);
}

hipError_t launch_pack_conv3d_weights(const void *w, void *out, int cin, int cout, bool bf16,
                                      hipStream_t s) {
    const int64_t total = packed_conv3d_weight_elems(cin, cout, bf16);
    if (total == 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
    if (bf16)
        pack_bf16_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t *>(w),
                                              static_cast<uint16_t *>(out), cin, cout,
                                              (cout + 31) / 32 * 32, 3, total);
    else
        pack_f32_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float *>(w),
                                                    static_cast<float *>(out), cin, cout, total);
    return hipGetLastError();
}

int64_t packed_conv2d_weight_elems(int cin, int cout) {
    return (int64_t)(upsample_by_phase(cout) ? 16 : 9) * cin * ((cout + 31) / 32 * 32);
}

hipError_t launch_pack_conv2d_weights(const void *w, void *out, int cin, int cout, hipStream_t s) {
    const int64_t total = packed_conv2d_weight_elems(cin, cout);
    if (total == 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
    if (upsample_by_phase(cout))
        pack_phase_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t *>(w), static_cast<uint16_t *>(out), cin,
                                               cout, (cout + 31) / 32 * 32, total);
    else
        pack_bf16_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t *>(w), static_cast<uint16_t *>(out), cin,
                                              cout, (cout + 31) / 32 * 32, 1, total);
    return hipGetLastError();
}

}  // namespace wanvae
