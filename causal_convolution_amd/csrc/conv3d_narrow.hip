// Causal 3x3x3 conv with very few output channels (C_out <= 3), bf16: the
// decoder's conv_out, 96 -> 3 at the output resolution ("Sharding of WAN 2.2
// VAE", decoder module tree).  Same definition as the general bf16 conv
// ("Closing the gap: Wan 2.2 14B VAE decoder", section 2: causal T pad of 2
// frames, zero pad of 1 in H and W):
//   y[t][h][w][co] = b[co] + sum_{kt,kh,kw,ci} W[co][ci][kt][kh][kw] x[t+kt-2][h+kh-1][w+kw-1][ci]
//
// With the output channels as the MFMA M dimension, 3 of every 32 rows would do
// useful work.  Here the taps go there instead: per input position p, one GEMM
// gives every (tap, co) product at once,
//   Z[p][tap * C_out + co] = sum_ci W[co][ci][tap] x[p][ci]      (27 C_out <= 81 rows of 96)
// and each output sums 27 of them from its neighbours:
//   y[t][h][w][co] = b[co] + sum_tap Z[(t+kt-2, h+kh-1, w+kw-1)][tap * C_out + co]
// (the zero-padded positions contribute nothing and are skipped).
//
// One wave per workgroup owns 8 output rows x 62 output columns of one batch
// item and a chunk of frames.  Per input frame it walks the 10 input rows the
// tile reads; per row it computes Z for 64 input columns (two 32-position MFMA
// tiles, v_mfma_f32_32x32x16_bf16: A = the (tap, co) weight rows, held in
// registers all along; B = 16 input channels of 32 positions, read straight
// from memory, the next row's requested before the current row's tap sums),
// writes Z to LDS, and every lane (one output column) adds the 3 horizontally
// adjacent products of each (kt, kh, co) into its accumulators.  Accumulators are kept for the 3 output frames an input frame
// feeds (t', t'+1, t'+2), rotated after each input frame, when frame t' is
// complete and stored; so each input frame's Z is computed once.  A chunk of
// frames starts 2 frames early (from the cache, or skipped before frame 0) to
// rebuild its accumulators.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 8;               // output rows per tile
constexpr int kCols = 62;              // output columns per tile (64 input columns)
constexpr int kChunk = 27;             // frames per work item
constexpr int kMT = 3;                 // 32-row MFMA tiles over the 27 C_out (tap, co) rows
constexpr int kZS = 64;                // LDS row stride of Z (transposed: [row][position]) in floats

template <int KS, int COUT>
__global__ __launch_bounds__(64) void conv3d_narrow_kernel(const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ cache,
                                                           const uint16_t *__restrict__ wp,
                                                           const float *__restrict__ bias,
                                                           uint16_t *__restrict__ y, int T, int H, int W,
                                                           int tiles_h, int tiles_w, int chunks) {
    constexpr int CIN = 16 * KS;
    __shared__ __attribute__((aligned(16))) float zl[96 * kZS];
    const int lane = threadIdx.x;
    const int l32 = lane & 31, g = lane >> 5;

    int64_t item = blockIdx.x;
    const int chunk = (int)(item % chunks);
    item /= chunks;
    const int w0 = (int)(item % tiles_w) * kCols;
    item /= tiles_w;
    const int h0 = (int)(item % tiles_h) * kRows;
    const int64_t n = item / tiles_h;
    const int t_begin = chunk * kChunk;
    const int t_end = t_begin + kChunk < T ? t_begin + kChunk : T;

    // ---- weight fragments (A operand): row r = 32 m + l32 is (tap, co) =
    // (r / COUT, r % COUT), k = 16 s + 8 g .. +7; from the packed layout
    // [kt][CIN/16][kh kw][32][16] (C_out padded to 32)
    bf16x8 wa[kMT][KS];
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
        const int r = 32 * m + l32;
        const int tap = r / COUT, co = r % COUT;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (tap < 27) {
                const int kt = tap / 9, khw = tap % 9;
                v = *reinterpret_cast<const u32x4 *>(wp + ((((int64_t)kt * KS + s) * 9 + khw) * 32 + co) * 16 + 8 * g);
            }
            wa[m][s] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // accumulators of output column w0 + lane: acc[f][row][co] for output
    // frames t', t' + 1, t' + 2 of the current input frame t'
    float acc[3][kRows][COUT];
#pragma unroll
    for (int f = 0; f < 3; ++f)
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int c = 0; c < COUT; ++c) acc[f][r][c] = 0.0f;
    float bv[COUT];
#pragma unroll
    for (int c = 0; c < COUT; ++c) bv[c] = bias ? bias[c] : 0.0f;

    const int64_t HW = (int64_t)H * W;
    for (int tp = t_begin - 2; tp < t_end; ++tp) {
        // input frame tp: x, or the cache for tp < 0 (skipped without one)
        const uint16_t *src = nullptr;
        if (tp >= 0)
            src = x + ((n * T + tp) * HW) * CIN;
        else if (cache)
            src = cache + ((n * 2 + (tp + 2)) * HW) * CIN;
        if (src != nullptr) {
            // Row ir: its inputs are requested first, then the tap sums of
            // row ir - 1 run (from LDS) while they load, then the MFMAs turn
            // them into Z of row ir.
            u32x4 bfr[2][KS];
            auto load_row = [&](int h) __attribute__((always_inline)) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int wc = w0 - 1 + 32 * nt + l32;
                    const bool inside = wc >= 0 && wc < W;
                    const uint16_t *px = src + ((int64_t)h * W + (inside ? wc : 0)) * CIN + 8 * g;
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        bfr[nt][s] = inside ? *reinterpret_cast<const u32x4 *>(px + 16 * s) : u32x4{0u, 0u, 0u, 0u};
                }
            };
            // Z is stored transposed, zl[row][position]: the tap sums read 64
            // consecutive floats per instruction
            auto compute_row = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    floatx16 z[kMT];
#pragma unroll
                    for (int m = 0; m < kMT; ++m)
#pragma unroll
                        for (int e = 0; e < 16; ++e) z[m][e] = 0.0f;
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const bf16x8 b = __builtin_bit_cast(bf16x8, bfr[nt][s]);
#pragma unroll
                        for (int m = 0; m < kMT; ++m)
                            z[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[m][s], b, z[m], 0, 0, 0);
                    }
                    // lane holds rows 32 m + 8 jj + 4 g + i of position 32 nt + l32
                    float *zp = zl + 32 * nt + l32;
#pragma unroll
                    for (int m = 0; m < kMT; ++m)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int r = 32 * m + 8 * (e >> 2) + 4 * g + (e & 3);
                            if (32 * m + 8 * (e >> 2) + (e & 3) < 27 * COUT) zp[r * kZS] = z[m][e];
                        }
                }
            };
            // output row ir - kh gets taps (kt, kh, kw) from the input columns lane + kw
            auto tap_sums = [&](int ir) __attribute__((always_inline)) {
                if (lane < kCols) {
#pragma unroll
                    for (int kh = 0; kh < 3; ++kh) {
                        const int ro = ir - kh;
                        if (ro < 0 || ro >= kRows) continue;
#pragma unroll
                        for (int kt = 0; kt < 3; ++kt)
#pragma unroll
                            for (int c = 0; c < COUT; ++c) {
                                float v = 0.0f;
#pragma unroll
                                for (int kw = 0; kw < 3; ++kw)
                                    v += zl[(((kt * 3 + kh) * 3 + kw) * COUT + c) * kZS + lane + kw];
                                acc[2 - kt][ro][c] += v;
                            }
                    }
                }
            };
            bool prev = false;   // row ir - 1 has a Z in LDS
#pragma unroll
            for (int ir = 0; ir < kRows + 2; ++ir) {
                const int h = h0 - 1 + ir;
                const bool valid = h >= 0 && h < H;
                if (valid) load_row(h);
                if (prev) tap_sums(ir - 1);
                // (one wave: its LDS accesses are served in order; the fences
                // keep the compiler from moving them across each other)
                asm volatile("" ::: "memory");
                if (valid) compute_row();
                asm volatile("" ::: "memory");
                prev = valid;
            }
            if (prev) tap_sums(kRows + 1);
            asm volatile("" ::: "memory");
        }
        // output frame tp is complete
        if (tp >= t_begin) {
            const int wc = w0 + lane;
            if (lane < kCols && wc < W) {
#pragma unroll
                for (int r = 0; r < kRows; ++r) {
                    const int h = h0 + r;
                    if (h < H) {
                        uint16_t *py = y + (((n * T + tp) * H + h) * (int64_t)W + wc) * COUT;
#pragma unroll
                        for (int c = 0; c < COUT; ++c) py[c] = (uint16_t)f32_to_bf16_bits(acc[0][r][c] + bv[c]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int c = 0; c < COUT; ++c) {
                acc[0][r][c] = acc[1][r][c];
                acc[1][r][c] = acc[2][r][c];
                acc[2][r][c] = 0.0f;
            }
    }
}

template <int KS, int COUT>
hipError_t launch_ks(const ConvLaunch &c, hipStream_t s) {
    const int tiles_h = (int)((c.h + kRows - 1) / kRows), tiles_w = (int)((c.w_ + kCols - 1) / kCols);
    const int chunks = (int)((c.t + kChunk - 1) / kChunk);
    const int64_t items = c.n * tiles_h * tiles_w * chunks;
    if (items == 0) return hipSuccess;
    conv3d_narrow_kernel<KS, COUT><<<dim3((unsigned)items), dim3(64), 0, s>>>(
        static_cast<const uint16_t *>(c.x), static_cast<const uint16_t *>(c.cache),
        static_cast<const uint16_t *>(c.w), c.bias, static_cast<uint16_t *>(c.y), (int)c.t, (int)c.h, (int)c.w_,
        tiles_h, tiles_w, chunks);
    return hipGetLastError();
}

template <int COUT>
hipError_t launch_cout(const ConvLaunch &c, hipStream_t s) {
    switch (c.cin / 16) {
        case 1: return launch_ks<1, COUT>(c, s);
        case 2: return launch_ks<2, COUT>(c, s);
        case 3: return launch_ks<3, COUT>(c, s);
        case 4: return launch_ks<4, COUT>(c, s);
        case 5: return launch_ks<5, COUT>(c, s);
        case 6: return launch_ks<6, COUT>(c, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool conv3d_narrow_supported(const ConvLaunch &c) {
    return c.cout >= 1 && c.cout <= 3 && c.cin >= 16 && c.cin <= 96 && c.cin % 16 == 0 && !c.x_sliced &&
           !c.gemm && !c.up2 && c.res == nullptr && c.wsc == nullptr;
}

hipError_t launch_conv3d_narrow(const ConvLaunch &c, hipStream_t s) {
    if (!conv3d_narrow_supported(c)) return hipErrorInvalidValue;
    switch (c.cout) {
        case 1: return launch_cout<1>(c, s);
        case 2: return launch_cout<2>(c, s);
        case 3: return launch_cout<3>(c, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wanvae
