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
//
// NORM: the decoder's tail norm_out -> SiLU -> conv_out in one pass.  The
// kernel then reads the norm's input and normalises each input position as
// its row arrives, before the MFMAs: the RMS_norm + SiLU of "Closing the gap",
// section 4 (d = max(sqrt(sum_c v_c^2), eps), u_c = v_c sqrt(C) / d gamma_c +
// beta_c, silu(u_c)), rounded to bf16 as a separate norm's output would be.
// Lane (l32, g) holds 8 of every 16 channels of its position and lane ^ 32
// the other 8, so the sum of squares takes one exchange.  Positions outside
// the frame stay 0 (the conv's zero pad applies to the norm's output), and a
// cache holds the norm's input frames, normalised on the way in like x.  The
// activation's round trip through memory (the norm writing it, the conv
// reading it back) is gone: x is read once, with the tiles' halos.
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

__device__ inline float silu(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

// the norm of NORM kernels: scale gamma (sqrt(C) applied here), shift beta
// (or null), clamp eps
struct InNorm {
    const float *gamma = nullptr, *beta = nullptr;
    float eps = 0.0f, sqrt_c = 0.0f;
};

template <int KS, int COUT, bool NORM>
__global__ __launch_bounds__(64) void conv3d_narrow_kernel(const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ cache,
                                                           const uint16_t *__restrict__ wp,
                                                           const float *__restrict__ bias,
                                                           uint16_t *__restrict__ y, int T, int H, int W,
                                                           int tiles_h, int tiles_w, int chunks, InNorm nm) {
    constexpr int CIN = 16 * KS;
    __shared__ __attribute__((aligned(16))) float zl[96 * kZS];
    // NORM: gamma * sqrt(C) of each input channel, then beta
    __shared__ __attribute__((aligned(16))) float nrm[NORM ? 2 * CIN : 4];
    const int lane = threadIdx.x;
    const int l32 = lane & 31, g = lane >> 5;
    if constexpr (NORM) {
        for (int c = lane; c < CIN; c += 64) {
            nrm[c] = nm.gamma[c] * nm.sqrt_c;
            nrm[CIN + c] = nm.beta ? nm.beta[c] : 0.0f;
        }
        __syncthreads();
    }

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
            uint32_t in_mask[2];   // all ones where the position is inside the frame
            auto load_row = [&](int h) __attribute__((always_inline)) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int wc = w0 - 1 + 32 * nt + l32;
                    const bool inside = wc >= 0 && wc < W;
                    in_mask[nt] = inside ? ~0u : 0u;
                    const uint16_t *px = src + ((int64_t)h * W + (inside ? wc : 0)) * CIN + 8 * g;
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        bfr[nt][s] = inside ? *reinterpret_cast<const u32x4 *>(px + 16 * s) : u32x4{0u, 0u, 0u, 0u};
                }
            };
            // NORM: the loaded row in place, channel 16 s + 8 g + 2 k (+1) in
            // bfr[nt][s][k]; sum of squares in that order, then lane ^ 32's
            auto normalize_row = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    float ss = 0.0f;
#pragma unroll
                    for (int s = 0; s < KS; ++s)
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float lo = bf16_bits_to_f32(bfr[nt][s][k] & 0xffffu);
                            const float hi = bf16_bits_to_f32(bfr[nt][s][k] >> 16);
                            ss = fmaf(lo, lo, ss);
                            ss = fmaf(hi, hi, ss);
                        }
                    ss += __shfl_xor(ss, 32);
                    const float inv = 1.0f / fmaxf(sqrtf(ss), nm.eps);
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const int c0 = 16 * s + 8 * g;
                        const u32x4 q = bfr[nt][s];
                        uint32_t o[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float2 gv = *reinterpret_cast<const float2 *>(nrm + c0 + 2 * k);
                            const float2 bv = *reinterpret_cast<const float2 *>(nrm + CIN + c0 + 2 * k);
                            const float lo = bf16_bits_to_f32(q[k] & 0xffffu);
                            const float hi = bf16_bits_to_f32(q[k] >> 16);
                            o[k] = pack_bf16x2(silu(fmaf(lo * inv, gv.x, bv.x)), silu(fmaf(hi * inv, gv.y, bv.y))) &
                                   in_mask[nt];
                        }
                        bfr[nt][s] = u32x4{o[0], o[1], o[2], o[3]};
                    }
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
                if constexpr (NORM)
                    if (valid) normalize_row();
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

template <int KS, int COUT, bool NORM>
hipError_t launch_ks(const ConvLaunch &c, hipStream_t s) {
    const int tiles_h = (int)((c.h + kRows - 1) / kRows), tiles_w = (int)((c.w_ + kCols - 1) / kCols);
    const int chunks = (int)((c.t + kChunk - 1) / kChunk);
    const int64_t items = c.n * tiles_h * tiles_w * chunks;
    if (items == 0) return hipSuccess;
    InNorm nm;
    if (NORM) {
        nm.gamma = c.in_norm_gamma;
        nm.beta = c.in_norm_beta;
        nm.eps = c.in_norm_eps;
        nm.sqrt_c = sqrtf((float)c.cin);
    }
    conv3d_narrow_kernel<KS, COUT, NORM><<<dim3((unsigned)items), dim3(64), 0, s>>>(
        static_cast<const uint16_t *>(c.x), static_cast<const uint16_t *>(c.cache),
        static_cast<const uint16_t *>(c.w), c.bias, static_cast<uint16_t *>(c.y), (int)c.t, (int)c.h, (int)c.w_,
        tiles_h, tiles_w, chunks, nm);
    return hipGetLastError();
}

template <int COUT, bool NORM>
hipError_t launch_cout(const ConvLaunch &c, hipStream_t s) {
    switch (c.cin / 16) {
        case 1: return launch_ks<1, COUT, NORM>(c, s);
        case 2: return launch_ks<2, COUT, NORM>(c, s);
        case 3: return launch_ks<3, COUT, NORM>(c, s);
        case 4: return launch_ks<4, COUT, NORM>(c, s);
        case 5: return launch_ks<5, COUT, NORM>(c, s);
        case 6: return launch_ks<6, COUT, NORM>(c, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool NORM>
hipError_t launch_norm(const ConvLaunch &c, hipStream_t s) {
    switch (c.cout) {
        case 1: return launch_cout<1, NORM>(c, s);
        case 2: return launch_cout<2, NORM>(c, s);
        case 3: return launch_cout<3, NORM>(c, s);
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
    if (c.in_norm_gamma != nullptr) return launch_norm<true>(c, s);
    return launch_norm<false>(c, s);
}

}  // namespace wanvae
