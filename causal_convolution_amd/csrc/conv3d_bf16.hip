// Causal 3x3x3 conv as an implicit GEMM on CDNA4 bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// What it computes ("Sharding of WAN 2.2 VAE", Available Sharding Dimensions;
// "Closing the gap: Wan 2.2 14B VAE decoder", sections 2 and 6):
//   y[p, co] = bias[co] + sum_{kt,kh,kw,ci} w[co][kt][kh][kw][ci] * Z[t+kt-2, h+kh-1, w+kw-1, ci]
//              (+ the shortcut: x[p, co], or sum_ci w_sc[co][ci] * x[p, ci] + b_sc[co])
// with Z = 0 outside the image in H and W, and frames -2, -1 taken from the
// feat_cache when one is given (else the causal zero pad).
//
// GEMM view: M = output channels (MFMA A operand = weights), N = output
// positions (MFMA B operand = input), K = 27 taps x C_in (+ C_res for the
// fused 1x1x1 shortcut).  Both operands are K-contiguous in HBM (weights
// [co][tap][ci], activations [pos][ci]), which is exactly the per-lane layout
// the MFMA wants, so no operand is transposed anywhere.
//
// Tiling (one workgroup): one frame t, HB output rows x 32 output columns, NB
// output channels.  Waves are arranged WM (rows) x WN (channels); each wave
// holds FM x FN 32x32 accumulator tiles.
//
// K loop in stages.  One stage = (kt, kh, 32-channel slice):
//   A tile (LDS): HB rows x 34 columns (32 + the 1-pixel W halo) x 32 channels
//                 of input frame t+kt-2, rows shifted by kh-1; pad positions are
//                 written as zeros, so the padding costs no branches in the MFMA
//                 loop and the 3 kw taps reuse the same tile.
//   B tile (LDS): NB channels x 3 taps (kw) x 32 channels of the weights.
// Stages are double-buffered through registers: the global loads of stage
// s+1 are issued before the MFMAs of stage s and written to the other LDS
// buffer after them, one barrier per stage.  LDS rows are padded from 64 to
// 80 bytes so the 16-byte per-lane operand reads of 8 (or 16) consecutive
// lanes fall in distinct banks.
//
// Causal pad: for a frame t < 2 without a cache, the stages whose source
// frame is before 0 would only add exact zeros and are skipped (uniform per
// workgroup).  With a cache they read the cached frames instead.
//
// Epilogue: each lane owns one output position and 4 consecutive output
// channels per accumulator quad; bias, then the identity residual or the
// 1x1x1 shortcut bias, are added in fp32 and the result is rounded once to
// bf16 and written as 8-byte stores.  The 1x1x1 shortcut GEMM itself runs as
// extra K stages (C_res / 32 of them) of the same accumulators: its A tile is
// x at the output positions and its B tile the shortcut weight.
//
// Workgroup order: tiles are numbered output-channel-block slowest, then
// (batch, frame), then row block, then column block, and the dispatch index is
// remapped so that each of the 8 XCDs walks a contiguous range of tiles: the
// XCD's L2 then serves one weight slice and neighbouring input rows.
#include "internal.h"

namespace wanvae {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kKC = 32;           // input channels per stage
constexpr int kPS = kKC + 8;      // LDS position stride in bf16 elements (80 bytes)
constexpr int kWB = 32;           // output columns per tile (one MFMA N block)
constexpr int kAW = kWB + 2;      // A tile columns including the W halo
constexpr int kXCD = 8;           // MI355X: 8 XCDs, workgroups dispatched round-robin

enum Epilogue { EPI_BIAS = 0, EPI_IDENTITY = 1, EPI_SHORTCUT = 2 };

struct Args {
    const uint16_t *x;      // conv input [n][t][h][w][cin]
    const uint16_t *cache;  // [n][2][h][w][cin] or null
    const uint16_t *w;      // [cout][27][cin]
    const float *bias;      // [cout] or null
    const uint16_t *res;    // [n][t][h][w][cres] or null
    const uint16_t *wsc;    // [cout][cres] or null
    const float *bsc;       // [cout] or null
    uint16_t *y;            // [n][t][h][w][cout]
    int64_t N, T, H, W;
    int cin, cout, cres;
    int tiles_w, tiles_h;
};

__device__ inline uint32_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);  // round to nearest even
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b));
}

__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

template <int WM, int WN, int FM, int FN>
struct Tile {
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int HB = WM * FM;                      // output rows
    static constexpr int NB = WN * FN * 32;                 // output channels
    static constexpr int A_POS = HB * kAW;                  // positions in the A tile
    static constexpr int A_ELEMS = A_POS * kPS;             // bf16 elements per A buffer
    static constexpr int B_ELEMS = 3 * NB * kPS;            // bf16 elements per B buffer
    static constexpr int A_CHUNKS = A_POS * (kKC / 8);      // 16-byte chunks per stage
    static constexpr int B_CHUNKS = 3 * NB * (kKC / 8);
    static constexpr int A_PER_T = (A_CHUNKS + kThreads - 1) / kThreads;
    static constexpr int B_PER_T = (B_CHUNKS + kThreads - 1) / kThreads;
    static constexpr int LDS_BYTES = 2 * (A_ELEMS + B_ELEMS) * 2;
    static_assert(LDS_BYTES <= 160 * 1024, "tile does not fit the 160 KB LDS");
};

template <int WM, int WN, int FM, int FN, int EPI>
__global__ __launch_bounds__(WM *WN * 64) void conv3d_bf16_kernel(Args a) {
    using TL = Tile<WM, WN, FM, FN>;
    constexpr int NT = TL::kThreads;
    constexpr int HB = TL::HB;
    constexpr int NB = TL::NB;

    __shared__ __attribute__((aligned(16))) uint16_t smA[2][TL::A_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t smB[2][TL::B_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;

    // ---- XCD-aware tile index: XCD k runs a contiguous range of tiles
    const int64_t nwg = gridDim.x;
    const int64_t bid = blockIdx.x;
    const int64_t q = nwg / kXCD, rmd = nwg % kXCD;
    const int64_t xcd = bid % kXCD, loc = bid / kXCD;
    int64_t tile = xcd < rmd ? xcd * (q + 1) + loc : rmd * (q + 1) + (xcd - rmd) * q + loc;

    const int wt = (int)(tile % a.tiles_w);
    tile /= a.tiles_w;
    const int ht = (int)(tile % a.tiles_h);
    tile /= a.tiles_h;
    const int64_t nt_idx = tile % (a.N * a.T);
    const int ntile = (int)(tile / (a.N * a.T));
    const int64_t tq = nt_idx % a.T;
    const int64_t nq = nt_idx / a.T;
    const int h0 = ht * HB;
    const int w0 = wt * kWB;
    const int n0 = ntile * NB;
    const int H = (int)a.H, W = (int)a.W;

    // ---- stage list: conv stages (kt from kt_begin, kh, channel slice), then shortcut stages
    const int ck = a.cin / kKC;
    const int kt_begin = (a.cache != nullptr || tq >= 2) ? 0 : (int)(2 - tq);
    const int s_conv = (3 - kt_begin) * 3 * ck;
    const int s_total = s_conv + (EPI == EPI_SHORTCUT ? a.cres / kKC : 0);
    const int64_t HW = (int64_t)H * W;

    uint4 ra[TL::A_PER_T];
    uint4 rb[TL::B_PER_T];

    auto load_stage = [&](int s) {
        const uint16_t *abase;
        int cstride, dh, ntaps, wrow, tapstride;
        const uint16_t *wbase;
        if (s < s_conv) {
            const int kt = kt_begin + s / (3 * ck);
            const int kh = (s / ck) % 3;
            const int cc = s % ck;
            const int64_t ts = tq + kt - 2;
            abase = ts >= 0 ? a.x + ((nq * a.T + ts) * HW) * a.cin
                            : a.cache + ((nq * 2 + (ts + 2)) * HW) * a.cin;
            abase += cc * kKC;
            cstride = a.cin;
            dh = kh - 1;
            ntaps = 3;
            wrow = 27 * a.cin;
            tapstride = a.cin;
            wbase = a.w + ((int64_t)n0 * 27 + kt * 9 + kh * 3) * a.cin + cc * kKC;
        } else {
            const int cc = s - s_conv;
            abase = a.res + ((nq * a.T + tq) * HW) * a.cres + cc * kKC;
            cstride = a.cres;
            dh = 0;
            ntaps = 1;
            wrow = a.cres;
            tapstride = 0;
            wbase = a.wsc + (int64_t)n0 * a.cres + cc * kKC;
        }
#pragma unroll
        for (int i = 0; i < TL::A_PER_T; ++i) {
            const int idx = tid + i * NT;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (idx < TL::A_CHUNKS) {
                const int pos = idx >> 2, qd = idx & 3;
                const int r = pos / kAW, c = pos % kAW;
                const int hh = h0 + r + dh, ww = w0 + c - 1;
                if (hh >= 0 && hh < H && ww >= 0 && ww < W)
                    v = *reinterpret_cast<const uint4 *>(abase + ((int64_t)hh * W + ww) * cstride +
                                                         qd * 8);
            }
            ra[i] = v;
        }
#pragma unroll
        for (int i = 0; i < TL::B_PER_T; ++i) {
            const int idx = tid + i * NT;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (idx < ntaps * NB * 4) {
                const int tap = idx / (NB * 4), rem = idx % (NB * 4);
                const int nl = rem >> 2, qd = rem & 3;
                v = *reinterpret_cast<const uint4 *>(wbase + (int64_t)nl * wrow + tap * tapstride +
                                                     qd * 8);
            }
            rb[i] = v;
        }
    };

    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < TL::A_PER_T; ++i) {
            const int idx = tid + i * NT;
            if (idx < TL::A_CHUNKS) {
                const int pos = idx >> 2, qd = idx & 3;
                *reinterpret_cast<uint4 *>(&smA[buf][pos * kPS + qd * 8]) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < TL::B_PER_T; ++i) {
            const int idx = tid + i * NT;
            if (idx < TL::B_CHUNKS) {
                const int tn = idx >> 2, qd = idx & 3;  // tn = tap * NB + nl
                *reinterpret_cast<uint4 *>(&smB[buf][tn * kPS + qd * 8]) = rb[i];
            }
        }
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int l32 = lane & 31;
    const int lhi = lane >> 5;

    auto compute = [&](int buf, int ntaps) {
        for (int kw = 0; kw < ntaps; ++kw) {
            const int coloff = ntaps == 1 ? 1 : kw;
#pragma unroll
            for (int ks = 0; ks < kKC / 16; ++ks) {
                const int qd = ks * 2 + lhi;
                bf16x8 bx[FM], bw[FN];
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int row = wm * FM + fm;
                    const uint4 v = *reinterpret_cast<const uint4 *>(
                        &smA[buf][(row * kAW + l32 + coloff) * kPS + qd * 8]);
                    bx[fm] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int nl = wn * FN * 32 + fn * 32 + l32;
                    const uint4 v =
                        *reinterpret_cast<const uint4 *>(&smB[buf][(kw * NB + nl) * kPS + qd * 8]);
                    bw[fn] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[fn], bx[fm],
                                                                              acc[fm][fn], 0, 0, 0);
            }
        }
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int s = 0; s < s_total; ++s) {
        const bool more = s + 1 < s_total;
        if (more) load_stage(s + 1);
        if (s < s_conv)
            compute(s & 1, 3);
        else
            compute(s & 1, 1);
        if (more) store_stage((s + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: lane owns position (row, w0 + l32) and channels 8g + 4*lhi + [0,4)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int hh = h0 + wm * FM + fm;
        const int ww = w0 + l32;
        if (hh >= H || ww >= W) continue;
        const int64_t p = ((nq * a.T + tq) * H + hh) * (int64_t)W + ww;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int co = n0 + wn * FN * 32 + fn * 32 + 8 * g + 4 * lhi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[fm][fn][4 * g + e];
                if (a.bias) {
                    const float4 bv = *reinterpret_cast<const float4 *>(a.bias + co);
                    v[0] += bv.x; v[1] += bv.y; v[2] += bv.z; v[3] += bv.w;
                }
                if constexpr (EPI == EPI_IDENTITY) {
                    const uint2 rv = *reinterpret_cast<const uint2 *>(a.res + p * a.cres + co);
                    v[0] += bf16_bits_to_f32(rv.x & 0xffffu);
                    v[1] += bf16_bits_to_f32(rv.x >> 16);
                    v[2] += bf16_bits_to_f32(rv.y & 0xffffu);
                    v[3] += bf16_bits_to_f32(rv.y >> 16);
                }
                if constexpr (EPI == EPI_SHORTCUT) {
                    if (a.bsc) {
                        const float4 bv = *reinterpret_cast<const float4 *>(a.bsc + co);
                        v[0] += bv.x; v[1] += bv.y; v[2] += bv.z; v[3] += bv.w;
                    }
                }
                uint2 o;
                o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                *reinterpret_cast<uint2 *>(a.y + p * a.cout + co) = o;
            }
        }
    }
}

template <int WM, int WN, int FM, int FN>
hipError_t launch_cfg(const ConvLaunch &c, hipStream_t s) {
    using TL = Tile<WM, WN, FM, FN>;
    Args a;
    a.x = static_cast<const uint16_t *>(c.x);
    a.cache = static_cast<const uint16_t *>(c.cache);
    a.w = static_cast<const uint16_t *>(c.w);
    a.bias = c.bias;
    a.res = static_cast<const uint16_t *>(c.res);
    a.wsc = static_cast<const uint16_t *>(c.wsc);
    a.bsc = c.bsc;
    a.y = static_cast<uint16_t *>(c.y);
    a.N = c.n;
    a.T = c.t;
    a.H = c.h;
    a.W = c.w_;
    a.cin = c.cin;
    a.cout = c.cout;
    a.cres = c.cres;
    a.tiles_w = (int)((c.w_ + kWB - 1) / kWB);
    a.tiles_h = (int)((c.h + TL::HB - 1) / TL::HB);
    const int64_t tiles = (int64_t)a.tiles_w * a.tiles_h * c.n * c.t * (c.cout / TL::NB);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles), block(TL::kThreads);
    if (!c.res)
        conv3d_bf16_kernel<WM, WN, FM, FN, EPI_BIAS><<<grid, block, 0, s>>>(a);
    else if (!c.wsc)
        conv3d_bf16_kernel<WM, WN, FM, FN, EPI_IDENTITY><<<grid, block, 0, s>>>(a);
    else
        conv3d_bf16_kernel<WM, WN, FM, FN, EPI_SHORTCUT><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool conv3d_bf16_supported(int cin, int cout) {
    return cin >= 32 && cin <= 1024 && cin % 32 == 0 && cout >= 32 && cout <= 1024 &&
           cout % 32 == 0;
}

// Tile choice per output-channel count: the widest channel block that divides
// C_out, 8 output rows x 32 columns per workgroup.
hipError_t launch_conv3d_bf16(const ConvLaunch &c, hipStream_t s) {
    if (c.cout % 192 == 0) return launch_cfg<2, 2, 4, 3>(c, s);   // NB = 192, 4 waves
    if (c.cout % 128 == 0) return launch_cfg<2, 2, 4, 2>(c, s);   // NB = 128, 4 waves
    if (c.cout % 96 == 0) return launch_cfg<4, 1, 2, 3>(c, s);    // NB = 96, 4 waves
    if (c.cout % 64 == 0) return launch_cfg<4, 1, 2, 2>(c, s);    // NB = 64
    return launch_cfg<4, 1, 2, 1>(c, s);                          // NB = 32
}

}  // namespace wanvae
