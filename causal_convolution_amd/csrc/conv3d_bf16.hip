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
//                 loop and the 3 kw taps reuse the same tile.  Tiles are fetched
//                 with raw buffer loads over one frame slab: a pad position gets an
//                 out-of-range offset and the hardware returns zeros for it.
//   B tile (LDS): NB channels x 3 taps (kw) x 32 channels of the weights.
// Stages are double-buffered through registers: the global loads of stage
// s+1 are issued before the MFMAs of stage s and written to the other LDS
// buffer after them, one barrier per stage.  LDS rows are padded from 64 to
// 80 bytes so the 16-byte per-lane operand reads and writes of 8 (or 16)
// consecutive lanes, which touch consecutive rows, fall in distinct banks.
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
// batch, row block, column block, and frame fastest, and the dispatch index is
// remapped so that each of the 8 XCDs walks a contiguous range of tiles: the
// workgroups resident on one XCD then share one weight slice and the input
// frames t-2..t of one spatial block through that XCD's L2.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for raw (unformatted, stride 0) buffers on gfx9-family
// GPUs; loads past num_records return zero.
constexpr int kBufFlags = 0x00020000;

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



template <int WM, int WN, int FM, int FN>
struct Tile {
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int HB = WM * FM;                      // output rows
    static constexpr int NB = WN * FN * 32;                 // output channels
    static constexpr int A_POS = HB * kAW;                  // positions in the A tile
    static constexpr int A_ELEMS = A_POS * kPS;             // bf16 elements per A buffer
    static constexpr int B_ELEMS = 3 * NB * kPS;            // bf16 elements per B buffer
    static constexpr int UPR = kThreads / 4;                // units loaded per round
    static constexpr int A_PER_T = (A_POS + UPR - 1) / UPR;  // load rounds per stage
    static constexpr int B_PER_T = (3 * NB + UPR - 1) / UPR;
    static_assert(kThreads % 32 == 0, "chunk mapping needs whole 32-lane groups");
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

    // frame fastest: consecutive tiles are the same spatial block in consecutive
    // frames, so the input frames t-2..t of neighbouring workgroups overlap in L2
    const int64_t tq = tile % a.T;
    tile /= a.T;
    const int wt = (int)(tile % a.tiles_w);
    tile /= a.tiles_w;
    const int ht = (int)(tile % a.tiles_h);
    tile /= a.tiles_h;
    const int64_t nq = tile % a.N;
    const int ntile = (int)(tile / a.N);
    const int h0 = ht * HB;
    const int w0 = wt * kWB;
    const int n0 = ntile * NB;
    const int H = (int)a.H, W = (int)a.W;
    const int64_t HW = (int64_t)H * W;

    // ---- stage list: conv stages (kt from kt_begin, kh, channel slice), then shortcut stages
    const int ck = a.cin / kKC;
    const int kt_begin = (a.cache != nullptr || tq >= 2) ? 0 : (int)(2 - tq);
    const int s_conv = (3 - kt_begin) * 3 * ck;
    const int s_total = s_conv + (EPI == EPI_SHORTCUT ? a.cres / kKC : 0);

    // ---- per-thread load descriptors, fixed for the whole K loop.
    // A tile unit = one position (r, c) of the HB x 34 halo tile; B tile unit =
    // one (kw tap, output channel) row.  Each unit holds 4 sixteen-byte quarters
    // of the 32-channel slice.  Chunk j = tid + i * NT maps to unit
    // 8 * (j >> 5) + (j & 7) and quarter (j >> 3) & 3: the 8 lanes of each LDS
    // access group write 8 different units with the same quarter, which the
    // 80-byte unit stride spreads over distinct banks, and one wavefront
    // instruction still covers 16 whole units (64 contiguous bytes each) in HBM.
    const int qd = (tid >> 3) & 3;
    const int u0 = 8 * (tid >> 5) + (tid & 7);
    constexpr int UPR = NT / 4;  // units advanced per round
    int a_pix[TL::A_PER_T];      // input pixel index (h0 + r) * W + (w0 + c - 1)
    int a_row[TL::A_PER_T];      // input row h0 + r, or a large negative value if unused
#pragma unroll
    for (int i = 0; i < TL::A_PER_T; ++i) {
        const int u = u0 + i * UPR;
        const int r = u / kAW, c = u % kAW;
        const int ww = w0 + c - 1;
        const bool ok = u < TL::A_POS && ww >= 0 && ww < W;
        a_pix[i] = (h0 + r) * W + ww;
        a_row[i] = ok ? h0 + r : -(1 << 29);
    }
    constexpr uint32_t kOOB = 0x80000000u;  // beyond every buffer: the load returns zeros
    const uint32_t wrow2 = (uint32_t)(27 * a.cin * 2), tap2 = (uint32_t)(a.cin * 2);
    uint32_t b_off[TL::B_PER_T];   // weight byte offset of the unit (stage part excluded)
    uint32_t b_sc[EPI == EPI_SHORTCUT ? TL::B_PER_T : 1];
#pragma unroll
    for (int i = 0; i < TL::B_PER_T; ++i) {
        const int u = u0 + i * UPR;
        const int tap = u / NB, nl = u % NB;
        b_off[i] = u < 3 * NB ? (uint32_t)(n0 + nl) * wrow2 + (uint32_t)tap * tap2 + qd * 16 : kOOB;
        if constexpr (EPI == EPI_SHORTCUT)
            b_sc[i] = u < NB ? (uint32_t)((n0 + nl) * a.cres * 2 + qd * 16) : kOOB;
    }
    const int lds_a0 = u0 * kPS + qd * 8;
    const int lds_b0 = u0 * kPS + qd * 8;

    u32x4 ra[TL::A_PER_T];
    u32x4 rb[TL::B_PER_T];

    // Buffer loads: a pad position (outside H or W) or an unused chunk gets an
    // out-of-range offset, for which the hardware returns zeros, so the loads
    // are branch-free.
    auto load_stage = [&](int s) {
        const uint16_t *abase;
        uint32_t aslab, cs2;
        int dh;
        if (s < s_conv) {
            const int kt = kt_begin + s / (3 * ck);
            const int kh = (s / ck) % 3;
            const int cc = s % ck;
            const int64_t ts = tq + kt - 2;
            abase = ts >= 0 ? a.x + ((nq * a.T + ts) * HW) * a.cin
                            : a.cache + ((nq * 2 + (ts + 2)) * HW) * a.cin;
            abase += cc * kKC;
            aslab = (uint32_t)(HW * a.cin * 2 - cc * kKC * 2);
            cs2 = (uint32_t)a.cin * 2;
            dh = kh - 1;
            const uint32_t woff = (uint32_t)(((kt * 9 + kh * 3) * a.cin + cc * kKC) * 2);
            const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
                (void *)a.w, (short)0, (int)((int64_t)a.cout * 27 * a.cin * 2), kBufFlags);
#pragma unroll
            for (int i = 0; i < TL::B_PER_T; ++i)
                rb[i] = __builtin_amdgcn_raw_buffer_load_b128(br, b_off[i] + woff, 0, 0);
        } else {
            const int cc = s - s_conv;
            abase = a.res + ((nq * a.T + tq) * HW) * a.cres + cc * kKC;
            aslab = (uint32_t)(HW * a.cres * 2 - cc * kKC * 2);
            cs2 = (uint32_t)a.cres * 2;
            dh = 0;
            if constexpr (EPI == EPI_SHORTCUT) {
                const uint32_t woff = (uint32_t)(cc * kKC * 2);
                const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)a.wsc, (short)0, (int)((int64_t)a.cout * a.cres * 2), kBufFlags);
#pragma unroll
                for (int i = 0; i < TL::B_PER_T; ++i)
                    rb[i] = __builtin_amdgcn_raw_buffer_load_b128(br, b_sc[i] + woff, 0, 0);
            }
        }
        const __amdgpu_buffer_rsrc_t ar =
            __builtin_amdgcn_make_buffer_rsrc((void *)abase, (short)0, (int)aslab, kBufFlags);
        const int dpix = dh * W;
#pragma unroll
        for (int i = 0; i < TL::A_PER_T; ++i) {
            const int hh = a_row[i] + dh;
            const bool ok = hh >= 0 && hh < H;
            const uint32_t off = ok ? (uint32_t)(a_pix[i] + dpix) * cs2 + qd * 16 : kOOB;
            ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
        }
    };

    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < TL::A_PER_T; ++i)
            if ((i + 1) * UPR <= TL::A_POS || u0 + i * UPR < TL::A_POS)
                *reinterpret_cast<u32x4 *>(&smA[buf][lds_a0 + i * UPR * kPS]) = ra[i];
#pragma unroll
        for (int i = 0; i < TL::B_PER_T; ++i)
            if ((i + 1) * UPR <= 3 * NB || u0 + i * UPR < 3 * NB)
                *reinterpret_cast<u32x4 *>(&smB[buf][lds_b0 + i * UPR * kPS]) = rb[i];
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

    // One stage of MFMAs: NTAPS kw taps x 2 sixteen-channel k-steps.  The
    // operand fragments of the next k-step are read from LDS while the MFMAs of
    // the current one run.
    auto compute = [&]<int NTAPS>(int buf) {
        constexpr int NSTEP = NTAPS * (kKC / 16);
        bf16x8 fx[2][FM], fw[2][FN];
        auto ldfrag = [&](int step, int slot) {
            const int kw = step / (kKC / 16), ks = step % (kKC / 16);
            const int coloff = NTAPS == 1 ? 1 : kw;
            const int qd = ks * 2 + lhi;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = wm * FM + fm;
                fx[slot][fm] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(
                                &smA[buf][(row * kAW + l32 + coloff) * kPS + qd * 8]));
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int nl = wn * FN * 32 + fn * 32 + l32;
                fw[slot][fn] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(&smB[buf][(kw * NB + nl) * kPS + qd * 8]));
            }
        };
        ldfrag(0, 0);
#pragma unroll
        for (int step = 0; step < NSTEP; ++step) {
            // the reads of step + 1 are issued before, and complete under, the
            // MFMAs of this step (sched_barrier keeps the compiler from sinking them)
            if (step + 1 < NSTEP) ldfrag(step + 1, (step + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        fw[step & 1][fn], fx[step & 1][fm], acc[fm][fn], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int s = 0; s < s_total; ++s) {
        const bool more = s + 1 < s_total;
        if (more) load_stage(s + 1);
        if constexpr (EPI == EPI_SHORTCUT) {
            if (s < s_conv)
                compute.template operator()<3>(s & 1);
            else
                compute.template operator()<1>(s & 1);
        } else {
            compute.template operator()<3>(s & 1);
        }
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

template <int WM, int WN, int FM, int FN, int EPI>
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
    conv3d_bf16_kernel<WM, WN, FM, FN, EPI><<<dim3((unsigned)tiles), dim3(TL::kThreads), 0, s>>>(a);
    return hipGetLastError();
}

// bias-only or identity-residual epilogue, chosen at run time
template <int WM, int WN, int FM, int FN>
hipError_t launch_plain(const ConvLaunch &c, hipStream_t s) {
    return c.res ? launch_cfg<WM, WN, FM, FN, EPI_IDENTITY>(c, s)
                 : launch_cfg<WM, WN, FM, FN, EPI_BIAS>(c, s);
}

}  // namespace

bool conv3d_bf16_supported(int cin, int cout) {
    return cin >= 32 && cin <= 1024 && cin % 32 == 0 && cout >= 32 && cout <= 1024 &&
           cout % 32 == 0;
}

// Tile choice, measured on MI355X over the decoder's channel counts (latent
// 384, mid 192, output 96): 8-wave workgroups (2 waves per SIMD) beat 4-wave
// ones at every shape.  The fused 1x1x1 shortcut variant keeps 4-wave tiles,
// whose register budget holds its second operand stream without spilling.
hipError_t launch_conv3d_bf16(const ConvLaunch &c, hipStream_t s) {
    if (c.res != nullptr && c.wsc != nullptr) {
        if (c.cout % 96 == 0) return launch_cfg<4, 1, 2, 3, EPI_SHORTCUT>(c, s);  // 8 rows x 96 ch
        if (c.cout % 64 == 0) return launch_cfg<4, 1, 2, 2, EPI_SHORTCUT>(c, s);  // 8 rows x 64 ch
        return launch_cfg<4, 1, 2, 1, EPI_SHORTCUT>(c, s);                        // 8 rows x 32 ch
    }
    if (c.cout % 128 == 0) return launch_plain<4, 2, 4, 2>(c, s);   // 16 rows x 128 ch
    if (c.cout % 192 == 0) return launch_plain<4, 2, 2, 3>(c, s);   // 8 rows x 192 ch
    if (c.cout % 96 == 0) return launch_plain<8, 1, 2, 3>(c, s);    // 16 rows x 96 ch
    if (c.cout % 64 == 0) return launch_plain<4, 1, 2, 2>(c, s);    // 8 rows x 64 ch
    return launch_plain<4, 1, 2, 1>(c, s);                          // 8 rows x 32 ch
}

}  // namespace wanvae
