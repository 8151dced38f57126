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
// [co][tap][ci], activations [pos][ci]), which is the per-lane operand layout
// of the MFMA, so nothing is transposed.
//
// Workgroup tile: one frame t, HB = WM*FM output rows x 32 output columns x
// NB = WN*FN*32 output channels; wave (wm, wn) owns FM rows x FN channel blocks
// (FM*FN 32x32 fp32 accumulators).
//
// K loop in stages of (kt, 16 input channels):
//   A tile (LDS): HB+2 input rows (the H halo) x 34 columns (the W halo) x 16
//     channels of frame t+kt-2.  Every (kh, kw) tap of the stage reads it.
//   B tile (LDS): the 9 (kh, kw) taps x NB channels x 16 input channels.
// A wave walks its FM+2 input rows once per stage ("row-stationary"): for each
// row it reads the three kw-shifted operand fragments from LDS and feeds them
// to every (kh, output row) pair that uses that input row, with all 9*FN weight
// fragments held in registers for the stage.  Per MFMA that is about
// (3(FM+2) + 9 FN) / (9 FM FN) KB of LDS reads, against one fragment pair per
// MFMA when every tap re-reads its operands.
//
// A workgroup has WM*WN MFMA waves and one load wave.  The load wave moves
// every byte of the tile from L2 straight to LDS (buffer_load ... lds): each of
// its instructions fills one 1 KB block of a stage buffer, lane l writing
// bytes 16l..16l+15, so no VGPRs stage the data and no LDS-write instructions
// run.  Issuing these loads stalls the issuing wave on the LDS-DMA queue; with
// a wave of its own for them, the MFMA waves never wait on the memory pipe.
// They are raw buffer loads over one frame slab: an input position outside
// the image gets an out-of-range offset and the hardware writes zeros, so
// padding costs no branch.  Because the tile already holds the H and W halo,
// every per-lane load offset is fixed for the whole K loop; a stage only moves
// the buffer base (frame and channel slice).  Stages rotate through a ring of
// NBUF LDS buffers: stage s+NBUF-1 is requested while stage s computes; per
// stage the load wave waits once (vmcnt) and all waves meet one barrier.
//
// LDS layout: 32-byte units (16 bf16 channels of one position or one weight
// row), the two 16-byte halves swapped when bit 3 of the unit index is set.
// 16 lanes reading one half of 16 consecutive units then hit 16 distinct
// 16-byte bank groups (gfx950 serves 16 lanes x 16 bytes per LDS cycle).  A
// tile rows are padded to 40 units so a lane's swizzle bit for (row, kw) is a
// compile-time function of the row parity.
//
// Causal pad: without a cache, the stages of a frame before 0 only add exact
// zeros and are skipped (uniform per workgroup); with a cache they read it.
//
// Epilogue: each lane owns one output position and 4 consecutive output
// channels per accumulator quad; bias, then the identity residual or the
// shortcut bias, are added in fp32 and the result is rounded once to bf16
// (8-byte stores).  The 1x1x1 shortcut GEMM runs as C_res/16 extra stages of
// the same accumulators: A tile = x at the output positions, B tile = w_sc.
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
constexpr uint32_t kOOB = 0x80000000u;  // beyond every buffer: the load returns zeros

constexpr int kKC = 16;          // input channels per stage = one MFMA k-step
constexpr int kUnit = 32;        // bytes per LDS unit (16 bf16)
constexpr int kWB = 32;          // output columns per tile (one MFMA N block)
constexpr int kAW = kWB + 2;     // A tile columns including the W halo
constexpr int kAS = 40;          // A tile row stride in units (34 used)
constexpr int kXCD = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin

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
    static constexpr int NWAVE = WM * WN;                    // MFMA waves
    static constexpr int kThreads = (NWAVE + 1) * 64;        // + one load wave
    static constexpr int HB = WM * FM;                       // output rows
    static constexpr int NB = WN * FN * 32;                  // output channels
    static constexpr int AR = HB + 2;                        // A tile rows (H halo)
    static constexpr int A_BLOCKS = (AR * kAS + 31) / 32;    // 1 KB blocks = 32 units
    static constexpr int B_BLOCKS = 9 * NB / 32;
    static constexpr int BLOCKS = A_BLOCKS + B_BLOCKS;       // load instructions per stage
    static constexpr int STAGE_BYTES = BLOCKS * 1024;
    static constexpr int NBUF = 3 * STAGE_BYTES <= 160 * 1024 ? 3 : 2;  // LDS ring depth
    static_assert(NBUF * STAGE_BYTES <= 160 * 1024, "tile does not fit the 160 KB LDS");
    static_assert(BLOCKS < 64, "vmcnt holds at most 63 outstanding loads");
};

// byte offset of half `h` (0/1) of LDS unit `u`
__device__ __host__ constexpr int lds_off(int u, int h) { return u * kUnit + ((h ^ ((u >> 3) & 1)) << 4); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (stride 0, num_records bytes) for a wave-uniform base.
__device__ inline i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)), (int)bytes, kBufFlags};
}

// One wavefront-wide 16-byte-per-lane load from a buffer straight into LDS:
// lane l's 16 bytes at byte offset voff land at LDS byte address
// lds_addr + 16 * l (lds_addr wave-uniform).  Written as inline assembly so the
// compiler does not wait for these loads before unrelated LDS reads; the
// kernel orders them itself with explicit vmcnt waits and barriers.  M0 is set
// inside the same statement, immediately before its only use.
__device__ inline void lds_dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "memory");
}

__device__ inline uint32_t lds_address(const unsigned char *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

template <int WM, int WN, int FM, int FN, int EPI>
__global__ __launch_bounds__((WM *WN + 1) * 64) void conv3d_bf16_kernel(Args a) {
    using TL = Tile<WM, WN, FM, FN>;
    constexpr int NT = TL::kThreads;
    constexpr int HB = TL::HB;
    constexpr int NB = TL::NB;

    __shared__ __attribute__((aligned(1024))) unsigned char smem[TL::NBUF * TL::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // NWAVE = the load wave
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

    // ---- stage list: conv stages (kt from kt_begin, channel slice), then shortcut stages
    const int ck = a.cin / kKC;
    const int kt_begin = (a.cache != nullptr || tq >= 2) ? 0 : (int)(2 - tq);
    const int s_conv = (3 - kt_begin) * ck;
    const int s_total = s_conv + (EPI == EPI_SHORTCUT ? a.cres / kKC : 0);

    constexpr int NBUF = TL::NBUF;
    const uint32_t smem_base = lds_address(smem);

    if (wave == TL::NWAVE) {
        // ================= load wave: all global -> LDS traffic of the tile
        // Block b of a stage: lane l writes half (l & 1) ^ swizzle(u) of unit
        // u = 32 * b' + l / 2 (b' relative to the A or B region), so the lane
        // fetches that half of that unit.  Offsets are fixed for the K loop; a
        // stage only moves the buffer base (frame and channel slice).
        const uint32_t cs2 = (uint32_t)a.cin * 2;
        const uint32_t wrow2 = (uint32_t)(27 * a.cin * 2), tap2 = (uint32_t)(a.cin * 2);
        // byte offset of block b's piece for a conv stage (sc = false) or a
        // shortcut stage (sc = true: x at the output positions, w_sc as one tap)
        auto block_off = [&](int b, bool sc) -> uint32_t {
            if (b < TL::A_BLOCKS) {
                const int u = b * 32 + (lane >> 1);
                const int hf = (lane & 1) ^ ((u >> 3) & 1);
                const int r = u / kAS, c = u % kAS;
                const int hh = h0 - 1 + r, ww = w0 - 1 + c;
                const bool inside = r < TL::AR && c < kAW && hh >= 0 && hh < H && ww >= 0 && ww < W;
                if (!sc) return inside ? (uint32_t)(hh * W + ww) * cs2 + hf * 16 : kOOB;
                return inside && r >= 1 && r <= HB && c >= 1 && c <= kWB
                           ? (uint32_t)(hh * W + ww) * (uint32_t)(a.cres * 2) + hf * 16
                           : kOOB;
            }
            const int u = (b - TL::A_BLOCKS) * 32 + (lane >> 1);
            const int hf = (lane & 1) ^ ((u >> 3) & 1);
            const int tap = u / NB, nl = u % NB;
            if (!sc) return (uint32_t)(n0 + nl) * wrow2 + (uint32_t)tap * tap2 + hf * 16;
            return tap == 0 ? (uint32_t)((n0 + nl) * a.cres * 2) + hf * 16 : kOOB;
        };
        uint32_t l_off[TL::BLOCKS];   // conv-stage offsets, kept for the whole K loop
#pragma unroll
        for (int b = 0; b < TL::BLOCKS; ++b) l_off[b] = block_off(b, false);

        // request stage s into ring buffer s % NBUF (asynchronous; completion via vmcnt)
        auto issue = [&](int s) {
            i32x4 ar, br;
            const bool sc = s >= s_conv;
            if (!sc) {
                const int kt = kt_begin + s / ck;
                const int cc = s % ck;
                const int64_t ts = tq + kt - 2;
                const uint16_t *abase = (ts >= 0 ? a.x + ((nq * a.T + ts) * HW) * a.cin
                                                 : a.cache + ((nq * 2 + (ts + 2)) * HW) * a.cin) +
                                        cc * kKC;
                ar = buffer_rsrc(abase, (uint32_t)(HW * a.cin * 2 - cc * kKC * 2));
                const int wskip = (kt * 9) * a.cin + cc * kKC;   // elements before this slice
                br = buffer_rsrc(a.w + wskip, (uint32_t)((int64_t)a.cout * 27 * a.cin * 2 - wskip * 2));
            } else {
                const int cc = s - s_conv;
                ar = buffer_rsrc(a.res + ((nq * a.T + tq) * HW) * a.cres + cc * kKC,
                                 (uint32_t)(HW * a.cres * 2 - cc * kKC * 2));
                br = buffer_rsrc(a.wsc + cc * kKC,
                                 (uint32_t)((int64_t)a.cout * a.cres * 2 - cc * kKC * 2));
            }
            const uint32_t base = smem_base + (uint32_t)(s % NBUF) * TL::STAGE_BYTES;
#pragma unroll
            for (int b = 0; b < TL::BLOCKS; ++b) {
                uint32_t off = l_off[b];
                if constexpr (EPI == EPI_SHORTCUT)
                    if (sc) off = block_off(b, true);
                lds_dma16(b < TL::A_BLOCKS ? ar : br, base + b * 1024, off);
            }
        };

        // s_waitcnt immediates for "vmcnt <= BLOCKS" (one stage may stay in
        // flight) and "vmcnt = 0"; other counters left alone (gfx9 encoding:
        // vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
        constexpr int kWaitOne = (TL::BLOCKS & 15) | ((TL::BLOCKS >> 4) << 14) | (7 << 4) | (15 << 8);
        constexpr int kWaitAll = (7 << 4) | (15 << 8);
        for (int p = 0; p < NBUF - 1 && p < s_total; ++p) issue(p);
        for (int s = 0; s < s_total; ++s) {
            // stage s has landed in LDS once at most the next stage is outstanding
            if (NBUF == 3 && s + 1 < s_total)
                __builtin_amdgcn_s_waitcnt(kWaitOne);
            else
                __builtin_amdgcn_s_waitcnt(kWaitAll);
            // A plain barrier, not __syncthreads(): its release fence would wait
            // for every outstanding load, including the prefetched stage.
            __builtin_amdgcn_s_barrier();
            // the barrier also means every MFMA wave has finished stage s - 1, so
            // its buffer ((s + NBUF - 1) % NBUF) can be refilled
            if (s + NBUF - 1 < s_total) issue(s + NBUF - 1);
        }
        return;
    }

    // ================= MFMA waves
    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int l32 = lane & 31;
    const int g = lane >> 5;   // k-group: which 8-channel half of the 16-channel unit
    // B fragment (tap, fn): unit tap*NB + wn*FN*32 + fn*32 + l32; NB and 32 are
    // multiples of 16, so its swizzle bit is bit 3 of l32
    const int b_rd0 = TL::A_BLOCKS * 1024 + lds_off(wn * FN * 32 + l32, g);
    // A fragment (row wm*FM + qr, column l32 + kw): the swizzle bit is bit 3 of
    // (row * 40 + l32 + kw) = parity(row) ^ bit 3 of (l32 + kw); a_rd[par] serves
    // the rows qr with qr & 1 == par, whose parity is par ^ parity(wm * FM)
    int a_rd[2][3];
#pragma unroll
    for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int u = l32 + kw;
            const int row_par = par ^ ((wm * FM) & 1);
            a_rd[par][kw] = (wm * FM) * kAS * kUnit + u * kUnit + ((g ^ ((u >> 3) & 1) ^ row_par) << 4);
        }

    auto ldA = [&](const unsigned char *buf, int qr, int kw) {
        const int off = a_rd[qr & 1][kw] + qr * kAS * kUnit;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(buf + off));
    };
    auto ldB = [&](const unsigned char *buf, int tap, int fn) {
        const int off = b_rd0 + (tap * NB + fn * 32) * kUnit;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(buf + off));
    };

    constexpr int NROW = FM + 2;
    // One conv stage: 9 taps x FM rows x FN channel blocks of MFMAs.  LDS
    // reads complete in order, so they are issued in the order of first use:
    // input row 0 and the kh = 0 weights, then the kh = 1 weights and row 1
    // (used from row group 1 on), then the kh = 2 weights (row group 2).
    auto compute_conv = [&](const unsigned char *buf) {
        bf16x8 fw[9][FN];
        bf16x8 fx[2][3];
#pragma unroll
        for (int kw = 0; kw < 3; ++kw) fx[0][kw] = ldA(buf, 0, kw);
#pragma unroll
        for (int tap = 0; tap < 3; ++tap)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) fw[tap][fn] = ldB(buf, tap, fn);
#pragma unroll
        for (int qr = 0; qr < NROW; ++qr) {
            if (qr + 1 < 3) {
#pragma unroll
                for (int tap = 3 * (qr + 1); tap < 3 * (qr + 2); ++tap)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) fw[tap][fn] = ldB(buf, tap, fn);
            }
            // input row qr feeds output rows fm = qr - kh; the next row is read meanwhile
            if (qr + 1 < NROW) {
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) fx[(qr + 1) & 1][kw] = ldA(buf, qr + 1, kw);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                for (int kh = 0; kh < 3; ++kh) {
                    const int fm = qr - kh;
                    if (fm < 0 || fm >= FM) continue;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fw[kh * 3 + kw][fn], fx[qr & 1][kw], acc[fm][fn], 0, 0, 0);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One shortcut stage: the centre position of each output row, w_sc as the only tap.
    auto compute_shortcut = [&](const unsigned char *buf) {
        bf16x8 fw[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) fw[fn] = ldB(buf, 0, fn);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const bf16x8 fx = ldA(buf, fm + 1, 1);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[fn], fx, acc[fm][fn], 0, 0, 0);
        }
    };

    // one barrier per stage, matching the load wave's: after it, stage s is in LDS
    for (int s = 0; s < s_conv; ++s) {
        __builtin_amdgcn_s_barrier();
        compute_conv(smem + (s % NBUF) * TL::STAGE_BYTES);
    }
    if constexpr (EPI == EPI_SHORTCUT) {
        for (int s = s_conv; s < s_total; ++s) {
            __builtin_amdgcn_s_barrier();
            compute_shortcut(smem + (s % NBUF) * TL::STAGE_BYTES);
        }
    }

    // ---- epilogue: lane owns position (row, w0 + l32) and channels 8j + 4g + [0,4)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int hh = h0 + wm * FM + fm;
        const int ww = w0 + l32;
        if (hh >= H || ww >= W) continue;
        const int64_t p = ((nq * a.T + tq) * H + hh) * (int64_t)W + ww;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int co = n0 + wn * FN * 32 + fn * 32 + 8 * j + 4 * g;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[fm][fn][4 * j + e];
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

// Tile choice per output-channel count (measured on the workload shapes):
// 16 output rows x 32 columns per workgroup as a 2 x 2 grid of MFMA waves,
// each wave 8 rows x 32 columns x 32 channels (128 accumulators), plus the
// load wave; a 2 x 3 grid (96 channels) when C_out is a multiple of 96 but
// not of 64; 16 rows x 32 channels from four 4-row waves otherwise.
hipError_t launch_conv3d_bf16(const ConvLaunch &c, hipStream_t s) {
    if (c.res != nullptr && c.wsc != nullptr) {
        if (c.cout % 64 == 0) return launch_cfg<2, 2, 8, 1, EPI_SHORTCUT>(c, s);
        if (c.cout % 96 == 0) return launch_cfg<2, 3, 8, 1, EPI_SHORTCUT>(c, s);
        return launch_cfg<4, 1, 4, 1, EPI_SHORTCUT>(c, s);
    }
    if (c.cout % 64 == 0) return launch_plain<2, 2, 8, 1>(c, s);
    if (c.cout % 96 == 0) return launch_plain<2, 3, 8, 1>(c, s);
    return launch_plain<4, 1, 4, 1>(c, s);
}

}  // namespace wanvae
