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
// fused 1x1x1 shortcut).  Both operands are K-contiguous in 16-channel units
// (packed weights [kt][C_in/16][tap][co][16], activations [pos][ci]), which is
// the per-lane operand layout of the MFMA, so nothing is transposed.  The
// packed weight order makes a stage's weights for one tap one contiguous run
// of C_out x 32 bytes: whole L2 lines, where [co][tap][ci] would cost one
// 128-byte line request per 32 useful bytes.
//
// Input layout: each frame of x (and of the cache) is either channels-last,
// [h][w][cin], or cut into 16-channel slices, [cin/16][h][w][16] (the layout
// the ResidualBlock's norm writes for its convs).  A stage's input is then one
// slice of one frame either way; in the sliced layout its positions are
// contiguous 32-byte units, so the loads move whole cache lines (a
// channels-last stage reads 32 bytes of every position's line).
//
// Output tile: one frame t, HB = WM*FM output rows x 32 output columns x
// NB = WN*FN*32 output channels; MFMA wave (wm, wn) owns FM rows x FN channel
// blocks (FM*FN 32x32 fp32 accumulators).
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
// A workgroup has WM*WN MFMA waves and one load wave, and is persistent: one
// per compute unit, looping over its share of the output tiles.  The load
// wave moves every byte of every stage from L2 straight to LDS
// (buffer_load ... lds): each instruction fills one 1 KB block of a stage
// buffer, lane l writing bytes 16l..16l+15, so no VGPRs stage the data and no
// LDS-write instructions run.  Issuing these loads stalls the issuing wave on
// the LDS-DMA queue; with a wave of its own for them, the MFMA waves never
// wait on the memory pipe.  They are raw buffer loads over one frame slab: an
// input position outside the image gets an out-of-range offset and the
// hardware writes zeros, so padding costs no branch.  Because the tile holds
// the H and W halo, every per-lane load offset is fixed for a tile's K loop; a
// stage only moves the buffer base (frame and channel slice).
//
// Stages rotate through a ring of NBUF LDS buffers, across tile boundaries (the
// next tile's first stages load while the MFMA waves run the epilogue).  There
// is no per-stage barrier: the load wave publishes in LDS how many stages have
// landed, each MFMA wave publishes how many it has consumed, and a slot is
// refilled once every MFMA wave has consumed the stage it held.  MFMA waves
// thus drift apart by up to a few stages, which spreads their LDS read bursts
// instead of lining them up behind a barrier.  Every wait on a flag is bounded;
// a wait that reaches its bound goes on and is counted (g_wait_giveups), so a
// stalled protocol shows up as a non-zero count instead of a hang.
// With one MFMA wave per SIMD nothing hides a stage's first LDS round trip, so
// each stage reads the next one's first operands during its last rows (when
// that stage has landed), and every row's fragment reads are issued one per
// MFMA rather than as a burst.
//
// The decoder's upsampler conv (up2: nearest x2 in H and W, then a 3x3 conv
// with one temporal tap) runs by output phase where C_out is a multiple of 96
// (PH kernels): output row 2i + py reads input rows i + py - 1 and i + py
// only (likewise columns), so each phase (py, px) is a 2x2 conv of the
// half-resolution input with merged weights (packed that way by
// launch_pack_conv2d_weights).  A PH tile is 12 input rows x 32 columns x 96
// channels of one phase; a stage holds that phase's 4 taps, 36 MFMAs per wave,
// and two load waves share its DMA (A and B blocks).  Other C_out read the
// doubled image through the loader (output position (h, w) from input
// (h/2, w/2)) and run the 9 taps.
//
// LDS layout: 32-byte units (16 bf16 channels of one position or one weight
// row), A tile rows 34 units apart.  The two 16-byte halves of a unit are
// swapped when bit 3 of its column (A) or unit index (B) is set: 16 lanes
// reading one half of 16 consecutive units then hit 16 distinct 16-byte bank
// groups (gfx950 serves 16 lanes x 16 bytes per LDS cycle).
//
// Causal pad: without a cache, the stages of a frame before 0 only add exact
// zeros and are skipped (uniform per tile); with a cache they read it.
//
// Epilogue: each lane owns one output position and 4 consecutive output
// channels per accumulator quad.  The accumulators start at the bias (plus
// the shortcut bias), the identity residual is added in fp32 at the end, and
// the result is rounded once to bf16 (8-byte stores).  The 1x1x1 shortcut GEMM runs as extra stages of the same
// accumulators, each holding two 16-channel slices (one when two do not fit a
// stage buffer) of x at the output positions and of w_sc: every load of such
// a stage is useful data, and x (channels-last) comes in 64-byte pieces per
// position, which the LDS-DMA moves at twice the rate of 32-byte ones.
//
// Conv A of a ResidualBlock whose out_dim is one tile's channel block (96 or
// 32) computes norm2 + SiLU in its epilogue (EPI_NORM): each wave holds every
// channel of its output positions, so the sum of squares is one exchange
// between a lane and its partner lane ^ 32, and n2 is written straight into
// the 16-channel-slice layout conv B reads (a is never stored, nor read back
// by a norm kernel).
//
// Tile order: batch slowest, then row block, column block, frame, and
// output-channel block fastest.  Without a cache the tiles of frames 0 and 1
// (a third and two thirds of the stages) form one work item, every other tile
// is an item of its own, so all items carry the same work and the persistent
// workgroups finish together.  Each of the 8 XCDs (workgroup index mod 8)
// owns a contiguous range of items, so the workgroups on one XCD work on
// neighbouring frames of one spatial block, all channel blocks of each side
// by side: every input frame (and the residual / shortcut input) of the block
// comes from HBM once and is then shared through the XCD's L2 by the tiles of
// frames t .. t+2 and of every channel block, and the weights (at most 2 MB
// for 384 -> 384 channels in bf16... 5.3 MB for 1024) stay in L2 as well.
#include <atomic>
#include <utility>

#include "bf16.h"
#include "internal.h"
#include "mfma_sched.h"

namespace wanvae {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource word 3 for raw (unformatted, stride 0) buffers on gfx9-family
// GPUs; loads past num_records return zero.
constexpr int kBufFlags = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kSuperBlock = 20;   // frame groups per super-block of the tile order (launch_cfg)  // beyond every buffer: the load returns zeros

constexpr int kKC = 16;          // input channels per stage = one MFMA k-step
constexpr int kUnit = 32;        // bytes per LDS unit (16 bf16)
constexpr int kWB = 32;          // output columns per tile (one MFMA N block)
constexpr int kAS = kWB + 2;     // A tile columns including the W halo = row stride in units
constexpr int kXCD = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int kSyncBytes = 256;  // LDS for the stage flags
// Epilogue staging, per MFMA wave: one output row of 32 positions x 32
// channels, positions 80 bytes apart (64 used; the pad spreads the 8-byte
// writes of 16 lanes over distinct bank groups)
constexpr int kEpiStride = 80;
constexpr int kEpiBytes = 32 * kEpiStride;
// Default bound on every flag wait: 2^15 polls ~64 cycles apart (about 2M
// cycles, far beyond any real wait).  Past it the wave goes on rather than
// hang, and counts the event in g_wait_giveups: the stage it then reads (or
// the slot it refills) may not be the one the protocol meant, so the launch's
// output is suspect.  The bound is a kernel argument (set_wait_bound) so that
// a test can force the give-up path from the host.
constexpr int kSpinCapDefault = 1 << 15;

// s_waitcnt immediate for "vmcnt <= n" (n <= 63), other counters left alone
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitVm0 = waitcnt_vm(0);

// EPI_NORM: conv A of the ResidualBlock with norm2 + SiLU in its epilogue,
// for tiles whose waves hold every output channel of their positions (one
// channel block per tile, WN = 1): y is then n2, in the 16-channel-slice
// layout conv B reads, instead of a.
enum Epilogue { EPI_BIAS = 0, EPI_IDENTITY = 1, EPI_SHORTCUT = 2, EPI_NORM = 3 };

// u / (1 + exp(-u)); exp(-u) = inf for very negative u gives -0
__device__ inline float silu(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

// sum of v over lanes l and l ^ 32: v_permlane32_swap on two copies of v
// leaves each lane its own value and its partner's, one in each result
__device__ inline float halves_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Division of a work-item index by a launch constant d (1 <= d < 2^31) as a
// multiply and a shift, q = (n m) >> (31 + s) with s = ceil(log2 d) and
// m = ceil(2^(31+s) / d) (a 32-bit value): m / 2^(31+s) exceeds 1/d by less
// than 2^-(31+s), so for 0 <= n < 2^31 the product exceeds n/d by less than
// 2^-s <= 1/d and never reaches the next integer (the fraction of n/d is at
// most (d-1)/d).  A tile decode then costs a few scalar instructions instead
// of 64-bit divisions by kernel arguments.
// The launch holds six multipliers and their shifts 31 + s, packed four to a
// word (a byte each), to spare scalar registers.
struct FastDiv {
    uint32_t m[6];
    uint32_t shifts[2];
};

inline void set_fastdiv(FastDiv &f, int k, uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.m[k] = (uint32_t)(((1ull << (31 + s)) + d - 1) / d);
    uint32_t &w = f.shifts[k / 4];
    w = (w & ~(0xffu << (8 * (k % 4)))) | ((31 + s) << (8 * (k % 4)));
}

// the quotient n / d_k, for 0 <= n < 2^31
template <int K>
__device__ inline uint32_t fdiv(uint32_t n, const FastDiv &f) {
    return (uint32_t)(((uint64_t)n * f.m[K]) >> ((f.shifts[K / 4] >> (8 * (K % 4))) & 0xff));
}

struct Args {
    const uint16_t *x;      // conv input [n][t][h][w][cin]
    const uint16_t *cache;  // [n][2][h][w][cin] or null
    const uint16_t *w;      // packed: [3 kt][cin/16][9 taps][cout][16] (upsampler: 1 kt; PH: [cin/16][4 phases][4 taps][cout][16])
    const float *bias;      // [cout] or null
    const uint16_t *res;    // [n][t][h][w][cres] or null
    const uint16_t *wsc;    // [cout][cres] or null
    const float *bsc;       // [cout] or null
    uint16_t *y;            // [n][t][h][w][cout], or for EPI_NORM [n][t][cout/16][h][w][16]
    // EPI_NORM: norm2 scale and shift ([cout] fp32, shift may be null) and eps
    const float *ngamma, *nbeta;
    float neps;
    int64_t N, T, H, W;
    int cin, cout, cres;
    int cout_p;             // cout rounded up to 32: the packed weight's channel count
    int tiles_w, tiles_h;
    // Tile order within one (batch item, row block): frame groups in
    // super-blocks of sbg, and within a super-block the frame group fastest,
    // then the column block (the last super-block holds sb_r groups).  The
    // decode's divisors: output-channel blocks (0), the items of one (batch
    // item, row block) (1), of one full super-block (2), row blocks (3),
    // sbg (4) and sb_r (5).
    FastDiv div;
    int region;     // frame groups x column blocks
    int sbg, sb_gw; // frame groups per super-block, and times the column blocks
    int sb_full;    // items of the full super-blocks: (super-blocks - 1) sb_gw
    int sb_last0;   // first frame group of the last super-block
    int sb_r;       // its frame groups
    // work items of the launch (fewer than 2^31): one output tile each, or with pair = 1 (no
    // cache: frames 0 and 1 skip the stages of the causal pad) the tiles of
    // frames 0 and 1 of one block together, so every item runs three frames'
    // worth of stages
    int64_t items;
    int pair;
    int x_sliced;           // x and cache frames are [cin/16][h][w][16], not [h][w][cin]
    // 1x1x1 stages (SC kernels): input [n][t][h][w][sc_c] at the output
    // positions and weight wsc [cout][sc_c]: the block's shortcut (sc_in =
    // res), or the whole product of a GEMM launch (gemm = 1: no 3x3x3 stages,
    // sc_in = x)
    const uint16_t *sc_in;
    int sc_c;
    int gemm;
    // upsampler conv (up2 = 1): x holds frames of (H/2) x (W/2) positions,
    // read as their nearest-neighbour doubling (position (h, w) of the H x W
    // image is x[h/2][w/2]); only the current frame's taps, packed weight
    // [cin/16][9 taps][cout][16]; no cache
    int up2;
    // with up2: the frames doubled in time as well (upsample3d): x holds
    // xT = (T + 1) / 2 frames per batch item and output frame t reads input
    // frame (t + 1) / 2; otherwise xT = T and frame t reads frame t
    int up_t;
    int64_t xT;
    // polls before a flag wait gives up (and is counted)
    int spin_cap;
};

// One output tile: batch item, frame, first row / column / output channel,
// and its K stages (conv stages from temporal tap kt_begin, then shortcut);
// ntiles: the tiles of its work item.
struct TileInfo {
    int64_t nq, tq;
    int h0, w0, n0;
    int kt_begin, s_conv, s_total;
    int ntiles;
    int ph;   // PH kernels: output phase 2 py + px (output row 2 i + py, column 2 j + px)
};

// PH: the upsampler conv by output phase (see the kernel's comment): rows
// and columns are the input's (half-resolution) ones, a stage holds the 4
// merged taps of one phase, and the A tile needs one halo row, not two.
template <int WM, int WN, int FM, int FN, bool PH = false>
struct Tile {
    static constexpr int NWAVE = WM * WN;                    // MFMA waves
    // load waves: one; two for PH, whose short stages (36 MFMAs a wave) need
    // more DMA in flight than one wave's 63 outstanding loads cover: the first
    // moves each stage's A blocks, the second its B blocks
    static constexpr int NLW = PH ? 2 : 1;
    static constexpr int kThreads = (NWAVE + NLW) * 64;
    static constexpr int HB = WM * FM;                       // output rows
    static constexpr int NB = WN * FN * 32;                  // output channels
    static constexpr int AR = HB + (PH ? 1 : 2);             // A tile rows (H halo)
    static constexpr int A_BLOCKS = (AR * kAS + 31) / 32;    // 1 KB blocks = 32 units
    static constexpr int B_BLOCKS = (PH ? 4 : 9) * NB / 32;
    static constexpr int BLOCKS = A_BLOCKS + B_BLOCKS;       // load instructions per stage
    static constexpr int STAGE_BYTES = BLOCKS * 1024;
    // FN > 1: each wave owns several channel blocks and walks the taps kh by kh
    // (9 FN weight fragments in registers would not fit beside the
    // accumulators).  The bias of every tile sits in LDS, not in registers.
    static constexpr bool KH_OUTER = FN > 1 && !PH;
    static constexpr int kBiasBytes = 8 * 1024;   // bias in LDS: [cout_p] fp32, cout <= 2048
    static constexpr int kLds = 160 * 1024 - kSyncBytes - NWAVE * kEpiBytes - kBiasBytes;
    static constexpr int NBUF = 5 * STAGE_BYTES <= kLds   ? 5
                                : 4 * STAGE_BYTES <= kLds ? 4
                                : 3 * STAGE_BYTES <= kLds ? 3
                                                          : 2;
    static_assert(NBUF * STAGE_BYTES <= kLds, "tile does not fit the 160 KB LDS");
    static_assert(NWAVE + 1 <= kSyncBytes / 4, "one flag per wave");
    static constexpr int kPerCU =
        (160 * 1024) / (NBUF * STAGE_BYTES + kSyncBytes + NWAVE * kEpiBytes + kBiasBytes);
    // shortcut stages: SCS 16-channel slices of x at the output positions
    // and of w_sc.  SCS = 2 (when it fits): x as 64-byte pieces (32 channels)
    // per position, two 1 KB blocks per row, then the two slices' w_sc units.
    // SCS = 1: one slice, one 1 KB block per row of x, then its w_sc units.
    static constexpr int SC_UNITS = HB * kWB + NB;                // units per slice
    static constexpr int SCS = 2 * SC_UNITS / 32 <= BLOCKS ? 2 : 1;
    static constexpr int SC_BLOCKS = SCS * SC_UNITS / 32;         // useful loads per stage
    static constexpr int SC_W_UNIT0 = SCS * HB * kWB;             // first w_sc unit
    static_assert(SC_BLOCKS <= BLOCKS, "a shortcut slice fits a stage buffer");
};

// byte offset of half `h` (0/1) of A unit (row r, column c) and of B unit u
__device__ __host__ constexpr int a_off(int r, int c, int h) {
    return (r * kAS + c) * kUnit + ((h ^ ((c >> 3) & 1)) << 4);
}
__device__ __host__ constexpr int b_off(int u, int h) { return u * kUnit + ((h ^ ((u >> 3) & 1)) << 4); }

// Raw buffer resource (stride 0, num_records bytes) for a wave-uniform base
// and size (made scalar explicitly: the resource must live in SGPRs).
__device__ inline i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)),
                 __builtin_amdgcn_readfirstlane((int)bytes), kBufFlags};
}

// One wavefront-wide 16-byte-per-lane load from a buffer straight into LDS:
// lane l's 16 bytes at byte offset voff land at LDS byte address
// lds_addr + 16 * l (lds_addr wave-uniform).  Written as inline assembly so the
// compiler does not wait for these loads before unrelated LDS accesses; the
// kernel orders them itself with explicit vmcnt waits.  M0 is set inside the
// same statement, immediately before its only use.
__device__ inline void lds_dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane((int)lds_addr)), "v"(voff), "s"(rsrc)
                 : "memory");
}

// The same resource as a typed value for the buffer load/store builtins.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(u), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), kBufFlags);
}

// rows of group gi when FM rows are taken EG at a time
template <int FM, int EG>
__device__ __host__ constexpr int group_rows(int gi) { return FM - gi * EG < EG ? FM - gi * EG : EG; }

__device__ inline uint32_t lds_address(const unsigned char *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

// compiler-only fence: no memory access moves across it
__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

}  // namespace

// Flag waits that reached their bound, per device, since the library was
// loaded or the count was last reset (a vector atomic by one lane per event).
__device__ unsigned int g_wait_giveups;

namespace {

__device__ inline void count_giveup(int lane) {
    if (lane == 0) __hip_atomic_fetch_add(&g_wait_giveups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int WM, int WN, int FM, int FN, int EPI, bool SC, bool PH>
__global__ __launch_bounds__((WM *WN + (PH ? 2 : 1)) * 64) void conv3d_bf16_kernel(Args a) {
    using TL = Tile<WM, WN, FM, FN, PH>;
    static_assert(!PH || (WM == 4 && WN == 1 && FM == 3 && EPI == EPI_BIAS && !SC),
                  "the phase upsampler runs on the 96-channel tile with a bias epilogue");
    constexpr int HB = TL::HB;
    constexpr int NB = TL::NB;
    constexpr int NBUF = TL::NBUF;

    __shared__ __attribute__((aligned(1024))) unsigned char smem[NBUF * TL::STAGE_BYTES];
    // sync[0]: stages landed (load wave); sync[1 + w]: stages consumed by MFMA
    // wave w; sync[1 + NWAVE]: stages landed, second load wave (NLW = 2)
    __shared__ int sync[kSyncBytes / 4];
    __shared__ __attribute__((aligned(16))) unsigned char epi_stage[TL::NWAVE * kEpiBytes];
    // bias (+ shortcut bias) of every output channel
    __shared__ __attribute__((aligned(16))) float bias_lds[TL::kBiasBytes / 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // NWAVE = the load wave
    const int H = (int)a.H, W = (int)a.W;
    const int64_t HW = (int64_t)H * W;
    const int ck = a.cin / kKC;

    static_assert(TL::NLW == 1 || !SC, "two load waves split conv stages only");
    static_assert(TL::NWAVE + 2 <= kSyncBytes / 4, "flags");
    if (tid <= TL::NWAVE + 1) sync[tid] = 0;
    for (int c = tid; c < a.cout_p; c += TL::kThreads) {
        float b = a.bias && c < a.cout ? a.bias[c] : 0.0f;
        if constexpr (SC)
            if (a.bsc && c < a.cout) b += a.bsc[c];
        bias_lds[c] = b;
        if constexpr (EPI == EPI_NORM) {
            // gamma * sqrt(C) and beta after the bias
            bias_lds[a.cout_p + c] = a.ngamma[c] * sqrtf((float)a.cout);
            bias_lds[2 * a.cout_p + c] = a.nbeta ? a.nbeta[c] : 0.0f;
        }
    }
    static_assert(EPI != EPI_NORM || (WN == 1 && 3 * NB <= TL::kBiasBytes / 4),
                  "the norm epilogue needs every channel of a position in one wave");
    __syncthreads();
    // flag accesses: relaxed atomics on the LDS array itself, so they stay
    // ds_read / ds_write (through a generic pointer they would become FLAT
    // accesses, which the compiler must also wait for with vmcnt)
    auto flag_read = [&](int i) { return __builtin_amdgcn_readfirstlane(__atomic_load_n(&sync[i], __ATOMIC_RELAXED)); };
    auto flag_write = [&](int i, int v) { __atomic_store_n(&sync[i], v, __ATOMIC_RELAXED); };
    // stages landed (both load waves' parts, with two): a VGPR value, made
    // uniform where it is used
    auto landed_count = [&]() __attribute__((always_inline)) {
        const int l0 = __atomic_load_n(&sync[0], __ATOMIC_RELAXED);
        if constexpr (TL::NLW == 2) {
            const int l1 = __atomic_load_n(&sync[1 + TL::NWAVE], __ATOMIC_RELAXED);
            return l0 < l1 ? l0 : l1;
        }
        return l0;
    };

    // ---- this workgroup's work items.  XCD x (= workgroup index mod 8) holds
    // wg_x of the grid's workgroups and owns a contiguous item range of
    // matching share, [x_begin, x_begin + x_count); its workgroups take the
    // items of that range round-robin.  (With at least as many items as
    // workgroups, every workgroup gets one or more.)  Items carry equal work
    // (pairing frames 0 and 1 when their pad stages are skipped): with a tile
    // per item, the workgroups that drew no frame-0/1 tiles would run up to
    // a tenth longer than the mean at the latent resolution.
    const int64_t nwg = gridDim.x, bid = blockIdx.x;
    const int64_t xcd = bid % kXCD, loc = bid / kXCD;
    const int64_t wg_x = nwg / kXCD + (xcd < nwg % kXCD ? 1 : 0);
    const int64_t wg_before = xcd * (nwg / kXCD) + (xcd < nwg % kXCD ? xcd : nwg % kXCD);
    const int64_t x_begin = a.items * wg_before / nwg;
    const int64_t x_count = a.items * (wg_before + wg_x) / nwg - x_begin;

    const int ncb = a.cout_p / NB;   // output-channel blocks (the last may be partly padding)
    // tile `sub` of work item `item` (a scalar decode: multiply-shift
    // divisions by the launch's precomputed divisors)
    auto decode = [&](int64_t item, int sub) __attribute__((always_inline)) {
        uint32_t tile = (uint32_t)item, q;
        TileInfo ti;
        q = fdiv<0>(tile, a.div);
        ti.n0 = (int)(tile - q * (uint32_t)ncb) * NB;
        tile = q;
        ti.ph = 0;
        if constexpr (PH) {
            // the four phases of a block side by side (they read the same input)
            ti.ph = (int)(tile & 3);
            tile >>= 2;
        }
        // frame groups ({0, 1}, 2, 3, ... when paired) and column blocks of
        // one (batch item, row block), by super-block
        q = fdiv<1>(tile, a.div);
        uint32_t idx = tile - q * (uint32_t)a.region, wb, g0, gl;
        tile = q;
        if (idx < (uint32_t)a.sb_full) {
            q = fdiv<2>(idx, a.div);
            g0 = q * (uint32_t)a.sbg;
            idx -= q * (uint32_t)a.sb_gw;
            wb = fdiv<4>(idx, a.div);
            gl = idx - wb * (uint32_t)a.sbg;
        } else {
            idx -= (uint32_t)a.sb_full;
            g0 = (uint32_t)a.sb_last0;
            wb = fdiv<5>(idx, a.div);
            gl = idx - wb * (uint32_t)a.sb_r;
        }
        const int64_t grp = g0 + gl;
        ti.ntiles = a.pair && grp == 0 ? 2 : 1;
        ti.tq = a.pair ? (grp == 0 ? sub : grp + 1) : grp;
        ti.w0 = (int)wb * kWB;
        q = fdiv<3>(tile, a.div);
        ti.h0 = (int)(tile - q * (uint32_t)a.tiles_h) * HB;
        ti.nq = q;
        // without a cache the stages of frames before 0 only add zeros: skipped
        const int kt_begin = a.up2 ? 2 : (a.cache != nullptr || ti.tq >= 2) ? 0 : (int)(2 - ti.tq);
        ti.kt_begin = kt_begin;
        ti.s_conv = a.gemm ? 0 : (3 - kt_begin) * ck;
        ti.s_total = ti.s_conv + (SC ? a.sc_c / (kKC * TL::SCS) : 0);
        return ti;
    };

    const uint32_t smem_base = lds_address(smem);

    if (wave >= TL::NWAVE) {
        // load wave lw: everything (one load wave), or with two the A (lw = 0)
        // or B (lw = 1) blocks of every stage
        const int lw = wave - TL::NWAVE;
        // ================= load wave: all global -> LDS traffic of every tile.
        // Block b of a stage: lane l writes physical half (l & 1) of unit
        // 32 * b' + l / 2 (b' relative to the A or B region), so it fetches the
        // logical half that the swizzle puts there.
        // bytes between neighbouring positions of a frame slab, and elements
        // between its 16-channel slices
        // the input frame: H x W, or (H/2) x (W/2) read doubled (up2)
        const int up = a.up2;
        const int Wi = W >> up;
        const int64_t HWi = HW >> (2 * up);
        const uint32_t cs2 = a.x_sliced ? (uint32_t)kUnit : (uint32_t)a.cin * 2;
        const int64_t slice_elems = a.x_sliced ? HWi * kKC : kKC;
        const uint32_t tap2 = (uint32_t)a.cout_p * kUnit;   // bytes per tap of a packed stage
        // byte offset of block b's piece for a conv stage (sc = false) or a
        // shortcut stage (sc = true: x at the output positions, w_sc as one tap)
        auto block_off = [&](const TileInfo &ti, int b) __attribute__((always_inline)) -> uint32_t {
            if (b < TL::A_BLOCKS) {
                const int u = b * 32 + (lane >> 1);
                const int r = u / kAS, c = u % kAS;
                const int hf = (lane & 1) ^ ((c >> 3) & 1);
                if constexpr (PH) {
                    // input rows h0 + py - 1 .. and columns w0 + px - 1 .. of
                    // the half-resolution frame
                    const int hh = ti.h0 + (ti.ph >> 1) - 1 + r, ww = ti.w0 + (ti.ph & 1) - 1 + c;
                    const bool inside = r < TL::AR && hh >= 0 && hh < (H >> 1) && ww >= 0 && ww < Wi;
                    return inside ? (uint32_t)(hh * Wi + ww) * cs2 + hf * 16 : kOOB;
                }
                const int hh = ti.h0 - 1 + r, ww = ti.w0 - 1 + c;
                const bool inside = r < TL::AR && hh >= 0 && hh < H && ww >= 0 && ww < W;
                return inside ? (uint32_t)((hh >> up) * Wi + (ww >> up)) * cs2 + hf * 16 : kOOB;
            }
            const int u = (b - TL::A_BLOCKS) * 32 + (lane >> 1);
            const int hf = (lane & 1) ^ ((u >> 3) & 1);
            const int tap = u / NB, nl = u % NB;
            return (uint32_t)tap * tap2 + (uint32_t)(ti.n0 + nl) * kUnit + hf * 16;
        };
        // shortcut stage, SCS = 2: block b < 2 HB holds row b / 2, positions
        // 16 (b % 2) .. +15 of x, 64 bytes (the stage's 32 channels) each:
        // lane l fetches position l / 4, 16-byte quarter q = (l % 4) ^ ((pos
        // >> 2) & 3), so each position's four quarters stay in four
        // consecutive lanes (one 64-byte piece per lane quad) and a fragment
        // read (one quarter of 16 positions) hits 16 distinct bank groups.
        // SCS = 1: block b < HB is row b of x, 32 bytes per position.  Then
        // the w_sc units of the SCS slices.  Blocks past the useful ones load
        // zeros into the unused tail of the buffer, so every stage issues
        // BLOCKS loads (the vmcnt accounting counts whole stages).  Returns
        // the offset and whether it is relative to the w_sc resource.
        auto sc_block_off = [&](const TileInfo &ti, int b, bool &from_w) -> uint32_t {
            from_w = false;
            if (b >= TL::SC_BLOCKS) return kOOB;
            if (b < TL::SCS * HB) {
                int r, c, q;
                if constexpr (TL::SCS == 2) {
                    r = b / 2;
                    c = (b % 2) * 16 + (lane >> 2);
                    q = (lane & 3) ^ ((c >> 2) & 3);
                } else {
                    r = b;
                    c = lane >> 1;
                    q = (lane & 1) ^ ((c >> 3) & 1);
                }
                const int hh = ti.h0 + r, ww = ti.w0 + c;
                return hh < H && ww < W ? (uint32_t)(hh * W + ww) * (uint32_t)(a.sc_c * 2) + q * 16 : kOOB;
            }
            from_w = true;
            const int u = (b - TL::SCS * HB) * 32 + (lane >> 1);   // w_sc unit: slice j, channel nl
            const int j = u / NB, nl = u % NB;
            const int hf = (lane & 1) ^ ((nl >> 3) & 1);
            return (uint32_t)((ti.n0 + nl) * a.sc_c * 2) + j * kUnit + hf * 16;
        };

        // request cursor: stage si of tile sub of local item it (item
        // x_begin + it), ring slot
        TileInfo ti{};
        int64_t it = loc;
        int si = 0, sub = 0, slot = 0;
        uint32_t l_off[TL::BLOCKS];   // conv-stage offsets of the cursor's tile
        auto start_tile = [&]() __attribute__((always_inline)) {
            ti = decode(x_begin + it, sub);
#pragma unroll
            for (int b = 0; b < TL::BLOCKS; ++b) l_off[b] = block_off(ti, b);
        };
        if (it < x_count) start_tile();

        // request the cursor's stage into its ring slot (asynchronous; completion
        // via vmcnt), then advance the cursor, into the next tile if need be
        auto issue_next = [&]() __attribute__((always_inline)) {
            const uint16_t *abase, *bbase;
            uint32_t abytes, bbytes;
            const bool sc = si >= ti.s_conv;   // conv stages first, then the shortcut stages
            if (!sc) {
                const int cs = si;   // conv stage index
                int kt, cc;
                if (a.x_sliced) {
                    // 16-channel slice outer, temporal tap inner: the tiles of
                    // frames t, t+1, t+2, which run side by side on one XCD,
                    // then read each slice of a frame within a few stages of
                    // each other, while it is still in the L2
                    const int nkt = 3 - ti.kt_begin;
                    cc = cs / nkt;
                    kt = ti.kt_begin + (cs - cc * nkt);
                } else {
                    // channels-last input: the slices of one frame share cache
                    // lines, so they are read back to back
                    kt = ti.kt_begin + cs / ck;
                    cc = cs % ck;
                }
                // (the temporal upsampler reads input frame (t + 1) / 2 for
                // output frame t; it has only the current-frame tap)
                const int64_t ts = a.up_t ? (ti.tq + 1) >> 1 : ti.tq + kt - 2;
                abase = (ts >= 0 ? a.x + ((ti.nq * a.xT + ts) * HWi) * a.cin
                                 : a.cache + ((ti.nq * 2 + (ts + 2)) * HWi) * a.cin) +
                        cc * slice_elems;
                abytes = (uint32_t)(HWi * a.cin * 2 - cc * slice_elems * 2);
                // elements of the packed weight before stage (kt, cc); an
                // upsampler's weight holds the current frame's taps only, and
                // by phase its 4 merged taps of each phase
                const int wkt = up ? kt - 2 : kt;
                const int64_t wskip = PH ? (int64_t)(cc * 4 + ti.ph) * 4 * a.cout_p * kKC
                                         : (int64_t)(wkt * ck + cc) * 9 * a.cout_p * kKC;
                bbase = a.w + wskip;
                bbytes = (uint32_t)(((int64_t)(PH ? 16 : up ? 9 : 27) * a.cin * a.cout_p - wskip) * 2);
            } else {
                // first 16-channel slice of this shortcut stage
                const int cc = (si - ti.s_conv) * TL::SCS;
                abase = a.sc_in + ((ti.nq * a.T + ti.tq) * HW) * a.sc_c + cc * kKC;
                abytes = (uint32_t)(HW * a.sc_c * 2 - cc * kKC * 2);
                bbase = a.wsc + cc * kKC;
                bbytes = (uint32_t)((int64_t)a.cout * a.sc_c * 2 - cc * kKC * 2);
            }
            // the cursor is uniform; buffer_rsrc makes that explicit to the compiler
            const i32x4 ar = buffer_rsrc(abase, abytes);
            const i32x4 br = buffer_rsrc(bbase, bbytes);
            const uint32_t base = smem_base + (uint32_t)slot * TL::STAGE_BYTES;
            if constexpr (TL::NLW == 2) {
                if (lw == 0) {
#pragma unroll
                    for (int b = 0; b < TL::A_BLOCKS; ++b) lds_dma16(ar, base + b * 1024, l_off[b]);
                } else {
#pragma unroll
                    for (int b = TL::A_BLOCKS; b < TL::BLOCKS; ++b) lds_dma16(br, base + b * 1024, l_off[b]);
                }
            } else {
#pragma unroll
                for (int b = 0; b < TL::BLOCKS; ++b) {
                    uint32_t off = l_off[b];
                    bool from_b = b >= TL::A_BLOCKS;
                    if constexpr (SC)
                        if (sc) off = sc_block_off(ti, b, from_b);
                    lds_dma16(from_b ? br : ar, base + b * 1024, off);
                }
            }
            slot = slot + 1 == NBUF ? 0 : slot + 1;
            if (++si == ti.s_total) {
                si = 0;
                if (++sub == ti.ntiles) {
                    sub = 0;
                    it += wg_x;
                }
                if (it < x_count) start_tile();
            }
        };

        // the slowest MFMA wave's consumed-stage count
        auto min_done = [&]() __attribute__((always_inline)) {
            int m = flag_read(1);
#pragma unroll
            for (int w = 1; w < TL::NWAVE; ++w) {
                const int d = flag_read(1 + w);
                m = d < m ? d : m;
            }
            return m;
        };

        int issued = 0, landed = 0, done = 0;
        for (;;) {
            // request stages while a ring slot is free: the slot of stage
            // `issued` last held stage issued - NBUF, which every MFMA wave
            // must have consumed
            while (it < x_count && issued < done + NBUF) {
                issue_next();
                ++issued;
            }
            if (landed < issued) {
                // the oldest requested stage has landed once at most the loads
                // requested after it are outstanding (vmcnt counts to 63 at most,
                // and at most 63 loads are ever in flight); B: this wave's
                // loads per stage
                auto wait_oldest = [&]<int B>() __attribute__((always_inline)) {
                    switch (issued - landed - 1) {
                        case 0: __builtin_amdgcn_s_waitcnt(kWaitVm0); break;
                        case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(B < 63 ? B : 63)); break;
                        case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * B < 63 ? 2 * B : 63)); break;
                        default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * B < 63 ? 3 * B : 63)); break;
                    }
                };
                if constexpr (TL::NLW == 2) {
                    if (lw == 0)
                        wait_oldest.template operator()<TL::A_BLOCKS>();
                    else
                        wait_oldest.template operator()<TL::BLOCKS - TL::A_BLOCKS>();
                } else {
                    wait_oldest.template operator()<TL::BLOCKS>();
                }
                compiler_fence();
                ++landed;
                if (lane == 0) flag_write(lw == 0 ? 0 : 1 + TL::NWAVE, landed);
                compiler_fence();
                done = min_done();
                continue;
            }
            if (it >= x_count) break;   // everything requested has landed and been published
            // every slot holds a published, unconsumed stage: wait for the slowest wave
            for (int spin = 0; spin < a.spin_cap; ++spin) {
                __builtin_amdgcn_s_sleep(1);
                done = min_done();
                if (issued < done + NBUF) break;
            }
            if (issued >= done + NBUF) {   // bound reached: go on, and say so
                done = issued - NBUF + 1;
                count_giveup(lane);
            }
        }
        return;
    }

    // ================= MFMA waves
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int l32 = lane & 31;
    const int g = lane >> 5;   // k-group: which 8-channel half of the 16-channel unit
    // B fragment (tap, fn): unit tap*NB + wn*FN*32 + fn*32 + l32; NB and 32 are
    // multiples of 16, so its swizzle bit is bit 3 of l32
    const int b_rd0 = TL::A_BLOCKS * 1024 + b_off(wn * FN * 32 + l32, g);
    // A fragment (row wm*FM + qr, column l32 + kw)
    int a_rd[3];
#pragma unroll
    for (int kw = 0; kw < 3; ++kw) a_rd[kw] = a_off(wm * FM, l32 + kw, g);

    auto ldA = [&](const unsigned char *buf, int qr, int kw) __attribute__((always_inline)) {
        const int off = a_rd[kw] + qr * kAS * kUnit;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(buf + off));
    };
    auto ldB = [&](const unsigned char *buf, int tap, int fn) __attribute__((always_inline)) {
        const int off = b_rd0 + (tap * NB + fn * 32) * kUnit;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(buf + off));
    };

    floatx16 acc[FM][FN];
    constexpr int NROW = FM + 2;
    // Stage operands, kept across stages: the next stage's first operands
    // (input row 0 and the kh = 0 weights) are read during this stage's last
    // two rows, straight into the registers they are used from.  With one
    // MFMA wave per SIMD nothing else would hide that LDS round trip at every
    // stage start.  fx is a two-row ring: row r of a stage with parity PAR is
    // in fx[(r + PAR) & 1], and the next stage's row 0 goes into the buffer
    // this stage's last row does not use, so with an odd row count the parity
    // alternates from stage to stage.
    bf16x8 fw[9][FN];
    bf16x8 fx[2][3];
    // KH_OUTER tiles keep input rows across kernel rows instead: input row i
    // of a stage (0 .. FM + 1) in fk[i % 3], the next stage's row 0 in fk[0]
    bf16x8 fk[3][3];
    // PH tiles: the merged weights of row tap a and column tap b (pw[a][b]),
    // input rows 0 .. FM of the wave (pr[r][b]: columns l32 + b)
    bf16x8 pw[2][2][FN];
    bf16x8 pr[FM + 1][2];
    constexpr bool ALT = !TL::KH_OUTER && !PH && NROW % 2 == 1;   // rows per stage odd
    // row 0 and the kh = 0 weights of the stage in `buf` (parity par)
    auto load_first = [&](const unsigned char *buf, int par) __attribute__((always_inline)) {
        if constexpr (PH) {
#pragma unroll
            for (int b = 0; b < 2; ++b) pr[0][b] = ldA(buf, 0, b);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) pw[0][b][fn] = ldB(buf, b, fn);
            return;
        } else if constexpr (TL::KH_OUTER) {
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) fk[0][kw] = ldA(buf, 0, kw);
        } else if (par) {
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) fx[1][kw] = ldA(buf, 0, kw);
        } else {
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) fx[0][kw] = ldA(buf, 0, kw);
        }
#pragma unroll
        for (int tap = 0; tap < 3; ++tap)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) fw[tap][fn] = ldB(buf, tap, fn);
    };

    int consumed = 0, seen = 0, slot = 0;
    // wait until stage `consumed` has landed
    auto wait_landed = [&]() __attribute__((always_inline)) {
        for (int spin = 0; seen <= consumed && spin < a.spin_cap; ++spin) {
            seen = __builtin_amdgcn_readfirstlane(landed_count());
            if (seen <= consumed) __builtin_amdgcn_s_sleep(1);
        }
        if (seen <= consumed) count_giveup(lane);   // bound reached: go on, and say so
        compiler_fence();   // the stage's reads stay below the flag read
    };

    // One conv stage: 9 taps x FM rows x FN channel blocks of MFMAs, from row
    // 0 and the kh = 0 weights already requested.  LDS reads complete in
    // order, so they are issued in the order of first use: the kh = 1 weights
    // and row 1 (used from row group 1 on), then the kh = 2 weights (row group
    // 2).  The following ring slot's first operands are read once this
    // stage's kh = 0 taps are done (row FM) and during its last row.  Those
    // reads are unconditional (reading a slot that is still being filled is
    // harmless, and with no branch around them every LDS wait stays exact);
    // the result is whether that slot's stage had landed before they were
    // issued, from a flag read issued early in the stage, so the stage never
    // blocks on it.
    auto compute_conv = [&]<int PAR>(const unsigned char *buf, const unsigned char *next)
                            __attribute__((always_inline)) {
        bool landed = false;
        int early = 0;
#pragma unroll
        for (int qr = 0; qr < NROW; ++qr) {
            const int cur = (qr + PAR) & 1;
            if (qr + 1 < 3) {
#pragma unroll
                for (int tap = 3 * (qr + 1); tap < 3 * (qr + 2); ++tap)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) fw[tap][fn] = ldB(buf, tap, fn);
            }
            // input row qr feeds output rows fm = qr - kh; the next row is read meanwhile
            if (qr + 1 < NROW) {
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) fx[cur ^ 1][kw] = ldA(buf, qr + 1, kw);
            }
            if (qr == 1) early = landed_count();
            if (qr == NROW - 2) {
                const int f = __builtin_amdgcn_readfirstlane(early);
                seen = f > seen ? f : seen;
                landed = seen > consumed + 1;
#pragma unroll
                for (int tap = 0; tap < 3; ++tap)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) fw[tap][fn] = ldB(next, tap, fn);
            }
            if (qr == NROW - 1) {
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) fx[cur ^ 1][kw] = ldA(next, 0, kw);
            }
            int nm = 0;
#pragma unroll
            for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                for (int kh = 0; kh < 3; ++kh) {
                    const int fm = qr - kh;
                    if (fm < 0 || fm >= FM) continue;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fw[kh * 3 + kw][fn], fx[cur][kw], acc[fm][fn], 0, 0, 0);
                        ++nm;
                    }
                }
            // the row's LDS reads go one after each MFMA (issued as a burst
            // they leave the matrix core idle for a few cycles each)
            const int nr = (qr + 1 < 3 ? 3 * FN : 0) + (qr + 1 < NROW ? 3 : 0) + (qr == 1 ? 1 : 0) +
                           (qr == NROW - 2 ? 3 * FN : 0) + (qr == NROW - 1 ? 3 : 0);
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                if (k < nr && k < nm) {
                    sched_group<kSchedMfma>(1);
                    sched_group<kSchedDsRead>(1);
                }
            }
            if (nr > nm) sched_group<kSchedDsRead>(nr - nm);
            if (nm > nr) sched_group<kSchedMfma>(nm - nr);
            __builtin_amdgcn_sched_barrier(0);
        }
        return landed;
    };

    // The same stage for KH_OUTER tiles: for each kh, the 3 kw x FN weight
    // fragments of that kernel row (in fw[0..2]), then each output row fm
    // with input row fm + kh.  An input row's fragments are read once per
    // stage and kept while a later kernel row still uses them (rows 1 .. FM
    // serve two or three kh): 3 (FM + 2) input reads per stage instead of
    // 9 FM.  With FM = 3 at most three rows are live, so row i sits in
    // fk[i % 3]: row 1 and 2 are read during the rows before their first
    // use, row 3 (into row 0's registers) during kh = 1's first row, row 4
    // during its second, and the following ring slot's row 0 during the
    // stage's last row, which also reads that slot's kh = 0 weights
    // (unconditionally, as in the row-stationary stage).  The weights of
    // kh + 1 replace those of kh, kw by kw, during the last row of kh.
    auto compute_conv_kh = [&]<int PAR>(const unsigned char *buf, const unsigned char *next)
                               __attribute__((always_inline)) {
        static_assert(FM == 3, "three live input rows hold exactly the rows a kernel-row change keeps");
        bool landed = false;
        int early = 0;
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = kh * FM + fm;
                const int row = fm + kh;
                const bool last_row = fm + 1 == FM;
                const bool final_row = kh == 2 && last_row;
                if (r == 1) early = landed_count();
                if (final_row) {
                    const int f = __builtin_amdgcn_readfirstlane(early);
                    seen = f > seen ? f : seen;
                    landed = seen > consumed + 1;
                }
                // input row read during this row: rows 1 and 2 (kh = 0), 3 and 4 (kh = 1), the next slot's row 0
                const int nr = kh == 0 && fm < 2 ? fm + 1 : kh == 1 && fm < 2 ? fm + 3 : final_row ? 0 : -1;
                if (nr >= 0) {
                    const unsigned char *rb = final_row ? next : buf;
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw) fk[nr % 3][kw] = ldA(rb, nr, kw);
                }
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) {
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[kw][fn], fk[row % 3][kw],
                                                                              acc[fm][fn], 0, 0, 0);
                    if (last_row) {
                        const unsigned char *wb = kh < 2 ? buf : next;
                        const int tap = kh < 2 ? (kh + 1) * 3 + kw : kw;
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn) fw[kw][fn] = ldB(wb, tap, fn);
                    }
                }
                // LDS reads one after each MFMA, as in the row-stationary stage
                constexpr int nm = 3 * FN;
                const int nrd = (nr >= 0 ? 3 : 0) + (last_row ? 3 * FN : 0) + (r == 1 ? 1 : 0);
#pragma unroll
                for (int k = 0; k < 9; ++k) {
                    if (k < nrd && k < nm) {
                        sched_group<kSchedMfma>(1);
                        sched_group<kSchedDsRead>(1);
                    }
                }
                if (nrd > nm) sched_group<kSchedDsRead>(nrd - nm);
                if (nm > nrd) sched_group<kSchedMfma>(nm - nrd);
                __builtin_amdgcn_sched_barrier(0);
            }
        return landed;
    };

    // The upsampler stage by phase (PH): output row fm of the wave (input row
    // i = wm FM + fm of the tile) takes row tap a from A row fm + a and
    // column tap b from column l32 + b, with the 4 merged weights of the
    // tile's phase.  Row tap 0 runs first with rows 0 .. FM - 1, while the
    // row tap 1 weights and rows 1 .. FM are read; row tap 1 then reads the
    // following ring slot's tap 0 weights and row 0 (unconditionally, kept
    // if that stage had landed, as in the other stages).
    auto compute_conv_ph = [&]<int PAR>(const unsigned char *buf, const unsigned char *next)
                               __attribute__((always_inline)) {
        bool landed = false;
        int early = 0;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                int nrd = 0;
                if (a == 0) {
                    if (fm == 0) {
                        // every input row of the stage, in the order of use, then the tap 1 weights
#pragma unroll
                        for (int r = 1; r <= FM; ++r)
#pragma unroll
                            for (int b = 0; b < 2; ++b) pr[r][b] = ldA(buf, r, b);
#pragma unroll
                        for (int b = 0; b < 2; ++b)
#pragma unroll
                            for (int fn = 0; fn < FN; ++fn) pw[1][b][fn] = ldB(buf, 2 + b, fn);
                        nrd += 2 * FM + 2 * FN;
                    }
                    if (fm == FM - 1) {
                        // the landed count as late as its read still returns
                        // before the next slot's operands are requested
                        early = landed_count();
                        nrd += TL::NLW;
                    }
                } else if (fm == 0) {
                    const int f = __builtin_amdgcn_readfirstlane(early);
                    seen = f > seen ? f : seen;
                    landed = seen > consumed + 1;
#pragma unroll
                    for (int b = 0; b < 2; ++b) pr[0][b] = ldA(next, 0, b);
#pragma unroll
                    for (int b = 0; b < 2; ++b)
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn) pw[0][b][fn] = ldB(next, b, fn);
                    nrd += 2 + 2 * FN;
                }
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pw[a][b][fn], pr[fm + a][b],
                                                                              acc[fm][fn], 0, 0, 0);
                // LDS reads after the row's first MFMAs, two per MFMA while
                // more are left than MFMAs to follow, then one
                constexpr int nm = 2 * FN;
                int left = nrd;
#pragma unroll
                for (int k = 0; k < nm; ++k) {
                    const int per = left > nm - k - 1 ? (left >= 2 ? 2 : left) : left > 0 ? 1 : 0;
                    sched_group<kSchedMfma>(1);
                    sched_group<kSchedDsRead>(per);
                    left -= per;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        return landed;
    };

    // One shortcut stage: SCS slices of 16 channels, each x at this wave's
    // output rows times that slice of w_sc.
    auto ldU = [&](const unsigned char *buf, int u) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(buf + b_off(u, g)));
    };
    // x fragment of slice j at tile row `row`: position l32, quarter 2j + g
    auto ldX = [&](const unsigned char *buf, int row, int j) __attribute__((always_inline)) {
        if constexpr (TL::SCS == 2) {
            const int q = (2 * j + g) ^ ((l32 >> 2) & 3);
            const int off = ((row * 2 + (l32 >> 4)) * 64 + (l32 & 15) * 4 + q) * 16;
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(buf + off));
        } else {
            return ldU(buf, row * kWB + l32);
        }
    };
    auto compute_shortcut = [&](const unsigned char *buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < TL::SCS; ++j) {
            bf16x8 fw[FN];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                fw[fn] = ldU(buf, TL::SC_W_UNIT0 + j * NB + wn * FN * 32 + fn * 32 + l32);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const bf16x8 fx = ldX(buf, wm * FM + fm, j);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[fn], fx, acc[fm][fn], 0, 0, 0);
            }
        }
    };

    // stage consumed: its reads were issued (and, LDS being in order, execute)
    // before this flag write
    auto release = [&]() __attribute__((always_inline)) {
        compiler_fence();
        ++consumed;
        if (lane == 0) flag_write(1 + wave, consumed);
        slot = slot + 1 == NBUF ? 0 : slot + 1;
    };

    // tile sub of local item i, in the load wave's order
    for (int64_t i = loc, sub = 0; i < x_count;) {
        const TileInfo ti = decode(x_begin + i, (int)sub);
        if (++sub == ti.ntiles) {
            sub = 0;
            i += wg_x;
        }

        // A tile's first stage reads its own operands: marking the carried
        // ones undefined here keeps them from being held across the epilogue
        // (which the KH_OUTER tiles' identity epilogue has no registers for).
        if constexpr (PH) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                pr[0][b] = __builtin_nondeterministic_value(pr[0][b]);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) pw[0][b][fn] = __builtin_nondeterministic_value(pw[0][b][fn]);
            }
        }
        if constexpr (TL::KH_OUTER) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                fk[0][j] = __builtin_nondeterministic_value(fk[0][j]);
                fk[1][j] = __builtin_nondeterministic_value(fk[1][j]);
                fk[2][j] = __builtin_nondeterministic_value(fk[2][j]);
            }
#pragma unroll
            for (int tap = 0; tap < 3; ++tap)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) fw[tap][fn] = __builtin_nondeterministic_value(fw[tap][fn]);
        }

        // the accumulators start at the bias (+ shortcut bias) of their
        // channels: accumulator element 4j + q of channel block fn is
        // channel 8j + 4g + q of the block
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            floatx16 b0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 bv =
                    *reinterpret_cast<const float4 *>(bias_lds + ti.n0 + wn * FN * 32 + fn * 32 + 8 * j + 4 * g);
                b0[4 * j] = bv.x;
                b0[4 * j + 1] = bv.y;
                b0[4 * j + 2] = bv.z;
                b0[4 * j + 3] = bv.w;
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fm][fn] = b0;
        }

        {
            // Stages run in pairs of parity 0 and 1 (straight-line code, so
            // both use the same registers), a tile's first stage with parity
            // 0.  The next stage's operands are kept when it is a conv stage
            // of this tile and had landed; kernels with shortcut stages read
            // every stage's first operands at its start.
            bool preloaded = false;
            auto stage = [&]<int PAR>(bool more) __attribute__((always_inline)) {
                const unsigned char *cur = smem + slot * TL::STAGE_BYTES;
                if (!preloaded) {
                    wait_landed();
                    load_first(cur, PAR);
                }
                const unsigned char *nxt = smem + (slot + 1 == NBUF ? 0 : slot + 1) * TL::STAGE_BYTES;
                bool landed;
                if constexpr (PH)
                    landed = compute_conv_ph.template operator()<PAR>(cur, nxt);
                else if constexpr (TL::KH_OUTER)
                    landed = compute_conv_kh.template operator()<PAR>(cur, nxt);
                else
                    landed = compute_conv.template operator()<PAR>(cur, nxt);
                preloaded = !SC && more && landed;
                release();
            };
            int s = 0;
            for (; s + 2 <= ti.s_conv; s += 2) {
                stage.template operator()<0>(true);
                stage.template operator()<ALT ? 1 : 0>(s + 2 < ti.s_conv);
            }
            if (s < ti.s_conv) stage.template operator()<0>(false);
        }
        if constexpr (SC) {
            for (int s = ti.s_conv; s < ti.s_total; ++s) {
                wait_landed();
                compute_shortcut(smem + slot * TL::STAGE_BYTES);
                release();
            }
        }

        // ---- epilogue: lane owns position (row, w0 + l32) and channels
        // 8j + 4g + [0,4) of each channel block.  The load wave is meanwhile
        // already filling the ring with the next tile's first stages.
        // Branch-free: residual loads and output stores are raw buffer
        // accesses over this frame, and a position outside the image gets an
        // out-of-range offset (its load returns zero, its store is dropped).
        // The identity residual is fetched in row groups (two rows, or one
        // with 96-channel tiles), one group ahead of the stores, with exact
        // vmcnt waits, in the stores' whole-line layout.
        const int64_t frame = ti.nq * a.T + ti.tq;
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y + frame * HW * a.cout, HW * a.cout * 2);
        // store pieces: position p = lane / 4 + 16 half, 16-byte quarter lane % 4
        // (PH: tile positions are the input's; output column 2 w + px, row 2 h + py)
        uint32_t col_off[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int ww = ti.w0 + (lane >> 2) + 16 * half;
            const int wo = PH ? 2 * ww + (ti.ph & 1) : ww;
            col_off[half] = ww < (PH ? W >> 1 : W)
                                ? (uint32_t)(wo * a.cout + ti.n0 + wn * FN * 32) * 2 + (lane & 3) * 16
                                : kOOB;
        }
        // A row of results goes out through this wave's LDS staging buffer:
        // written as the MFMA layout holds it (lane = position, 4 channels per
        // accumulator quad), read back as 16 bytes per lane with 4 lanes per
        // position, and stored as 64 contiguous bytes per position, so a store
        // touches 16 cache lines instead of 32 and there are half as many.
        unsigned char *const epi = epi_stage + wave * kEpiBytes;
        // A tile whose channel block runs past C_out (C_out not a multiple of
        // 32), or whose rows are not 16-byte aligned (C_out % 8 != 0), stores
        // each valid output channel by itself instead.  Only the 32-channel
        // tile with a bias epilogue meets such C_out (the others need
        // multiples of 64 or 96, the residual epilogues multiples of 32).
        constexpr bool CAN_NARROW = EPI == EPI_BIAS && NB == 32;
        const bool narrow = CAN_NARROW && ((a.cout & 7) != 0 || ti.n0 + NB > a.cout);
        // res: the residual of these rows as loaded, in the store layout
        // (16 bytes per lane, per row, channel block and half); it goes
        // through the staging buffer into the accumulator layout.
        auto store_rows = [&](int f0, int nrows, const u32x4 (*res)[FN][2]) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < nrows; ++e) {
                const int hh = ti.h0 + wm * FM + f0 + e;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    if (res != nullptr) {
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int p = (lane >> 2) + 16 * half, qq = lane & 3;
                            *reinterpret_cast<u32x4 *>(epi + p * kEpiStride + qq * 16) = res[e][fn][half];
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float v[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = acc[f0 + e][fn][4 * j + q];
                        if (res != nullptr) {
                            const u32x2 r = *reinterpret_cast<const u32x2 *>(epi + l32 * kEpiStride + j * 16 + g * 8);
                            v[0] += bf16_bits_to_f32(r.x & 0xffffu);
                            v[1] += bf16_bits_to_f32(r.x >> 16);
                            v[2] += bf16_bits_to_f32(r.y & 0xffffu);
                            v[3] += bf16_bits_to_f32(r.y >> 16);
                        }
                        if (narrow) {
                            const int ww = ti.w0 + l32;
                            const int c0 = ti.n0 + wn * FN * 32 + fn * 32 + 8 * j + 4 * g;
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (hh < H && ww < W && c0 + q < a.cout)
                                    __builtin_amdgcn_raw_buffer_store_b16(
                                        (unsigned short)f32_to_bf16_bits(v[q]), ry,
                                        (uint32_t)((hh * W + ww) * a.cout + c0 + q) * 2, 0, 0);
                            continue;
                        }
                        const u32x2 o = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *reinterpret_cast<u32x2 *>(epi + l32 * kEpiStride + j * 16 + g * 8) = o;
                    }
                    if (narrow) continue;
                    const int ho = PH ? 2 * hh + (ti.ph >> 1) : hh;
                    const bool row_in = hh < (PH ? H >> 1 : H);
                    const uint32_t row_off = (uint32_t)(ho * W * a.cout) * 2 + fn * 64;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int p = (lane >> 2) + 16 * half, q = lane & 3;
                        const u32x4 d = *reinterpret_cast<const u32x4 *>(epi + p * kEpiStride + q * 16);
                        const uint32_t off = row_in && col_off[half] != kOOB ? row_off + col_off[half] : kOOB;
                        __builtin_amdgcn_raw_buffer_store_b128(d, ry, off, 0, 0);
                    }
                }
            }
        };
        if constexpr (EPI == EPI_IDENTITY) {
            constexpr int EG = FN > 1 ? 1 : 2;             // rows per residual group (registers)
            constexpr int NG = (FM + EG - 1) / EG;
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.res + frame * HW * a.cres, HW * a.cres * 2);
            // residual pieces as the stores write them: position
            // lane / 4 + 16 half, 16-byte quarter lane % 4 (64 contiguous
            // bytes per position and channel block)
            u32x4 rv[2][EG][FN][2];
            uint32_t rcol[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int ww = ti.w0 + (lane >> 2) + 16 * half;
                rcol[half] = ww < W ? (uint32_t)(ww * a.cres + ti.n0 + wn * FN * 32) * 2 + (lane & 3) * 16 : kOOB;
            }
            auto load_group = [&](int gi) __attribute__((always_inline)) {
#pragma unroll
                for (int e = 0; e < group_rows<FM, EG>(gi); ++e) {
                    const int hh = ti.h0 + wm * FM + gi * EG + e;
                    const uint32_t rrow = (uint32_t)(hh * W * a.cres) * 2;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const uint32_t off = hh < H && rcol[half] != kOOB ? rrow + fn * 64 + rcol[half] : kOOB;
                            rv[gi & 1][e][fn][half] = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0);
                        }
                }
            };
            load_group(0);
            if (NG > 1) load_group(1);
            // group GI has landed once at most the VMEM operations issued
            // after its loads are outstanding: the stores of group GI - 1 and
            // the loads of group GI + 1 (2 each per row and channel block); an
            // immediate, hence the template
            auto step = [&]<int GI>() __attribute__((always_inline)) {
                constexpr int kAfter = (GI >= 1 ? group_rows<FM, EG>(GI - 1) * FN * 2 : 0) +
                                       (GI + 1 < NG ? group_rows<FM, EG>(GI + 1) * FN * 2 : 0);
                static_assert(kAfter <= 63, "vmcnt counts to 63");
                compiler_fence();
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAfter));
                compiler_fence();
                store_rows(GI * EG, group_rows<FM, EG>(GI), rv[GI & 1]);
                if (GI + 2 < NG) load_group(GI + 2);
            };
            [&]<int... GI>(std::integer_sequence<int, GI...>) {
                (step.template operator()<GI>(), ...);
            }(std::make_integer_sequence<int, NG>{});
        } else if constexpr (EPI == EPI_NORM) {
            // norm2 + SiLU of each output position from the fp32 accumulators
            // (bias included): the lane holds 16 of every 32-channel block's
            // channels (8j + 4g + q), its partner lane ^ 32 the other 16, so
            // the sum of squares takes one exchange.  n2 goes out in the
            // 16-channel-slice layout: through the staging buffer, each slice
            // of a row is one 1 KB run (32 positions x 32 bytes), a lane
            // storing half of one position's unit.
            const float *gs = bias_lds + a.cout_p;        // gamma * sqrt(C)
            const float *gb = bias_lds + 2 * a.cout_p;    // beta
            const int p2 = lane >> 1, h2 = lane & 1;     // read-back: position, half unit
            const int ww2 = ti.w0 + p2;
#pragma unroll
            for (int e = 0; e < FM; ++e) {
                const int hh = ti.h0 + wm * FM + e;
                float ss = 0.0f;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int k = 0; k < 16; ++k) ss = fmaf(acc[e][fn][k], acc[e][fn][k], ss);
                ss = halves_sum(ss);
                const float inv = 1.0f / fmaxf(sqrtf(ss), a.neps);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c0 = fn * 32 + 8 * j + 4 * g;
                        const float4 gv = *reinterpret_cast<const float4 *>(gs + c0);
                        const float4 bv = *reinterpret_cast<const float4 *>(gb + c0);
                        const float v0 = silu(fmaf(acc[e][fn][4 * j] * inv, gv.x, bv.x));
                        const float v1 = silu(fmaf(acc[e][fn][4 * j + 1] * inv, gv.y, bv.y));
                        const float v2 = silu(fmaf(acc[e][fn][4 * j + 2] * inv, gv.z, bv.z));
                        const float v3 = silu(fmaf(acc[e][fn][4 * j + 3] * inv, gv.w, bv.w));
                        *reinterpret_cast<u32x2 *>(epi + l32 * kEpiStride + j * 16 + g * 8) =
                            u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    }
                    // slice (2 fn + sl) of this row: position p2, bytes 16 h2 .. + 15
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl) {
                        const u32x4 d = *reinterpret_cast<const u32x4 *>(epi + p2 * kEpiStride + sl * 32 + h2 * 16);
                        const uint32_t off = hh < H && ww2 < W
                            ? (uint32_t)(((int64_t)(2 * fn + sl) * HW + hh * W + ww2) * kUnit) + h2 * 16
                            : kOOB;
                        __builtin_amdgcn_raw_buffer_store_b128(d, ry, off, 0, 0);
                    }
                    // one channel block's scales in registers at a time
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            store_rows(0, FM, nullptr);
        }
    }
}

}  // namespace

namespace {
std::atomic<int> g_spin_cap{kSpinCapDefault};
}  // namespace

void set_wait_bound(int polls) { g_spin_cap.store(polls < 0 ? kSpinCapDefault : polls, std::memory_order_relaxed); }

hipError_t read_wait_giveups(uint64_t *count) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    unsigned int v = 0;
    e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_wait_giveups), sizeof v, 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess) *count = v;
    return e;
}

hipError_t reset_wait_giveups() {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    const unsigned int zero = 0;
    return hipMemcpyToSymbol(HIP_SYMBOL(g_wait_giveups), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
}

// Compute units of the current device (cached per device; also used by the
// other persistent kernels).
hipError_t device_cu_count(int *out) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) {
            *out = v;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return hipSuccess;
}

namespace {

template <int WM, int WN, int FM, int FN, int EPI, bool SC = EPI == EPI_SHORTCUT, bool PH = false>
hipError_t launch_cfg(const ConvLaunch &c, hipStream_t s) {
    using TL = Tile<WM, WN, FM, FN, PH>;
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
    a.cout_p = (c.cout + 31) / 32 * 32;
    a.cres = c.cres;
    a.x_sliced = c.x_sliced ? 1 : 0;
    a.gemm = c.gemm ? 1 : 0;
    a.up2 = c.up2 ? 1 : 0;
    a.up_t = c.up2 && c.up_t ? 1 : 0;
    a.xT = a.up_t ? (c.t + 1) / 2 : c.t;
    a.spin_cap = g_spin_cap.load(std::memory_order_relaxed);
    a.ngamma = c.norm_gamma;
    a.nbeta = c.norm_beta;
    a.neps = c.norm_eps;
    a.sc_in = static_cast<const uint16_t *>(c.gemm ? c.x : c.res);
    a.sc_c = c.gemm ? c.cin : c.cres;
    if (c.gemm) a.wsc = static_cast<const uint16_t *>(c.w);
    // (PH: tiles over the half-resolution input, four phases each)
    const int64_t th = PH ? c.h / 2 : c.h, tw = PH ? c.w_ / 2 : c.w_;
    a.tiles_w = (int)((tw + kWB - 1) / kWB);
    a.tiles_h = (int)((th + TL::HB - 1) / TL::HB);
    a.pair = c.cache == nullptr && !c.up2 && !c.gemm && c.t >= 2 ? 1 : 0;
    a.items = (int64_t)a.tiles_w * a.tiles_h * c.n * (c.t - a.pair) * (a.cout_p / TL::NB) * (PH ? 4 : 1);
    if (a.items <= 0) return hipSuccess;
    if (a.items >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // the decode's 31-bit item indices
    // Super-blocks of 20 frame groups where one channel block spans every
    // output channel (c4's 96-channel tiles): an XCD's 32 workgroups then run
    // neighbouring column blocks of the same frames together as well as
    // neighbouring frames, and the tiles' column halos are read from L2.
    // Where several channel blocks share a frame (C_out 192, 384), and for
    // the upsampler by phase (four phase tiles per block already), the frame
    // groups stay undivided: measured neutral to slightly slower there.
    const int ngroups = (int)(c.t - a.pair), ncb = a.cout_p / TL::NB;
    a.sbg = ncb == 1 && !PH ? (ngroups < kSuperBlock ? ngroups : kSuperBlock) : ngroups;
    const int nsb = (ngroups + a.sbg - 1) / a.sbg;
    a.region = ngroups * a.tiles_w;
    a.sb_gw = a.sbg * a.tiles_w;
    a.sb_full = (nsb - 1) * a.sb_gw;
    a.sb_last0 = (nsb - 1) * a.sbg;
    a.sb_r = ngroups - a.sb_last0;
    a.div.shifts[0] = a.div.shifts[1] = 0;
    set_fastdiv(a.div, 0, (uint32_t)ncb);
    set_fastdiv(a.div, 1, (uint32_t)a.region);
    set_fastdiv(a.div, 2, (uint32_t)a.sb_gw);
    set_fastdiv(a.div, 3, (uint32_t)a.tiles_h);
    set_fastdiv(a.div, 4, (uint32_t)a.sbg);
    set_fastdiv(a.div, 5, (uint32_t)a.sb_r);
    // persistent grid: one workgroup per compute unit (the LDS ring takes most
    // of a CU's 160 KB), each looping over its share of the tiles
    int ncu = 0;
    const hipError_t e = device_cu_count(&ncu);
    if (e != hipSuccess) return e;
    const int64_t grid = a.items < (int64_t)ncu * TL::kPerCU ? a.items : (int64_t)ncu * TL::kPerCU;
    conv3d_bf16_kernel<WM, WN, FM, FN, EPI, SC, PH><<<dim3((unsigned)grid), dim3(TL::kThreads), 0, s>>>(a);
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
    return cin >= 16 && cin <= 1024 && cin % 16 == 0 && cout >= 1 && cout <= 1024;
}

// The norm epilogue needs one channel block per tile (WN = 1): the
// 96-channel kh-outer tile or the 32-channel one.
bool conv3d_bf16_norm_supported(int cout) { return cout == 96 || cout == 32; }

// Rows a tile height computes for an image height (the last tile is padded).
int64_t rows_computed(int64_t h, int hb) { return (h + hb - 1) / hb * hb; }

// A launch too small for the large tiles to fill the chip evenly (a one-frame
// stream step: 300 tiles of 18 x 32 x 64 on 256 compute units run as two
// rounds, the second a sixth full) runs on the 32-channel tile instead when
// its rounds cost less: the large tiles' rounds times their outputs, against
// the small ones' times theirs and the small tile's higher cost per output
// (measured 1.4x: more weight reads per MFMA).  Full-T launches have many
// rounds and keep the large tiles.
bool prefer_small_tiles(const ConvLaunch &c, bool tall) {
    if (c.res != nullptr && c.wsc != nullptr) return false;   // the shortcut stages are sized per tile
    int ncu = 0;
    if (device_cu_count(&ncu) != hipSuccess || ncu <= 0) return false;
    const bool pair = c.cache == nullptr && c.t >= 2;
    const int64_t frames = c.n * (c.t - (pair ? 1 : 0));
    const int64_t tw = (c.w_ + kWB - 1) / kWB;
    auto rounds = [&](int hb, int nb) {
        const int64_t items = tw * ((c.h + hb - 1) / hb) * frames * (((c.cout + 31) / 32 * 32) / nb);
        return (items + ncu - 1) / ncu;
    };
    const int hb = c.cout % 64 == 0 ? (tall ? 18 : 16) : 12, nb = c.cout % 64 == 0 ? 64 : 96;
    const double big = (double)rounds(hb, nb) * hb * nb;
    const double small = 1.4 * (double)rounds(16, 32) * 16 * 32;
    return small < big;
}

// Tile choice (measured on the workload shapes):
//  - C_out a multiple of 64: a 2 x 2 grid of MFMA waves, each 8 or 9 rows x 32
//    columns x 32 channels (128 or 144 accumulators), plus the load wave.  The
//    18-row tile is taken unless it pads more rows than the 16-row one (every
//    decoder resolution, 90 x 160 up to 720 x 1280, is a multiple of 18 rows).
//  - other multiples of 96: four MFMA waves of 3 rows x 96 channels (one wave
//    per SIMD; a 2 x 3 grid of 32-channel waves puts two waves on two of the
//    four SIMDs and one on the others, and measured 7% slower).
//  - any other C_out: four waves of 4 rows x 32 channels, the last channel
//    block padded with zero weights (the decoder's 3-channel conv_out).
hipError_t launch_conv3d_bf16(const ConvLaunch &c, hipStream_t s) {
    if (c.cout < 1 || c.cout > 1024) return hipErrorInvalidValue;
    if (c.norm_out) {
        // one channel block per tile: the 96-channel kh-outer tile, or the
        // 32-channel one
        if (c.res != nullptr || c.norm_gamma == nullptr || c.up2 || c.gemm) return hipErrorInvalidValue;
        if (c.cout == 96) return launch_cfg<4, 1, 3, 3, EPI_NORM>(c, s);
        if (c.cout == 32) return launch_cfg<4, 1, 4, 1, EPI_NORM>(c, s);
        return hipErrorInvalidValue;
    }
    if (c.up2 && upsample_by_phase(c.cout)) {
        if (c.res != nullptr || c.cache != nullptr || (c.h | c.w_) & 1) return hipErrorInvalidValue;
        return launch_cfg<4, 1, 3, 3, EPI_BIAS, false, true>(c, s);
    }
    const bool tall = rows_computed(c.h, 18) <= rows_computed(c.h, 16);
    if (c.res != nullptr && c.wsc != nullptr) {
        if (c.cout % 64 == 0)
            return tall ? launch_cfg<2, 2, 9, 1, EPI_SHORTCUT>(c, s) : launch_cfg<2, 2, 8, 1, EPI_SHORTCUT>(c, s);
        if (c.cout % 96 == 0) return launch_cfg<4, 1, 3, 3, EPI_SHORTCUT>(c, s);
        return launch_cfg<4, 1, 4, 1, EPI_SHORTCUT>(c, s);
    }
    if ((c.cout % 64 == 0 || c.cout % 96 == 0) && prefer_small_tiles(c, tall)) return launch_plain<4, 1, 4, 1>(c, s);
    if (c.cout % 64 == 0) return tall ? launch_plain<2, 2, 9, 1>(c, s) : launch_plain<2, 2, 8, 1>(c, s);
    if (c.cout % 96 == 0) return launch_plain<4, 1, 3, 3>(c, s);
    return launch_plain<4, 1, 4, 1>(c, s);
}

// The same kernels with only 1x1x1 stages: y = w x + bias (+ res), the plain
// channel GEMM of a pointwise projection, tiled like the conv.
template <int WM, int WN, int FM, int FN>
hipError_t launch_gemm_cfg(const ConvLaunch &c, hipStream_t s) {
    return c.res ? launch_cfg<WM, WN, FM, FN, EPI_IDENTITY, true>(c, s)
                 : launch_cfg<WM, WN, FM, FN, EPI_BIAS, true>(c, s);
}

hipError_t launch_gemm_bf16(const ConvLaunch &c, hipStream_t s) {
    // the bias of every output channel must fit the kernel's LDS copy; the 1x1x1
    // stages take 32 input channels at a time
    if (!c.gemm || c.cout < 1 || c.cout > 2048 || c.cin < 32 || c.cin % 32 != 0) return hipErrorInvalidValue;
    const bool tall = rows_computed(c.h, 18) <= rows_computed(c.h, 16);
    if (c.cout % 64 == 0) return tall ? launch_gemm_cfg<2, 2, 9, 1>(c, s) : launch_gemm_cfg<2, 2, 8, 1>(c, s);
    if (c.cout % 96 == 0) return launch_gemm_cfg<4, 1, 3, 3>(c, s);
    return launch_gemm_cfg<4, 1, 4, 1>(c, s);
}

}  // namespace wanvae
