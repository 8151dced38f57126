// Pointwise projection as a plain channel GEMM on MFMA:
//   y[p][n] = sum_k x[p][k] w[n][k] + bias[n] (+ res[p][n])
// x [P][K], w [N][K], res and y [P][N], all bf16 channels-last; fp32
// accumulation, bias and residual added in fp32, one RNE rounding.  These are
// the 1x1x1 projections around the decoder's mid-block attention (q, k and v
// from the normed input, C -> 3C, and the output projection with the residual,
// C -> C; "Closing the gap: Wan 2.2 14B VAE decoder", section 5, and
// "Sharding of WAN 2.2 VAE", decoder module tree), and the 1x1x1 shortcut of a
// channel-changing ResidualBlock.
//
// A workgroup owns 256 positions and all N output channels; its four waves
// (one per SIMD) own 64 positions each and keep their x rows for the whole K
// (K <= 384) in registers, as MFMA B operands: x comes from HBM exactly once
// and never passes through LDS.  The weight (small, L2-resident) streams
// through LDS in stages of 128 output channels x 128 k (32 KB), moved by
// LDS-DMA (buffer_load ... lds, 1 KB per instruction, each wave a quarter of
// every stage), in a ring of 4 slots loaded 3 stages ahead; the weight stream
// does not depend on the positions, so it runs on across tiles.  Per stage a
// wave runs 4 channel blocks x 2 position blocks x 8 k-steps of
// v_mfma_f32_32x32x16_bf16 (weights as the A operand, channels as M), each
// weight fragment read from LDS once for two MFMAs.  A lane ends up holding 4
// consecutive output channels of one position per 4 accumulators and stores
// them as one 8-byte piece.  The accumulators start at the bias.  The next
// tile's x is loaded k-slice by k-slice as the last output-channel chunk of
// the current tile finishes with each slice.  Weight rows are swizzled in
// 16-byte chunks (chunk ^ (row & 15)) so that fragment reads hit distinct
// banks.  The grid is persistent, one workgroup per CU, each XCD a contiguous
// range of tiles.
//
// Waits on the weight stages are exact: vector-memory operations complete in
// issue order, so "stage s has landed" is "at most the operations issued
// after its loads are outstanding"; each wave counts what it issues (weight
// loads, x loads, residual loads, stores) and waits for that count.
#include <type_traits>
#include <utility>

#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;                       // positions per tile
constexpr int kBN = 128;                       // output channels per chunk
constexpr int kBK = 128;                       // K per weight stage
constexpr int kKMax = 384;                     // x of 64 positions in registers: K <= 384
constexpr int kRowBytes = kBK * 2;             // 256 bytes of a weight row per stage
constexpr int kPart = kBN * kRowBytes;         // 32 KB: one weight stage
constexpr int kNBuf = 4;                       // weight ring slots
constexpr int kNMax = 2048;                    // output channels (the bias is kept in LDS)
constexpr int kAhead = 3;                      // stages loaded ahead
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kWBlocksPerWave = kPart / 1024 / kWaves;   // 8
constexpr int kXCD = 8;
// The epilogue goes through LDS: per wave, 32 positions x 64 channels of
// bf16 at a time (rows kStageRow bytes apart), read back as 8 lanes x 16
// bytes per position, so a store writes 8 whole 128-byte rows (and a residual
// is loaded the same way).
constexpr int kStageRow = 144;
constexpr int kStagedStores = 2 * 2 * 4;       // stores (and residual loads) per lane in an epilogue
constexpr int kBufFlags = 0x00020000;          // raw buffer: loads past num_records return zeros
constexpr uint32_t kOOB = 0x80000000u;
static_assert(kNBuf * kPart + kNMax * 4 + kWaves * 32 * kStageRow <= 160 * 1024, "LDS");
static_assert(kAhead < kNBuf, "a slot is refilled only after the stage it held was consumed");

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }

__device__ inline i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)),
                 __builtin_amdgcn_readfirstlane((int)bytes), kBufFlags};
}

// one wavefront-wide 16-byte-per-lane load into LDS at lds_addr + 16 * lane
__device__ inline void lds_dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane((int)lds_addr)), "v"(voff), "s"(rsrc)
                 : "memory");
}

// the same resource as a typed value for the buffer load/store builtins
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(u), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), kBufFlags);
}

__device__ inline uint32_t lds_address(const unsigned char *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt for "at most n vector-memory operations outstanding", n known only
// at run time (the instruction takes an immediate): n is rounded down to a
// multiple of 8 (at most 56), which only waits longer
__device__ inline void wait_vm_at_most(int n) {
    if (n >= 32) {
        if (n >= 48) {
            if (n >= 56) __builtin_amdgcn_s_waitcnt(waitcnt_vm(56));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(48));
        } else {
            if (n >= 40) __builtin_amdgcn_s_waitcnt(waitcnt_vm(40));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(32));
        }
    } else {
        if (n >= 16) {
            if (n >= 24) __builtin_amdgcn_s_waitcnt(waitcnt_vm(24));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));
        } else {
            if (n >= 8) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
    }
}

template <int K, bool RES, bool ONE_CHUNK>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ w,
                                                             const float *__restrict__ bias,
                                                             const uint16_t *__restrict__ res,
                                                             uint16_t *__restrict__ y, int64_t P, int N,
                                                             int64_t mtiles) {
    constexpr int KS = K / 16;   // MFMA k-steps
    constexpr int S = K / kBK;   // weight stages per output-channel chunk
    static_assert(K % kBK == 0 && K <= kKMax, "K");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kNBuf * kPart];
    // the bias of every output channel, read from LDS: a vector-memory load
    // of it would make the compiler wait for every load in flight (it does
    // not see the weight loads, which are inline assembly)
    __shared__ __attribute__((aligned(16))) float bias_lds[kNMax];
    __shared__ __attribute__((aligned(16))) unsigned char ostage[kWaves * 32 * kStageRow];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int nchunks = ONE_CHUNK ? 1 : (N + kBN - 1) / kBN;   // the last may be 64 wide

    // ---- this workgroup's position tiles: XCD x (= workgroup index mod 8)
    // owns a contiguous range, its workgroups take them round-robin
    const int64_t nwg = gridDim.x, bid = blockIdx.x;
    const int64_t xcd = bid % kXCD, loc = bid / kXCD;
    const int64_t wg_x = nwg / kXCD + (xcd < nwg % kXCD ? 1 : 0);
    const int64_t wg_before = xcd * (nwg / kXCD) + (xcd < nwg % kXCD ? xcd : nwg % kXCD);
    const int64_t x_begin = mtiles * wg_before / nwg;
    const int64_t x_count = mtiles * (wg_before + wg_x) / nwg - x_begin;
    const int64_t my_tiles = x_count > loc ? (x_count - loc + wg_x - 1) / wg_x : 0;
    if (my_tiles == 0) return;   // uniform over the workgroup: no barrier is left waiting
    for (int c = tid; c < N; c += kThreads) bias_lds[c] = bias != nullptr ? bias[c] : 0.0f;
    __syncthreads();
    const int per_tile = nchunks * S;            // weight stages per tile
    const int64_t total = my_tiles * per_tile;   // weight stages of this workgroup
    auto tile_m0 = [&](int64_t it) __attribute__((always_inline)) { return (x_begin + loc + it * wg_x) * kBM; };

    int issued = 0;   // vector-memory operations this wave has issued (they complete in order)

    // ---- weight stage gst (chunk nc, k stage kq, the same for every tile):
    // 32 blocks of 1 KB, 8 per wave; block b holds rows 4b .. 4b + 3 of the
    // 128 channels, lane row 4b + l / 16, stored chunk l % 16
    const uint32_t lds_base = lds_address(lds);
    // lane offset of block i (computed at each issue: eight live registers
    // fewer beside the x fragments)
    auto w_off = [&](int i) __attribute__((always_inline)) {
        const int row = 4 * (wave * kWBlocksPerWave + i) + (lane >> 4), cs = lane & 15;
        return (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)((cs ^ (row & 15)) * 16);
    };
    // source and LDS destination of stage gst's loads; past the last stage
    // the buffer is empty (its loads write zeros into a slot already consumed)
    struct WLoad {
        i32x4 r;
        uint32_t dst;
    };
    auto w_load = [&](int64_t gst) __attribute__((always_inline)) {
        const int st = (int)(gst % per_tile);
        const int nc = st / S, kk = (st % S) * kBK;
        // channels past N (a 64-wide last chunk) fall beyond the buffer's end: zeros
        const int rows = N - nc * kBN < kBN ? N - nc * kBN : kBN;
        const uint32_t bytes = gst < total ? (uint32_t)(rows * K * 2 - kk * 2) : 0u;
        return WLoad{buffer_rsrc(w + (int64_t)nc * kBN * K + kk, bytes),
                     lds_base + (uint32_t)((int)(gst % kNBuf) * kPart + wave * kWBlocksPerWave * 1024)};
    };
    auto issue_w = [&](int64_t gst) __attribute__((always_inline)) {
        const WLoad l = w_load(gst);
#pragma unroll
        for (int i = 0; i < kWBlocksPerWave; ++i) lds_dma16(l.r, l.dst + i * 1024, w_off(i));
        issued += kWBlocksPerWave;
    };

    // ---- x of this wave's 64 positions: fragment (k-step ks, position block
    // jn) = x[m0 + 64 wave + 32 jn + l32][16 ks + 8 g .. + 7], one 16-byte
    // load; positions past P read zeros
    bf16x8 xf[KS][2];
    auto load_x = [&](int64_t m0, int ks0, int ks1) __attribute__((always_inline)) {
        const int64_t rows = P - m0 < kBM ? P - m0 : kBM;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + m0 * K, (uint32_t)(rows * K * 2));
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int pl = wave * 64 + 32 * jn + l32;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks < ks0 || ks >= ks1) continue;
                const uint32_t off = pl < rows ? (uint32_t)(pl * K * 2 + ks * 32 + g * 16) : kOOB;
                xf[ks][jn] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
            }
        }
        issued += 2 * (ks1 - ks0);
    };

    floatx16 acc[4][2];
    // the accumulators start at the bias: element 4 jj + q of channel block i
    // is channel n0 + 32 i + 8 jj + 4 g + q
    auto init_acc = [&](int n0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            floatx16 b0;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c = n0 + 32 * i + 8 * jj + 4 * g;
                const float4 bv =
                    c < N ? *reinterpret_cast<const float4 *>(bias_lds + c) : float4{0.0f, 0.0f, 0.0f, 0.0f};
                b0[4 * jj] = bv.x;
                b0[4 * jj + 1] = bv.y;
                b0[4 * jj + 2] = bv.z;
                b0[4 * jj + 3] = bv.w;
            }
            acc[i][0] = b0;
            acc[i][1] = b0;
        }
    };
    // ---- epilogue of chunk n0.  Accumulator element 4 jj + q of (channel
    // block i, position block jn) is channel n0 + 32 i + 8 jj + 4 g + q of
    // position m0 + 64 wave + 32 jn + l32.  The number of vector-memory
    // operations per lane is fixed whatever the tile: positions past P and
    // channels past N get an offset beyond the buffer's end (the load returns
    // zeros, the store is dropped).
    auto store = [&](int64_t m0, int n0) __attribute__((always_inline)) {
        const int64_t rows = P - m0 < kBM ? P - m0 : kBM;
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + m0 * N, (uint32_t)(rows * N * 2));
        // Through this wave's LDS staging rows, 32 positions x 64 channels
        // (channel half h of the chunk) at a time: written in the
        // accumulator layout, stored as 16 bytes per lane, 128 contiguous
        // bytes per position.  A residual is loaded in that store layout,
        // all of it before the first store (a load behind a store would wait
        // for it), and reaches the accumulator layout through the same rows,
        // so the output keeps its single rounding.  The lane index is made
        // opaque so that the addresses are computed in place instead of being
        // hoisted out of the stage loop into registers that the x fragments
        // need.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lq = ln & 31, gq = ln >> 5;
        unsigned char *stg = ostage + wave * 32 * kStageRow;
        // piece r of (position block jn, channel half h): position (ln >> 3) + 8 r, 16-byte part ln & 7
        auto piece_off = [&](int jn, int h, int r) __attribute__((always_inline)) -> uint32_t {
            const int pl = wave * 64 + 32 * jn + (ln >> 3) + 8 * r;
            return pl < rows && n0 + 64 * h < N ? (uint32_t)((pl * N + n0 + 64 * h + 8 * (ln & 7)) * 2) : kOOB;
        };
        [[maybe_unused]] u32x4 rq[RES ? 2 : 1][2][4];
        if constexpr (RES) {
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(res + m0 * N, (uint32_t)(rows * N * 2));
#pragma unroll
            for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        rq[jn][h][r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, piece_off(jn, h, r), 0, 0));
            issued += kStagedStores;   // as many loads as stores
        }
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (RES) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<u32x4 *>(stg + ((ln >> 3) + 8 * r) * kStageRow + (ln & 7) * 16) = rq[jn][h][r];
                }
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const floatx16 &a = acc[2 * h + i2][jn];
                        u32x2 *slot = reinterpret_cast<u32x2 *>(stg + lq * kStageRow + (32 * i2 + 8 * jj + 4 * gq) * 2);
                        float v0 = a[4 * jj], v1 = a[4 * jj + 1], v2 = a[4 * jj + 2], v3 = a[4 * jj + 3];
                        if constexpr (RES) {
                            const u32x2 rv = *slot;
                            v0 += bf16_bits_to_f32(rv.x & 0xffffu);
                            v1 += bf16_bits_to_f32(rv.x >> 16);
                            v2 += bf16_bits_to_f32(rv.y & 0xffffu);
                            v3 += bf16_bits_to_f32(rv.y >> 16);
                        }
                        *slot = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + ((ln >> 3) + 8 * r) * kStageRow + (ln & 7) * 16);
                    __builtin_amdgcn_raw_buffer_store_b128(v, ry, piece_off(jn, h, r), 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);   // one unit's values live at a time
            }
        issued += kStagedStores;
    };

    // weight fragment: row `row` of a stage, k-step ks (k = 16 ks + 8 g .. +7)
    auto wfrag = [&](const unsigned char *ws, int row, int ks) __attribute__((always_inline)) {
        const int c = (2 * ks + g) ^ (row & 15);
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(ws + row * kRowBytes + c * 16));
    };

    // ---- prologue: x of the first tile, then the first kAhead weight stages;
    // mark[d] is the issue count just after the loads of stage gst + d
    load_x(tile_m0(0), 0, KS);
    int mark[kAhead];
#pragma unroll
    for (int d = 0; d < kAhead; ++d) {
        issue_w(d);
        mark[d] = issued;
    }
    // One weight stage: k stage Q of output-channel chunk nc of tile it.  In
    // the tile's last chunk (LAST) the k-slice Q of x is used for the last
    // time, and the next tile's is loaded into its registers.
    auto stage = [&]<int Q, bool LAST>(int64_t gst, int nc, int64_t it) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);   // nothing moves between stages (register pressure)
        // stage gst landed (this wave's quarter: at most the operations issued
        // after it are outstanding; every wave's: the barrier), and every wave
        // is done with the slot the next load refills (it held stage gst - 1)
        compiler_fence();
        wait_vm_at_most(issued - mark[0]);
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());   // this wave's LDS reads of stage gst - 1 done
        __builtin_amdgcn_s_barrier();
        compiler_fence();
#pragma unroll
        for (int d = 0; d + 1 < kAhead; ++d) mark[d] = mark[d + 1];
        // stage gst + kAhead's loads go out one per k-step below (issued as a
        // burst, the four waves' loads queue behind each other on the CU's
        // texture path while the matrix cores wait)
        const WLoad wl = w_load(gst + kAhead);
        static_assert(kWBlocksPerWave == kBK / 16, "one load per k-step");

        if (Q == 0) init_acc(nc * kBN);
        const unsigned char *ws = lds + (int)(gst % kNBuf) * kPart;
        // 8 k-steps; the 4 channel blocks' weight fragments are read one
        // k-step ahead, each feeds both position blocks
        bf16x8 fa[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[0][i] = wfrag(ws, 32 * i + l32, 0);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < kBK / 16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[cur ^ 1][i] = wfrag(ws, 32 * i + l32, ks + 1);
            }
            lds_dma16(wl.r, wl.dst + ks * 1024, w_off(ks));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jn = 0; jn < 2; ++jn)
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], xf[Q * 8 + ks][jn],
                                                                         acc[i][jn], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        issued += kWBlocksPerWave;
        mark[kAhead - 1] = issued;
        if (Q == S - 1) store(tile_m0(it), nc * kBN);
        if (LAST && it + 1 < my_tiles) load_x(tile_m0(it + 1), Q * 8, Q * 8 + 8);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto chunk = [&]<bool LAST>(int64_t &gst, int nc, int64_t it) __attribute__((always_inline)) {
        [&]<int... Q>(std::integer_sequence<int, Q...>) {
            ((stage.template operator()<Q, LAST>(gst + Q, nc, it)), ...);
        }(std::make_integer_sequence<int, S>{});
        gst += S;
    };
    // The chunks of a tile as three code paths (one when N <= 128, a separate
    // instantiation): the first (its stages wait
    // for the x loads still in flight), the middle ones (in a loop that no x
    // load enters, so no wait for x is placed in it) and the last (which
    // loads the next tile's x).  With a single loop over all chunks the
    // compiler would place the waits for x in every stage, and those waits,
    // which do not see the inline-assembly weight loads, would drain them and
    // the stores at every stage.
    int64_t gst = 0;
    for (int64_t it = 0; it < my_tiles; ++it) {
        if constexpr (ONE_CHUNK) {
            chunk.template operator()<true>(gst, 0, it);
        } else {
            chunk.template operator()<false>(gst, 0, it);
            for (int nc = 1; nc + 1 < nchunks; ++nc) chunk.template operator()<false>(gst, nc, it);
            chunk.template operator()<true>(gst, nchunks - 1, it);
        }
    }
    // the loads issued past the last stage (into consumed slots) have landed
    // before the workgroup ends and its LDS is handed on
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

}  // namespace

bool gemm_bf16_tiled_supported(int K, int N) {
    return K >= kBK && K <= kKMax && K % kBK == 0 && N >= 64 && N % 64 == 0 && N <= kNMax;
}

hipError_t launch_gemm_bf16_tiled(const void *x, const void *w, const float *bias, const void *res, void *y,
                                  int64_t P, int K, int N, hipStream_t s) {
    if (!gemm_bf16_tiled_supported(K, N)) return hipErrorInvalidValue;
    if (P <= 0) return hipSuccess;
    const int64_t mtiles = (P + kBM - 1) / kBM;
    int ncu = 0;
    const hipError_t e = device_cu_count(&ncu);
    if (e != hipSuccess) return e;
    const int64_t grid = mtiles < ncu ? mtiles : ncu;
    const auto *xp = static_cast<const uint16_t *>(x);
    const auto *wp = static_cast<const uint16_t *>(w);
    const auto *rp = static_cast<const uint16_t *>(res);
    auto *yp = static_cast<uint16_t *>(y);
    auto go = [&](auto kernel) {
        kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(xp, wp, bias, rp, yp, P, N, mtiles);
        return hipGetLastError();
    };
    auto by_k = [&](auto one) {
        constexpr bool ONE = decltype(one)::value;
        switch (K) {
            case 128: return res ? go(gemm_bf16_kernel<128, true, ONE>) : go(gemm_bf16_kernel<128, false, ONE>);
            case 256: return res ? go(gemm_bf16_kernel<256, true, ONE>) : go(gemm_bf16_kernel<256, false, ONE>);
            default: return res ? go(gemm_bf16_kernel<384, true, ONE>) : go(gemm_bf16_kernel<384, false, ONE>);
        }
    };
    return N <= kBN ? by_k(std::true_type{}) : by_k(std::false_type{});
}

}  // namespace wanvae
