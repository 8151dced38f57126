// Pointwise projection as a plain channel GEMM on MFMA:
//   y[p][n] = sum_k x[p][k] w[n][k] + bias[n] (+ res[p][n])
// x [P][K], w [N][K], res and y [P][N], all bf16 channels-last; fp32
// accumulation, bias and residual added in fp32, one RNE rounding.  These are
// the 1x1x1 projections around the decoder's mid-block attention (q, k and v
// from the normed input, C -> 3C, and the output projection with the residual,
// C -> C; "Closing the gap: Wan 2.2 14B VAE decoder", section 5, and
// "Sharding of WAN 2.2 VAE", decoder module tree).
//
// A workgroup owns 128 positions and all N output channels.  Their x rows
// (K <= 384, up to 96 KB) are loaded into LDS once, by LDS-DMA (buffer_load
// ... lds, 1 KB per instruction), and stay there while the output channels go
// by in chunks of 128: the weight (small, L2-resident) streams through a double
// buffer in stages of 128 channels x 128 k, the next stage loading while the
// current one computes.  x thus comes from HBM exactly once and only the weight
// is re-read, from L2.  Four waves, one per SIMD, each own 64 channels x 64
// positions of a chunk: 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 with the
// weights as the A operand (channels as M) and x as the B operand (positions
// as N), so a lane ends up holding 4 consecutive output channels of one
// position per 4 accumulators and stores them as one 8-byte piece.  Rows are
// swizzled in 16-byte chunks (chunk ^ (row & 15)) so that fragment reads hit
// distinct banks.  The grid is persistent, one workgroup per CU.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;                       // positions per tile
constexpr int kBN = 128;                       // output channels per chunk
constexpr int kBK = 128;                       // K per weight stage
constexpr int kKMax = 384;                     // the resident x tile holds K <= 384
constexpr int kXMax = kBM * kKMax * 2;         // 96 KB
constexpr int kRowBytes = kBK * 2;             // 256 bytes of a weight row per stage
constexpr int kPart = kBN * kRowBytes;         // 32 KB: one weight stage
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kWBlocksPerWave = kPart / 1024 / kWaves;   // 8
constexpr int kXCD = 8;
constexpr int kStores = 16;                    // buffer stores per lane in an epilogue
constexpr int kBufFlags = 0x00020000;          // raw buffer: loads past num_records return zeros
constexpr uint32_t kOOB = 0x80000000u;
static_assert(kXMax + 2 * kPart <= 160 * 1024, "LDS");

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

template <bool RES>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ w,
                                                             const float *__restrict__ bias,
                                                             const uint16_t *__restrict__ res,
                                                             uint16_t *__restrict__ y, int64_t P, int N, int K,
                                                             int64_t mtiles) {
    // LDS: the x tile [128 positions][K] (resident for all output channels),
    // then two w stages [128 channels][128 k]
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kXMax + 2 * kPart];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;       // channel half, position half
    const int l32 = lane & 31, g = lane >> 5;
    const int nchunks = (N + kBN - 1) / kBN, kstages = K / kBK;   // (the last chunk may be 64 wide)
    const int xrow = 2 * K;                        // bytes of an x row

    // ---- this workgroup's position tiles: XCD x (= workgroup index mod 8)
    // owns a contiguous range, its workgroups take them round-robin
    const int64_t nwg = gridDim.x, bid = blockIdx.x;
    const int64_t xcd = bid % kXCD, loc = bid / kXCD;
    const int64_t wg_x = nwg / kXCD + (xcd < nwg % kXCD ? 1 : 0);
    const int64_t wg_before = xcd * (nwg / kXCD) + (xcd < nwg % kXCD ? xcd : nwg % kXCD);
    const int64_t x_begin = mtiles * wg_before / nwg;
    const int64_t x_count = mtiles * (wg_before + wg_x) / nwg - x_begin;
    const int64_t my_tiles = x_count > loc ? (x_count - loc + wg_x - 1) / wg_x : 0;

    const uint32_t lds_base = lds_address(lds);
    const uint32_t w_base = lds_base + kXMax;
    // x tile: K/4 blocks of 1 KB, wave w the blocks w, w + 4, ...; byte o of
    // the tile is row o / xrow, stored chunk (o % xrow) / 16 = global chunk ^
    // (row & 15)
    auto issue_x = [&](int64_t m0) __attribute__((always_inline)) {
        const int64_t rows = P - m0 < kBM ? P - m0 : kBM;
        const i32x4 r = buffer_rsrc(x + m0 * K, (uint32_t)(rows * xrow));
        for (int b = wave; b < K / 4; b += kWaves) {
            const int o = b * 1024 + lane * 16;
            const int row = o / xrow, cs = (o % xrow) / 16;
            const uint32_t off = row < rows ? (uint32_t)(row * xrow + ((cs ^ (row & 15)) * 16)) : kOOB;
            lds_dma16(r, lds_base + (uint32_t)(b * 1024), off);
        }
    };
    // w stage (chunk nc, k stage ks): 32 blocks, 8 per wave; block b rows
    // 4b .. 4b + 3 of the 128 channels, lane row 4b + l / 16, stored chunk l % 16
    uint32_t w_off[kWBlocksPerWave];
#pragma unroll
    for (int i = 0; i < kWBlocksPerWave; ++i) {
        const int b = wave * kWBlocksPerWave + i;
        const int row = 4 * b + (lane >> 4), cs = lane & 15;
        w_off[i] = (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)((cs ^ (row & 15)) * 16);
    }
    auto issue_w = [&](int st) __attribute__((always_inline)) {
        const int nc = st / kstages, kk = (st % kstages) * kBK;
        // channels past N (a 64-wide last chunk) fall beyond the buffer's end: zeros
        const int rows = N - nc * kBN < kBN ? N - nc * kBN : kBN;
        const i32x4 r = buffer_rsrc(w + (int64_t)nc * kBN * K + kk, (uint32_t)(rows * K * 2 - kk * 2));
        const uint32_t dst = w_base + (uint32_t)((st & 1) * kPart + wave * kWBlocksPerWave * 1024);
#pragma unroll
        for (int i = 0; i < kWBlocksPerWave; ++i) lds_dma16(r, dst + i * 1024, w_off[i]);
    };
    // wait for this wave's LDS-DMA (all but the last `after` vector-memory
    // operations, which counts in issue order) and LDS reads, then barrier
    auto sync = [&](bool after_stores) __attribute__((always_inline)) {
        compiler_fence();
        if (after_stores)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(kStores) & waitcnt_lgkm0());
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & waitcnt_lgkm0());
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    };

    // fragments: weight row `row` of a stage, k-step ks (k = 16 ks + 8 g .. +7);
    // x row `row`, global 16-byte chunk kc
    auto wfrag = [&](const unsigned char *ws, int row, int ks) __attribute__((always_inline)) {
        const int c = (2 * ks + g) ^ (row & 15);
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(ws + row * kRowBytes + c * 16));
    };
    auto xfrag = [&](int row, int kc) __attribute__((always_inline)) {
        const int c = kc ^ (row & 15);
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(lds + row * xrow + c * 16));
    };

    floatx16 acc[2][2];
    float4 bv[2][4];   // bias of this lane's channels in the current chunk
    auto load_bias = [&](int n0) __attribute__((always_inline)) {
        if (bias) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    bv[i][jj] = n0 + wm * 64 < N ? *reinterpret_cast<const float4 *>(bias + n0 + wm * 64 + 32 * i + 8 * jj + 4 * g)
                                                 : float4{0.0f, 0.0f, 0.0f, 0.0f};
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) bv[i][jj] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    // ---- epilogue of chunk n0: channel n0 + 64 wm + 32 i + 8 jj + 4 g + {0..3}
    // of position m0 + 64 wn + 32 jn + l32: 8 contiguous bytes.  Exactly
    // kStores buffer stores per lane whatever the tile: positions past P fall
    // beyond the buffer's end and are dropped (the stage wait counts on it).
    auto store = [&](int64_t m0, int n0) __attribute__((always_inline)) {
        const int64_t rows = P - m0 < kBM ? P - m0 : kBM;
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + m0 * N, (uint32_t)(rows * N * 2));
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(RES ? res + m0 * N : y, RES ? (uint32_t)(rows * N * 2) : 0u);
        uint32_t off[2][2][4];
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int pl = wn * 64 + 32 * jn + l32;   // position within the tile
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    off[jn][i][jj] = pl < rows && n0 + wm * 64 < N
                                         ? (uint32_t)((pl * N + n0 + wm * 64 + 32 * i + 8 * jj + 4 * g) * 2)
                                         : kOOB;
        }
        // residual pieces all requested before the first store (a load behind
        // a store would wait for it)
        u32x2 rv[2][2][4];
        if constexpr (RES) {
#pragma unroll
            for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        rv[jn][i][jj] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rr, off[jn][i][jj], 0, 0));
        }
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float v0 = acc[i][jn][4 * jj] + bv[i][jj].x, v1 = acc[i][jn][4 * jj + 1] + bv[i][jj].y;
                    float v2 = acc[i][jn][4 * jj + 2] + bv[i][jj].z, v3 = acc[i][jn][4 * jj + 3] + bv[i][jj].w;
                    if constexpr (RES) {
                        v0 += bf16_bits_to_f32(rv[jn][i][jj].x & 0xffffu);
                        v1 += bf16_bits_to_f32(rv[jn][i][jj].x >> 16);
                        v2 += bf16_bits_to_f32(rv[jn][i][jj].y & 0xffffu);
                        v3 += bf16_bits_to_f32(rv[jn][i][jj].y >> 16);
                    }
                    const u32x2 d = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, d), ry, off[jn][i][jj], 0, 0);
                }
    };

    const int wstages = nchunks * kstages;
    for (int64_t it = 0; it < my_tiles; ++it) {
        const int64_t m0 = (x_begin + loc + it * wg_x) * kBM;
        // every wave is done with the previous tile's x and w buffers (LDS
        // reads only: its stores may still be in flight)
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        issue_x(m0);
        issue_w(0);
        for (int st = 0; st < wstages; ++st) {
            // stage st (and, first, the x tile) landed; buffer (st + 1) & 1
            // free.  After an epilogue exactly kStores stores follow the
            // stage's loads.
            sync(st > 0 && st % kstages == 0);
            if (st + 1 < wstages) issue_w(st + 1);
            const int nc = st / kstages, kq = st % kstages;
            if (kq == 0) {
                load_bias(nc * kBN);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.0f;
            }
            const unsigned char *ws = lds + kXMax + (st & 1) * kPart;
            // fragments are read one k-step ahead of their MFMAs
            bf16x8 fa[2][2], fb[2][2];
            auto load_frags = [&](int ks, int buf) __attribute__((always_inline)) {
                const int kc = kq * (kBK / 8) + 2 * ks + g;   // x chunk of this k-step
                fa[buf][0] = wfrag(ws, wm * 64 + l32, ks);
                fa[buf][1] = wfrag(ws, wm * 64 + 32 + l32, ks);
                fb[buf][0] = xfrag(wn * 64 + l32, kc);
                fb[buf][1] = xfrag(wn * 64 + 32 + l32, kc);
            };
            load_frags(0, 0);
#pragma unroll
            for (int ks = 0; ks < kBK / 16; ++ks) {
                const int cur = ks & 1;
                if (ks + 1 < kBK / 16) load_frags(ks + 1, cur ^ 1);
                __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of these MFMAs
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int jn = 0; jn < 2; ++jn)
                        acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][jn], acc[i][jn], 0, 0, 0);
            }
            if (kq + 1 == kstages) store(m0, nc * kBN);
        }
    }
}
}  // namespace

bool gemm_bf16_tiled_supported(int K, int N) {
    return K >= kBK && K <= kKMax && K % kBK == 0 && N >= 64 && N % 64 == 0;
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
    if (res)
        gemm_bf16_kernel<true><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(xp, wp, bias, rp, yp, P, N, K, mtiles);
    else
        gemm_bf16_kernel<false><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(xp, wp, bias, rp, yp, P, N, K, mtiles);
    return hipGetLastError();
}

}  // namespace wanvae
