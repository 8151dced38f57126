// Pointwise projection as a plain channel GEMM on MFMA:
//   y[p][n] = sum_k x[p][k] w[n][k] + bias[n] (+ res[p][n])
// x [P][K], w [N][K], res and y [P][N], all bf16 channels-last; fp32
// accumulation, bias and residual added in fp32, one RNE rounding.  These are
// the 1x1x1 projections around the decoder's mid-block attention (q, k and v
// from the normed input, C -> 3C, and the output projection with the residual,
// C -> C; "Closing the gap: Wan 2.2 14B VAE decoder", section 5, and
// "Sharding of WAN 2.2 VAE", decoder module tree).
//
// A workgroup owns a tile of 128 positions x 128 output channels and walks K in
// stages of 128 (256 bytes of every row): both operands are K-contiguous, so a
// stage is 128 + 128 rows of 256 contiguous bytes, staged by LDS-DMA
// (buffer_load ... lds, 1 KB per instruction, 16 per wave) into a double
// buffer, the next stage loading while the current one computes.  Four waves,
// one per SIMD, each own 64 channels x 64 positions: 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 with the weights as the A operand (channels as M)
// and x as the B operand (positions as N), so a lane ends up holding 4
// consecutive output channels of one position per 4 accumulators and stores
// them as one 8-byte piece.  Rows are swizzled in 16-byte chunks (chunk ^ (row
// & 15)) so that fragment reads hit distinct banks.  The grid is persistent,
// one workgroup per CU, each XCD owning a contiguous range of tiles with the
// channel tile fastest, so the workgroups of an XCD share each x tile through
// its L2 and the whole weight stays L2-resident.
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
constexpr int kBN = 128;                       // output channels per tile
constexpr int kBK = 128;                       // K per stage
constexpr int kRowBytes = kBK * 2;             // 256 bytes of a row per stage
constexpr int kPart = kBM * kRowBytes;         // 32 KB: the x part (and the w part) of a stage
constexpr int kStage = 2 * kPart;              // 64 KB
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kDmaPerWave = kStage / 1024 / kWaves;   // 16
constexpr int kXCD = 8;
constexpr int kBufFlags = 0x00020000;          // raw buffer: loads past num_records return zeros
constexpr uint32_t kOOB = 0x80000000u;
static_assert(kBM == kBN, "x and w parts share the DMA mapping");

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
                                                             int64_t tiles) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;       // channel half, position half
    const int l32 = lane & 31, g = lane >> 5;
    const int ntn = N / kBN;
    const int ks_per_tile = K / kBK;

    // ---- this workgroup's tiles: XCD x (= workgroup index mod 8) owns a
    // contiguous range; its workgroups take that range's tiles round-robin
    const int64_t nwg = gridDim.x, bid = blockIdx.x;
    const int64_t xcd = bid % kXCD, loc = bid / kXCD;
    const int64_t wg_x = nwg / kXCD + (xcd < nwg % kXCD ? 1 : 0);
    const int64_t wg_before = xcd * (nwg / kXCD) + (xcd < nwg % kXCD ? xcd : nwg % kXCD);
    const int64_t x_begin = tiles * wg_before / nwg;
    const int64_t x_count = tiles * (wg_before + wg_x) / nwg - x_begin;
    const int64_t my_tiles = x_count > loc ? (x_count - loc + wg_x - 1) / wg_x : 0;
    const int64_t stages = my_tiles * ks_per_tile;

    // ---- DMA: wave w issues the 1 KB blocks 16w .. 16w + 15 of a stage;
    // blocks 0..31 are the x part, 32..63 the w part.  Block b holds rows
    // 4(b % 32) .. +3 of its part; lane l row 4(b % 32) + l / 16, stored
    // chunk l % 16 = global chunk ^ (row & 15).
    const uint32_t lds_base = lds_address(lds);
    const bool x_wave = wave < 2;
    uint32_t row_off[kDmaPerWave];   // byte offset of this lane's piece within the part's rows
    int row_of[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int b = (wave & 1) * kDmaPerWave + i;   // block within the part
        const int row = 4 * b + (lane >> 4), cs = lane & 15;
        row_of[i] = row;
        row_off[i] = (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)((cs ^ (row & 15)) * 16);
    }
    const uint32_t dma_lds0 = lds_base + (x_wave ? 0u : (uint32_t)kPart) + (uint32_t)((wave & 1) * kDmaPerWave * 1024);
    auto tile_of = [&](int64_t t) __attribute__((always_inline)) { return x_begin + loc + t * wg_x; };
    // request stage st (of this workgroup's sequence) into buffer st & 1
    auto issue = [&](int64_t st) __attribute__((always_inline)) {
        const int64_t tile = tile_of(st / ks_per_tile);
        const int kk = (int)(st % ks_per_tile) * kBK;
        const int64_t m0 = (tile / ntn) * kBM;
        const int n0 = (int)(tile % ntn) * kBN;
        const uint32_t dst = dma_lds0 + (uint32_t)((st & 1) * kStage);
        if (x_wave) {
            // rows past P fall beyond the buffer's end: zeros
            const int64_t rows = P - m0 < kBM ? P - m0 : kBM;
            const i32x4 r = buffer_rsrc(x + m0 * K + kk, (uint32_t)(rows * K * 2 - kk * 2));
#pragma unroll
            for (int i = 0; i < kDmaPerWave; ++i) lds_dma16(r, dst + i * 1024, row_of[i] < rows ? row_off[i] : kOOB);
        } else {
            const i32x4 r = buffer_rsrc(w + (int64_t)n0 * K + kk, (uint32_t)(kBN * K * 2 - kk * 2));
#pragma unroll
            for (int i = 0; i < kDmaPerWave; ++i) lds_dma16(r, dst + i * 1024, row_off[i]);
        }
    };

    // fragment of row `row` of a part, MFMA k-step ks (k = 16 ks + 8 g .. +7)
    auto frag = [&](const unsigned char *part, int row, int ks) __attribute__((always_inline)) {
        const int c = (2 * ks + g) ^ (row & 15);
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(part + row * kRowBytes + c * 16));
    };

    floatx16 acc[2][2];
    auto zero = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.0f;
    };
    zero();

    if (stages > 0) issue(0);
    for (int64_t st = 0; st < stages; ++st) {
        // stage st landed (own loads), every wave done with buffer (st + 1) & 1
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & waitcnt_lgkm0());
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (st + 1 < stages) issue(st + 1);

        const unsigned char *xs = lds + (st & 1) * kStage;
        const unsigned char *ws = xs + kPart;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const bf16x8 a0 = frag(ws, wm * 64 + l32, ks), a1 = frag(ws, wm * 64 + 32 + l32, ks);
            const bf16x8 b0 = frag(xs, wn * 64 + l32, ks), b1 = frag(xs, wn * 64 + 32 + l32, ks);
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
        }

        if ((st + 1) % ks_per_tile == 0) {
            // ---- epilogue: channel n0 + 64 wm + 32 i + 8 jj + 4 g + {0..3} of
            // position m0 + 64 wn + 32 jn + l32: 8 contiguous bytes
            const int64_t tile = tile_of(st / ks_per_tile);
            const int64_t m0 = (tile / ntn) * kBM;
            const int n0 = (int)(tile % ntn) * kBN;
#pragma unroll
            for (int jn = 0; jn < 2; ++jn) {
                const int64_t p = m0 + wn * 64 + 32 * jn + l32;
                if (p < P) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int n = n0 + wm * 64 + 32 * i + 8 * jj + 4 * g;
                            const float4 bv = bias ? *reinterpret_cast<const float4 *>(bias + n)
                                                   : float4{0.0f, 0.0f, 0.0f, 0.0f};
                            float v0 = acc[i][jn][4 * jj] + bv.x, v1 = acc[i][jn][4 * jj + 1] + bv.y;
                            float v2 = acc[i][jn][4 * jj + 2] + bv.z, v3 = acc[i][jn][4 * jj + 3] + bv.w;
                            if constexpr (RES) {
                                const u32x2 rv = *reinterpret_cast<const u32x2 *>(res + p * N + n);
                                v0 += bf16_bits_to_f32(rv.x & 0xffffu);
                                v1 += bf16_bits_to_f32(rv.x >> 16);
                                v2 += bf16_bits_to_f32(rv.y & 0xffffu);
                                v3 += bf16_bits_to_f32(rv.y >> 16);
                            }
                            *reinterpret_cast<u32x2 *>(y + p * N + n) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                        }
                }
            }
            zero();
        }
    }
}

}  // namespace

bool gemm_bf16_tiled_supported(int K, int N) { return K >= kBK && K % kBK == 0 && N >= kBN && N % kBN == 0; }

hipError_t launch_gemm_bf16_tiled(const void *x, const void *w, const float *bias, const void *res, void *y,
                                  int64_t P, int K, int N, hipStream_t s) {
    if (!gemm_bf16_tiled_supported(K, N)) return hipErrorInvalidValue;
    // the x part of a stage addresses a tile's rows with 32-bit offsets
    if ((int64_t)kBM * K * 2 >= (int64_t)1 << 31) return hipErrorInvalidValue;
    if (P <= 0) return hipSuccess;
    const int64_t tiles = (P + kBM - 1) / kBM * (N / kBN);
    int ncu = 0;
    const hipError_t e = device_cu_count(&ncu);
    if (e != hipSuccess) return e;
    const int64_t grid = tiles < ncu ? tiles : ncu;
    const auto *xp = static_cast<const uint16_t *>(x);
    const auto *wp = static_cast<const uint16_t *>(w);
    const auto *rp = static_cast<const uint16_t *>(res);
    auto *yp = static_cast<uint16_t *>(y);
    if (res)
        gemm_bf16_kernel<true><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(xp, wp, bias, rp, yp, P, N, K, tiles);
    else
        gemm_bf16_kernel<false><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(xp, wp, bias, rp, yp, P, N, K, tiles);
    return hipGetLastError();
}

}  // namespace wanvae
