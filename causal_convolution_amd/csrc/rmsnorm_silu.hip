// Fused channel RMS_norm + SiLU, HBM-bound.
//
// Per C-vector v (one NDHWC position):
//   d = max(sqrt(sum_c v_c^2), eps),  u_c = v_c * (sqrt(C) / d) * gamma_c + beta_c,
//   y_c = u_c / (1 + exp(-u_c))
// which is the F.normalize-based RMS_norm of "Closing the gap: Wan 2.2 14B VAE
// decoder", section 4, with SiLU fused into the same pass as that section
// describes for tt-metal's kernel.
//
// Mapping: 16 consecutive lanes own G consecutive rows, G the fewest rows
// that span a whole number of 256-byte runs (G = 1 for 384 bf16 channels, 2
// for 192, 4 for 96).  The G rows are cut into 16-byte pieces and piece p
// belongs to lane p % 16, so every load or store instruction of a 16-lane
// group covers one whole 256-byte run: each instruction uses its cache lines
// entirely, which lets the accesses stream past the caches (nontemporal) at
// close to the device's copy bandwidth.  Pieces never straddle rows (C is a
// multiple of 8); a lane keeps one partial sum of squares per row of its
// group, and each is reduced across the 16 lanes with xor shuffles (no LDS).
// gamma * sqrt(C) and beta are held in registers for the whole grid-stride
// loop; U groups of rows are in flight per lane to cover HBM latency.  y may
// equal x (in place): each element is read and then written by the same
// lane.  x is read once and y written once: 2 * rows * C * sizeof(T) bytes of
// HBM traffic.
//
// A second form writes y in the layout the bf16 conv reads: rows are the
// positions of frames of hw positions, and each frame is stored as 16-channel
// slices, [C/16][hw][16].  A block then normalises its R = 16 G U rows of a
// pass, loaded as above, into LDS in slice order and stores each slice of the
// tile as one contiguous run of R * 32 bytes (1 KB for C = 384, 2 KB for 192,
// 4 KB for 96): whole cache lines and long DRAM bursts, where storing the
// pieces straight from their lanes would leave lines half written.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

constexpr int kGroupLanes = 16;
constexpr int kThreads = 256;
constexpr int kGroups = kThreads / kGroupLanes;   // 16-lane groups per block
constexpr int kGridCap = 16384;                   // blocks; the grid strides over the rows
constexpr int kNoRow = 1 << 20;                   // row index of a ragged group's empty pieces

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }

__device__ inline float silu(float u) {
    // u / (1 + exp(-u)); exp(-u) = inf for very negative u gives -0
    return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

template <bool ACT>
__device__ inline float act(float u) {
    if constexpr (ACT) return silu(u);
    return u;
}

// 16 bytes = EP elements of T as fp32 and back
template <typename T> struct Piece;
template <> struct Piece<float> {
    static constexpr int EP = 4;
    static __device__ inline void unpack(const u32x4 &d, float (&v)[4]) {
        v[0] = __uint_as_float(d.x); v[1] = __uint_as_float(d.y);
        v[2] = __uint_as_float(d.z); v[3] = __uint_as_float(d.w);
    }
    static __device__ inline u32x4 pack(const float (&v)[4]) {
        return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    }
};
template <> struct Piece<uint16_t> {  // bf16 bits
    static constexpr int EP = 8;
    static __device__ inline void unpack(const u32x4 &d, float (&v)[8]) {
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = bf16_bits_to_f32(w[k] & 0xffffu);
            v[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
        }
    }
    static __device__ inline u32x4 pack(const float (&v)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = f32_to_bf16_bits(v[2 * k]) | (f32_to_bf16_bits(v[2 * k + 1]) << 16);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
};

template <typename T, int C>
struct Shape {
    static constexpr int RB = C * (int)sizeof(T);          // row bytes
    static constexpr int G0 = 256 / gcd(256, RB);          // fewest rows spanning whole runs
    // Channel counts whose G0 rows would give a lane more than 16 pieces
    // (odd multiples of 32 above 512) take one row per group instead, its last
    // 256-byte run only partly used ("ragged": some lanes own one piece less).
    static constexpr bool RAGGED = G0 * RB / 256 > 16;
    static constexpr int G = RAGGED ? 1 : G0;              // rows per 16-lane group
    static constexpr int NP = RAGGED ? (RB + 255) / 256 : G * RB / 256;   // 16-byte pieces per lane
    static constexpr int EP = Piece<T>::EP;                // elements per piece
    // groups of rows in flight per lane: about 96 bytes of loads or more
    static constexpr int U = NP * 16 >= 96 ? 1 : (96 + NP * 16 - 1) / (NP * 16) > 8 ? 8
                                                    : (96 + NP * 16 - 1) / (NP * 16);
    static constexpr int ROWS_PER_BLOCK = kGroups * G * U;  // per pass of the grid-stride loop
    // gamma, beta and the unpacked values of a lane's pieces stay in registers
    // when there are few; otherwise (channel counts with many pieces per lane)
    // gamma and beta are re-read from the cache and the pieces unpacked twice
    static constexpr bool IN_REGS = NP * EP <= 48;
};

// SLICED: y is written in the conv input layout, frame f = row / hw cut into
// 16-channel slices, y[f][c / 16][row % hw][c % 16] (inv_hw = 1 / hw).
// ACT: SiLU after the norm (the ResidualBlock); without it, the plain
// RMS_norm (the attention block's input norm).
template <typename T, int C, bool SLICED, bool ACT>
__global__ __launch_bounds__(kThreads) void rmsnorm_silu_kernel(
    const T *x, T *y, int64_t rows, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, float sqrt_c, int64_t hw, double inv_hw) {
    using S = Shape<T, C>;
    using PC = Piece<T>;
    constexpr int G = S::G, NP = S::NP, EP = S::EP, U = S::U;

    const int lane = threadIdx.x % kGroupLanes;
    const int grp = threadIdx.x / kGroupLanes;

    // piece i of this lane: byte (i * 16 + lane) * 16 of its group's G rows,
    // i.e. row prow[i] of the group, channels pch[i] .. pch[i] + EP - 1
    int prow[NP], pch[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int byte = (i * kGroupLanes + lane) * 16;
        prow[i] = G == 1 ? 0 : byte / S::RB;
        pch[i] = (byte % S::RB) / (int)sizeof(T);
        // a ragged group's pieces past the row: no data, channel 0's gamma
        if (S::RAGGED && byte >= S::RB) prow[i] = kNoRow, pch[i] = 0;
    }
    // gamma * sqrt(C) and beta of those channels, loaded once
    constexpr int NR = S::IN_REGS ? NP : 1;
    float g[NR][EP], b[NR][EP];
#pragma unroll
    for (int i = 0; i < (S::IN_REGS ? NP : 0); ++i)
#pragma unroll
        for (int k = 0; k < EP; k += 4) {
            const float4 gv = *reinterpret_cast<const float4 *>(gamma + pch[i] + k);
            const float4 bv = beta ? *reinterpret_cast<const float4 *>(beta + pch[i] + k)
                                   : float4{0.f, 0.f, 0.f, 0.f};
            g[i][k] = gv.x * sqrt_c; g[i][k + 1] = gv.y * sqrt_c;
            g[i][k + 2] = gv.z * sqrt_c; g[i][k + 3] = gv.w * sqrt_c;
            b[i][k] = bv.x; b[i][k + 1] = bv.y; b[i][k + 2] = bv.z; b[i][k + 3] = bv.w;
        }

    const unsigned char *xb = reinterpret_cast<const unsigned char *>(x);
    unsigned char *yb = reinterpret_cast<unsigned char *>(y);

    // SLICED: the block's R rows of a pass are normalised into LDS in slice
    // order, [C/16][R][16] with a 16-byte pad per slice against bank
    // conflicts, and stored from there as R * 32 contiguous bytes per slice.
    constexpr int R = S::ROWS_PER_BLOCK;
    constexpr int SLICE_STRIDE = R * 32 + 16;
    __shared__ __attribute__((aligned(16))) unsigned char tile_lds[SLICED ? (C / 16) * SLICE_STRIDE : 16];
    auto group_row0 = [&](int64_t r0, int u) -> int64_t { return r0 + (int64_t)(u * kGroups + grp) * G; };
    const int64_t step = (int64_t)gridDim.x * S::ROWS_PER_BLOCK;

    // this lane's pieces of the pass starting at row r0
    auto load_pass = [&](int64_t r0, u32x4 (&d)[U][NP]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g0 = group_row0(r0, u);   // the group's first row
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                if ((!S::RAGGED || prow[i] != kNoRow) && g0 + prow[i] < rows)
                    d[u][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                        xb + g0 * S::RB + (i * kGroupLanes + lane) * 16));
                else
                    d[u][i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // SLICED passes end in a block barrier and an LDS round trip, so the next
    // pass's loads are issued before this pass is processed
    u32x4 d_next[SLICED ? U : 1][NP];
    if constexpr (SLICED) load_pass((int64_t)blockIdx.x * S::ROWS_PER_BLOCK, d_next);

    for (int64_t r0 = (int64_t)blockIdx.x * S::ROWS_PER_BLOCK; r0 < rows; r0 += step) {
        u32x4 d[U][NP];
        if constexpr (SLICED) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < NP; ++i) d[u][i] = d_next[u][i];
            if (r0 + step < rows) load_pass(r0 + step, d_next);
        } else {
            load_pass(r0, d);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g0 = group_row0(r0, u);
            float v[NR][EP];
            float ss[G];
#pragma unroll
            for (int q = 0; q < G; ++q) ss[q] = 0.0f;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                float (&vi)[EP] = v[S::IN_REGS ? i : 0];
                PC::unpack(d[u][i], vi);
                float s = 0.0f;
#pragma unroll
                for (int k = 0; k < EP; ++k) s = fmaf(vi[k], vi[k], s);
#pragma unroll
                for (int q = 0; q < G; ++q) ss[q] += prow[i] == q ? s : 0.0f;
            }
            float inv[G];
#pragma unroll
            for (int q = 0; q < G; ++q) {
                // all 64 lanes take part: the xor masks stay inside each 16-lane group
                float t = ss[q];
                // Row q's first piece sits at lane (q * RB / 16) % 16 of the
                // group; rotating the partial sums so that it comes to lane 0
                // makes the order of the sum below (and so its rounding) the
                // same wherever a row falls in its group.  A position then
                // gets the same norm whether it is normalised with its whole
                // clip or in a chunk of frames (rows shift by the frames
                // before it, h * w rows each, which need not be a multiple
                // of G).
                constexpr int kRowPieces = S::RB / 16;
                if (G > 1 && (q * kRowPieces) % kGroupLanes != 0) {
                    const int wl = threadIdx.x & 63;
                    t = __shfl(t, (wl & ~(kGroupLanes - 1)) | ((wl + q * kRowPieces) & (kGroupLanes - 1)));
                }
                t += __shfl_xor(t, 1);
                t += __shfl_xor(t, 2);
                t += __shfl_xor(t, 4);
                t += __shfl_xor(t, 8);
                inv[q] = 1.0f / fmaxf(sqrtf(t), eps);
            }
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                float ip = inv[0];
#pragma unroll
                for (int q = 1; q < G; ++q) ip = prow[i] == q ? inv[q] : ip;
                float (&vi)[EP] = v[S::IN_REGS ? i : 0];
                if constexpr (S::IN_REGS) {
#pragma unroll
                    for (int k = 0; k < EP; ++k) vi[k] = act<ACT>(fmaf(vi[k] * ip, g[i][k], b[i][k]));
                } else {
                    PC::unpack(d[u][i], vi);
#pragma unroll
                    for (int k = 0; k < EP; k += 4) {
                        const float4 gv = *reinterpret_cast<const float4 *>(gamma + pch[i] + k);
                        const float4 bv = beta ? *reinterpret_cast<const float4 *>(beta + pch[i] + k)
                                               : float4{0.f, 0.f, 0.f, 0.f};
                        vi[k] = act<ACT>(fmaf(vi[k] * ip, gv.x * sqrt_c, bv.x));
                        vi[k + 1] = act<ACT>(fmaf(vi[k + 1] * ip, gv.y * sqrt_c, bv.y));
                        vi[k + 2] = act<ACT>(fmaf(vi[k + 2] * ip, gv.z * sqrt_c, bv.z));
                        vi[k + 3] = act<ACT>(fmaf(vi[k + 3] * ip, gv.w * sqrt_c, bv.w));
                    }
                }
                if constexpr (SLICED) {
                    if (!S::RAGGED || prow[i] != kNoRow) {
                        const int rt = (u * kGroups + grp) * G + prow[i];   // row within the block tile
                        *reinterpret_cast<u32x4 *>(tile_lds + (pch[i] / 16) * SLICE_STRIDE + rt * 32 +
                                                   (pch[i] % 16) * (int)sizeof(T)) = PC::pack(vi);
                    }
                } else if ((!S::RAGGED || prow[i] != kNoRow) && g0 + prow[i] < rows) {
                    __builtin_nontemporal_store(PC::pack(vi), reinterpret_cast<u32x4 *>(
                        yb + g0 * S::RB + (i * kGroupLanes + lane) * 16));
                }
            }
        }
        if constexpr (SLICED) {
            __syncthreads();   // the whole tile is in LDS
            constexpr int TOTAL = R * S::RB;   // bytes of the block tile
            const int64_t t0 = r0;
            // frame and position of the tile's first row: a double-precision
            // quotient, exact after one correction step
            int64_t f0 = (int64_t)((double)t0 * inv_hw);
            int64_t q0 = t0 - f0 * hw;
            if (q0 < 0) --f0, q0 += hw;
            else if (q0 >= hw) ++f0, q0 -= hw;
#pragma unroll
            for (int j = 0; j < (TOTAL + kThreads * 16 - 1) / (kThreads * 16); ++j) {
                const int o = (j * kThreads + (int)threadIdx.x) * 16;   // byte of the tile in [C/16][R][32] order
                const int k = o / (R * 32), rem = o % (R * 32);
                const int rt = rem / 32;
                if (o < TOTAL && t0 + rt < rows) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(tile_lds + k * SLICE_STRIDE + rem);
                    int64_t f = f0, q = q0 + rt;
                    while (q >= hw) q -= hw, ++f;   // at most R / hw + 1 steps
                    const int64_t off = ((f * C + k * 16) * hw + q * 16) * (int64_t)sizeof(T) + rem % 32;
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(yb + off));
                }
            }
            __syncthreads();   // read back before the next pass overwrites the tile
        }
    }
}

template <typename T, int C, bool SLICED, bool ACT>
hipError_t launch_c(const void *x, void *y, int64_t rows, const float *gamma, const float *beta,
                    float eps, int64_t hw, hipStream_t s) {
    using S = Shape<T, C>;
    int64_t blocks = (rows + S::ROWS_PER_BLOCK - 1) / S::ROWS_PER_BLOCK;
    if (blocks > kGridCap) blocks = kGridCap;
    if (blocks < 1) blocks = 1;
    rmsnorm_silu_kernel<T, C, SLICED, ACT><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
        static_cast<const T *>(x), static_cast<T *>(y), rows, gamma, beta, eps, sqrtf((float)C), hw,
        1.0 / (double)hw);
    return hipGetLastError();
}

template <typename T, bool SLICED, bool ACT = true>
hipError_t dispatch(const void *x, void *y, int64_t rows, int C, const float *gamma,
                    const float *beta, float eps, int64_t hw, hipStream_t s) {
    switch (C) {
#define WANVAE_NORM_CASE(K) \
    case 32 * K: return launch_c<T, 32 * K, SLICED, ACT>(x, y, rows, gamma, beta, eps, hw, s);
        WANVAE_NORM_CASE(1) WANVAE_NORM_CASE(2) WANVAE_NORM_CASE(3) WANVAE_NORM_CASE(4)
        WANVAE_NORM_CASE(5) WANVAE_NORM_CASE(6) WANVAE_NORM_CASE(7) WANVAE_NORM_CASE(8)
        WANVAE_NORM_CASE(9) WANVAE_NORM_CASE(10) WANVAE_NORM_CASE(11) WANVAE_NORM_CASE(12)
        WANVAE_NORM_CASE(13) WANVAE_NORM_CASE(14) WANVAE_NORM_CASE(15) WANVAE_NORM_CASE(16)
        WANVAE_NORM_CASE(17) WANVAE_NORM_CASE(18) WANVAE_NORM_CASE(19) WANVAE_NORM_CASE(20)
        WANVAE_NORM_CASE(21) WANVAE_NORM_CASE(22) WANVAE_NORM_CASE(23) WANVAE_NORM_CASE(24)
        WANVAE_NORM_CASE(25) WANVAE_NORM_CASE(26) WANVAE_NORM_CASE(27) WANVAE_NORM_CASE(28)
        WANVAE_NORM_CASE(29) WANVAE_NORM_CASE(30) WANVAE_NORM_CASE(31) WANVAE_NORM_CASE(32)
#undef WANVAE_NORM_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool rmsnorm_silu_supported(int C) { return C >= 32 && C <= 1024 && C % 32 == 0; }

hipError_t launch_rmsnorm_silu_bf16(const void *x, void *y, int64_t rows, int C,
                                    const float *gamma, const float *beta, float eps,
                                    hipStream_t s) {
    return dispatch<uint16_t, false>(x, y, rows, C, gamma, beta, eps, 1, s);
}

hipError_t launch_rmsnorm_silu_bf16_sliced(const void *x, void *y, int64_t rows, int C, int64_t hw,
                                           const float *gamma, const float *beta, float eps,
                                           hipStream_t s) {
    if (hw <= 0) return hipErrorInvalidValue;
    return dispatch<uint16_t, true>(x, y, rows, C, gamma, beta, eps, hw, s);
}

hipError_t launch_rms_norm_bf16(const void *x, void *y, int64_t rows, int C, const float *gamma,
                                const float *beta, float eps, hipStream_t s) {
    return dispatch<uint16_t, false, false>(x, y, rows, C, gamma, beta, eps, 1, s);
}

hipError_t launch_rmsnorm_silu_f32(const void *x, void *y, int64_t rows, int C, const float *gamma,
                                   const float *beta, float eps, hipStream_t s) {
    return dispatch<float, false>(x, y, rows, C, gamma, beta, eps, 1, s);
}

}  // namespace wanvae
