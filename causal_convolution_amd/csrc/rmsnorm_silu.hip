// Fused channel RMS_norm + SiLU, HBM-bound.
//
// Per C-vector v (one NDHWC position):
//   d = max(sqrt(sum_c v_c^2), eps),  u_c = v_c * (sqrt(C) / d) * gamma_c + beta_c,
//   y_c = u_c / (1 + exp(-u_c))
// which is the F.normalize-based RMS_norm of "Closing the gap: Wan 2.2 14B VAE
// decoder", section 4, with SiLU fused into the same pass as that section
// describes for tt-metal's kernel.
//
// Mapping: a row of C channels is owned by a group of 16 consecutive lanes,
// each holding E = C/16 contiguous channels, so one wavefront works on 4 rows
// and every load instruction of the wavefront covers 4 x 2C contiguous bytes.
// The sum of squares is reduced across the 16 lanes with xor shuffles (no LDS).
// gamma * sqrt(C) and beta are held in registers for the whole grid-stride
// loop; each lane keeps U rows in flight to cover HBM latency.  y may equal x
// (in place): each element is read and then written by the same lane.  x is read once
// and y written once: 2 * rows * C * sizeof(T) bytes of HBM traffic.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

constexpr int kLanesPerRow = 16;
constexpr int kThreads = 256;
constexpr int kRowsPerPass = kThreads / kLanesPerRow;  // 16 rows per block per pass



// Load NDW dwords from a pointer aligned to VW dwords.
template <int NDW, int VW>
__device__ inline void load_dwords(const uint32_t *__restrict__ p, uint32_t (&d)[NDW]) {
#pragma unroll
    for (int i = 0; i < NDW; i += VW) {
        if constexpr (VW == 4) {
            uint4 q = *reinterpret_cast<const uint4 *>(p + i);
            d[i] = q.x; d[i + 1] = q.y; d[i + 2] = q.z; d[i + 3] = q.w;
        } else if constexpr (VW == 2) {
            uint2 q = *reinterpret_cast<const uint2 *>(p + i);
            d[i] = q.x; d[i + 1] = q.y;
        } else {
            d[i] = p[i];
        }
    }
}

template <int NDW, int VW>
__device__ inline void store_dwords(uint32_t *__restrict__ p, const uint32_t (&d)[NDW]) {
#pragma unroll
    for (int i = 0; i < NDW; i += VW) {
        if constexpr (VW == 4) {
            *reinterpret_cast<uint4 *>(p + i) = make_uint4(d[i], d[i + 1], d[i + 2], d[i + 3]);
        } else if constexpr (VW == 2) {
            *reinterpret_cast<uint2 *>(p + i) = make_uint2(d[i], d[i + 1]);
        } else {
            p[i] = d[i];
        }
    }
}

constexpr int pow2_vec(int ndw) { return ndw % 4 == 0 ? 4 : (ndw % 2 == 0 ? 2 : 1); }

// Per-element storage traits: E elements as NDW dwords.
template <typename T, int E> struct Row;

template <int E> struct Row<float, E> {
    static constexpr int NDW = E;
    static __device__ inline void unpack(const uint32_t (&d)[NDW], float (&v)[E]) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = __uint_as_float(d[e]);
    }
    static __device__ inline void pack(const float (&v)[E], uint32_t (&d)[NDW]) {
#pragma unroll
        for (int e = 0; e < E; ++e) d[e] = __float_as_uint(v[e]);
    }
};

template <int E> struct Row<uint16_t, E> {  // bf16 bits
    static_assert(E % 2 == 0, "bf16 rows need an even count per lane");
    static constexpr int NDW = E / 2;
    static __device__ inline void unpack(const uint32_t (&d)[NDW], float (&v)[E]) {
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            v[2 * i] = bf16_bits_to_f32(d[i] & 0xffffu);
            v[2 * i + 1] = bf16_bits_to_f32(d[i] >> 16);
        }
    }
    static __device__ inline void pack(const float (&v)[E], uint32_t (&d)[NDW]) {
#pragma unroll
        for (int i = 0; i < NDW; ++i)
            d[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
    }
};

// E consecutive fp32 values (16-byte aligned when E is a multiple of 4, 8-byte when even).
template <int E>
__device__ inline void load_params(const float *__restrict__ p, float (&v)[E]) {
    constexpr int VW = E % 4 == 0 ? 4 : (E % 2 == 0 ? 2 : 1);
    uint32_t d[E];
    load_dwords<E, VW>(reinterpret_cast<const uint32_t *>(p), d);
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = __uint_as_float(d[e]);
}

__device__ inline float silu(float u) {
    // u / (1 + exp(-u)); exp(-u) = inf for very negative u gives -0
    return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

template <typename T, int E, int U>
__global__ __launch_bounds__(kThreads) void rmsnorm_silu_kernel(
    const T *x, T *y, int64_t rows, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, float sqrt_c) {
    using R = Row<T, E>;
    constexpr int NDW = R::NDW;
    constexpr int VW = pow2_vec(NDW);
    constexpr int C = E * kLanesPerRow;
    constexpr int ROW_DW = C * (int)sizeof(T) / 4;

    const int lane = threadIdx.x % kLanesPerRow;
    const int slot = threadIdx.x / kLanesPerRow;

    // gamma * sqrt(C) and beta for this lane's E channels, loaded once
    float g[E], b[E];
    load_params<E>(gamma + lane * E, g);
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] *= sqrt_c;
    if (beta) {
        load_params<E>(beta + lane * E, b);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) b[e] = 0.0f;
    }

    const uint32_t *xs = reinterpret_cast<const uint32_t *>(x);
    uint32_t *ys = reinterpret_cast<uint32_t *>(y);
    const int64_t step = (int64_t)gridDim.x * kRowsPerPass * U;

    for (int64_t r0 = (int64_t)blockIdx.x * kRowsPerPass * U; r0 < rows; r0 += step) {
        uint32_t d[U][NDW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = r0 + u * kRowsPerPass + slot;
            if (r < rows) {
                load_dwords<NDW, VW>(xs + r * ROW_DW + lane * NDW, d[u]);
            } else {
#pragma unroll
                for (int i = 0; i < NDW; ++i) d[u][i] = 0u;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = r0 + u * kRowsPerPass + slot;
            float v[E];
            R::unpack(d[u], v);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) ss = fmaf(v[e], v[e], ss);
            // all 64 lanes take part: the xor masks stay inside each 16-lane group
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            ss += __shfl_xor(ss, 8);
            const float inv = 1.0f / fmaxf(sqrtf(ss), eps);
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = silu(fmaf(v[e] * inv, g[e], b[e]));
            uint32_t o[NDW];
            R::pack(v, o);
            if (r < rows) store_dwords<NDW, VW>(ys + r * ROW_DW + lane * NDW, o);
        }
    }
}

template <typename T, int E>
hipError_t launch_e(const void *x, void *y, int64_t rows, int C, const float *gamma,
                    const float *beta, float eps, hipStream_t s) {
    // rows in flight per lane: at least ~96 bytes of loads outstanding per lane
    constexpr int ROW_BYTES = E * (int)sizeof(T);
    constexpr int U = ROW_BYTES >= 96 ? 1 : (96 + ROW_BYTES - 1) / ROW_BYTES > 8 ? 8
                                                 : (96 + ROW_BYTES - 1) / ROW_BYTES;
    const int64_t per_block = (int64_t)kRowsPerPass * U;
    int64_t blocks = (rows + per_block - 1) / per_block;
    // a resident grid (8 blocks of 256 threads per CU on 256 CUs) that strides over the rows
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    rmsnorm_silu_kernel<T, E, U><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
        static_cast<const T *>(x), static_cast<T *>(y), rows, gamma, beta, eps,
        sqrtf((float)C));
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const void *x, void *y, int64_t rows, int C, const float *gamma,
                    const float *beta, float eps, hipStream_t s) {
    switch (C / kLanesPerRow) {
#define WANVAE_NORM_CASE(E) \
    case E: return launch_e<T, E>(x, y, rows, C, gamma, beta, eps, s);
        WANVAE_NORM_CASE(2) WANVAE_NORM_CASE(4) WANVAE_NORM_CASE(6) WANVAE_NORM_CASE(8)
        WANVAE_NORM_CASE(10) WANVAE_NORM_CASE(12) WANVAE_NORM_CASE(14) WANVAE_NORM_CASE(16)
        WANVAE_NORM_CASE(18) WANVAE_NORM_CASE(20) WANVAE_NORM_CASE(22) WANVAE_NORM_CASE(24)
        WANVAE_NORM_CASE(26) WANVAE_NORM_CASE(28) WANVAE_NORM_CASE(30) WANVAE_NORM_CASE(32)
        WANVAE_NORM_CASE(34) WANVAE_NORM_CASE(36) WANVAE_NORM_CASE(38) WANVAE_NORM_CASE(40)
        WANVAE_NORM_CASE(42) WANVAE_NORM_CASE(44) WANVAE_NORM_CASE(46) WANVAE_NORM_CASE(48)
        WANVAE_NORM_CASE(50) WANVAE_NORM_CASE(52) WANVAE_NORM_CASE(54) WANVAE_NORM_CASE(56)
        WANVAE_NORM_CASE(58) WANVAE_NORM_CASE(60) WANVAE_NORM_CASE(62) WANVAE_NORM_CASE(64)
#undef WANVAE_NORM_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool rmsnorm_silu_supported(int C) { return C >= 32 && C <= 1024 && C % 32 == 0; }

hipError_t launch_rmsnorm_silu_bf16(const void *x, void *y, int64_t rows, int C,
                                    const float *gamma, const float *beta, float eps,
                                    hipStream_t s) {
    return dispatch<uint16_t>(x, y, rows, C, gamma, beta, eps, s);
}

hipError_t launch_rmsnorm_silu_f32(const void *x, void *y, int64_t rows, int C, const float *gamma,
                                   const float *beta, float eps, hipStream_t s) {
    return dispatch<float>(x, y, rows, C, gamma, beta, eps, s);
}

}  // namespace wanvae
