// Internal launch interface between the C-ABI layer (abi.cpp) and the HIP
// kernels.  Every launcher assumes its arguments were validated by abi.cpp:
// shapes supported, pointers non-null where required and 16-byte aligned.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace wanvae {

// One causal 3x3x3 conv launch.  Activations channels-last.  The optional
// residual source `res` ([n][t][h][w][cres]) is added in the epilogue: as is
// (identity shortcut, cres == cout) when `wsc` is null, or through the 1x1x1
// shortcut weight `wsc` ([cout][cres]) plus `bsc` otherwise.
struct ConvLaunch {
    const void *x = nullptr;      // conv input [n][t][h][w][cin]
    const void *cache = nullptr;  // frames -2, -1: [n][2][h][w][cin], or null
    const void *w = nullptr;      // packed by launch_pack_conv3d_weights
    const float *bias = nullptr;  // [cout] or null
    const void *res = nullptr;    // residual / shortcut input, or null
    const void *wsc = nullptr;    // [cout][cres] or null
    const float *bsc = nullptr;   // [cout] or null
    void *y = nullptr;            // [n][t][h][w][cout]
    int64_t n = 0, t = 0, h = 0, w_ = 0;
    int cin = 0, cout = 0, cres = 0;
    // bf16 only: x and cache frames are [cin/16][h][w][16] (16-channel
    // slices) instead of [h][w][cin]; res and y stay channels-last
    bool x_sliced = false;
    // GEMM launch (launch_gemm_bf16): y = w x + bias (+ res), w plain
    // [cout][cin], x channels-last; cin a multiple of 32, cout of 32
    bool gemm = false;
    // upsampler conv (bf16): h, w_ are the output's (even) sizes, x frames are
    // (h/2) x (w/2) read by nearest neighbour, w packed by
    // launch_pack_conv2d_weights; no cache, no residual
    bool up2 = false;
    // with up2: the frames doubled in time too (upsample3d): t is the
    // output's 2 t_in - 1 frames, x has t_in = (t + 1) / 2 frames per batch
    // item, and output frame t' reads input frame (t' + 1) / 2
    bool up_t = false;
    // bf16 only, conv3d_bf16_norm_supported(cout): y is silu(RMS_norm(conv)),
    // the ResidualBlock's n2, with scale norm_gamma, shift norm_beta (or
    // null) and clamp norm_eps, written in the 16-channel-slice layout
    // [n][t][cout/16][h][w][16]; no residual
    bool norm_out = false;
    const float *norm_gamma = nullptr, *norm_beta = nullptr;
    float norm_eps = 0.0f;
    // bf16 narrow conv only (conv3d_narrow_supported): x and cache hold the
    // input of an RMS_norm + SiLU (scale in_norm_gamma, shift in_norm_beta or
    // null, clamp in_norm_eps) that the conv applies to each position as it
    // reads it (the decoder's norm_out -> SiLU -> conv_out); null: no norm
    const float *in_norm_gamma = nullptr, *in_norm_beta = nullptr;
    float in_norm_eps = 0.0f;
};

// Fused RMS_norm + SiLU over rows of C channels (C % 32 == 0, 32..1024).
bool rmsnorm_silu_supported(int C);
hipError_t launch_rmsnorm_silu_bf16(const void *x, void *y, int64_t rows, int C,
                                    const float *gamma, const float *beta, float eps,
                                    hipStream_t s);
// The same over rows that are the positions of frames of hw positions each,
// writing y in the 16-channel-slice layout the bf16 conv reads:
// y[f][c / 16][q][c % 16] for row f * hw + q.  bf16 only; y must not overlap x.
hipError_t launch_rmsnorm_silu_bf16_sliced(const void *x, void *y, int64_t rows, int C, int64_t hw,
                                           const float *gamma, const float *beta, float eps,
                                           hipStream_t s);
// The norm alone (no SiLU), channels-last bf16 in and out; y == x allowed.
hipError_t launch_rms_norm_bf16(const void *x, void *y, int64_t rows, int C, const float *gamma,
                                const float *beta, float eps, hipStream_t s);
hipError_t launch_rmsnorm_silu_f32(const void *x, void *y, int64_t rows, int C, const float *gamma,
                                   const float *beta, float eps, hipStream_t s);

// bf16 implicit-GEMM conv on MFMA: cin a multiple of 16, any cout (padded to a
// multiple of 32 in the packed weight); cres (the block's shortcut input) a
// multiple of 32.
bool conv3d_bf16_supported(int cin, int cout);
// C_out for which the conv can compute norm2 + SiLU in its epilogue (a tile
// holds every channel of its positions): 32 and 96.
bool conv3d_bf16_norm_supported(int cout);
// The bf16 causal conv for C_out <= 3 (the taps on the MFMA M dimension, then
// a tap sum per output): channels-last x and cache, 16 <= C_in <= 96, C_in a
// multiple of 16; no residual or shortcut.
bool conv3d_narrow_supported(const ConvLaunch &c);
// The upsampler conv by output phase (C_out a multiple of 96): its weight is
// packed as the 4 merged 2 x 2 taps of each of the 4 output phases, and the
// conv runs on the half-resolution input (launch_pack_conv2d_weights and the
// up2 launches agree through this test).
inline bool upsample_by_phase(int cout) { return cout % 96 == 0; }
hipError_t launch_conv3d_narrow(const ConvLaunch &c, hipStream_t s);
hipError_t launch_conv3d_bf16(const ConvLaunch &a, hipStream_t s);

// Bounded flag waits of the bf16 conv: polls per wait before it gives up
// (negative: the default), and the per-device count of waits that gave up
// (read and reset wait for the device to go idle first).
void set_wait_bound(int polls);
hipError_t read_wait_giveups(uint64_t *count);
hipError_t reset_wait_giveups();

// Channel GEMM over positions (a pointwise projection) on the conv kernel's
// 1x1x1 stages: ConvLaunch with gemm = true.
hipError_t launch_gemm_bf16(const ConvLaunch &a, hipStream_t s);
// The same product by the dedicated GEMM kernel (128 positions resident in
// LDS, the weight streamed in 128 x 128 stages): y [P][N] = x [P][K] w[N][K]^T
// + bias (+ res), bf16 channels-last; K in {128, 256, 384}, N a multiple of 64.
// Compute units of the current device (cached per device).
hipError_t device_cu_count(int *out);
bool gemm_bf16_tiled_supported(int K, int N);
hipError_t launch_gemm_bf16_tiled(const void *x, const void *w, const float *bias, const void *res, void *y,
                                  int64_t P, int K, int N, hipStream_t s);

// Attention core of the decoder mid-block (attention.hip): head width D in
// {64, 128, 384}; keys padded to a multiple of 32 in the transposed v.
bool attention_supported(int D);
int64_t attention_keys_padded(int64_t hw);
// vt[f][d][k] = qkv[f][k][2D + d] (zero for HW <= k < HWp)
hipError_t launch_transpose_v(const void *qkv, void *vt, int64_t frames, int HW, int D, hipStream_t s);
// o[f][q] = softmax_k(q . k / sqrt(D)) v over the frame's HW positions
hipError_t launch_flash_attention(const void *qkv, const void *vt, void *o, int64_t frames, int HW, int D,
                                  hipStream_t s);

// Packs PyTorch-layout conv weights [cout][cin][3][3][3] for the conv kernels
// (bf16: [3][cin/16][3][3][cout_p][16], cin % 16 == 0, cout_p = cout rounded
// up to 32 with zero weights in the padding; fp32: [cout][3][3][3][cin]).
int64_t packed_conv3d_weight_elems(int cin, int cout, bool bf16);
// 2D 3x3 weights [cout][cin][3][3] (bf16) -> [cin/16][9][cout_p][16]
int64_t packed_conv2d_weight_elems(int cin, int cout);
hipError_t launch_pack_conv2d_weights(const void *w, void *out, int cin, int cout, hipStream_t s);
hipError_t launch_pack_conv3d_weights(const void *w, void *out, int cin, int cout, bool bf16,
                                      hipStream_t s);

// 1x1x1 conv over rows of channels: y[r][co] = bias[co] + sum_ci w[co][ci] * x[r][ci],
// x, w, y of one dtype, fp32 accumulation; cin, cout in [1, 64]; y must not overlap x.
hipError_t launch_pointwise_conv(const void *x, const void *w, const float *bias, void *y,
                                 int64_t rows, int cin, int cout, bool bf16, hipStream_t s);

// Streaming copy of `bytes` (a multiple of 16) with `unroll` 16-byte pieces
// per lane in flight (1, 2, 4 or 8) and at most blocks_per_cu workgroups of
// 256 lanes per compute unit.
hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, int unroll, int blocks_per_cu,
                              hipStream_t s);

// frames x hw positions x C channels (C % 16 == 0, bf16) between the
// 16-channel-slice layout [frame][C/16][hw][16] and channels-last
// [frame][hw][C]; to_sliced picks the direction.  src and dst must not overlap.
hipError_t launch_cache_layout(const void *src, void *dst, int64_t frames, int64_t hw, int C, bool to_sliced,
                               hipStream_t s);

// fp32 direct conv, any channel counts.
hipError_t launch_conv3d_f32(const ConvLaunch &a, hipStream_t s);

// cache[nb][0..1] <- last two frames of [cache[nb], chunk[nb]] for each batch
// item; a frame is `slab_bytes` bytes (a multiple of 4).
hipError_t launch_roll_cache(void *cache, const void *chunk, int64_t nbatch, int64_t tc,
                             int64_t slab_bytes, hipStream_t s);

}  // namespace wanvae
