/*
 * wanvae.h — C ABI of the Wan 2.2 VAE-decoder ResidualBlock library
 * (libwanvae.so, hand-written HIP kernels for MI355X / gfx950).
 *
 * The block is the decoder's residual unit as described on "Sharding of WAN
 * 2.2 VAE" (Channel sharding: residual = RMS_norm, SiLU, CausalConv3d k3,
 * RMS_norm, SiLU, CausalConv3d k3; shortcut = CausalConv3d k1, or Identity
 * when in_dim == out_dim; output = residual + shortcut), run over all frames
 * at once ("Closing the gap: Wan 2.2 14B VAE decoder", gap #1 / section 1,
 * full-T) or frame-chunk by frame-chunk with a feat_cache ("Sharding of WAN
 * 2.2 VAE", Why depth sharding is not beneficial).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers to dense tensors.  Activations are
 *    channels-last [n][t][h][w][C] (C innermost), the NDHWC layout of
 *    "Closing the gap", gap #6; nothing is permuted inside the library.
 *  - 3x3x3 conv weights are passed PACKED: the buffer that
 *    wanvae_pack_conv3d_weights fills from the pages' [C_out, C_in, kD, kH, kW]
 *    weight ("Sharding of WAN 2.2 VAE", Available Sharding Dimensions; the
 *    PyTorch Conv3d layout).  A packed weight holds the same 27*C_in*C_out
 *    elements of the conv dtype, reordered for the kernel that streams it.
 *    The 1x1x1 shortcut weight is plain [C_out][C_in].
 *  - dtype (wanvae_dtype) applies to activations and conv weights.  Norm
 *    scales/shifts and all biases are fp32 [C].  Arithmetic is fp32 (norm
 *    statistics, conv accumulation, bias and residual adds); bf16 outputs are
 *    rounded once, to nearest even.
 *  - Alignment: every pointer must be 16-byte aligned (torch allocations
 *    are); a misaligned pointer returns WANVAE_ERR_SHAPE.
 *  - Ownership: the caller allocates and owns every buffer (tensors, weights,
 *    caches, workspace).  The library allocates no device memory and keeps no
 *    pointer after a call returns.  Its only device memory of its own is
 *    static, part of its loaded code: the workspace array of
 *    wanvae_resblock_forward_noalloc and the wait give-up counter.
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream).  All
 *    work is enqueued on it; no call synchronizes the device or the stream
 *    (except wanvae_timing_read, which waits for its own events).
 *  - Errors: every entry point validates all arguments on the host before it
 *    enqueues anything and returns a wanvae_status.  On an error nothing has
 *    been enqueued, except WANVAE_ERR_HIP, which reports a launch failure
 *    (earlier launches of the same call may already be enqueued).
 *    wanvae_last_error() describes the most recent failure of this thread.
 *  - Threads: entry points may be called from several host threads; calls
 *    that share output buffers must be ordered by the caller.
 */
#ifndef WANVAE_H
#define WANVAE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define WANVAE_API __attribute__((visibility("default")))
#else
#define WANVAE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WANVAE_OK = 0,
    WANVAE_ERR_NULL = 1,      /* a required pointer is NULL                      */
    WANVAE_ERR_SHAPE = 2,     /* negative extent, unsupported channel count, ... */
    WANVAE_ERR_DTYPE = 3,     /* unknown dtype                                   */
    WANVAE_ERR_ALIAS = 4,     /* an output overlaps an input it must not overlap */
    WANVAE_ERR_WORKSPACE = 5, /* workspace missing or smaller than required      */
    WANVAE_ERR_HIP = 6        /* a HIP launch or runtime call failed             */
} wanvae_status;

typedef enum { WANVAE_F32 = 0, WANVAE_BF16 = 1 } wanvae_dtype;

/* Activation extent: a tensor is [n][t][h][w][C].  Any extent may be 0
 * (an empty tensor: the call does nothing and returns WANVAE_OK). */
typedef struct {
    int64_t n, t, h, w;
} wanvae_dims;

/* Parameters of one ResidualBlock.  All pointers are device pointers. */
typedef struct {
    int32_t in_dim, out_dim;  /* channel counts of x and y                          */
    int32_t dtype;            /* wanvae_dtype of activations and conv weights        */
    float eps;                /* clamp of the channel L2 norm (1e-12 in the decoder) */
    const float *gamma1;      /* [in_dim]  norm1 scale                                */
    const float *beta1;       /* [in_dim]  norm1 shift, or NULL for 0                 */
    const void *w_a;          /* conv A weight (out_dim x in_dim), packed             */
    const float *b_a;         /* [out_dim] conv A bias, or NULL                        */
    const float *gamma2;      /* [out_dim] norm2 scale                                */
    const float *beta2;       /* [out_dim] norm2 shift, or NULL                        */
    const void *w_b;          /* conv B weight (out_dim x out_dim), packed            */
    const float *b_b;         /* [out_dim] conv B bias, or NULL                        */
    const void *w_sc;         /* [out_dim][in_dim] 1x1x1 shortcut weight, or NULL for
                                 the identity shortcut (requires in_dim == out_dim)   */
    const float *b_sc;        /* [out_dim] shortcut bias, or NULL                      */
} wanvae_resblock_params;

/*
 * Fused channel RMS_norm + SiLU over `rows` independent C-vectors:
 *   d = max(sqrt(sum_c x_c^2), eps)
 *   y_c = silu(x_c / d * sqrt(C) * gamma_c + beta_c),  silu(u) = u / (1 + exp(-u))
 * The norm is the F.normalize chain of "Closing the gap", section 4 (RMSNorm
 * not fused: abs, pow 2, sum over channels, sqrt, clamp(eps), divide, scale
 * by sqrt(D)*gamma), with beta added after the scale; SiLU is fused into the
 * same pass as tt-metal's fused norm kernel does (same section).
 *   x, y   : [rows][C] of dtype.  y == x (in place) is allowed; any other
 *            overlap returns WANVAE_ERR_ALIAS.
 *   C      : a multiple of 32 in [32, 1024].
 *   gamma  : [C] fp32; beta: [C] fp32 or NULL.
 */
WANVAE_API int wanvae_rmsnorm_silu(const void *x, void *y, int64_t rows, int32_t C, const float *gamma,
                        const float *beta, float eps, int32_t dtype, void *stream);

/*
 * Packs a 3x3x3 conv weight for wanvae_causal_conv3d and the ResidualBlock
 * calls.  Input: w = [cout][cin][3][3][3] of dtype, the pages' weight layout
 * [C_out, C_in, kD, kH, kW] ("Sharding of WAN 2.2 VAE", Available Sharding
 * Dimensions).  Output: `packed`, wanvae_packed_conv3d_weight_elems elements
 * of dtype, laid out as
 *   fp32: [cout][kt][kh][kw][cin]                    (27*cin*cout elements)
 *   bf16: [kt][cin/16][kh][kw][cout_p][16]           (27*cin*cout_p elements)
 * with cout_p = cout rounded up to a multiple of 32 (the MFMA tile's channel
 * block) and zero weights for the padding channels; cin a multiple of 16 for
 * bf16.  The bf16 order is the MFMA conv's K loop (temporal tap, 16-channel
 * slice, then the 9 spatial taps), so each tap's slice for all output
 * channels is one contiguous run.  Runs one GPU gather kernel on `stream`;
 * meant for set-up, once per weight.  `packed` must not overlap `w`; both are
 * owned by the caller.
 */
WANVAE_API int wanvae_pack_conv3d_weights(const void *w, void *packed, int32_t cin, int32_t cout,
                                          int32_t dtype, void *stream);

/* Elements of a packed conv weight (cin -> cout, dtype): the buffer size
 * wanvae_pack_conv3d_weights fills.  Host only; writes *elems. */
WANVAE_API int wanvae_packed_conv3d_weight_elems(int32_t cin, int32_t cout, int32_t dtype,
                                                 int64_t *elems);

/*
 * Decoder upsampler, spatial part (upsample2d): each frame doubled in H and W
 * by nearest neighbour, then a 3x3 conv with zero padding 1 over the frame
 * ("Sharding of WAN 2.2 VAE": the decoder module tree ends three up blocks
 * with an upsampler, and "Further sharding consideration: WanResample" names
 * its conv, resample[1], with a C_out to split; the tree's channel counts make
 * that conv halve the channels):
 *   y[n][t][h][w][co] = bias[co] + sum_{kh,kw,ci} w[co][ci][kh][kw] *
 *                       x[n][t][(h+kh-1)/2][(w+kw-1)/2][ci]
 * with the terms outside the 2h x 2w image left out.  The doubled image is
 * never stored: the conv reads each input position for the output positions
 * it covers; for cout a multiple of 96 it runs by output phase, 4 merged taps
 * of the input per output (the weights as wanvae_pack_conv2d_weights merges
 * them, rounded to bf16 once).  bf16 only (other dtypes: WANVAE_ERR_DTYPE);
 * fp32 accumulation, bias added in fp32, one RNE rounding.
 * wanvae_upsample3d_conv adds the temporal doubling of upsample3d.
 *   x     : [n][t][h][w][cin] bf16, channels-last (d gives this extent).
 *   w     : packed by wanvae_pack_conv2d_weights (cin x cout).
 *   bias  : [cout] fp32 or NULL.
 *   y     : [n][t][2h][2w][cout] bf16, channels-last; must not overlap x or w.
 *   cin a multiple of 16 in [16, 1024]; cout in [1, 1024]; a frame of x and of
 *   y below 2 GiB.  Asynchronous on `stream`; allocates nothing.
 */
WANVAE_API int wanvae_upsample2d_conv(const void *x, const void *w, const float *bias, void *y,
                                      const wanvae_dims *d, int32_t cin, int32_t cout, int32_t dtype,
                                      void *stream);

/*
 * Decoder upsampler with the frames doubled in time (upsample3d): T frames
 * become 2T - 1, then each frame goes through wanvae_upsample2d_conv's
 * spatial doubling and 3x3 conv.  The pages fix only the frame counts (up
 * blocks 0 and 1 of "Sharding of WAN 2.2 VAE"'s decoder module tree end in
 * upsample3d; 21 latent frames, "Closing the gap", gap #1, become the 81 of
 * the decoded video, "Optimize attention ... WAN 2.2 Training on TPU 7x",
 * inference validation table); the frames are made by nearest neighbour in
 * time with the first kept once:
 *   output frame 0 = input frame 0, output frames 2k - 1 and 2k = input frame k
 * (output frame t' reads input frame (t' + 1) / 2, no later frame), so
 *   y[n][t'][h][w][co] = bias[co] + sum_{kh,kw,ci} w[co][ci][kh][kw] *
 *                        x[n][(t'+1)/2][(h+kh-1)/2][(w+kw-1)/2][ci]
 * with the terms outside the 2h x 2w image left out.  bf16 only; fp32
 * accumulation, one RNE rounding.
 *   x : [n][t][h][w][cin] bf16, channels-last (d gives this extent).
 *   w : packed by wanvae_pack_conv2d_weights; bias: [cout] fp32 or NULL.
 *   y : [n][2t - 1][2h][2w][cout] bf16; must not overlap x or w.
 *   Same channel and frame-size limits as wanvae_upsample2d_conv.
 */
WANVAE_API int wanvae_upsample3d_conv(const void *x, const void *w, const float *bias, void *y,
                                      const wanvae_dims *d, int32_t cin, int32_t cout, int32_t dtype,
                                      void *stream);

/* Packs a 2D 3x3 conv weight [cout][cin][3][3] (bf16) for the upsampler
 * convs.  cout a multiple of 96 (every decoder upsampler): by output phase,
 * [cin/16][phase][a][b][cout_p][16], phase = 2 py + px and (a, b) the 2 x 2
 * taps on the half-resolution input, each the fp32 sum of the 3x3 taps that
 * land on that input position after the nearest x2 doubling (output row
 * 2i + py reads input rows i + py - 1 + a: kernel rows {-1} and {0, +1} for
 * py = 0, {-1, 0} and {+1} for py = 1; columns alike), rounded to bf16 once.
 * Other cout: [cin/16][kh][kw][cout_p][16], the bf16 conv layout with one
 * temporal tap.  cout_p = cout rounded up to 32, zero padding.  Same rules as
 * wanvae_pack_conv3d_weights; bf16 only. */
WANVAE_API int wanvae_pack_conv2d_weights(const void *w, void *packed, int32_t cin, int32_t cout,
                                          int32_t dtype, void *stream);

/* Elements of a packed 2D conv weight: 16*cin*cout_p by phase (cout a
 * multiple of 96), else 9*cin*cout_p.  Host only. */
WANVAE_API int wanvae_packed_conv2d_weight_elems(int32_t cin, int32_t cout, int32_t dtype,
                                                 int64_t *elems);

/*
 * Pointwise (1x1x1) conv over `rows` positions:
 *   y[r][co] = bias[co] + sum_ci w[co][ci] * x[r][ci]
 * The decoder's post_quant_conv, a CausalConv3d of kernel size 1 over the
 * latent channels ("Sharding of WAN 2.2 VAE", the decoder module tree); with
 * kernel size 1 there is no causal pad and no cache.  fp32 accumulation over
 * ascending ci, bias added last, one rounding for bf16 outputs.
 *   x : [rows][cin] of dtype (channels-last positions);  y : [rows][cout] of
 *       dtype, must not overlap x, w or bias.
 *   w : [cout][cin] of dtype;  bias : [cout] fp32 or NULL.
 *   cin, cout in [1, 64] (small-channel kernel: one thread per output value).
 */
WANVAE_API int wanvae_pointwise_conv(const void *x, const void *w, const float *bias, void *y,
                                     int64_t rows, int32_t cin, int32_t cout, int32_t dtype,
                                     void *stream);

/*
 * Causal 3x3x3 convolution, stride 1, with bias:
 *   y[n,t,h,w,co] = bias[co] + sum_{kt,kh,kw,ci} w[co,ci,kt,kh,kw] *
 *                   Z[n, t+kt-2, h+kh-1, w+kw-1, ci]
 * ("Sharding of WAN 2.2 VAE", Available Sharding Dimensions, for the conv and
 * its weight; causal in time, zero pad of one pixel in H and W: "Closing the
 * gap", section 2, the padding mask and causal-T-pad).  Z is x inside the
 * tensor and 0 outside it in H and W.  Frames -2 and -1 are cache[:,0] and
 * cache[:,1] when a cache is given (the feat_cache of "Sharding of WAN 2.2
 * VAE", Why depth sharding is not beneficial), else 0 (causal zero pad).
 *   x     : [d.n][d.t][d.h][d.w][cin] of dtype.
 *   cache : [d.n][2][d.h][d.w][cin] of dtype, or NULL.  Only read.
 *   w     : packed weight (wanvae_pack_conv3d_weights, cin x cout, dtype).
 *   bias  : [cout] fp32 or NULL.
 *   y     : [d.n][d.t][d.h][d.w][cout] of dtype; must not overlap x, cache, w.
 *   Channels: bf16 (MFMA implicit GEMM) needs cin a multiple of 16 in
 *   [16, 1024] and cout in [1, 1024] (the decoder's conv_in, 16 latent
 *   channels in, and conv_out, 3 channels out, included); fp32 (direct
 *   kernel) accepts 1..1024 for both.
 */
WANVAE_API int wanvae_causal_conv3d(const void *x, const void *cache, const void *w, const float *bias,
                         void *y, const wanvae_dims *d, int32_t cin, int32_t cout, int32_t dtype,
                         void *stream);

/*
 * The decoder's tail, norm_out -> SiLU -> conv_out, in one pass ("Sharding of
 * WAN 2.2 VAE", decoder module tree; the norm and SiLU as in "Closing the gap:
 * Wan 2.2 14B VAE decoder", section 4):
 *   n = silu(x / max(||x||_2, eps) * sqrt(cin) * gamma + beta)   per position
 *   y = causal_conv3d(n; w, bias)   (as wanvae_causal_conv3d)
 * The conv reads x and normalises each position as it loads it, so n never
 * goes through memory; n is rounded to bf16 before the products, as the
 * separate wanvae_rmsnorm_silu + wanvae_causal_conv3d would store it.  The
 * conv's zero padding (H, W, and frames before 0 without a cache) applies to
 * n.  bf16 only.
 *   x     : [d.n][d.t][d.h][d.w][cin], the norm's input.
 *   cache : [d.n][2][d.h][d.w][cin], the norm's INPUT for frames -2 and -1
 *           (normalised on the way in like x), or NULL.
 *   gamma : [cin] fp32 (required); beta: [cin] fp32 or NULL; eps >= 0.
 *   w     : packed by wanvae_pack_conv3d_weights(cin, cout, bf16).
 *   bias  : [cout] fp32 or NULL.   y : [..][cout], must not overlap x, cache or w.
 *   cin a multiple of 16 in [16, 96]; cout in [1, 3] (the decoder: 96 -> 3).
 * Asynchronous on `stream`; timed as WANVAE_KERNEL_CONV_BF16.  Errors:
 * WANVAE_ERR_DTYPE (not bf16), WANVAE_ERR_SHAPE, WANVAE_ERR_NULL,
 * WANVAE_ERR_ALIAS; nothing is launched then.
 */
WANVAE_API int wanvae_rmsnorm_silu_conv_out(const void *x, const void *cache, const float *gamma,
                                            const float *beta, float eps, const void *w, const float *bias,
                                            void *y, const wanvae_dims *d, int32_t cin, int32_t cout,
                                            int32_t dtype, void *stream);

/*
 * Workspace bytes that wanvae_resblock_forward / wanvae_resblock_stream_step
 * need for extent *d (for the stream step, d->t is the chunk length), with
 * P = n*t*h*w, two 256-byte aligned regions:
 *   - the conv inputs, P * max(in_dim, out_dim) elements: n1 (conv A's input),
 *     then n2 (conv B's input) once conv A has read n1;
 *   - conv A's output a, P * out_dim elements.
 * For bf16 the norms write n1 and n2 in the MFMA conv's input layout (each
 * frame cut into 16-channel slices, [C/16][h][w][16]); for fp32 n1 is
 * channels-last and n2 is a normalised in place.  Validates p and d as the
 * forward call does.
 */
WANVAE_API int wanvae_resblock_workspace_size(const wanvae_resblock_params *p, const wanvae_dims *d,
                                   size_t *bytes);

/*
 * Whole ResidualBlock over every frame in one pass (full-T, no cache):
 *   n1 = rmsnorm_silu(x; gamma1, beta1); a = conv3d(n1; w_a, b_a)
 *   n2 = rmsnorm_silu(a; gamma2, beta2)
 *   y  = conv3d(n2; w_b, b_b) + shortcut(x)
 * shortcut(x) = x for the identity, else w_sc . x + b_sc per position; the
 * shortcut reads the block's original input ("Sharding of WAN 2.2 VAE",
 * Channel sharding and the op-sequence diagram; "Closing the gap", gap #6:
 * the 1x1x1 conv is a matmul).  Conv B's accumulator, its bias and the
 * shortcut are summed in fp32 and rounded once.
 *   x : [d.n][d.t][d.h][d.w][in_dim];  y : [..][out_dim]; y must not overlap x.
 *   workspace: device buffer of at least wanvae_resblock_workspace_size bytes.
 * Kernel launches on `stream`: norm1 (into the conv input region), conv A
 * (into the region of a), norm2 (a into the conv input region; for fp32, a
 * normalised in place), then conv B with the residual add in its epilogue.
 * For bf16 with out_dim 96 or 32 conv A computes norm2 + SiLU in its own
 * epilogue and writes conv B's input directly (a is never stored, no norm2
 * launch).  The 1x1x1 shortcut is added in conv B's epilogue too: computed
 * inside conv B's K loop, or, for bf16 with in_dim 128, 256 or 384 and
 * out_dim a multiple of 64, by a projection GEMM launched ahead of conv B
 * into the region of a (free once norm2 has read it), S rounded to bf16 and
 * then added like the identity residual.  Three to five launches in all.
 */
WANVAE_API int wanvae_resblock_forward(const wanvae_resblock_params *p, const void *x, void *y,
                            const wanvae_dims *d, void *workspace, size_t ws_bytes, void *stream);

/*
 * wanvae_resblock_forward for callers that cannot allocate device memory:
 * code under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace; the block's intermediates live in a
 * device array of the library's own (64 MiB, held by each GPU the library
 * runs on until the process ends), so only blocks whose
 * wanvae_resblock_workspace_size is at most 64 MiB are accepted (else
 * WANVAE_ERR_WORKSPACE, nothing enqueued).  The call allocates nothing and
 * is never timed (wanvae_timing_*); its first call on a device looks the
 * array's address up once.  Same kernels and results as
 * wanvae_resblock_forward.  Every call on one device shares that array:
 * calls that overlap on a device (other streams, other threads) race and
 * must be ordered by the caller.  Nothing in it needs clearing between calls.
 * The current device must be the one `stream` belongs to.
 */
WANVAE_API int wanvae_resblock_forward_noalloc(const wanvae_resblock_params *p, const void *x, void *y,
                                               const wanvae_dims *d, void *stream);

/*
 * One streaming step over a chunk of d->t >= 1 frames with the feat_cache
 * ("Sharding of WAN 2.2 VAE", Why depth sharding is not beneficial: one frame
 * at a time with a cache of the last frames of every CausalConv3d's input;
 * "Closing the gap", section 1: the per-frame decode loop carrying feat_cache).
 *   cache_a : d.n*2*d.h*d.w*in_dim elements: conv A input frames -2, -1 (in/out)
 *   cache_b : d.n*2*d.h*d.w*out_dim elements: conv B input frames -2, -1 (in/out)
 * Each conv reads its cache as the two frames before the chunk; afterwards
 * the cache holds the last two frames of [cache, this chunk's conv input].
 * The frames are stored as the library stores conv inputs: [n][2][h][w][C]
 * for fp32, [n][2][C/16][h][w][16] (16-channel slices) for bf16; callers
 * treat the caches as opaque buffers of that many elements and read or set
 * their frames channels-last with wanvae_stream_cache_export / _import.  A
 * fresh stream starts from zero-filled caches (zero is the causal pad in
 * either layout), so running a clip chunk by chunk gives the full-T result.
 * Caches must not overlap each other, x, y or the workspace.
 */
WANVAE_API int wanvae_resblock_stream_step(const wanvae_resblock_params *p, const void *x_chunk,
                                void *y_chunk, const wanvae_dims *d, void *cache_a, void *cache_b,
                                void *workspace, size_t ws_bytes, void *stream);

/*
 * A stream cache's frames, channels-last.  The feat_cache is the streaming
 * decoder's only state ("Sharding of WAN 2.2 VAE", Why depth sharding is not
 * beneficial: the last frames of every CausalConv3d's input); these calls let
 * a caller save it and resume later, or seed it from frames of its own.
 *   export: out = the cache's frames -2, -1 as [d.n][2][d.h][d.w][C];
 *   import: the cache set from in = [d.n][2][d.h][d.w][C].
 * C is in_dim for cache_a and out_dim for cache_b (a multiple of 16 for
 * bf16); d.t is ignored.  For bf16 a permutation kernel on `stream` (bit for
 * bit); for fp32, whose caches are channels-last already, a device copy on
 * `stream`.  Device pointers, 16-byte aligned, not overlapping; asynchronous.
 */
WANVAE_API int wanvae_stream_cache_export(const void *cache, void *out, const wanvae_dims *d, int32_t C,
                                          int32_t dtype, void *stream);
WANVAE_API int wanvae_stream_cache_import(const void *in, void *cache, const wanvae_dims *d, int32_t C,
                                          int32_t dtype, void *stream);

/* Parameters of the decoder mid-block attention block (bf16).  All pointers
 * are device pointers. */
typedef struct {
    int32_t dim;              /* C: channels = head width (64, 128 or 384)        */
    float eps;                /* clamp of the channel L2 norm                       */
    const float *gamma;       /* [dim] norm scale                                   */
    const float *beta;        /* [dim] norm shift, or NULL                          */
    const void *w_qkv;        /* [3*dim][dim] bf16: rows of q, then k, then v       */
    const float *b_qkv;       /* [3*dim] or NULL                                     */
    const void *w_o;          /* [dim][dim] bf16 output projection                  */
    const float *b_o;         /* [dim] or NULL                                       */
} wanvae_attention_params;

/*
 * Workspace bytes of wanvae_attention_block for extent *d (P = n*t*h*w
 * positions, F = n*t frames, HWp = h*w rounded up to 32): u [P][C], qkv
 * [P][3C], v transposed per frame [F][C][HWp] and o [P][C], bf16, each region
 * 256-byte aligned.
 */
WANVAE_API int wanvae_attention_workspace_size(const wanvae_attention_params *p, const wanvae_dims *d,
                                               size_t *bytes);

/*
 * The decoder mid-block's attention block over every frame ("Closing the gap:
 * Wan 2.2 14B VAE decoder", section 5: a spatial self-attention in which,
 * within a frame, every position attends to every other, the sequence being
 * the H*W grid and each (batch, frame) an independent problem; "Sharding of
 * WAN 2.2 VAE", decoder module tree: WanAttentionBlock(384)).  The pages give
 * no more; this computes, per frame and position i:
 *   u = RMS_norm(x; gamma, beta)               (the decoder's norm, no SiLU)
 *   [q | k | v] = w_qkv u + b_qkv              (1x1x1 projection)
 *   o_i = sum_j softmax_j(q_i . k_j / sqrt(C)) v_j   (one head, all H*W j)
 *   y_i = x_i + w_o o_i + b_o
 * bf16 activations and weights, fp32 norm statistics, accumulation and
 * softmax; u, q, k, v, o and y rounded to bf16.
 *   x, y: [d.n][d.t][d.h][d.w][dim] bf16, channels-last; y must not overlap x.
 * Five launches on `stream`: norm, q/k/v projection (MFMA GEMM), v transpose,
 * flash attention (MFMA, scores kept on chip), output projection with the
 * residual add (MFMA GEMM).
 */
WANVAE_API int wanvae_attention_block(const wanvae_attention_params *p, const void *x, void *y,
                                      const wanvae_dims *d, void *workspace, size_t ws_bytes, void *stream);

/*
 * Bounded waits.  The bf16 conv's waves synchronise through flags in LDS
 * (stage landed / stage consumed), and every wait on a flag is bounded so a
 * launch can never hang.  A wait that reaches its bound goes on and is
 * counted: the launch's output is then suspect.
 *   wanvae_wait_giveups: waits for the current device to go idle, then
 *     writes the number of waits that gave up on it since the library was
 *     loaded or the count was last reset.  Zero means no launch on this device
 *     left its synchronisation protocol.
 *   wanvae_wait_giveups_reset: waits for the device to go idle, sets the
 *     count to zero.
 *   wanvae_set_wait_bound: polls (about 64 cycles apart) before a wait gives
 *     up, for launches enqueued after the call, process-wide; negative
 *     restores the default (2^15 polls, about 2M cycles, far beyond any real
 *     wait).  A test hook: a bound of 0 makes the waits give up at once, so
 *     that the counting can be checked from the host (the kernels still run
 *     to completion, their results then meaningless).
 */
WANVAE_API int wanvae_wait_giveups(uint64_t *count);
WANVAE_API int wanvae_wait_giveups_reset(void);
WANVAE_API int wanvae_set_wait_bound(int32_t polls);

/*
 * A plain streaming copy, for measurement: dst = src over `bytes` bytes, each
 * read once and written once, as the fused RMS_norm + SiLU reads its input
 * and writes its output.  Its rate is the attainable HBM rate that the
 * library's bandwidth-bound kernels are compared with (the 8 TB/s of the HBM
 * specification is not reached by any copy).  16-byte nontemporal accesses
 * per lane, `unroll` (1, 2, 4 or 8) of them in flight, at most blocks_per_cu
 * (1..64) workgroups of 256 lanes per compute unit, striding over the buffer.
 *   src, dst: device pointers, 16-byte aligned, not overlapping; bytes a
 *   multiple of 16.  Asynchronous on `stream`; timed as WANVAE_KERNEL_COPY.
 */
WANVAE_API int wanvae_stream_copy(const void *src, void *dst, int64_t bytes, int32_t unroll,
                                  int32_t blocks_per_cu, void *stream);

/* Text of this thread's most recent error (library-owned, valid until the
 * thread's next call into the library).  "" when there was none. */
WANVAE_API const char *wanvae_last_error(void);

/*
 * Per-kernel timing, for measurement.  While enabled, every kernel the
 * library launches is bracketed by a pair of hipEvents recorded on the same
 * stream.  wanvae_timing_read waits for the recorded events and returns, for
 * one kernel kind, the number of launches and their summed duration in ms.
 * Kinds: 0 = fused RMS_norm+SiLU, 1 = bf16 MFMA conv, 2 = fp32 conv,
 * 3 = cache roll, 4 = pointwise conv, 5 = attention projection GEMM,
 * 6 = v transpose, 7 = flash attention, 8 = upsampler conv, 9 = stream copy.
 * wanvae_timing_reset forgets all records; at most 65536 launches are
 * recorded between resets (later ones go untimed).  Timing state is process-wide; enable it only while one thread
 * drives the library.
 */
enum { WANVAE_KERNEL_NORM = 0, WANVAE_KERNEL_CONV_BF16 = 1, WANVAE_KERNEL_CONV_F32 = 2,
       WANVAE_KERNEL_ROLL = 3, WANVAE_KERNEL_POINTWISE = 4, WANVAE_KERNEL_GEMM = 5,
       WANVAE_KERNEL_TRANSPOSE = 6, WANVAE_KERNEL_ATTENTION = 7, WANVAE_KERNEL_UPSAMPLE = 8,
       WANVAE_KERNEL_COPY = 9, WANVAE_KERNEL_KINDS = 10 };
WANVAE_API int wanvae_timing_enable(int on);
WANVAE_API int wanvae_timing_reset(void);
WANVAE_API int wanvae_timing_read(int32_t kind, int64_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* WANVAE_H */
