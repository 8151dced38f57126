/*
 * CPU oracle for the Wan 2.2 VAE-decoder ResidualBlock (causal Conv3d).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference that the
 * HIP library is checked against.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the product path never
 * does.  It shares no code, header, table or helper with the HIP library.
 *
 * Arithmetic: every value is stored as fp32 (inputs, intermediates, outputs);
 * every reduction (the channel sum of squares, the convolution sum, the
 * shortcut dot product) is accumulated in fp64 in ascending index order and
 * rounded to fp32 once.  Each output element is computed by exactly one
 * thread, in a fixed order, so results do not depend on the thread count.
 *
 * Layouts: activations are channels-last, [N][T][H][W][C] (C innermost), the
 * layout both pages describe for the convolution ("Closing the gap", gap #6:
 * NDHWC end-to-end).  Conv weights keep the pages' own order
 * [C_out][C_in][kD][kH][kW] ("Sharding of WAN 2.2 VAE", Conv3D Sharding
 * Strategy, Available Sharding Dimensions).  A 1x1x1 shortcut weight is
 * [C_out][C_in].
 *
 * What each function follows is cited in its comment.  Readings of points the
 * pages leave open are stated where they are used.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Parameters of one ResidualBlock.                                          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int cin, cout;        /* in_dim, out_dim */
    double eps;           /* clamp of the channel L2 norm */
    const float *gamma1;  /* [cin]                       */
    const float *beta1;   /* [cin] or NULL (= 0)         */
    const float *wa;      /* [cout][cin][3][3][3]        */
    const float *ba;      /* [cout] or NULL              */
    const float *gamma2;  /* [cout]                      */
    const float *beta2;   /* [cout] or NULL              */
    const float *wb;      /* [cout][cout][3][3][3]       */
    const float *bb;      /* [cout] or NULL              */
    const float *ws;      /* [cout][cin] or NULL: NULL means identity shortcut */
    const float *bs;      /* [cout] or NULL              */
} oracle_block;

/*
 * A stored region of a channels-last activation tensor whose full extent is
 * [N][T][H][W][C].  The region holds frames [t0, t0+nt), rows [h0, h0+nh) and
 * columns [w0, w0+nw) of every batch item, packed as [N][nt][nh][nw][C].
 */
typedef struct {
    const float *data;
    int64_t N, T, H, W, C;     /* full extent                    */
    int64_t t0, h0, w0;        /* origin of the stored region    */
    int64_t nt, nh, nw;        /* extent of the stored region    */
} oracle_field;

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* SiLU.  The pages name it as the activation after each RMS_norm            */
/* ("Sharding of WAN 2.2 VAE", Channel sharding: the ResidualBlock           */
/* structure) and never define it; this is its standard definition           */
/* x * sigmoid(x) = x / (1 + exp(-x)), evaluated in fp64.                    */
/* ------------------------------------------------------------------------ */
double oracle_silu(double u)
{
    return u / (1.0 + exp(-u));
}

/* ------------------------------------------------------------------------ */
/* RMS_norm over the channel axis followed by SiLU, for one C-vector.        */
/*                                                                           */
/* "Closing the gap", section 4 (RMSNorm not fused) spells the norm out as   */
/* the chain abs -> pow 2 -> sum over channels -> sqrt -> clamp(eps) ->      */
/* divide -> scale by sqrt(D)*gamma, and says the sqrt(D) factor makes it    */
/* RMSNorm.  D is the size of the normalised (channel) axis, here C.  The    */
/* affine shift beta is added after the scale (beta = 0 reduces to the       */
/* pages' chain).  abs() before squaring changes nothing and is omitted.     */
/* The clamp applies to the L2 norm itself, so a zero vector maps to beta.   */
/* ------------------------------------------------------------------------ */
static double rms_denominator(const float *v, int C, double eps)
{
    double ss = 0.0;
    for (int c = 0; c < C; ++c) ss += (double)v[c] * (double)v[c];
    double r = sqrt(ss);
    return r > eps ? r : eps;
}

static double norm_value(float vc, double d, int C, float gamma_c, const float *beta, int c)
{
    return (double)vc / d * sqrt((double)C) * (double)gamma_c + (beta ? (double)beta[c] : 0.0);
}

/* rows independent C-vectors, packed [rows][C]: y = round_fp32(norm(x)). */
void oracle_rms_norm(const float *x, float *y, int64_t rows, int C, const float *gamma,
                     const float *beta, double eps)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *v = x + r * (int64_t)C;
        double d = rms_denominator(v, C, eps);
        for (int c = 0; c < C; ++c)
            y[r * (int64_t)C + c] = (float)norm_value(v[c], d, C, gamma[c], beta, c);
    }
}

/* rows independent C-vectors, packed [rows][C]: y = round_fp32(silu(norm(x))),
 * with the norm value kept in fp64 up to the single rounding. */
void oracle_norm_silu(const float *x, float *y, int64_t rows, int C, const float *gamma,
                      const float *beta, double eps)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *v = x + r * (int64_t)C;
        double d = rms_denominator(v, C, eps);
        for (int c = 0; c < C; ++c)
            y[r * (int64_t)C + c] = (float)oracle_silu(norm_value(v[c], d, C, gamma[c], beta, c));
    }
}

/* ------------------------------------------------------------------------ */
/* Value of the causal conv's (padded) input at one index.                   */
/*                                                                           */
/* The 3x3x3 conv is causal in time and zero-padded by one pixel in H and W  */
/* ("Closing the gap", section 2: the halo exchange folds in the padding     */
/* mask and the causal-T-pad; "Sharding of WAN 2.2 VAE", Spatial sharding:   */
/* a kernel of size k needs (k-1)/2 border elements per side).  Frames       */
/* before the first one are the feat_cache ("Sharding of WAN 2.2 VAE", Why   */
/* depth sharding is not beneficial: the cache holds the last one or two     */
/* frames of each CausalConv3d's input), or zero when no cache is given.     */
/* The cache is [N][2][H][W][C]; its frame 0 stands for frame -2 and its     */
/* frame 1 for frame -1.  Padding is applied to the conv input, i.e. after   */
/* the norm and SiLU, so a padded position is 0, not silu(beta).             */
/* ------------------------------------------------------------------------ */
static const float *field_ptr(const oracle_field *f, const float *cache, int64_t n, int64_t t,
                              int64_t h, int64_t w)
{
    if (h < 0 || h >= f->H || w < 0 || w >= f->W) return NULL;         /* spatial zero pad */
    if (t < 0) {
        if (!cache) return NULL;                                         /* causal zero pad  */
        if (t < -2) { fprintf(stderr, "oracle: frame %lld before the 2-frame cache\n", (long long)t); abort(); }
        return cache + ((((n * 2 + (t + 2)) * f->H + h) * f->W + w) * f->C);
    }
    if (t >= f->T) { fprintf(stderr, "oracle: frame %lld past the end\n", (long long)t); abort(); }
    int64_t lt = t - f->t0, lh = h - f->h0, lw = w - f->w0;
    if (lt < 0 || lt >= f->nt || lh < 0 || lh >= f->nh || lw < 0 || lw >= f->nw) {
        fprintf(stderr, "oracle: read (%lld,%lld,%lld) outside the stored region\n",
                (long long)t, (long long)h, (long long)w);
        abort();
    }
    return f->data + ((((n * f->nt + lt) * f->nh + lh) * f->nw + lw) * f->C);
}

/*
 * Causal 3x3x3 convolution sum at one output element, without bias:
 *   sum over kt, kh, kw in 0..2 and ci of
 *     W[co][ci][kt][kh][kw] * Z[n][t+kt-2][h+kh-1][w+kw-1][ci]
 * ("Sharding of WAN 2.2 VAE", Available Sharding Dimensions: weight
 * [C_out, C_in, kD, kH, kW]; the conv is a cross-correlation as in PyTorch's
 * Conv3d, and kt = 2 is the current frame so only past frames are read).
 * Accumulated in fp64 in ascending (kt, kh, kw, ci) order; a padded input
 * contributes W * 0.
 */
static double conv3_sum(const oracle_field *z, const float *cache, const float *wt, int cin,
                        int64_t n, int64_t t, int64_t h, int64_t w, int co)
{
    double acc = 0.0;
    for (int kt = 0; kt < 3; ++kt)
        for (int kh = 0; kh < 3; ++kh)
            for (int kw = 0; kw < 3; ++kw) {
                const float *zp = field_ptr(z, cache, n, t + kt - 2, h + kh - 1, w + kw - 1);
                for (int ci = 0; ci < cin; ++ci) {
                    double wv = (double)wt[(((int64_t)co * cin + ci) * 3 + kt) * 9 + kh * 3 + kw];
                    double zv = zp ? (double)zp[ci] : 0.0;
                    acc += wv * zv;
                }
            }
    return acc;
}

/*
 * Shortcut branch at one output element.  Identity when in_dim == out_dim
 * ("Sharding of WAN 2.2 VAE", the op-sequence diagram: conv_shortcut is
 * Identity when in_dim == out_dim); otherwise the 1x1x1 CausalConv3d, which
 * is a plain matmul over channels per position ("Closing the gap", gap #6:
 * 1x1 convs are Linear).  A kernel of size 1 reads only the current frame.
 */
static double shortcut_at(const oracle_block *p, const oracle_field *x, int64_t n, int64_t t,
                          int64_t h, int64_t w, int co)
{
    const float *xp = field_ptr(x, NULL, n, t, h, w);
    if (!p->ws) return (double)xp[co];
    double acc = 0.0;
    for (int ci = 0; ci < p->cin; ++ci)
        acc += (double)p->ws[(int64_t)co * p->cin + ci] * (double)xp[ci];
    return acc + (p->bs ? (double)p->bs[co] : 0.0);
}

/*
 * One causal conv over an output box [ot0,ot0+ont) x [oh0,..) x [ow0,..),
 * written packed as [N][ont][onh][onw][cout].  The result is rounded to fp32
 * once: y = round(sum + bias) when resid == NULL (conv A), or
 * y = round(sum + bias + shortcut(x)) (conv B with the residual add: the
 * shortcut reads the block's original input, "Sharding of WAN 2.2 VAE",
 * Channel sharding: "return residual + shortcut").
 */
static void conv3_box(const oracle_field *z, const float *cache, const float *wt,
                      const float *bias, int cout, int64_t ot0, int64_t oh0, int64_t ow0,
                      int64_t ont, int64_t onh, int64_t onw, float *out,
                      const oracle_block *resid_p, const oracle_field *resid_x)
{
    int cin = (int)z->C;
    int64_t N = z->N;
    #pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t lt = 0; lt < ont; ++lt)
            for (int64_t lh = 0; lh < onh; ++lh)
                for (int64_t lw = 0; lw < onw; ++lw) {
                    int64_t t = ot0 + lt, h = oh0 + lh, w = ow0 + lw;
                    float *o = out + ((((n * ont + lt) * onh + lh) * onw + lw) * cout);
                    for (int co = 0; co < cout; ++co) {
                        double v = conv3_sum(z, cache, wt, cin, n, t, h, w, co);
                        v += bias ? (double)bias[co] : 0.0;
                        if (resid_x) v += shortcut_at(resid_p, resid_x, n, t, h, w, co);
                        o[co] = (float)v;
                    }
                }
}

/* Public single conv: x [N][T][H][W][cin] (whole tensor), optional cache
 * [N][2][H][W][cin], w [cout][cin][3][3][3], bias [cout] or NULL,
 * y [N][T][H][W][cout]. */
void oracle_causal_conv3d(const float *x, const float *cache, const float *w, const float *bias,
                          float *y, int64_t N, int64_t T, int64_t H, int64_t W, int cin, int cout)
{
    oracle_field z = {x, N, T, H, W, cin, 0, 0, 0, T, H, W};
    conv3_box(&z, cache, w, bias, cout, 0, 0, 0, T, H, W, y, NULL, NULL);
}

/* 1x1x1 shortcut or identity alone, for testing the branch by itself. */
void oracle_shortcut(const oracle_block *p, const float *x, float *y, int64_t N, int64_t T,
                     int64_t H, int64_t W)
{
    oracle_field xf = {x, N, T, H, W, p->cin, 0, 0, 0, T, H, W};
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t w = 0; w < W; ++w)
                    for (int co = 0; co < p->cout; ++co)
                        y[((((n * T + t) * H + h) * W + w) * p->cout) + co] =
                            (float)shortcut_at(p, &xf, n, t, h, w, co);
}

/* ------------------------------------------------------------------------ */
/* Whole ResidualBlock, full-T: every frame in one pass, no cache            */
/* ("Closing the gap", gap #1 and section 1: full-T temporal pass).          */
/*   n1 = silu(norm1(x)); a = convA(n1) + bA; n2 = silu(norm2(a));           */
/*   y  = convB(n2) + bB + shortcut(x)                                       */
/* ("Sharding of WAN 2.2 VAE", Channel sharding: the residual Sequential     */
/* and "return residual + shortcut").                                         */
/* ------------------------------------------------------------------------ */
void oracle_resblock_full(const oracle_block *p, const float *x, float *y, int64_t N, int64_t T,
                          int64_t H, int64_t W)
{
    int64_t P = N * T * H * W;
    float *n1 = (float *)malloc(sizeof(float) * (size_t)(P * p->cin));
    float *a = (float *)malloc(sizeof(float) * (size_t)(P * p->cout));
    float *n2 = (float *)malloc(sizeof(float) * (size_t)(P * p->cout));
    if (!n1 || !a || !n2) { fprintf(stderr, "oracle: out of memory\n"); abort(); }

    oracle_norm_silu(x, n1, P, p->cin, p->gamma1, p->beta1, p->eps);
    oracle_field f1 = {n1, N, T, H, W, p->cin, 0, 0, 0, T, H, W};
    conv3_box(&f1, NULL, p->wa, p->ba, p->cout, 0, 0, 0, T, H, W, a, NULL, NULL);
    oracle_norm_silu(a, n2, P, p->cout, p->gamma2, p->beta2, p->eps);
    oracle_field f2 = {n2, N, T, H, W, p->cout, 0, 0, 0, T, H, W};
    oracle_field fx = {x, N, T, H, W, p->cin, 0, 0, 0, T, H, W};
    conv3_box(&f2, NULL, p->wb, p->bb, p->cout, 0, 0, 0, T, H, W, y, p, &fx);

    free(n1); free(a); free(n2);
}

/* Keep the last two frames of [cache, chunk] in cache ([N][2][H][W][C]). */
static void roll_cache(float *cache, const float *chunk, int64_t N, int64_t Tc, int64_t H,
                       int64_t W, int64_t C)
{
    int64_t slab = H * W * C;
    for (int64_t n = 0; n < N; ++n) {
        float *c = cache + n * 2 * slab;
        const float *z = chunk + n * Tc * slab;
        if (Tc >= 2) {
            memcpy(c, z + (Tc - 2) * slab, sizeof(float) * (size_t)slab);
            memcpy(c + slab, z + (Tc - 1) * slab, sizeof(float) * (size_t)slab);
        } else {
            memmove(c, c + slab, sizeof(float) * (size_t)slab);
            memcpy(c + slab, z, sizeof(float) * (size_t)slab);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* One streaming step over a chunk of Tc >= 1 frames with the feat_cache     */
/* ("Sharding of WAN 2.2 VAE", Why depth sharding is not beneficial: one      */
/* frame at a time with a cache of the last one or two frames of every       */
/* CausalConv3d's input; "Closing the gap", section 1: the per-frame loop    */
/* carrying feat_cache).  cache_a holds conv A's input (n1) frames, cache_b  */
/* conv B's input (n2) frames; both are read as frames -2, -1 and then       */
/* updated in place.  A fresh stream starts from zero caches, which is the   */
/* causal zero pad.                                                          */
/* ------------------------------------------------------------------------ */
void oracle_resblock_stream_step(const oracle_block *p, const float *x, float *y, int64_t N,
                                 int64_t Tc, int64_t H, int64_t W, float *cache_a, float *cache_b)
{
    int64_t P = N * Tc * H * W;
    float *n1 = (float *)malloc(sizeof(float) * (size_t)(P * p->cin));
    float *a = (float *)malloc(sizeof(float) * (size_t)(P * p->cout));
    float *n2 = (float *)malloc(sizeof(float) * (size_t)(P * p->cout));
    if (!n1 || !a || !n2) { fprintf(stderr, "oracle: out of memory\n"); abort(); }

    oracle_norm_silu(x, n1, P, p->cin, p->gamma1, p->beta1, p->eps);
    oracle_field f1 = {n1, N, Tc, H, W, p->cin, 0, 0, 0, Tc, H, W};
    conv3_box(&f1, cache_a, p->wa, p->ba, p->cout, 0, 0, 0, Tc, H, W, a, NULL, NULL);
    roll_cache(cache_a, n1, N, Tc, H, W, p->cin);
    oracle_norm_silu(a, n2, P, p->cout, p->gamma2, p->beta2, p->eps);
    oracle_field f2 = {n2, N, Tc, H, W, p->cout, 0, 0, 0, Tc, H, W};
    oracle_field fx = {x, N, Tc, H, W, p->cin, 0, 0, 0, Tc, H, W};
    conv3_box(&f2, cache_b, p->wb, p->bb, p->cout, 0, 0, 0, Tc, H, W, y, p, &fx);
    roll_cache(cache_b, n2, N, Tc, H, W, p->cout);

    free(n1); free(a); free(n2);
}

/* Whole clip in chunks of t_step frames, starting from zero caches. */
void oracle_resblock_stream(const oracle_block *p, const float *x, float *y, int64_t N, int64_t T,
                            int64_t H, int64_t W, int64_t t_step)
{
    int64_t slab_in = H * W * p->cin, slab_out = H * W * p->cout;
    float *ca = (float *)calloc((size_t)(N * 2 * slab_in), sizeof(float));
    float *cb = (float *)calloc((size_t)(N * 2 * slab_out), sizeof(float));
    float *xc = (float *)malloc(sizeof(float) * (size_t)(N * t_step * slab_in));
    float *yc = (float *)malloc(sizeof(float) * (size_t)(N * t_step * slab_out));
    if (!ca || !cb || !xc || !yc) { fprintf(stderr, "oracle: out of memory\n"); abort(); }
    for (int64_t t0 = 0; t0 < T; t0 += t_step) {
        int64_t tc = T - t0 < t_step ? T - t0 : t_step;
        for (int64_t n = 0; n < N; ++n)
            memcpy(xc + n * tc * slab_in, x + (n * T + t0) * slab_in,
                   sizeof(float) * (size_t)(tc * slab_in));
        oracle_resblock_stream_step(p, xc, yc, N, tc, H, W, ca, cb);
        for (int64_t n = 0; n < N; ++n)
            memcpy(y + (n * T + t0) * slab_out, yc + n * tc * slab_out,
                   sizeof(float) * (size_t)(tc * slab_out));
    }
    free(ca); free(cb); free(xc); free(yc);
}

/* ------------------------------------------------------------------------ */
/* Output box of the full-T block computed from its receptive field only.    */
/*                                                                           */
/* The block output on a box depends on x only within the box widened by 4   */
/* frames back in T and 2 pixels each way in H and W (two 3x3x3 causal       */
/* convs), which is the halo argument of "Sharding of WAN 2.2 VAE", Spatial  */
/* sharding.  x_region holds x on that widened box clipped to the tensor,    */
/* with origin (xt0, xh0, xw0) and extent (xnt, xnh, xnw).  Conv A outputs   */
/* outside the tensor are conv B's zero pad and are never computed.          */
/* y_box is [N][bt1-bt0][bh1-bh0][bw1-bw0][cout].                            */
/* ------------------------------------------------------------------------ */
static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }
static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

void oracle_resblock_window(const oracle_block *p, const float *x_region, int64_t N, int64_t T,
                            int64_t H, int64_t W, int64_t xt0, int64_t xh0, int64_t xw0,
                            int64_t xnt, int64_t xnh, int64_t xnw, int64_t bt0, int64_t bt1,
                            int64_t bh0, int64_t bh1, int64_t bw0, int64_t bw1, float *y_box)
{
    /* conv A is needed on the box widened by (2 back, 1, 1), clipped */
    int64_t at0 = max64(bt0 - 2, 0), at1 = bt1;
    int64_t ah0 = max64(bh0 - 1, 0), ah1 = min64(bh1 + 1, H);
    int64_t aw0 = max64(bw0 - 1, 0), aw1 = min64(bw1 + 1, W);
    int64_t ant = at1 - at0, anh = ah1 - ah0, anw = aw1 - aw0;

    int64_t Px = N * xnt * xnh * xnw, Pa = N * ant * anh * anw;
    float *n1 = (float *)malloc(sizeof(float) * (size_t)(Px * p->cin));
    float *a = (float *)malloc(sizeof(float) * (size_t)(Pa * p->cout));
    float *n2 = (float *)malloc(sizeof(float) * (size_t)(Pa * p->cout));
    if (!n1 || !a || !n2) { fprintf(stderr, "oracle: out of memory\n"); abort(); }

    oracle_norm_silu(x_region, n1, Px, p->cin, p->gamma1, p->beta1, p->eps);
    oracle_field f1 = {n1, N, T, H, W, p->cin, xt0, xh0, xw0, xnt, xnh, xnw};
    conv3_box(&f1, NULL, p->wa, p->ba, p->cout, at0, ah0, aw0, ant, anh, anw, a, NULL, NULL);
    oracle_norm_silu(a, n2, Pa, p->cout, p->gamma2, p->beta2, p->eps);
    oracle_field f2 = {n2, N, T, H, W, p->cout, at0, ah0, aw0, ant, anh, anw};
    oracle_field fx = {x_region, N, T, H, W, p->cin, xt0, xh0, xw0, xnt, xnh, xnw};
    conv3_box(&f2, NULL, p->wb, p->bb, p->cout, bt0, bh0, bw0, bt1 - bt0, bh1 - bh0, bw1 - bw0,
              y_box, p, &fx);

    free(n1); free(a); free(n2);
}

/* ------------------------------------------------------------------------ */
/* Decoder mid-block attention over one frame.                               */
/* "Closing the gap: Wan 2.2 14B VAE decoder", section 5: the decoder's one  */
/* attention block is a spatial self-attention in which, within a frame,     */
/* every position attends to every other; the sequence is the H*W grid and  */
/* each (batch, frame) is an independent problem.  "Sharding of WAN 2.2     */
/* VAE", decoder module tree: WanAttentionBlock(384) between the mid-block's */
/* two ResidualBlocks.  The pages give nothing more; the readings used:      */
/*   u = RMS_norm(x; gamma, beta)          (the decoder's norm, no SiLU)     */
/*   [q | k | v] = wqkv u + bqkv           (one 1x1x1 projection, [3C][C];   */
/*                                           rows 0..C-1 q, C..2C-1 k, then v)*/
/*   p_ij = softmax_j(q_i . k_j / sqrt(C)) (one head of width C, over all    */
/*                                           H*W positions j of the frame)   */
/*   o_i = sum_j p_ij v_j                                                    */
/*   y_i = x_i + wo o_i + bo               (1x1x1 output projection, [C][C], */
/*                                           and the residual)              */
/* u, q, k, v and o are stored as fp32; every sum runs in fp64 in ascending  */
/* index order; the softmax subtracts the row maximum before exp (exact in   */
/* real arithmetic).                                                         */
/* x: one frame [HW][C]; y: [nq][C] for the query positions qidx[0..nq-1]    */
/* (qidx NULL: all HW positions in order, nq = HW).                          */
/* ------------------------------------------------------------------------ */
void oracle_attention_frame(const float *x, int64_t HW, int C, const float *gamma,
                            const float *beta, double eps, const float *wqkv, const float *bqkv,
                            const float *wo, const float *bo, const int64_t *qidx, int64_t nq,
                            float *y)
{
    float *u = (float *)malloc(sizeof(float) * (size_t)(HW * C));
    float *k = (float *)malloc(sizeof(float) * (size_t)(HW * C));
    float *v = (float *)malloc(sizeof(float) * (size_t)(HW * C));
    if (!u || !k || !v) { fprintf(stderr, "oracle: out of memory\n"); abort(); }
    oracle_rms_norm(x, u, HW, C, gamma, beta, eps);

    /* k and v of every position of the frame */
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < HW; ++j) {
        const float *uj = u + j * (int64_t)C;
        for (int c = 0; c < C; ++c) {
            double sk = 0.0, sv = 0.0;
            const float *wk = wqkv + ((int64_t)C + c) * C;
            const float *wv = wqkv + ((int64_t)2 * C + c) * C;
            for (int i = 0; i < C; ++i) {
                sk += (double)wk[i] * (double)uj[i];
                sv += (double)wv[i] * (double)uj[i];
            }
            k[j * (int64_t)C + c] = (float)(sk + (bqkv ? (double)bqkv[C + c] : 0.0));
            v[j * (int64_t)C + c] = (float)(sv + (bqkv ? (double)bqkv[2 * C + c] : 0.0));
        }
    }

    const double scale = 1.0 / sqrt((double)C);
    #pragma omp parallel
    {
        float *q = (float *)malloc(sizeof(float) * (size_t)C);
        float *o = (float *)malloc(sizeof(float) * (size_t)C);
        double *s = (double *)malloc(sizeof(double) * (size_t)HW);
        double *acc = (double *)malloc(sizeof(double) * (size_t)C);
        if (!q || !o || !s || !acc) { fprintf(stderr, "oracle: out of memory\n"); abort(); }
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < nq; ++r) {
            const int64_t i = qidx ? qidx[r] : r;
            const float *ui = u + i * (int64_t)C;
            for (int c = 0; c < C; ++c) {
                double sq = 0.0;
                const float *wq = wqkv + (int64_t)c * C;
                for (int t = 0; t < C; ++t) sq += (double)wq[t] * (double)ui[t];
                q[c] = (float)(sq + (bqkv ? (double)bqkv[c] : 0.0));
            }
            double m = -INFINITY;
            for (int64_t j = 0; j < HW; ++j) {
                double d = 0.0;
                const float *kj = k + j * (int64_t)C;
                for (int c = 0; c < C; ++c) d += (double)q[c] * (double)kj[c];
                s[j] = d * scale;
                if (s[j] > m) m = s[j];
            }
            double z = 0.0;
            for (int c = 0; c < C; ++c) acc[c] = 0.0;
            for (int64_t j = 0; j < HW; ++j) {
                const double e = exp(s[j] - m);
                z += e;
                const float *vj = v + j * (int64_t)C;
                for (int c = 0; c < C; ++c) acc[c] += e * (double)vj[c];
            }
            for (int c = 0; c < C; ++c) o[c] = (float)(acc[c] / z);
            const float *xi = x + i * (int64_t)C;
            for (int co = 0; co < C; ++co) {
                double t = 0.0;
                const float *w = wo + (int64_t)co * C;
                for (int c = 0; c < C; ++c) t += (double)w[c] * (double)o[c];
                y[r * (int64_t)C + co] =
                    (float)((double)xi[co] + t + (bo ? (double)bo[co] : 0.0));
            }
        }
        free(q); free(o); free(s); free(acc);
    }
    free(u); free(k); free(v);
}

/* ------------------------------------------------------------------------ */
/* Spatial upsampler of the decoder (upsample2d): every frame doubled in H   */
/* and W by nearest neighbour, then one 3x3 conv over the frame.             */
/* "Sharding of WAN 2.2 VAE", decoder module tree: the up blocks end in an    */
/* upsample2d or upsample3d; "Further sharding consideration: WanResample"   */
/* names the upsampler's conv, resample[1], and its C_out.  The tree's       */
/* channel counts (an up block that ends at 384 channels feeds one that      */
/* starts at 192) make that conv halve the channels, and the decoder goes    */
/* from the 90 x 160 latent to 720 x 1280 through three upsamplers, x2 each. */
/* The pages say no more; the readings used:                                 */
/*   up[h][w][ci] = x[h / 2][w / 2][ci]       (nearest, integer division)    */
/*   y[h][w][co]  = sum_{kh, kw, ci} w[co][ci][kh][kw] up[h+kh-1][w+kw-1][ci] */
/*                  + b[co]                    (zero outside the 2H x 2W image)*/
/* frame by frame, with no temporal taps (the temporal half of upsample3d is */
/* not described on the pages and is not modelled here).  The sum runs in    */
/* fp64 in ascending (kh, kw, ci) order, the bias last, one rounding.        */
/* x: nf frames [nf][H][W][cin]; w: [cout][cin][3][3]; b: [cout] or NULL;     */
/* y: rows [r0, r1) of each upsampled frame, [nf][r1 - r0][2W][cout].        */
/* ------------------------------------------------------------------------ */
void oracle_upsample2d_conv(const float *x, int64_t nf, int64_t H, int64_t W, int cin, int cout,
                            const float *w, const float *b, int64_t r0, int64_t r1, float *y)
{
    const int64_t Ho = 2 * H, Wo = 2 * W, nr = r1 - r0;
    #pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < nf * nr * Wo; ++o) {
        const int64_t f = o / (nr * Wo), h = r0 + (o / Wo) % nr, wc = o % Wo;
        const float *xf = x + f * H * W * (int64_t)cin;
        float *yo = y + o * (int64_t)cout;
        for (int co = 0; co < cout; ++co) {
            double acc = 0.0;
            for (int kh = 0; kh < 3; ++kh) {
                const int64_t uh = h + kh - 1;
                if (uh < 0 || uh >= Ho) continue;
                for (int kw = 0; kw < 3; ++kw) {
                    const int64_t uw = wc + kw - 1;
                    if (uw < 0 || uw >= Wo) continue;
                    const float *xs = xf + ((uh / 2) * W + uw / 2) * (int64_t)cin;
                    for (int ci = 0; ci < cin; ++ci)
                        acc += (double)w[(((int64_t)co * cin + ci) * 3 + kh) * 3 + kw] * (double)xs[ci];
                }
            }
            if (b) acc += (double)b[co];
            yo[co] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* The decoder's upsample3d: the frames doubled in time, then each frame     */
/* through the spatial upsampler above.  "Sharding of WAN 2.2 VAE", decoder  */
/* module tree: up_blocks[0] and up_blocks[1] end in upsample3d, and the     */
/* decoder takes the 21 latent frames to 81 output frames ("Optimize         */
/* attention ... WAN 2.2 Training on TPU 7x", inference validation workload:  */
/* 81 frames; the mid-resolution block runs 41): each upsample3d takes T     */
/* frames to 2T - 1.  How the frames are made is not on the pages; the       */
/* reading used is the plainest causal one that gives 2T - 1, nearest        */
/* neighbour in time with the first frame kept once:                          */
/*   output frame 0 = input frame 0;                                          */
/*   output frames 2k - 1 and 2k = input frame k   (k = 1 .. T - 1),          */
/* i.e. output frame t' takes input frame (t' + 1) / 2 (integer division),    */
/* so an output frame depends on no later input frame.                        */
/* x: [N][T][H][W][cin]; w: [cout][cin][3][3]; b: [cout] or NULL;             */
/* y: [N][2T - 1][2H][2W][cout].                                              */
/* ------------------------------------------------------------------------ */
void oracle_upsample3d_conv(const float *x, int64_t N, int64_t T, int64_t H, int64_t W, int cin, int cout,
                            const float *w, const float *b, float *y)
{
    const int64_t To = 2 * T - 1;
    const int64_t in_frame = H * W * (int64_t)cin, out_frame = 4 * H * W * (int64_t)cout;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t t = 0; t < To; ++t) {
            const int64_t src = (t + 1) / 2;
            oracle_upsample2d_conv(x + (n * T + src) * in_frame, 1, H, W, cin, cout, w, b, 0, 2 * H,
                                   y + (n * To + t) * out_frame);
        }
}
