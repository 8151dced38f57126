// Decoder mid-block attention core: per frame, o = softmax(q k^T / sqrt(D)) v
// over the frame's H*W positions ("Closing the gap: Wan 2.2 14B VAE decoder",
// section 5: a spatial self-attention in which, within a frame, every position
// attends to every other; each (batch, frame) is an independent problem).
// One head of width D = C.
//
// Inputs: qkv [F][HW][3D] bf16 (q, k, v of each position side by side, the
// output of the block's 1x1x1 projection) and vt [F][HWp/32][D][32] bf16, v
// transposed per frame and block of 32 keys (transpose_v_kernel, keys padded
// with zeros to HWp; within every 16 keys the groups of 4 are stored in the
// order 0, 2, 1, 3, see below), so each key block's V^T is one contiguous
// run.  Output o [F][HW][D] bf16.
//
// Flash-attention form, bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 softmax and
// accumulation, the scores never leave the chip.  A workgroup owns 128 queries
// of one frame and walks the frame's keys in blocks of 32.  Its 8 waves are 4
// query groups of 32, each a producer and a consumer wave on the same SIMD
// (waves qg and qg + 4):
//  - the producer keeps q of its 32 queries over the whole head in registers
//    and, per key block, computes the scores S^T = K q^T (keys as the MFMA M
//    rows, queries as N columns) and the online softmax: row maximum (the two
//    32-lane halves exchange theirs with v_permlane32_swap), exp2, running
//    sum, with the reference maximum moved only when some query's maximum
//    passes it by more than 2^8 in the exponential (lazy rescaling; exact).
//    It publishes P in LDS, in the consumer's B-operand layout, and, when
//    the reference moved, the factors that rescale O;
//  - the consumer keeps O^T for most of the head (D/32 tiles of 32 x 32, all
//    but the producer's share) and, one key block behind, rescales it if
//    told to and adds V^T P^T; the producer does the same for its share of
//    the tiles (a sixth) from its own P, which its lanes already hold in the
//    B-operand layout.  A producer
//    lane holds the scores of one query for keys 8j + 4g + i (j, i < 4; g =
//    lane / 32); taking j = 2ks, 2ks + 1 as MFMA k-step ks, the 8 k values of
//    lane group g are keys 16ks + 4g + {0..3, 8..11}: the consumer lane reads
//    its P straight from its twin's slot, and the V^T operand is read in that
//    same key order: vt stores the 4-key groups of every 16 keys as 0, 2, 1,
//    3, so that order is 16 contiguous bytes (one read per fragment);
//  - so the two waves of a SIMD overlap: the producer's softmax (VALU) runs
//    beside the consumer's MFMAs.  One barrier per key block; the K and V^T
//    blocks (2 x 24 KB at D = 384) are staged by LDS-DMA (buffer_load ...
//    lds) into 2-slot rings a block ahead of use, the loads issued by the
//    consumers.
// LDS: K rows are swizzled in 16-byte chunks (chunk ^ (key & 15)) and V^T rows
// (64 bytes) by (d >> 2) & 3, so fragment reads spread over the banks.
// Scores of keys past HW are -inf; queries past HW compute on zero q and are
// not stored.
#include "bf16.h"
#include "internal.h"

namespace wanvae {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufFlags = 0x00020000;   // raw buffer, loads past num_records return zeros
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kBQ = 128;                // queries per workgroup
constexpr int kBK = 32;                 // keys per block
constexpr int kGroups = 4;              // query groups of 32 per workgroup
constexpr int kWaves = 2 * kGroups;     // a producer and a consumer wave per group
constexpr float kRescaleLog2 = 8.0f;    // softmax reference moves when a maximum passes it by this (log2)
constexpr int kThreads = kWaves * 64;

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }   // lgkmcnt(0), others untouched

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

template <int D>
struct AttnShape {
    static constexpr int KS = D / 16;                   // MFMA k-steps of the score product
    static constexpr int DT = D / 32;                   // O^T tiles
    // of them, the producer's (the consumer has the rest): the consumer, which
    // also issues every load, is the longer chain; 2 of 12 measured best at
    // D = 384 (1 to 3 within 1%, 4 and more slower)
    static constexpr int PT = DT / 6;
    static constexpr int CPR = D / 8;                   // 16-byte chunks per K row
    static constexpr int KSWZ = CPR < 16 ? CPR - 1 : 15;   // chunk swizzle mask of K rows
    static constexpr int K_BYTES = kBK * D * 2;         // one K block
    static constexpr int V_BYTES = D * kBK * 2;         // one V^T block
    static constexpr int KB = K_BYTES / 1024;           // 1 KB LDS-DMA blocks of K (and of V^T)
    // LDS: 2 K slots, 2 V^T slots, then per query group and buffer: P (64
    // lanes x 32 bytes), the rescale factors (32 floats) and a flag
    static constexpr int K_OFF = 0, V_OFF = 2 * K_BYTES;
    static constexpr int P_OFF = V_OFF + 2 * V_BYTES;
    static constexpr int P_BYTES = 64 * 32;
    static constexpr int A_OFF = P_OFF + 2 * kGroups * P_BYTES;
    static constexpr int F_OFF = A_OFF + 2 * kGroups * 32 * 4;
    static constexpr int L_OFF = F_OFF + 2 * kGroups * 4;
    static constexpr int LDS = L_OFF + kGroups * 32 * 4;
    static_assert(D % 64 == 0 && D <= 384, "head width a multiple of 64, at most 384");
    static_assert(KB % kGroups == 0, "each producer (consumer) wave issues the same K (V^T) loads");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// max and sum of v over lanes l and l ^ 32.  v_permlane32_swap on two copies
// of v leaves each lane holding its own value and its partner's, one in each
// result, so the combination needs no knowledge of which is which.
__device__ __forceinline__ float halves_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kThreads) void flash_attention_kernel(const uint16_t *__restrict__ qkv,
                                                                   const uint16_t *__restrict__ vt,
                                                                   uint16_t *__restrict__ o, int64_t frames,
                                                                   int HW, int HWp, float scale_log2) {
    using S = AttnShape<D>;
    constexpr int KS = S::KS, DT = S::DT;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[S::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave < kGroups;          // waves w and w + 4 share SIMD w
    const int qg = wave & (kGroups - 1);
    const int l32 = lane & 31, g = lane >> 5;
    const int qblocks = (HW + kBQ - 1) / kBQ;
    const int64_t f = blockIdx.x / qblocks;
    const int q0 = (int)(blockIdx.x % qblocks) * kBQ + qg * 32;   // this group's first query
    const int row3 = 3 * D;                                        // qkv row stride (elements)
    const uint16_t *qkv_f = qkv + f * (int64_t)HW * row3;
    const uint16_t *vt_f = vt + f * (int64_t)D * HWp;   // this frame's key blocks, D * 32 each
    const int nblk = (HW + kBK - 1) / kBK;
    const uint32_t lds_base = lds_address(lds);

    // ---- LDS-DMA, issued by the consumers (the producers carry the softmax,
    // the longer chain): consumer qg moves the 1 KB blocks qg, qg + 4, ... of
    // each K and V^T block.  Piece P (16 bytes) of a K block is K row P / CPR,
    // stored chunk P % CPR = global chunk ^ (row & KSWZ); piece P of a V^T
    // block is V^T row d = P / 4 (64 bytes, 4 chunks), stored chunk = global
    // chunk ^ ((d >> 2) & 3).
    // lane offsets within a block do not depend on the block: block j moves
    // the buffers' bases (scalar), and keys past HW fall beyond the K
    // buffer's end (zeros)
    constexpr int NDMA = S::KB / kGroups;
    uint32_t koff[NDMA], voff[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int b = qg + i * kGroups;
        const int P = b * 64 + lane;
        const int row = P / S::CPR, cs = P % S::CPR;
        koff[i] = (uint32_t)row * (uint32_t)(row3 * 2) + (uint32_t)((cs ^ (row & S::KSWZ)) * 16);
        const int d = P >> 2, c4 = P & 3;
        voff[i] = (uint32_t)d * (uint32_t)(kBK * 2) + (uint32_t)((c4 ^ ((d >> 2) & 3)) * 16);
    }
    auto issue_k = [&](int j) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)j * kBK;
        const i32x4 r = buffer_rsrc(qkv_f + k0 * row3 + D, (uint32_t)((HW - k0) * row3 * 2 - D * 2));
        const uint32_t dst = lds_base + (uint32_t)(S::K_OFF + (j & 1) * S::K_BYTES + qg * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) lds_dma16(r, dst + (uint32_t)(i * kGroups * 1024), koff[i]);
    };
    auto issue_v = [&](int j) __attribute__((always_inline)) {
        const i32x4 r = buffer_rsrc(vt_f + (int64_t)j * D * kBK, (uint32_t)(D * kBK * 2));
        const uint32_t dst = lds_base + (uint32_t)(S::V_OFF + (j & 1) * S::V_BYTES + qg * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) lds_dma16(r, dst + (uint32_t)(i * kGroups * 1024), voff[i]);
    };
    // every wave: its loads landed, its LDS accesses done; then the barrier
    auto sync = [&]() __attribute__((always_inline)) {
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & waitcnt_lgkm0());
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    };
    unsigned char *p_buf = lds + S::P_OFF + qg * S::P_BYTES;        // + (j & 1) * kGroups * P_BYTES
    float *a_buf = reinterpret_cast<float *>(lds + S::A_OFF) + qg * 32;   // + (j & 1) * kGroups * 32
    int *f_buf = reinterpret_cast<int *>(lds + S::F_OFF) + qg;             // + (j & 1) * kGroups
    float *l_buf = reinterpret_cast<float *>(lds + S::L_OFF) + qg * 32;

    // Phase p (0 .. nblk, one barrier each): the producer of a query group
    // computes the scores of key block p and their softmax and publishes P_p
    // (and, when the reference maximum moved, the factors that rescale O); the
    // consumer adds V_{p-1} P_{p-1} to O.  Loads: K_{p+1} and V^T_p, into the
    // slots of K_{p-1} and V^T_{p-2}, which the last barrier freed.
    if (producer) {
        // ---- producer: q of its 32 queries over the whole head, in registers
        bf16x8 qf[KS];
        {
            const int q = q0 + l32;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (q < HW) v = *reinterpret_cast<const u32x4 *>(qkv_f + (int64_t)q * row3 + 16 * s + 8 * g);
                qf[s] = __builtin_bit_cast(bf16x8, v);
            }
        }
        float m_run = -INFINITY, l_run = 0.0f;
        // O^T tiles 0 .. PT - 1 of the group's queries, one key block behind
        // like the consumer's, from this wave's own P, factor and flag of the
        // previous block (P is already in the B-operand layout: the consumer
        // lane reads its twin's P as it is)
        floatx16 oacc[S::PT > 0 ? S::PT : 1];
#pragma unroll
        for (int t = 0; t < S::PT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[t][r] = 0.0f;
        u32x4 pw0 = u32x4{0u, 0u, 0u, 0u}, pw1 = pw0;
        float alpha_prev = 1.0f;
        bool grow_prev = false;
        sync();
        for (int p = 0; p <= nblk; ++p) {
            if (S::PT > 0 && p >= 1) {
                const int j = p - 1;
                if (grow_prev) {
#pragma unroll
                    for (int t = 0; t < S::PT; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha_prev;
                }
                const bf16x8 pf0 = __builtin_bit_cast(bf16x8, pw0);
                const bf16x8 pf1 = __builtin_bit_cast(bf16x8, pw1);
                const unsigned char *vs = lds + S::V_OFF + (j & 1) * S::V_BYTES;
#pragma unroll
                for (int t = 0; t < S::PT; ++t) {
                    const int d = 32 * t + l32;
                    const unsigned char *row = vs + d * (kBK * 2);
                    const int sw = (d >> 2) & 3;
                    const bf16x8 v0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + ((0 + g) ^ sw) * 16));
                    const bf16x8 v1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + ((2 + g) ^ sw) * 16));
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pf0, oacc[t], 0, 0, 0);
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pf1, oacc[t], 0, 0, 0);
                }
            }
            if (p < nblk) {
                const unsigned char *ks = lds + S::K_OFF + (p & 1) * S::K_BYTES;
                // scores S^T = K q^T: keys as the MFMA rows, this lane's query l32
                floatx16 sc;
#pragma unroll
                for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int c = (2 * s + g) ^ (l32 & S::KSWZ);
                    const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(ks + (l32 * S::CPR + c) * 16));
                    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sc, 0, 0, 0);
                }
                // online softmax for the lane's query, keys 8jj + 4g + i; only the
                // last block can hold keys past HW
                if (p * kBK + kBK > HW) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (p * kBK + 8 * (r >> 2) + 4 * g + (r & 3) >= HW) sc[r] = -INFINITY;
                }
                float mx = sc[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
                mx = halves_max(mx) * scale_log2;
                // Lazy rescaling: m_run, the reference the exponentials are taken
                // against, moves (and O is rescaled) only when some query's
                // maximum exceeds it by more than kRescaleLog2.  The softmax stays
                // exact (P, l and O share the reference); P is then at most
                // 2^kRescaleLog2, well inside bf16 and fp32.  With the reference
                // tracking every increase, about a quarter of the key blocks of a
                // 90 x 160 frame rescaled O; now almost only the first does.
                const bool grow = __builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0;
                grow_prev = grow;
                if (grow) {
                    const float m_new = fmaxf(m_run, mx);
                    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                    l_run *= alpha;
                    m_run = m_new;
                    alpha_prev = alpha;
                    if (g == 0) a_buf[(p & 1) * kGroups * 32 + l32] = alpha;
                }
                if (lane == 0) f_buf[(p & 1) * kGroups] = grow ? 1 : 0;
                // P in the consumer's B-operand layout: the lane's keys 16 ks + 4 g +
                // {0..3, 8..11} are k-step ks; l_run: the lane's share
                uint32_t w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * e], scale_log2, -m_run));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * e + 1], scale_log2, -m_run));
                    l_run += p0 + p1;
                    w[e] = pack_bf16x2(p0, p1);
                }
                u32x4 *pp = reinterpret_cast<u32x4 *>(p_buf + (p & 1) * kGroups * S::P_BYTES + lane * 32);
                pw0 = u32x4{w[0], w[1], w[2], w[3]};
                pw1 = u32x4{w[4], w[5], w[6], w[7]};
                pp[0] = pw0;
                pp[1] = pw1;
            }
            sync();
        }
        // the row sums, for the consumer's normalisation
        l_run = halves_sum(l_run);
        if (g == 0) l_buf[l32] = l_run;
        sync();
        // o = O / l for this wave's tiles: d = 32 t + 8 jj + 4 g + i
        const int q = q0 + l32;
        if (S::PT > 0 && q < HW) {
            const float inv = 1.0f / l_run;
            uint16_t *orow = o + (f * (int64_t)HW + q) * D;
#pragma unroll
            for (int t = 0; t < S::PT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float v0 = oacc[t][4 * jj], v1 = oacc[t][4 * jj + 1];
                    const float v2 = oacc[t][4 * jj + 2], v3 = oacc[t][4 * jj + 3];
                    *reinterpret_cast<u32x2 *>(orow + 32 * t + 8 * jj + 4 * g) =
                        u32x2{pack_bf16x2(v0 * inv, v1 * inv), pack_bf16x2(v2 * inv, v3 * inv)};
                }
        }
    } else {
        // ---- consumer: O^T tiles PT .. DT - 1 for the group's 32 queries
        constexpr int CT = DT - S::PT;
        floatx16 acc[CT];
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
        issue_k(0);
        sync();
        for (int p = 0; p <= nblk; ++p) {
            if (p + 1 < nblk) issue_k(p + 1);
            if (p < nblk) issue_v(p);
            if (p >= 1) {
                const int j = p - 1;
                if (f_buf[(j & 1) * kGroups] != 0) {
                    const float alpha = a_buf[(j & 1) * kGroups * 32 + l32];
#pragma unroll
                    for (int t = 0; t < CT; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
                }
                const u32x4 *pp = reinterpret_cast<const u32x4 *>(p_buf + (j & 1) * kGroups * S::P_BYTES + lane * 32);
                const bf16x8 pf0 = __builtin_bit_cast(bf16x8, pp[0]);
                const bf16x8 pf1 = __builtin_bit_cast(bf16x8, pp[1]);
                // O^T += V^T P^T; V^T fragment of tile t, k-step ks: d = 32 t + l32,
                // keys 16 ks + 4 g + {0..3, 8..11}: 16 contiguous bytes, logical
                // chunk 2 ks + g of the 64-byte row, swizzled by (d >> 2) & 3
                const unsigned char *vs = lds + S::V_OFF + (j & 1) * S::V_BYTES;
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    const int d = 32 * (S::PT + t) + l32;
                    const unsigned char *row = vs + d * (kBK * 2);
                    const int sw = (d >> 2) & 3;
                    const bf16x8 v0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + ((0 + g) ^ sw) * 16));
                    const bf16x8 v1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + ((2 + g) ^ sw) * 16));
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pf0, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pf1, acc[t], 0, 0, 0);
                }
            }
            sync();
        }
        sync();   // the producer's row sums
        // ---- o = O / l for this lane's query: d = 32 t + 8 jj + 4 g + i
        const int q = q0 + l32;
        if (q < HW) {
            const float inv = 1.0f / l_buf[l32];
            uint16_t *orow = o + (f * (int64_t)HW + q) * D;
#pragma unroll
            for (int t = 0; t < CT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float v0 = acc[t][4 * jj], v1 = acc[t][4 * jj + 1];
                    const float v2 = acc[t][4 * jj + 2], v3 = acc[t][4 * jj + 3];
                    *reinterpret_cast<u32x2 *>(orow + 32 * (S::PT + t) + 8 * jj + 4 * g) =
                        u32x2{pack_bf16x2(v0 * inv, v1 * inv), pack_bf16x2(v2 * inv, v3 * inv)};
                }
        }
    }
}

// vt[f][s / 32][d][s % 32] = v of key key(s) (qkv[f][key][2D + d]) for key <
// HW, 0 for HW <= key < HWp, where stored position s = 16 m + 4 a + b holds
// key 16 m + 4 sigma(a) + b, sigma = (0, 2, 1, 3): the 4-key groups of every
// 16 keys in the order the attention kernel's value product reads them, each
// block of 32 keys one contiguous [D][32] run.  64 keys x 64 dims per
// workgroup through LDS: 16-byte reads along d, 16-byte writes along s.
constexpr int kTT = 64;
__global__ __launch_bounds__(256) void transpose_v_kernel(const uint16_t *__restrict__ qkv, uint16_t *__restrict__ vt,
                                                          int64_t frames, int HW, int HWp, int D) {
    __shared__ uint16_t tile[kTT][kTT + 2];
    const int kb = (HWp + kTT - 1) / kTT, db = D / kTT;
    int64_t bid = blockIdx.x;
    const int dbi = (int)(bid % db);
    bid /= db;
    const int kbi = (int)(bid % kb);
    const int64_t f = bid / kb;
    const int k0 = kbi * kTT, d0 = dbi * kTT;
    const int tid = threadIdx.x;
    // read: 64 keys x 8 pieces of 8 dims
    for (int p = tid; p < kTT * 8; p += 256) {
        const int kr = p >> 3, dc = (p & 7) * 8;
        const int key = k0 + kr;
        u32x4 d = u32x4{0u, 0u, 0u, 0u};
        if (key < HW) d = *reinterpret_cast<const u32x4 *>(qkv + (f * HW + key) * (int64_t)(3 * D) + 2 * D + d0 + dc);
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[kr][dc + e] = (uint16_t)(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xffffu);
    }
    __syncthreads();
    // write: 64 dims x 8 pieces of 8 keys
    for (int p = tid; p < kTT * 8; p += 256) {
        const int dr = p >> 3, kc = (p & 7) * 8;
        if (k0 + kc >= HWp) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // stored positions kc + 2e, kc + 2e + 1 (same 4-key group)
            const int s = (kc & 15) + 2 * e, a = s >> 2;
            const int key = (kc & ~15) + 4 * (((a & 1) << 1) | (a >> 1)) + (s & 3);
            w[e] = (uint32_t)tile[key][dr] | ((uint32_t)tile[key + 1][dr] << 16);
        }
        // block (k0 + kc) / 32 of the frame, row d, positions (k0 + kc) % 32 ..
        const int64_t kblk = (k0 + kc) / kBK;
        *reinterpret_cast<u32x4 *>(vt + ((f * (HWp / kBK) + kblk) * D + d0 + dr) * (int64_t)kBK + (k0 + kc) % kBK) =
            u32x4{w[0], w[1], w[2], w[3]};
    }
}

template <int D>
hipError_t launch_flash(const void *qkv, const void *vt, void *o, int64_t frames, int HW, int HWp, hipStream_t s) {
    const int64_t qblocks = (HW + kBQ - 1) / kBQ;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    flash_attention_kernel<D><<<dim3((unsigned)(frames * qblocks)), dim3(kThreads), 0, s>>>(
        static_cast<const uint16_t *>(qkv), static_cast<const uint16_t *>(vt), static_cast<uint16_t *>(o), frames,
        HW, HWp, scale_log2);
    return hipGetLastError();
}

}  // namespace

bool attention_supported(int D) { return D == 64 || D == 128 || D == 384; }

int64_t attention_keys_padded(int64_t hw) { return (hw + kBK - 1) / kBK * kBK; }

hipError_t launch_transpose_v(const void *qkv, void *vt, int64_t frames, int HW, int D, hipStream_t s) {
    const int HWp = (int)attention_keys_padded(HW);
    const int64_t blocks = frames * ((HWp + kTT - 1) / kTT) * (D / kTT);
    if (blocks == 0) return hipSuccess;
    transpose_v_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(static_cast<const uint16_t *>(qkv),
                                                                    static_cast<uint16_t *>(vt), frames, HW, HWp, D);
    return hipGetLastError();
}

hipError_t launch_flash_attention(const void *qkv, const void *vt, void *o, int64_t frames, int HW, int D,
                                  hipStream_t s) {
    if (frames == 0 || HW == 0) return hipSuccess;
    const int HWp = (int)attention_keys_padded(HW);
    switch (D) {
        case 64: return launch_flash<64>(qkv, vt, o, frames, HW, HWp, s);
        case 128: return launch_flash<128>(qkv, vt, o, frames, HW, HWp, s);
        case 384: return launch_flash<384>(qkv, vt, o, frames, HW, HWp, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wanvae
