// fa_fwd.hip -- exact attention forward for MI355X (gfx950, CDNA4), and its C ABI.
//
// The method: the tiled online-softmax forward ("Flash Attention, tiled: exact
// attention without the T x T HBM matrix", section "From the example to tiled
// GPU work"; "FlashAttention: the IO-aware Attention Kernel", sections 3.2-3.3).
// A workgroup owns one tile of query rows of one (batch, head); it walks the
// key/value tiles, computes the score tile with matrix-core instructions, folds
// it into each row's running (max, sum, output) state, multiplies the tile's
// probabilities by V at once, and writes O = o / l and the row log-sum-exp after
// the last tile.  Score and probability tiles live only in registers.
//
// gfx950 mapping: one workgroup of 8 waves (256 query rows) per CU; waves w and
// w + 4 share SIMD w % 4.
//   * Each wave owns 32 query rows and computes the TRANSPOSED score tile
//     S^T = K_j Q^T with v_mfma_f32_32x32x16_bf16: in the accumulator every lane
//     holds 32 scores of ONE query row (lane % 32), the other 32 keys of the
//     64-key tile sitting in lane ^ 32.  Row max and row sums are in-register
//     reductions plus one v_permlane32_swap.
//   * The output is accumulated transposed too, O^T += V_j^T P^T: its B operand
//     is the bf16-converted score accumulator as it stands (no LDS round trip
//     for P) and its accumulator again keeps one query row per lane, so a row's
//     rescale factor is lane-local.
//   * Ping-pong between the two waves of a SIMD.  Waves 0-3 run one phase ahead
//     of waves 4-7, and a workgroup barrier at every key tile (every second
//     phase) keeps them there, so one wave of each SIMD runs a matrix phase (PV
//     of tile j and S^T of tile j+1: 32 MFMAs, at raised wave priority) while
//     the other runs a softmax phase (max, exponentials, row sums of tile j+1:
//     VALU work).  The two kinds of work then co-issue on the SIMD instead of
//     competing for the same unit.  This is the
//     producer/consumer overlap of softmax with the matrix products described
//     for FlashAttention-3 on "FlashAttention and Fused Kernels: Attention
//     Without the n x n Matrix" ("Four generations"), done here with wave groups
//     and barriers.
//   * K_j and V_j are copied HBM -> LDS by buffer_load ... lds (no VGPR
//     staging), one 16-byte chunk per lane, into row-major tiles whose 16-byte
//     chunks are XOR-swizzled by row so that both the K operand reads
//     (ds_read_b128) and the transposed V operand reads (ds_read_b64_tr_b16,
//     which hands each lane 4 keys of one head-dim column) are free of bank
//     conflicts.  The buffer descriptor of each tile covers only the rows that
//     exist, so the ragged end of the sequence reads as zeros.  All 8 waves share
//     each tile; LDS holds two K and two V tiles, fetched two phases ahead.
//   * The softmax scale is folded into the exponent (one FMA per score, exp2 with
//     scale*log2(e)); a negative scale negates Q once instead.
//   * The max is tracked lazily: a row is rescaled only when its tile maximum
//     exceeds the running reference by more than 2^8 (in exp2 units), the
//     conditional rescale described for FlashAttention-4 on the same page.
//     Weights exp2(x - m) then stay at most 256, and the result is unchanged up
//     to rounding.  The weights are first computed against the current
//     reference; only when some lane's tile sum exceeds 256 (so that some weight
//     may) is the tile max taken and the weights recomputed, which gives the
//     same bits as always taking the max.  Two row sums are kept: the fp32 sum of the weights (for the
//     log-sum-exp) and the sum of their bf16 roundings, which are the weights
//     the PV product actually used (for O = o / l).
//   * Causal: key tiles past a wave's last query are skipped; only a wave's
//     last tile can cross its diagonal or the end of the sequence, and only that
//     tile runs the masked softmax.
//   * Workgroup order: the grid is remapped so that a contiguous range of the
//     work list lands on one XCD (workgroups are dealt round-robin over the 8
//     XCDs), keeping one head's K/V in that XCD's L2; within a head the heaviest
//     causal query tiles go first.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_internal.h"

namespace {

#define FA_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;         // keys per K/V tile
constexpr int kXcds = 8;
constexpr double kLog2e = 1.4426950408889634;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;   // log2 units: rescale when the max grows by > 2^8
constexpr uint32_t kBufferFlags = 0x00020000u;   // gfx9 raw buffer descriptor word 3
constexpr uint32_t kNaN32 = 0x7FC00000u;         // quiet NaN, fp32 bits
constexpr uint32_t kNaN16x2 = 0x7FC07FC0u;       // two quiet NaNs, bf16 bits
constexpr float kMaxRef = 8388608.0f;             // 2^23: largest |reference| (log2 units) with an accurate result


// Tile geometry for head size D and NG wave groups per workgroup (4 waves of
// 32 query rows each per group).
template <int D, int NG>
struct Geo {
    static constexpr int kWaves = 4 * NG;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBM = 32 * kWaves;          // query rows per workgroup
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;            // 16-byte chunks per row
    static constexpr int kTileBytes = kBN * kRowBytes;
    static constexpr int kLoads = kTileBytes / 1024 / kWaves;  // 1 KB buffer->LDS loads per wave per tile
    static constexpr int kDSteps = D / 16;            // MFMA k-steps over d for S^T
    static constexpr int kDBlocks = D / 32;           // 32-row blocks of O^T
    static constexpr int kLdsBytes = 4 * kTileBytes;  // K slot 0, K slot 1, V slot 0, V slot 1
};

// Waves per SIMD (and so the register budget: 512 / waves): NG = 2 is one
// 8-wave workgroup per CU whose wave groups alternate phases, two waves per
// SIMD; NG = 1 is independent 4-wave workgroups, two per CU at d = 128 and
// three at d = 64, whose smaller tiles leave the registers for a third wave.
template <int D, int NG>
constexpr int kWavesPerSimd = NG == 1 && D == 64 ? 3 : 2;

// XOR swizzle of the 16-byte chunk index within a tile row.  D = 128 (16
// chunks): the two 2-bit fields of row % 16 swapped; D = 64 (8 chunks): a
// 3-bit permutation of (row / 2) % 8.  Either way 16 consecutive rows map one
// logical chunk to 16 (resp. 8 x 2 half-rows of) distinct banks, and 4
// consecutive rows move a 4-chunk group to 4 distinct bank quarters.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// max / sum of a value and its copy in lane ^ 32 (the other half of the row's keys)
__device__ __forceinline__ float xhalf_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return fmaxf(as_f32(r[0]), as_f32(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return as_f32(r[0]) + as_f32(r[1]);
}

// Max of the 32 raw scores a lane holds, then across the lane pair.
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
    float a0 = max3f(s[0][0], s[0][1], s[0][2]), a1 = max3f(s[0][3], s[0][4], s[0][5]);
    float a2 = max3f(s[0][6], s[0][7], s[0][8]), a3 = max3f(s[0][9], s[0][10], s[0][11]);
    float a4 = max3f(s[0][12], s[0][13], s[0][14]), a5 = max3f(s[0][15], s[1][0], s[1][1]);
    float a6 = max3f(s[1][2], s[1][3], s[1][4]), a7 = max3f(s[1][5], s[1][6], s[1][7]);
    float a8 = max3f(s[1][8], s[1][9], s[1][10]), a9 = max3f(s[1][11], s[1][12], s[1][13]);
    float a10 = fmaxf(s[1][14], s[1][15]);
    float b0 = max3f(a0, a1, a2), b1 = max3f(a3, a4, a5), b2 = max3f(a6, a7, a8), b3 = fmaxf(a9, a10);
    return xhalf_max(fmaxf(max3f(b0, b1, b2), b3));
}

// FA4's polynomial exponential ("FlashAttention and Fused Kernels", "Four
// generations of FlashAttention"): a share of the weights is computed on the
// FMA path instead of the transcendental unit.  kPolyExp2<D> is how many of a
// lane's 32 weights per key tile take it, per head size.  On gfx950 the
// transcendental instruction issues through the same VALU port as the FMAs,
// and the polynomial costs eight VALU instructions where v_exp_f32 costs one,
// so no head size takes it; building with FA_EXP2_POLY=n gives n at every
// head size, the variant that measures the trade.
#ifdef FA_EXP2_POLY
template <int D>
constexpr int kPolyExp2 = FA_EXP2_POLY;
#else
template <int D>
constexpr int kPolyExp2 = 0;
#endif
static_assert(kPolyExp2<64> >= 0 && kPolyExp2<64> <= 32 && (kPolyExp2<64> == 0 || 32 % kPolyExp2<64> == 0));
static_assert(kPolyExp2<128> >= 0 && kPolyExp2<128> <= 32 && (kPolyExp2<128> == 0 || 32 % kPolyExp2<128> == 0));

// 2^x as 2^floor(x) * q(frac(x)), q the cubic with q(0) = 1 that minimises the
// largest relative error against 2^f on [0, 1) (fitted by iteratively
// reweighted least squares on [0, 1]: 9.5e-5).  x is first clamped to [-160, 128], so
// masked scores (-inf) give exactly 0 and overflow gives +inf, as v_exp_f32.
__device__ __forceinline__ float exp2_poly(float x) {
    const float y = __builtin_amdgcn_fmed3f(x, -160.0f, 128.0f);
    const float fl = __builtin_floorf(y);
    const float f = y - fl;          // in [0, 1]: 1 only where y is just below an integer, and q(1) ~ 2
    const int e = static_cast<int>(fl);
    float q = __builtin_fmaf(f, 0.07714322f, 0.22765102f);
    q = __builtin_fmaf(f, q, 0.69507057f);
    q = __builtin_fmaf(f, q, 1.0f);
    return __builtin_amdgcn_ldexpf(q, e);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}


template <int D>
struct WaveState {
    f32x16 o[Geo<D, 1>::kDBlocks];   // O^T accumulator: lane holds d-rows of its query
    // Running reference max (exp2 units).  It starts at the most negative
    // finite float rather than -inf, so that the first tile's weights are +inf
    // (never NaN, also for masked -inf scores) and take the max.
    float m = -3.402823466e38f;
    float l32 = 0.0f;             // sum of fp32 weights
    float l16 = 0.0f;             // sum of bf16-rounded weights
};

// Lazily move the reference max to m_new when it grew by more than the threshold.
template <int D>
__device__ __forceinline__ void maybe_rescale(WaveState<D>& st, float m_new) {
    const bool need = m_new > st.m + kRescaleThreshold;
    if (__any(need)) {
        const float r = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.0f;
        st.m = need ? m_new : st.m;
        st.l32 *= r;
        st.l16 *= r;
#pragma unroll
        for (int b = 0; b < Geo<D, 1>::kDBlocks; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.o[b][i] *= r;
    }
}


// Launch arguments.  Query head h of batch b reads key/value head
// b * (hq / group) + h / group.  The query rows are the last tq positions of
// a tk-long sequence (causal: query i sees keys j <= i + tk - tq).  Key range
// [s * chunk, (s + 1) * chunk) goes to split s; with SPLIT the workgroup
// writes that split's normalised fp32 output and log-sum-exp to op / lp.
struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    float* op;     // [n_split][rows][D]
    float* lp;     // [n_split][rows]
    long long rows;   // B * hq * tq
    int tq, tk, n_qt, total, hq, group, chunk, n_split;
    float c;       // scale * log2(e)
};

// One workgroup's work; `lds` is the workgroup's Geo<D, NG>::kLdsBytes of LDS.
// The pointers come in as __restrict__ parameters (not through `a`): their
// no-alias scopes also tell the compiler that the LDS reads of one tile do
// not wait on the LDS DMA of another.
template <int D, bool CAUSAL, int NG, bool SPLIT>
__device__ __forceinline__ void fa_fwd_block(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                             const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                             float* __restrict__ LSE, float* __restrict__ OP,
                                             float* __restrict__ LP, const FwdArgs& a, FA_LDS char* const lds) {
    using G = Geo<D, NG>;
    constexpr int kBM = G::kBM;
    const int Tq = a.tq, Tk = a.tk, n_qt = a.n_qt, total = a.total;
    const float c_in = a.c;
    FA_LDS char* const kslot[2] = {lds, lds + G::kTileBytes};
    FA_LDS char* const vslot[2] = {lds + 2 * G::kTileBytes, lds + 3 * G::kTileBytes};

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = NG == 2 ? wave >> 2 : 0;   // 0: leading wave group, 1: one phase behind
    const int col = lane & 31;   // this lane's query row within the wave
    const int half = lane >> 5;

    // Work decode: XCD-contiguous remap, then (head, query tile), heavy tiles first.
    const int id = blockIdx.x;
    const int xcd = id % kXcds, xslot = id / kXcds;
    const int q8 = total / kXcds, r8 = total % kXcds;
    const int w = xcd < r8 ? xcd * (q8 + 1) + xslot : r8 * (q8 + 1) + (xcd - r8) * q8 + xslot;
    int bh = w / (n_qt * a.n_split);
    const int split = (w / n_qt) % a.n_split;
    int qt = CAUSAL ? n_qt - 1 - (w % n_qt) : (w % n_qt);
    // Causal work with few workgroups per CU (at most 8 rounds of the 256 CUs)
    // is tail-bound: when every XCD owns whole heads, its heads are walked
    // query-tile-major, so the heaviest tiles of all of them go first.  Longer
    // grids keep the head-major order, which keeps one head's K/V in L2.
    constexpr int kRoundSlots = 256 * (NG == 2 ? 1 : kWavesPerSimd<D, NG>);   // CUs x workgroups per CU
    if (CAUSAL && a.n_split == 1 && r8 == 0 && q8 % n_qt == 0 && total <= 8 * kRoundSlots) {
        const int hx = q8 / n_qt;                 // heads per XCD
        bh = xcd * hx + xslot % hx;
        qt = n_qt - 1 - xslot / hx;
    }

    const int kvh = (bh / a.hq) * (a.hq / a.group) + (bh % a.hq) / a.group;   // key/value head
    const size_t qbase = (size_t)bh * (size_t)Tq * D;
    const size_t kvbase = (size_t)kvh * (size_t)Tk * D;
    const uint16_t* __restrict__ kbh = K + kvbase;
    const uint16_t* __restrict__ vbh = V + kvbase;
    const uint32_t q_bytes = (uint32_t)Tq * G::kRowBytes;

    const int blk = NG == 2 ? 2 * (wave & 3) + grp : wave;   // the two waves of a SIMD take adjacent row blocks
    const int qw0 = qt * kBM + blk * 32;   // first query row of this wave
    const int qrow = qw0 + col;
    // Keys of this split, [k_lo, k_hi); causal query i sees keys <= i + off.
    const int off = Tk - Tq;
    const int k_lo = split * a.chunk;
    const int k_hi = min(Tk, k_lo + a.chunk);
    const int kv_end = CAUSAL ? min(k_hi, min(Tq, qt * kBM + kBM) + off) : k_hi;
    const int n_kt = kv_end > k_lo ? (kv_end - k_lo + kBN - 1) / kBN : 0;   // tiles the workgroup loads
    const int w_end = CAUSAL ? min(k_hi, qw0 + 32 + off) : k_hi;            // keys this wave may see
    const int n_w = qw0 >= Tq || w_end <= k_lo ? 0 : (w_end - k_lo + kBN - 1) / kBN;   // tiles it uses
    // Tiles from j_mask on can hold keys some row of the wave must not see
    // (past its diagonal, or past the split): at most the last two.
    const int j_mask = CAUSAL ? min(n_w - 1, max(0, (qw0 + off + 1 - k_lo) / kBN))
                              : (k_hi - k_lo) % kBN == 0 ? n_w : n_w - 1;   // a full last tile needs no mask

    // Per-lane byte offsets of this lane's 16-byte chunk in each tile load; the
    // wave's 1 KB blocks of a tile are contiguous in LDS.
    uint32_t goff[G::kLoads];
#pragma unroll
    for (int c = 0; c < G::kLoads; ++c) {
        const int q = (wave * G::kLoads + c) * 64 + lane;
        const int r = q / G::kChunks, p = q % G::kChunks;
        goff[c] = r * G::kRowBytes + 16 * (p ^ swz<D>(r));
    }
    auto load_tile = [&] __device__ (const uint16_t* src, int key0, FA_LDS char* slot) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (size_t)key0 * D, (uint32_t)(Tk - key0) * G::kRowBytes);
#pragma unroll
        for (int c = 0; c < G::kLoads; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(slot + (wave * G::kLoads + c) * 1024), 16,
                                                     goff[c], 0, 0, 0);
    };

    // LDS read offsets.  K (A operand of S^T): row = key col, logical chunk 2 s + half.
    uint32_t koff[G::kDSteps];
#pragma unroll
    for (int s = 0; s < G::kDSteps; ++s) koff[s] = col * G::kRowBytes + 16 * ((2 * s + half) ^ swz<D>(col));
    // V (A operand of O^T, transposed read): in 16-lane group g, lane i fetches 4 d-values of
    // row 8 e + 4 half + i / 4 (plus 16 per key step) at column 32 db + 16 (g % 2) + 4 (i % 4).
    uint32_t voff[G::kDBlocks][2];
    {
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = 8 * e + 4 * half + (i >> 2);
                const int cc = 32 * db + 16 * (g & 1) + 4 * (i & 3);
                voff[db][e] = r * G::kRowBytes + 16 * ((cc >> 3) ^ swz<D>(r)) + 2 * (cc & 7);
            }
    }

    if (n_kt > 0) load_tile(kbh, k_lo, kslot[0]);   // K_0; K_1 and V_0 follow in phase 0

    // Q^T operand (B operand of S^T): lane holds Q[qrow][16 s + 8 half .. +7]; zeros past T.
    bf16x8 qf[G::kDSteps];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qbase, q_bytes);
        const uint32_t neg = c_in < 0.0f ? 0x80008000u : 0u;
#pragma unroll
        for (int s = 0; s < G::kDSteps; ++s) {
            u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)qrow * G::kRowBytes + 32 * s + 16 * half,
                                                              0, 0);
            raw ^= neg;
            qf[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    // A zero scale runs as 1e-30: every product s * c then rounds away against
    // the reference in exp2 (all weights are 1, as for zero), and masked scores
    // (-inf) still give -inf instead of -inf * 0 = NaN.
    const float c = fmaxf(fabsf(c_in), 1e-30f);

    WaveState<D> st;
#pragma unroll
    for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[b][i] = 0.0f;
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    // S^T = K_j Q^T.  All K operand reads are written first; the scheduling
    // barriers then pin a pipeline that keeps kQkAhead reads in flight ahead of
    // the MFMA that consumes them.
    auto qk = [&] __device__ (FA_LDS const char* ks, f32x16 (&s)[2]) {
        constexpr int N = 2 * G::kDSteps;
        constexpr int kQkAhead = 4;   // K operand reads in flight ahead of their product
        bf16x8 a[N];
#pragma unroll
        for (int i = 0; i < N; ++i)
            a[i] = *(FA_LDS const bf16x8*)(ks + (i & 1) * 32 * G::kRowBytes + koff[i >> 1]);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[b][i] = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qf[i >> 1], s[i & 1], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kQkAhead, 0);
#pragma unroll
        for (int i = 0; i < N - kQkAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kQkAhead, 0);
    };
    // The V^T operand of O^T for key step ks and head-dim block db: two transposed 8-byte reads.
    auto v_operand = [&] __device__ (FA_LDS const char* vs, int ks, int db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (FA_LDS i16x4*)(vs + ks * 16 * G::kRowBytes + voff[db][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (FA_LDS i16x4*)(vs + ks * 16 * G::kRowBytes + voff[db][1]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 araw = {l2[0], l2[1], h2[0], h2[1]};
        return __builtin_bit_cast(bf16x8, araw);
    };
    // O^T += V_j^T P^T, with the V operands of the next key step read ahead.
    auto pv = [&] __device__ (FA_LDS const char* vs, const uint32_t (&pk)[16]) {
        bf16x8 va[2][G::kDBlocks];
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db) va[0][db] = v_operand(vs, 0, db);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) {
#pragma unroll
                for (int db = 0; db < G::kDBlocks; ++db) va[(ks + 1) & 1][db] = v_operand(vs, ks + 1, db);
            }
            const u32x4 praw = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, praw);
#pragma unroll
            for (int db = 0; db < G::kDBlocks; ++db) {
                st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks & 1][db], pb, st.o[db], 0, 0, 0);
                // The row sum of the bf16 weights rides in the MFMA shadow, in key order.
#pragma unroll
                for (int n = 4 * ks + db * 4 / G::kDBlocks; n < 4 * ks + (db + 1) * 4 / G::kDBlocks; ++n)
                    st.l16 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[n]), ones, st.l16, false);
            }
        }
    };

    f32x16 sc[2];       // score tile of the wave's current key tile
    uint32_t pk[16];    // its bf16 weights, consumed by the next matrix phase


    // Matrix phase for tile j (parity P = j & 1): PV of tile j, then the scores
    // of tile j+1 (K_{j+1} sits in slot P ^ 1, V_j in slot P).
    auto matrix_phase = [&] __device__ (int j, auto parity) {
        constexpr int P = decltype(parity)::value;
        // Issue priority for the matrix phase: otherwise the older waves' softmax
        // work wins the SIMD's arbitration and starves the other group's MFMAs.
        __builtin_amdgcn_s_setprio(1);
        const bool do_pv = j >= 0 && j < n_w;
        const bool do_qk = j + 1 < n_w;
        if (do_pv) pv(vslot[P], pk);
        if (do_qk) qk(kslot[P ^ 1], sc);
        __builtin_amdgcn_s_setprio(0);
    };
    // Softmax phase for tile j: running max, weights, fp32 row sum.  Only a
    // wave's last tile can cross its diagonal or the end of the sequence; there
    // the hidden scores are set to -inf in place, so that every tile then takes
    // the same path (a single code path keeps the O accumulator in place).
    auto softmax_phase = [&] __device__ (int j) {
        if (j < 0 || j >= n_w) return;
        if (j >= j_mask) {
            const int key0 = k_lo + j * kBN;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool vis = key < k_hi && (!CAUSAL || key <= qrow + off);
                    sc[kb][i] = vis ? sc[kb][i] : -INFINITY;
                }
        }
        // Weights against the current reference.  With speculation the tile max
        // is only taken when some weight may exceed 2^8, detected by the lane's
        // tile sum exceeding 2^8 (every weight is <= 2^8 otherwise).  Before the
        // first rescale the reference is -FLT_MAX and the visible weights are
        // inf, which also takes the max.
        // The first tile takes its max at once: against the initial reference
        // every weight would be infinite and the speculation would fail.
        if (j == 0) maybe_rescale<D>(st, tile_max(sc) * c);
        float p[32];
        float ts;
        auto weights = [&] __device__ () {
            const float mneg = -st.m;
#pragma unroll
            for (int n = 0; n < 32; ++n) {
                const float x = __builtin_fmaf(n < 16 ? sc[0][n] : sc[1][n - 16], c, mneg);
                constexpr int kEvery = kPolyExp2<D> ? 32 / kPolyExp2<D> : 0;
                p[n] = kEvery && n % kEvery == 0 ? exp2_poly(x) : __builtin_amdgcn_exp2f(x);
            }
            float t8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) t8[q] = (p[4 * q] + p[4 * q + 1]) + (p[4 * q + 2] + p[4 * q + 3]);
            ts = ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
        };
        weights();
        if (__any(!(ts <= 256.0f))) {
            maybe_rescale<D>(st, tile_max(sc) * c);
            weights();
        }
        st.l32 += ts;
#pragma unroll
        for (int n = 0; n < 16; ++n) pk[n] = pack_bf16x2(p[2 * n], p[2 * n + 1]);
    };

    // Phase ph: the leading group runs step ph, the trailing group step ph - 1,
    // where the steps are M(-1), S(0), M(0), S(1), M(1), ... (M = matrix phase,
    // S = softmax phase).  Even phases 2 j first wait for the loads issued two
    // phases earlier, then fetch K_{j+1} and V_j into the slots freed by M(j-2).
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    const int n_ph = 2 * n_kt + 2;
    // Barrier + loads at the start of phase ph (identical in both groups' loops).
    auto phase_start = [&] __device__ (int ph) {
        if ((ph & 1) == 0) {
            const int j = ph >> 1;
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the loads of phase ph - 2 have landed
            __syncthreads();
            if (j + 1 < n_kt) load_tile(kbh, k_lo + (j + 1) * kBN, kslot[(j + 1) & 1]);
            if (j < n_kt) load_tile(vbh, k_lo + j * kBN, vslot[j & 1]);
        }
    };
    // Each group runs its own straight-line loop; both loops pass the same
    // sequence of barriers.  Four phases (two key tiles) per iteration keep the
    // LDS slot of every access a compile-time constant.
    if (grp == 0) {
        for (int ph = 0; ph < n_ph; ph += 4) {
            const int j = ph >> 1;
            phase_start(ph);
            matrix_phase(j - 1, Odd{});
            if (ph + 1 >= n_ph) break;
            phase_start(ph + 1);
            softmax_phase(j);
            if (ph + 2 >= n_ph) break;
            phase_start(ph + 2);
            matrix_phase(j, Even{});
            if (ph + 3 >= n_ph) break;
            phase_start(ph + 3);
            softmax_phase(j + 1);
        }
    } else {
        for (int ph = 0; ph < n_ph; ph += 4) {
            const int j = ph >> 1;
            phase_start(ph);
            softmax_phase(j - 1);
            if (ph + 1 >= n_ph) break;
            phase_start(ph + 1);
            matrix_phase(j - 1, Odd{});
            if (ph + 2 >= n_ph) break;
            phase_start(ph + 2);
            softmax_phase(j);
            if (ph + 3 >= n_ph) break;
            phase_start(ph + 3);
            matrix_phase(j, Even{});
        }
    }

    // Epilogue: O = o / l, lse = ln2 * (m + log2 l).  A row that saw no key
    // (possible only for one split of a split problem) gets O = 0, lse = -inf.
    // The weights are exp2(fma(s, c, -m)): exact up to a common factor 2^e,
    // where e is the rounding error of the reference m, at most half an ulp of
    // m.  That factor cancels in O and lse, and stays within 2^(+-1/4) while
    // |m| < 2^23.  A row whose largest scaled score reaches 2^23 in magnitude
    // (or leaves fp32) has no accurate result and gets NaN, written as a bit
    // pattern (the build assumes no NaN arithmetic).  m = -FLT_MAX means the
    // row saw no key.
    const float l32 = xhalf_sum(st.l32);
    const float l16 = xhalf_sum(st.l16);
    const bool in_range = fabsf(st.m) < kMaxRef || st.m == -3.402823466e38f;
    const float inv = l16 > 0.0f ? 1.0f / l16 : 0.0f;
    const uint32_t lse_bits = in_range ? as_u32(kLn2 * (st.m + __builtin_amdgcn_logf(l32))) : kNaN32;
    if constexpr (!SPLIT) {
        if (n_w == 0) return;
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + qbase, q_bytes);   // rows past Tq are dropped
        const uint32_t orow = (uint32_t)qrow * G::kRowBytes;
#pragma unroll
        for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 wv;
                wv.x = in_range ? pack_bf16x2(st.o[b][4 * g + 0] * inv, st.o[b][4 * g + 1] * inv) : kNaN16x2;
                wv.y = in_range ? pack_bf16x2(st.o[b][4 * g + 2] * inv, st.o[b][4 * g + 3] * inv) : kNaN16x2;
                __builtin_amdgcn_raw_buffer_store_b64(wv, ro, orow + 2 * (b * 32 + 8 * g + 4 * half), 0, 0);
            }
        if (half == 0) {
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(LSE + (size_t)bh * Tq, (uint32_t)Tq * 4u);
            __builtin_amdgcn_raw_buffer_store_b32(lse_bits, rl, (uint32_t)qrow * 4u, 0, 0);
        }
    } else {
        // Every row of the split is written, also those that saw no key.
        const size_t prow = (size_t)split * (size_t)a.rows + (size_t)bh * Tq;
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(OP + prow * D, (uint32_t)Tq * D * 4u);
        const uint32_t orow = (uint32_t)qrow * D * 4u;
#pragma unroll
        for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x4 wv = {as_u32(st.o[b][4 * g + 0] * inv), as_u32(st.o[b][4 * g + 1] * inv),
                            as_u32(st.o[b][4 * g + 2] * inv), as_u32(st.o[b][4 * g + 3] * inv)};
                if (!in_range) wv = kNaN32;
                __builtin_amdgcn_raw_buffer_store_b128(wv, ro, orow + 4 * (b * 32 + 8 * g + 4 * half), 0, 0);
            }
        if (half == 0) {
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(LP + prow, (uint32_t)Tq * 4u);
            __builtin_amdgcn_raw_buffer_store_b32(lse_bits, rl, (uint32_t)qrow * 4u, 0, 0);
        }
    }
}

template <int D, bool CAUSAL, int NG, bool SPLIT>
__global__ __launch_bounds__(256 * NG)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D, NG>, kWavesPerSimd<D, NG>)))
void fa_fwd_kernel(FwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[Geo<D, NG>::kLdsBytes];
    fa_fwd_block<D, CAUSAL, NG, SPLIT>(a.q, a.k, a.v, a.o, a.lse, a.op, a.lp, a, (FA_LDS char*)smem);
}

// Merge of the splits' partial results, the log-sum-exp combine of "FlashAttention
// and Fused Kernels: Attention Without the n x n Matrix", Step 4: with M the
// largest split lse, w_s = exp(lse_s - M), O = sum_s w_s O_s / sum_s w_s and
// lse = M + ln sum_s w_s.  D / 4 lanes per row, four values each; a split
// that saw no key (lse_s = -inf) gets weight zero.
template <int D>
__global__ __launch_bounds__(256) void fa_combine_kernel(const float* __restrict__ op, const float* __restrict__ lp,
                                                         uint16_t* __restrict__ o, float* __restrict__ lse,
                                                         long long rows, int n_split) {
    constexpr int kLanes = D / 4;
    constexpr int kRowsPerBlock = 256 / kLanes;
    const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
    const int t = threadIdx.x % kLanes;
    if (row >= rows) return;
    float m = -INFINITY;
    bool nan = false;   // a split that flagged its row (score outside fp32): the row is NaN
    for (int s = 0; s < n_split; ++s) {
        const float ls = lp[(size_t)s * rows + row];
        nan |= (as_u32(ls) & 0x7FFFFFFFu) > 0x7F800000u;
        m = fmaxf(m, ls);
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float l = 0.0f;
    for (int s = 0; s < n_split; ++s) {
        const float ls = lp[(size_t)s * rows + row];
        const float w = ls == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((ls - m) * (float)kLog2e);
        const u32x4 raw = *reinterpret_cast<const u32x4*>(op + ((size_t)s * rows + row) * D + 4 * t);
        l += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, as_f32(raw[e]), acc[e]);
    }
    const float inv = 1.0f / l;
    u32x2 wv;
    wv.x = nan ? kNaN16x2 : pack_bf16x2(acc[0] * inv, acc[1] * inv);
    wv.y = nan ? kNaN16x2 : pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2*>(o + (size_t)row * D + 4 * t) = wv;
    if (t == 0) reinterpret_cast<uint32_t*>(lse)[row] = nan ? kNaN32 : as_u32(m + kLn2 * __builtin_amdgcn_logf(l));
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

template <int D, bool CAUSAL, int NG, bool SPLIT>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, NG, SPLIT>), dim3(a.total), dim3(Geo<D, NG>::kThreads), 0, stream,
                       a);
    return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_d(const FwdArgs& a, bool causal, int ng, hipStream_t stream) {
    if (ng == 2) return causal ? launch<D, true, 2, SPLIT>(a, stream) : launch<D, false, 2, SPLIT>(a, stream);
    return causal ? launch<D, true, 1, SPLIT>(a, stream) : launch<D, false, 1, SPLIT>(a, stream);
}

// Keys per split: the split count spread evenly, rounded up to whole key tiles.
int64_t split_chunk(int64_t Tk, int64_t n_split) {
    const int64_t per = (Tk + n_split - 1) / n_split;
    return (per + kBN - 1) / kBN * kBN;
}

// The library's fixed split-key scratch, for callers that cannot allocate
// (fa_fwd_split_noalloc).  Each GPU holds its own copy until the process
// ends.  Host code never passes `scratch` itself to a kernel: its device
// address, per device, comes from hipGetSymbolAddress (fixed_scratch).
constexpr size_t kScratchBytes = FA_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device that `stream` runs on, looked
// up once per device with that device current.
fa_status fixed_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (err != hipSuccess) {
        fa_internal::record_hip_error(err);
        return FA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        err = hipGetDevice(&cur);
        if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
        void* ptr = nullptr;
        if (err == hipSuccess) err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess || !ptr) {
            fa_internal::record_hip_error(err != hipSuccess ? err : hipErrorInvalidSymbol);
            return FA_ERR_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

// The general forward behind every entry point.  With fixed_ws, the split
// workspace is the library's fixed scratch instead of the caller's.
fa_status run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                  int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal, float scale, int64_t n_split,
                  void* workspace, size_t workspace_bytes, hipStream_t stream, bool fixed_ws = false) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (causal && Tq > Tk) return FA_ERR_SHAPE;
    if (n_split < 1) return FA_ERR_ARG;
    if (!std::isfinite(scale)) return FA_ERR_SCALE;
    // The kernels take the exponent factor scale * log2(e) in fp32; past
    // ~2.4e38 it would be infinite and a zero score would give 0 * inf = NaN.
    if (!std::isfinite(static_cast<float>(static_cast<double>(scale) * kLog2e))) return FA_ERR_SCALE;
    const auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if ((addr(q) | addr(k) | addr(v) | addr(o) | addr(workspace)) & 15u) return FA_ERR_ALIGN;

    // Grouped heads whose rows all see the same keys (no mask, or one query
    // row, which sees every key) are one problem per key/value head: the
    // group's query rows [h0, h0 + group) x [0, Tq) are contiguous in q, o and
    // lse, so they run as group * Tq query rows of that head, and each K/V
    // tile is loaded once for the whole group.
    if (Hq != Hkv && (!causal || Tq == 1)) {
        if (Tq > INT32_MAX / (Hq / Hkv)) return FA_ERR_OVERFLOW;   // folded rows are 32-bit indices
        Tq *= Hq / Hkv;
        Hq = Hkv;
        causal = 0;   // a single query row per head sees every key either way
    }
    if (addr(lse) & 3u) return FA_ERR_ALIGN;

    // Workgroup shape: the phase-alternating 8-wave workgroup pays off when
    // d = 128 and each query tile walks many key tiles (T >= 8192 causal, or
    // T >= 4096 without the mask); otherwise two independent 4-wave workgroups
    // per CU are faster.  Both shapes give bit-identical results.
    const int ng = d == 128 && Tq * (causal ? 1 : 2) >= 8192 ? 2 : 1;
    const int64_t bm = 128 * ng;

    // Sizes: every byte count must fit int64; in-kernel row and key indices are 32-bit.
    const int64_t kMax = INT64_MAX;
    if (B > kMax / Hq) return FA_ERR_OVERFLOW;
    const int64_t BH = B * Hq, BHkv = B * Hkv;
    if (BH > kMax / Tq || BHkv > kMax / Tk) return FA_ERR_OVERFLOW;
    const int64_t rows = BH * Tq, kv_rows = BHkv * Tk;
    if (rows > kMax / (4 * (d + 1)) || kv_rows > kMax / (2 * d)) return FA_ERR_OVERFLOW;
    if (Tq > INT32_MAX - 2 * bm || Tk > INT32_MAX - 2 * bm) return FA_ERR_OVERFLOW;
    // Buffer descriptors address one head: (T + 2 tiles) rows must fit in 32-bit byte offsets.
    if ((Tq + 2 * bm) * 4 * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;
    if ((Tk + 2 * bm) * 2 * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;
    const int64_t chunk = split_chunk(Tk, n_split);
    const int64_t n_eff = (Tk + chunk - 1) / chunk;   // splits that hold at least one key
    const int64_t n_qt = (Tq + bm - 1) / bm;
    if (BH > INT32_MAX / (n_qt * n_eff)) return FA_ERR_OVERFLOW;

    const size_t q_bytes = static_cast<size_t>(rows) * static_cast<size_t>(d) * 2u;
    const size_t kv_bytes = static_cast<size_t>(kv_rows) * static_cast<size_t>(d) * 2u;
    const size_t lse_bytes = static_cast<size_t>(rows) * 4u;
    const size_t ws_need = n_eff > 1 ? static_cast<size_t>(n_eff) * static_cast<size_t>(rows) * (d + 1) * 4u : 0;
    if (n_eff > 1 && rows > static_cast<int64_t>(INT32_MAX) * (256 / (d / 4))) return FA_ERR_OVERFLOW;   // combine grid
    const struct { const void* p; size_t n; } ins[3] = {{q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}};
    for (const auto& in : ins)
        if (overlaps(o, q_bytes, in.p, in.n) || overlaps(lse, lse_bytes, in.p, in.n)) return FA_ERR_ARG;
    if (overlaps(o, q_bytes, lse, lse_bytes)) return FA_ERR_ARG;
    if (fixed_ws) {   // every argument is checked by now: the HIP calls start here
        if (ws_need > kScratchBytes) return FA_ERR_SCRATCH;
        workspace = nullptr;
        workspace_bytes = 0;
        if (ws_need > 0) {
            const fa_status st = fixed_scratch(stream, &workspace);
            if (st != FA_OK) return st;
            workspace_bytes = kScratchBytes;
        }
    }
    if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return workspace ? FA_ERR_ARG : FA_ERR_NULL;
    for (const auto& in : ins)
        if (ws_need && overlaps(workspace, ws_need, in.p, in.n)) return FA_ERR_ARG;
    if (ws_need && (overlaps(workspace, ws_need, o, q_bytes) || overlaps(workspace, ws_need, lse, lse_bytes)))
        return FA_ERR_ARG;

    FwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.op = static_cast<float*>(workspace);
    a.lp = ws_need ? static_cast<float*>(workspace) + static_cast<size_t>(n_eff) * rows * d : nullptr;
    a.rows = rows;
    a.tq = static_cast<int>(Tq);
    a.tk = static_cast<int>(Tk);
    a.n_qt = static_cast<int>(n_qt);
    a.total = static_cast<int>(BH * n_qt * n_eff);
    a.hq = static_cast<int>(Hq);
    a.group = static_cast<int>(Hq / Hkv);
    a.chunk = static_cast<int>(chunk);
    a.n_split = static_cast<int>(n_eff);
    a.c = static_cast<float>(static_cast<double>(scale) * kLog2e);

    hipError_t err;
    if (n_eff == 1) {
        err = d == 128 ? launch_d<128, false>(a, causal, ng, stream) : launch_d<64, false>(a, causal, ng, stream);
    } else {
        err = d == 128 ? launch_d<128, true>(a, causal, ng, stream) : launch_d<64, true>(a, causal, ng, stream);
        if (err == hipSuccess)
            err = fa_internal::launch_split_combine(a.op, a.lp, a.o, lse, rows, a.n_split, static_cast<int>(d), stream);
    }
    if (err != hipSuccess) {
        fa_internal::record_hip_error(err);
        return FA_ERR_HIP;
    }
    fa_internal::clear_hip_error();
    return FA_OK;
}

}  // namespace

namespace fa_internal {

thread_local char g_hip_error[256] = "";

void record_hip_error(hipError_t err) {
    std::snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", hipGetErrorName(err), hipGetErrorString(err));
}

void clear_hip_error() { g_hip_error[0] = '\0'; }

hipError_t launch_split_combine(const float* op, const float* lp, uint16_t* o, float* lse, long long rows, int n_split,
                                int d, hipStream_t stream) {
    const int rpb = 256 / (d / 4);   // rows per 256-thread block
    const long long blocks = (rows + rpb - 1) / rpb;
    if (d == 128)
        hipLaunchKernelGGL(fa_combine_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, op, lp, o,
                           lse, rows, n_split);
    else
        hipLaunchKernelGGL(fa_combine_kernel<64>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, op, lp, o,
                           lse, rows, n_split);
    return hipGetLastError();
}

}  // namespace fa_internal

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                            int64_t H, int64_t T, int64_t d, int causal, float scale, hipStream_t stream) {
    return run_fwd(q, k, v, o, lse, B, H, H, T, T, d, causal, scale, 1, nullptr, 0, stream);
}

extern "C" fa_status fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t T, int64_t d, int causal, float scale,
                                hipStream_t stream) {
    return run_fwd(q, k, v, o, lse, B, Hq, Hkv, T, T, d, causal, scale, 1, nullptr, 0, stream);
}

extern "C" size_t fa_fwd_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Tq, int64_t Tk, int64_t d,
                                               int64_t n_split) {
    if (B < 1 || Hq < 1 || Tq < 1 || Tk < 1 || d < 1 || n_split < 1) return 0;
    const int64_t chunk = split_chunk(Tk, n_split);
    const int64_t n_eff = (Tk + chunk - 1) / chunk;
    if (n_eff == 1) return 0;
    const double bytes = (double)n_eff * (double)B * (double)Hq * (double)Tq * (double)(d + 1) * 4.0;
    if (bytes > 9.0e18) return 0;
    return static_cast<size_t>(n_eff * B * Hq * Tq * (d + 1) * 4);
}

extern "C" int64_t fa_fwd_split_count(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                                      int causal) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Tq < 1 || Tk < 1 || (d != 64 && d != 128)) return 1;
    if (Hq != Hkv && (!causal || Tq == 1)) {   // folded as in the forward itself
        if (Tq > INT32_MAX / (Hq / Hkv)) return 1;   // the forward rejects this shape
        Tq *= Hq / Hkv;
        Hq = Hkv;
        causal = 0;
    }
    const int64_t ng = d == 128 && Tq * (causal ? 1 : 2) >= 8192 ? 2 : 1;
    const int64_t slots = 256 * (ng == 2 ? 1 : (d == 64 ? 3 : 2));   // CUs x resident workgroups per CU
    if (B >= slots || Hq >= slots) return 1;                   // a full round already (and no overflow below)
    const int64_t wgs = B * Hq * ((Tq + 128 * ng - 1) / (128 * ng));
    if (wgs >= slots) return 1;
    // About one round of workgroups: a decode sweep on MI355X (64 query
    // workgroups, 32768 keys) ran fastest at 4-8 splits and 5% slower at 16.
    int64_t n = (slots + wgs - 1) / wgs;
    n = std::min<int64_t>(n, std::max<int64_t>(1, Tk / 128));  // at least two key tiles per split
    return std::min<int64_t>(n, 64);
}

extern "C" fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                  int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal,
                                  float scale, int64_t n_split, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    return run_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, n_split, workspace, workspace_bytes,
                   stream);
}

extern "C" fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                          int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal,
                                          float scale, int64_t n_split, hipStream_t stream) {
    return run_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, n_split, nullptr, 0, stream, true);
}

extern "C" const char* fa_status_string(int status) {
    switch (status) {   // an int: a C caller may pass any value, and only the listed ones are fa_status values
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "sizes must be >= 1, Hq a multiple of Hkv, and Tq <= Tk when causal";
        case FA_ERR_HEAD_DIM: return "head size d must be 64 or 128";
        case FA_ERR_SCALE: return "scale (and scale * log2(e) in fp32; FP8: the descales, > 0) must be finite";
        case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case FA_ERR_OVERFLOW: return "sizes overflow the supported index range";
        case FA_ERR_HIP: return "HIP kernel launch failed";
        case FA_ERR_ARG: return "bad argument: causal not 0/1, n_split < 1, workspace too small, or overlapping buffers";
        case FA_ERR_SCRATCH: return "the split keys need more scratch than the library's fixed buffer (FA_SCRATCH_BYTES)";
    }
    return "unknown status";
}

extern "C" const char* fa_hip_error_string(void) { return fa_internal::g_hip_error; }
