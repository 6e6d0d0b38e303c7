// fa_fwd_fp8.hip -- exact attention forward with FP8 E4M3 inputs for MI355X
// (gfx950, CDNA4), and its C ABI.
//
// The method is the tiled online-softmax forward of the bf16 path ("Flash
// Attention, tiled: exact attention without the T x T HBM matrix", section
// "From the example to tiled GPU work"; "FlashAttention: the IO-aware Attention
// Kernel", sections 3.2-3.3), fed with Q, K, V in OCP FP8 E4M3 and one fp32
// descale factor per tensor, the FP8 mode that "FlashAttention and Fused
// Kernels: Attention Without the n x n Matrix" ("Four generations") names for
// FlashAttention-3.  Both products run on the FP8 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, k = 64, twice the bf16 rate); the probability
// weights enter the PV product as E4M3, which is the one approximation beyond
// rounding order.
//
// gfx950 mapping (the same pipeline as the bf16 kernel):
//   * Waves own 32 query rows each and compute S^T = K_j Q^T.  With one MFMA
//     covering 64 values of the contraction, a lane's A/B operand is 32 bytes:
//     K row (lane % 32) and Q row (lane % 32), head-dim bytes
//     64 s + 32 (lane / 32) + [0, 32).  The operand layout is symmetric in
//     (lane / 32, byte), so any assignment of the contraction index to bytes
//     that A and B share is valid.
//   * O^T += V_j^T P^T.  The 32 fp32 scores a lane holds (one query row, the
//     keys 32 kb + 8 (i / 4) + 4 (lane / 32) + i % 4 of accumulator element i
//     of block kb) are converted to E4M3 in that order and are the B operand
//     as they stand: one MFMA per 32 head-dim rows covers the whole 64-key
//     tile.  The A operand (V^T, 32 keys of one head-dim column per lane, in
//     the same key order) comes from four ds_read_b64_tr_b8: in each 16-lane
//     group, lane i receives column i of an 8-row x 16-byte block whose row b
//     is addressed by lanes 2b and 2b + 1, so each lane addresses the key row
//     that its byte slot needs.
//   * The weights are formed as 2^3 * 2^(x - m) against a lazily moved
//     reference m (the conditional rescale of FlashAttention-4 on the same
//     page): the tile max is taken only when a lane's tile sum exceeds 448
//     (so that some weight may), and then a row's reference moves to its max
//     if that grew by more than 2^5.  So every weight lies in (0, 448], inside
//     E4M3's range (the conversion does not saturate), the reference never
//     exceeds the row max, so the largest weight of a row is at least 8, which
//     keeps the subnormal rounding of the small weights negligible, and rows of
//     equal scores (weights 8, tile sums 256) never take the max.
//   * O is normalised by the sum of the E4M3 weights the product actually
//     used, taken by one more MFMA against an all-ones A operand (the matrix
//     cores have slack here, the exponentials set the pace); the log-sum-exp
//     uses the fp32 sum.  The descale factors are folded into the exponent
//     constant (Q, K) and into the final division (V).
//   * K_j and V_j tiles (64 keys x d bytes) go HBM -> LDS by buffer_load ... lds,
//     16-byte chunks XOR-swizzled by row so that the ds_read_b128 K reads and
//     the transposed V reads are free of bank conflicts.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_internal.h"

namespace {

#define FA_LDS __attribute__((address_space(3)))

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;          // keys per K/V tile
constexpr int kXcds = 8;
constexpr double kLog2e = 1.4426950408889634;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kWeightShift = 3.0f;       // weights are 2^3 * 2^(x - m_ref)
constexpr float kRescaleThreshold = 8.0f;  // rescale when 2^(x - m) may exceed 2^8 (max grew by > 2^5)
constexpr float kSpecSum = 448.0f;         // a lane's tile sum <= 448 bounds each weight by E4M3's largest
constexpr uint32_t kBufferFlags = 0x00020000u;
constexpr uint32_t kNaN32 = 0x7FC00000u;     // quiet NaN, fp32 bits
constexpr uint32_t kNaN16x2 = 0x7FC07FC0u;   // two quiet NaNs, bf16 bits
constexpr int kOnesE4m3 = 0x38383838;      // four E4M3 ones

template <int D, int NG>
struct Geo8 {
    static constexpr int kWaves = 4 * NG;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBM = 32 * kWaves;
    static constexpr int kRowBytes = D;               // one byte per element
    static constexpr int kChunks = D / 16;            // 16-byte chunks per row
    static constexpr int kTileBytes = kBN * kRowBytes;
    static constexpr int kLoads = kTileBytes / 1024 / kWaves;
    static constexpr int kDSteps = D / 64;            // MFMA steps over d for S^T
    static constexpr int kDBlocks = D / 32;           // 32-row blocks of O^T
    static constexpr int kLdsBytes = 4 * kTileBytes;  // K slot 0, K slot 1, V slot 0, V slot 1
    static_assert(kLoads >= 1, "each wave must load at least one 1 KB block per tile");
};

// XOR swizzle of the 16-byte chunk index within a tile row.  D = 128 (8 chunks
// of 128-byte rows, two rows per 64 banks): a bit permutation of (row / 2) % 8
// that also keeps rows 4 apart on chunk parities of their own, so the two
// 16-lane halves of a transposed read (chunks c and c ^ 1, the same 8 keys)
// meet disjoint banks.  D = 64 (4 chunks, four rows per 64 banks): (row / 4) % 4.
template <int D>
__device__ __forceinline__ int swz8(int r) {
    if constexpr (D == 128) {
        const int t = (r >> 1) & 7;
        return ((t >> 1) & 1) | ((t & 1) << 1) | (t & 4);
    } else {
        return (r >> 2) & 3;
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float xhalf_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return fmaxf(as_f32(r[0]), as_f32(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return as_f32(r[0]) + as_f32(r[1]);
}

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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

// Four fp32 weights -> four E4M3 bytes (round to nearest even), first weight in byte 0.
__device__ __forceinline__ int pack_e4m3x4(float a, float b, float c, float d) {
    int t = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, t, true);
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    // cbsz = blgp = 0: both operands E4M3; zero scale operands select the unscaled form.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D>
struct WaveState8 {
    f32x16 o[Geo8<D, 1>::kDBlocks];   // O^T accumulator (one query row per lane)
    f32x16 l8;                        // sum of the E4M3 weights, in every element
    float m = -3.402823466e38f;       // reference, exp2 units, minus the weight shift
    float l32 = 0.0f;                 // sum of the fp32 weights
};

template <int D>
__device__ __forceinline__ void maybe_rescale8(WaveState8<D>& st, float m_new) {
    const bool need = m_new > st.m + kRescaleThreshold;
    if (__any(need)) {
        const float m_to = m_new - kWeightShift;
        const float r = need ? __builtin_amdgcn_exp2f(st.m - m_to) : 1.0f;
        st.m = need ? m_to : st.m;
        st.l32 *= r;
#pragma unroll
        for (int i = 0; i < 16; ++i) st.l8[i] *= r;
#pragma unroll
        for (int b = 0; b < Geo8<D, 1>::kDBlocks; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.o[b][i] *= r;
    }
}

// Launch arguments; head mapping, causal alignment and key splits as for the
// bf16 forward: key range [s * chunk, (s + 1) * chunk) goes to split s, and
// with SPLIT the workgroup writes that split's normalised fp32 output and
// log-sum-exp to op / lp for the combine kernel.
struct Fwd8Args {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    uint16_t* o;
    float* lse;
    float* op;     // [n_split][rows][D]
    float* lp;     // [n_split][rows]
    long long rows;
    int tq, tk, n_qt, total, hq, group, chunk, n_split;
    float c;        // scale * q_descale * k_descale * log2(e)
    float vscale;   // v_descale
};

template <int D, bool CAUSAL, int NG, bool SPLIT>
__device__ __forceinline__ void fa_fwd8_block(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                              const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
                                              float* __restrict__ LSE, float* __restrict__ OP, float* __restrict__ LP,
                                              const Fwd8Args& a, FA_LDS char* const lds) {
    using G = Geo8<D, NG>;
    constexpr int kBM = G::kBM;
    const int Tq = a.tq, Tk = a.tk, n_qt = a.n_qt, total = a.total;
    const float c_in = a.c;
    FA_LDS char* const kslot[2] = {lds, lds + G::kTileBytes};
    FA_LDS char* const vslot[2] = {lds + 2 * G::kTileBytes, lds + 3 * G::kTileBytes};

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = NG == 2 ? wave >> 2 : 0;
    const int col = lane & 31;
    const int half = lane >> 5;

    // Work decode: XCD-contiguous remap, heavy causal tiles first (as the bf16 forward).
    const int id = blockIdx.x;
    const int xcd = id % kXcds, xslot = id / kXcds;
    const int q8 = total / kXcds, r8 = total % kXcds;
    const int w = xcd < r8 ? xcd * (q8 + 1) + xslot : r8 * (q8 + 1) + (xcd - r8) * q8 + xslot;
    int bh = w / (n_qt * a.n_split);
    const int split = (w / n_qt) % a.n_split;
    int qt = CAUSAL ? n_qt - 1 - (w % n_qt) : (w % n_qt);
    constexpr int kRoundSlots = 256 * (NG == 2 ? 1 : 2);
    if (CAUSAL && a.n_split == 1 && r8 == 0 && q8 % n_qt == 0 && total <= 8 * kRoundSlots) {
        const int hx = q8 / n_qt;
        bh = xcd * hx + xslot % hx;
        qt = n_qt - 1 - xslot / hx;
    }

    const int kvh = (bh / a.hq) * (a.hq / a.group) + (bh % a.hq) / a.group;
    const size_t qbase = (size_t)bh * (size_t)Tq * D;
    const size_t kvbase = (size_t)kvh * (size_t)Tk * D;
    const uint8_t* __restrict__ kbh = K + kvbase;
    const uint8_t* __restrict__ vbh = V + kvbase;

    const int blk = NG == 2 ? 2 * (wave & 3) + grp : wave;
    const int qw0 = qt * kBM + blk * 32;
    const int qrow = qw0 + col;
    const int off = Tk - Tq;
    const int k_lo = split * a.chunk;
    const int k_hi = min(Tk, k_lo + a.chunk);
    const int kv_end = CAUSAL ? min(k_hi, min(Tq, qt * kBM + kBM) + off) : k_hi;
    const int n_kt = kv_end > k_lo ? (kv_end - k_lo + kBN - 1) / kBN : 0;   // tiles the workgroup loads
    const int w_end = CAUSAL ? min(k_hi, qw0 + 32 + off) : k_hi;            // keys this wave may see
    const int n_w = qw0 >= Tq || w_end <= k_lo ? 0 : (w_end - k_lo + kBN - 1) / kBN;
    // Tiles from j_mask on can hold keys some row of the wave must not see.
    const int j_mask = CAUSAL ? min(n_w - 1, max(0, (qw0 + off + 1 - k_lo) / kBN)) : n_w - 1;

    uint32_t goff[G::kLoads];
#pragma unroll
    for (int c = 0; c < G::kLoads; ++c) {
        const int q = (wave * G::kLoads + c) * 64 + lane;
        const int r = q / G::kChunks, p = q % G::kChunks;
        goff[c] = r * G::kRowBytes + 16 * (p ^ swz8<D>(r));
    }
    auto load_tile = [&] __device__ (const uint8_t* src, int key0, FA_LDS char* slot) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (size_t)key0 * D, (uint32_t)(Tk - key0) * G::kRowBytes);
#pragma unroll
        for (int c = 0; c < G::kLoads; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(slot + (wave * G::kLoads + c) * 1024), 16,
                                                     goff[c], 0, 0, 0);
    };

    // K operand (A of S^T): key row `col` (+ 32 kb), logical chunks 4 s + 2 half + {0, 1}.
    uint32_t koff[G::kDSteps][2];
#pragma unroll
    for (int s = 0; s < G::kDSteps; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) koff[s][h] = col * G::kRowBytes + 16 * ((4 * s + 2 * half + h) ^ swz8<D>(col));
    // V^T operand: in 16-lane group g, lane i addresses key row
    // 8 (b / 4) + 4 half + b % 4 (b = i / 2; plus 16 per read e) at the 8-byte
    // half i % 2 of logical chunk 2 db + g % 2.  The swizzle of those rows does
    // not depend on e, so the four reads differ by an immediate 16 rows.
    uint32_t voff[G::kDBlocks];
    {
        const int g = lane >> 4, i = lane & 15, b = i >> 1;
        const int r = 8 * (b >> 2) + 4 * half + (b & 3);
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db)
            voff[db] = r * G::kRowBytes + 16 * ((2 * db + (g & 1)) ^ swz8<D>(r)) + 8 * (i & 1);
    }

    if (n_kt > 0) load_tile(kbh, k_lo, kslot[0]);

    // Q^T operand (B of S^T): Q row qrow, bytes 64 s + 32 half + [0, 32); zeros past Tq.
    i32x8 qf[G::kDSteps];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qbase, (uint32_t)Tq * G::kRowBytes);
        const uint32_t neg = c_in < 0.0f ? 0x80808080u : 0u;   // a negative scale negates Q
#pragma unroll
        for (int s = 0; s < G::kDSteps; ++s) {
            const uint32_t base = (uint32_t)qrow * G::kRowBytes + 64 * s + 32 * half;
            u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rq, base, 0, 0);
            u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rq, base + 16, 0, 0);
            lo ^= neg;
            hi ^= neg;
            const i32x8 v8 = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            qf[s] = v8;
        }
    }
    const float c = fmaxf(fabsf(c_in), 1e-30f);

    WaveState8<D> st;
#pragma unroll
    for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[b][i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) st.l8[i] = 0.0f;
    const i32x8 ones = {kOnesE4m3, kOnesE4m3, kOnesE4m3, kOnesE4m3, kOnesE4m3, kOnesE4m3, kOnesE4m3, kOnesE4m3};

    auto qk = [&] __device__ (FA_LDS const char* ks, f32x16 (&s)[2]) {
        i32x8 a[2][G::kDSteps];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st_ = 0; st_ < G::kDSteps; ++st_) {
                const u32x4 lo = *(FA_LDS const u32x4*)(ks + kb * 32 * G::kRowBytes + koff[st_][0]);
                const u32x4 hi = *(FA_LDS const u32x4*)(ks + kb * 32 * G::kRowBytes + koff[st_][1]);
                const i32x8 v8 = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                a[kb][st_] = v8;
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
        for (int st_ = 0; st_ < G::kDSteps; ++st_)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma8(a[kb][st_], qf[st_], s[kb]);
    };
    auto v_operand = [&] __device__ (FA_LDS const char* vs, int db) {
        i32x2 r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[e] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)(vs + e * 16 * G::kRowBytes + voff[db]));
        const i32x8 v8 = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
        return v8;
    };
    auto pv = [&] __device__ (FA_LDS const char* vs, const i32x8& pk) {
        i32x8 va[G::kDBlocks];
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db) va[db] = v_operand(vs, db);
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db) st.o[db] = mfma8(va[db], pk, st.o[db]);
        st.l8 = mfma8(ones, pk, st.l8);
    };

    f32x16 sc[2];
    // fp32 weights of the current tile.  The next matrix phase converts them
    // to E4M3 (the conversion hides under its first LDS reads): with FP8
    // products the matrix phase is the shorter one, and moving this VALU work
    // there keeps a wave's softmax phase from outlasting its partner's matrix
    // phase (the two waves of a SIMD then contend less for the VALU).
    float pw[32];

    auto matrix_phase = [&] __device__ (int j, auto parity) {
        constexpr int P = decltype(parity)::value;
        __builtin_amdgcn_s_setprio(1);
        const bool do_pv = j >= 0 && j < n_w;
        const bool do_qk = j + 1 < n_w;
        if (do_pv) {
            i32x8 pk;
#pragma unroll
            for (int n = 0; n < 8; ++n) pk[n] = pack_e4m3x4(pw[4 * n], pw[4 * n + 1], pw[4 * n + 2], pw[4 * n + 3]);
            pv(vslot[P], pk);
        }
        if (do_qk) qk(kslot[P ^ 1], sc);
        __builtin_amdgcn_s_setprio(0);
    };
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
        // Weights against the current reference; only when some lane's tile sum
        // exceeds 448 (so that some weight may) is the tile max taken.
        float p[32];
        float ts;
        auto weights = [&] __device__ () {
            const float mneg = -st.m;
#pragma unroll
            for (int n = 0; n < 32; ++n)
                p[n] = __builtin_amdgcn_exp2f(__builtin_fmaf(n < 16 ? sc[0][n] : sc[1][n - 16], c, mneg));
            float t8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) t8[q] = (p[4 * q] + p[4 * q + 1]) + (p[4 * q + 2] + p[4 * q + 3]);
            ts = ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
        };
        weights();
        if (__any(!(ts <= kSpecSum))) {
            maybe_rescale8<D>(st, tile_max(sc) * c);
            weights();
        }
        st.l32 += ts;
#pragma unroll
        for (int n = 0; n < 32; ++n) pw[n] = p[n];
    };

    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    const int n_ph = 2 * n_kt + 2;
    auto phase_start = [&] __device__ (int ph) {
        if ((ph & 1) == 0) {
            const int j = ph >> 1;
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the loads of phase ph - 2 have landed
            __syncthreads();
            if (j + 1 < n_kt) load_tile(kbh, k_lo + (j + 1) * kBN, kslot[(j + 1) & 1]);
            if (j < n_kt) load_tile(vbh, k_lo + j * kBN, vslot[j & 1]);
        }
    };
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

    // Epilogue: O = v_descale * o / l8, lse = ln2 * (m + log2 l32).  A row that
    // saw no key (possible only for one split of a split problem) gets O = 0,
    // lse = -inf.  A row whose largest scaled score reaches 2^23 in magnitude
    // (log2 units) has no accurate result, as in the bf16 forward (there the
    // reference's rounding could also push a weight past 448), and gets NaN,
    // written as a bit pattern (the build assumes no NaN arithmetic).
    const float l32 = xhalf_sum(st.l32);
    const float l8 = st.l8[0];
    const bool in_range = fabsf(st.m) < 8388608.0f || st.m == -3.402823466e38f;
    const float inv = l8 > 0.0f ? a.vscale / l8 : 0.0f;
    const uint32_t lse_bits = in_range ? as_u32(kLn2 * (st.m + __builtin_amdgcn_logf(l32))) : kNaN32;
    if constexpr (SPLIT) {
        // Every row of the split is written, also those that saw no key.
        const size_t prow = (size_t)split * (size_t)a.rows + (size_t)bh * Tq;
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(OP + prow * D, (uint32_t)Tq * D * 4u);
        const uint32_t prow_b = (uint32_t)qrow * D * 4u;
#pragma unroll
        for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x4 wv = {as_u32(st.o[b][4 * g + 0] * inv), as_u32(st.o[b][4 * g + 1] * inv),
                            as_u32(st.o[b][4 * g + 2] * inv), as_u32(st.o[b][4 * g + 3] * inv)};
                if (!in_range) wv = kNaN32;
                __builtin_amdgcn_raw_buffer_store_b128(wv, rp, prow_b + 4 * (b * 32 + 8 * g + 4 * half), 0, 0);
            }
        if (half == 0) {
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(LP + prow, (uint32_t)Tq * 4u);
            __builtin_amdgcn_raw_buffer_store_b32(lse_bits, rl, (uint32_t)qrow * 4u, 0, 0);
        }
        return;
    }
    if (n_w == 0) return;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + qbase, (uint32_t)Tq * D * 2u);
    const uint32_t orow = (uint32_t)qrow * D * 2u;
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
}

template <int D, bool CAUSAL, int NG, bool SPLIT>
__global__ __launch_bounds__(256 * NG) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(Fwd8Args a) {
    __shared__ __attribute__((aligned(1024))) char smem[Geo8<D, NG>::kLdsBytes];
    fa_fwd8_block<D, CAUSAL, NG, SPLIT>(a.q, a.k, a.v, a.o, a.lse, a.op, a.lp, a, (FA_LDS char*)smem);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

template <int D, bool CAUSAL, int NG, bool SPLIT>
hipError_t launch8(const Fwd8Args& a, hipStream_t stream) {
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, NG, SPLIT>), dim3(a.total), dim3(Geo8<D, NG>::kThreads), 0, stream,
                       a);
    return hipGetLastError();
}

template <bool SPLIT>
hipError_t launch8_d(const Fwd8Args& a, int64_t d, bool causal, int ng, hipStream_t stream) {
    if (d == 128) {
        if (ng == 2) return causal ? launch8<128, true, 2, SPLIT>(a, stream) : launch8<128, false, 2, SPLIT>(a, stream);
        return causal ? launch8<128, true, 1, SPLIT>(a, stream) : launch8<128, false, 1, SPLIT>(a, stream);
    }
    return causal ? launch8<64, true, 1, SPLIT>(a, stream) : launch8<64, false, 1, SPLIT>(a, stream);
}

// Keys per split: the split count spread evenly, rounded up to whole key tiles
// (the layout fa_fwd_split_workspace_bytes sizes).
int64_t split_chunk8(int64_t Tk, int64_t n_split) {
    const int64_t per = (Tk + n_split - 1) / n_split;
    return (per + kBN - 1) / kBN * kBN;
}

fa_status run_fwd8(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal, float scale, float q_descale,
                   float k_descale, float v_descale, int64_t n_split, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (causal && Tq > Tk) return FA_ERR_SHAPE;
    if (n_split < 1) return FA_ERR_ARG;
    if (!std::isfinite(scale)) return FA_ERR_SCALE;
    for (float ds : {q_descale, k_descale, v_descale})
        if (!std::isfinite(ds) || !(ds > 0.0f)) return FA_ERR_SCALE;
    const double cd = static_cast<double>(scale) * q_descale * k_descale * kLog2e;
    if (!std::isfinite(static_cast<float>(cd))) return FA_ERR_SCALE;
    const auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if ((addr(q) | addr(k) | addr(v) | addr(o) | addr(workspace)) & 15u) return FA_ERR_ALIGN;
    if (addr(lse) & 3u) return FA_ERR_ALIGN;

    // Grouped heads whose rows all see the same keys run as one problem per
    // key/value head (the group's query rows are contiguous), as for bf16.
    if (Hq != Hkv && (!causal || Tq == 1)) {
        if (Tq > INT32_MAX / (Hq / Hkv)) return FA_ERR_OVERFLOW;   // folded rows are 32-bit indices
        Tq *= Hq / Hkv;
        Hq = Hkv;
        causal = 0;
    }
    const int ng = d == 128 && Tq * (causal ? 1 : 2) >= 8192 ? 2 : 1;
    const int64_t bm = 128 * ng;

    const int64_t kMax = INT64_MAX;
    if (B > kMax / Hq) return FA_ERR_OVERFLOW;
    const int64_t BH = B * Hq, BHkv = B * Hkv;
    if (BH > kMax / Tq || BHkv > kMax / Tk) return FA_ERR_OVERFLOW;
    const int64_t rows = BH * Tq, kv_rows = BHkv * Tk;
    if (rows > kMax / (2 * d) || kv_rows > kMax / d) return FA_ERR_OVERFLOW;
    if (Tq > INT32_MAX - 2 * bm || Tk > INT32_MAX - 2 * bm) return FA_ERR_OVERFLOW;
    // Buffer descriptors address one head: (T + 2 tiles) rows of O (2 bytes an
    // element) must fit in 32-bit byte offsets, and so must the FP8 K/V rows.
    if ((Tq + 2 * bm) * 2 * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;
    if ((Tk + 2 * bm) * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;
    if (rows > kMax / (4 * (d + 1))) return FA_ERR_OVERFLOW;   // split workspace
    const int64_t chunk = split_chunk8(Tk, n_split);
    const int64_t n_eff = (Tk + chunk - 1) / chunk;   // splits that hold at least one key
    const int64_t n_qt = (Tq + bm - 1) / bm;
    if (BH > INT32_MAX / (n_qt * n_eff)) return FA_ERR_OVERFLOW;
    if (n_eff > 1 && rows > static_cast<int64_t>(INT32_MAX) * (256 / (d / 4))) return FA_ERR_OVERFLOW;   // combine grid
    // The fp32 partial rows of one head (4 bytes an element) must fit in 32-bit byte offsets too.
    if (n_eff > 1 && (Tq + 2 * bm) * 4 * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;

    const size_t q_bytes = static_cast<size_t>(rows) * static_cast<size_t>(d);
    const size_t o_bytes = 2u * q_bytes;
    const size_t kv_bytes = static_cast<size_t>(kv_rows) * static_cast<size_t>(d);
    const size_t lse_bytes = static_cast<size_t>(rows) * 4u;
    const struct { const void* p; size_t n; } ins[3] = {{q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}};
    const size_t ws_need = n_eff > 1 ? static_cast<size_t>(n_eff) * static_cast<size_t>(rows) * (d + 1) * 4u : 0;
    if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return workspace ? FA_ERR_ARG : FA_ERR_NULL;
    for (const auto& in : ins) {
        if (overlaps(o, o_bytes, in.p, in.n) || overlaps(lse, lse_bytes, in.p, in.n)) return FA_ERR_ARG;
        if (ws_need && overlaps(workspace, ws_need, in.p, in.n)) return FA_ERR_ARG;
    }
    if (overlaps(o, o_bytes, lse, lse_bytes)) return FA_ERR_ARG;
    if (ws_need && (overlaps(workspace, ws_need, o, o_bytes) || overlaps(workspace, ws_need, lse, lse_bytes)))
        return FA_ERR_ARG;

    Fwd8Args a;
    a.q = static_cast<const uint8_t*>(q);
    a.k = static_cast<const uint8_t*>(k);
    a.v = static_cast<const uint8_t*>(v);
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
    a.c = static_cast<float>(cd);
    a.vscale = v_descale;

    hipError_t err;
    if (n_eff == 1) {
        err = launch8_d<false>(a, d, causal, ng, stream);
    } else {
        err = launch8_d<true>(a, d, causal, ng, stream);
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

extern "C" fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal, float scale,
                                float q_descale, float k_descale, float v_descale, hipStream_t stream) {
    return run_fwd8(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, q_descale, k_descale, v_descale, 1, nullptr,
                    0, stream);
}

extern "C" fa_status fa_fwd_fp8_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                      int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal,
                                      float scale, float q_descale, float k_descale, float v_descale, int64_t n_split,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return run_fwd8(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, q_descale, k_descale, v_descale, n_split,
                    workspace, workspace_bytes, stream);
}
