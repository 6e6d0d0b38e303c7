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
// gfx950 mapping (one workgroup = 4 waves of 64 lanes, 128 query rows, 2
// workgroups per CU):
//   * Each wave owns 32 query rows and computes the TRANSPOSED score tile
//     S^T = K_j Q^T with v_mfma_f32_32x32x16_bf16: in the accumulator every lane
//     holds 32 scores of ONE query row (lane % 32), the other 32 keys of the
//     64-key tile sitting in lane ^ 32.  Row max and row sums are in-register
//     reductions plus one v_permlane32_swap.
//   * The output is accumulated transposed too, O^T += V_j^T P^T: its B operand
//     is the bf16-converted score accumulator as it stands (no LDS round trip
//     for P) and its accumulator again keeps one query row per lane, so a row's
//     rescale factor is lane-local.
//   * K_j and V_j are copied HBM -> LDS by buffer_load ... lds (no VGPR
//     staging), one 16-byte chunk per lane, into row-major tiles whose 16-byte
//     chunks are XOR-swizzled by row so that both the K operand reads
//     (ds_read_b128) and the transposed V operand reads (ds_read_b64_tr_b16,
//     which hands each lane 4 keys of one head-dim column) are free of bank
//     conflicts.  The buffer descriptor of each tile covers only the rows that
//     exist, so the ragged end of the sequence reads as zeros.
//   * Software pipeline per wave: while the exponentials of tile j run on the
//     VALU, the MFMAs of tile j+1's scores are already in flight, and the row
//     max of tile j+1 is taken while tile j's PV MFMAs run.  LDS holds two K and
//     two V tiles; tile j+2's K and tile j+1's V are fetched during iteration j.
//   * The softmax scale is folded into the exponent (one FMA per score, exp2 with
//     scale*log2(e)); a negative scale negates Q once instead.
//   * The max is tracked lazily: a row is rescaled only when its tile maximum
//     exceeds the running reference by more than 2^8 (in exp2 units), the
//     conditional rescale described for FlashAttention-4 on "FlashAttention and
//     Fused Kernels: Attention Without the n x n Matrix" ("Four generations").
//     Weights exp2(x - m) then stay at most 256, and the result is unchanged up
//     to rounding.  Two row sums are kept: the fp32 sum of the weights (for the
//     log-sum-exp) and the sum of their bf16 roundings, which are the weights
//     the PV product actually used (for O = o / l).
//   * Causal: key tiles past a wave's last query are skipped; only a wave's
//     last tile can cross its diagonal or the end of the sequence, and only that
//     tile runs the masked path.
//   * Workgroup order: the grid is remapped so that a contiguous range of the
//     work list lands on one XCD (workgroups are dealt round-robin over the 8
//     XCDs), keeping one head's K/V in that XCD's L2; within a head the heaviest
//     causal query tiles go first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <type_traits>

#include "fa.h"

namespace {

#define FA_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;        // query rows per workgroup
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kThreads = 256;   // 4 waves
constexpr int kXcds = 8;
constexpr double kLog2e = 1.4426950408889634;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;   // log2 units: rescale when the max grows by > 2^8
constexpr uint32_t kBufferFlags = 0x00020000u;   // gfx9 raw buffer descriptor word 3

// Waves of one workgroup per SIMD: 1 gives each wave the full 512-entry
// register file (VGPR + AGPR); 2 halves it and lets two workgroups share a CU.
#ifndef FA_WAVES_PER_EU
#define FA_WAVES_PER_EU 2
#endif
// 1: a wave keeps the next tile's scores in flight under the current softmax;
// 0: one score tile at a time (fewer registers; the other wave on the SIMD overlaps).
#ifndef FA_PIPELINE
#define FA_PIPELINE 0
#endif

template <int D>
struct Geo {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;            // 16-byte chunks per row
    static constexpr int kTileBytes = kBN * kRowBytes;
    static constexpr int kLoads = D / 32;             // 1 KB buffer->LDS loads per wave per tile
    static constexpr int kDSteps = D / 16;            // MFMA k-steps over d for S^T
    static constexpr int kDBlocks = D / 32;           // 32-row blocks of O^T
    static constexpr int kLdsBytes = 4 * kTileBytes;  // K slot 0, K slot 1, V slot 0, V slot 1
};

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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

template <int D>
struct WaveState {
    f32x16 o[Geo<D>::kDBlocks];   // O^T accumulator: lane holds d-rows of its query
    float m = -INFINITY;          // running reference max (exp2 units)
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
        for (int b = 0; b < Geo<D>::kDBlocks; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.o[b][i] *= r;
    }
}

// One workgroup's work; `lds` is the workgroup's Geo<D>::kLdsBytes of LDS.
template <int D, bool CAUSAL>
__device__ __forceinline__ void fa_fwd_block(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                             const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                             float* __restrict__ LSE, int T, int n_qt, int total, float c_in,
                                             FA_LDS char* const lds) {
    using G = Geo<D>;
    FA_LDS char* const kslot[2] = {lds, lds + G::kTileBytes};
    FA_LDS char* const vslot[2] = {lds + 2 * G::kTileBytes, lds + 3 * G::kTileBytes};

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;   // this lane's query row within the wave
    const int half = lane >> 5;

    // Work decode: XCD-contiguous remap, then (head, query tile), heavy tiles first.
    const int id = blockIdx.x;
    const int xcd = id % kXcds, xslot = id / kXcds;
    const int q8 = total / kXcds, r8 = total % kXcds;
    const int w = xcd < r8 ? xcd * (q8 + 1) + xslot : r8 * (q8 + 1) + (xcd - r8) * q8 + xslot;
    const int bh = w / n_qt;
    const int qt = CAUSAL ? n_qt - 1 - (w % n_qt) : (w % n_qt);

    const size_t base = (size_t)bh * (size_t)T * D;
    const uint16_t* __restrict__ kbh = K + base;
    const uint16_t* __restrict__ vbh = V + base;
    const uint32_t head_bytes = (uint32_t)T * G::kRowBytes;

    const int qw0 = qt * kBM + wave * 32;   // first query row of this wave
    const int qrow = qw0 + col;
    const int n_all = (T + kBN - 1) / kBN;
    const int kv_end = CAUSAL ? min(T, qt * kBM + kBM) : T;
    const int n_kt = (kv_end + kBN - 1) / kBN;                       // tiles the workgroup loads
    const int n_w = qw0 >= T ? 0 : (CAUSAL ? min(n_all, (qw0 + 31) / kBN + 1) : n_all);  // tiles this wave uses

    // Per-lane byte offsets of this lane's 16-byte chunk in each tile load, and
    // the matching LDS destination of the wave's 1 KB block.
    uint32_t goff[G::kLoads];
#pragma unroll
    for (int c = 0; c < G::kLoads; ++c) {
        const int q = (wave * G::kLoads + c) * 64 + lane;
        const int r = q / G::kChunks, p = q % G::kChunks;
        goff[c] = r * G::kRowBytes + 16 * (p ^ swz<D>(r));
    }
    auto load_tile = [&] __device__ (const uint16_t* src, int key0, FA_LDS char* slot) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (size_t)key0 * D, (uint32_t)(T - key0) * G::kRowBytes);
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

    // Start fetching: K_0, V_0, K_1.
    load_tile(kbh, 0, kslot[0]);
    load_tile(vbh, 0, vslot[0]);
#if FA_PIPELINE
    if (n_kt > 1) load_tile(kbh, kBN, kslot[1]);
#endif

    // Q^T operand (B operand of S^T): lane holds Q[qrow][16 s + 8 half .. +7]; zeros past T.
    bf16x8 qf[G::kDSteps];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + base, head_bytes);
        const uint32_t neg = c_in < 0.0f ? 0x80008000u : 0u;
#pragma unroll
        for (int s = 0; s < G::kDSteps; ++s) {
            u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)qrow * G::kRowBytes + 32 * s + 16 * half,
                                                              0, 0);
            raw ^= neg;
            qf[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    const float c = fabsf(c_in);

    WaveState<D> st;
#pragma unroll
    for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[b][i] = 0.0f;

    auto qk = [&] __device__ (FA_LDS const char* ks, f32x16 (&s)[2]) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[b][i] = 0.0f;
#pragma unroll
        for (int t = 0; t < G::kDSteps; ++t)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = *(FA_LDS const bf16x8*)(ks + kb * 32 * G::kRowBytes + koff[t]);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kb], 0, 0, 0);
            }
    };
    auto pv = [&] __device__ (FA_LDS const char* vs, const uint32_t (&pk)[16]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 praw = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, praw);
#pragma unroll
            for (int db = 0; db < G::kDBlocks; ++db) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (FA_LDS i16x4*)(vs + ks * 16 * G::kRowBytes + voff[db][0]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (FA_LDS i16x4*)(vs + ks * 16 * G::kRowBytes + voff[db][1]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 araw = {l2[0], l2[1], h2[0], h2[1]};
                st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, araw), pb, st.o[db],
                                                                    0, 0, 0);
            }
        }
    };
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile loads have landed
    __syncthreads();

    // Two score buffers: even steps turn sa into probabilities while sb fills, odd
    // steps the other way round (a static register renaming, no copies).
    f32x16 sa[2], sb[2];
#if FA_PIPELINE
    if (n_w > 0) {
        qk(kslot[0], sa);
        if (n_w > 1) st.m = tile_max(sa) * c;
    }
#endif

    // Tiles every wave of the workgroup treats as unmasked, with a successor:
    // wave 0 has the fewest tiles, and its last one is left to the tail.
    const int n_w0 = qt * kBM >= T ? 0 : (CAUSAL ? min(n_all, (qt * kBM + 31) / kBN + 1) : n_all);
    const int n_steady = max(0, n_w0 - 1);

    // Steady tile j (parity P): tile j+1's score MFMAs overlap tile j's
    // exponentials; tile j+1's max is taken while tile j's PV MFMAs run.
    auto steady = [&] __device__ (int j, auto parity, f32x16 (&sc)[2], f32x16 (&sn)[2], bool next_steady) {
        constexpr int P = decltype(parity)::value;   // j % 2
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();   // K_{j+1}, V_j landed; every wave is done with K_j and V_{j-1}
        if (j + 2 < n_kt) load_tile(kbh, (j + 2) * kBN, kslot[P]);
        if (j + 1 < n_kt) load_tile(vbh, (j + 1) * kBN, vslot[P ^ 1]);
        qk(kslot[P ^ 1], sn);
        uint32_t pk[16];
        const float mneg = -st.m;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const float x0 = n < 8 ? sc[0][2 * n] : sc[1][2 * n - 16];
            const float x1 = n < 8 ? sc[0][2 * n + 1] : sc[1][2 * n - 15];
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x0, c, mneg));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x1, c, mneg));
            st.l32 += p0;
            st.l32 += p1;
            pk[n] = pack_bf16x2(p0, p1);
        }
        pv(vslot[P], pk);
#pragma unroll
        for (int n = 0; n < 16; ++n)
            st.l16 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[n]), ones, st.l16, false);
        if (next_steady) maybe_rescale<D>(st, tile_max(sn) * c);
    };

    // Steady tile j without the in-wave pipeline: scores, max, weights, PV.
    auto steady_np = [&] __device__ (int j, auto parity, f32x16 (&sc)[2]) {
        constexpr int P = decltype(parity)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();   // K_j, V_j landed; every wave is done with K_{j-1}, V_{j-1}
        if (j + 1 < n_kt) {
            load_tile(kbh, (j + 1) * kBN, kslot[P ^ 1]);
            load_tile(vbh, (j + 1) * kBN, vslot[P ^ 1]);
        }
        qk(kslot[P], sc);
        maybe_rescale<D>(st, tile_max(sc) * c);
        uint32_t pk[16];
        const float mneg = -st.m;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const float x0 = n < 8 ? sc[0][2 * n] : sc[1][2 * n - 16];
            const float x1 = n < 8 ? sc[0][2 * n + 1] : sc[1][2 * n - 15];
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x0, c, mneg));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x1, c, mneg));
            st.l32 += p0;
            st.l32 += p1;
            pk[n] = pack_bf16x2(p0, p1);
            st.l16 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[n]), ones, st.l16, false);
        }
        pv(vslot[P], pk);
    };

    // A wave's last tile (parity P): mask keys past its diagonal or past T.
    auto last = [&] __device__ (int j, auto parity, f32x16 (&sc)[2]) {
        constexpr int P = decltype(parity)::value;
        const int key0 = j * kBN;
        float x[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                const bool vis = key < T && (!CAUSAL || key <= qrow);
                x[kb * 16 + i] = vis ? sc[kb][i] * c : -INFINITY;
            }
        float mt = x[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) mt = fmaxf(mt, x[i]);
        maybe_rescale<D>(st, fmaxf(st.m, xhalf_max(mt)));
        const float mu = st.m == -INFINITY ? 0.0f : st.m;
        uint32_t pk[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const float p0 = __builtin_amdgcn_exp2f(x[2 * n] - mu);
            const float p1 = __builtin_amdgcn_exp2f(x[2 * n + 1] - mu);
            st.l32 += p0;
            st.l32 += p1;
            pk[n] = pack_bf16x2(p0, p1);
            st.l16 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[n]), ones, st.l16, false);
        }
        pv(vslot[P], pk);
    };

    // Tail tile j (parity P): per-wave steady / last / idle, plus the loads.
    auto tail = [&] __device__ (int j, auto parity, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
        constexpr int P = decltype(parity)::value;
        if (j + 1 < n_w) {
            steady(j, parity, sc, sn, j + 2 < n_w);
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (j + 2 < n_kt) load_tile(kbh, (j + 2) * kBN, kslot[P]);
            if (j + 1 < n_kt) load_tile(vbh, (j + 1) * kBN, vslot[P ^ 1]);
            if (j + 1 == n_w) last(j, parity, sc);
        }
    };

    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
#if !FA_PIPELINE
    // Non-pipelined order: K_j and V_j share a stage; tile j+1 loads during tile j.
    auto tail_np = [&] __device__ (int j, auto parity, f32x16 (&sc)[2]) {
        constexpr int P = decltype(parity)::value;
        if (j + 1 < n_w) {
            steady_np(j, parity, sc);
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (j + 1 < n_kt) {
                load_tile(kbh, (j + 1) * kBN, kslot[P ^ 1]);
                load_tile(vbh, (j + 1) * kBN, vslot[P ^ 1]);
            }
            if (j + 1 == n_w) {
                qk(kslot[P], sc);
                last(j, parity, sc);
            }
        }
    };
    int j = 0;
    for (; j + 1 < n_steady; j += 2) {
        steady_np(j, Even{}, sa);
        steady_np(j + 1, Odd{}, sa);
    }
    for (; j < n_kt; j += 2) {
        if (j < n_steady) steady_np(j, Even{}, sa);
        else tail_np(j, Even{}, sa);
        if (j + 1 < n_kt) tail_np(j + 1, Odd{}, sa);
    }
#else
    int j = 0;
    for (; j + 1 < n_steady; j += 2) {
        steady(j, Even{}, sa, sb, true);
        steady(j + 1, Odd{}, sb, sa, true);
    }
    // Tiles n_steady_even .. n_kt-1: the odd leftover steady tile and the masked ends.
    for (; j < n_kt; j += 2) {
        if (j < n_steady) steady(j, Even{}, sa, sb, true);
        else tail(j, Even{}, sa, sb);
        if (j + 1 < n_kt) tail(j + 1, Odd{}, sb, sa);
    }
#endif

    // Epilogue: O = o / l (bf16, round to nearest even), lse = ln2 * (m + log2 l).
    const float l32 = xhalf_sum(st.l32);
    const float l16 = xhalf_sum(st.l16);
    if (n_w == 0) return;
    const float inv = 1.0f / l16;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + base, head_bytes);   // rows past T are dropped
    const uint32_t orow = (uint32_t)qrow * G::kRowBytes;
#pragma unroll
    for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 wv;
            wv.x = pack_bf16x2(st.o[b][4 * g + 0] * inv, st.o[b][4 * g + 1] * inv);
            wv.y = pack_bf16x2(st.o[b][4 * g + 2] * inv, st.o[b][4 * g + 3] * inv);
            __builtin_amdgcn_raw_buffer_store_b64(wv, ro, orow + 2 * (b * 32 + 8 * g + 4 * half), 0, 0);
        }
    if (half == 0) {
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(LSE + (size_t)bh * T, (uint32_t)T * 4u);
        __builtin_amdgcn_raw_buffer_store_b32(as_u32(kLn2 * (st.m + __builtin_amdgcn_logf(l32))), rl,
                                              (uint32_t)qrow * 4u, 0, 0);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(FA_WAVES_PER_EU, FA_WAVES_PER_EU)))
void fa_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                   int T, int n_qt, int total, float c_in /* scale * log2(e) */) {
    __shared__ __attribute__((aligned(1024))) char smem[Geo<D>::kLdsBytes];
    fa_fwd_block<D, CAUSAL>(Q, K, V, O, LSE, T, n_qt, total, c_in, (FA_LDS char*)smem);
}

thread_local char g_hip_error[256] = "";

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int T, int n_qt, int total,
                  float c, hipStream_t stream) {
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), dim3(total), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, T, n_qt, total, c);
    return hipGetLastError();
}

}  // namespace

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                            int64_t H, int64_t T, int64_t d, int causal, float scale, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || T < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (!std::isfinite(scale)) return FA_ERR_SCALE;
    const auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if ((addr(q) | addr(k) | addr(v) | addr(o)) & 15u) return FA_ERR_ALIGN;
    if (addr(lse) & 3u) return FA_ERR_ALIGN;

    // Sizes: every byte count must fit int64; in-kernel row indices are 32-bit.
    const int64_t kMax = INT64_MAX;
    if (B > kMax / H) return FA_ERR_OVERFLOW;
    const int64_t BH = B * H;
    if (BH > kMax / T) return FA_ERR_OVERFLOW;
    const int64_t rows = BH * T;
    if (rows > kMax / (2 * d)) return FA_ERR_OVERFLOW;
    if (T > INT32_MAX - 2 * kBM) return FA_ERR_OVERFLOW;
    // Buffer descriptors address one head: (T + 2 query tiles) rows must fit in 32-bit byte offsets.
    if ((T + 2 * kBM) * 2 * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;
    const int64_t n_qt = (T + kBM - 1) / kBM;
    if (BH > INT32_MAX / n_qt) return FA_ERR_OVERFLOW;
    const int total = static_cast<int>(BH * n_qt);

    const size_t tensor_bytes = static_cast<size_t>(rows) * static_cast<size_t>(d) * 2u;
    const size_t lse_bytes = static_cast<size_t>(rows) * 4u;
    for (const void* in : {q, k, v}) {
        if (overlaps(o, tensor_bytes, in, tensor_bytes)) return FA_ERR_ARG;
        if (overlaps(lse, lse_bytes, in, tensor_bytes)) return FA_ERR_ARG;
    }
    if (overlaps(o, tensor_bytes, lse, lse_bytes)) return FA_ERR_ARG;

    const float c = static_cast<float>(static_cast<double>(scale) * kLog2e);
    hipError_t err;
    const int Ti = static_cast<int>(T), nq = static_cast<int>(n_qt);
    if (d == 128)
        err = causal ? launch<128, true>(q, k, v, o, lse, Ti, nq, total, c, stream)
                     : launch<128, false>(q, k, v, o, lse, Ti, nq, total, c, stream);
    else
        err = causal ? launch<64, true>(q, k, v, o, lse, Ti, nq, total, c, stream)
                     : launch<64, false>(q, k, v, o, lse, Ti, nq, total, c, stream);
    if (err != hipSuccess) {
        std::snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", hipGetErrorName(err), hipGetErrorString(err));
        return FA_ERR_HIP;
    }
    g_hip_error[0] = '\0';
    return FA_OK;
}

extern "C" const char* fa_status_string(fa_status status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "B, H and T must all be >= 1";
        case FA_ERR_HEAD_DIM: return "head size d must be 64 or 128";
        case FA_ERR_SCALE: return "scale must be finite";
        case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case FA_ERR_OVERFLOW: return "sizes overflow the supported index range";
        case FA_ERR_HIP: return "HIP kernel launch failed";
        case FA_ERR_ARG: return "causal must be 0 or 1, and outputs must not overlap inputs";
    }
    return "unknown status";
}

extern "C" const char* fa_hip_error_string(void) { return g_hip_error; }
