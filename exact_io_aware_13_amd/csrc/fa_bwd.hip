// fa_bwd.hip -- exact attention backward for MI355X (gfx950, CDNA4), and its C ABI.
//
// The method: the training backward that keeps only O and the per-row
// statistics from the forward and recomputes the score and probability tiles
// ("FlashAttention and Fused Kernels: Attention Without the n x n Matrix",
// "Training: recompute instead of store"; "Flash Attention, tiled: exact
// attention without the T x T HBM matrix", "More arithmetic can still be
// faster").  With s = scale * q.k, P_ij = exp(s_ij - lse_i) (the forward's row
// log-sum-exp gives the softmax row directly, no running max), dP = dO V^T,
// D_i = sum_j P_ij dP_ij = dO_i . O_i and dS = P * (dP - D):
//     dV = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K.
// The T x T tiles S, P, dP, dS exist only in registers, tile by tile.
//
// gfx950 mapping: three launches on the caller's stream, none with atomics, so
// the gradients are bit-reproducible.
//   * prep: D_i = dO_i . O_i (fp32 from the bf16 O the forward wrote) and
//     lse_i * log2(e), one pass over O and dO into the workspace.
//   * dK/dV kernel, key-major: a workgroup of 8 waves owns 128 keys of one
//     key/value head.  The two waves of a SIMD take the same 32 keys and split
//     the work: one holds K and computes S = Q K^T, P and dV^T += dO^T P, the
//     other holds V and computes dP = dO V^T, dS = P (dP - D) and
//     dK^T += Q^T dS, with P passed through LDS.  It walks the 32-row query
//     tiles (every query head of the group) that see its keys, copying Q, dO,
//     lse and D tiles HBM -> LDS (buffer_load ... lds, a ring of four slots).
//     S and dP are computed with the keys on the lanes
//     (v_mfma_f32_32x32x16_bf16; each lane holds 32 query rows of ONE key), so
//     the bf16 P and dS accumulators are directly the B operands of the dV and
//     dK products, whose A operands are transposed LDS reads
//     (ds_read_b64_tr_b16) of the same dO and Q tiles.  The two waves of a
//     SIMD are phase-shifted by software pipelining, so that one's
//     exponentials overlap the other's matrix products.
//   * dQ kernel, query-major: the forward's shape.  A workgroup of 4 waves
//     owns 128 query rows, each lane one row, with Q and dO held in registers;
//     it streams 64-key K and V tiles through LDS, computes S^T = K Q^T and
//     dP^T = V dO^T with the queries on the lanes, and accumulates
//     dQ^T += K^T dS^T with the bf16 dS^T accumulator as the B operand and
//     transposed K reads as the A operand.
//   The dQ products are recomputed in the second kernel instead of being
//   summed across key-major workgroups with atomics: 7 instead of 5 matrix
//   products per tile pair, no fp32 atomic traffic, a deterministic result.
//   * Tiles in LDS are row-major with 16-byte chunks XOR-swizzled by row, so
//     that the row reads (ds_read_b128) and the transposed reads are free of
//     bank conflicts; buffer descriptors end at the last existing row, so
//     ragged tails read as zeros.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <type_traits>

#include "fa.h"
#include "fa_internal.h"

namespace {

#define FB_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 64;        // rows per LDS tile: query rows (dK/dV kernel) or keys (dQ kernel)
constexpr int kKeysPerWg = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int kQueriesPerWg = 128;   // query rows per dQ workgroup (32 per wave)
constexpr int kXcds = 8;
constexpr double kLog2e = 1.4426950408889634;
constexpr uint32_t kBufferFlags = 0x00020000u;   // gfx9 raw buffer descriptor word 3

template <int D>
struct BGeo {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;              // 16-byte chunks per row
    static constexpr int kTileBytes = kRows * kRowBytes;
    static constexpr int kLoads = kTileBytes / 1024 / 4;   // 1 KB buffer->LDS loads per wave per tile
    static constexpr int kDSteps = D / 16;              // MFMA k-steps over d
    static constexpr int kDBlocks = D / 32;             // 32-row blocks over d
};

// XOR swizzle of the 16-byte chunk index within a tile row (see the header
// comment): it depends only on row % 16, so 32- and 16-row offsets keep it.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 r = {a, b, c, d};
    return __builtin_bit_cast(bf16x8, r);
}

// Per-lane LDS offsets into a 64-row tile.
//   row(s):   the row-read operand: row `col` (+ 32 per row block), d-chunk 2 s + half.
//   tr(db,e): the transposed operand: in 16-lane group g, lane i fetches four
//             d-values of row 8 e + 4 half + i / 4 (+ 16 per step) at column
//             32 db + 16 (g % 2) + 4 (i % 4); after the transpose, lane l holds
//             column 32 db + l % 32 at rows {4 half .. 4 half + 3} (e = 0) and
//             {8 + 4 half .. 8 + 4 half + 3} (e = 1) of the step, the k order of
//             the rows an accumulator's elements 0-7 (or 8-15) hold.
template <int D>
struct TileOffsets {
    uint32_t row[BGeo<D>::kDSteps];
    uint32_t tr[BGeo<D>::kDBlocks][2];
    __device__ __forceinline__ TileOffsets(int lane) {
        using G = BGeo<D>;
        const int col = lane & 31, half = lane >> 5;
#pragma unroll
        for (int s = 0; s < G::kDSteps; ++s) row[s] = col * G::kRowBytes + 16 * ((2 * s + half) ^ swz<D>(col));
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = 8 * e + 4 * half + (i >> 2);
                const int cc = 32 * db + 16 * (g & 1) + 4 * (i & 3);
                tr[db][e] = r * G::kRowBytes + 16 * ((cc >> 3) ^ swz<D>(r)) + 2 * (cc & 7);
            }
    }
};

// Row operand: rows 32 rb + lane % 32 of the tile, d-values 16 s + 8 half .. + 7.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(FB_LDS const char* t, const TileOffsets<D>& off, int rb, int s) {
    return *(FB_LDS const bf16x8*)(t + rb * 32 * BGeo<D>::kRowBytes + off.row[s]);
}

// Transposed operand for 16-row step ks (rows 16 ks ..) and d-block db.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(FB_LDS const char* t, const TileOffsets<D>& off, int ks, int db) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (FB_LDS i16x4*)(t + ks * 16 * BGeo<D>::kRowBytes + off.tr[db][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (FB_LDS i16x4*)(t + ks * 16 * BGeo<D>::kRowBytes + off.tr[db][1]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return as_bf16x8(l2[0], l2[1], h2[0], h2[1]);
}

// Work-list index of this workgroup: contiguous ranges of the list go to one
// XCD (the hardware deals workgroups round-robin over the 8 XCDs), so the
// workgroups of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
    const int xcd = id % kXcds, xslot = id / kXcds;
    const int q8 = total / kXcds, r8 = total % kXcds;
    return xcd < r8 ? xcd * (q8 + 1) + xslot : r8 * (q8 + 1) + (xcd - r8) * q8 + xslot;
}

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    const float* lse2;   // [B * hq * tq] lse * log2(e)
    const float* dd;     // [B * hq * tq] D_i
    int tq, tk, hq, group;
    int n_kt;            // key workgroups per key/value head (dK/dV kernel)
    int n_qt;            // query workgroups per query head (dQ kernel)
    int total;           // workgroups of the launch
    float c;             // scale * log2(e)
    float scale;
};

// ---------------------------------------------------------------------------
// prep: D_i = sum_c dO[i][c] * O[i][c] and lse_i * log2(e); D / 8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                          const uint16_t* __restrict__ dout,
                                                          const float* __restrict__ lse, float* __restrict__ lse2,
                                                          float* __restrict__ dd, long long rows) {
    constexpr int kLanes = D / 8;
    const long long row = (long long)blockIdx.x * (256 / kLanes) + threadIdx.x / kLanes;
    const int t = threadIdx.x % kLanes;
    float acc = 0.0f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + (size_t)row * D + 8 * t);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dout + (size_t)row * D + 8 * t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(as_f32(a[e] << 16), as_f32(b[e] << 16), acc);
            acc = __builtin_fmaf(as_f32(a[e] & 0xFFFF0000u), as_f32(b[e] & 0xFFFF0000u), acc);
        }
    }
#pragma unroll
    for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (row < rows && t == 0) {
        dd[row] = acc;
        lse2[row] = lse[row] * (float)kLog2e;
    }
}

// ---------------------------------------------------------------------------
// dK/dV kernel.  A workgroup of 8 waves owns 128 keys.  Waves w and w + 4
// share SIMD w % 4 and the same 32 keys: wave w (the "P wave") holds K and
// computes S = Q K^T, P and dV^T += dO^T P; wave w + 4 (the "dS wave") holds
// V and computes dP = dO V^T, dS = P (dP - D) and dK^T += Q^T dS, taking P
// from LDS.  Each wave holds one of K, V and one of dK, dV (about 150
// registers), so two waves fit a SIMD.  Query tiles of 32 rows; each tile is
// two phases, and in each phase one wave of a SIMD does VALU work while the
// other keeps the matrix unit busy:
//   phase A(i):  P wave:  P(i) from S(i) (to LDS and to bf16)
//                dS wave: dP(i) = dO_i V^T, then dK^T += Q_{i-1}^T dS(i-1)
//   phase B(i):  P wave:  dV^T += dO_i^T P(i), then S(i+1) = Q_{i+1} K^T
//                dS wave: dS(i) = P(i) (dP(i) - D)
// LDS: a ring of tile slots (Q, dO, lse2, D) and the P exchange area (4 KB
// per wave pair and 32-row block).  A tile is in use from phase B of the tile
// before it to phase A of the tile after it; it is fetched into the slot of
// the tile before that as soon as that one is done, at least a tile ahead.
// 32-row tiles: 64-row tiles (three slots) measured the same at d = 128 and
// slower at d = 64.
constexpr int kQRows = 32;                     // query rows per dK/dV tile
constexpr int kRB = kQRows / 32;               // 32-row blocks per tile
constexpr int kRing = kQRows == 32 ? 4 : 3;    // tile slots
template <int D>
struct KvLds {
    static constexpr int kTile = kQRows * 2 * D;
    static constexpr int kSlot = 2 * kTile;                 // Q tile, then dO tile
    static constexpr int kStats = kRing * kSlot;            // per slot: 64 lse2, then 64 D (one copy each)
    static constexpr int kPad = kStats + kRing * 512;       // 6 waves x 256 B of dummy copies
    static constexpr int kX = kPad + 6 * 256;               // P exchange: [pair][row block][4][64 lanes][16 B]
    static constexpr int kBytes = kX + 4 * 4096 * kRB;
    static constexpr int kBlocks = kTile / 1024;            // 1 KB blocks per tile of one tensor
    static constexpr int kLoads = 2 * kBlocks / 8;          // 1 KB copies per wave per tile (Q, then dO)
};

template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_block(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V, const uint16_t* __restrict__ DO,
                                           const float* __restrict__ LSE2, const float* __restrict__ DD,
                                           uint16_t* __restrict__ DK, uint16_t* __restrict__ DV, const BwdArgs& a,
                                           FB_LDS char* const lds) {
    using G = BGeo<D>;
    using L = KvLds<D>;
    const int Tq = a.tq, Tk = a.tk;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = wave & 3;
    const bool pwave = wave < 4;   // wave-uniform role
    const int half = lane >> 5;

    // Work decode: (key/value head, key tile), key tiles of a head in order,
    // which for causal work is heaviest first.
    const int w = xcd_remap(blockIdx.x, a.total);
    const int bkv = w / a.n_kt;
    const int kt = w % a.n_kt;
    const int hkv = a.hq / a.group;
    const int b = bkv / hkv, hk = bkv % hkv;
    const int kw0 = kt * kKeysPerWg;      // first key of the workgroup
    const int k0 = kw0 + 32 * pair;       // first key of this wave pair
    const int key = k0 + (lane & 31);     // this lane's key
    const int off = Tk - Tq;              // causal: query i sees keys j <= i + off

    const size_t kvbase = (size_t)bkv * (size_t)Tk * D;
    // The wave's K (P wave) or V (dS wave) rows as B operands: lane holds row
    // `key`, d-values 16 s + 8 half .. + 7; zeros past Tk.
    bf16x8 bf[G::kDSteps];
    {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc((pwave ? K : V) + kvbase, (uint32_t)Tk * G::kRowBytes);
#pragma unroll
        for (int s = 0; s < G::kDSteps; ++s)
            bf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rb, (uint32_t)key * G::kRowBytes + 32 * s + 16 * half, 0, 0));
    }

    // Query tiles that see some key of the workgroup, for every query head of
    // the group.  A tile that a wave pair's keys reach only partly (or not at
    // all: then every weight is masked) is one of the first few of each head.
    const int n_q = (Tq + kQRows - 1) / kQRows;
    const int qt0 = CAUSAL ? max(0, kw0 - off) / kQRows : 0;
    const int per_head = n_q - qt0;
    const int n_it = per_head * a.group;
    // Tiles t < t_mask of each head hold a row that must not see some key of this pair.
    const int t_mask = CAUSAL ? max(0, (k0 + 31 - off + kQRows - 1) / kQRows - qt0) : 0;

    // Buffer->LDS copies: the Q tile's and then the dO tile's 1 KB blocks are
    // dealt to the 8 waves; this lane copies one 16-byte chunk of each.  Each
    // wave issues kLoads + 1 copies per tile (waves 0, 1: lse2, D; the others
    // a dummy), so that a tile's copies are one fixed count in every wave.
    constexpr int kPerTile = L::kLoads + 1;
    uint32_t goff[L::kLoads];
    int gdst[L::kLoads];
    bool gdo[L::kLoads];
#pragma unroll
    for (int c = 0; c < L::kLoads; ++c) {
        const int j = wave * L::kLoads + c;
        gdo[c] = j >= L::kBlocks;
        const int jb = j % L::kBlocks;
        const int qd = jb * 64 + lane;
        const int r = qd / G::kChunks, p = qd % G::kChunks;
        goff[c] = r * G::kRowBytes + 16 * (p ^ swz<D>(r));
        gdst[c] = jb * 1024;
    }
    auto slot_of = [&] __device__ (int it) { return kRing == 4 ? (it & 3) : it % kRing; };
    auto load = [&] __device__ (int it) {
        const int k = slot_of(it);
        const int h = hk * a.group + it / per_head;
        const int q0 = (qt0 + it % per_head) * kQRows;
        const size_t row0 = ((size_t)b * a.hq + h) * (size_t)Tq + q0;
        const uint32_t bytes = (uint32_t)(Tq - q0) * G::kRowBytes;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + row0 * D, bytes);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(DO + row0 * D, bytes);
#pragma unroll
        for (int c = 0; c < L::kLoads; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(gdo[c] ? rd : rq,
                                                     (FB_LDS void*)(lds + k * L::kSlot + (gdo[c] ? L::kTile : 0) + gdst[c]),
                                                     16, goff[c], 0, 0, 0);
        // lse2 (wave 0) and D (wave 1) of the tile's rows; 64 values per copy.
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((wave == 1 ? DD : LSE2) + row0, (uint32_t)(Tq - q0) * 4u);
        const int dst = wave == 0 ? L::kStats + k * 512 : wave == 1 ? L::kStats + k * 512 + 256 : L::kPad + 256 * (wave - 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FB_LDS void*)(lds + dst), 4, (uint32_t)lane * 4u, 0, 0, 0);
    };

    const TileOffsets<D> to(lane);
    f32x16 acc[G::kDBlocks];   // dV^T (P wave) or dK^T (dS wave): lane holds d-rows of its key
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
    const float c = a.c;
    FB_LDS char* const xp = lds + L::kX + pair * 4096 * kRB + lane * 16;   // this lane's P exchange slots

    // S = Q K^T (P wave) or dP = dO V^T (dS wave) of the tile in slot k.
    auto product = [&] __device__ (int k, f32x16 (&r)[kRB]) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i) r[rb][i] = 0.0f;
        FB_LDS const char* const src = lds + k * L::kSlot + (pwave ? 0 : L::kTile);
        constexpr int N = G::kDSteps * kRB;
        bf16x8 op[N];
#pragma unroll
        for (int i = 0; i < N; ++i) op[i] = row_operand<D>(src, to, i % kRB, i / kRB);
#pragma unroll
        for (int i = 0; i < N; ++i)
            r[i % kRB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], bf[i / kRB], r[i % kRB], 0, 0, 0);
        // Keep kAhead operand reads in flight ahead of the MFMA that uses them.
        constexpr int kAhead = 3 < N ? 3 : N;
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int i = 0; i < N - kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    };
    // acc += A^T B over a tile's query rows (steps of 16): A = dO (P wave) or
    // Q (dS wave) of slot k read transposed, B = the bf16 weights.
    auto accumulate = [&] __device__ (int k, const uint32_t (&wb)[8 * kRB]) {
        FB_LDS const char* const src = lds + k * L::kSlot + (pwave ? L::kTile : 0);
        constexpr int N = 2 * kRB * G::kDBlocks;
        bf16x8 op[N];
#pragma unroll
        for (int i = 0; i < N; ++i) op[i] = tr_operand<D>(src, to, i / G::kDBlocks, i % G::kDBlocks);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int ks = i / G::kDBlocks, db = i % G::kDBlocks;
            const bf16x8 bb = as_bf16x8(wb[4 * ks], wb[4 * ks + 1], wb[4 * ks + 2], wb[4 * ks + 3]);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], bb, acc[db], 0, 0, 0);
        }
        // Each operand is two transposed reads; keep kAhead operands in flight.
        constexpr int kAhead = 3 < N ? 3 : N;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
        for (int i = 0; i < N - kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    };

    // Each role runs its own loop over the tiles; both loops pass the same
    // barriers in the same order (two per tile).  Element i of 32-row block rb
    // is query row q0 + 32 rb + 8 (i / 4) + 4 half + i % 4 of key `key`.
    auto phase_b_start = [&] __device__ (int it) {
        // Tile it + 1 has landed (with four slots, tile it + 2 may still be in flight).
        if (kRing == 4 && it + 2 < n_it) __builtin_amdgcn_s_waitcnt(0x0F70 | kPerTile);   // vmcnt(kPerTile)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                                          // vmcnt(0)
        __syncthreads();
        if (it + kRing - 1 < n_it) load(it + kRing - 1);   // into tile it - 1's slot
    };

    // The last slot's Q tile is read (with zero weights) by the dS waves'
    // first, empty dK step before any tile lands there: clear it, so that the
    // product is exactly zero.
#pragma unroll
    for (int z0 = 0; z0 < L::kTile; z0 += 8 * 1024)
        if (z0 + wave * 1024 < L::kTile) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            *(FB_LDS u32x4*)(lds + (kRing - 1) * L::kSlot + z0 + wave * 1024 + lane * 16) = z;
        }
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j)
        if (j < n_it) load(j);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (pwave) {
        // Phase A: P (to LDS and bf16); phase B: dV^T += dO^T P, then the next
        // tile's S (after the last tile: a dummy on stale LDS data, never used).
        f32x16 s_next[kRB];
        product(0, s_next);
        for (int it = 0; it < n_it; ++it) {
            const int k = slot_of(it);
            const int t = it % per_head;
            const int q0 = (qt0 + t) * kQRows;
            __syncthreads();
            const bool masked = CAUSAL && t < t_mask;
            FB_LDS const char* const lse_t = lds + L::kStats + k * 512;
            uint32_t pb[8 * kRB];
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                const int vis0 = q0 + 32 * rb + off + 4 * half - key;   // element visible iff vis0 + 8 g + e >= 0
                float p[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 l4 = *(FB_LDS const f32x4*)(lse_t + 4 * (32 * rb + 8 * g + 4 * half));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s_next[rb][4 * g + e], c, -l4[e]));
                        p[4 * g + e] = masked && vis0 < -(8 * g + e) ? 0.0f : pv;
                    }
                    const f32x4 pw = {p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
                    *(FB_LDS f32x4*)(xp + rb * 4096 + g * 1024) = pw;
                }
#pragma unroll
                for (int n = 0; n < 8; ++n) pb[8 * rb + n] = pack_bf16x2(p[2 * n], p[2 * n + 1]);
            }
            phase_b_start(it);
            accumulate(k, pb);
            product(slot_of(it + 1), s_next);
        }
    } else {
        // Phase A: dP, then dK^T += Q^T dS of the previous tile; phase B:
        // dS = P (dP - D).
        uint32_t ds_prev[8 * kRB];
#pragma unroll
        for (int n = 0; n < 8 * kRB; ++n) ds_prev[n] = 0u;
        for (int it = 0; it < n_it; ++it) {
            const int k = slot_of(it);
            __syncthreads();
            f32x16 dp[kRB];
            product(k, dp);
            accumulate(slot_of(it + kRing - 1), ds_prev);   // first tile: zero weights on a zeroed tile
            phase_b_start(it);
            FB_LDS const char* const d_t = lds + L::kStats + k * 512 + 256;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                float ds[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 p4 = *(FB_LDS const f32x4*)(xp + rb * 4096 + g * 1024);
                    const f32x4 d4 = *(FB_LDS const f32x4*)(d_t + 4 * (32 * rb + 8 * g + 4 * half));
#pragma unroll
                    for (int e = 0; e < 4; ++e) ds[4 * g + e] = p4[e] * (dp[rb][4 * g + e] - d4[e]);
                }
#pragma unroll
                for (int n = 0; n < 8; ++n) ds_prev[8 * rb + n] = pack_bf16x2(ds[2 * n], ds[2 * n + 1]);
            }
        }
        // The last tile's dK^T += Q^T dS (its Q tile is still in place).
        if (n_it > 0) accumulate(slot_of(n_it - 1), ds_prev);
    }

    // dV = dV^T (P wave), dK = scale * dK^T (dS wave), bf16; rows past Tk dropped by the descriptor.
    if (k0 >= Tk) return;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((pwave ? DV : DK) + kvbase, (uint32_t)Tk * G::kRowBytes);
    const uint32_t orow = (uint32_t)key * G::kRowBytes;
    const float sc = pwave ? 1.0f : a.scale;
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 wv;
            wv.x = pack_bf16x2(acc[db][4 * g + 0] * sc, acc[db][4 * g + 1] * sc);
            wv.y = pack_bf16x2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
            __builtin_amdgcn_raw_buffer_store_b64(wv, ro, orow + 2 * (db * 32 + 8 * g + 4 * half), 0, 0);
        }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void fa_bwd_dkdv_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[KvLds<D>::kBytes];
    dkdv_block<D, CAUSAL>(a.q, a.k, a.v, a.dout, a.lse2, a.dd, a.dk, a.dv, a, (FB_LDS char*)smem);
}

// ---------------------------------------------------------------------------
// dQ kernel.  LDS per slot: K tile, V tile.
// Operand reads the dQ kernel keeps in flight ahead of the MFMAs (3-6 measured alike).
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_block(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                         const uint16_t* __restrict__ V, const uint16_t* __restrict__ DO,
                                         const float* __restrict__ LSE2, const float* __restrict__ DD,
                                         uint16_t* __restrict__ DQ, const BwdArgs& a, FB_LDS char* const lds) {
    using G = BGeo<D>;
    const int Tq = a.tq, Tk = a.tk, n_qt = a.n_qt;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, half = lane >> 5;

    // Work decode: (head, query tile), heaviest causal tiles of a head first.
    const int w = xcd_remap(blockIdx.x, a.total);
    const int bh = w / n_qt;
    const int qt = CAUSAL ? n_qt - 1 - (w % n_qt) : (w % n_qt);
    const int kvh = (bh / a.hq) * (a.hq / a.group) + (bh % a.hq) / a.group;
    const size_t qbase = (size_t)bh * (size_t)Tq * D;
    const size_t kvbase = (size_t)kvh * (size_t)Tk * D;
    const uint16_t* __restrict__ kbh = K + kvbase;
    const uint16_t* __restrict__ vbh = V + kvbase;

    const int qw0 = qt * kQueriesPerWg + 32 * wave;   // first query row of this wave
    const int qrow = qw0 + col;
    const int off = Tk - Tq;
    const int kv_end = CAUSAL ? min(Tk, min(Tq, qt * kQueriesPerWg + kQueriesPerWg) + off) : Tk;
    const int n_kt = (kv_end + kRows - 1) / kRows;                 // tiles the workgroup loads
    const int w_end = CAUSAL ? min(Tk, qw0 + 32 + off) : Tk;        // keys this wave may see
    const int n_w = qw0 >= Tq ? 0 : (w_end + kRows - 1) / kRows;     // tiles it uses
    // Tiles from j_mask on can hold keys some row of the wave must not see.
    const int j_mask = CAUSAL ? min(n_w - 1, max(0, (qw0 + off + 1) / kRows)) : n_w - 1;

    uint32_t goff[G::kLoads];
#pragma unroll
    for (int c = 0; c < G::kLoads; ++c) {
        const int qd = (wave * G::kLoads + c) * 64 + lane;
        const int r = qd / G::kChunks, p = qd % G::kChunks;
        goff[c] = r * G::kRowBytes + 16 * (p ^ swz<D>(r));
    }
    auto load = [&] __device__ (int j, FB_LDS char* slot) {
        const int key0 = j * kRows;
        const uint32_t bytes = (uint32_t)(Tk - key0) * G::kRowBytes;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbh + (size_t)key0 * D, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbh + (size_t)key0 * D, bytes);
#pragma unroll
        for (int c = 0; c < G::kLoads; ++c) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FB_LDS void*)(slot + (wave * G::kLoads + c) * 1024), 16,
                                                     goff[c], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (FB_LDS void*)(slot + G::kTileBytes + (wave * G::kLoads + c) * 1024), 16, goff[c], 0, 0, 0);
        }
    };
    if (n_kt > 0) load(0, lds);

    // Q and dO rows as B operands; lse2 and D of the lane's row.
    bf16x8 qf[G::kDSteps], df[G::kDSteps];
    float lse2 = 0.0f, dd = 0.0f;
    {
        const uint32_t qb = (uint32_t)Tq * G::kRowBytes;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qbase, qb);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(DO + qbase, qb);
#pragma unroll
        for (int s = 0; s < G::kDSteps; ++s) {
            const uint32_t o = (uint32_t)qrow * G::kRowBytes + 32 * s + 16 * half;
            qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0));
            df[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rd, o, 0, 0));
        }
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(LSE2 + (size_t)bh * Tq, (uint32_t)Tq * 4u);
        const __amdgpu_buffer_rsrc_t rdd = make_rsrc(DD + (size_t)bh * Tq, (uint32_t)Tq * 4u);
        lse2 = as_f32(__builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)qrow * 4u, 0, 0));
        dd = as_f32(__builtin_amdgcn_raw_buffer_load_b32(rdd, (uint32_t)qrow * 4u, 0, 0));
    }

    const TileOffsets<D> to(lane);
    f32x16 dqa[G::kDBlocks];   // dQ^T: lane holds d-rows of its query row
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqa[db][i] = 0.0f;
    const float c = a.c;

    auto compute = [&] __device__ (int j, FB_LDS const char* slot) {
        if (j >= n_w) return;
        FB_LDS const char* ks = slot;
        FB_LDS const char* vs = slot + G::kTileBytes;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[kb][i] = 0.0f;
                dp[kb][i] = 0.0f;
            }
        // S^T = K Q^T and dP^T = V dO^T, the K and V operand reads interleaved
        // and kAhead of them kept in flight ahead of the MFMA that uses them.
        {
            constexpr int N = 4 * G::kDSteps;   // operands: (step, key block, K or V)
            bf16x8 op[N];
#pragma unroll
            for (int i = 0; i < N; ++i)
                op[i] = row_operand<D>((i & 1) ? vs : ks, to, (i >> 1) & 1, i >> 2);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int kb = (i >> 1) & 1, st = i >> 2;
                if (i & 1) dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], df[st], dp[kb], 0, 0, 0);
                else s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], qf[st], s[kb], 0, 0, 0);
            }
            constexpr int kAhead = 4 < N ? 4 : N;   // operand reads in flight
            __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
            for (int i = 0; i < N - kAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
        }
        // Element i of key block kb is key 64 j + 32 kb + 8 (i / 4) + 4 half + i % 4.
        // Exponent arguments first; only a wave's last tiles can hold keys a row
        // must not see, and there they are set to -inf (P = 0) in place.
        float x[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) x[kb][i] = __builtin_fmaf(s[kb][i], c, -lse2);
        if (j >= j_mask) {
            const int key0 = j * kRows;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kj = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool vis = kj < Tk && (!CAUSAL || kj <= qrow + off);
                    x[kb][i] = vis ? x[kb][i] : -INFINITY;
                }
        }
        uint32_t dsp[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float dsv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) dsv[i] = __builtin_amdgcn_exp2f(x[kb][i]) * (dp[kb][i] - dd);
#pragma unroll
            for (int n = 0; n < 8; ++n) dsp[kb][n] = pack_bf16x2(dsv[2 * n], dsv[2 * n + 1]);
        }
        // dQ^T += K^T dS^T over the tile's 64 keys (4 steps of 16); each operand
        // is two transposed reads, kAhead operands kept in flight.
        {
            constexpr int N = 4 * G::kDBlocks;
            bf16x8 op[N];
#pragma unroll
            for (int i = 0; i < N; ++i) op[i] = tr_operand<D>(ks, to, i / G::kDBlocks, i % G::kDBlocks);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int st = i / G::kDBlocks, db = i % G::kDBlocks;
                const int kb = st >> 1, h8 = 4 * (st & 1);
                const bf16x8 sb = as_bf16x8(dsp[kb][h8], dsp[kb][h8 + 1], dsp[kb][h8 + 2], dsp[kb][h8 + 3]);
                dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], sb, dqa[db], 0, 0, 0);
            }
            constexpr int kAhead = 4 < N ? 4 : N;   // operand reads in flight
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
            for (int i = 0; i < N - kAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
        }
    };

    constexpr int kSlot = 2 * G::kTileBytes;
    FB_LDS char* const slot0 = lds;
    FB_LDS char* const slot1 = lds + kSlot;
    for (int j = 0; j < n_kt; j += 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (j + 1 < n_kt) load(j + 1, slot1);
        compute(j, slot0);
        if (j + 1 >= n_kt) break;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (j + 2 < n_kt) load(j + 2, slot0);
        compute(j + 1, slot1);
    }

    if (n_w == 0) return;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(DQ + qbase, (uint32_t)Tq * G::kRowBytes);   // rows past Tq dropped
    const uint32_t orow = (uint32_t)qrow * G::kRowBytes;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 wv;
            wv.x = pack_bf16x2(dqa[db][4 * g + 0] * sc, dqa[db][4 * g + 1] * sc);
            wv.y = pack_bf16x2(dqa[db][4 * g + 2] * sc, dqa[db][4 * g + 3] * sc);
            __builtin_amdgcn_raw_buffer_store_b64(wv, ro, orow + 2 * (db * 32 + 8 * g + 4 * half), 0, 0);
        }
}

// Two workgroups per CU (two waves per SIMD).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dq_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[4 * BGeo<D>::kTileBytes];
    dq_block<D, CAUSAL>(a.q, a.k, a.v, a.dout, a.lse2, a.dd, a.dq, a, (FB_LDS char*)smem);
}

bool overlaps(const void* x, size_t nx, const void* y, size_t ny) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + ny && b < a + nx;
}

template <int D>
hipError_t launch_bwd(BwdArgs a, bool causal, long long rows, const uint16_t* o, const float* lse, float* lse2,
                      float* dd, int n_kv_wg, int n_q_wg, hipStream_t stream) {
    const int rpb = 256 / (D / 8);
    hipLaunchKernelGGL(fa_bwd_prep_kernel<D>, dim3(static_cast<unsigned>((rows + rpb - 1) / rpb)), dim3(256), 0,
                       stream, o, a.dout, lse, lse2, dd, rows);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    a.total = n_kv_wg;
    if (causal) hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, true>), dim3(n_kv_wg), dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, false>), dim3(n_kv_wg), dim3(512), 0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    a.total = n_q_wg;
    if (causal) hipLaunchKernelGGL((fa_bwd_dq_kernel<D, true>), dim3(n_q_wg), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((fa_bwd_dq_kernel<D, false>), dim3(n_q_wg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

fa_status run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk,
                  int64_t d, int causal, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (causal && Tq > Tk) return FA_ERR_SHAPE;
    if (!std::isfinite(scale)) return FA_ERR_SCALE;
    // The kernels take scale * log2(e) in fp32, which must stay finite.
    if (!std::isfinite(static_cast<float>(static_cast<double>(scale) * kLog2e))) return FA_ERR_SCALE;
    const auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if ((addr(q) | addr(k) | addr(v) | addr(o) | addr(dout) | addr(dq) | addr(dk) | addr(dv) | addr(workspace)) & 15u)
        return FA_ERR_ALIGN;
    if (addr(lse) & 3u) return FA_ERR_ALIGN;

    const int64_t kMax = INT64_MAX;
    if (B > kMax / Hq) return FA_ERR_OVERFLOW;
    const int64_t BH = B * Hq, BHkv = B * Hkv;
    if (BH > kMax / Tq || BHkv > kMax / Tk) return FA_ERR_OVERFLOW;
    const int64_t rows = BH * Tq, kv_rows = BHkv * Tk;
    if (rows > kMax / (4 * d) || kv_rows > kMax / (4 * d)) return FA_ERR_OVERFLOW;
    if (Tq > INT32_MAX - 4 * kRows || Tk > INT32_MAX - 4 * kRows) return FA_ERR_OVERFLOW;
    // Buffer descriptors address one head: (T + 2 tiles) rows in 32-bit byte offsets.
    if ((Tq + 2 * kQueriesPerWg) * 2 * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;
    if ((Tk + 2 * kKeysPerWg) * 2 * d > static_cast<int64_t>(UINT32_MAX)) return FA_ERR_OVERFLOW;
    const int64_t n_kt = (Tk + kKeysPerWg - 1) / kKeysPerWg;
    const int64_t n_qt = (Tq + kQueriesPerWg - 1) / kQueriesPerWg;
    if (BHkv > INT32_MAX / n_kt || BH > INT32_MAX / n_qt) return FA_ERR_OVERFLOW;
    if (rows / (256 / (d / 8)) >= INT32_MAX) return FA_ERR_OVERFLOW;   // prep grid

    const size_t q_bytes = static_cast<size_t>(rows) * static_cast<size_t>(d) * 2u;
    const size_t kv_bytes = static_cast<size_t>(kv_rows) * static_cast<size_t>(d) * 2u;
    const size_t lse_bytes = static_cast<size_t>(rows) * 4u;
    const size_t ws_need = 2u * static_cast<size_t>(rows) * 4u;
    if (workspace_bytes < ws_need) return FA_ERR_ARG;
    // Outputs must not overlap each other, the inputs or the workspace.
    const struct { const void* p; size_t n; } bufs[9] = {{q, q_bytes},  {k, kv_bytes}, {v, kv_bytes},
                                                         {o, q_bytes},  {dout, q_bytes}, {lse, lse_bytes},
                                                         {dq, q_bytes}, {dk, kv_bytes}, {dv, kv_bytes}};
    for (int x = 6; x < 9; ++x) {
        for (int y = 0; y < 9; ++y)
            if (y != x && overlaps(bufs[x].p, bufs[x].n, bufs[y].p, bufs[y].n)) return FA_ERR_ARG;
    }
    for (int y = 0; y < 9; ++y)
        if (overlaps(workspace, ws_need, bufs[y].p, bufs[y].n)) return FA_ERR_ARG;

    BwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.dout = static_cast<const uint16_t*>(dout);
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    float* lse2 = static_cast<float*>(workspace);
    float* dd = lse2 + rows;
    a.lse2 = lse2;
    a.dd = dd;
    a.tq = static_cast<int>(Tq);
    a.tk = static_cast<int>(Tk);
    a.hq = static_cast<int>(Hq);
    a.group = static_cast<int>(Hq / Hkv);
    a.n_kt = static_cast<int>(n_kt);
    a.n_qt = static_cast<int>(n_qt);
    a.total = 0;
    a.c = static_cast<float>(static_cast<double>(scale) * kLog2e);
    a.scale = scale;
    const int n_kv_wg = static_cast<int>(BHkv * n_kt), n_q_wg = static_cast<int>(BH * n_qt);
    const uint16_t* o16 = static_cast<const uint16_t*>(o);
    const hipError_t err =
        d == 128 ? launch_bwd<128>(a, causal != 0, rows, o16, lse, lse2, dd, n_kv_wg, n_q_wg, stream)
                 : launch_bwd<64>(a, causal != 0, rows, o16, lse, lse2, dd, n_kv_wg, n_q_wg, stream);
    if (err != hipSuccess) {
        fa_internal::record_hip_error(err);
        return FA_ERR_HIP;
    }
    fa_internal::clear_hip_error();
    return FA_OK;
}

}  // namespace

extern "C" size_t fa_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Tq) {
    if (B < 1 || Hq < 1 || Tq < 1) return 0;
    if ((double)B * (double)Hq * (double)Tq * 8.0 > 9.0e18) return 0;
    return static_cast<size_t>(B * Hq * Tq * 8);
}

extern "C" fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                            int64_t Tq, int64_t Tk, int64_t d, int causal, float scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Tq, Tk, d, causal, scale, workspace,
                   workspace_bytes, stream);
}
