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
// gfx950 mapping (one workgroup = 4 waves of 64 lanes, 128 query rows):
//   * Each wave owns 32 query rows.  It computes the TRANSPOSED score tile
//     S^T = K_j Q_i^T with v_mfma_f32_32x32x16_bf16, so that in the accumulator
//     every lane holds 32 scores of ONE query row (lane % 32) -- half the keys of
//     the tile, the other half in lane ^ 32.  Row max and row sum are then
//     in-register reductions plus one exchange between the two lane halves.
//   * The output is accumulated transposed as well, O^T += V_j^T P^T, whose
//     B operand is exactly the bf16-converted score accumulator (no LDS round
//     trip for P), and whose accumulator again keeps one query row per lane, so
//     the rescale factor of a row is lane-local.
//   * K_j is staged in LDS row-major; V_j is staged transposed (V^T) with the key
//     order inside each 16-key group permuted to match the accumulator layout of
//     S^T, so each MFMA operand is one 16-byte LDS read.  Rows are padded by 16
//     bytes against bank conflicts.  Two LDS stages: tile j+1 is fetched from
//     HBM into registers while tile j is computed.
//   * Causal: whole key tiles above a wave's diagonal are skipped; only tiles
//     that cross the diagonal (or the ragged end of the sequence) are masked.
//   * The max is tracked lazily: a row is rescaled only when its tile maximum
//     exceeds the running reference by more than 2^8 (in exp2 units), the
//     conditional rescale described for FlashAttention-4 on "FlashAttention and
//     Fused Kernels: Attention Without the n x n Matrix" ("Four generations").
//     Weights exp2(x - m) are then at most 256, exact in fp32 and bf16 range,
//     and the result is unchanged up to rounding.
//   * Workgroup order: the grid is remapped so that a contiguous range of the
//     work list lands on one XCD (workgroups are dealt round-robin over the 8
//     XCDs), keeping one head's K/V in that XCD's L2; within a head the heaviest
//     causal query tiles go first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

template <int D>
struct Tile {
    static constexpr int kKStride = D + 8;                   // bf16 per K row in LDS
    static constexpr int kVStride = kBN + 8;                 // bf16 per V^T row in LDS
    static constexpr int kKElems = kBN * kKStride;
    static constexpr int kVElems = D * kVStride;
    static constexpr int kStage = kKElems + kVElems;         // bf16 per LDS stage
    static constexpr int kKChunks = kBN * D / 8 / kThreads;  // 16-byte K chunks per thread
    static constexpr int kVKeys = D / 32;                    // V rows per thread (8 d values each)
    static constexpr int kVKeyGroups = kBN / kVKeys;
};

template <int D>
struct TileRegs {
    u32x4 k[Tile<D>::kKChunks];
    u32x4 v[Tile<D>::kVKeys];
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Position of key `key` (0..63 within a tile) in the transposed V tile: bits 2
// and 3 swapped.  The S^T accumulator gives lane half h, element e of the
// 16-key step the key 8*(e/4) + 4*h + e%4; with this permutation those eight
// keys are contiguous at slot 8*h + e.
__device__ __forceinline__ int vt_slot(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Fetch K/V tile rows [key0, key0+64) of one head into registers (zeros past T).
template <int D>
__device__ __forceinline__ void fetch_tile(TileRegs<D>& r, const uint16_t* __restrict__ kbh,
                                           const uint16_t* __restrict__ vbh, int key0, int T, int tid) {
    using TL = Tile<D>;
    constexpr int kChunksPerRow = D / 8;
#pragma unroll
    for (int c = 0; c < TL::kKChunks; ++c) {
        const int chunk = tid + c * kThreads;
        const int key = key0 + chunk / kChunksPerRow;
        const int col = chunk % kChunksPerRow;
        r.k[c] = key < T ? *reinterpret_cast<const u32x4*>(kbh + (size_t)key * D + col * 8)
                         : u32x4{0u, 0u, 0u, 0u};
    }
    const int kg = tid % TL::kVKeyGroups;
    const int dg = tid / TL::kVKeyGroups;
#pragma unroll
    for (int e = 0; e < TL::kVKeys; ++e) {
        const int key = key0 + kg * TL::kVKeys + e;
        r.v[e] = key < T ? *reinterpret_cast<const u32x4*>(vbh + (size_t)key * D + dg * 8)
                         : u32x4{0u, 0u, 0u, 0u};
    }
}

// Registers -> one LDS stage: K row-major, V transposed with the slot permutation.
template <int D>
__device__ __forceinline__ void stage_tile(const TileRegs<D>& r, uint16_t* ks, uint16_t* vts, int tid) {
    using TL = Tile<D>;
    constexpr int kChunksPerRow = D / 8;
#pragma unroll
    for (int c = 0; c < TL::kKChunks; ++c) {
        const int chunk = tid + c * kThreads;
        const int row = chunk / kChunksPerRow;
        const int col = chunk % kChunksPerRow;
        *reinterpret_cast<u32x4*>(ks + row * TL::kKStride + col * 8) = r.k[c];
    }
    const int kg = tid % TL::kVKeyGroups;
    const int dg = tid / TL::kVKeyGroups;
    const int slot0 = vt_slot(kg * TL::kVKeys);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        uint16_t* dst = vts + (dg * 8 + e) * TL::kVStride + slot0;
        if constexpr (TL::kVKeys == 4) {
            u32x2 w;
            w.x = ((r.v[0][e >> 1] >> sh) & 0xffffu) | (((r.v[1][e >> 1] >> sh) & 0xffffu) << 16);
            w.y = ((r.v[2][e >> 1] >> sh) & 0xffffu) | (((r.v[3][e >> 1] >> sh) & 0xffffu) << 16);
            *reinterpret_cast<u32x2*>(dst) = w;
        } else {
            static_assert(TL::kVKeys == 2, "head size must be 64 or 128");
            const uint32_t w = ((r.v[0][e >> 1] >> sh) & 0xffffu) | (((r.v[1][e >> 1] >> sh) & 0xffffu) << 16);
            *reinterpret_cast<uint32_t*>(dst) = w;
        }
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                   int T, int n_qt, int total, float c /* scale * log2(e) */) {
    using TL = Tile<D>;
    constexpr int kDSteps = D / 16;   // MFMA k-steps over the head dimension
    constexpr int kDBlocks = D / 32;  // 32-row blocks of O^T

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TL::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const uint16_t* __restrict__ qbh = Q + base;
    const uint16_t* __restrict__ kbh = K + base;
    const uint16_t* __restrict__ vbh = V + base;

    const int qw0 = qt * kBM + wave * 32;   // first query row of this wave
    const int qrow = qw0 + col;
    const bool wave_active = qw0 < T;
    const int wave_last_key = CAUSAL ? min(qw0 + 31, T - 1) : T - 1;

    // Q^T operand: lane holds Q[qrow][16 s + 8 half .. +7].
    bf16x8 qf[kDSteps];
#pragma unroll
    for (int s = 0; s < kDSteps; ++s) {
        u32x4 raw = qrow < T ? *reinterpret_cast<const u32x4*>(qbh + (size_t)qrow * D + 16 * s + 8 * half)
                             : u32x4{0u, 0u, 0u, 0u};
        qf[s] = __builtin_bit_cast(bf16x8, raw);
    }

    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] = 0.0f;
    float m = -INFINITY;   // running reference max, log2 units
    float l32 = 0.0f;      // sum of fp32 weights (for lse)
    float l16 = 0.0f;      // sum of the bf16-rounded weights fed to the PV product (for O)

    const int kv_end = CAUSAL ? min(T, qt * kBM + kBM) : T;
    const int n_kt = ceil_div(kv_end, kBN);

    TileRegs<D> tr;
    fetch_tile<D>(tr, kbh, vbh, 0, T, tid);
    stage_tile<D>(tr, smem, smem + TL::kKElems, tid);
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const uint16_t* ks = smem + (j & 1) * TL::kStage;
        const uint16_t* vts = ks + TL::kKElems;
        if (j + 1 < n_kt) fetch_tile<D>(tr, kbh, vbh, (j + 1) * kBN, T, tid);

        const int key0 = j * kBN;
        if (wave_active && key0 <= wave_last_key) {
            // S^T = K_j Q^T : two 32-key blocks.
            f32x16 sacc[2];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[b][i] = 0.0f;
#pragma unroll
            for (int s = 0; s < kDSteps; ++s) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + col) * TL::kKStride +
                                                                      16 * s + 8 * half);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
                }
            }

            // Scale into exp2 units; mask keys past the diagonal or past T.
            float x[32];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) x[kb * 16 + i] = sacc[kb][i] * c;
            const bool need_mask = (CAUSAL && key0 + kBN - 1 > qw0) || (key0 + kBN > T);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                        const bool hide = (CAUSAL && key > qrow) || key >= T;
                        x[kb * 16 + i] = hide ? -INFINITY : x[kb * 16 + i];
                    }
            }

            // Row max over the tile (in-register, then across the two lane halves).
            float mt = x[0];
#pragma unroll
            for (int i = 1; i < 32; ++i) mt = fmaxf(mt, x[i]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m, mt);
            const bool need = m_new > m + kRescaleThreshold;
            if (__any(need)) {
                const float r = need ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
                m = need ? m_new : m;
                l32 *= r;
                l16 *= r;
#pragma unroll
                for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[b][i] *= r;
            }
            const float mu = (m == -INFINITY) ? 0.0f : m;

            // Weights, both row sums, bf16 P^T operand.
            uint32_t pk[16];
            const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                const float p0 = __builtin_amdgcn_exp2f(x[2 * n] - mu);
                const float p1 = __builtin_amdgcn_exp2f(x[2 * n + 1] - mu);
                l32 += p0;
                l32 += p1;
                pk[n] = pack_bf16x2(p0, p1);
                l16 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[n]), ones, l16, false);
            }

            // O^T += V_j^T P^T : four 16-key steps.
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const u32x4 praw = {pk[4 * st], pk[4 * st + 1], pk[4 * st + 2], pk[4 * st + 3]};
                const bf16x8 pb = __builtin_bit_cast(bf16x8, praw);
#pragma unroll
                for (int b = 0; b < kDBlocks; ++b) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(vts + (b * 32 + col) * TL::kVStride +
                                                                      16 * st + 8 * half);
                    oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[b], 0, 0, 0);
                }
            }
        }

        if (j + 1 < n_kt)
            stage_tile<D>(tr, smem + ((j + 1) & 1) * TL::kStage, smem + ((j + 1) & 1) * TL::kStage + TL::kKElems,
                          tid);
        __syncthreads();
    }

    // Epilogue: O = o / l (bf16, round to nearest even), lse = ln2 * (m + log2 l).
    l32 += __shfl_xor(l32, 32);
    l16 += __shfl_xor(l16, 32);
    if (!wave_active || qrow >= T) return;
    const float inv = 1.0f / l16;
    uint16_t* orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 wv;
            wv.x = pack_bf16x2(oacc[b][4 * g + 0] * inv, oacc[b][4 * g + 1] * inv);
            wv.y = pack_bf16x2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + b * 32 + 8 * g + 4 * half) = wv;
        }
    if (half == 0) LSE[(size_t)bh * T + qrow] = kLn2 * (m + __builtin_amdgcn_logf(l32));
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
