// Output-side weight fusion W' = R^T . W along out_features (the rows of a
// row-major [out_features, in_features] weight), R = blockdiag(H_b) / sqrt(b)
// with the Sylvester H_b in natural order (AutoRound "Rotation Transform",
// section 1.5; section 1.1: R1 fused into the outputs of o_proj / down_proj,
// R2 per head of head_dim rows on v_proj). H_b is symmetric, so R^T = R.
//
// One workgroup transforms a tile of b rows x C columns (b C = 2^TB
// elements, C >= 8; b and TB are template parameters, so every LDS address
// is a per-thread base plus an immediate) held in LDS as float32,
// column-major with a padded stride:
//   * load: 16-byte pieces (8 columns of one row), widened to float32, up to
//     8 consecutive threads on consecutive pieces of one row;
//   * rounds of five row bits: each thread takes 32 rows of one column (the
//     five bits of the round vary, the others fixed), runs the butterflies
//     (a, b) -> (a + b, a - b) of the round's bits in registers and writes
//     them back; a barrier separates rounds;
//   * store: the normalisation 1/sqrt(b) and the conversion to the weight
//     dtype (nearest even), 16-byte pieces again.
// The grid is persistent (as many workgroups as fit on the device); each
// workgroup loads its next tile into registers while it transforms and
// stores the current one.  Tiles are numbered so that the strips of columns
// sharing cache lines land on the same XCD (workgroups are dealt to the 8
// XCDs round robin).  Blocks of 2048 rows or more leave only 8 columns
// (16 bytes of bf16) per row in a tile that fits LDS: those are bound by the
// partial-line traffic, not by the transform.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "codes.h"
#include "plan.h"

namespace hr {
namespace {

template <int LOGB, int TB, bool BF16>
__global__ void __launch_bounds__(1 << (TB - 5)) colrot_kernel(const ColArgs a) {
    constexpr int T = 1 << TB;           // tile elements
    constexpr int NT = T / 32;           // threads, 32 elements each
    constexpr int NR = BF16 ? 4 : 8;     // 16-byte registers of raw input per thread
    constexpr int logb = LOGB;
    constexpr int b = 1 << LOGB;
    constexpr int C = T >> LOGB;         // tile columns (at least 8)
    constexpr int ld = b + (b >> 5) + 1; // column stride in LDS (words)
    static_assert(LOGB >= 5 && C >= 8, "tile shape");
    __shared__ float lds[C * ld];
    const int tid = threadIdx.x;

    // persistent: this workgroup takes tiles base + t, t += step; with XCD
    // grouping each XCD owns a contiguous range of tiles
    const int64_t ntiles = a.row_blocks * a.strips;
    const bool xcd = (ntiles & 7) == 0 && (gridDim.x & 7) == 0;
    const int64_t count = xcd ? ntiles >> 3 : ntiles;
    const int64_t base = xcd ? (blockIdx.x & 7) * count : 0;
    const int64_t step = xcd ? gridDim.x >> 3 : gridDim.x;
    int64_t t = xcd ? blockIdx.x >> 3 : blockIdx.x;
    if (t >= count) return;

    // piece p (8 columns of one row) -> (row, first column): groups of up to
    // 8 consecutive threads take consecutive pieces of one row (whole 128-byte
    // lines for bf16), the groups run down the rows, then across the strip
    constexpr int lc = TB - LOGB - 3 < 3 ? TB - LOGB - 3 : 3;
    const auto piece = [&](int p, int& r, int& cc) {
        const int rest = p >> lc;
        r = rest & (b - 1);
        cc = 8 * ((p & ((1 << lc) - 1)) | ((rest >> logb) << lc));
    };
    const auto origin = [&](int64_t L) {    // element offset of the tile
        const int64_t rblk = L / a.strips;
        return rblk * b * a.in + (L - rblk * a.strips) * C;
    };
    uint4 raw[NR];
    const auto load_tile = [&](int64_t L) {
        const int64_t o = origin(L);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int r, cc;
            piece(tid + NT * k, r, cc);
            const int64_t e = o + r * a.in + cc;
            if constexpr (BF16) {
                raw[k] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.w) + e);
            } else {
                raw[2 * k] = reinterpret_cast<const uint4*>(static_cast<const float*>(a.w) + e)[0];
                raw[2 * k + 1] = reinterpret_cast<const uint4*>(static_cast<const float*>(a.w) + e)[1];
            }
        }
    };

    load_tile(base + t);
    for (;;) {
        const int64_t L = base + t;
        // ---- raw registers -> LDS as float32
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int r, cc;
            piece(tid + NT * k, r, cc);
            float v[8];
            if constexpr (BF16) {
                const uint32_t w4[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = __uint_as_float(w4[i] << 16);
                    v[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
                }
            } else {
                const uint4 d0 = raw[2 * k], d1 = raw[2 * k + 1];
                v[0] = __uint_as_float(d0.x); v[1] = __uint_as_float(d0.y);
                v[2] = __uint_as_float(d0.z); v[3] = __uint_as_float(d0.w);
                v[4] = __uint_as_float(d1.x); v[5] = __uint_as_float(d1.y);
                v[6] = __uint_as_float(d1.z); v[7] = __uint_as_float(d1.w);
            }
            const int pr = r + (r >> 5);
#pragma unroll
            for (int i = 0; i < 8; ++i) lds[(cc + i) * ld + pr] = v[i];
        }
        __syncthreads();
        // the next tile's loads stay in flight through the rounds and stores
        // (the barriers wait for LDS traffic only)
        const bool more = t + step < count;
        if (more) load_tile(L + step);

        // ---- rounds of five row bits; consecutive threads differ in q, so
        // the 32 lanes of a half-wave hit 32 banks
        const int q = tid & ((b >> 5) - 1);  // the row bits outside the round's window
        const int col = tid >> (logb - 5);
#pragma unroll
        for (int s = 0; s < logb; s += 5) {
            const int w0 = s + 5 <= logb ? s : logb - 5;   // window [w0, w0 + 5)
            const int lo = q & ((1 << w0) - 1);
            const int hi = (q >> w0) << (w0 + 5);
            // row r = hi | j << w0 | lo from disjoint bit fields, so its padded
            // index r + r / 32 splits into a per-thread base and a constant per j
            const int rb = hi | lo;
            float* const col_base = lds + col * ld + rb + (rb >> 5);
            float v[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) v[j] = col_base[(j << w0) + ((j << w0) >> 5)];
            // butterflies of the window bits not transformed in earlier rounds
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                if (w0 + k < s) continue;
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    if (!(j & (1 << k))) {
                        const float x0 = v[j], x1 = v[j + (1 << k)];
                        v[j] = x0 + x1;
                        v[j + (1 << k)] = x0 - x1;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 32; ++j) col_base[(j << w0) + ((j << w0) >> 5)] = v[j];
            __syncthreads();
        }

        // ---- store
        const int64_t o = origin(L);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int r, cc;
            piece(tid + NT * k, r, cc);
            const int pr = r + (r >> 5);
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = lds[(cc + i) * ld + pr] * a.norm;
            const int64_t e = o + r * a.in + cc;
            if constexpr (BF16) {
                uint4 d;
                d.x = f2bf(v[0]) | (f2bf(v[1]) << 16);
                d.y = f2bf(v[2]) | (f2bf(v[3]) << 16);
                d.z = f2bf(v[4]) | (f2bf(v[5]) << 16);
                d.w = f2bf(v[6]) | (f2bf(v[7]) << 16);
                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.w_rot) + e) = d;
            } else {
                float* dst = static_cast<float*>(a.w_rot) + e;
                reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
                reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
        if (!more) break;
        __syncthreads();      // every store read of LDS done before the next tile's writes
        t += step;
    }
}

template <int LOGB, int TB, bool BF16>
int launch_tb(const ColArgs& a, hipStream_t s) {
    // persistent grid: as many workgroups as the device holds at once
    static std::atomic<int> slots[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
    int cap = slots[dev].load(std::memory_order_relaxed);
    if (cap == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, colrot_kernel<LOGB, TB, BF16>, 1 << (TB - 5), 0) !=
                hipSuccess)
            return static_cast<int>(hipErrorInvalidValue);
        cap = cus * (per > 0 ? per : 1);
        slots[dev].store(cap, std::memory_order_relaxed);
    }
    const int64_t ntiles = a.row_blocks * a.strips;
    const int64_t grid = ntiles < cap ? ntiles : cap;
    hipLaunchKernelGGL((colrot_kernel<LOGB, TB, BF16>), dim3(static_cast<unsigned>(grid)), dim3(1 << (TB - 5)), 0, s,
                       a);
    return static_cast<int>(hipGetLastError());
}

// tile sizes 2^TB, TB from max(11, LOGB + 3) up to 15
template <int LOGB, int TB = 15>
int launch_logb(const ColArgs& a, hipStream_t s) {
    if (a.tb == TB) return a.bf16 ? launch_tb<LOGB, TB, true>(a, s) : launch_tb<LOGB, TB, false>(a, s);
    if constexpr (TB > 11 && TB > LOGB + 3) return launch_logb<LOGB, TB - 1>(a, s);
    return static_cast<int>(hipErrorInvalidValue);
}


// ---------------------------------------------------------------- colwide
// Output-side fusion along out_features = K * M rows held in one tile (the
// Kronecker form R = (H_K (x) H_M) / sqrt(K M) for out_features that are not
// a power of two, AutoRound "Rotation Transform", section 1.5; K = 1 is a
// Sylvester block of 8192 rows, too tall for colrot's tiles).  W'[(a, m)] =
// sum_c H_K[c][a] sum_m' H_M[m'][m] W[(c, m')] / sqrt(K M).
// A workgroup of 512 threads takes a tile of all K M rows x 4 columns
// (135 KB of LDS at 8192 rows), float32, column-major with a padded stride:
//   * load: one piece (4 columns of one row, 8 bytes of bf16) per row,
//     R / 512 per thread, kept in registers one tile ahead;
//   * H_M on each block of M rows: rounds of five row bits as in colrot,
//     work items (column, block, 32-row group) spread over the threads;
//   * the base-matrix mix (K > 1): work items (column, m), each reading the
//     K values of rows c M + m into registers and writing the K outputs back
//     (each item owns its rows); signs from the dense bits of H_K;
//   * store with the normalisation and the conversion to the weight dtype.
// Rows of 8 bytes are partial cache lines: the 16 tiles sharing a line run
// on one XCD (the numbering of colrot), and the transform is not the limit.
template <int LOGM, int K, bool BF16>
__global__ void __launch_bounds__(512, 1) colwide_kernel(const ColArgs a) {
    constexpr int M = 1 << LOGM;
    constexpr int R = K * M;             // rows of the tile
    constexpr int C = 4;                 // columns of the tile
    constexpr int NT = 512;
    constexpr int NP = R / NT;           // pieces (rows) per thread
    constexpr int ld = R + (R >> 5) + 1; // column stride in LDS (words)
    static_assert(LOGM >= 5 && R % NT == 0 && K <= 32, "tile shape");
    __shared__ float lds[C * ld];
    const int tid = threadIdx.x;

    const int64_t ntiles = a.row_blocks * a.strips;
    const bool xcd = (ntiles & 7) == 0 && (gridDim.x & 7) == 0;
    const int64_t count = xcd ? ntiles >> 3 : ntiles;
    const int64_t base = xcd ? (blockIdx.x & 7) * count : 0;
    const int64_t step = xcd ? gridDim.x >> 3 : gridDim.x;
    int64_t t = xcd ? blockIdx.x >> 3 : blockIdx.x;
    if (t >= count) return;

    const auto origin = [&](int64_t L) {
        const int64_t rblk = L / a.strips;
        return rblk * R * a.in + (L - rblk * a.strips) * C;
    };
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    // a piece is 2 words (bf16) or 4 (float32); the next tile is loaded into
    // registers ahead of time only where that takes at most 32 of them
    constexpr int WORDS = BF16 ? 2 : 4;
    constexpr bool PREFETCH = NP * WORDS <= 32;
    constexpr int NPR = PREFETCH ? NP : 1;
    uint32_t raw[NPR][WORDS];
    const auto load_piece = [&](int64_t o, int k, uint32_t (&d)[WORDS]) {
        const int64_t e = o + static_cast<int64_t>(tid + NT * k) * a.in;
        if constexpr (BF16) {
            const u32x2 x = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.w) + e);
            d[0] = x[0];
            d[1] = x[1];
        } else {
            const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const float*>(a.w) + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = x[i];
        }
    };
    const auto stage_piece = [&](int k, const uint32_t (&d)[WORDS]) {
        const int r = tid + NT * k;
        float v[4];
        if constexpr (BF16) {
            v[0] = __uint_as_float(d[0] << 16);
            v[1] = __uint_as_float(d[0] & 0xFFFF0000u);
            v[2] = __uint_as_float(d[1] << 16);
            v[3] = __uint_as_float(d[1] & 0xFFFF0000u);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(d[i]);
        }
        const int pr = r + (r >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds[i * ld + pr] = v[i];
    };
    const auto load_tile = [&](int64_t L) {
        const int64_t o = origin(L);
#pragma unroll
        for (int k = 0; k < NP; ++k) load_piece(o, k, raw[k]);
    };

    if constexpr (PREFETCH) load_tile(base + t);
    for (;;) {
        const int64_t L = base + t;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int k = 0; k < NP; ++k) stage_piece(k, raw[k]);
        } else {
            const int64_t o = origin(L);
            for (int k = 0; k < NP; ++k) {
                load_piece(o, k, raw[0]);
                stage_piece(k, raw[0]);
            }
        }
        __syncthreads();
        const bool more = t + step < count;
        if constexpr (PREFETCH) {
            if (more) load_tile(L + step);
        }

        // ---- H_M on each block of M rows: rounds of five row bits
        constexpr int G = M / 32;                 // 32-row groups per block per round
        constexpr int ITEMS = C * K * G;
#pragma unroll
        for (int s = 0; s < LOGM; s += 5) {
            const int w0 = s + 5 <= LOGM ? s : LOGM - 5;   // window [w0, w0 + 5)
#pragma unroll 1
            for (int it = tid; it < ITEMS; it += NT) {
                const int q = it % G;
                const int blk = (it / G) % K;
                const int col = it / (G * K);
                const int lo = q & ((1 << w0) - 1);
                const int hi = (q >> w0) << (w0 + 5);
                // row r = blk M + hi | j << w0 | lo from disjoint bit fields:
                // its padded index r + r / 32 is a per-item base plus a
                // constant per j
                const int rb = blk * M + (hi | lo);
                float* const cb = lds + col * ld + rb + (rb >> 5);
                float v[32];
#pragma unroll
                for (int j = 0; j < 32; ++j) v[j] = cb[(j << w0) + ((j << w0) >> 5)];
#pragma unroll
                for (int k = 0; k < 5; ++k) {
                    if (w0 + k < s) continue;
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        if (!(j & (1 << k))) {
                            const float x0 = v[j], x1 = v[j + (1 << k)];
                            v[j] = x0 + x1;
                            v[j + (1 << k)] = x0 - x1;
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < 32; ++j) cb[(j << w0) + ((j << w0) >> 5)] = v[j];
            }
            __syncthreads();
        }
        // ---- base-matrix mix across the K blocks: y_a = sum_c H_K[c][a] z_c
        if constexpr (K > 1) {
            // row c M + m has the padded index c (M + M / 32) + m + m / 32
            constexpr int PM = M + M / 32;
#pragma unroll 1
            for (int it = tid; it < C * M; it += NT) {
                const int m = it % M;
                const int col = it / M;
                float* const cb = lds + col * ld + m + (m >> 5);
                float z[K];
#pragma unroll
                for (int c = 0; c < K; ++c) z[c] = cb[c * PM];
#pragma unroll 1
                for (int o = 0; o < K; ++o) {
                    const uint64_t neg = a.hk_neg[o];   // bit c: H_K[c][o] == -1
                    float acc = 0.0f;
#pragma unroll
                    for (int c = 0; c < K; ++c) acc += ((neg >> c) & 1u) ? -z[c] : z[c];
                    cb[o * PM] = acc;
                }
            }
            __syncthreads();
        }

        // ---- store
        const int64_t o = origin(L);
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int r = tid + NT * k;
            const int pr = r + (r >> 5);
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = lds[i * ld + pr] * a.norm;
            const int64_t e = o + static_cast<int64_t>(r) * a.in;
            if constexpr (BF16) {
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.w_rot) + e) =
                    u32x2{f2bf(v[0]) | (f2bf(v[1]) << 16), f2bf(v[2]) | (f2bf(v[3]) << 16)};
            } else {
                *reinterpret_cast<u32x4*>(static_cast<float*>(a.w_rot) + e) =
                    u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
            }
        }
        if (!more) break;
        __syncthreads();
        t += step;
    }
}

template <int LOGM, int K, bool BF16>
int launch_wide(const ColArgs& a, hipStream_t s) {
    static std::atomic<int> slots[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
    int cap = slots[dev].load(std::memory_order_relaxed);
    if (cap == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, colwide_kernel<LOGM, K, BF16>, 512, 0) != hipSuccess)
            return static_cast<int>(hipErrorInvalidValue);
        cap = cus * (per > 0 ? per : 1);
        slots[dev].store(cap, std::memory_order_relaxed);
    }
    const int64_t ntiles = a.row_blocks * a.strips;
    const int64_t grid = ntiles < cap ? ntiles : cap;
    hipLaunchKernelGGL((colwide_kernel<LOGM, K, BF16>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, s, a);
    return static_cast<int>(hipGetLastError());
}

template <int LOGM, int K>
int launch_wide_dt(const ColArgs& a, hipStream_t s) {
    return a.bf16 ? launch_wide<LOGM, K, true>(a, s) : launch_wide<LOGM, K, false>(a, s);
}
}  // namespace

int launch_colrot(const ColArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.kron_k > 1 || a.logb > 12) {
        // whole-height tiles of 4 columns (colwide): K x M rows
        const int key = a.kron_k * 100 + a.logb;
        switch (key) {
            case 100 + 13: return launch_wide_dt<13, 1>(a, s);    // Sylvester 8192
            case 1200 + 7: return launch_wide_dt<7, 12>(a, s);
            case 1200 + 8: return launch_wide_dt<8, 12>(a, s);
            case 1200 + 9: return launch_wide_dt<9, 12>(a, s);
            case 2000 + 7: return launch_wide_dt<7, 20>(a, s);
            case 2000 + 8: return launch_wide_dt<8, 20>(a, s);
            case 2800 + 7: return launch_wide_dt<7, 28>(a, s);
            case 2800 + 8: return launch_wide_dt<8, 28>(a, s);
            default: return static_cast<int>(hipErrorInvalidValue);
        }
    }
    switch (a.logb) {
        case 5: return launch_logb<5>(a, s);
        case 6: return launch_logb<6>(a, s);
        case 7: return launch_logb<7>(a, s);
        case 8: return launch_logb<8>(a, s);
        case 9: return launch_logb<9>(a, s);
        case 10: return launch_logb<10>(a, s);
        case 11: return launch_logb<11>(a, s);
        case 12: return launch_logb<12>(a, s);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

}  // namespace hr
