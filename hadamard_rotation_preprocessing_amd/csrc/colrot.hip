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

}  // namespace

int launch_colrot(const ColArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
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
