// Rotation + quantization kernels for gfx950 (CDNA4, wave64).
//
// Generic kernel family `rot_kernel<LOGE, BF16, KMAX>`:
//   * The flattened [rows, n] tensor is cut into chunks of C elements (a
//     whole number of Hadamard blocks and quantizer groups).  A chunk is
//     owned by C / E consecutive threads; thread t of a chunk holds the E
//     contiguous elements [t E, t E + E) in registers (coalesced 16-byte
//     loads), widened to float32.
//   * Fast Walsh-Hadamard transform of each power-of-two block B = 2^logb
//     (the Sylvester matrix in natural order, AutoRound "Rotation
//     Transform", section 1.5): butterflies (a, b) -> (a + b, a - b) on the
//     index bits that are register bits, then a transpose through LDS that
//     makes the next LOGE unprocessed index bits register bits, and so on;
//     a final transpose returns every thread to its contiguous elements.
//     LDS rows are padded by one word per 16 to spread banks.
//   * Kronecker form (width K * 2^m, section 1.5 of the same page): after the
//     transform of each length-2^m piece, the K pieces of a row are mixed by
//     the base matrix: y_c = sum_a H_K[a][c] z_a, one column per thread.
//   * Randomised rotations (a permutation gather and +-1 signs before the
//     transform, +-1 signs after it: the random Hadamard H diag(+-1) of the
//     AutoRound page, section 1.5, and OrbitQuant's RPBH, Method
//     Conformance) read element by element; with a permutation the loads
//     are gathers within the row.
//   * One normalisation multiply, optional store of the rotated tensor, and
//     up to two fused quantizer epilogues (INT sym/asym groups, MXFP4, NVFP4) that
//     reduce group statistics across the threads of a group with lane
//     shuffles (and LDS across waves), round, pack nibbles and store.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "codes.h"
#include "plan.h"

namespace hr {
namespace {

// ----------------------------------------------------------------- vector IO

template <int E, bool BF16>
__device__ __forceinline__ void load_vals(const void* base, int64_t e0, float (&v)[E]) {
    if constexpr (BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(base) + e0;
        if constexpr (E >= 8) {
#pragma unroll
            for (int c = 0; c < E / 8; ++c) {
                const uint4 d = reinterpret_cast<const uint4*>(p)[c];
                const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[c * 8 + 2 * k] = __uint_as_float(w[k] << 16);
                    v[c * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                }
            }
        } else if constexpr (E == 4) {
            const uint2 d = *reinterpret_cast<const uint2*>(p);
            v[0] = __uint_as_float(d.x << 16);
            v[1] = __uint_as_float(d.x & 0xFFFF0000u);
            v[2] = __uint_as_float(d.y << 16);
            v[3] = __uint_as_float(d.y & 0xFFFF0000u);
        } else {
            const uint32_t d = *reinterpret_cast<const uint32_t*>(p);
            v[0] = __uint_as_float(d << 16);
            v[1] = __uint_as_float(d & 0xFFFF0000u);
        }
    } else {
        const float* p = static_cast<const float*>(base) + e0;
        if constexpr (E >= 4) {
#pragma unroll
            for (int c = 0; c < E / 4; ++c) {
                const float4 d = reinterpret_cast<const float4*>(p)[c];
                v[4 * c] = d.x;
                v[4 * c + 1] = d.y;
                v[4 * c + 2] = d.z;
                v[4 * c + 3] = d.w;
            }
        } else {
            const float2 d = *reinterpret_cast<const float2*>(p);
            v[0] = d.x;
            v[1] = d.y;
        }
    }
}

template <bool BF16>
__device__ __forceinline__ float load_one(const void* base, int64_t e) {
    if constexpr (BF16)
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[e]) << 16);
    else
        return static_cast<const float*>(base)[e];
}

template <int E, bool BF16>
__device__ __forceinline__ void store_vals(void* base, int64_t e0, const float (&v)[E]) {
    if constexpr (BF16) {
        uint16_t* p = static_cast<uint16_t*>(base) + e0;
        uint32_t w[E / 2];
#pragma unroll
        for (int k = 0; k < E / 2; ++k) w[k] = f2bf(v[2 * k]) | (f2bf(v[2 * k + 1]) << 16);
        if constexpr (E >= 8) {
#pragma unroll
            for (int c = 0; c < E / 8; ++c)
                reinterpret_cast<uint4*>(p)[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
        } else if constexpr (E == 4) {
            *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        } else {
            *reinterpret_cast<uint32_t*>(p) = w[0];
        }
    } else {
        float* p = static_cast<float*>(base) + e0;
        if constexpr (E >= 4) {
#pragma unroll
            for (int c = 0; c < E / 4; ++c)
                reinterpret_cast<float4*>(p)[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
        } else {
            *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
        }
    }
}

// Store E/2 packed code bytes.
template <int E>
__device__ __forceinline__ void store_codes(uint8_t* base, int64_t e0, const uint32_t (&w)[(E + 7) / 8]) {
    uint8_t* p = base + (e0 >> 1);
    if constexpr (E == 32) {
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (E == 16) {
        *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else if constexpr (E == 8) {
        *reinterpret_cast<uint32_t*>(p) = w[0];
    } else if constexpr (E == 4) {
        *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(w[0]);
    } else {
        *p = static_cast<uint8_t>(w[0]);
    }
}

// ---------------------------------------------------------------- transform

// Butterflies on the register-index bits selected by `mask`.
template <int LOGE>
__device__ __forceinline__ void bfly(float (&v)[1 << LOGE], unsigned mask) {
#pragma unroll
    for (int k = 0; k < LOGE; ++k) {
        if (mask & (1u << k)) {
#pragma unroll
            for (int j = 0; j < (1 << LOGE); ++j) {
                if (!(j & (1 << k))) {
                    const float a = v[j];
                    const float b = v[j + (1 << k)];
                    v[j] = a + b;
                    v[j + (1 << k)] = a - b;
                }
            }
        }
    }
}

// Block-relative index of register j of block-thread t when the register
// bits are the index bits [w, w + loge).
__device__ __forceinline__ int tpos(int t, int j, int w, int loge) {
    return ((t >> w) << (w + loge)) | (j << w) | (t & ((1 << w) - 1));
}

__device__ __forceinline__ int lpad(int i) { return i + (i >> 4); }

// Unnormalised FWHT of every block of 2^logb elements; on return each thread
// again holds its E contiguous elements.
template <int LOGE>
__device__ __forceinline__ void fwht(float (&v)[1 << LOGE], float* lds, int tid, int logb) {
    constexpr int E = 1 << LOGE;
    if (logb <= LOGE) {
        bfly<LOGE>(v, (1u << logb) - 1u);
        return;
    }
    bfly<LOGE>(v, (1u << LOGE) - 1u);
    const int tbl = logb - LOGE;
    const int t = tid & ((1 << tbl) - 1);
    const int base = (tid - t) * E;
    int done = LOGE;
    int wprev = 0;
    while (true) {
        const int w = (done < logb) ? min(done, logb - LOGE) : 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < E; ++j) lds[lpad(base + tpos(t, j, wprev, LOGE))] = v[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = lds[lpad(base + tpos(t, j, w, LOGE))];
        if (done >= logb) break;
        const int hi = w + LOGE;
        const unsigned m = ((1u << (hi - done)) - 1u) << (done - w);
        bfly<LOGE>(v, m);
        done = hi;
        wprev = w;
    }
}

// Kronecker mix across the K pieces (length M = 2^logb) of each chunk:
// y[c][col] = sum_a H_K[a][c] z[a][col].
template <int LOGE, int KMAX>
__device__ __forceinline__ void kron_mix(float (&v)[1 << LOGE], float* lds, int tid, const RotArgs& a) {
    constexpr int E = 1 << LOGE;
    const int K = a.kron_k;
    const int M = 1 << a.logb;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) lds[lpad(tid * E + j)] = v[j];
    __syncthreads();
    const int cl = tid / a.tpc;
    const int lt = tid - cl * a.tpc;
    const int cbase = cl * a.chunk;
    for (int col = lt; col < M; col += a.tpc) {
        float z[KMAX];
        float o[KMAX];
#pragma unroll
        for (int i = 0; i < KMAX; ++i) z[i] = (i < K) ? lds[lpad(cbase + i * M + col)] : 0.0f;
#pragma unroll
        for (int c = 0; c < KMAX; ++c) {
            float acc = 0.0f;
            if (c < K) {
                const uint64_t neg = a.hk_neg[c];
#pragma unroll
                for (int i = 0; i < KMAX; ++i) {
                    if (i < K) acc += ((neg >> i) & 1u) ? -z[i] : z[i];
                }
            }
            o[c] = acc;
        }
#pragma unroll
        for (int c = 0; c < KMAX; ++c)
            if (c < K) lds[lpad(cbase + c * M + col)] = o[c];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = lds[lpad(tid * E + j)];
}

// H_K[r][c] == -1 for the Kronecker base matrix of `a`: the dense bits, or
// for orders above 64 the Paley I construction over the integers mod a prime
// q: +1 on the diagonal and in row 0, -1 in column 0 below it, else the
// quadratic character of (r - c) mod q.
__device__ __forceinline__ bool hk_minus(const RotArgs& a, int r, int c) {
    if (a.kron_q == 0) return (a.hk_neg[c] >> r) & 1u;
    if (r == c || r == 0) return false;
    if (c == 0) return true;
    int d = r - c;
    if (d < 0) d += a.kron_q;
    return ((a.kron_chi[d >> 5] >> (d & 31)) & 1u) == 0u;
}

// Kronecker mix for orders above 64: each of the chunk's threads computes
// outputs (c, col) in turn from the K pieces staged in LDS, into a second
// LDS buffer (`out`), so no output overwrites an input still to be read.
template <int LOGE>
__device__ __forceinline__ void kron_mix_wide(float (&v)[1 << LOGE], float* lds, float* out, int tid, const RotArgs& a) {
    constexpr int E = 1 << LOGE;
    const int K = a.kron_k;
    const int M = 1 << a.logb;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) lds[lpad(tid * E + j)] = v[j];
    __syncthreads();
    const int cl = tid / a.tpc;
    const int lt = tid - cl * a.tpc;
    const int cbase = cl * a.chunk;
    for (int idx = lt; idx < K * M; idx += a.tpc) {
        const int c = idx >> a.logb;
        const int col = idx & (M - 1);
        float acc = 0.0f;
        for (int r = 0; r < K; ++r) {
            const float z = lds[lpad(cbase + r * M + col)];
            acc += hk_minus(a, r, c) ? -z : z;
        }
        out[lpad(cbase + c * M + col)] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = out[lpad(tid * E + j)];
}

// ---------------------------------------------------------------- epilogue

// Several whole groups of G = 2^LOGG elements in one thread's E = 2^LOGE
// (LOGG < LOGE): blocks wider than 1024 groups.  INT and NVFP4 (MXFP4's
// groups of 32 are never smaller than a thread's elements).  Every group is
// the thread's own, so nothing is exchanged and no barrier is needed.
template <int LOGE, int LOGG>
__device__ __forceinline__ void quantize_multi(const float (&y)[1 << LOGE], const QuantDev& q, bool valid,
                                               int64_t e0) {
    constexpr int E = 1 << LOGE, G = 1 << LOGG, NG = E / G;
    static_assert(NG >= 2 && E >= 8, "several groups, whole bytes of codes");
    const int64_t G0 = e0 >> LOGG;   // even: e0 is a multiple of E >= 2 G
    uint32_t w[E / 8];
#pragma unroll
    for (int k = 0; k < E / 8; ++k) w[k] = 0u;
    uint32_t zq[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        float r0 = y[k * G], r1 = -y[k * G];   // max y, max(-y)
#pragma unroll
        for (int j = 1; j < G; ++j) {
            r0 = fmaxf(r0, y[k * G + j]);
            r1 = fmaxf(r1, -y[k * G + j]);
        }
        zq[k] = 0u;
        if (q.format == 2) {
            const uint32_t byte = e4m3_byte(fmaxf(r0, r1) / (6.0f * q.tscale));
            const float s = e4m3_value(byte) * q.tscale;
            if (s > 0.0f) {
                const float inv = 1.0f / s;
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const int jj = k * G + j;
                    const float a = fabsf(y[jj] * inv);
                    uint32_t idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                                   (a >= 3.5f) + (a > 5.0f);
                    idx |= (y[jj] < 0.0f) ? 8u : 0u;
                    w[jj >> 3] |= idx << (4 * (jj & 7));
                }
            }
            if (valid) static_cast<uint8_t*>(q.scales)[G0 + k] = static_cast<uint8_t>(byte);
        } else {
            float s = q.sym ? fmaxf(r0, r1) / 7.0f : (fmaxf(r0, 0.0f) + fmaxf(r1, 0.0f)) / 15.0f;
            uint32_t sbits = 0;
            if (q.scale_dtype == 1) {
                sbits = f2bf(s);
                s = bf2f(sbits);
                if (s == 0.0f) {
                    s = 1.0f;
                    sbits = 0x3F80u;
                }
            } else if (s == 0.0f) {
                s = 1.0f;
            }
            const float inv = 1.0f / s;
            float zf = 0.0f;
            if (!q.sym) zf = fminf(fmaxf(rintf(fmaxf(r1, 0.0f) / s), 0.0f), 15.0f);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int jj = k * G + j;
                uint32_t c;
                if (q.sym) {
                    const float t = fminf(fmaxf(rintf(y[jj] * inv), -8.0f), 7.0f);
                    c = static_cast<uint32_t>(static_cast<int>(t)) & 0xFu;
                } else {
                    const float t = fminf(fmaxf(rintf(y[jj] * inv) + zf, 0.0f), 15.0f);
                    c = static_cast<uint32_t>(static_cast<int>(t));
                }
                w[jj >> 3] |= c << (4 * (jj & 7));
            }
            zq[k] = static_cast<uint32_t>(static_cast<int>(zf));
            if (valid) {
                if (q.scale_dtype == 1)
                    static_cast<uint16_t*>(q.scales)[G0 + k] = static_cast<uint16_t>(sbits);
                else
                    static_cast<float*>(q.scales)[G0 + k] = s;
            }
        }
    }
    if (valid && q.format == 0 && !q.sym) {
#pragma unroll
        for (int k = 0; k < NG; k += 2) q.zeros[(G0 + k) >> 1] = static_cast<uint8_t>((zq[k] & 0xFu) | ((zq[k + 1] & 0xFu) << 4));
    }
    if (valid) store_codes<E>(q.codes, e0, w);
}

template <int LOGE>
__device__ __forceinline__ void quantize_multi_any(const float (&y)[1 << LOGE], const QuantDev& q, bool valid,
                                                   int64_t e0) {
    if constexpr (LOGE >= 4) {
        switch (q.logg) {
            case 1: quantize_multi<LOGE, 1>(y, q, valid, e0); break;
            case 2: quantize_multi<LOGE, 2>(y, q, valid, e0); break;
            case 3: quantize_multi<LOGE, 3>(y, q, valid, e0); break;
            default:
                if constexpr (LOGE >= 5) quantize_multi<LOGE, 4>(y, q, valid, e0);
                break;
        }
    }
}

template <int LOGE>
__device__ __forceinline__ void quantize(const float (&y)[1 << LOGE], const QuantDev& q, int64_t total_groups,
                                         int tid, int nt, bool valid, int64_t e0, int64_t wg_e0,
                                         float* red, int* zst) {
    constexpr int E = 1 << LOGE;
    if (q.logg < LOGE) {           // several groups per thread (uniform over the workgroup)
        quantize_multi_any<LOGE>(y, q, valid, e0);
        return;
    }
    const int gl = q.logg - LOGE;  // log2(threads per group), >= 0
    const int gth = 1 << gl;

    // per-thread partial statistics: r0 = max y, r1 = max(-y)
    float r0 = y[0];
    float r1 = -y[0];
#pragma unroll
    for (int j = 1; j < E; ++j) {
        r0 = fmaxf(r0, y[j]);
        r1 = fmaxf(r1, -y[j]);
    }
    for (int m = 1; m < gth && m < 64; m <<= 1) {
        r0 = fmaxf(r0, __shfl_xor(r0, m));
        r1 = fmaxf(r1, __shfl_xor(r1, m));
    }
    if (gth > 64) {
        const int wave = tid >> 6;
        __syncthreads();
        if ((tid & 63) == 0) {
            red[2 * wave] = r0;
            red[2 * wave + 1] = r1;
        }
        __syncthreads();
        const int wpg = gth >> 6;
        const int w0 = wave & ~(wpg - 1);
        r0 = red[2 * w0];
        r1 = red[2 * w0 + 1];
        for (int k = 1; k < wpg; ++k) {
            r0 = fmaxf(r0, red[2 * (w0 + k)]);
            r1 = fmaxf(r1, red[2 * (w0 + k) + 1]);
        }
    }
    const bool leader = valid && ((tid & (gth - 1)) == 0);
    const int64_t G = e0 >> q.logg;

    uint32_t w[(E + 7) / 8];
#pragma unroll
    for (int k = 0; k < (E + 7) / 8; ++k) w[k] = 0u;

    if (q.format == 1) {
        // MXFP4: shared exponent e = floor(log2 amax) - 2, E2M1 elements
        const float amax = fmaxf(r0, r1);
        const int ex = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
        int e = (ex == 0) ? -127 : ex - 127 - 2;
        e = max(-127, min(127, e));
        const float sc = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);  // 2^-e
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float v = y[j] * sc;
            const float a = fabsf(v);
            // nearest E2M1 magnitude, ties to the even index
            uint32_t idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                           (a >= 3.5f) + (a > 5.0f);
            idx |= (y[j] < 0.0f) ? 8u : 0u;
            w[j >> 3] |= idx << (4 * (j & 7));
        }
        if (leader) static_cast<uint8_t*>(q.scales)[G] = static_cast<uint8_t>(e + 127);
    } else if (q.format == 2) {
        // NVFP4: E4M3 block scale of amax / (6 g); E2M1 elements of y / s with
        // s = E4M3 g; a zero scale leaves every code 0
        const float amax = fmaxf(r0, r1);
        const uint32_t byte = e4m3_byte(amax / (6.0f * q.tscale));
        const float s = e4m3_value(byte) * q.tscale;
        if (s > 0.0f) {
            const float inv = 1.0f / s;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float a = fabsf(y[j] * inv);
                uint32_t idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                               (a >= 3.5f) + (a > 5.0f);
                idx |= (y[j] < 0.0f) ? 8u : 0u;
                w[j >> 3] |= idx << (4 * (j & 7));
            }
        }
        if (leader) static_cast<uint8_t*>(q.scales)[G] = static_cast<uint8_t>(byte);
    } else {
        float s;
        float zf = 0.0f;
        if (q.sym) {
            s = fmaxf(r0, r1) / 7.0f;
        } else {
            const float hi = fmaxf(r0, 0.0f);
            const float lo = -fmaxf(r1, 0.0f);
            s = (hi - lo) / 15.0f;
        }
        uint32_t sbits = 0;
        if (q.scale_dtype == 1) {
            sbits = f2bf(s);
            s = bf2f(sbits);
            if (s == 0.0f) {
                s = 1.0f;
                sbits = 0x3F80u;
            }
        } else if (s == 0.0f) {
            s = 1.0f;
        }
        const float inv = 1.0f / s;
        if (q.sym) {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                float t = rintf(y[j] * inv);
                t = fminf(fmaxf(t, -8.0f), 7.0f);
                w[j >> 3] |= (static_cast<uint32_t>(static_cast<int>(t)) & 0xFu) << (4 * (j & 7));
            }
        } else {
            const float lo = -fmaxf(r1, 0.0f);
            zf = fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
#pragma unroll
            for (int j = 0; j < E; ++j) {
                float t = rintf(y[j] * inv) + zf;
                t = fminf(fmaxf(t, 0.0f), 15.0f);
                w[j >> 3] |= static_cast<uint32_t>(static_cast<int>(t)) << (4 * (j & 7));
            }
        }
        if (leader) {
            if (q.scale_dtype == 1)
                static_cast<uint16_t*>(q.scales)[G] = static_cast<uint16_t>(sbits);
            else
                static_cast<float*>(q.scales)[G] = s;
        }
        if (!q.sym) {
            // zero points: uint4, two per byte over the flattened group index;
            // every workgroup owns an even number of groups starting at an
            // even index, so it writes whole bytes.
            const int ngwg = (nt * E) >> q.logg;
            __syncthreads();
            if ((tid & (gth - 1)) == 0) zst[(tid * E) >> q.logg] = static_cast<int>(zf);
            __syncthreads();
            const int64_t G0 = wg_e0 >> q.logg;
            if (tid < (ngwg >> 1)) {
                const int64_t g = G0 + 2 * tid;
                if (g < total_groups) {
                    uint32_t b = static_cast<uint32_t>(zst[2 * tid]) & 0xFu;
                    if (g + 1 < total_groups) b |= (static_cast<uint32_t>(zst[2 * tid + 1]) & 0xFu) << 4;
                    q.zeros[g >> 1] = static_cast<uint8_t>(b);
                }
            }
        }
    }
    if (valid) store_codes<E>(q.codes, e0, w);
}

template <int LOGE, bool BF16, int KMAX>
__global__ void __launch_bounds__(1024) rot_kernel(const RotArgs a) {
    constexpr int E = 1 << LOGE;
    extern __shared__ float smem[];
    const int tid = static_cast<int>(threadIdx.x);
    const int nt = static_cast<int>(blockDim.x);
    float* lds = smem;
    float* lds2 = smem + lpad(nt * E);                          // wide Kronecker mix only
    float* red = lds2 + (KMAX < 0 ? lpad(nt * E) : 0);
    int* zst = reinterpret_cast<int*>(red + 2 * (nt / 64 + 1));

    const int cl = tid / a.tpc;
    const int lt = tid - cl * a.tpc;
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * a.cpw + cl;
    const bool valid = chunk < a.total_chunks;
    const int64_t e0 = chunk * a.chunk + static_cast<int64_t>(lt) * E;
    const int64_t wg_e0 = static_cast<int64_t>(blockIdx.x) * a.cpw * a.chunk;

    float v[E];
    // randomised rotation: the thread's E elements lie in one row
    const int64_t col0 = valid && (a.perm || a.in_signs || a.out_signs) ? e0 % a.row_n : 0;
    if (valid) {
        if (a.perm) {
            const int64_t rs = e0 - col0;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                int64_t src = a.perm[col0 + j];
                src = src < 0 ? 0 : (src >= a.row_n ? a.row_n - 1 : src);
                v[j] = load_one<BF16>(a.x, rs + src);
            }
        } else {
            load_vals<E, BF16>(a.x, e0, v);
        }
        if (a.in_signs) {
#pragma unroll
            for (int j = 0; j < E; ++j)
                if (a.in_signs[col0 + j] < 0) v[j] = -v[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = 0.0f;
    }
    fwht<LOGE>(v, lds, tid, a.logb);
    if constexpr (KMAX > 0) kron_mix<LOGE, KMAX>(v, lds, tid, a);
    if constexpr (KMAX < 0) kron_mix_wide<LOGE>(v, lds, lds2, tid, a);
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] *= a.norm;
    if (a.out_signs && valid) {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (a.out_signs[col0 + j] < 0) v[j] = -v[j];
    }
    if (a.y_rot != nullptr && valid) store_vals<E, BF16>(a.y_rot, e0, v);
    for (int i = 0; i < a.nq; ++i)
        quantize<LOGE>(v, a.q[i], a.total_groups[i], tid, nt, valid, e0, wg_e0, red, zst);
}

// ------------------------------------------------------------ dequantization

__device__ __forceinline__ float e2m1_mag(uint32_t idx) {
    // {0, 0.5, 1, 1.5, 2, 3, 4, 6}
    const float t[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    return t[idx & 7u];
}

// Dequantizes (and, with a.parts, measures against a.ref) the code bytes of
// a grid-stride range; each workgroup writes one partial of its statistics.
__global__ void __launch_bounds__(256) dequant_kernel(const DqArgs a) {
    double se2 = 0.0, sr2 = 0.0;
    unsigned long long nover = 0, nclamp = 0;
    float mx = 0.0f;
    const int64_t bytes = (a.total + 1) / 2;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < bytes;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const uint32_t byte = a.codes[i];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t e = 2 * i + h;
            if (e >= a.total) break;
            const uint32_t c = (byte >> (4 * h)) & 0xFu;
            const int64_t G = e >> a.logg;
            float deq, step, lo_lim = 0.0f, hi_lim = 0.0f, s = 1.0f, z = 0.0f;
            int ee = 0;
            if (a.format == 1) {
                ee = static_cast<int>(static_cast<const uint8_t*>(a.scales)[G]) - 127;
                const float m = e2m1_mag(c);
                deq = ldexpf((c & 8u) ? -m : m, ee);
                step = 0.0f;  // set below from the reference
            } else if (a.format == 2) {
                s = e4m3_value(static_cast<const uint8_t*>(a.scales)[G]) * a.tscale;
                const float m = e2m1_mag(c);
                deq = ((c & 8u) ? -m : m) * s;
                step = 0.0f;  // set below from the reference
            } else {
                s = (a.scale_dtype == 1) ? bf2f(static_cast<const uint16_t*>(a.scales)[G])
                                         : static_cast<const float*>(a.scales)[G];
                if (a.sym) {
                    const int qv = static_cast<int>(c) - ((c & 8u) ? 16 : 0);
                    deq = static_cast<float>(qv) * s;
                    lo_lim = -8.5f;
                    hi_lim = 7.5f;
                } else {
                    const uint32_t zb = a.zeros[G >> 1];
                    z = static_cast<float>((zb >> (4 * (G & 1))) & 0xFu);
                    deq = (static_cast<float>(c) - z) * s;
                    lo_lim = -0.5f;
                    hi_lim = 15.5f;
                }
                step = s;
            }
            if (a.deq) a.deq[e] = deq;
            if (a.parts) {
                const float r = a.ref_bf16 ? bf2f(static_cast<const uint16_t*>(a.ref)[e])
                                           : static_cast<const float*>(a.ref)[e];
                bool clamped;
                if (a.format == 1) {
                    const float v = fabsf(ldexpf(r, -ee));
                    const float sp = (v < 2.0f) ? 0.5f : ((v < 4.0f) ? 1.0f : 2.0f);
                    step = ldexpf(sp, ee);
                    clamped = v > 6.0f;
                } else if (a.format == 2) {
                    // a zero block scale is measured against the smallest one, 2^-9 g
                    const float sb = s > 0.0f ? s : 0.001953125f * a.tscale;
                    const float v = fabsf(r) / sb;
                    const float sp = (v < 2.0f) ? 0.5f : ((v < 4.0f) ? 1.0f : 2.0f);
                    step = sp * sb;
                    clamped = v > 6.0f;
                } else {
                    const float t = r / s + z;
                    clamped = (t < lo_lim) || (t > hi_lim);
                }
                const float err = fabsf(r - deq);
                const float es = err / step;
                mx = fmaxf(mx, es);
                nover += (err > 0.5f * step) ? 1ull : 0ull;
                nclamp += clamped ? 1ull : 0ull;
                se2 += static_cast<double>(err) * err;
                sr2 += static_cast<double>(r) * r;
            }
        }
    }
    if (a.parts) {
        // wave reduction, then the four waves in order: one partial per workgroup
        for (int m = 32; m >= 1; m >>= 1) {
            se2 += __shfl_xor(se2, m);
            sr2 += __shfl_xor(sr2, m);
            nover += __shfl_xor(nover, m);
            nclamp += __shfl_xor(nclamp, m);
            mx = fmaxf(mx, __shfl_xor(mx, m));
        }
        __shared__ DqPartial wsum[4];
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) wsum[w] = DqPartial{se2, sr2, nover, nclamp, mx, 0u};
        __syncthreads();
        if (threadIdx.x == 0) {
            DqPartial t = wsum[0];
            for (int k = 1; k < 4; ++k) {
                t.sum_err2 += wsum[k].sum_err2;
                t.sum_ref2 += wsum[k].sum_ref2;
                t.n_over += wsum[k].n_over;
                t.n_clamped += wsum[k].n_clamped;
                t.max_err = fmaxf(t.max_err, wsum[k].max_err);
            }
            static_cast<DqPartial*>(a.parts)[blockIdx.x] = t;
        }
    }
}

// Sums the `nparts` partials of dequant_kernel in a fixed order into slot
// kDqMaxParts (one workgroup of 64 threads).
__global__ void __launch_bounds__(64) dequant_finish(DqPartial* parts, int nparts) {
    const int t = threadIdx.x;
    DqPartial acc{0.0, 0.0, 0ull, 0ull, 0.0f, 0u};
    for (int i = t; i < nparts; i += 64) {
        const DqPartial p = parts[i];
        acc.sum_err2 += p.sum_err2;
        acc.sum_ref2 += p.sum_ref2;
        acc.n_over += p.n_over;
        acc.n_clamped += p.n_clamped;
        acc.max_err = fmaxf(acc.max_err, p.max_err);
    }
    for (int m = 32; m >= 1; m >>= 1) {
        acc.sum_err2 += __shfl_xor(acc.sum_err2, m);
        acc.sum_ref2 += __shfl_xor(acc.sum_ref2, m);
        acc.n_over += __shfl_xor(acc.n_over, m);
        acc.n_clamped += __shfl_xor(acc.n_clamped, m);
        acc.max_err = fmaxf(acc.max_err, __shfl_xor(acc.max_err, m));
    }
    if (t == 0) parts[kDqMaxParts] = acc;
}

template <int LOGE, bool BF16, int KMAX>
hipError_t launch_inst(const RotPlan& p, hipStream_t s) {
    auto fn = rot_kernel<LOGE, BF16, KMAX>;
    if (p.lds_bytes > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(p.lds_bytes));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(p.grid)), dim3(p.nt), p.lds_bytes, s, p.a);
    return hipGetLastError();
}

template <int LOGE, bool BF16>
hipError_t launch_k(const RotPlan& p, hipStream_t s) {
    if constexpr (LOGE >= 3) {
        switch (p.kmax) {
            case 16: return launch_inst<LOGE, BF16, 16>(p, s);
            case 32: return launch_inst<LOGE, BF16, 32>(p, s);
            case 64: return launch_inst<LOGE, BF16, 64>(p, s);
            case -1: return launch_inst<LOGE, BF16, -1>(p, s);
            default: break;
        }
    }
    if (p.kmax != 0) return hipErrorInvalidValue;
    return launch_inst<LOGE, BF16, 0>(p, s);
}

template <bool BF16>
hipError_t launch_e(const RotPlan& p, hipStream_t s) {
    switch (p.loge) {
        case 1: return launch_k<1, BF16>(p, s);
        case 2: return launch_k<2, BF16>(p, s);
        case 3: return launch_k<3, BF16>(p, s);
        case 4: return launch_k<4, BF16>(p, s);
        case 5: return launch_k<5, BF16>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int launch_rotate(const RotPlan& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return static_cast<int>(p.bf16 ? launch_e<true>(p, s) : launch_e<false>(p, s));
}

// Scratch of dequant_check_noalloc: the statistics partials, one copy per
// device, held until the process ends.  In host code `scratch` is only a
// handle for hipGetSymbolAddress; kernels get the device address from
// scratch_address().
static __device__ __align__(256) unsigned char scratch[kDqScratchBytes];

int scratch_address(void** out) {
    static std::atomic<void*> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        // with the device current: each device holds its own copy
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return static_cast<int>(e);
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return 0;
}

int launch_dequant(const DqArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t bytes = (a.total + 1) / 2;
    int64_t grid = (bytes + 255) / 256;
    if (grid > kDqMaxParts) grid = kDqMaxParts;   // grid-stride beyond that
    hipLaunchKernelGGL(dequant_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.parts) return static_cast<int>(e);
    hipLaunchKernelGGL(dequant_finish, dim3(1), dim3(64), 0, s, static_cast<DqPartial*>(a.parts),
                       static_cast<int>(grid));
    return static_cast<int>(hipGetLastError());
}

}  // namespace hr
