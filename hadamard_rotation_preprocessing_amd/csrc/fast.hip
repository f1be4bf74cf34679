// Specialised bfloat16 kernels for gfx950: every shape parameter is a
// compile-time constant, one wave owns whole Hadamard blocks, and there is
// no workgroup barrier.
//
// The Sylvester transform of a block (AutoRound "Rotation Transform",
// section 1.5: H_{2k} = [[H_k, H_k], [H_k, -H_k]], natural order) is a tensor
// product of 2x2 butterflies over the index bits, so the bits can be taken in
// any order and by any mechanism:
//   * four bits by one MFMA: a lane's four loaded bf16 values are one column
//     of the B operand of v_mfma_f32_16x16x16_bf16, the A operand is H_16
//     (entries +-1), so D = H_16 . X transforms four index bits exactly
//     (bf16 products with +-1 are exact, accumulation is float32) and leaves
//     every result in the lane and register position of its input;
//   * bits held in registers: butterflies a +- b;
//   * lane bits: DPP quad permutations (partner + sign * own);
//   * otherwise an in-wave transpose through a small padded LDS buffer.
//
// kwave<LOGB>: one wave per block of 2^LOGB (2048 or 4096) elements.
// k128: eight rows of 128 elements per wave; no LDS at all.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace hr {
namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// fma(y, c, kMagic) = kMagic + rne(y * c) for |y * c| < 2^22: the rounded
// integer sits in the low mantissa bits (one rounding of the exact product).
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

constexpr int kXor1 = 0xB1;        // DPP quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // DPP quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kMirror = 0x140;     // lane i <-> 15 - i within 16

template <int FMT, int SYM, int LOGG, int SDT>
struct QD {
    static constexpr int fmt = FMT, sym = SYM, logg = LOGG, sdt = SDT;
};
using QNone = QD<-1, 0, 0, 0>;

__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ u32x4_t ldg16(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void stg16(void* p, u32x4_t v) {
    __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
}

// A operand H_16: lane l holds H_16[l % 16][4 (l / 16) + t], t = 0..3.
__device__ __forceinline__ bf16x4_t h16_operand(int lane) {
    const int i = lane & 15;
    bf16x4_t h;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k = 4 * (lane >> 4) + t;
        h[t] = (__popc(i & k) & 1) ? static_cast<short>(0xBF80) : static_cast<short>(0x3F80);
    }
    return h;
}

// Transform of the four index bits (k & 3 within the lane, k >> 2 across
// lanes l, l + 16, l + 32, l + 48) of the four bf16 values in (lo, hi).
__device__ __forceinline__ f32x4_t mfma_h16(bf16x4_t h, uint32_t lo, uint32_t hi) {
    const u32x2_t u = {lo, hi};
    const bf16x4_t b = __builtin_bit_cast(bf16x4_t, u);
    const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(h, b, z, 0, 0, 0);
}

template <int N, unsigned MASK>
__device__ __forceinline__ void bfly(float (&v)[N]) {
#pragma unroll
    for (int k = 0; (1 << k) < N; ++k) {
        if (MASK & (1u << k)) {
#pragma unroll
            for (int j = 0; j < N; ++j) {
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

// Butterfly across a lane bit: lane with the bit clear gets own + partner,
// lane with the bit set gets partner - own (sgn = -1 there).
template <int CTRL, int N>
__device__ __forceinline__ void dpp_bfly(float (&v)[N], float sgn) {
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = fmaf(sgn, v[j], dpp<CTRL>(v[j]));
}

// Maximum over aligned groups of GL consecutive lanes.
template <int GL>
__device__ __forceinline__ float lanes_max(float v) {
    if constexpr (GL >= 2) v = fmaxf(v, dpp<kXor1>(v));
    if constexpr (GL >= 4) v = fmaxf(v, dpp<kXor2>(v));
    if constexpr (GL >= 8) v = fmaxf(v, dpp<kHalfMirror>(v));
    if constexpr (GL >= 16) v = fmaxf(v, dpp<kMirror>(v));
    if constexpr (GL >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (GL >= 64) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Eight rounded codes (floats kMagic + offset + q, offset + q in 0..15)
// -> eight nibbles, element 0 in the low nibble.
__device__ __forceinline__ uint32_t pack8(const float* t) {
    const uint32_t a0 = __float_as_uint(t[0]) | (__float_as_uint(t[1]) << 4) |
                        (__float_as_uint(t[2]) << 8) | (__float_as_uint(t[3]) << 12);
    const uint32_t a1 = __float_as_uint(t[4]) | (__float_as_uint(t[5]) << 4) |
                        (__float_as_uint(t[6]) << 8) | (__float_as_uint(t[7]) << 12);
    return __builtin_amdgcn_perm(a1, a0, 0x05040100u);
}

__device__ __forceinline__ uint32_t bf16x2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

// E2M1 code of v (already divided by the shared scale): nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6} with ties to the even index, saturating; sign
// set iff v < 0.  Used only for groups whose scale is 2^-127.
__device__ __forceinline__ uint32_t e2m1_soft(float v) {
    const float a = fabsf(v);
    uint32_t i = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return i | ((v < 0.0f) ? 8u : 0u);
}

// ------------------------------------------------------------ INT epilogue
// u[0..E) are the lane's E contiguous elements of one group of G >= E
// elements spread over GL = G / E lanes; y = u * f.
template <int E, class Q>
__device__ __forceinline__ void epi_int(const float (&u)[E], float f, const QuantDev& q, int64_t e0, bool valid,
                                        int lane, int64_t total_groups) {
    constexpr int G = 1 << Q::logg;
    static_assert(G >= E, "group spans whole lanes");
    constexpr int GL = G / E;
    float s, zf = 0.0f;
    if constexpr (Q::sym) {
        float am = fabsf(u[0]);
#pragma unroll
        for (int j = 1; j < E; ++j) am = fmaxf(am, fabsf(u[j]));
        am = lanes_max<GL>(am);
        s = (am * f) / 7.0f;
    } else {
        float hi = u[0], nl = -u[0];
#pragma unroll
        for (int j = 1; j < E; ++j) {
            hi = fmaxf(hi, u[j]);
            nl = fmaxf(nl, -u[j]);
        }
        hi = fmaxf(lanes_max<GL>(hi), 0.0f) * f;
        nl = fmaxf(lanes_max<GL>(nl), 0.0f) * f;  // -min(min y, 0)
        s = (hi + nl) / 15.0f;
        zf = nl;
    }
    uint32_t sbits = 0;
    if constexpr (Q::sdt == 1) {
        sbits = f2bf(s);
        s = bf2f(sbits);
        if (s == 0.0f) {
            s = 1.0f;
            sbits = 0x3F80u;
        }
    } else if (s == 0.0f) {
        s = 1.0f;
    }
    const float inv = f / s;
    uint32_t w[E / 8];
    if constexpr (Q::sym) {
        // |y| <= amax and s >= amax / 7 (1 - 2^-8): rne(y / s) stays in [-7, 7],
        // so no clamp is needed; +8 makes every nibble non-negative, and the
        // two's complement nibble is recovered by flipping its top bit.
        const float off = kMagic + 8.0f;
#pragma unroll
        for (int b = 0; b < E / 8; ++b) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = fmaf(u[8 * b + j], inv, off);
            w[b] = pack8(t) ^ 0x88888888u;
        }
    } else {
        const float z = fminf(fmaxf(rintf(zf / s), 0.0f), 15.0f);
        // clamp(rne(y / s) + z, 0, 15): round on y / s alone (ties to even
        // there), clamp to [-z, 15 - z], then add z as an integer.
        const uint32_t zi = static_cast<uint32_t>(z);
        const float lo = kMagic - z, hi = kMagic + 15.0f - z;
#pragma unroll
        for (int b = 0; b < E / 8; ++b) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float r = __builtin_amdgcn_fmed3f(fmaf(u[8 * b + j], inv, kMagic), lo, hi);
                t[j] = __uint_as_float(__float_as_uint(r) + zi);
            }
            w[b] = pack8(t);
        }
        // zero points: group pairs (2i, 2i + 1) -> one byte, written by the
        // first lane of the even group
        uint32_t zn = zi;
        uint32_t zodd;
        if constexpr (GL == 1) zodd = dppu<kXor1>(zn);
        else if constexpr (GL == 2) zodd = dppu<kXor2>(zn);
        else if constexpr (GL == 4) zodd = dppu<kHalfMirror>(zn);
        else if constexpr (GL == 8) zodd = dppu<kMirror>(zn);
        else zodd = static_cast<uint32_t>(__shfl_xor(static_cast<int>(zn), GL));
        const int64_t gidx = e0 >> Q::logg;
        if (valid && (lane & (2 * GL - 1)) == 0 && gidx < total_groups) {
            uint32_t byte = zn & 0xFu;
            if (gidx + 1 < total_groups) byte |= (zodd & 0xFu) << 4;
            q.zeros[gidx >> 1] = static_cast<uint8_t>(byte);
        }
    }
    if (valid) {
        uint8_t* cp = q.codes + (e0 >> 1);
        if constexpr (E / 8 == 8) {
            stg16(cp, u32x4_t{w[0], w[1], w[2], w[3]});
            stg16(cp + 16, u32x4_t{w[4], w[5], w[6], w[7]});
        } else if constexpr (E / 8 == 4) {
            stg16(cp, u32x4_t{w[0], w[1], w[2], w[3]});
        } else {
#pragma unroll
            for (int b = 0; b < E / 8; ++b) reinterpret_cast<uint32_t*>(cp)[b] = w[b];
        }
        if ((lane & (GL - 1)) == 0) {
            const int64_t gidx = e0 >> Q::logg;
            if constexpr (Q::sdt == 1)
                static_cast<uint16_t*>(q.scales)[gidx] = static_cast<uint16_t>(sbits);
            else
                static_cast<float*>(q.scales)[gidx] = s;
        }
    }
}

// ----------------------------------------------------------- MXFP4 epilogue
// y[0..E) contiguous normalised values, E a multiple of 32.
template <int E>
__device__ __forceinline__ void epi_mxfp4(const float (&y)[E], const QuantDev& q, int64_t e0, bool valid) {
    static_assert(E % 32 == 0, "whole MX blocks per lane");
    constexpr int NB = E / 32;
    uint32_t w[E / 8];
    uint32_t ebytes = 0;
#pragma unroll
    for (int g = 0; g < NB; ++g) {
        float am = fabsf(y[32 * g]);
#pragma unroll
        for (int j = 1; j < 32; ++j) am = fmaxf(am, fabsf(y[32 * g + j]));
        const int ex = static_cast<int>((__float_as_uint(am) >> 23) & 0xFFu);
        const int e = (ex == 0) ? -127 : ex - 129;  // floor(log2 amax) - 2, >= -127
        ebytes |= static_cast<uint32_t>(e + 127) << (8 * g);
        if (e > -127) {
            // the converter divides by the scale, rounds to nearest even
            // and saturates at +-6
            const float sc = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t r = 0;
                r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[32 * g + 8 * d + 0], y[32 * g + 8 * d + 1], sc, 0);
                r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[32 * g + 8 * d + 2], y[32 * g + 8 * d + 3], sc, 1);
                r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[32 * g + 8 * d + 4], y[32 * g + 8 * d + 5], sc, 2);
                r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[32 * g + 8 * d + 6], y[32 * g + 8 * d + 7], sc, 3);
                w[4 * g + d] = r;
            }
        } else {
            // scale 2^-127 (amax below 2^-124): scale by 2^127 in software
            const float up = __uint_as_float(254u << 23);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t r = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) r |= e2m1_soft(y[32 * g + 8 * d + j] * up) << (4 * j);
                w[4 * g + d] = r;
            }
        }
    }
    if (valid) {
        uint8_t* cp = q.codes + (e0 >> 1);
#pragma unroll
        for (int b = 0; b < E / 32; ++b) stg16(cp + 16 * b, u32x4_t{w[4 * b], w[4 * b + 1], w[4 * b + 2], w[4 * b + 3]});
        uint8_t* sp = static_cast<uint8_t*>(q.scales) + (e0 >> 5);
        if constexpr (NB == 2)
            *reinterpret_cast<uint16_t*>(sp) = static_cast<uint16_t>(ebytes);
        else
            *sp = static_cast<uint8_t>(ebytes);
    }
}

template <int E, class Q>
__device__ __forceinline__ void epilogue(const float (&u)[E], float f, const QuantDev& q, int64_t e0, bool valid,
                                         int lane, int64_t total_groups) {
    if constexpr (Q::fmt == 0) {
        epi_int<E, Q>(u, f, q, e0, valid, lane, total_groups);
    } else if constexpr (Q::fmt == 1) {
        epi_mxfp4<E>(u, q, e0, valid);  // caller passes normalised values
    }
}

// ---------------------------------------------------------------- kwave

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int LOGB>
struct KW {
    static constexpr int B = 1 << LOGB;
    static constexpr int E = B / 64;          // elements per lane: 32 or 64
    static constexpr int NC = E / 8;          // 16-byte chunks per lane
    static constexpr int NS = E / 16;         // transpose passes
    static constexpr int R = 8 / NS;          // chunk elements per pass
    static constexpr int LW = B / NS;         // elements per pass
    static constexpr int LDS = LW + (LW >> 5) + 1;
    static_assert(LW <= 1024, "padding formula assumes passes of at most 1024 elements");
};

// One wave per block of B = 2^LOGB elements (bf16 in).  Load layout L0:
// element e = 512 c + 8 lane + r (chunk c, r = 0..7).  The MFMA transforms
// bits {0, 1, 7, 8}; register butterflies bits 2 and 9.. ; an LDS transpose
// (in NS passes over r) gives each lane E contiguous elements; bits 3..6 are
// then register bits (below log2 E) or lane bits (DPP).
template <int LOGB, bool WROT, class Q0, class Q1>
__global__ void __launch_bounds__(256) kwave(const FastArgs a) {
    using K = KW<LOGB>;
    constexpr int B = K::B, E = K::E, NC = K::NC, NS = K::NS, R = K::R;
    constexpr int LOGE = (E == 64) ? 6 : 5;
    __shared__ float lds_all[4][K::LDS];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + wv;
    if (blk >= a.units) return;  // whole wave idle; no barrier follows
    float* lds = lds_all[wv];
    const uint16_t* src = static_cast<const uint16_t*>(a.x) + blk * B;

    u32x4_t raw[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] = ldg16(src + 512 * c + 8 * lane);

    const bf16x4_t hop = h16_operand(lane);
    float v[E];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4_t d0 = mfma_h16(hop, raw[c][0], raw[c][1]);
        const f32x4_t d1 = mfma_h16(hop, raw[c][2], raw[c][3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * c + j] = d0[j];
            v[8 * c + 4 + j] = d1[j];
        }
    }
    // register bits of L0: v-index bit 2 (e bit 2) and bits 3.. (e bits 9..)
    bfly<E, ~3u & (E - 1)>(v);

    // transpose L0 -> lane-contiguous, in NS passes over r
    float y[E];
    const int wbase = lane * R + ((lane * R) >> 5);
    const int rbase = 16 * lane + (lane >> 1);
#pragma unroll
    for (int p = 0; p < NS; ++p) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int rr = 0; rr < R; ++rr) lds[wbase + 64 * c * R + 2 * c * R + rr] = v[8 * c + p * R + rr];
        wave_sync();
#pragma unroll
        for (int jj = 0; jj < E / 8; ++jj)
#pragma unroll
            for (int rr = 0; rr < R; ++rr) y[8 * jj + p * R + rr] = lds[rbase + jj * R + rr];
        wave_sync();
    }
    // bits 3..6: registers below LOGE, lane bits from LOGE on
    constexpr unsigned regmask = (0x78u) & ((1u << LOGE) - 1u);
    bfly<E, regmask>(y);
    if constexpr (LOGE <= 5) dpp_bfly<kXor1>(y, (lane & 1) ? -1.0f : 1.0f);      // bit 5
    if constexpr (LOGE <= 6) {
        if constexpr (LOGE == 5) dpp_bfly<kXor2>(y, (lane & 2) ? -1.0f : 1.0f);  // bit 6
        else dpp_bfly<kXor1>(y, (lane & 1) ? -1.0f : 1.0f);                      // bit 6
    }

    const int64_t e0 = blk * B + static_cast<int64_t>(E) * lane;
    constexpr bool need_y = WROT || Q0::fmt == 1 || Q1::fmt == 1;
    float f = a.norm;
    if constexpr (need_y) {
#pragma unroll
        for (int j = 0; j < E; ++j) y[j] *= a.norm;
        f = 1.0f;
    }
    if constexpr (WROT) {
        uint16_t* dst = static_cast<uint16_t*>(a.y_rot) + e0;
#pragma unroll
        for (int b = 0; b < E / 8; ++b)
            stg16(dst + 8 * b, u32x4_t{bf16x2(y[8 * b], y[8 * b + 1]), bf16x2(y[8 * b + 2], y[8 * b + 3]),
                                       bf16x2(y[8 * b + 4], y[8 * b + 5]), bf16x2(y[8 * b + 6], y[8 * b + 7])});
    }
    if constexpr (Q0::fmt >= 0) epilogue<E, Q0>(y, f, a.q[0], e0, true, lane, a.total_groups[0]);
    if constexpr (Q1::fmt >= 0) epilogue<E, Q1>(y, f, a.q[1], e0, true, lane, a.total_groups[1]);
}

// ----------------------------------------------------------------- k128
// Eight rows of 128 per wave.  Lane l: n = l % 16, row = n >> 1, h = n & 1,
// q = l >> 4; chunk c in {0, 1} holds row elements 64 c + 32 h + 8 q + r.
// The MFMA transforms bits {0, 1, 3, 4}, registers bits 2 and 6, the DPP
// butterfly bit 5.  The 128 elements of a row sit in the 8 lanes sharing n >> 1.
template <bool WROT, class Q0>
__global__ void __launch_bounds__(256) k128(const FastArgs a) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n = lane & 15;
    const int h = n & 1;
    const int qq = lane >> 4;
    const int64_t row = (static_cast<int64_t>(blockIdx.x) * 4 + wv) * 8 + (n >> 1);
    const bool valid = row < a.units;
    const int col0 = 32 * h + 8 * qq;  // element of chunk 0 within the row
    const uint16_t* src = static_cast<const uint16_t*>(a.x) + row * 128 + col0;
    u32x4_t raw[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        if (valid) raw[c] = ldg16(src + 64 * c);
        else raw[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
    const bf16x4_t hop = h16_operand(lane);
    float v[16];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const f32x4_t d0 = mfma_h16(hop, raw[c][0], raw[c][1]);
        const f32x4_t d1 = mfma_h16(hop, raw[c][2], raw[c][3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * c + j] = d0[j];
            v[8 * c + 4 + j] = d1[j];
        }
    }
    bfly<16, 0xCu>(v);                           // bits 2 (v-index bit 2) and 6 (v-index bit 3)
    dpp_bfly<kXor1>(v, h ? -1.0f : 1.0f);        // bit 5
    const int64_t e0 = row * 128 + col0;

    if constexpr (WROT) {
        uint16_t* dst = static_cast<uint16_t*>(a.y_rot) + e0;
        float y[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = v[j] * a.norm;
        if (valid) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
                stg16(dst + 64 * c, u32x4_t{bf16x2(y[8 * c], y[8 * c + 1]), bf16x2(y[8 * c + 2], y[8 * c + 3]),
                                            bf16x2(y[8 * c + 4], y[8 * c + 5]), bf16x2(y[8 * c + 6], y[8 * c + 7])});
        }
    }
    if constexpr (Q0::fmt == 0) {
        static_assert(Q0::logg == 7, "one group per row");
        const float f = a.norm;
        float s, zf = 0.0f;
        if constexpr (Q0::sym) {
            float am = fabsf(v[0]);
#pragma unroll
            for (int j = 1; j < 16; ++j) am = fmaxf(am, fabsf(v[j]));
            am = fmaxf(am, dpp<kXor1>(am));
            am = fmaxf(am, __shfl_xor(am, 16));
            am = fmaxf(am, __shfl_xor(am, 32));
            s = (am * f) / 7.0f;
        } else {
            float hi = v[0], nl = -v[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) {
                hi = fmaxf(hi, v[j]);
                nl = fmaxf(nl, -v[j]);
            }
            hi = fmaxf(hi, dpp<kXor1>(hi));
            nl = fmaxf(nl, dpp<kXor1>(nl));
            hi = fmaxf(hi, __shfl_xor(hi, 16));
            nl = fmaxf(nl, __shfl_xor(nl, 16));
            hi = fmaxf(hi, __shfl_xor(hi, 32));
            nl = fmaxf(nl, __shfl_xor(nl, 32));
            hi = fmaxf(hi, 0.0f) * f;
            nl = fmaxf(nl, 0.0f) * f;
            s = (hi + nl) / 15.0f;
            zf = nl;
        }
        uint32_t sbits = 0;
        if constexpr (Q0::sdt == 1) {
            sbits = f2bf(s);
            s = bf2f(sbits);
            if (s == 0.0f) {
                s = 1.0f;
                sbits = 0x3F80u;
            }
        } else if (s == 0.0f) {
            s = 1.0f;
        }
        const float inv = f / s;
        uint32_t w[2];
        uint32_t zi = 0;
        if constexpr (Q0::sym) {
            const float off = kMagic + 8.0f;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t[j] = fmaf(v[8 * c + j], inv, off);
                w[c] = pack8(t) ^ 0x88888888u;
            }
        } else {
            const float z = fminf(fmaxf(rintf(zf / s), 0.0f), 15.0f);
            zi = static_cast<uint32_t>(z);
            const float lo = kMagic - z, hi = kMagic + 15.0f - z;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float r = __builtin_amdgcn_fmed3f(fmaf(v[8 * c + j], inv, kMagic), lo, hi);
                    t[j] = __uint_as_float(__float_as_uint(r) + zi);
                }
                w[c] = pack8(t);
            }
            // rows 2m, 2m + 1 live in lanes 4m, 4m + 2 (q = 0): one byte
            const uint32_t zodd = dppu<kXor2>(zi);
            if (valid && qq == 0 && (n & 3) == 0) {
                uint32_t byte = zi & 0xFu;
                if (row + 1 < a.units) byte |= (zodd & 0xFu) << 4;
                a.q[0].zeros[row >> 1] = static_cast<uint8_t>(byte);
            }
        }
        if (valid) {
            uint32_t* cp = reinterpret_cast<uint32_t*>(a.q[0].codes + (e0 >> 1));
            cp[0] = w[0];
            cp[8] = w[1];  // chunk 1 is 64 elements = 32 bytes further
            if (qq == 0 && h == 0) {
                if constexpr (Q0::sdt == 1)
                    static_cast<uint16_t*>(a.q[0].scales)[row] = static_cast<uint16_t>(sbits);
                else
                    static_cast<float*>(a.q[0].scales)[row] = s;
            }
        }
    }
}

// ------------------------------------------------------------- dispatch

template <class Q>
bool qmatch(const FastKey& k, int i) {
    if (Q::fmt < 0) return i >= k.nq;
    return i < k.nq && k.fmt[i] == Q::fmt && k.logg[i] == Q::logg && k.sdt[i] == Q::sdt &&
           (Q::fmt == 1 || k.sym[i] == Q::sym);
}

template <int LOGB, bool WROT, class Q0, class Q1>
int try_kwave(const FastKey& k, const FastArgs& a, hipStream_t s) {
    if (k.logb != LOGB || k.wrot != (WROT ? 1 : 0) || !qmatch<Q0>(k, 0) || !qmatch<Q1>(k, 1)) return 0;
    const int64_t grid = (a.units + 3) / 4;
    hipLaunchKernelGGL((kwave<LOGB, WROT, Q0, Q1>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 1 : -static_cast<int>(e);
}

template <bool WROT, class Q0>
int try_k128(const FastKey& k, const FastArgs& a, hipStream_t s) {
    if (k.logb != 7 || k.wrot != (WROT ? 1 : 0) || !qmatch<Q0>(k, 0) || k.nq > 1) return 0;
    const int64_t grid = (a.units + 31) / 32;
    hipLaunchKernelGGL((k128<WROT, Q0>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 1 : -static_cast<int>(e);
}

using IS128B = QD<0, 1, 7, 1>;   // INT sym g128 bf16 scales
using IA128B = QD<0, 0, 7, 1>;   // INT asym g128 bf16 scales
using IS128F = QD<0, 1, 7, 0>;
using IA128F = QD<0, 0, 7, 0>;
using MX = QD<1, 1, 5, 2>;       // MXFP4

}  // namespace

int launch_fast(const FastKey& k, const FastArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int r = 0;
#define HR_TRY(expr) \
    if ((r = (expr)) != 0) return r
    // 4096-wide blocks
    HR_TRY((try_kwave<12, false, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, true, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, false, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, true, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, true, MX, IS128B>(k, a, s)));
    HR_TRY((try_kwave<12, false, MX, IS128B>(k, a, s)));
    HR_TRY((try_kwave<12, false, MX, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, true, MX, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, true, QNone, QNone>(k, a, s)));
    // 2048-wide blocks
    HR_TRY((try_kwave<11, false, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, true, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, false, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, true, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, true, QNone, QNone>(k, a, s)));
    // 128-wide rows
    HR_TRY((try_k128<true, QNone>(k, a, s)));
    HR_TRY((try_k128<false, IA128B>(k, a, s)));
    HR_TRY((try_k128<true, IA128B>(k, a, s)));
    HR_TRY((try_k128<false, IS128B>(k, a, s)));
    HR_TRY((try_k128<true, IS128B>(k, a, s)));
#undef HR_TRY
    return 0;
}

}  // namespace hr
