// Specialised bfloat16 kernels for gfx950: every shape parameter is a
// compile-time constant.
//
// The Sylvester transform of a block (AutoRound "Rotation Transform",
// section 1.5: H_{2k} = [[H_k, H_k], [H_k, -H_k]], natural order) is a tensor
// product of 2x2 butterflies over the index bits, so the bits can be taken in
// any order and by any mechanism:
//   * bits of exact bf16 inputs by an MFMA: a lane's loaded bf16 values are
//     B operand columns and A is a +-1 matrix (H_32, blockdiag(H_16, H_16),
//     or H_K (x) H_4),
//     so D = A . X transforms those bits exactly (bf16 products with +-1 are
//     exact, accumulation is float32);
//   * bits held in registers: butterflies a +- b;
//   * lane bits: DPP quad permutations or v_permlane32_swap (partner + sign *
//     own);
//   * otherwise an in-wave transpose through a small padded LDS buffer.
//
// kwave<LOGB>: one wave per 4096 elements (one 4096 block or two 2048
//   blocks), no workgroup barrier.
// k128: eight rows of 128 elements per wave; no LDS at all.
// kkron<K>: one workgroup per row of K x 512 (Kronecker form).
// kb32 / kb16 (kbsmall): 128 blocks of 32 or 256 of 16 per wave
//   (rotation_size 32 with MXFP4, 16 with NVFP4).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "codes.h"
#include "plan.h"

namespace hr {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

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


__device__ __forceinline__ u32x4_t ldg16(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
}
// Cached loads for the small vectors every row reads again (permutation,
// signs): a streaming hint would send them back to HBM each time.
__device__ __forceinline__ u32x4_t ldc16(const void* p) { return *static_cast<const u32x4_t*>(p); }
// Streaming (non-temporal) stores for outputs nothing reads back in the same
// launch: codes, scales and rotated rows.  Measured against ordinary stores
// over the whole rotate + quantize step (kernel durations, same GPU), they
// cut the R1, R4 and R3 query kernels by 5-8% and the R3 key kernel by up
// to 2%.  The weight pass keeps one ordinary store (stg16c, its rotated
// rows): with all three of its outputs streaming it ran 1-4% slower than
// with ordinary stores, and with this one ordinary it runs 8% faster.
__device__ __forceinline__ void stg16(void* p, u32x4_t v) {
    __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void stg16c(void* p, u32x4_t v) { *static_cast<u32x4_t*>(p) = v; }

// A operands of v_mfma_f32_16x16x32_bf16 for a transform of five index bits
// of 32 values: lane (j, g = lane / 16) holds k = 8 g + t (t = 0..7) of B
// column j, and the two row halves h give lane (j, g) the outputs
// 8 g + 4 h + r (r = 0..3), i.e. the outputs land where their inputs were.
// HSmallTable<5> is H_32 on (t, g); HSmallTable<4> is blockdiag(H_16, H_16).
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
template <int LOGB>
struct HSmallTable {
    uint32_t w[2][64][4];   // [row half][lane][dword]
    constexpr HSmallTable() : w() {
        for (int h = 0; h < 2; ++h)
            for (int l = 0; l < 64; ++l)
                for (int t = 0; t < 8; ++t) {
                    const int i = l & 15, g = l >> 4;
                    const int out = 8 * (i >> 2) + 4 * h + (i & 3);   // output position of row i
                    const int in = 8 * g + t;                         // input position of k = 8 g + t
                    uint32_t v = 0;                                   // 0 across two blocks of 16
                    if ((out >> LOGB) == (in >> LOGB)) {
                        int p = out & in & ((1 << LOGB) - 1), par = 0;
                        while (p) {
                            par ^= p & 1;
                            p >>= 1;
                        }
                        v = par ? 0xBF80u : 0x3F80u;
                    }
                    w[h][l][t >> 1] |= v << (16 * (t & 1));
                }
    }
};
__constant__ constexpr HSmallTable<5> kH32 = HSmallTable<5>();
__constant__ constexpr HSmallTable<4> kH16x2 = HSmallTable<4>();   // blockdiag(H_16, H_16)
__constant__ constexpr HSmallTable<3> kH8x4 = HSmallTable<3>();    // blockdiag of four H_8

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

// Butterfly across lane bit 0 in one v_fmac_f32_dpp per value: the lane
// with the bit clear gets own + partner, the lane with the bit set own -
// partner (sgn = -1 there), which is exactly -(partner - own).  Those lanes
// therefore hold the negated transform from here on; the caller multiplies
// by sgn again where it normalises, or passes it on to the epilogue inside
// the factor f (a negative f).
// (The compiler does not fold a DPP move into v_fmac_f32, so the stage is
// written out, eight values per block.  Its hazard recognizer does not look
// inside inline asm, so the blocks carry their own wait states: a DPP read of
// a VGPR needs two after a VALU write of it (s_nop 1 before each block;
// inside a block no instruction reads a register another one writes), and
// five after a VALU write of EXEC (s_nop 4 before the first block: EXEC only
// changes at control flow, and the stage is one unrolled basic block).)
template <int N>
__device__ __forceinline__ void dpp_bfly_neg_xor1(float (&v)[N], float sgn) {
    static_assert(N % 8 == 0, "blocks of eight values");
#define HR_DPP_FMAC8(NOP)                                                                          \
    asm(NOP "\n\t"                                                                                 \
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"             \
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"             \
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"             \
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"             \
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"             \
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"             \
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"             \
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"                 \
        : "+v"(v[j]), "+v"(v[j + 1]), "+v"(v[j + 2]), "+v"(v[j + 3]), "+v"(v[j + 4]), "+v"(v[j + 5]), \
          "+v"(v[j + 6]), "+v"(v[j + 7])                                                           \
        : "v"(sgn))
#pragma unroll
    for (int j = 0; j < N; j += 8) {
        if (j == 0)
            HR_DPP_FMAC8("s_nop 4");
        else
            HR_DPP_FMAC8("s_nop 1");
    }
#undef HR_DPP_FMAC8
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

// Eight clamped rounded values (floats kMagic + c with c in [-z, 15 - z])
// and zmul = z * 0x1111 -> eight nibbles c + z, element 0 in the low nibble.
// Below bit 22 the bits of kMagic + c are those of the integer c, so the sum
// of the four shifted words is exact modulo 2^16; adding zmul once per four
// elements then gives the nibbles c + z in 0..15, which never carry.
// (a << 4) + b in one v_lshl_add_u32: the compiler forms separate shifts and
// v_add3_u32 from the plain expression, five instructions per four codes
// against four for this Horner chain.
__device__ __forceinline__ uint32_t shl4_add(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_lshl_add_u32 %0, %1, 4, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t pack8z(const float* r, uint32_t zmul) {
    const uint32_t* b = reinterpret_cast<const uint32_t*>(r);
    const uint32_t a0 = shl4_add(shl4_add(shl4_add(b[3], b[2]), b[1]), b[0]) + zmul;
    const uint32_t a1 = shl4_add(shl4_add(shl4_add(b[7], b[6]), b[5]), b[4]) + zmul;
    return __builtin_amdgcn_perm(a1, a0, 0x05040100u);
}

// Asymmetric INT4 codes of NB runs of eight values el(b, j), j < 8:
// clamp(rne(u inv), lo, hi) in kMagic units (lo = kMagic - z, hi = kMagic +
// 15 - z), packed by pack8z.  fma(u, inv, kMagic) rounds u inv + kMagic once,
// which is monotone in u (either direction, by the sign of inv), so when the
// codes of the lane's largest and smallest u both lie in [lo, hi] so does
// every code and the clamp is the identity.  A wave whose lanes all pass that
// test skips the clamp (one v_med3 per value); its codes are bit for bit the
// clamped ones.  On Gaussian-like rows about one group in a hundred needs the
// clamp: the bf16 scale can round below (hi - lo) / 15 and the two ends of
// the range can both round outwards.
template <int NB, class El>
__device__ __forceinline__ void codes_asym(El el, float inv, float lo, float hi, uint32_t zmul, float umax,
                                           float umin, uint32_t* w) {
    const float c0 = fmaf(umax, inv, kMagic), c1 = fmaf(umin, inv, kMagic);
    const bool inside = fminf(c0, c1) >= lo && fmaxf(c0, c1) <= hi;
    if (__builtin_amdgcn_ballot_w64(!inside) == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = fmaf(el(b, j), inv, kMagic);
            w[b] = pack8z(t, zmul);
        }
    } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = __builtin_amdgcn_fmed3f(fmaf(el(b, j), inv, kMagic), lo, hi);
            w[b] = pack8z(t, zmul);
        }
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two bfloat16 (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    const f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// ------------------------------------------------------------ INT epilogue
// u[0..E) are the lane's E elements of one group of G >= E elements spread
// over GL = G / E lanes, as E / 8 runs of 8 consecutive elements, run b
// starting at element e0 + b SR (SR = 8: E contiguous elements); y = u * f.
template <int E, class Q, int SR = 8>
__device__ __forceinline__ void epi_int(const float (&u)[E], float f, const QuantDev& q, int64_t e0, bool valid,
                                        int lane, int64_t total_groups) {
    constexpr int G = 1 << Q::logg;
    static_assert(G >= E, "group spans whole lanes");
    constexpr int GL = G / E;
    float s, zf = 0.0f;
    float umax = 0.0f, umin = 0.0f;   // the lane's extremes of u (asymmetric)
    if constexpr (Q::sym) {
        float am = fabsf(u[0]);
#pragma unroll
        for (int j = 1; j < E; ++j) am = fmaxf(am, fabsf(u[j]));
        am = lanes_max<GL>(am);
        s = (am * fabsf(f)) * (1.0f / 7.0f);
    } else {
        float hi = u[0], nl = -u[0];
#pragma unroll
        for (int j = 1; j < E; ++j) {
            hi = fmaxf(hi, u[j]);
            nl = fmaxf(nl, -u[j]);
        }
        umax = hi;
        umin = -nl;
        if (f < 0.0f) {   // the lane holds -y: max y = max(-u), -min y = max u
            const float t = hi;
            hi = nl;
            nl = t;
        }
        hi = fmaxf(lanes_max<GL>(hi), 0.0f) * fabsf(f);
        nl = fmaxf(lanes_max<GL>(nl), 0.0f) * fabsf(f);  // -min(min y, 0)
        s = (hi + nl) * (1.0f / 15.0f);
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
    // reciprocal within 1 ulp: moves y / s by about 1e-7 of a step
    const float rs = __builtin_amdgcn_rcpf(s);
    const float inv = f * rs;
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
        const float z = fminf(fmaxf(rintf(zf * rs), 0.0f), 15.0f);
        // clamp(rne(y / s) + z, 0, 15): round on y / s alone (ties to even
        // there), clamp to [-z, 15 - z], then add z to the packed nibbles.
        const uint32_t zi = static_cast<uint32_t>(z);
        const uint32_t zmul = zi * 0x1111u;
        const float lo = kMagic - z, hi = kMagic + 15.0f - z;
        codes_asym<E / 8>([&](int b, int j) { return u[8 * b + j]; }, inv, lo, hi, zmul, umax, umin, w);
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
        if constexpr (SR != 8) {
#pragma unroll
            for (int b = 0; b < E / 8; ++b) *reinterpret_cast<uint32_t*>(cp + (b * SR) / 2) = w[b];
        } else if constexpr (E / 8 == 8) {
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

// INT epilogue for groups smaller than the lane's E contiguous elements
// (G = 32: two groups per lane; G = 16: four): each group's extremes,
// scale, codes and zero point stay in the lane, with the arithmetic of
// epi_int.  The lane's NG scales are one store, and its NG zero-point
// nibbles (groups 2i, 2i + 1 share a byte, element order) one more.
template <int E, class Q>
__device__ __forceinline__ void epi_int_small(const float (&u)[E], float f, const QuantDev& q, int64_t e0,
                                              bool valid) {
    constexpr int G = 1 << Q::logg;
    constexpr int NG = E / G;
    static_assert(G >= 16 && G < E && NG <= 4, "two or four groups per lane");
    uint32_t w[E / 8];
    uint32_t sb[NG];
    float sf[NG];
    uint32_t zbits = 0;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const float* v = u + G * k;
        float s, zf = 0.0f;
        if constexpr (Q::sym) {
            float am = fabsf(v[0]);
#pragma unroll
            for (int j = 1; j < G; ++j) am = fmaxf(am, fabsf(v[j]));
            s = (am * fabsf(f)) * (1.0f / 7.0f);
        } else {
            float hi = v[0], nl = -v[0];
#pragma unroll
            for (int j = 1; j < G; ++j) {
                hi = fmaxf(hi, v[j]);
                nl = fmaxf(nl, -v[j]);
            }
            if (f < 0.0f) {   // the lane holds -y
                const float t = hi;
                hi = nl;
                nl = t;
            }
            hi = fmaxf(hi, 0.0f) * fabsf(f);
            nl = fmaxf(nl, 0.0f) * fabsf(f);  // -min(min y, 0)
            s = (hi + nl) * (1.0f / 15.0f);
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
        sb[k] = sbits;
        sf[k] = s;
        const float rs = __builtin_amdgcn_rcpf(s);
        const float inv = f * rs;
        if constexpr (Q::sym) {
            const float off = kMagic + 8.0f;
#pragma unroll
            for (int b = 0; b < G / 8; ++b) {
                float t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t[j] = fmaf(v[8 * b + j], inv, off);
                w[(G / 8) * k + b] = pack8(t) ^ 0x88888888u;
            }
        } else {
            const float z = fminf(fmaxf(rintf(zf * rs), 0.0f), 15.0f);
            const uint32_t zi = static_cast<uint32_t>(z);
            const uint32_t zmul = zi * 0x1111u;
            const float lo = kMagic - z, hi = kMagic + 15.0f - z;
#pragma unroll
            for (int b = 0; b < G / 8; ++b) {
                float t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) t[j] = __builtin_amdgcn_fmed3f(fmaf(v[8 * b + j], inv, kMagic), lo, hi);
                w[(G / 8) * k + b] = pack8z(t, zmul);
            }
            zbits |= zi << (4 * k);
        }
    }
    if (valid) {
        uint8_t* cp = q.codes + (e0 >> 1);
#pragma unroll
        for (int b = 0; b < E / 32; ++b) stg16(cp + 16 * b, u32x4_t{w[4 * b], w[4 * b + 1], w[4 * b + 2], w[4 * b + 3]});
        const int64_t g0 = e0 >> Q::logg;          // the lane's first group (a multiple of NG)
        if constexpr (Q::sdt == 1) {
            // one store of the NG scales where the buffer's alignment allows it
            // (the same for every lane: g0 is a multiple of NG), else NG
            uint16_t* sp = static_cast<uint16_t*>(q.scales) + g0;
            if ((reinterpret_cast<uintptr_t>(q.scales) & (2 * NG - 1)) == 0) {
                if constexpr (NG == 2)
                    *reinterpret_cast<uint32_t*>(sp) = sb[0] | (sb[1] << 16);
                else
                    *reinterpret_cast<u32x2_t*>(sp) = u32x2_t{sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16)};
            } else {
#pragma unroll
                for (int k = 0; k < NG; ++k) sp[k] = static_cast<uint16_t>(sb[k]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NG; ++k) static_cast<float*>(q.scales)[g0 + k] = sf[k];
        }
        if constexpr (!Q::sym) {
            q.zeros[g0 >> 1] = static_cast<uint8_t>(zbits);
            if constexpr (NG == 4) q.zeros[(g0 >> 1) + 1] = static_cast<uint8_t>(zbits >> 8);
        }
    }
}

// ----------------------------------------------------------- MXFP4 epilogue
// Eight values -> eight E2M1 nibbles (element 0 lowest) with the hardware
// converter, which divides by `sc`, rounds to nearest even and saturates.
__device__ __forceinline__ uint32_t cvt8_fp4(const float* v, float sc, float pre, bool scaled) {
    uint32_t r = 0;
    if (scaled) {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0] * pre, v[1] * pre, sc, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2] * pre, v[3] * pre, sc, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4] * pre, v[5] * pre, sc, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6] * pre, v[7] * pre, sc, 3);
    } else {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], sc, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], sc, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], sc, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], sc, 3);
    }
    return r;
}

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
        // 2^-127 is not a normal float: a group with that scale (amax below
        // 2^-124) is multiplied by 2^64 and divided by 2^-63 instead, both
        // exact; the branch is uniform over the wave.
        if (__builtin_amdgcn_ballot_w64(e == -127) == 0) {
            const float sc = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);  // 2^e
#pragma unroll
            for (int d = 0; d < 4; ++d) w[4 * g + d] = cvt8_fp4(y + 32 * g + 8 * d, sc, 1.0f, false);
        } else {
            const bool tiny = e == -127;
            const float sc = tiny ? __uint_as_float(64u << 23) : __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
            const float pre = tiny ? __uint_as_float(191u << 23) : 1.0f;  // 2^-63 and 2^64
#pragma unroll
            for (int d = 0; d < 4; ++d) w[4 * g + d] = cvt8_fp4(y + 32 * g + 8 * d, sc, pre, true);
        }
    }
    if (valid) {
        uint8_t* cp = q.codes + (e0 >> 1);
#pragma unroll
        for (int b = 0; b < E / 32; ++b) stg16(cp + 16 * b, u32x4_t{w[4 * b], w[4 * b + 1], w[4 * b + 2], w[4 * b + 3]});
        uint8_t* sp = static_cast<uint8_t*>(q.scales) + (e0 >> 5);
        if constexpr (NB == 2) {
            // the E8M0 buffer need only be byte-aligned; e0 is a multiple of 64,
            // so every lane's pair has the parity of the buffer
            if ((reinterpret_cast<uintptr_t>(q.scales) & 1u) == 0) {
                *reinterpret_cast<uint16_t*>(sp) = static_cast<uint16_t>(ebytes);
            } else {
                sp[0] = static_cast<uint8_t>(ebytes);
                sp[1] = static_cast<uint8_t>(ebytes >> 8);
            }
        } else {
            *sp = static_cast<uint8_t>(ebytes);
        }
    }
}

template <int E, class Q>
__device__ __forceinline__ void epilogue(const float (&u)[E], float f, const QuantDev& q, int64_t e0, bool valid,
                                         int lane, int64_t total_groups) {
    if constexpr (Q::fmt == 0 && (1 << Q::logg) < E) {
        epi_int_small<E, Q>(u, f, q, e0, valid);
    } else if constexpr (Q::fmt == 0) {
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

// A wave owns 4096 contiguous elements: one block of 4096, or 4096 / B
// blocks of B = 2048 .. 64 (half a block of 8192: a pair of waves).
struct KW {
    static constexpr int E = 64;              // elements per lane
    static constexpr int NC = E / 8;          // 16-byte chunks per lane
    static constexpr int NS = 4;              // transpose passes
    static constexpr int R = 8 / NS;          // chunk elements per pass
    static constexpr int LW = 4096 / NS;      // elements per pass
    static constexpr int LDS_T = LW + (LW >> 5) + 1;     // transpose pass buffer
    static constexpr int LDS_W = 2048 + (2048 >> 5);      // bf16 words of 4096 outputs
    static constexpr int LDS = LDS_T > LDS_W ? LDS_T : LDS_W;
    static_assert(LW <= 1024, "padding formula assumes passes of at most 1024 elements");
};

// Load layout L0: element e = 512 c + 8 lane + r of the wave's 4096 (chunk c,
// r = 0..7).  The MFMA (16x16x32, one 16-byte load as B) transforms index
// bits {0, 1, 2, 7, 8}; register butterflies bits 9, 10 and (4096-blocks)
// 11; an LDS transpose in NS
// passes over r gives each lane 64 contiguous elements (L2); bits 3..5 are
// then register bits and bit 6 is lane bit 0 (DPP).  Bits at or above log2 B
// select the block and are never mixed: 2048-blocks leave bit 11 alone,
// 512-blocks bits 9..11, 256-blocks also bit 8 (the MFMA applies
// blockdiag(H_16, H_16)), 64-blocks also bits 6, 7 (four H_8 on the MFMA, no
// DPP stage).
// Randomised rotation (MIX > 0): element j of a row reads x[perm[j]] and is
// multiplied by in_signs[j] before and by out_signs[j] after the transform
// (the random Hadamard H diag(+-1) of the AutoRound page, section 1.5;
// OrbitQuant's RPBH, Method Conformance: permutation, Rademacher signs,
// block FWHT); each vector is nullable. With a permutation (MIX = 2) one
// workgroup owns a whole row (n <= 16384), stages it in LDS and gathers from
// there: gathering from global memory (64 scattered 2-byte loads per lane)
// measured slower than the generic kernel. Column of element e of block b:
// (b mod row_blocks) B + e.
__device__ __forceinline__ uint32_t sign_mask2(uint32_t s, int k) {
    // bf16 pair (2k, 2k + 1) of the four int8 signs in s: bit 15 and bit 31
    const uint32_t lo = (s >> (16 * k)) & 0x80u, hi = (s >> (16 * k + 8)) & 0x80u;
    return (lo << 8) | (hi << 24);
}

template <int LOGB, bool WROT, class Q0, class Q1, int MIX = 0>
__global__ void __launch_bounds__(256) kwave(const FastArgs a) {
    static_assert(LOGB >= 6 && LOGB <= 13 && LOGB != 7, "blocks of 64, 256 .. 8192 (128: k128)");
    static_assert(MIX == 0 || LOGB == 11 || LOGB == 12, "randomised rotations on 2048- and 4096-blocks");
    constexpr int E = KW::E, NC = KW::NC, NS = KW::NS, R = KW::R;
    constexpr int B = 1 << LOGB;
    // blocks of 8192: a pair of waves (w, w ^ 1) per block, each holding one
    // half; index bit 12 is a butterfly across the pair through LDS
    constexpr bool PAIR = LOGB == 13;
    constexpr int BPW = PAIR ? 1 : 4096 / B;  // blocks per wave
    constexpr bool MIXED = MIX > 0;           // signs (1) or a permutation and signs (2)
    constexpr bool PERM = MIX == 2;
    // permutation: one workgroup per row of n <= 16384, staged in rowbuf, whose
    // space then holds the waves' transpose buffers
    constexpr int RB16 = 2 * 4 * KW::LDS > 16384 ? 2 * 4 * KW::LDS : 16384;   // uint16 words
    // per-wave buffer: the transpose, plus (rotated output) the bf16 store staging
    constexpr int LDSZ = WROT ? KW::LDS : KW::LDS_T;
    __shared__ float lds_all[PERM ? 1 : 4][PERM ? 1 : LDSZ];
    __shared__ __attribute__((aligned(16))) uint16_t rowbuf[PERM ? RB16 : 8];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    int64_t blk0;
    bool hi_ok;
    int mcol[2] = {0, 0};   // randomised rotation: column of the wave's blocks in their rows
    if constexpr (PERM) {
        const int rb = static_cast<int>(a.row_blocks);
        const int n = rb * B;
        const int64_t row = blockIdx.x;
        const uint16_t* xr = static_cast<const uint16_t*>(a.x) + row * n;
        // batches of 8 loads in flight per thread
        const int nq = n / 8, nt = blockDim.x;
        for (int q0 = threadIdx.x; q0 < nq; q0 += 8 * nt) {
            u32x4_t t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = q0 + i * nt;
                t[i] = ldg16(xr + 8 * (q < nq ? q : q0));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = q0 + i * nt;
                if (q < nq) *reinterpret_cast<u32x4_t*>(rowbuf + 8 * q) = t[i];
            }
        }
        __syncthreads();
        blk0 = row * rb + wv * BPW;
        hi_ok = BPW == 1 || wv * BPW + 1 < rb;
        mcol[0] = wv * BPW * B;
        mcol[1] = mcol[0] + B;
    } else if constexpr (PAIR) {
        // both waves of a pair reach the exchange barriers: a pair past the
        // end re-reads the last block and stores nothing
        const int64_t blk = (static_cast<int64_t>(blockIdx.x) * 4 + wv) >> 1;
        hi_ok = blk < a.units;
        blk0 = hi_ok ? blk : a.units - 1;
    } else {
        const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + wv;
        blk0 = wave * BPW;
        if (blk0 >= a.units) return;  // whole wave idle; no barrier follows
        // with two blocks per wave the second may lie past the end
        hi_ok = BPW == 1 || blk0 + 1 < a.units;
        if constexpr (MIXED) {
            const int64_t rb = a.row_blocks;
            const int b0 = __builtin_amdgcn_readfirstlane(static_cast<int>(blk0 % rb));
            mcol[0] = b0 * B;
            mcol[1] = b0 + 1 == rb ? 0 : mcol[0] + B;
        }
    }
    float* lds = PERM ? reinterpret_cast<float*>(rowbuf) + wv * KW::LDS : lds_all[wv];
    // first element of the wave's 4096 (the wave's half of a block of 8192)
    const int64_t ebase = blk0 * B + (PAIR ? 4096 * (wv & 1) : 0);
    const uint16_t* src = static_cast<const uint16_t*>(a.x) + ebase;
    // blocks of the wave that it stores: those before the end of the tensor
    // (BPW > 1: the rest re-read the first block, finite data that is never
    // stored); with a permutation, those inside the workgroup's row
    const int64_t nvalid = BPW == 1 ? 1
                         : PERM     ? (hi_ok ? 2 : 1)
                                    : (a.units - blk0 < BPW ? a.units - blk0 : BPW);
    u32x4_t raw[NC];
    if constexpr (PERM) {
        // gather from the staged row: element j of the row is x[perm[j]]
        const int nn = static_cast<int>(a.row_blocks) * B;
        const bool idle = wv * BPW >= a.row_blocks;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (idle) break;
            const int k = ((512 * c) >> LOGB) & (hi_ok ? 1 : 0);
            const int col = mcol[k] + ((512 * c + 8 * lane) & (B - 1));
            const u32x4_t p0 = ldc16(a.perm + col), p1 = ldc16(a.perm + col + 4);
            const int idx[8] = {static_cast<int>(p0[0]), static_cast<int>(p0[1]), static_cast<int>(p0[2]),
                                static_cast<int>(p0[3]), static_cast<int>(p1[0]), static_cast<int>(p1[1]),
                                static_cast<int>(p1[2]), static_cast<int>(p1[3])};
            uint32_t h[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) h[r] = rowbuf[min(max(idx[r], 0), nn - 1)];
            raw[c] = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
        __syncthreads();   // every gather done: rowbuf becomes the transpose buffers
        if (idle) return;  // whole wave idle; no barrier follows
    } else if constexpr (LOGB >= 9) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            constexpr int CPB = B / 512 < NC ? B / 512 : NC;      // chunks per block
            const int kb = (512 * c) >> LOGB;                    // block of the chunk in the wave
            raw[c] = ldg16(src + (kb < nvalid ? 512 * c : 512 * (c % CPB)) + 8 * lane);
        }
    } else {
        // blocks under 512: a chunk spans several blocks, so the test is per
        // lane; a piece past the end re-reads its place in the first block
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = 512 * c + 8 * lane;
            raw[c] = ldg16(src + ((e >> LOGB) < nvalid ? e : (e & (B - 1))));
        }
    }
    if constexpr (MIXED) {
        if (a.in_signs) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int k = ((512 * c) >> LOGB) & (hi_ok ? 1 : 0);   // block of the wave
                const int col = mcol[k] + ((512 * c + 8 * lane) & (B - 1));
                const u32x2_t sg = *reinterpret_cast<const u32x2_t*>(a.in_signs + col);
                raw[c][0] ^= sign_mask2(sg[0], 0);
                raw[c][1] ^= sign_mask2(sg[0], 1);
                raw[c][2] ^= sign_mask2(sg[1], 0);
                raw[c][3] ^= sign_mask2(sg[1], 1);
            }
        }
    }

    // the MFMA mixes index bits 0..2 with 7, 8 (H_32), with 7 only (blocks
    // of 256: blockdiag(H_16, H_16)) or with neither (blocks of 64: four H_8)
    const uint32_t* tw = LOGB >= 9 ? &kH32.w[0][lane][0] : (LOGB == 8 ? &kH16x2.w[0][lane][0] : &kH8x4.w[0][lane][0]);
    const u32x4_t* hp = reinterpret_cast<const u32x4_t*>(tw);   // hp[64]: row half 1
    const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, hp[0]);
    const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, hp[64]);
    float v[E];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const bf16x8_t Bc = __builtin_bit_cast(bf16x8_t, raw[c]);
        const f32x4v_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Bc, f32x4v_t{}, 0, 0, 0);
        const f32x4v_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Bc, f32x4v_t{}, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * c + j] = d0[j];
            v[8 * c + 4 + j] = d1[j];
        }
    }
    // register bits of L0: v-index bits 3..5 (e bits 9..11), those inside a
    // block
    bfly<E, (LOGB >= 12) ? 0x38u : (LOGB == 11 ? 0x18u : (LOGB == 10 ? 0x08u : 0u))>(v);

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
    bfly<E, 0x38u>(y);                                   // bits 3, 4, 5
    // bit 6; odd lanes then hold -y (sig), undone at the normalisation or in
    // the epilogue's factor
    const float sig = (LOGB >= 7 && (lane & 1)) ? -1.0f : 1.0f;
    if constexpr (LOGB >= 7) dpp_bfly_neg_xor1(y, sig);
    if constexpr (PAIR) {
        // bit 12 across the pair: four passes of 16 values per lane through
        // the transpose buffers (value j of lane l at 65 j + l: no bank
        // conflicts); wave w ^ 1 holds the same positions of the other half
        const float* pl = lds_all[wv ^ 1];
        const float sgn = (wv & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int j = 0; j < 16; ++j) lds[65 * j + lane] = y[16 * p + j];
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 16; ++j) y[16 * p + j] = fmaf(sgn, y[16 * p + j], pl[65 * j + lane]);
            __syncthreads();
        }
    }

    // the lane's 64 elements lie in block (64 lane) >> LOGB of the wave
    const bool valid = PAIR ? hi_ok : ((64 * lane) >> LOGB) < nvalid;
    const int64_t e0 = ebase + static_cast<int64_t>(E) * lane;
    if constexpr (MIXED) {
        if (a.out_signs) {
            // the lane's 64 contiguous elements lie in one block
            const int k = ((E * lane) >> LOGB) & (valid ? 1 : 0);
            const int col = mcol[k] + ((E * lane) & (B - 1));
#pragma unroll
            for (int q4 = 0; q4 < E / 16; ++q4) {
                const u32x4_t sg = ldc16(a.out_signs + col + 16 * q4);
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const uint32_t bit = ((sg[t >> 2] >> (8 * (t & 3))) & 0x80u) << 24;
                    y[16 * q4 + t] = __uint_as_float(__float_as_uint(y[16 * q4 + t]) ^ bit);
                }
            }
        }
    }
    constexpr bool need_y = WROT || Q0::fmt == 1 || Q1::fmt == 1;
    float f = sig * a.norm;   // y = f * (the lane's values)
    if constexpr (need_y) {
#pragma unroll
        for (int j = 0; j < E; ++j) y[j] *= f;
        f = 1.0f;
    }
    if constexpr (WROT) {
        // bf16 words go back through LDS to the load layout so that each
        // store instruction writes 1 KiB of consecutive bytes: word
        // w = 32 lane + m (padded by one per 32) is read back as chunk c,
        // word k of lane l: w = 256 c + 4 l + k.
        uint32_t* lw = reinterpret_cast<uint32_t*>(lds);
#pragma unroll
        for (int m = 0; m < 32; ++m) lw[33 * lane + m] = bf16x2(y[2 * m], y[2 * m + 1]);
        wave_sync();
        uint16_t* dst = static_cast<uint16_t*>(a.y_rot) + ebase;
        const int rb = 4 * lane + (lane >> 3);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4_t wv4 = {lw[rb + 264 * c], lw[rb + 264 * c + 1], lw[rb + 264 * c + 2], lw[rb + 264 * c + 3]};
            const bool cvalid = PAIR ? hi_ok : ((512 * c + (LOGB < 9 ? 8 * lane : 0)) >> LOGB) < nvalid;
            if (cvalid) stg16c(dst + 512 * c + 8 * lane, wv4);
        }
        wave_sync();
    }
    if constexpr (Q0::fmt >= 0) epilogue<E, Q0>(y, f, a.q[0], e0, valid, lane, a.total_groups[0]);
    if constexpr (Q1::fmt >= 0) epilogue<E, Q1>(y, f, a.q[1], e0, valid, lane, a.total_groups[1]);
}

// ----------------------------------------------------------------- k128
// Eight rows of 128 per wave.  Lane l: n = l % 16, row = n >> 1, h = n & 1,
// q = l >> 4; chunk c in {0, 1} holds row elements 64 c + 32 h + 8 q + r.
// The MFMA (16x16x32, one 16-byte load as B) transforms bits {0..4},
// registers bit 6, the DPP butterfly bit 5.  The 128 elements of a row sit in the 8 lanes sharing n >> 1.
// Groups of eight 128-element rows per k128 wave.  The quantising instances
// load two groups up front (twice the bytes in flight per wave, the set-up
// shared): the R3 key kernel measured 60.5 -> 58.9 us with two, 60.3 with four
// (79 VGPRs, six waves per SIMD) and 63.5 with eight.  The plain rotation
// keeps one, which measured faster there.  (Quantising without a rotated
// output now runs k128q; this applies to the instances that also write y.)
template <class Q0>
__host__ __device__ constexpr int k128_groups() {
    return Q0::fmt == 0 ? 2 : 1;
}

template <bool WROT, class Q0>
__global__ void __launch_bounds__(256) k128(const FastArgs a) {
    constexpr int G = k128_groups<Q0>();   // groups of eight rows per wave
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n = lane & 15;
    const int h = n & 1;
    const int qq = lane >> 4;
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + wv) * 8 * G + (n >> 1);
    const int col0 = 32 * h + 8 * qq;  // element of chunk 0 within the row
    // every group's loads first; rows past the end re-read the last row
    // (finite data, never stored)
    u32x4_t raws[G][2];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        const int64_t row = row0 + 8 * gi;
        const int64_t lrow = row < a.units ? row : a.units - 1;
        const uint16_t* src = static_cast<const uint16_t*>(a.x) + lrow * 128 + col0;
#pragma unroll
        for (int c = 0; c < 2; ++c) raws[gi][c] = ldg16(src + 64 * c);
    }
    const u32x4_t* hp = reinterpret_cast<const u32x4_t*>(&kH32.w[0][lane][0]);   // hp[64]: row half 1
    const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, hp[0]);
    const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, hp[64]);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        const int64_t row = row0 + 8 * gi;
        const bool valid = row < a.units;
        const u32x4_t (&raw)[2] = raws[gi];
        float v[16];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8_t Bc = __builtin_bit_cast(bf16x8_t, raw[c]);
            const f32x4v_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Bc, f32x4v_t{}, 0, 0, 0);
            const f32x4v_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Bc, f32x4v_t{}, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * c + j] = d0[j];
                v[8 * c + 4 + j] = d1[j];
            }
        }
        bfly<16, 0x8u>(v);                           // bit 6 (v-index bit 3)
        // bit 5: odd lanes then hold -y, undone by the signed factor f
        const float sig = h ? -1.0f : 1.0f;
        dpp_bfly_neg_xor1(v, sig);
        const int64_t e0 = row * 128 + col0;

        if constexpr (WROT) {
            uint16_t* dst = static_cast<uint16_t*>(a.y_rot) + e0;
            float y[16];
            const float fy = sig * a.norm;
#pragma unroll
            for (int j = 0; j < 16; ++j) y[j] = v[j] * fy;
            if (valid) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    stg16(dst + 64 * c, u32x4_t{bf16x2(y[8 * c], y[8 * c + 1]), bf16x2(y[8 * c + 2], y[8 * c + 3]),
                                                bf16x2(y[8 * c + 4], y[8 * c + 5]), bf16x2(y[8 * c + 6], y[8 * c + 7])});
            }
        }
        if constexpr (Q0::fmt == 0) {
            static_assert(Q0::logg == 7, "one group per row");
            const float f = a.norm;   // y = sig * f * v
            float s, zf = 0.0f;
            float umax = 0.0f, umin = 0.0f;   // the lane's extremes of v (asymmetric)
            if constexpr (Q0::sym) {
                float am = fabsf(v[0]);
#pragma unroll
                for (int j = 1; j < 16; ++j) am = fmaxf(am, fabsf(v[j]));
                am = fmaxf(am, dpp<kXor1>(am));
                am = fmaxf(am, __shfl_xor(am, 16));
                am = fmaxf(am, __shfl_xor(am, 32));
                s = (am * f) * (1.0f / 7.0f);
            } else {
                float hi = v[0], nl = -v[0];
#pragma unroll
                for (int j = 1; j < 16; ++j) {
                    hi = fmaxf(hi, v[j]);
                    nl = fmaxf(nl, -v[j]);
                }
                umax = hi;
                umin = -nl;
                if (h) {   // the lane holds -y: max y = max(-v), -min y = max v
                    const float t = hi;
                    hi = nl;
                    nl = t;
                }
                hi = fmaxf(hi, dpp<kXor1>(hi));
                nl = fmaxf(nl, dpp<kXor1>(nl));
                hi = fmaxf(hi, __shfl_xor(hi, 16));
                nl = fmaxf(nl, __shfl_xor(nl, 16));
                hi = fmaxf(hi, __shfl_xor(hi, 32));
                nl = fmaxf(nl, __shfl_xor(nl, 32));
                hi = fmaxf(hi, 0.0f) * f;
                nl = fmaxf(nl, 0.0f) * f;
                s = (hi + nl) * (1.0f / 15.0f);
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
            const float rs = __builtin_amdgcn_rcpf(s);
            const float inv = sig * (f * rs);
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
                const float z = fminf(fmaxf(rintf(zf * rs), 0.0f), 15.0f);
                zi = static_cast<uint32_t>(z);
                const uint32_t zmul = zi * 0x1111u;
                const float lo = kMagic - z, hi = kMagic + 15.0f - z;
                codes_asym<2>([&](int c, int j) { return v[8 * c + j]; }, inv, lo, hi, zmul, umax, umin, w);
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
}

// ----------------------------------------------------------------- k128q
// R3 keys: 128-element rows quantised as one group each, no rotated output.
// Sixteen rows per wave: lane l = n + 16 q holds row n's elements
// 32 c + 8 q + r (c = 0..3, r = 0..7).  The MFMA takes index bits 0..4 (r and
// q) exactly as in k128; bits 5 and 6 (c) are register butterflies, so no
// lane stage is left, and a lane's share of its group's reductions, scale and
// zero point covers 32 elements instead of 16.  A row's group spans lanes
// n + 16 q: its extremes are reduced over lane bits 4 and 5.
// In that layout a load instruction would read 64-byte halves of sixteen
// lines (measured: 76 us against 59 for k128 on the R3 keys), so the wave's
// 4 KiB go through LDS: whole-line loads in, the layout out; and the 1 KiB
// of codes back the same way, so that each store writes 1 KiB of
// consecutive bytes.
constexpr int kQRow = 272;    // LDS bytes per staged row (256 + 16: no bank conflicts)
constexpr int kQCode = 80;    // LDS bytes per row of codes (64 + 16)
template <class Q0>
__global__ void __launch_bounds__(256) k128q(const FastArgs a) {
    static_assert(Q0::fmt == 0 && Q0::logg == 7, "INT, one group per row");
    __shared__ __attribute__((aligned(16))) char smem[4][16 * kQRow];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    char* ws = smem[wv];
    const int n = lane & 15;
    const int qq = lane >> 4;
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + wv) * 16;
    const int64_t row = row0 + n;
    const bool valid = row < a.units;
    // whole-line loads: piece k of lane l is byte 1024 k + 16 l of the
    // wave's 16 rows; rows past the end re-read the last row (finite data,
    // never stored)
    u32x4_t g[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = 1024 * k + 16 * lane;
        const int64_t gr = row0 + (p >> 8);
        const int64_t lr = gr < a.units ? gr : a.units - 1;
        g[k] = ldg16(static_cast<const char*>(a.x) + lr * 256 + (p & 255));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = 1024 * k + 16 * lane;
        *reinterpret_cast<u32x4_t*>(ws + (p >> 8) * kQRow + (p & 255)) = g[k];
    }
    wave_sync();
    u32x4_t raw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = *reinterpret_cast<const u32x4_t*>(ws + n * kQRow + 64 * c + 16 * qq);
    const u32x4_t* hp = reinterpret_cast<const u32x4_t*>(&kH32.w[0][lane][0]);   // hp[64]: row half 1
    const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, hp[0]);
    const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, hp[64]);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const bf16x8_t Bc = __builtin_bit_cast(bf16x8_t, raw[c]);
        const f32x4v_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Bc, f32x4v_t{}, 0, 0, 0);
        const f32x4v_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Bc, f32x4v_t{}, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * c + j] = d0[j];
            v[8 * c + 4 + j] = d1[j];
        }
    }
    bfly<32, 0x18u>(v);   // bits 5, 6 (v-index bits 3, 4)

    const float f = a.norm;
    float s, zf = 0.0f;
    float umax = 0.0f, umin = 0.0f;   // the lane's extremes of v (asymmetric)
    if constexpr (Q0::sym) {
        float am = fabsf(v[0]);
#pragma unroll
        for (int j = 1; j < 32; ++j) am = fmaxf(am, fabsf(v[j]));
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        s = (am * f) * (1.0f / 7.0f);
    } else {
        float hi = v[0], nl = -v[0];
#pragma unroll
        for (int j = 1; j < 32; ++j) {
            hi = fmaxf(hi, v[j]);
            nl = fmaxf(nl, -v[j]);
        }
        umax = hi;
        umin = -nl;
        hi = fmaxf(hi, __shfl_xor(hi, 16));
        nl = fmaxf(nl, __shfl_xor(nl, 16));
        hi = fmaxf(hi, __shfl_xor(hi, 32));
        nl = fmaxf(nl, __shfl_xor(nl, 32));
        hi = fmaxf(hi, 0.0f) * f;
        nl = fmaxf(nl, 0.0f) * f;   // -min(min y, 0)
        s = (hi + nl) * (1.0f / 15.0f);
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
    const float rs = __builtin_amdgcn_rcpf(s);
    const float inv = f * rs;
    uint32_t w[4];
    if constexpr (Q0::sym) {
        const float off = kMagic + 8.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = fmaf(v[8 * c + j], inv, off);
            w[c] = pack8(t) ^ 0x88888888u;
        }
    } else {
        const float z = fminf(fmaxf(rintf(zf * rs), 0.0f), 15.0f);
        const uint32_t zi = static_cast<uint32_t>(z);
        const uint32_t zmul = zi * 0x1111u;
        const float lo = kMagic - z, hi = kMagic + 15.0f - z;
        codes_asym<4>([&](int c, int j) { return v[8 * c + j]; }, inv, lo, hi, zmul, umax, umin, w);
        // rows 2m, 2m + 1 live in lanes 2m, 2m + 1 (q = 0): one byte
        const uint32_t zodd = dppu<kXor1>(zi);
        if (valid && qq == 0 && (n & 1) == 0) {
            uint32_t byte = zi & 0xFu;
            if (row + 1 < a.units) byte |= (zodd & 0xFu) << 4;
            a.q[0].zeros[row >> 1] = static_cast<uint8_t>(byte);
        }
    }
    // codes: chunk c of lane (n, q) is byte 16 c + 4 q of row n's 64; through
    // LDS so that lane l stores bytes 16 l .. 16 l + 15 of the wave's 1 KiB
    wave_sync();   // every lane has read its operands from ws
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(ws + n * kQCode + 16 * c + 4 * qq) = w[c];
    wave_sync();
    const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(ws + (lane >> 2) * kQCode + 16 * (lane & 3));
    if (row0 + (lane >> 2) < a.units) stg16(a.q[0].codes + row0 * 64 + 16 * lane, cw);
    if (valid) {
        if (qq == 0) {
            if constexpr (Q0::sdt == 1)
                static_cast<uint16_t*>(a.q[0].scales)[row] = static_cast<uint16_t>(sbits);
            else
                static_cast<float*>(a.q[0].scales)[row] = s;
        }
    }
}

// ----------------------------------------------------------------- kkron
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Hides a value from the optimiser, so that per-lane LDS bases stay whole
// and the constant parts of addresses stay in the instruction offsets.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// (lanes 0-31 of x, lanes 0-31 of y), (lanes 32-63 of x, lanes 32-63 of y)
__device__ __forceinline__ void swap_halves(float& x, float& y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}
// maximum of v over lanes l and l ^ 32
__device__ __forceinline__ float max_halves(float v) {
    float a = v, b = v;
    swap_halves(a, b);
    return fmaxf(a, b);
}

// One workgroup (4 waves) per row of n = K * 512 bf16 elements, K <= 32,
// computing y = x (H_K (x) H_512) / sqrt(n) (AutoRound "Rotation Transform",
// section 1.5: a base matrix of order K combined with a Sylvester block).
// Write the row as x[a][b] (piece a < K, column b < 512, bits b0..b8).
// Phase 1: stage the row in LDS, 16 bytes per (piece octet, column): dword j
//   of octet q at column b holds x[8q + 2j][b] (low half) and x[8q + 2j + 1][b];
//   pieces >= K are zero. Within each run of 8 columns the 16-byte slots are
//   XOR-swizzled so that both the staging writes and the operand reads are
//   free of bank conflicts.
// Phase 2: v_mfma_f32_32x32x16_bf16 contracts over (u, a) at once, u being
//   column bits b7, b8: for output bits s and piece c,
//   Y[c][b' + 128 s] = sum_u sum_a H_4[u][s] H_K[a][c] x[a][b' + 128 u]
//   (b' = i + 32 blk + 64 b6 < 128, i = b0..b4, blk = b5). A = 32 columns i
//   by 16 pieces a of x (one u, one 16-byte read per lane), B = +-H_K slice
//   (the sign H_4[u][s] picks the copy). bf16 times +-1 is exact; the sum is
//   float32. This takes the base-matrix mix and two of the nine column stages
//   (the MFMA does 4 times the useful work of the mix alone, which costs less
//   than the vector stages it saves only up to about two column bits). Wave w
//   owns output bits (b7, b8) = (w & 1, w >> 1) and all of b0..b6: four tiles
//   (blk, b6). Lane l then holds piece c = l % 32, b2 = l / 32, and b0, b1,
//   b3, b4, b5, b6 in registers: six butterfly stages, then one across the
//   two half-waves (v_permlane32_swap) for b2, after which lane l holds the
//   64 consecutive columns of piece c with b6 = l / 32.
// Epilogue: a group of 128 columns (b0..b6) sits in lanes l and l ^ 32.
template <int W, int HALVES, int LOGM>
__device__ __forceinline__ void kkron_mix(const uint32_t* smem, int lane, float (&v)[64]) {
    constexpr int M = 1 << LOGM;
    constexpr int U = M / 128;               // column blocks contracted on the MFMA
    constexpr int BT = 16 * M;               // B table offset, dwords (after the staging)
    const int il = lane & 31;
    const int g = lane >> 5;
    // B operand: lane (c, g) element t = H_K[16 h + 8 g + t][c]
    u32x4_t bp[HALVES], bn[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t x = smem[BT + lane + 64 * (p + 4 * h)];
            bp[h][p] = x;
            bn[h][p] = x ^ 0x80008000u;
        }
    }
    // A operand: lane (i, g) element t = x[16 h + 8 g + t][i + 32 blk + 64 b6 + 128 u],
    // the 16-byte slot of octet 2 h + g at the swizzled column
    const u32x4_t* ab[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int hs = ((il >> 3) + 4 * blk) & 7;
        ab[blk] = reinterpret_cast<const u32x4_t*>(smem + opaque(4 * (g * M + (il & ~7) + 32 * blk + ((il & 7) ^ hs))));
    }
    f32x16_t d[4];   // tile blk + 2 b6
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool neg = __builtin_popcount(u & W) & 1;   // H_U[u][W]
#pragma unroll
        for (int h = 0; h < HALVES; ++h) {
            const bf16x8_t B = __builtin_bit_cast(bf16x8_t, neg ? bn[h] : bp[h]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int blk = t & 1, b6 = t >> 1;
                const bf16x8_t A = __builtin_bit_cast(bf16x8_t, ab[blk][2 * h * M + 64 * b6 + 128 * u]);
                if (u == 0 && h == 0)
                    d[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, f32x16_t{}, 0, 0, 0);
                else
                    d[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, d[t], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[16 * t + r] = d[t][r];
}

// kkron_mix for the wave-uniform output block w: one instance per block,
// so the signs H_U[u][w] are compile-time constants.
template <int W, int NW, int HALVES, int LOGM>
__device__ __forceinline__ void kkron_mix_sel(int w, const uint32_t* smem, int lane, float (&v)[64]) {
    if constexpr (W + 1 < NW) {
        if (w == W)
            kkron_mix<W, HALVES, LOGM>(smem, lane, v);
        else
            kkron_mix_sel<W + 1, NW, HALVES, LOGM>(w, smem, lane, v);
    } else {
        kkron_mix<W, HALVES, LOGM>(smem, lane, v);
    }
}

// Element index of column 8 m + q (m, q < 8) within the lane's 64-column run.
__host__ __device__ constexpr int kron_elem(int m, int q) {
    return (q & 3) | ((m & 3) << 2) | ((m >> 2) << 4) | ((q >> 2) << 5);
}

// INT4 g128 epilogue of the lane's 64 consecutive columns (the other 64 of
// the group in lane l ^ 32). Arithmetic as in epi_int. cp: the 32 code bytes;
// gidx: group index.  Returns the group's zero point (0 if symmetric); the
// caller packs zero points.
template <class Q>
__device__ __forceinline__ uint32_t epi_kron(const float (&u)[64], float f, const QuantDev& q, uint8_t* cp,
                                             int64_t gidx, bool valid, bool first) {
    static_assert(Q::logg == 7, "groups of 128 columns");
    float s, zf = 0.0f;
    float umax = 0.0f, umin = 0.0f;   // the lane's extremes of u (asymmetric)
    if constexpr (Q::sym) {
        float am = fabsf(u[0]);
#pragma unroll
        for (int j = 1; j < 64; ++j) am = fmaxf(am, fabsf(u[j]));
        am = max_halves(am);
        s = (am * f) * (1.0f / 7.0f);
    } else {
        float hi = u[0], nl = -u[0];
#pragma unroll
        for (int j = 1; j < 64; ++j) {
            hi = fmaxf(hi, u[j]);
            nl = fmaxf(nl, -u[j]);
        }
        umax = hi;
        umin = -nl;
        // after the swap, max(hi, nl) is the group's max y in lanes 0-31 and
        // its -min y in lanes 32-63; a second swap hands each to every lane
        swap_halves(hi, nl);
        float mhi = fmaxf(hi, nl);
        float mnl = mhi;
        swap_halves(mhi, mnl);
        hi = fmaxf(mhi, 0.0f) * f;
        nl = fmaxf(mnl, 0.0f) * f;  // -min(min y, 0)
        s = (hi + nl) * (1.0f / 15.0f);
        zf = nl;
    }
    uint32_t sbits = f2bf(s);
    s = bf2f(sbits);
    if (s == 0.0f) {
        s = 1.0f;
        sbits = 0x3F80u;
    }
    const float rs = __builtin_amdgcn_rcpf(s);
    const float inv = f * rs;
    uint32_t w[8];
    uint32_t zret = 0;
    if constexpr (Q::sym) {
        const float off = kMagic + 8.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            float t[8];
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) t[qq] = fmaf(u[kron_elem(m, qq)], inv, off);
            w[m] = pack8(t) ^ 0x88888888u;
        }
    } else {
        const float z = fminf(fmaxf(rintf(zf * rs), 0.0f), 15.0f);
        const uint32_t zi = static_cast<uint32_t>(z);
        const uint32_t zmul = zi * 0x1111u;
        const float lo = kMagic - z, hi = kMagic + 15.0f - z;
        codes_asym<8>([&](int m, int qq) { return u[kron_elem(m, qq)]; }, inv, lo, hi, zmul, umax, umin, w);
        zret = zi;
    }
    if (valid) {
        // ordinary stores: the four quarters of a 128-byte line of codes come
        // from four waves, and the L2 merges them (streaming stores of these
        // pieces wrote 1.48 times the code bytes to HBM)
        stg16c(cp, u32x4_t{w[0], w[1], w[2], w[3]});
        stg16c(cp + 16, u32x4_t{w[4], w[5], w[6], w[7]});
        if (first) static_cast<uint16_t*>(q.scales)[gidx] = static_cast<uint16_t>(sbits);
    }
    return zret;
}

template <int K, int LOGM, bool WROT, class Q0>
__global__ void __launch_bounds__(64 * (1 << LOGM) / 128, (16 * 128 >> LOGM) < 4 ? (16 * 128 >> LOGM) : 4)
kkron(const KronArgs a) {
    static_assert(K <= 32, "one MFMA K-padding of 32");
    static_assert(LOGM >= 8 && LOGM <= 10, "pieces of 256, 512 or 1024");
    constexpr int M = 1 << LOGM;
    constexpr int NW = M / 128;              // waves: one block of 128 output columns each
    constexpr int NT = 64 * NW;
    constexpr int n = K * M;
    // K <= 16: two rows per iteration, row r of the pair in piece slots
    // 16 r .. 16 r + 15 (the lanes of a half-wave, and the MFMA's input and
    // output dimensions), with H_K block-diagonal over the pair.  (The host
    // regroups K x M as 2K x M / 2 where M / 2 >= 256, so this serves rows of
    // K x 256, such as 3072 = 12 x 256.)
    constexpr int PACK = K <= 16 ? 2 : 1;
    constexpr int HALVES = 2;                // 16-slot halves of the contraction
    constexpr int OCT = 4;                   // staged slot octets
    constexpr int BT = 16 * M;               // B table offset, dwords (staging below)
    constexpr int ZB = BT + 512;             // zero-point bytes, NW per piece
    __shared__ uint32_t smem[ZB + 8 * NW];
    uint8_t* zbuf = reinterpret_cast<uint8_t*>(smem + ZB);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform

    // Staging pairs (slot octet, run of 8 columns): OCT * M / 8 of them, one
    // per thread.  Slot s of an octet is piece s (PACK = 1) or piece s % 16 of
    // row s / 16 of the pair (PACK = 2); slots without a piece stage zeros.
    const int so = tid / (M / 8);            // octet
    const int cg = tid % (M / 8);            // columns 8 cg .. 8 cg + 7
    const bool stager = so < OCT;
    const int srow = PACK == 2 ? so >> 1 : 0;             // row of the pair
    const int spc = PACK == 2 ? 8 * (so & 1) : 8 * so;    // first piece of the octet
    u32x4_t ld[8];
    auto load = [&](int64_t r0) {
        const int64_t r = r0 + srow;
        const bool rok = r < a.rows;
        const uint16_t* src = static_cast<const uint16_t*>(a.x) + (rok ? r : r0) * n + 8 * cg;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (rok && spc + j < K) ld[j] = ldg16(src + (spc + j) * M);
            else ld[j] = u32x4_t{0u, 0u, 0u, 0u};
        }
    };

    // B table entry e = lane' + 64 (p + 4 h): slot 16 h + 8 g + 2p (+1) of
    // input to slot c = lane' % 32 of output, g = lane' / 32, as packed bf16:
    // H_K of the two pieces (+-1), or 0 across the rows of a pair.  Never
    // overwritten.
    for (int e = tid; e < 512; e += NT) {
        const int c = e & 31, g = (e >> 5) & 1, p = (e >> 6) & 3, h = e >> 8;
        if (PACK == 2 && h != (c >> 4)) {
            smem[BT + e] = 0u;
        } else {
            const int co = PACK == 2 ? c & 15 : c;
            const int ri = PACK == 2 ? 8 * g + 2 * p : 16 * h + 8 * g + 2 * p;
            const uint32_t nb = static_cast<uint32_t>(a.hk_neg[co] >> ri);
            smem[BT + e] = 0x3F803F80u | ((nb & 1u) << 15) | ((nb & 2u) << 30);
        }
    }

    // Rows (pairs of rows for PACK = 2) blockIdx.x, blockIdx.x + gridDim.x,
    // ...  Each row is loaded just before it is staged: without a prefetch
    // the kernel fits 128 VGPRs, so four waves per SIMD hide one another's
    // load latency.
    int64_t row = static_cast<int64_t>(blockIdx.x) * PACK;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * PACK;
    const int c = lane & 31;                   // output slot
    const int g = lane >> 5;                   // column bit b6 after the mix
    const int pc = PACK == 2 ? c & 15 : c;     // piece of the slot
    const int prow = PACK == 2 ? c >> 4 : 0;   // row of the pair
    for (;;) {
        if (stager) load(row);
        // ---- phase 1: stage the row (16-byte slot of column 8 cg + cc at
        // 8 cg + (cc ^ (cg & 7)) within octet so)
        if (stager) {
            const int base = 16 * (so * M + 8 * cg);     // bytes
            const int hs16 = 16 * (cg & 7);
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_perm(ld[2 * j + 1][cc >> 1], ld[2 * j][cc >> 1], sel);
                *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(smem) + ((base | hs16) ^ (16 * cc))) = o;
            }
        }
        const int64_t next = row + stride;
        __syncthreads();

        // ---- phase 2: mix on the MFMA, six register stages, one across halves
        float v[64];
        kkron_mix_sel<0, NW, HALVES, LOGM>(w, smem, lane, v);
        // v[16 (blk + 2 b6) + r]: column b0, b1 = r & 3, b3, b4 = r >> 2, b5 = blk; b2 = lane / 32
        bfly<64, 0x3Fu>(v);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            float x0 = v[j], x1 = v[j + 32];
            swap_halves(x0, x1);      // (b6 = lane / 32; b2 = 0, 1)
            v[j] = x0 + x1;
            v[j + 32] = x0 - x1;
        }
        // v[j]: column 8 m + q of the run of 64 starting at 64 (g + 2 w),
        // with j = kron_elem(m, q)
        const bool valid = pc < K && row + prow < a.rows;
        const int64_t e0 = (row + prow) * n + pc * M + 64 * (g + 2 * w);
        if constexpr (WROT) {
            if (valid) {
                uint16_t* dst = static_cast<uint16_t*>(a.y_rot) + e0;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    u32x4_t o;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        o[p] = bf16x2(v[kron_elem(m, 2 * p)] * a.norm, v[kron_elem(m, 2 * p + 1)] * a.norm);
                    stg16c(dst + 8 * m, o);   // a lane's 8 pieces fill one line: merged in L2
                }
            }
        }
        if constexpr (Q0::fmt == 0) {
            const uint32_t zi = epi_kron<Q0>(v, a.norm, a.q, a.q.codes + (e0 >> 1), e0 >> 7, valid, valid && g == 0);
            if constexpr (!Q0::sym) {
                if (valid && g == 0) zbuf[NW * c + w] = static_cast<uint8_t>(zi);
            }
        }
        __syncthreads();   // operand reads and zero-point bytes done
        if constexpr (Q0::fmt == 0 && !Q0::sym) {
            // zero points of groups (2i, 2i + 1) -> one byte: NW / 2 per piece
            // (the groups of a piece are its NW column blocks, one per wave)
            constexpr int ZR = K * NW / 2;     // zero bytes per row
            for (int b = tid; b < PACK * ZR; b += NT) {
                const int r = b / ZR, bb = b % ZR;
                const int zpc = bb / (NW / 2), k2 = bb % (NW / 2);
                const uint8_t* zp = zbuf + NW * (16 * r * (PACK - 1) + zpc) + 2 * k2;
                if (row + r < a.rows) a.q.zeros[(row + r) * ZR + bb] = static_cast<uint8_t>(zp[0] | (zp[1] << 4));
            }
        }
        row = next;
        if (row >= a.rows) break;
    }
}

// ---------------------------------------------------------------- kkronw
// H_K[r][c] == -1 for the base matrix of `a` (dense bits for K <= 64, else
// the Paley I construction over the integers mod the prime q = K - 1: +1 on
// the diagonal and in row 0, -1 in column 0 below it, else the quadratic
// character of (r - c) mod q).
__device__ __forceinline__ bool kron_minus(const KronArgs& a, int r, int c) {
    if (a.kron_q == 0) return (a.hk_neg[c] >> r) & 1u;
    if (r == c || r == 0) return false;
    if (c == 0) return true;
    int d = r - c;
    if (d < 0) d += a.kron_q;
    return ((a.kron_chi[d >> 5] >> (d & 31)) & 1u) == 0u;
}

// Rows of n = K * 128 bf16 with 32 < K <= 160 (AutoRound "Rotation
// Transform", section 1.5: base orders such as 108 and 140 combined with a
// Sylvester block of 128): y = x (H_K (x) H_128) / sqrt(n).  One workgroup of
// NW = ceil(K / 32) waves per row, persistent over rows.  Write the row as
// x[a][b] (piece a < K, column b < 128).
// Staging: the row goes to LDS as 16 bytes per (piece octet, column), dword j
//   holding pieces 2j, 2j + 1 of the octet (as in kkron); octets past K are
//   zero.  Each wave stages four octets: lane (octet 4w + l / 16, columns
//   8 (l % 16) .. + 7).
// Mix: wave w owns output pieces c = 32 w + l % 32.  For each tile t of 32
//   columns, v_mfma_f32_32x32x16_bf16 over the 16-piece halves h:
//   D[col][c] += sum_a x[16 h + a][col] H_K[16 h + a][c], A = 32 columns by 16
//   pieces (one 16-byte LDS read per lane), B = the +-1 slice of H_K.  Exact
//   bf16 products, float32 sums.  For these base orders (q = K - 1 prime)
//   H_K is +1 in row 0, -1 in column 0 below it, and elsewhere a function
//   of (r - c) mod q.  So lane (c, g)'s B for half h, H_K[16 h + 8 g + t][c]
//   for t = 0..7, is one 16-byte entry of a table in LDS: entry o holds the
//   signs at (r - c) mod q = o .. o + 7 (mod q), entry q is all -1 (column
//   0), and row 0 is one element set to +1.  Rows past K meet zero A slots.
// Then the 128-point transform of each output piece: bits b0, b1, b3, b4
//   (tile rows) and b5, b6 (tiles) are register butterflies, b2 one
//   v_permlane32_swap stage, after which lane l holds the 64 consecutive
//   columns of piece c with b6 = l / 32 (the layout of kkron).
// Epilogue: INT g128 = one piece per group (lanes l, l ^ 32); zero points of
//   pieces c, c + 1 (lanes l, l ^ 1) share a byte.
template <int K, bool WROT, class Q0>
__global__ void __launch_bounds__(64 * ((K + 31) / 32), 4) kkronw(const KronArgs a) {
    static_assert(K > 32 && K <= 160 && K % 4 == 0, "base orders 36..160");
    constexpr int M = 128;
    constexpr int n = K * M;
    constexpr int NW = (K + 31) / 32;
    constexpr int KH = (K + 15) / 16;          // 16-piece halves of the contraction
    constexpr int NOCT = 2 * KH;               // staged octets
    static_assert(NOCT <= 4 * NW, "each wave stages four octets");
    constexpr int q = K - 1;
    __shared__ u32x4_t stage[NOCT * M];
    __shared__ u32x4_t btab[K];                 // entries 0 .. q - 1: windows; q: column 0
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = 32 * w + (lane & 31);         // output piece
    const int g = lane >> 5;
    const bool valid = c < K;

    // the sign table (read after the first staging barrier)
    for (int o = tid; o < K; o += 64 * NW) {
        u32x4_t e;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t dw = 0;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                int d = o + 2 * p + h2;
                if (d >= q) d -= q;
                // H_K at (1 + d, 1): the value at (r - c) mod q = d
                const bool minus = o == q || kron_minus(a, 1 + d, 1);
                dw |= (minus ? 0xBF80u : 0x3F80u) << (16 * h2);
            }
            e[p] = dw;
        }
        btab[o] = e;
    }
    // lane (c, g), half h: entry (16 h + 8 g - c) mod q, or q for column 0
    // (stepped from o0 inside the mix, which keeps one register live)
    int o0 = (8 * g - c) % q;
    if (o0 < 0) o0 += q;
    // A operand bases: lane (i, g) of tile t reads octet 2 h + g at column
    // i + 32 t, slot (col & ~7) + ((col & 7) ^ ((col >> 3) & 7)); the swizzle
    // depends on t & 1 only
    const int il = lane & 31;
    const u32x4_t* ab[2];
#pragma unroll
    for (int t1 = 0; t1 < 2; ++t1) {
        const int hs = ((il >> 3) + 4 * t1) & 7;
        ab[t1] = stage + opaque(g * M + (il & ~7) + 32 * t1 + ((il & 7) ^ hs));
    }
    // staging role: octet so = 4 w + l / 16, columns 8 cg .. 8 cg + 7
    const int so = 4 * w + (lane >> 4);
    const int cg = lane & 15;
    const bool stager = so < NOCT;

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        if (stager) {
            const uint16_t* src = static_cast<const uint16_t*>(a.x) + row * n + 8 * cg;
            u32x4_t ld[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int pc = 8 * so + j;
                ld[j] = pc < K ? ldg16(src + pc * M) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_perm(ld[2 * j + 1][cc >> 1], ld[2 * j][cc >> 1], sel);
                stage[so * M + 8 * cg + (cc ^ (cg & 7))] = o;
            }
        }
        __syncthreads();

        f32x16_t d[4];   // tile t = b5 + 2 b6
        int o = o0;
#pragma unroll
        for (int h = 0; h < KH; ++h) {
            u32x4_t bw = btab[c == 0 ? q : o];
            o += 16;
            if (o >= q) o -= q;
            if (h == 0 && g == 0) bw[0] = (bw[0] & 0xFFFF0000u) | 0x3F80u;   // row 0: +1
            const bf16x8_t B = __builtin_bit_cast(bf16x8_t, bw);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8_t A = __builtin_bit_cast(bf16x8_t, ab[t & 1][2 * h * M + 64 * (t >> 1)]);
                if (h == 0)
                    d[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, f32x16_t{}, 0, 0, 0);
                else
                    d[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, d[t], 0, 0, 0);
            }
        }
        float v[64];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) v[16 * t + r] = d[t][r];
        // v[16 t + r]: column b0, b1 = r & 3, b3, b4 = r >> 2, b5, b6 = t; b2 = lane / 32
        bfly<64, 0x3Fu>(v);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            float x0 = v[j], x1 = v[j + 32];
            swap_halves(x0, x1);      // (b6 = lane / 32; b2 = 0, 1)
            v[j] = x0 + x1;
            v[j + 32] = x0 - x1;
        }
        const int64_t e0 = row * n + c * M + 64 * g;
        if constexpr (WROT) {
            if (valid) {
                uint16_t* dst = static_cast<uint16_t*>(a.y_rot) + e0;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    u32x4_t o;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        o[p] = bf16x2(v[kron_elem(m, 2 * p)] * a.norm, v[kron_elem(m, 2 * p + 1)] * a.norm);
                    stg16c(dst + 8 * m, o);   // a lane's 8 pieces fill one line: merged in L2
                }
            }
        }
        if constexpr (Q0::fmt == 0) {
            const uint32_t zi = epi_kron<Q0>(v, a.norm, a.q, a.q.codes + (e0 >> 1), e0 >> 7, valid, valid && g == 0);
            if constexpr (!Q0::sym) {
                // pieces c, c + 1 (K even) -> one byte, written by the even one
                const uint32_t zodd = dppu<kXor1>(zi);
                if (valid && g == 0 && (c & 1) == 0)
                    a.q.zeros[(row * K + c) >> 1] = static_cast<uint8_t>((zi & 0xFu) | ((zodd & 0xFu) << 4));
            }
        }
        __syncthreads();   // operand reads done before the next row is staged
    }
}

// ----------------------------------------------------------- kb32 / kb16
// Blocks of 32 (rotation_size 32, the MX block; MXFP4 codes or rotated bf16)
// and of 16 (the NVFP block; NVFP4 codes or rotated bf16).
// v_mfma_f32_16x16x32_bf16 with B = the data: column j is 32 consecutive
// elements of a run of 512 (one block of 32, or two of 16) and lane
// (j, g = lane / 16) holds its elements 8 g .. 8 g + 7, one 16-byte load (so
// each load instruction reads 1 KiB of consecutive bytes). Two MFMAs (A = the
// two row halves of H_32, or of blockdiag(H_16, H_16), rows permuted) give
// lane (j, g) the outputs 8 g .. 8 g + 7 of column j: D row 4 g + r of half h
// is output 8 g + 4 h + r. The whole transform is exact bf16 x +-1 products
// summed in float32; no butterfly runs on the vector ALU. A block of 32 sits
// in lanes j, j + 16, j + 32, j + 48; a block of 16 in lanes l, l ^ 16.
// maximum over lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float max_quad16(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));   // xor 16
    return max_halves(v);
}

template <int LOGB, bool WROT, class Q0>
__global__ void __launch_bounds__(256) kbsmall(const FastArgs a) {
    static_assert(LOGB == 4 || LOGB == 5, "blocks of 16 or 32");
    static_assert(Q0::fmt < 0 || (LOGB == 5 && Q0::fmt == 1) || (LOGB == 4 && Q0::fmt == 2),
                  "MXFP4 on blocks of 32, NVFP4 on blocks of 16, or rotation only");
    constexpr int CH = 8;                       // runs of 512 elements per wave
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t runs = a.units >> (9 - LOGB);  // units: blocks (a whole number of runs)
    const int64_t run0 = wave * CH;
    if (run0 >= runs) return;
    const int j = lane & 15, g = lane >> 4;
    const uint32_t* tw = LOGB == 5 ? &kH32.w[0][lane][0] : &kH16x2.w[0][lane][0];
    const u32x4_t* hp = reinterpret_cast<const u32x4_t*>(tw);   // hp[64]: the second row half
    const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, hp[0]);
    const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, hp[64]);
    const uint16_t* src = static_cast<const uint16_t*>(a.x);
    const int lo = 32 * j + 8 * g;              // the lane's first element within a run
    u32x4_t raw[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        // a run past the end re-reads the first (finite data, never stored)
        const int64_t run = run0 + c < runs ? run0 + c : run0;
        raw[c] = ldg16(src + run * 512 + lo);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, raw[c]);
        const f32x4v_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, f32x4v_t{}, 0, 0, 0);
        const f32x4v_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, f32x4v_t{}, 0, 0, 0);
        float y[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            y[r] = d0[r] * a.norm;
            y[4 + r] = d1[r] * a.norm;
        }
        const bool store = run0 + c < runs;
        const int64_t e0 = (run0 + c) * 512 + lo;     // first of the lane's 8 elements
        if constexpr (WROT) {
            if (store)
                stg16(static_cast<uint16_t*>(a.y_rot) + e0,
                      u32x4_t{bf16x2(y[0], y[1]), bf16x2(y[2], y[3]), bf16x2(y[4], y[5]), bf16x2(y[6], y[7])});
        }
        if constexpr (Q0::fmt == 1) {
            float am = fabsf(y[0]);
#pragma unroll
            for (int r = 1; r < 8; ++r) am = fmaxf(am, fabsf(y[r]));
            am = max_quad16(am);
            const int ex = static_cast<int>((__float_as_uint(am) >> 23) & 0xFFu);
            const int e = (ex == 0) ? -127 : ex - 129;  // floor(log2 amax) - 2, >= -127
            uint32_t wc;
            // 2^-127 is not a normal float: such a block is multiplied by 2^64
            // and divided by 2^-63 instead, both exact (uniform branch).
            if (__builtin_amdgcn_ballot_w64(e == -127) == 0) {
                wc = cvt8_fp4(y, __uint_as_float(static_cast<uint32_t>(e + 127) << 23), 1.0f, false);
            } else {
                const bool tiny = e == -127;
                const float sc = tiny ? __uint_as_float(64u << 23) : __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
                const float pre = tiny ? __uint_as_float(191u << 23) : 1.0f;
                wc = cvt8_fp4(y, sc, pre, true);
            }
            if (store) {
                *reinterpret_cast<uint32_t*>(a.q[0].codes + (e0 >> 1)) = wc;
                if (g == 0) static_cast<uint8_t*>(a.q[0].scales)[e0 >> 5] = static_cast<uint8_t>(e + 127);
            }
        }
        if constexpr (Q0::fmt == 2) {
            // NVFP4: E4M3 byte of amax / (6 g); codes of y / s, s = E4M3 g, by
            // the converter at scale 1 (a zero byte stores zero codes)
            float am = fabsf(y[0]);
#pragma unroll
            for (int r = 1; r < 8; ++r) am = fmaxf(am, fabsf(y[r]));
            am = fmaxf(am, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(am), 0x401F)));   // xor 16
            const float ts = a.q[0].tscale;
            const uint32_t byte = e4m3_byte(am / (6.0f * ts));
            const float sc = e4m3_value(byte) * ts;
            const float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
            float t[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) t[r] = y[r] * inv;
            uint32_t wc = cvt8_fp4(t, 1.0f, 1.0f, false);
            if (!(sc > 0.0f)) wc = 0u;
            if (store) {
                *reinterpret_cast<uint32_t*>(a.q[0].codes + (e0 >> 1)) = wc;
                if ((g & 1) == 0) static_cast<uint8_t*>(a.q[0].scales)[e0 >> 4] = static_cast<uint8_t>(byte);
            }
        }
    }
}

// ------------------------------------------------------------- dispatch

template <class Q>
bool qmatch(const FastKey& k, int i) {
    if (Q::fmt < 0) return i >= k.nq;
    return i < k.nq && k.fmt[i] == Q::fmt && k.logg[i] == Q::logg && k.sdt[i] == Q::sdt &&
           (Q::fmt >= 1 || k.sym[i] == Q::sym);
}

template <int LOGB, bool WROT, class Q0, class Q1, int MIX = 0>
int try_kwave(const FastKey& k, const FastArgs& a, hipStream_t s) {
    if (k.logb != LOGB || k.wrot != (WROT ? 1 : 0) || k.mixed != MIX || !qmatch<Q0>(k, 0) || !qmatch<Q1>(k, 1))
        return 0;
    constexpr int64_t bpw = LOGB <= 12 ? 4096 >> LOGB : 1;
    if constexpr (MIX == 2) {
        // one workgroup per row, its waves owning 4096 elements each
        if ((a.row_blocks << LOGB) > 16384 || (reinterpret_cast<uintptr_t>(a.perm) & 15) != 0) return 0;
        const int64_t rows = a.units / a.row_blocks;
        const int wpr = static_cast<int>((a.row_blocks + bpw - 1) / bpw);
        hipLaunchKernelGGL((kwave<LOGB, WROT, Q0, Q1, MIX>), dim3(static_cast<unsigned>(rows)), dim3(64 * wpr), 0, s, a);
        const hipError_t e = hipGetLastError();
        return e == hipSuccess ? 1 : -static_cast<int>(e);
    }
    // blocks of 8192: two waves per block
    const int64_t waves = LOGB == 13 ? 2 * a.units : (a.units + bpw - 1) / bpw;
    const int64_t grid = (waves + 3) / 4;
    hipLaunchKernelGGL((kwave<LOGB, WROT, Q0, Q1, MIX>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 1 : -static_cast<int>(e);
}

template <bool WROT, class Q0>
int try_k128(const FastKey& k, const FastArgs& a, hipStream_t s) {
    if (k.mixed || k.logb != 7 || k.wrot != (WROT ? 1 : 0) || !qmatch<Q0>(k, 0) || k.nq > 1) return 0;
    if constexpr (!WROT && Q0::fmt == 0) {
        // quantised without a rotated output: sixteen rows per wave
        const int64_t grid = (a.units + 63) / 64;
        hipLaunchKernelGGL((k128q<Q0>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    } else {
        constexpr int64_t rows_per_block = 32 * k128_groups<Q0>();
        const int64_t grid = (a.units + rows_per_block - 1) / rows_per_block;
        hipLaunchKernelGGL((k128<WROT, Q0>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 1 : -static_cast<int>(e);
}

template <int LOGB, bool WROT, class Q0>
int try_kbsmall(const FastKey& k, const FastArgs& a, hipStream_t s) {
    constexpr int64_t per_run = 512 >> LOGB;    // blocks per run of 512 elements
    if (k.mixed || k.logb != LOGB || k.wrot != (WROT ? 1 : 0) || !qmatch<Q0>(k, 0) || k.nq > 1 ||
        (a.units & (per_run - 1)) != 0)
        return 0;
    const int64_t waves = (a.units / per_run + 7) / 8;
    const int64_t grid = (waves + 3) / 4;
    hipLaunchKernelGGL((kbsmall<LOGB, WROT, Q0>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 1 : -static_cast<int>(e);
}

template <int K, int LOGM, bool WROT, class Q0>
int try_kkron(const FastKey& k, const KronArgs& a, hipStream_t s) {
    if (a.k != K || k.logb != LOGM || k.wrot != (WROT ? 1 : 0) || !qmatch<Q0>(k, 0) || k.nq > 1) return 0;
    constexpr int NT = 64 * (1 << LOGM) / 128;
    // persistent grid: as many workgroups as the device holds at once
    static std::atomic<int> slots[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -static_cast<int>(hipErrorInvalidDevice);
    int cap = slots[dev].load(std::memory_order_relaxed);
    if (cap == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kkron<K, LOGM, WROT, Q0>, NT, 0) != hipSuccess)
            return -static_cast<int>(hipErrorInvalidValue);
        cap = cus * (per > 0 ? per : 1);
        slots[dev].store(cap, std::memory_order_relaxed);
    }
    const int64_t units = K <= 16 ? (a.rows + 1) / 2 : a.rows;   // rows, or pairs of rows (K <= 16)
    const int64_t grid = units < cap ? units : cap;
    hipLaunchKernelGGL((kkron<K, LOGM, WROT, Q0>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 1 : -static_cast<int>(e);
}

template <int K, bool WROT, class Q0>
int try_kkronw(const FastKey& k, const KronArgs& a, hipStream_t s) {
    if (a.k != K || k.wrot != (WROT ? 1 : 0) || !qmatch<Q0>(k, 0) || k.nq > 1) return 0;
    constexpr int NT = 64 * ((K + 31) / 32);
    static std::atomic<int> slots[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -static_cast<int>(hipErrorInvalidDevice);
    int cap = slots[dev].load(std::memory_order_relaxed);
    if (cap == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kkronw<K, WROT, Q0>, NT, 0) != hipSuccess)
            return -static_cast<int>(hipErrorInvalidValue);
        cap = cus * (per > 0 ? per : 1);
        slots[dev].store(cap, std::memory_order_relaxed);
    }
    const int64_t grid = a.rows < cap ? a.rows : cap;
    hipLaunchKernelGGL((kkronw<K, WROT, Q0>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 1 : -static_cast<int>(e);
}

using IS128B = QD<0, 1, 7, 1>;   // INT sym g128 bf16 scales
using IA128B = QD<0, 0, 7, 1>;   // INT asym g128 bf16 scales
using IS128F = QD<0, 1, 7, 0>;
using IA128F = QD<0, 0, 7, 0>;
using IS32B = QD<0, 1, 5, 1>;     // INT groups of 32, 64, 256 (bf16 scales)
using IA32B = QD<0, 0, 5, 1>;
using IS64B = QD<0, 1, 6, 1>;
using IA64B = QD<0, 0, 6, 1>;
using IS256B = QD<0, 1, 8, 1>;
using IA256B = QD<0, 0, 8, 1>;
using MX = QD<1, 1, 5, 2>;       // MXFP4
using NV = QD<2, 1, 4, 3>;       // NVFP4

}  // namespace
int launch_kron(const FastKey& k, const KronArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int r = 0;
#define HR_TRY(expr) \
    if ((r = (expr)) != 0) return r
    if (k.logb == 7) {
        // rows of K x 128, 32 < K <= 160
        HR_TRY((try_kkronw<108, false, IA128B>(k, a, s)));
        HR_TRY((try_kkronw<108, false, IS128B>(k, a, s)));
        HR_TRY((try_kkronw<108, true, QNone>(k, a, s)));
        HR_TRY((try_kkronw<108, true, IA128B>(k, a, s)));
        HR_TRY((try_kkronw<108, true, IS128B>(k, a, s)));
        HR_TRY((try_kkronw<140, false, IA128B>(k, a, s)));
        HR_TRY((try_kkronw<140, false, IS128B>(k, a, s)));
        HR_TRY((try_kkronw<140, true, QNone>(k, a, s)));
        HR_TRY((try_kkronw<140, true, IA128B>(k, a, s)));
        HR_TRY((try_kkronw<140, true, IS128B>(k, a, s)));
        HR_TRY((try_kkronw<60, false, IA128B>(k, a, s)));
        HR_TRY((try_kkronw<60, false, IS128B>(k, a, s)));
        HR_TRY((try_kkronw<60, true, QNone>(k, a, s)));
        return 0;
    }
    // rows of K x 512
    HR_TRY((try_kkron<28, 9, false, IA128B>(k, a, s)));
    HR_TRY((try_kkron<28, 9, true, IA128B>(k, a, s)));
    HR_TRY((try_kkron<28, 9, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<28, 9, true, IS128B>(k, a, s)));
    HR_TRY((try_kkron<28, 9, true, QNone>(k, a, s)));
    HR_TRY((try_kkron<24, 9, false, IA128B>(k, a, s)));   // 12 x 1024, regrouped
    HR_TRY((try_kkron<24, 9, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<24, 9, true, QNone>(k, a, s)));
    HR_TRY((try_kkron<20, 9, false, IA128B>(k, a, s)));
    HR_TRY((try_kkron<20, 9, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<20, 9, true, QNone>(k, a, s)));
    // rows of K x 256 (e.g. 5120 = 20 x 256)
    HR_TRY((try_kkron<20, 8, false, IA128B>(k, a, s)));
    HR_TRY((try_kkron<20, 8, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<20, 8, true, QNone>(k, a, s)));
    HR_TRY((try_kkron<12, 8, false, IA128B>(k, a, s)));
    HR_TRY((try_kkron<12, 8, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<12, 8, true, QNone>(k, a, s)));
    HR_TRY((try_kkron<24, 8, false, IA128B>(k, a, s)));   // 12 x 512, regrouped
    HR_TRY((try_kkron<24, 8, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<24, 8, true, QNone>(k, a, s)));
    HR_TRY((try_kkron<28, 8, false, IA128B>(k, a, s)));
    HR_TRY((try_kkron<28, 8, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<28, 8, true, QNone>(k, a, s)));
    // rows of K x 1024 (e.g. 20480 = 20 x 1024)
    HR_TRY((try_kkron<20, 10, false, IA128B>(k, a, s)));
    HR_TRY((try_kkron<20, 10, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<20, 10, true, QNone>(k, a, s)));
    HR_TRY((try_kkron<28, 10, false, IA128B>(k, a, s)));
    HR_TRY((try_kkron<28, 10, false, IS128B>(k, a, s)));
    HR_TRY((try_kkron<28, 10, true, QNone>(k, a, s)));
#undef HR_TRY
    return 0;
}


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
    // 8192-wide blocks (a pair of waves per block)
    HR_TRY((try_kwave<13, false, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<13, true, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<13, false, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<13, true, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<13, true, MX, IS128B>(k, a, s)));
    HR_TRY((try_kwave<13, false, MX, IS128B>(k, a, s)));
    HR_TRY((try_kwave<13, true, QNone, QNone>(k, a, s)));
    // 1024-wide blocks (four per wave)
    HR_TRY((try_kwave<10, false, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<10, true, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<10, false, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<10, true, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<10, true, QNone, QNone>(k, a, s)));
    // INT groups of 32, 64 and 256 on 2048- and 4096-wide blocks
    HR_TRY((try_kwave<11, false, IA32B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, false, IS32B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, false, IA64B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, false, IS64B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, false, IA256B, QNone>(k, a, s)));
    HR_TRY((try_kwave<11, false, IS256B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, false, IA32B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, false, IS32B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, false, IA64B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, false, IS64B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, false, IA256B, QNone>(k, a, s)));
    HR_TRY((try_kwave<12, false, IS256B, QNone>(k, a, s)));
    // 512-, 256- and 64-wide blocks (8, 16 or 64 per wave)
    HR_TRY((try_kwave<9, false, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<9, true, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<9, false, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<9, true, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<9, false, MX, QNone>(k, a, s)));
    HR_TRY((try_kwave<9, true, QNone, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, false, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, true, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, false, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, true, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, false, MX, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, true, QNone, QNone>(k, a, s)));
    HR_TRY((try_kwave<6, false, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<6, true, IA128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<6, false, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<6, true, IS128B, QNone>(k, a, s)));
    HR_TRY((try_kwave<6, false, MX, QNone>(k, a, s)));
    HR_TRY((try_kwave<6, true, QNone, QNone>(k, a, s)));
    // one group per block (R3 per head vector for head_dim 64 or 256)
    HR_TRY((try_kwave<6, false, IA64B, QNone>(k, a, s)));
    HR_TRY((try_kwave<6, false, IS64B, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, false, IA256B, QNone>(k, a, s)));
    HR_TRY((try_kwave<8, false, IS256B, QNone>(k, a, s)));
    // randomised rotations: signs (random Hadamard), permutation + signs (RPBH)
    HR_TRY((try_kwave<12, false, IS128B, QNone, 1>(k, a, s)));
    HR_TRY((try_kwave<12, false, IA128B, QNone, 1>(k, a, s)));
    HR_TRY((try_kwave<12, true, MX, IS128B, 1>(k, a, s)));
    HR_TRY((try_kwave<12, true, QNone, QNone, 1>(k, a, s)));
    HR_TRY((try_kwave<11, false, IA128B, QNone, 1>(k, a, s)));
    HR_TRY((try_kwave<11, false, IS128B, QNone, 1>(k, a, s)));
    HR_TRY((try_kwave<11, true, QNone, QNone, 1>(k, a, s)));
    HR_TRY((try_kwave<12, false, IS128B, QNone, 2>(k, a, s)));
    HR_TRY((try_kwave<12, false, IA128B, QNone, 2>(k, a, s)));
    HR_TRY((try_kwave<12, true, QNone, QNone, 2>(k, a, s)));
    HR_TRY((try_kwave<11, false, IA128B, QNone, 2>(k, a, s)));
    HR_TRY((try_kwave<11, false, IS128B, QNone, 2>(k, a, s)));
    HR_TRY((try_kwave<11, true, QNone, QNone, 2>(k, a, s)));
    // 128-wide rows
    HR_TRY((try_k128<true, QNone>(k, a, s)));
    HR_TRY((try_k128<false, IA128B>(k, a, s)));
    HR_TRY((try_k128<true, IA128B>(k, a, s)));
    HR_TRY((try_k128<false, IS128B>(k, a, s)));
    HR_TRY((try_k128<true, IS128B>(k, a, s)));
    // blocks of 32
    HR_TRY((try_kbsmall<5, false, MX>(k, a, s)));
    HR_TRY((try_kbsmall<5, true, MX>(k, a, s)));
    HR_TRY((try_kbsmall<5, true, QNone>(k, a, s)));
    HR_TRY((try_kbsmall<4, false, NV>(k, a, s)));
    HR_TRY((try_kbsmall<4, true, NV>(k, a, s)));
    HR_TRY((try_kbsmall<4, true, QNone>(k, a, s)));
#undef HR_TRY
    return 0;
}

}  // namespace hr
