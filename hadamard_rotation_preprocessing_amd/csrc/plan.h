// Launch plan and kernel argument structs shared by the host dispatcher and
// the kernels.  Plain data only.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace hr {

// per-device launch caches (persistent grid sizes) hold this many devices
constexpr int kMaxDevices = 64;

constexpr int kMaxQuant = 2;
constexpr int kMaxKron = 160;      // largest Kronecker base order handled on the GPU
constexpr int kMaxKronDense = 64;  // orders up to this pass the whole base matrix

// One quantizer epilogue, resolved to device pointers.
struct QuantDev {
    int32_t format;       // 0 INT, 1 MXFP4, 2 NVFP4
    int32_t sym;          // INT: 1 symmetric, 0 asymmetric
    int32_t logg;         // log2(group_size)
    int32_t scale_dtype;  // 0 f32, 1 bf16, 2 e8m0, 3 e4m3
    float tscale;         // NVFP4 tensor scale g (1 otherwise)
    uint8_t* codes;
    void* scales;
    uint8_t* zeros;       // INT asymmetric only
};

// Arguments of the rotate(+quantize) kernel family.
struct RotArgs {
    const void* x;
    void* y_rot;              // nullable: rotated output in the input dtype
    int64_t total_chunks;     // chunks in the flattened tensor
    int64_t total_groups[kMaxQuant];
    float norm;               // 1/sqrt(block) or 1/sqrt(n) (Kronecker)
    int32_t logb;             // Hadamard block (Sylvester) or M (Kronecker) bits
    int32_t chunk;            // elements per chunk (C)
    int32_t tpc;              // threads per chunk (C / E)
    int32_t cpw;              // chunks per workgroup
    int32_t kron_k;           // 0: none; else the base order K (C = K * 2^logb)
    int32_t nq;
    QuantDev q[kMaxQuant];
    // Kronecker base matrix, by output column c: bit a of hk_neg[c] set iff
    // H_K[a][c] == -1, so that y_c = sum_a H_K[a][c] z_a (y = H_K^T z).
    // Orders above kMaxKronDense (prime q = K - 1 only) pass the quadratic
    // character of GF(q) instead: kron_q = q, bit d of kron_chi set iff d is
    // a nonzero square mod q (the matrix then follows from the Paley I
    // construction; kron_q = 0 means hk_neg holds the matrix).
    uint64_t hk_neg[kMaxKronDense];
    uint32_t kron_chi[kMaxKron / 32];
    int32_t kron_q;
    // randomised rotation (all nullable): element j of a row reads
    // x[perm[j]], is multiplied by in_signs[j] before and out_signs[j] after
    // the rotation; row_n is the row width n
    const int32_t* perm;
    const int8_t* in_signs;
    const int8_t* out_signs;
    int64_t row_n;
};

// Host-side plan.
struct RotPlan {
    int bf16;        // input/output dtype is bfloat16
    int loge;        // log2 elements per thread
    int kmax;        // 0, 16, 32, 64: register bound for the Kronecker mix;
                     // -1: orders above 64, mixed through a second LDS buffer
    int nt;          // threads per workgroup
    int64_t grid;    // workgroups
    size_t lds_bytes;
    RotArgs a;
};

struct DqArgs {
    const uint8_t* codes;
    const void* scales;
    const uint8_t* zeros;
    const void* ref;       // nullable
    float* deq;            // nullable
    void* parts;           // nullable: DqPartial[kDqMaxParts + 1] on the device (statistics)
    int64_t total;         // elements
    int32_t format, sym, logg, scale_dtype, ref_bf16;
    float tscale;          // NVFP4 tensor scale
};

// Statistics of dequant_check: one partial per workgroup of a grid of at
// most kDqMaxParts workgroups, then their sum (in a fixed order, so the
// result does not depend on scheduling) in slot kDqMaxParts.
struct DqPartial {
    double sum_err2;
    double sum_ref2;
    unsigned long long n_over;
    unsigned long long n_clamped;
    float max_err;
    uint32_t pad;
};
constexpr int kDqMaxParts = 1024;
constexpr size_t kDqWorkBytes = sizeof(DqPartial) * (kDqMaxParts + 1);
// static device scratch of dequant_check_noalloc (holds kDqWorkBytes)
constexpr size_t kDqScratchBytes = 65536;
static_assert(kDqWorkBytes <= kDqScratchBytes, "statistics partials fit the static scratch");

// Arguments of the specialised bfloat16 kernels (one wave per block).
struct FastArgs {
    const void* x;
    void* y_rot;              // nullable
    int64_t units;            // blocks (one wave each) or rows (128-wide kernel)
    int64_t total_groups[kMaxQuant];
    float norm;               // 1/sqrt(block)
    QuantDev q[kMaxQuant];
    // randomised rotation (kwave only; nullable): as in RotArgs, with
    // row_blocks = n / block
    const int32_t* perm;
    const int8_t* in_signs;
    const int8_t* out_signs;
    int64_t row_blocks;
};

// Arguments of the specialised Kronecker kernels (rows of K * 512 bf16 with
// K <= 32, or K * 128 with 32 < K <= 160).
struct KronArgs {
    const void* x;
    void* y_rot;              // nullable
    int64_t rows;
    int64_t total_groups;
    float norm;               // 1/sqrt(K * M)
    int32_t k;                // base order
    QuantDev q;
    // base matrix as in RotArgs: bit a of hk_neg[c] set iff H_K[a][c] == -1
    // (K <= 64), or the quadratic character of GF(q), q = kron_q = K - 1
    // prime (K > 64)
    uint64_t hk_neg[kMaxKronDense];
    uint32_t kron_chi[kMaxKron / 32];
    int32_t kron_q;
};

// Compile-time shape of a specialised kernel, matched at dispatch.
struct FastKey {
    int logb;                 // 5, 7, 11 or 12
    int wrot;                 // rotated output written
    int mixed;                // randomised rotation (perm / signs)
    int nq;
    int fmt[kMaxQuant], sym[kMaxQuant], logg[kMaxQuant], sdt[kMaxQuant];
};

// Output-side weight fusion (colrot.hip): W' = R^T W along out_features.
struct ColArgs {
    const void* w;
    void* w_rot;
    int64_t in;               // in_features (row length)
    int64_t row_blocks;       // out_features / b
    int64_t strips;           // in_features / C
    float norm;               // 1 / sqrt(b)
    int32_t logb;             // b = 2^logb, 5..12 (colrot); M = 2^logb (colwide)
    int32_t tb;               // tile of 2^tb elements (b C), 11..15 (colrot)
    int32_t bf16;
    // colwide (whole-height tiles of 4 columns): kron_k = K (1 for a
    // Sylvester block of 8192) and the base matrix, bit c of hk_neg[a] set
    // iff H_K[c][a] == -1
    int32_t kron_k;
    uint64_t hk_neg[32];
};

int launch_rotate(const RotPlan& p, void* stream);        // returns hipError_t
int launch_colrot(const ColArgs& a, void* stream);        // returns hipError_t
// Launches a specialised kernel if one matches `k`: returns 1 if launched,
// 0 if none matches, or a negative hipError_t on a launch error.
int launch_fast(const FastKey& k, const FastArgs& a, void* stream);
// Launches a specialised Kronecker kernel if one matches (bf16; K <= 32 with
// M = 512, or 32 < K <= 160 with M = 128; no quantizer or INT g128 with bf16
// scales): 1 launched, 0 no match, negative hipError_t on a launch error.
int launch_kron(const FastKey& k, const KronArgs& a, void* stream);
int launch_dequant(const DqArgs& a, void* stream);        // returns hipError_t
// Device address of the static scratch of the current device (resolved once
// per device); returns hipError_t.
int scratch_address(void** out);

}  // namespace hr
