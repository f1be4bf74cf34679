/*
 * hadarot -- Hadamard rotation fused with group quantization, for MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain pointers and sizes, returns an int
 * status (hr_status), and enqueues its work asynchronously on the HIP stream
 * passed as `stream` (a hipStream_t cast to void*; NULL = the null stream).
 *
 * Operations (cited by page title and section):
 *   - Orthogonal rotation y = x . R, applied to the last dimension of a
 *     row-major tensor.  R is a Sylvester Hadamard matrix normalised by
 *     1/sqrt(size) (AutoRound "Rotation Transform", section 1.5), applied
 *     block-diagonally with a power-of-two block (the same page, sections
 *     1.2 `rotation_size` and 2.1 `block_size`), or, for a full-width
 *     rotation of a width that is not a power of two, the Kronecker product
 *     of a base Hadamard matrix of order K with a Sylvester matrix
 *     (section 1.5).  Because R R^T = I, x R (W R)^T = x W^T (the page's
 *     introduction), so the same call serves the online activation side and
 *     the offline weight side (section 1.1, online vs offline).
 *   - Group round-to-nearest quantization with the (wbits, groupsize, sym)
 *     specification (OneCompression "Pre-Process", Workflow note; orbitquant
 *     0.2.0, Method Conformance: INT4 group RTN), MXFP4 with blocks of 32
 *     and NVFP4 with blocks of 16 (AutoRound page, sections 2 and 2.1).
 *
 * Conventions shared by every call
 *   - Tensors are contiguous row-major; the rotated dimension n is the last
 *     one and leading dimensions are flattened into `rows` (orbitquant 0.2.0,
 *     "Quantize An Instantiated Module": arbitrary leading dims, final dim =
 *     features).  Weights are [out_features, in_features] and are rotated
 *     along in_features.
 *   - Rotation arithmetic is float32 (AutoRound page, section 1.2, `dtype`),
 *     with one normalisation by 1/sqrt(block) (or 1/sqrt(n) for the
 *     Kronecker form).  Quantizers see the unrounded float32 rotated values,
 *     not a bfloat16-rounded copy.
 *   - Groups are contiguous runs of group_size elements along the last
 *     dimension.  Symmetric: s = amax / (2^(b-1) - 1), q = clamp(rne(y/s),
 *     -2^(b-1), 2^(b-1)-1).  Asymmetric: lo = min(min y, 0), hi = max(max y,
 *     0), s = (hi - lo) / (2^b - 1), z = clamp(rne(-lo/s), 0, 2^b - 1),
 *     q = clamp(rne(y/s) + z, 0, 2^b - 1).  s is rounded (to nearest even) to
 *     the scale dtype and the stored value is used for the codes; an all-zero
 *     group stores s = 1.  rne = round half to even.
 *   - MXFP4: per 32 elements e = clamp(floor(log2 amax) - 2, -127, 127)
 *     (amax = 0 gives -127), stored as the E8M0 byte e + 127; each element is
 *     the E2M1 code of y / 2^e, round to nearest with ties to the even
 *     mantissa, saturating at +-6; code = sign << 3 | index, index 0..7 for
 *     magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; sign set iff y < 0.
 *   - Packing: 4-bit codes two per byte, element 2j in the low nibble
 *     (symmetric codes as two's complement nibbles), `rows * n / 2` bytes.
 *     Scales: rows * n / group_size values of the scale dtype (E8M0 and
 *     E4M3: bytes).
 *     Zero points (asymmetric only): uint4, two per byte over the row-major
 *     flattened group index, ceil(groups / 2) bytes, a trailing odd nibble
 *     set to 0.
 *   - Ownership: the caller allocates every buffer on the device of the
 *     stream, including dequant_check's statistics workspace, and keeps it
 *     alive until the stream work has completed.  The library keeps no
 *     pointer after returning and allocates no device memory.  Its only
 *     mutable state is the per-thread error text, per-device launch sizes
 *     cached on first use, and the process-wide dispatch switch of
 *     hr_set_generic_only.
 *   - Alignment: x, y, y_rot, w, w_rot and codes must be 16-byte aligned;
 *     scales and zeros naturally aligned.  Outputs may not overlap inputs or
 *     each other, except y == x (hadamard_rotate) and y_rot == x
 *     (rotate_quantize_act), which rotate in place.
 *   - Errors: every argument is checked before anything is enqueued, so on
 *     a non-zero status no output has been touched (all-or-nothing, as the
 *     AIMET SpinQuant page applies its passes: validate every pass, then
 *     mutate).  There is no fallback to another algorithm.  Faults inside a
 *     kernel surface at the caller's next synchronisation.  hr_last_error()
 *     returns the message of the last failing call on this thread.
 *   - rows == 0 is a valid empty tensor: the call returns HR_OK and enqueues
 *     nothing (pointers may then be NULL).
 *   - Graph capture: apart from dequant_check with `stats` (which copies
 *     to the host and synchronises), a call enqueues
 *     kernel launches only (no allocation, copy or memset), so it may be
 *     captured in a HIP graph and replayed.  The first call for a kernel on a
 *     device also queries the device's occupancy on the host; making one call
 *     before capturing keeps that query out of the capture (the tested use).
 */
#ifndef HADAROT_H
#define HADAROT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hr_status {
    HR_OK = 0,
    HR_EINVAL = -1,        /* bad argument: NULL, size, layout, alignment, aliasing */
    HR_EUNSUPPORTED = -2,  /* well-formed but not implemented (bits != 4, K > 160, ...) */
    HR_EDEVICE = -3        /* HIP runtime error while enqueueing */
} hr_status;

typedef enum hr_dtype {
    HR_F32 = 0,
    HR_BF16 = 1,
    HR_E8M0 = 2,           /* scales only: MXFP4 shared exponent byte */
    HR_E4M3 = 3            /* scales only: NVFP4 block scale byte (OCP e4m3fn) */
} hr_dtype;

typedef enum hr_qformat {
    HR_Q_INT = 0,          /* round-to-nearest integer groups */
    HR_Q_MXFP4 = 1,        /* E2M1 elements, E8M0 scale per 32 */
    HR_Q_NVFP4 = 2         /* E2M1 elements, E4M3 scale per 16, times a tensor scale */
} hr_qformat;

/* Quantizer specification: the pages' (wbits, groupsize, sym) plus format
 * and scale storage type.  INT: bits must be 4, group_size an even power of
 * two dividing n, scale_dtype HR_F32 or HR_BF16.  MXFP4: bits 4,
 * group_size 32, sym ignored, scale_dtype HR_E8M0.
 * NVFP4 (named on the AutoRound page, sections 2 and 2.1, with rotation
 * blocks of 16; the encoding is the public two-level one): bits 4,
 * group_size 16, sym ignored, scale_dtype HR_E4M3; tensor_scale g > 0 and
 * finite (0 means 1).  Block byte = E4M3 of amax / (6 g), nearest even,
 * saturating at 448; element codes = E2M1 of y / (E4M3 g), nearest even,
 * saturating at 6 (all 0 when the byte is 0).  tensor_scale is ignored by
 * the other formats. */
typedef struct hr_qspec {
    int32_t format;        /* hr_qformat */
    int32_t bits;
    int32_t group_size;
    int32_t sym;           /* 1 symmetric, 0 asymmetric (INT only) */
    int32_t scale_dtype;   /* hr_dtype */
    float tensor_scale;    /* NVFP4 only */
} hr_qspec;

/* Output buffers of one quantizer. zeros is NULL unless INT asymmetric. */
typedef struct hr_qout {
    void* codes;
    void* scales;
    void* zeros;
} hr_qout;

/* Statistics of a dequantization against a reference (dequant_check). */
typedef struct hr_dq_stats {
    double max_err_steps;      /* max |ref - deq| / local step */
    int64_t n_over_half_step;  /* elements with |ref - deq| > step / 2 */
    int64_t n_clamped;         /* elements outside the representable range */
    double rel_l2_err;         /* ||ref - deq||_2 / ||ref||_2 (0 if ref is 0) */
} hr_dq_stats;

/*
 * y = x . R on the last dimension (rotation only; the R3 query path and the
 * plain rotation of the AutoRound page, section 1.1).
 *   x, y   device, [rows, n] of `dtype` (HR_F32 or HR_BF16); y may equal x.
 *   block  > 0: block-diagonal Hadamard with blocks of `block` (a power of
 *          two dividing n, at most 32768); <= 0 or == n: full width, which is
 *          Sylvester if n is a power of two (n <= 32768), else the Kronecker
 *          form n = K * 2^m with K the smallest supported order K = odd(n) 2^j
 *          dividing n that has a Paley I construction (K - 1 a prime power
 *          = 3 mod 4), K <= 160 (above 64: K - 1 prime, e.g. 108 and 140),
 *          n <= 32768.  Specialised kernels take bfloat16 rows of K x 512
 *          (K <= 32) and K x 128 (K = 60, 108, 140); other Kronecker shapes,
 *          and float32, run the generic kernel, which for K > 64 needs LDS
 *          for two copies of the row (about 18000 elements at most).
 * Output is rounded to `dtype` (nearest even).
 */
int hadamard_rotate(const void* x, void* y, int dtype, int64_t rows, int64_t n,
                    int64_t block, void* stream);

/*
 * Online activation path (R1 residual stream, R3 keys, R4 down_proj input;
 * AutoRound page, sections 1.1 and 2, input mode): rotate x as in
 * hadamard_rotate and quantize the float32 rotated values with `q`.
 *   codes  device, rows * n / 2 bytes.
 *   scales device, rows * n / group_size elements of q->scale_dtype.
 *   zeros  device, ceil(rows * n / group_size / 2) bytes if INT asymmetric,
 *          else must be NULL.
 *   y_rot  device or NULL: if set, also writes the rotated tensor in `dtype`
 *          (may equal x).
 */
int rotate_quantize_act(const void* x, int dtype, int64_t rows, int64_t n, int64_t block,
                        const hr_qspec* q, void* codes, void* scales, void* zeros,
                        void* y_rot, void* stream);

/*
 * Offline weight fusion W' = W . R on in_features (AutoRound page, sections
 * 1 and 1.1: offline rotations are absorbed into the weights; section 2,
 * weight mode), with up to two quantized forms of W' from one read of W.
 *   w      device, [out_features, in_features] of `dtype`.
 *   w_rot  device or NULL: W' in `dtype` (may not alias w).
 *   q      array of nq quantizer specs (nq = 0, 1 or 2); outs[i] holds the
 *          buffers for q[i], sized as in rotate_quantize_act with
 *          rows = out_features, n = in_features.
 * At least one of w_rot and nq > 0 must be given.
 */
int rotate_fuse_weight(const void* w, int dtype, int64_t out_features, int64_t in_features,
                       int64_t block, void* w_rot, const hr_qspec* q, int nq,
                       const hr_qout* outs, void* stream);

/*
 * Output-side weight fusion W' = R^T . W along out_features (AutoRound page,
 * section 1.1: R1 fused into the outputs of o_proj / down_proj / embed when
 * online_r1_rotation is False, and R2 per head of head_dim rows on the v_proj
 * output).  For a layer y = x . W^T this gives y . R = x . W'^T.
 *   w      device, [out_features, in_features] of `dtype`.
 *   w_rot  device, the same shape and dtype; may equal w (in place), may not
 *          partially overlap it.
 *   block  > 0: R = blockdiag(H_block) / sqrt(block) over groups of `block`
 *          consecutive rows; <= 0 or == out_features: full width.  The block
 *          must be a power of two dividing out_features with 32 <= block <=
 *          4096, and in_features a multiple of max(8, 2048 / block):
 *          HR_EUNSUPPORTED otherwise (including full width on a
 *          non-power-of-two out_features).
 * out_features == 0 is an empty weight (HR_OK, nothing enqueued).
 * Output is rounded to `dtype` (nearest even).  Quantize W' along
 * in_features afterwards with rotate_fuse_weight and block = 1 (H_1 = 1).
 */
int rotate_fuse_weight_out(const void* w, int dtype, int64_t out_features, int64_t in_features,
                           int64_t block, void* w_rot, void* stream);

/*
 * Dequantize packed codes (orbitquant 0.2.0, "Packed Runtime": an explicit
 * dequantized reference mode for numerical debugging):
 *   INT symmetric q * s; INT asymmetric (q - z) * s; MXFP4 E2M1 * 2^e;
 *   NVFP4 E2M1 * E4M3 * tensor_scale.
 *   codes, scales, zeros  as written by the calls above for [rows, n].
 *   ref    device or NULL: [rows, n] of ref_dtype (HR_F32 / HR_BF16).
 *   deq    device or NULL: [rows, n] float32 output.
 *   stats  host or NULL: requires ref and work.  Filled after the stream
 *          has been synchronised (this call then blocks).  The local step is
 *          s for INT; for MXFP4 it is 2^e times the E2M1 spacing around
 *          |ref| / 2^e (0.5 below 2, 1 below 4, 2 above).  Clamped: INT
 *          ref/s (+ z) outside [qmin - 1/2, qmax + 1/2]; MXFP4 |ref| / 2^e > 6.
 *          The sums are reduced in a fixed order (per-workgroup partials,
 *          then one pass over them), so repeated calls give identical stats.
 *   work   device or NULL: HR_DQ_WORK_BYTES of scratch for the statistics
 *          reduction, 16-byte aligned, owned by the caller; required with
 *          stats, ignored without.  Its contents on entry do not matter;
 *          it may not overlap any other buffer of the call.
 * At least one of deq and stats must be given.
 */
#define HR_DQ_WORK_BYTES 65536
int dequant_check(const void* codes, const void* scales, const void* zeros,
                  const hr_qspec* q, int64_t rows, int64_t n, const void* ref,
                  int ref_dtype, float* deq, hr_dq_stats* stats, void* work,
                  void* stream);

/*
 * dequant_check without the `work` argument, for callers that cannot
 * allocate device memory (harnesses or serving loops that forbid hipMalloc):
 * the statistics partials go to a 64 KiB scratch array in the library's
 * device code, one copy per GPU, resolved on the first call on each device
 * and held until the process ends.  Nothing is allocated.  The scratch a call
 * needs does not grow with the input (at most 1025 partials of 40 bytes: the
 * grid is capped at 1024 workgroups, which stride over any size), so every
 * size dequant_check accepts fits; there is no size limit beyond its own.
 * Every call writes each scratch slot it reads, so nothing needs clearing
 * between calls.  Calls with `stats` on one GPU share that scratch: two such
 * calls in flight at once (other streams or other host threads) race, and
 * the caller must order them.  Without `stats` the call is dequant_check's
 * and touches no scratch.  Results equal dequant_check's bit for bit.
 */
int dequant_check_noalloc(const void* codes, const void* scales, const void* zeros,
                          const hr_qspec* q, int64_t rows, int64_t n, const void* ref,
                          int ref_dtype, float* deq, hr_dq_stats* stats, void* stream);

/*
 * Randomised rotations: the rotation becomes R' = P . D_in . R . D_out with
 *   P      the permutation with (x . P)[j] = x[perm[j]] (a gather),
 *   D_in   diag(in_signs), D_out = diag(out_signs) (+-1 entries),
 * so y = ((x gathered by perm) * in_signs) . R * out_signs, element j of a
 * row using perm[j], in_signs[j] and out_signs[j].  The random Hadamard of
 * the AutoRound page (section 1.5, "Random": H times diag(+-1) over
 * sqrt(N); section 1.2, random_r1..random_r4) is R . D_out; OrbitQuant's
 * RPBH (Method Conformance: permutation, Rademacher signs, block FWHT,
 * orthonormal scaling) is P . D_in . R.  Every member may be NULL (that
 * factor is the identity).
 *   perm       device, n int32, 4-byte aligned: a permutation of 0..n-1.
 *              Entries outside [0, n) are clamped into it (no fault); an
 *              array that is not a permutation gives an unspecified result.
 *   in_signs   device, n int8: negative means -1, anything else +1.
 *   out_signs  device, n int8: likewise.
 * n must be below 2^31.  The vectors are shared by every row and only read.  They may not overlap
 * an output.  With perm set, the rotation cannot run in place (y == x,
 * y_rot == x): HR_EINVAL.  The specialised kernels take mixed calls of
 * 2048- and 4096-blocks when the vectors are 16-byte aligned (or NULL) and,
 * with a permutation, n <= 16384; other mixed calls run the generic kernel.
 */
typedef struct hr_mix {
    const int32_t* perm;
    const int8_t* in_signs;
    const int8_t* out_signs;
} hr_mix;

/* hadamard_rotate, rotate_quantize_act and rotate_fuse_weight with the
 * rotation R' of hr_mix; mix == NULL is the plain call. */
int hadamard_rotate_mixed(const void* x, void* y, int dtype, int64_t rows, int64_t n,
                          int64_t block, const hr_mix* mix, void* stream);
int rotate_quantize_act_mixed(const void* x, int dtype, int64_t rows, int64_t n, int64_t block,
                              const hr_qspec* q, void* codes, void* scales, void* zeros,
                              void* y_rot, const hr_mix* mix, void* stream);
int rotate_fuse_weight_mixed(const void* w, int dtype, int64_t out_features, int64_t in_features,
                             int64_t block, void* w_rot, const hr_qspec* q, int nq,
                             const hr_qout* outs, const hr_mix* mix, void* stream);

/* Message of the last non-zero status returned on this thread ("" if none). */
const char* hr_last_error(void);

/*
 * Host-only query of the Kronecker factorisation the library uses for a
 * full-width rotation of a width n that is not a power of two: writes K and
 * M = n / K.  Returns HR_EUNSUPPORTED if no supported order exists, HR_EINVAL
 * for n <= 0 or a power of two.  Also, when `hk` is non-NULL, writes the K x K
 * base matrix entries (+1 / -1, row-major int8) the library applies.
 */
int hr_kron_order(int64_t n, int32_t* K, int64_t* M, int8_t* hk);

/*
 * Host-only query: the status that hadamard_rotate (nq = 0),
 * rotate_quantize_act (nq = 1) or rotate_fuse_weight (nq = 0..2) would
 * return for this dtype, shape, block and quantizer specs q[0..nq), from the
 * same argument checks and launch planning, before any pointer is looked at.
 * Touches no device.  rows <= 0 is planned as one row.  Lets a caller learn
 * whether a shape is implemented (HR_OK) or not (HR_EUNSUPPORTED, with the
 * reason in hr_last_error) before allocating anything.
 */
int hr_check_shape(int dtype, int64_t rows, int64_t n, int64_t block, const hr_qspec* q, int nq);

/*
 * Dispatch switch for testing: on != 0 sends every later call in the
 * process to the generic kernel, which handles every supported shape, even
 * where a specialised kernel matches; 0 (the default) restores the normal
 * dispatch.  Results agree within the tolerances of the library's tests,
 * not bit for bit.  Process-wide; not synchronised with calls in flight on
 * other threads.
 */
void hr_set_generic_only(int on);

#ifdef __cplusplus
}
#endif

#endif /* HADAROT_H */
