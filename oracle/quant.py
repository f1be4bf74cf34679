"""Group quantizers evaluated element by element in float64 (oracle; test infrastructure only).

Sources (cited by page title and section):

* OneCompression "Pre-Process (Rotation Preprocessing)", the note under
  "Workflow": the round-to-nearest quantizer is specified by (wbits,
  groupsize, sym).
* orbitquant 0.2.0, "Method Conformance": INT4 group round-to-nearest; and
  "Features": packed low-bit storage.
* AutoRound "Rotation Transform", sections 2 and 2.1: MXFP4 uses blocks of 32
  elements.
* QuIP note, "The math, slowly": per-element round-off of nearest rounding
  lies in [-1/2, 1/2] of a step, with mean square 1/12 of a step squared.

The pages give no formula for the quantizer; the plainest reading is taken
and stated here:

* groups are contiguous runs of ``group_size`` elements along the last dim;
* symmetric: s = amax / (2^(b-1) - 1), q = clamp(rne(y / s), -2^(b-1), 2^(b-1) - 1);
* asymmetric: lo = min(min y, 0), hi = max(max y, 0), s = (hi - lo) / (2^b - 1),
  z = clamp(rne(-lo / s), 0, 2^b - 1), q = clamp(rne(y / s) + z, 0, 2^b - 1);
* s is rounded to its storage type (float32 or bfloat16, round to nearest
  even, directly from float64) and the stored value is the one used for the
  codes; a zero stored scale (all-zero group) is replaced by 1;
* MXFP4: e = clamp(floor(log2 amax) - 2, -127, 127) taken exactly from the
  binary exponent (amax = 0 gives -127), E8M0 byte = e + 127; every element
  is E2M1 of y / 2^e with round-to-nearest, ties to the even mantissa,
  saturating at +-6; the 4-bit code is sign << 3 | index with
  index 0..7 <-> {0, 0.5, 1, 1.5, 2, 3, 4, 6}; the sign bit is set iff y < 0
  (a negative value that rounds to zero keeps its sign, code 0x8);
* NVFP4 (named on the AutoRound page, sections 2 and 2.1, with rotation
  blocks of 16; its encoding is not on the pages, so this reading is the
  public two-level one): blocks of 16 consecutive elements; a float32 tensor
  scale g > 0 chosen by the caller (1 for a single-level scale); the block
  scale byte is E4M3 (OCP e4m3fn: bias 7, 3 mantissa bits, subnormals down
  to 2^-9, no infinities) of d = amax / (6 g), round to nearest even,
  saturating at 448; every element is E2M1 of y / (E4M3(d) g) with the
  MXFP4 rounding rules; a block whose scale byte is 0 stores code 0 for
  every element;
* rne is round half to even (numpy.rint);
* codes are packed two per byte, element 2j in the low nibble; symmetric
  codes are stored as two's complement nibbles; zero points are packed the
  same way over the row-major flattened group index (a trailing odd nibble
  is padded with 0).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# midpoints between consecutive E2M1 magnitudes
E2M1_BOUNDS = (E2M1_VALUES[1:] + E2M1_VALUES[:-1]) / 2.0


# ----------------------------------------------------------- storage rounding

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float64.  Done directly from float64 (no intermediate float32), by
    scaling the binary significand to 8 bits and rounding with numpy.rint.
    Values below the float32 normal range are not handled."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0) / 256.0     # 8 significant bits
    return np.ldexp(r, e)


def fp32_round(x) -> np.ndarray:
    """Round float64 values to float32 (numpy conversion is round to nearest
    even) and return them as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_scale(s, scale_dtype: str) -> np.ndarray:
    if scale_dtype == "f32":
        return fp32_round(s)
    if scale_dtype == "bf16":
        return bf16_round(s)
    raise ValueError("scale dtype must be 'f32' or 'bf16'")


# ------------------------------------------------------------------ RTN int

@dataclass
class QuantResult:
    """Quantizer output for a [rows, n] input, unpacked.

    codes   int64 [rows, n]        RTN: signed (sym) or unsigned (asym) codes;
                                   MXFP4: 4-bit codes 0..15
    scales  float64 [rows, n/g]    stored scale values (RTN), or int64 E8M0
                                   bytes (MXFP4)
    zeros   int64 [rows, n/g] | None
    raw     float64 [rows, n/g]    unrounded scale (RTN) or amax (MXFP4)
    pre     float64 [rows, n]      value that is rounded: y / s_stored (RTN,
                                   before + z), or y / 2^e (MXFP4)
    zero_pre float64 [rows, n/g] | None   -lo / s_stored (asymmetric RTN)
    """
    codes: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray | None
    raw: np.ndarray
    pre: np.ndarray
    zero_pre: np.ndarray | None = None


def _groups(y: np.ndarray, g: int) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    if g <= 0 or n % g:
        raise ValueError("group size must divide the last dimension")
    return y.reshape(-1, n // g, g)


def rtn_codes(pre: np.ndarray, zero, bits: int, sym: bool) -> np.ndarray:
    """Codes from pre-rounding values pre = y / s_stored: clamp(rne(pre) [+ z])."""
    if sym:
        lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
        return np.clip(np.rint(pre), lo, hi).astype(np.int64)
    return np.clip(np.rint(pre) + zero, 0, (1 << bits) - 1).astype(np.int64)


def rtn_quant(y, group_size: int, bits: int = 4, sym: bool = True,
              scale_dtype: str = "bf16") -> QuantResult:
    """Round-to-nearest group quantization of y [..., n] (see module text)."""
    yg = _groups(y, group_size)
    rows = yg.shape[0]
    n = yg.shape[1] * group_size
    if sym:
        qmax = (1 << (bits - 1)) - 1
        raw = np.abs(yg).max(axis=-1) / qmax
        s = round_scale(raw, scale_dtype)
        s = np.where(s == 0.0, 1.0, s)
        pre = yg / s[..., None]
        codes = rtn_codes(pre, None, bits, True)
        zeros = None
        zero_pre = None
    else:
        levels = (1 << bits) - 1
        lo = np.minimum(yg.min(axis=-1), 0.0)
        hi = np.maximum(yg.max(axis=-1), 0.0)
        raw = (hi - lo) / levels
        s = round_scale(raw, scale_dtype)
        s = np.where(s == 0.0, 1.0, s)
        zero_pre = -lo / s
        zeros = np.clip(np.rint(zero_pre), 0, levels).astype(np.int64)
        pre = yg / s[..., None]
        codes = rtn_codes(pre, zeros[..., None], bits, False)
    return QuantResult(codes.reshape(rows, n), s, zeros, raw, pre.reshape(rows, n), zero_pre)


def dequant_int(codes, scales, zeros, group_size: int) -> np.ndarray:
    """q * s (symmetric, zeros None) or (q - z) * s (asymmetric)."""
    c = np.asarray(codes, dtype=np.float64)
    rows, n = c.shape
    cg = c.reshape(rows, n // group_size, group_size)
    if zeros is not None:
        cg = cg - np.asarray(zeros, dtype=np.float64)[..., None]
    return (cg * np.asarray(scales, dtype=np.float64)[..., None]).reshape(rows, n)


# -------------------------------------------------------------------- MXFP4

def e2m1_round(v) -> np.ndarray:
    """E2M1 code (sign << 3 | index) of v: nearest magnitude in E2M1_VALUES,
    ties to the even index (even mantissa), saturating above 6; sign set iff
    v < 0."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    idx = np.zeros(a.shape, dtype=np.int64)
    for k, b in enumerate(E2M1_BOUNDS):
        up = a > b
        if k % 2 == 1:              # tie goes up to index k + 1, which is even
            up = up | (a == b)
        idx += up.astype(np.int64)
    return np.where(v < 0, idx | 8, idx)


def mxfp4_quant(y, group_size: int = 32) -> QuantResult:
    """MXFP4 quantization of y [..., n] with one E8M0 scale per group."""
    yg = _groups(y, group_size)
    rows = yg.shape[0]
    n = yg.shape[1] * group_size
    amax = np.abs(yg).max(axis=-1)
    _, ex = np.frexp(amax)              # amax = m 2^ex, 0.5 <= m < 1
    e = np.where(amax > 0, ex.astype(np.int64) - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    pre = np.ldexp(yg, -e[..., None])   # exact power-of-two scaling
    codes = e2m1_round(pre)
    return QuantResult(codes.reshape(rows, n), e + 127, None, amax, pre.reshape(rows, n))


def dequant_mxfp4(codes, e8m0, group_size: int = 32) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    rows, n = c.shape
    mag = E2M1_VALUES[c & 7]
    val = np.where(c & 8, -mag, mag).reshape(rows, n // group_size, group_size)
    e = np.asarray(e8m0, dtype=np.int64) - 127
    return np.ldexp(val, e[..., None]).reshape(rows, n)


# -------------------------------------------------------------------- NVFP4

E4M3_MAX = 448.0


def e4m3_decode(byte) -> np.ndarray:
    """Value of E4M3 (e4m3fn) bytes: sign, 4 exponent bits (bias 7), 3
    mantissa bits; exponent field 0 is subnormal (m / 8 * 2^-6); 0x7F / 0xFF
    are NaN."""
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    ef = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(ef == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, ef - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(v) -> np.ndarray:
    """E4M3 byte of non-negative values: nearest representable magnitude,
    ties to the even mantissa, saturating at 448 (so no NaN is produced)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("E4M3 scales are encoded from non-negative values")
    a = np.minimum(v, E4M3_MAX)
    # exponent of the binade, clamped to the subnormal binade below 2^-6
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f 2^ex, 0.5 <= f < 1
    e = np.maximum(ex.astype(np.int64) - 1, -6)        # floor(log2 a), >= -6
    q = np.rint(np.ldexp(a, 3 - e))                    # units of 2^(e - 3), ties to even
    # q in 8..16 for normals (16 carries into the next binade), 0..8 subnormal
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, q / 2, q)
    normal = q >= 8
    ef = np.where(normal, e + 7, 0)
    mant = np.where(normal, q - 8, q).astype(np.int64)
    return np.where(a > 0, (ef.astype(np.int64) << 3) | mant, 0).astype(np.int64)


def nvfp4_quant(y, group_size: int = 16, tensor_scale: float = 1.0) -> QuantResult:
    """NVFP4 quantization of y [..., n] (see module text): E4M3 block scale
    bytes of amax / (6 g), E2M1 codes of y / (E4M3 g)."""
    if not tensor_scale > 0 or not np.isfinite(tensor_scale):
        raise ValueError("tensor scale must be positive and finite")
    yg = _groups(y, group_size)
    rows = yg.shape[0]
    n = yg.shape[1] * group_size
    g = float(tensor_scale)
    amax = np.abs(yg).max(axis=-1)
    d = amax / (6.0 * g)
    byte = e4m3_encode(d)
    s = e4m3_decode(byte) * g
    safe = np.where(s > 0, s, 1.0)
    pre = np.where(s[..., None] > 0, yg / safe[..., None], 0.0)
    codes = np.where(s[..., None] > 0, e2m1_round(pre), 0)
    return QuantResult(codes.reshape(rows, n), byte, None, d, pre.reshape(rows, n))


def dequant_nvfp4(codes, e4m3, group_size: int = 16, tensor_scale: float = 1.0) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    rows, n = c.shape
    mag = E2M1_VALUES[c & 7]
    val = np.where(c & 8, -mag, mag).reshape(rows, n // group_size, group_size)
    s = e4m3_decode(e4m3) * float(tensor_scale)
    return (val * s[..., None]).reshape(rows, n)


# ------------------------------------------------------------------ packing

def pack_nibbles(codes) -> np.ndarray:
    """Pack integer codes two per byte over the flattened order: element 2j in
    the low nibble, 2j + 1 in the high nibble (values taken mod 16, so signed
    codes become two's complement nibbles).  An odd count is padded with 0."""
    c = (np.asarray(codes, dtype=np.int64).reshape(-1) & 0xF).astype(np.uint8)
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, dtype=np.uint8)])
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed, count: int, signed: bool = False) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    c = np.empty(p.size * 2, dtype=np.int64)
    c[0::2] = p & 0xF
    c[1::2] = p >> 4
    c = c[:count]
    if signed:
        c = np.where(c >= 8, c - 16, c)
    return c
