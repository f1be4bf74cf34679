"""Pins for the oracle's quantizers, storage rounding and packing (CPU only).

Independent checks: hand-worked golden cases, brute-force nearest-grid-point
search in exact rational arithmetic (fractions.Fraction) on tiny groups, the
round-off bounds from the QuIP note ("The math, slowly": per-element error
within half a step, mean square a twelfth of a step squared), torch's
float32 -> bfloat16 conversion as a library cross-check for the bfloat16
rounding, and the MXFP4 scale bracket amax / 2^e in [4, 8).  NVFP4: the E4M3
scale byte against PyTorch's float8_e4m3fn conversion (an independent
implementation of the public format), hand-worked blocks, and exact brute
force over every E4M3 and E2M1 value.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import quant as Q

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


# --------------------------------------------------------------- bf16 / fp32

def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-20, 20, 200000).astype(np.float32),
        np.array([1.0, -1.0, 0.0, 3.0e38, 1.1754944e-38], dtype=np.float32),
    ]).astype(np.float32)
    v = v[np.isfinite(v)]
    ours = Q.bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_round_ties_to_even():
    one = 1.0
    assert Q.bf16_round(one + 2.0 ** -8) == 1.0                       # tie, 1.0 is even
    assert Q.bf16_round(one + 3 * 2.0 ** -8) == one + 2.0 ** -6       # tie, goes up to even
    assert Q.bf16_round(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    assert Q.bf16_round(-(one + 2.0 ** -8)) == -1.0


def test_bf16_round_direct_from_float64_no_double_rounding():
    # 1 + 2^-8 - 2^-40 is below the bf16 midpoint; a detour through float32
    # would round it to 1 + 2^-8 (a tie) first and could then land on the
    # other side.  Direct rounding gives 1.0.
    assert Q.bf16_round(1.0 + 2.0 ** -8 - 2.0 ** -40) == 1.0
    assert Q.bf16_round(1.0 + 3 * 2.0 ** -8 - 2.0 ** -40) == 1.0 + 2.0 ** -7


def _f32_c(v: float) -> float:
    """float64 -> float32 by the C library's conversion (struct), an
    implementation independent of numpy's."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def test_fp32_round_ties_to_even_and_direction():
    one = 1.0
    u = 2.0 ** -23                                         # float32 ulp at 1
    assert Q.fp32_round(one + u / 2) == 1.0                # tie, 1.0 is even
    assert Q.fp32_round(one + 3 * u / 2) == one + 2 * u    # tie, goes up to even
    assert Q.fp32_round(one + u / 2 + 2.0 ** -50) == one + u   # above the midpoint
    assert Q.fp32_round(one + u / 2 - 2.0 ** -50) == 1.0       # below it
    assert Q.fp32_round(-(one + 3 * u / 2)) == -(one + 2 * u)  # sign symmetric
    assert Q.fp32_round(one + 0.75 * u) == one + u         # nearest, not toward zero
    assert Q.fp32_round(-(one + 0.75 * u)) == -(one + u)


def test_fp32_round_matches_torch_and_c_at_midpoints():
    """Exact float32 midpoints (ties) and points just beside them, compared
    with torch's float64 -> float32 conversion and the C library's."""
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    a = a[np.isfinite(a) & (np.abs(a) > 1e-30)].astype(np.float64)
    b = np.nextafter(a.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    mid = 0.5 * (a + b)                    # exact in float64
    vals = np.concatenate([mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), a])
    ours = Q.fp32_round(vals)
    ref = torch.from_numpy(vals).to(torch.float32).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    for i in range(0, vals.size, 97):
        assert ours[i] == _f32_c(float(vals[i]))


def test_fp32_scales_of_hand_cases_are_exact():
    """The stored float32 scales of the hand-worked cases equal the C library's
    float32 of 5/7 and 7/15 exactly (not merely within a tolerance)."""
    r = oracle.rtn_quant(np.array([[5.0, -1.0, -2.0, 0.0]]), 4, 4, True, "f32")
    assert r.scales[0, 0] == _f32_c(5.0 / 7.0)
    r = oracle.rtn_quant(np.array([[5.0, -1.0, -2.0, 0.0]]), 4, 4, False, "f32")
    assert r.scales[0, 0] == _f32_c(7.0 / 15.0)


# --------------------------------------------------------------------- RTN

def test_rtn_hand_cases():
    c = GOLDEN["rtn_sym_g4"]
    r = oracle.rtn_quant(np.array([c["y"]]), 4, 4, True, "f32")
    assert r.codes[0].tolist() == c["codes"]
    assert math.isclose(r.scales[0, 0], c["scale"], rel_tol=1e-7)
    assert oracle.pack_nibbles(r.codes).tolist() == c["packed_bytes"]
    c = GOLDEN["rtn_asym_g4"]
    r = oracle.rtn_quant(np.array([c["y"]]), 4, 4, False, "f32")
    assert r.codes[0].tolist() == c["codes"]
    assert r.zeros[0, 0] == c["zero"]
    assert math.isclose(r.scales[0, 0], c["scale"], rel_tol=1e-7)
    deq = oracle.dequant_int(r.codes, r.scales, r.zeros, 4)
    assert np.allclose(deq[0], c["dequant"], rtol=1e-6)


def _brute_rtn(vals, bits, sym, scale_dtype):
    """Nearest grid point by exhaustive search in exact arithmetic."""
    fr = [Fraction(float(v)) for v in vals]
    if sym:
        qmax = (1 << (bits - 1)) - 1
        amax = max(abs(f) for f in fr)
        s = float(oracle.round_scale(np.float64(amax / qmax), scale_dtype)) if amax else 0.0
        s = s if s != 0.0 else 1.0
        S = Fraction(s)
        grid = range(-(1 << (bits - 1)), qmax + 1)
        z = 0
    else:
        lo = min(min(fr), Fraction(0))
        hi = max(max(fr), Fraction(0))
        levels = (1 << bits) - 1
        s = float(oracle.round_scale(np.float64((hi - lo) / levels), scale_dtype)) if hi > lo else 0.0
        s = s if s != 0.0 else 1.0
        S = Fraction(s)
        # zero point: nearest integer to -lo / s, ties to even, clamped
        t = -lo / S
        z = min(max(_rne_fraction(t), 0), levels)
        grid = range(0, levels + 1)
    codes = []
    for f in fr:
        best = None
        for q in grid:
            d = abs(f - (q - z) * S)
            key = (d, (q - z) % 2)          # ties: even (q - z)
            if best is None or key < best[0]:
                best = (key, q)
        codes.append(best[1])
    return codes, s, z


def _rne_fraction(t: Fraction) -> int:
    f = math.floor(t)
    r = t - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("scale_dtype", ["f32", "bf16"])
def test_rtn_brute_force_tiny_groups(sym, scale_dtype):
    rng = np.random.default_rng(11 if sym else 12)
    for trial in range(400):
        g = int(rng.integers(1, 5))
        kind = trial % 4
        if kind == 0:
            vals = rng.standard_normal(g)
        elif kind == 1:
            vals = rng.uniform(0.1, 3.0, g)                     # one-signed group
        elif kind == 2:
            # values on half-integer multiples of a power-of-two scale: exact ties
            vals = (rng.integers(-15, 16, g) + 0.5) * 0.25
            vals[0] = 7 * 0.25 if sym else vals[0]
        else:
            vals = rng.standard_normal(g) * 10.0 ** rng.integers(-3, 3)
        r = oracle.rtn_quant(vals[None, :], g, 4, sym, scale_dtype)
        codes, s, z = _brute_rtn(vals, 4, sym, scale_dtype)
        assert r.codes[0].tolist() == codes, (vals, r.codes, codes)
        assert r.scales[0, 0] == s
        if not sym:
            assert r.zeros[0, 0] == z


def test_rtn_all_zero_group():
    r = oracle.rtn_quant(np.zeros((2, 8)), 4, 4, True, "bf16")
    assert np.all(r.scales == 1.0) and np.all(r.codes == 0)
    r = oracle.rtn_quant(np.zeros((2, 8)), 4, 4, False, "bf16")
    assert np.all(r.scales == 1.0) and np.all(r.codes == 0) and np.all(r.zeros == 0)


def test_rtn_symmetric_amax_maps_to_full_scale():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((64, 128))
    r = oracle.rtn_quant(y, 128, 4, True, "bf16")
    i = np.abs(y).argmax(axis=1)
    top = r.codes[np.arange(64), i]
    assert np.all(np.abs(top) == 7)
    assert r.codes.min() >= -7 and r.codes.max() <= 7


@pytest.mark.parametrize("sym", [True, False])
def test_rtn_error_bounds(sym):
    """|y - yhat| <= s/2 for unclamped elements; mean square error close to
    s^2/12 over many elements (QuIP note, 'The math, slowly')."""
    rng = np.random.default_rng(4)
    y = rng.standard_normal((2000, 128))
    r = oracle.rtn_quant(y, 128, 4, sym, "f32")
    deq = oracle.dequant_int(r.codes, r.scales, r.zeros, 128)
    s = np.repeat(r.scales, 128, axis=1)
    err = (y - deq) / s
    assert np.all(np.abs(err) <= 0.5 + 1e-9)
    # interior elements: exclude codes at the ends of the grid
    q = r.codes
    interior = (np.abs(q) < 7) if sym else ((q > 0) & (q < 15))
    e = err[interior]
    assert e.size > 100000
    assert abs(np.mean(e * e) - 1.0 / 12.0) < 0.03 / 12.0


# ------------------------------------------------------------------- MXFP4

def test_mxfp4_hand_cases():
    c = GOLDEN["mxfp4_amax5"]
    y = np.array(c["y"] + [0.0] * (32 - len(c["y"])))
    r = oracle.mxfp4_quant(y[None, :], 32)
    assert r.scales[0, 0] == c["e8m0"]
    assert r.codes[0, :len(c["codes"])].tolist() == c["codes"]
    deq = oracle.dequant_mxfp4(r.codes, r.scales, 32)[0, :len(c["values"])]
    assert deq.tolist() == c["values"]
    assert np.signbit(deq[4])
    s = GOLDEN["mxfp4_scale"]
    for amax, e in zip(s["amax"], s["e"]):
        y = np.zeros(32)
        y[5] = -amax
        assert oracle.mxfp4_quant(y[None, :], 32).scales[0, 0] == e + 127


def _brute_e2m1(v: float) -> int:
    """Nearest of the 15 distinct E2M1 values, exact arithmetic, ties to the
    even mantissa (even index); sign bit kept for negative v."""
    f = Fraction(float(v))
    a = abs(f)
    best = None
    for idx, val in enumerate(oracle.E2M1_VALUES):
        d = abs(a - Fraction(float(val)))
        key = (d, idx % 2)
        if best is None or key < best[0]:
            best = (key, idx)
    return best[1] | (8 if f < 0 else 0)


def test_e2m1_brute_force():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.uniform(-8, 8, 5000),
        np.arange(-64, 65) / 8.0,            # every multiple of 1/8 in [-8, 8]: all ties
        [6.0, -6.0, 100.0, -1e9, 0.0, -0.0, 1e-30, -1e-30],
    ])
    got = oracle.e2m1_round(vals)
    exp = np.array([_brute_e2m1(v) for v in vals])
    assert np.array_equal(got, exp)


def test_mxfp4_brute_force_groups():
    rng = np.random.default_rng(6)
    for trial in range(60):
        y = rng.standard_normal(32) * 10.0 ** rng.integers(-6, 6)
        r = oracle.mxfp4_quant(y[None, :], 32)
        e = int(r.scales[0, 0]) - 127
        amax = np.abs(y).max()
        assert 4.0 <= amax / 2.0 ** e < 8.0
        # brute force over the 15 distinct values times 2^e
        for k in range(32):
            v = Fraction(float(y[k])) / Fraction(2) ** e
            assert r.codes[0, k] == _brute_e2m1(float(v))


def test_mxfp4_zero_group():
    r = oracle.mxfp4_quant(np.zeros((1, 64)), 32)
    assert r.scales.tolist() == [[0, 0]] and np.all(r.codes == 0)


# -------------------------------------------------------------------- NVFP4

def test_e4m3_closed_forms():
    c = GOLDEN["e4m3_values"]
    got = oracle.e4m3_decode(np.array(c["bytes"]))
    assert got.tolist() == c["values"]
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert oracle.e4m3_decode(np.array([0x80 | 56]))[0] == -1.0
    assert oracle.e4m3_encode(np.array(c["values"])).tolist() == c["bytes"]


def _e4m3_grid():
    """Every finite non-negative E4M3 value by byte, from torch's own decoder."""
    b = torch.arange(0, 127, dtype=torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_torch():
    assert np.array_equal(oracle.e4m3_decode(np.arange(127)), _e4m3_grid())


def test_e4m3_encode_matches_torch():
    """PyTorch's float32 -> float8_e4m3fn conversion is an independent
    implementation of the same rounding (nearest, ties to even); it is
    compared below 464, above which it gives NaN where the oracle saturates."""
    grid = _e4m3_grid()
    mids = (grid[1:] + grid[:-1]) / 2                # every tie, exact in float32
    rng = np.random.default_rng(11)
    rand = np.exp2(rng.uniform(-13, np.log2(463.9), 20000))
    v = np.concatenate([grid, mids, rand, [464.0]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), ref)


def test_e4m3_saturates_and_rejects_negative():
    assert oracle.e4m3_encode(np.array([448.0, 464.0, 465.0, 1e30, np.inf])).tolist() == [126] * 5
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([-1.0]))


def _brute_e4m3(d: Fraction) -> int:
    """Nearest E4M3 byte to d >= 0 in exact arithmetic, ties to the even
    mantissa, saturating at 448."""
    grid = _e4m3_grid()
    best = None
    for byte, val in enumerate(grid):
        key = (abs(d - Fraction(float(val))), byte & 1)
        if best is None or key < best[0]:
            best = (key, byte)
    return best[1]


def test_nvfp4_hand_cases():
    for c in GOLDEN["nvfp4_cases"]["cases"]:
        y = np.array(c["y"] + [0.0] * (16 - len(c["y"])))
        r = oracle.nvfp4_quant(y[None, :], 16, c["g"])
        assert r.scales[0, 0] == c["byte"], c["note"]
        assert r.codes[0, :len(c["codes"])].tolist() == c["codes"], c["note"]
        if c["byte"]:
            assert np.all(r.codes[0, len(c["codes"]):] == 0)
        deq = oracle.dequant_nvfp4(r.codes, r.scales, 16, c["g"])[0, :len(c["values"])]
        assert deq.tolist() == c["values"], c["note"]


def test_nvfp4_brute_force_blocks():
    rng = np.random.default_rng(12)
    for trial in range(80):
        y = rng.standard_normal(16) * 10.0 ** rng.integers(-4, 4)
        g = float(np.float32(2.0 ** rng.uniform(-6, 3))) if trial % 2 else 1.0
        r = oracle.nvfp4_quant(y[None, :], 16, g)
        d = Fraction(float(np.abs(y).max())) / (6 * Fraction(g))
        byte = _brute_e4m3(d)
        assert r.scales[0, 0] == byte
        s = Fraction(float(_e4m3_grid()[byte])) * Fraction(g)
        for k in range(16):
            want = _brute_e2m1(float(Fraction(float(y[k])) / s)) if s else 0
            assert r.codes[0, k] == want


def test_nvfp4_error_bound():
    """Each element dequantizes within half of the local E2M1 spacing times
    the block scale, unless y / s is beyond 6 (saturated)."""
    rng = np.random.default_rng(13)
    y = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-8, 8, (64, 1)))
    r = oracle.nvfp4_quant(y, 16, 0.5)
    deq = oracle.dequant_nvfp4(r.codes, r.scales, 16, 0.5)
    s = np.repeat(oracle.e4m3_decode(r.scales) * 0.5, 16, axis=1)
    a = np.abs(y) / s
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    ok = a <= 6
    assert np.all(np.abs(deq - y)[ok] <= (half * s)[ok] * (1 + 1e-12))
    # the block maximum lands on a code near 6: its scale is amax / 6 rounded
    # to 4 significant bits, within 1/16 relative
    amax_codes = np.abs(y).reshape(64, 16, 16).argmax(-1)
    top = np.take_along_axis(r.codes.reshape(64, 16, 16), amax_codes[..., None], -1)[..., 0] & 7
    assert np.all(top >= 6)


def test_nvfp4_zero_and_invalid():
    r = oracle.nvfp4_quant(np.zeros((1, 32)), 16)
    assert r.scales.tolist() == [[0, 0]] and np.all(r.codes == 0)
    with pytest.raises(ValueError):
        oracle.nvfp4_quant(np.zeros((1, 16)), 16, 0.0)


# ----------------------------------------------------------------- packing

def test_pack_unpack():
    assert oracle.pack_nibbles([1, 2, 3, 4]).tolist() == [0x21, 0x43]
    assert oracle.pack_nibbles([-1, 7, -8]).tolist() == [0x7F, 0x08]
    rng = np.random.default_rng(9)
    c = rng.integers(-8, 8, 1001)
    p = oracle.pack_nibbles(c)
    assert p.size == 501
    assert np.array_equal(oracle.unpack_nibbles(p, 1001, signed=True), c)
