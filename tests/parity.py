"""Comparison of GPU outputs with the oracle, under the stated tolerances.

Rotated values: per element |gpu - oracle| <= tol * ||oracle row||_2, with
tol = 2e-3 for bfloat16 outputs and 1e-5 for float32 (the oracle value is the
unrounded float64 rotation).

Integer codes (INT, MXFP4 and NVFP4) must be bit-exact except where the oracle's
pre-rounding value lies within 1e-3 of a step from a rounding boundary, and
then the codes may differ by one step only (adjacent code).  Scales: float32
within 1e-6 relative; bfloat16 and E8M0 exact, except a group whose unrounded
oracle scale (bfloat16) or amax (E8M0) lies within 1e-6 relative of a
rounding midpoint (bfloat16) or a power of two (E8M0), where the GPU may
hold the neighbouring value; such a group's codes are re-derived by the
oracle from the GPU's stored scale before the code rule is applied.  Zero
points follow the code rule with pre-rounding value -lo / s.  A code 0x0 /
0x8 (MXFP4 +0 / -0) difference is accepted where |y / 2^e| < 5e-4 (the sign of
a value at the float32 rounding-noise level).  NVFP4 E4M3 block bytes follow
the bfloat16 scale rule (the rounding point is the midpoint between adjacent
E4M3 values), and its codes the MXFP4 code rule with y / s in place of
y / 2^e.

Two bounds derived from the arithmetic extend the stated tolerances where
those cannot hold for any correct implementation:

* bfloat16 outputs: a value within one bfloat16 ulp of the exact rotation
  (one of its two bfloat16 neighbours) is accepted even where that exceeds
  2e-3 of the row norm; this happens for rows of 2..16 elements, where one
  element carries most of the norm and round-to-nearest alone errs by up to
  2^-8 of it.
* float32 rotation error: the transform's rounding error is relative to the
  magnitude of the row, not to each group, so groups much smaller than the
  row see larger relative errors.  The comparator widens the scale (1e-6
  relative), boundary (1e-3 step) and flip windows to cover an absolute
  error of EPS_ROW = 4 (log2 n + K + 3) 2^-24 rms(row) in every rotated
  value (K: Kronecker base order, else 0).  For groups of typical magnitude
  (amax about 3 rms) this is about 1e-5 of a step and 2e-6 relative on a
  scale; it dominates only for groups far below the row's magnitude
  (groups of 2..8 elements).  Report.max_scale_rel records the largest
  float32 scale deviation actually seen.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import oracle

ROT_TOL = {"bf16": 2e-3, "f32": 1e-5}
CODE_TOL = 1e-3        # steps from a rounding boundary
SCALE_REL = 1e-6


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


@dataclass
class Report:
    n_elems: int = 0
    n_groups: int = 0
    code_mismatch: int = 0
    scale_flips: int = 0
    zero_flips: int = 0
    max_rot_err: float = 0.0
    max_scale_rel: float = 0.0
    # acceptances outside the stated tolerances, counted by the rule that
    # allowed them: the float32 rotation-error widening (EPS_ROW), the
    # one-ulp rule for bfloat16 outputs, and the +0 / -0 rule of E2M1 codes
    widened: int = 0
    ulp_accepted: int = 0
    zero_sign: int = 0
    notes: list = field(default_factory=list)

    def __str__(self):
        return ("elems=%d groups=%d tolerated code mismatches=%d scale flips=%d zero flips=%d "
                "max rot err/rownorm=%.3g max f32 scale rel dev=%.3g widened-window acceptances=%d "
                "bf16 one-ulp acceptances=%d signed-zero acceptances=%d"
                % (self.n_elems, self.n_groups, self.code_mismatch, self.scale_flips,
                   self.zero_flips, self.max_rot_err, self.max_scale_rel, self.widened,
                   self.ulp_accepted, self.zero_sign))


def eps_row(y: np.ndarray, kron_k: int = 0) -> np.ndarray:
    """Per-row absolute error allowance of float32 rotated values [rows, 1]."""
    n = y.shape[-1]
    rms = np.sqrt(np.mean(y.reshape(-1, n) ** 2, axis=1, keepdims=True))
    return 4.0 * (np.log2(n) + kron_k + 3) * 2.0 ** -24 * rms


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check_rotated(gpu: np.ndarray, ref: np.ndarray, out_dtype: str, rep: Report | None = None):
    n = ref.shape[-1]
    g = gpu.reshape(-1, n)
    r = ref.reshape(-1, n)
    norm = np.linalg.norm(r, axis=1, keepdims=True)
    err = np.abs(g - r)
    lim = ROT_TOL[out_dtype] * norm
    over = err > lim
    bad = over
    if out_dtype == "bf16":
        bad = over & ~(err < bf16_ulp(r))
    rel = float(np.max(err / np.where(norm > 0, norm, 1.0))) if err.size else 0.0
    if rep is not None:
        rep.max_rot_err = max(rep.max_rot_err, rel)
        rep.ulp_accepted += int((over & ~bad).sum())
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("rotated output out of tolerance at %s: gpu %r oracle %r (row norm %r)"
                             % (tuple(i), g[tuple(i)], r[tuple(i)], norm[i[0], 0]))
    return rel


def _near_half(pre: np.ndarray) -> np.ndarray:
    """Distance (in steps) of pre from the nearest rounding boundary k + 1/2."""
    return np.abs(pre - (np.floor(pre) + 0.5))


def unpack_gpu_codes(codes: torch.Tensor, count: int, signed: bool) -> np.ndarray:
    return oracle.unpack_nibbles(codes.detach().cpu().numpy().reshape(-1), count, signed)


def check_int(gpu: dict, y: np.ndarray, g: int, sym: bool, scale_dtype: str, rep: Report,
              zeros_gpu: np.ndarray | None = None, kron_k: int = 0):
    """gpu: dict(codes uint8, scales tensor, zeros uint8 or None) for the rows
    of y (float64 [rows, n]).  ``zeros_gpu`` overrides the unpacked zero points
    (used for sampled rows)."""
    rows, n = y.shape
    ref = oracle.rtn_quant(y, g, 4, sym, scale_dtype)
    codes = unpack_gpu_codes(gpu["codes"], rows * n, sym).reshape(rows, n)
    s_gpu = to_np64(gpu["scales"]).reshape(rows, n // g)
    ng = rows * n // g
    rep.n_elems += rows * n
    rep.n_groups += ng
    s_ref = ref.scales
    levels = 7.0 if sym else 15.0
    ey = eps_row(y, kron_k)                           # [rows, 1]
    s_tol = np.maximum(SCALE_REL * np.abs(ref.raw), 2.0 * ey / levels)
    # ---- scales
    flip = s_gpu != s_ref
    if scale_dtype == "f32":
        dev = np.abs(s_gpu - s_ref)
        rep.max_scale_rel = max(rep.max_scale_rel, float(np.max(dev / np.abs(s_ref))) if dev.size else 0.0)
        bad = dev > s_tol
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("f32 scale mismatch at group %s: gpu %r oracle %r" % (tuple(i), s_gpu[tuple(i)], s_ref[tuple(i)]))
        rep.widened += int((dev > SCALE_REL * np.abs(ref.raw)).sum())
    else:
        ok_flip = (np.abs(ref.raw - 0.5 * (s_gpu + s_ref)) <= s_tol) & (
            np.abs(s_gpu - s_ref) <= np.abs(s_ref) * 2.0 ** -7 * 1.0001)
        bad = flip & ~ok_flip
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("bf16 scale mismatch at group %s: gpu %r oracle %r (unrounded %r)"
                                 % (tuple(i), s_gpu[tuple(i)], s_ref[tuple(i)], ref.raw[tuple(i)]))
        rep.widened += int((flip & (np.abs(ref.raw - 0.5 * (s_gpu + s_ref)) > SCALE_REL * np.abs(ref.raw))).sum())
    rep.scale_flips += int(flip.sum())
    # oracle's codes and zeros, re-derived from the GPU scale where it flipped
    s_use = np.where(flip, s_gpu, s_ref)
    yg = y.reshape(rows, n // g, g)
    pre = yg / s_use[..., None]
    if sym:
        exp = oracle.rtn_codes(pre, None, 4, True)
    else:
        lo = np.minimum(yg.min(axis=-1), 0.0)
        zpre = -lo / s_use
        z_ref = np.clip(np.rint(zpre), 0, 15).astype(np.int64)
        z_gpu = zeros_gpu.reshape(rows, n // g) if zeros_gpu is not None else \
            oracle.unpack_nibbles(gpu["zeros"].cpu().numpy(), ng).reshape(rows, n // g)
        zd = z_gpu != z_ref
        ztol = np.maximum(CODE_TOL, ey / s_use)
        zbad = zd & ~((_near_half(zpre) <= ztol) & (np.abs(z_gpu - z_ref) == 1))
        if zbad.any():
            i = np.argwhere(zbad)[0]
            raise AssertionError("zero point mismatch at group %s: gpu %d oracle %d (pre %r)"
                                 % (tuple(i), z_gpu[tuple(i)], z_ref[tuple(i)], zpre[tuple(i)]))
        rep.zero_flips += int(zd.sum())
        rep.widened += int((zd & (_near_half(zpre) > CODE_TOL)).sum())
        exp = oracle.rtn_codes(pre, z_gpu[..., None], 4, False)
    ctol = np.repeat(np.maximum(CODE_TOL, ey / s_use), g, axis=1)
    exp = exp.reshape(rows, n)
    pre = pre.reshape(rows, n)
    d = codes != exp
    if d.any():
        ok = (_near_half(pre) <= ctol) & (np.abs(codes - exp) == 1)
        bad = d & ~ok
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("code mismatch at %s: gpu %d oracle %d (pre %r)"
                                 % (tuple(i), codes[tuple(i)], exp[tuple(i)], pre[tuple(i)]))
        rep.code_mismatch += int(d.sum())
        rep.widened += int((d & (_near_half(pre) > CODE_TOL)).sum())


_BOUNDS = oracle.quant.E2M1_BOUNDS
_SPACING = np.diff(oracle.E2M1_VALUES)


def check_mxfp4(gpu: dict, y: np.ndarray, rep: Report, kron_k: int = 0):
    rows, n = y.shape
    g = 32
    ref = oracle.mxfp4_quant(y, g)
    codes = unpack_gpu_codes(gpu["codes"], rows * n, False).reshape(rows, n)
    e_gpu = gpu["scales"].cpu().numpy().astype(np.int64).reshape(rows, n // g)
    e_ref = ref.scales
    rep.n_elems += rows * n
    rep.n_groups += rows * n // g
    ey = eps_row(y, kron_k)
    flip = e_gpu != e_ref
    if flip.any():
        amax = ref.raw
        near = np.abs(amax - 2.0 ** np.round(np.log2(np.where(amax > 0, amax, 1.0)))) <= \
            np.maximum(SCALE_REL * amax, ey)
        bad = flip & ~(near & (np.abs(e_gpu - e_ref) == 1))
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("E8M0 mismatch at group %s: gpu %d oracle %d (amax %r)"
                                 % (tuple(i), e_gpu[tuple(i)], e_ref[tuple(i)], amax[tuple(i)]))
        rep.scale_flips += int(flip.sum())
        strict = np.abs(amax - 2.0 ** np.round(np.log2(np.where(amax > 0, amax, 1.0)))) <= SCALE_REL * amax
        rep.widened += int((flip & ~strict).sum())
    e_use = np.where(flip, e_gpu, e_ref) - 127
    pre = np.ldexp(y.reshape(rows, n // g, g), -e_use[..., None]).reshape(rows, n)
    exp = oracle.e2m1_round(pre)
    d = codes != exp
    if d.any():
        a = np.abs(pre)
        k = np.clip(np.searchsorted(_BOUNDS, a), 0, len(_BOUNDS) - 1)
        # distance to the nearest boundary, in units of the spacing there
        dist = np.minimum(
            np.abs(a - _BOUNDS[np.clip(k - 1, 0, 6)]) / _SPACING[np.clip(k - 1, 0, 6)],
            np.abs(a - _BOUNDS[k]) / _SPACING[k])
        same_sign = (codes & 8) == (exp & 8)
        adjacent = same_sign & (np.abs((codes & 7) - (exp & 7)) == 1)
        etol = np.repeat(np.maximum(CODE_TOL, ey / 2.0 ** e_use / 0.5), g, axis=1)
        zero_sign = ((codes & 7) == 0) & ((exp & 7) == 0) & (a < 0.5 * etol)
        ok = ((dist <= etol) & adjacent) | zero_sign
        bad = d & ~ok
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("MXFP4 code mismatch at %s: gpu %d oracle %d (pre %r)"
                                 % (tuple(i), codes[tuple(i)], exp[tuple(i)], pre[tuple(i)]))
        rep.code_mismatch += int(d.sum())
        by_sign = d & zero_sign & ~((dist <= etol) & adjacent)
        rep.zero_sign += int(by_sign.sum())
        rep.widened += int((d & ~by_sign & (dist > CODE_TOL)).sum())


def check_nvfp4(gpu: dict, y: np.ndarray, rep: Report, tensor_scale: float = 1.0, kron_k: int = 0):
    """NVFP4 under the MXFP4 rules: E4M3 block bytes exact except an adjacent
    byte where amax / (6 g) lies within 1e-6 relative of the midpoint between
    the two values (that block's codes are then re-derived from the GPU's
    byte); codes exact except adjacent codes near a rounding boundary, and
    +0 / -0 at the rounding-noise level."""
    rows, n = y.shape
    g = 16
    ts = float(np.float32(tensor_scale)) if tensor_scale else 1.0
    ref = oracle.nvfp4_quant(y, g, ts)
    codes = unpack_gpu_codes(gpu["codes"], rows * n, False).reshape(rows, n)
    b_gpu = gpu["scales"].cpu().numpy().astype(np.int64).reshape(rows, n // g)
    b_ref = ref.scales
    rep.n_elems += rows * n
    rep.n_groups += rows * n // g
    ey = eps_row(y, kron_k)
    flip = b_gpu != b_ref
    if flip.any():
        mid = 0.5 * (oracle.e4m3_decode(np.clip(b_gpu, 0, 126)) + oracle.e4m3_decode(b_ref))
        near = np.abs(ref.raw - mid) <= np.maximum(SCALE_REL * ref.raw, ey / (6.0 * ts))
        bad = flip & ~(near & (np.abs(b_gpu - b_ref) == 1))
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("E4M3 mismatch at group %s: gpu %d oracle %d (amax / 6g %r)"
                                 % (tuple(i), b_gpu[tuple(i)], b_ref[tuple(i)], ref.raw[tuple(i)]))
        rep.scale_flips += int(flip.sum())
        rep.widened += int((flip & (np.abs(ref.raw - mid) > SCALE_REL * ref.raw)).sum())
    s_use = oracle.e4m3_decode(np.where(flip, b_gpu, b_ref)) * ts
    yg = y.reshape(rows, n // g, g)
    safe = np.where(s_use > 0, s_use, 1.0)
    pre = np.where(s_use[..., None] > 0, yg / safe[..., None], 0.0).reshape(rows, n)
    exp = np.where(np.repeat(s_use, g, axis=1) > 0, oracle.e2m1_round(pre), 0)
    d = codes != exp
    if d.any():
        a = np.abs(pre)
        k = np.clip(np.searchsorted(_BOUNDS, a), 0, len(_BOUNDS) - 1)
        dist = np.minimum(
            np.abs(a - _BOUNDS[np.clip(k - 1, 0, 6)]) / _SPACING[np.clip(k - 1, 0, 6)],
            np.abs(a - _BOUNDS[k]) / _SPACING[k])
        same_sign = (codes & 8) == (exp & 8)
        adjacent = same_sign & (np.abs((codes & 7) - (exp & 7)) == 1)
        etol = np.repeat(np.maximum(CODE_TOL, ey / safe / 0.5), g, axis=1)
        zero_sign = ((codes & 7) == 0) & ((exp & 7) == 0) & (a < 0.5 * etol)
        ok = ((dist <= etol) & adjacent) | zero_sign
        bad = d & ~ok
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("NVFP4 code mismatch at %s: gpu %d oracle %d (pre %r)"
                                 % (tuple(i), codes[tuple(i)], exp[tuple(i)], pre[tuple(i)]))
        rep.code_mismatch += int(d.sum())
        by_sign = d & zero_sign & ~((dist <= etol) & adjacent)
        rep.zero_sign += int(by_sign.sum())
        rep.widened += int((d & ~by_sign & (dist > CODE_TOL)).sum())
