"""Seeded synthetic tensors with the shapes and value structure of the pages' workloads.

The rotation pages evaluate on real models (Qwen3, Qwen2.5, Llama-3.1, OPT)
and datasets that are not available here; these generators stand in for the
activations and weights those runs would feed the rotation.  Shapes follow the
8B-class layer geometry the pages name (hidden 4096, intermediate 14336,
32 heads of 128); the value structure follows the premise of the AutoRound
"Rotation Transform" page (introduction: rotation spreads outliers) and the
QuIP note ("Incoherence" section: a single large outlier dominates the
incoherence of a matrix).

Every generator draws from ``numpy.random.default_rng(seed)`` in a fixed order,
in float32, and casts to bfloat16 with round-to-nearest-even through torch on
the CPU.  The same bits feed the GPU path and the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def _to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 array -> bfloat16 CPU tensor (round to nearest even)."""
    assert a.dtype == np.float32
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)


def gaussian(shape, seed: int, dtype=torch.float32, std: float = 1.0) -> torch.Tensor:
    """iid N(0, std^2) tensor drawn in float32, cast to ``dtype`` (CPU)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == torch.bfloat16:
        return _to_bf16(a)
    return torch.from_numpy(a).to(dtype)


def rademacher(n: int, seed: int) -> torch.Tensor:
    """n independent +-1 signs (int8), as drawn for a random Hadamard or the
    Rademacher step of RPBH; the draw is an input of both implementations."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.choice(np.array([-1, 1], dtype=np.int8), n))


def permutation(n: int, seed: int) -> torch.Tensor:
    """A uniformly random permutation of 0..n-1 (int32)."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.permutation(n).astype(np.int32))


def tiny_activations(seed: int = 1, rows: int = 256, n: int = 128) -> torch.Tensor:
    """Tiny case: rows x n float32, N(0, 1)."""
    return gaussian((rows, n), seed, torch.float32)


def r1_activations(seed: int = 2, tokens: int = 4096, hidden: int = 4096,
                   n_outliers: int = 8, outlier_scale: float = 50.0) -> torch.Tensor:
    """Residual-stream activations: Student-t (nu = 3, unit scale) entries with
    ``n_outliers`` distinct channels (chosen uniformly without replacement)
    multiplied by ``outlier_scale`` before the bfloat16 cast."""
    rng = np.random.default_rng(seed)
    a = rng.standard_t(3.0, size=(tokens, hidden)).astype(np.float32)
    cols = rng.choice(hidden, size=min(n_outliers, hidden), replace=False)
    a[:, cols] *= np.float32(outlier_scale)
    return _to_bf16(a)


def r4_activations(seed: int = 3, tokens: int = 8192, inter: int = 14336) -> torch.Tensor:
    """down_proj inputs of a SwiGLU MLP: a * SiLU(b) with a, b iid N(0, 1) in float32."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=(tokens, inter), dtype=np.float32)
    b = rng.standard_normal(size=(tokens, inter), dtype=np.float32)
    # SiLU(b) = b * sigmoid(b), evaluated in float32
    silu = b / (np.float32(1.0) + np.exp(-b))
    del b
    a *= silu
    del silu
    return _to_bf16(a)


def _rope_inplace(x: np.ndarray, base: float = 10000.0) -> None:
    """Rotary position embedding in the rotate-half pairing (i, i + D/2) on a
    float32 array [B, S, H, D]; position = sequence index."""
    d = x.shape[-1]
    half = d // 2
    inv_freq = base ** (-np.arange(0, half, dtype=np.float64) * 2.0 / d)
    pos = np.arange(x.shape[1], dtype=np.float64)
    ang = np.outer(pos, inv_freq)                       # [S, D/2]
    cos = np.cos(ang).astype(np.float32)[None, :, None, :]
    sin = np.sin(ang).astype(np.float32)[None, :, None, :]
    x1 = x[..., :half].copy()
    x2 = x[..., half:]
    x[..., :half] = x1 * cos - x2 * sin
    x[..., half:] = x2 * cos + x1 * sin


def r3_query_key(seed: int = 4, batch: int = 16, seq: int = 2048, heads: int = 32,
                 head_dim: int = 128):
    """Post-RoPE queries and keys [B, S, H, D], N(0, 1) before RoPE (base 10000),
    cast to bfloat16.  Q is drawn before K."""
    rng = np.random.default_rng(seed)
    shape = (batch, seq, heads, head_dim)
    q = rng.standard_normal(size=shape, dtype=np.float32)
    k = rng.standard_normal(size=shape, dtype=np.float32)
    _rope_inplace(q)
    _rope_inplace(k)
    return _to_bf16(q), _to_bf16(k)


def weight_with_outliers(seed: int = 5, out_features: int = 14336, in_features: int = 4096,
                         std: float = 0.02, frac: float = 0.001,
                         outlier_scale: float = 20.0) -> torch.Tensor:
    """Linear weight [out, in]: N(0, std^2) with round(frac * numel) distinct
    entries (uniform without replacement) multiplied by ``outlier_scale``."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(size=(out_features, in_features), dtype=np.float32)
    w *= np.float32(std)
    cnt = int(round(frac * w.size))
    if cnt:
        pos = rng.choice(w.size, size=cnt, replace=False)
        w.reshape(-1)[pos] *= np.float32(outlier_scale)
    return _to_bf16(w)


@dataclass(frozen=True)
class Workload:
    """One named workload: generator arguments plus the rotation/quantizer
    settings the path runs on it.  ``qspecs`` entries are plain dicts
    (format, bits, group_size, sym, scale_dtype)."""
    name: str
    kind: str                 # "act" | "rotate_act" (Q/K) | "weight"
    seed: int
    n: int                    # rotated (last) dimension
    block: int                # Hadamard block; <= 0 means full width
    dtype: str                # "f32" | "bf16"
    qspecs: tuple = field(default_factory=tuple)
    write_rotated: bool = False
    gen_kwargs: dict = field(default_factory=dict)
    description: str = ""


def _q(fmt, bits, g, sym, scale_dtype):
    return dict(format=fmt, bits=bits, group_size=g, sym=sym, scale_dtype=scale_dtype)


WORKLOADS = {
    "tiny": Workload(
        "tiny", "act", 1, 128, 0, "f32", (_q("int", 4, 32, 1, "f32"),), True,
        dict(rows=256, n=128),
        "256x128 fp32 N(0,1); Sylvester n=128; int4 sym g32 fp32 scales; rotated fp32 written"),
    "r1": Workload(
        "r1", "act", 2, 4096, 0, "bf16", (_q("int", 4, 128, 1, "bf16"),), False,
        dict(tokens=4096, hidden=4096),
        "R1 4096 tokens x 4096 bf16 Student-t(3), 8 outlier channels x50; full FWHT 4096; "
        "int4 sym g128 bf16 scales"),
    "r4": Workload(
        "r4", "act", 3, 14336, 2048, "bf16", (_q("int", 4, 128, 0, "bf16"),), False,
        dict(tokens=8192, inter=14336),
        "R4 8192 tokens x 14336 bf16 a*SiLU(b); block-diagonal 7 x 2048; int4 asym g128 "
        "bf16 scales + uint4 zeros"),
    "r4_kron": Workload(
        "r4_kron", "act", 3, 14336, 0, "bf16", (_q("int", 4, 128, 0, "bf16"),), False,
        dict(tokens=8192, inter=14336),
        "R4 at full width 14336 = 28 x 512 (Kronecker H28 (x) H512) on the R4 input; "
        "int4 asym g128"),
    "r3": Workload(
        "r3", "rotate_act", 4, 128, 0, "bf16", (_q("int", 4, 128, 0, "bf16"),), False,
        dict(batch=16, seq=2048, heads=32, head_dim=128),
        "R3 Q,K 16x2048x32x128 bf16 post-RoPE; FWHT 128 per head; Q -> rotated bf16, "
        "K -> int4 asym g128"),
    "weight": Workload(
        "weight", "weight", 5, 4096, 0, "bf16",
        (_q("mxfp4", 4, 32, 1, "e8m0"), _q("int", 4, 128, 1, "bf16")), True,
        dict(out_features=14336, in_features=4096),
        "W 14336x4096 bf16 N(0,0.02^2) with 0.1% entries x20; W.H4096 bf16 + MXFP4 + int4 sym g128"),
}


def make_inputs(w: Workload, **override):
    """Generate the input tensor(s) of a workload (CPU).  ``override`` replaces
    generator size arguments (used for reduced-size parity cases)."""
    kw = dict(w.gen_kwargs)
    kw.update(override)
    if w.name == "tiny":
        return tiny_activations(w.seed, **kw)
    if w.name == "r1":
        return r1_activations(w.seed, **kw)
    if w.name in ("r4", "r4_kron"):
        return r4_activations(w.seed, **kw)
    if w.name == "r3":
        return r3_query_key(w.seed, **kw)
    if w.name == "weight":
        return weight_with_outliers(w.seed, **kw)
    raise KeyError(w.name)
