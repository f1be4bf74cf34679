"""Hadamard matrices and the rotation y = x . R, in float64 (oracle; test infrastructure only).

Sources (cited by page title and section):

* AutoRound "Rotation Transform", section 1.5 (Deterministic vs random
  Hadamard): the deterministic matrix is the Sylvester recursion
  H -> [[H, H], [H, -H]], normalised by sqrt(size), size a power of two; for
  other sizes n is factored as K * 2^m and a base Hadamard of order K is
  combined with a Sylvester block.
* Same page, section 1.2 (rotation_size must be a positive power of two and
  replaces the full width) and section 2.1 (block_size: grouped, i.e.
  block-diagonal, Hadamard; None or -1 means full width).
* Same page, introduction: an orthogonal R with R R^T = I leaves
  x R R^T W^T = x W^T unchanged.

Readings taken where the pages are silent:

* natural (Sylvester) order, H[i][j] = (-1)^popcount(i & j);
* row-vector convention y = x . R, and the weight pairing W' = W . R;
* blocks are contiguous runs of ``block`` elements along the last dimension;
* Kronecker form R = (H_K (x) H_M) / sqrt(K M) with K outer, so the length-M
  pieces of a row are contiguous; K is the smallest order K = odd(n) * 2^j
  (j >= 0) dividing n for which a Paley I matrix exists (K - 1 a prime power
  congruent to 3 mod 4);
* the Paley I matrix for q = K - 1: field elements of GF(p^r) are indexed by
  i = c0 + c1 p + ... (base-p digits are the coefficients of the polynomial
  basis) modulo the first monic irreducible polynomial of degree r when
  monic polynomials are enumerated by the integer a0 + a1 p + ... + a_{r-1}
  p^{r-1}; Q[i][j] = chi(x_i - x_j) (quadratic character);
  H = I + [[0, 1^T], [-1, Q]].  The pages' table of known matrices is not
  available, so which Hadamard matrix of order K is used is a reading; the
  construction is pinned to H H^T = K I and to its closed form for prime q.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------- Sylvester

def sylvester(n: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix of order n (int64), built by the
    recursion H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]] (AutoRound
    "Rotation Transform", section 1.5)."""
    if n < 1 or n & (n - 1):
        raise ValueError("Sylvester Hadamard order must be a power of two, got %d" % n)
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# ------------------------------------------------------- finite fields, Paley

def _prime_power(q: int):
    """Return (p, r) with q = p^r, p prime, or None."""
    if q < 2:
        return None
    p = None
    for d in range(2, int(math.isqrt(q)) + 1):
        if q % d == 0:
            p = d
            break
    if p is None:
        return (q, 1)
    r = 0
    while q % p == 0:
        q //= p
        r += 1
    return (p, r) if q == 1 else None


def _poly_mulmod(a, b, mod, p):
    """Multiply polynomials a, b (coefficient lists, low degree first) over
    GF(p) and reduce modulo the monic polynomial ``mod`` (length r + 1)."""
    r = len(mod) - 1
    prod = [0] * (2 * r - 1)
    for i, ai in enumerate(a):
        if ai:
            for j, bj in enumerate(b):
                prod[i + j] = (prod[i + j] + ai * bj) % p
    for d in range(len(prod) - 1, r - 1, -1):
        c = prod[d]
        if c:
            for k in range(r + 1):
                prod[d - r + k] = (prod[d - r + k] - c * mod[k]) % p
    return prod[:r]


def _is_irreducible(mod, p):
    """True if the monic polynomial ``mod`` (degree r) is irreducible over
    GF(p), by brute force: no monic factor of degree 1..r//2 divides it."""
    r = len(mod) - 1

    def divides(f, g):
        # f monic of degree < deg g; polynomial long division g mod f == 0 ?
        g = list(g)
        df = len(f) - 1
        for d in range(len(g) - 1, df - 1, -1):
            c = g[d] % p
            if c:
                for k in range(df + 1):
                    g[d - df + k] = (g[d - df + k] - c * f[k]) % p
        return all(x % p == 0 for x in g[:df])

    for deg in range(1, r // 2 + 1):
        for code in range(p ** deg):
            f = [(code // p ** k) % p for k in range(deg)] + [1]
            if divides(f, mod):
                return False
    return True


def _field_modulus(p: int, r: int):
    """First monic irreducible polynomial of degree r over GF(p), enumerating
    monic polynomials by the integer a0 + a1 p + ... + a_{r-1} p^{r-1}."""
    if r == 1:
        return [0, 1]
    for code in range(p ** r):
        mod = [(code // p ** k) % p for k in range(r)] + [1]
        if _is_irreducible(mod, p):
            return mod
    raise AssertionError("no irreducible polynomial found")


def _quadratic_character(q: int):
    """Return (elements, chi, sub) for GF(q): elements as coefficient tuples in
    index order, chi as a length-q int array over indices, and a function
    sub(i, j) giving the index of x_i - x_j."""
    pr = _prime_power(q)
    if pr is None:
        raise ValueError("%d is not a prime power" % q)
    p, r = pr
    mod = _field_modulus(p, r)
    elems = [tuple((i // p ** k) % p for k in range(r)) for i in range(q)]

    def index(c):
        return sum(int(ck) * p ** k for k, ck in enumerate(c))

    squares = set()
    for e in elems[1:]:
        squares.add(index(_poly_mulmod(list(e), list(e), mod, p)))
    chi = np.array([0] + [1 if i in squares else -1 for i in range(1, q)], dtype=np.int64)

    def sub(i, j):
        return index([(a - b) % p for a, b in zip(elems[i], elems[j])])

    return elems, chi, sub


def paley_hadamard(k: int) -> np.ndarray:
    """Paley I Hadamard matrix of order k = q + 1 with q a prime power and
    q = 3 (mod 4), as int64 entries +-1 (base matrix for the Kronecker driver,
    AutoRound "Rotation Transform", section 1.5; the pages' table is not
    available, so the choice of this matrix is a reading; pinned to
    H H^T = k I and, for prime q, to the bordered-circulant closed form)."""
    q = k - 1
    if _prime_power(q) is None or q % 4 != 3:
        raise ValueError("no Paley I construction for order %d" % k)
    _, chi, sub = _quadratic_character(q)
    jac = np.empty((q, q), dtype=np.int64)
    for i in range(q):
        for j in range(q):
            jac[i, j] = chi[sub(i, j)]
    s = np.zeros((k, k), dtype=np.int64)
    s[0, 1:] = 1
    s[1:, 0] = -1
    s[1:, 1:] = jac
    return np.eye(k, dtype=np.int64) + s


def _paley_exists(k: int) -> bool:
    q = k - 1
    return k % 4 == 0 and _prime_power(q) is not None and q % 4 == 3


def kron_factor(n: int):
    """Factor a width n that is not a power of two as n = K * M, M = 2^m, with
    K the smallest order odd(n) * 2^j (j >= 0) that divides n and has a Paley I
    matrix (AutoRound "Rotation Transform", section 1.5: a width that is not
    a power of two is split into a base order times a power of two).  Returns (K, M); raises ValueError when no order works."""
    if n < 1:
        raise ValueError("width must be positive")
    if n & (n - 1) == 0:
        raise ValueError("%d is a power of two; no Kronecker factor needed" % n)
    odd = n
    while odd % 2 == 0:
        odd //= 2
    k = odd
    while n % k == 0:
        if _paley_exists(k):
            return k, n // k
        k *= 2
    raise ValueError("no supported Hadamard order K with n = K * 2^m for n = %d" % n)


# ------------------------------------------------------------ rotation matrix

def rotation_matrix(n: int, block: int = 0) -> np.ndarray:
    """Dense orthogonal rotation R (float64, n x n) for width n and block size:

    * block <= 0 (None / -1 on the pages means full width) and n a power of
      two: H_n / sqrt(n);
    * block <= 0 and n not a power of two: (H_K (x) H_M) / sqrt(n) with
      (K, M) = kron_factor(n);
    * block > 0: block-diagonal diag(H_b, ..., H_b) / sqrt(b); b must be a
      power of two dividing n (AutoRound page, sections 1.2 and 2.1).
    """
    if block is None or block <= 0 or block == n:
        if n & (n - 1) == 0:
            return sylvester(n).astype(np.float64) / math.sqrt(n)
        k, m = kron_factor(n)
        return np.kron(paley_hadamard(k), sylvester(m)).astype(np.float64) / math.sqrt(n)
    if block & (block - 1) or n % block:
        raise ValueError("block must be a power of two dividing n (n=%d, block=%d)" % (n, block))
    r = np.zeros((n, n), dtype=np.float64)
    hb = sylvester(block).astype(np.float64) / math.sqrt(block)
    for s in range(0, n, block):
        r[s:s + block, s:s + block] = hb
    return r


def rotate(x, n: int, block: int = 0, chunk_rows: int = 2048) -> np.ndarray:
    """y = x . R in float64 for x of shape [..., n] (any float dtype; bfloat16
    torch tensors are widened exactly).  Rows are processed in chunks to bound
    memory.  For block-diagonal R each block's product is taken separately,
    which is the same product with the zero blocks skipped."""
    x64 = _as_f64(x)
    if x64.shape[-1] != n:
        raise ValueError("last dimension must be n")
    lead = x64.shape[:-1]
    x2 = x64.reshape(-1, n)
    y = np.empty_like(x2)
    if block is None or block <= 0 or block == n:
        r = rotation_matrix(n, 0)
        for s in range(0, x2.shape[0], chunk_rows):
            y[s:s + chunk_rows] = x2[s:s + chunk_rows] @ r
    else:
        if block & (block - 1) or n % block:
            raise ValueError("block must be a power of two dividing n")
        hb = sylvester(block).astype(np.float64) / math.sqrt(block)
        for s in range(0, x2.shape[0], chunk_rows):
            xs = x2[s:s + chunk_rows]
            for b0 in range(0, n, block):
                y[s:s + chunk_rows, b0:b0 + block] = xs[:, b0:b0 + block] @ hb
    return y.reshape(*lead, n)


def mixing_matrices(n: int, perm=None, in_signs=None, out_signs=None):
    """Dense factors of the randomised rotations (float64, n x n each):

    * P with P[perm[j], j] = 1, so (x . P)[j] = x[perm[j]] (a gather; the
      identity when perm is None);
    * D_in = diag(in_signs) and D_out = diag(out_signs), a negative entry
      meaning -1 and any other +1 (the identity when None).

    The random Hadamard of the AutoRound page (section 1.5, "Random": H times
    diag(+-1) over sqrt(N)) is R . D_out; OrbitQuant's RPBH ("Method
    Conformance": permutation, Rademacher signs, block FWHT, orthonormal
    scaling) is P . D_in . R.
    """
    pm = np.eye(n)
    if perm is not None:
        perm = np.asarray(perm, dtype=np.int64).reshape(-1)
        if perm.shape != (n,) or not np.array_equal(np.sort(perm), np.arange(n)):
            raise ValueError("perm must be a permutation of 0..n-1")
        pm = np.zeros((n, n))
        pm[perm, np.arange(n)] = 1.0

    def diag(s):
        if s is None:
            return np.eye(n)
        s = np.asarray(s).reshape(-1)
        if s.shape != (n,):
            raise ValueError("sign vectors must have n entries")
        return np.diag(np.where(s < 0, -1.0, 1.0))

    return pm, diag(in_signs), diag(out_signs)


def rotate_mixed(x, n: int, block: int = 0, perm=None, in_signs=None, out_signs=None) -> np.ndarray:
    """y = x . P . D_in . R . D_out in float64 (factors as in mixing_matrices,
    R = rotation_matrix(n, block)): four dense matrix products, taken left to
    right on the rows."""
    pm, di, do = mixing_matrices(n, perm, in_signs, out_signs)
    x64 = _as_f64(x)
    if x64.shape[-1] != n:
        raise ValueError("last dimension must be n")
    y = x64.reshape(-1, n) @ pm @ di @ rotation_matrix(n, block) @ do
    return y.reshape(x64.shape)


def rotate_out(w, out_features: int, block: int = 0) -> np.ndarray:
    """W' = R^T . W for a weight W [out_features, in_features] (float64): the
    rotation of the layer's output, absorbed into its weight. For a layer
    y = x . W^T the rotated output is y . R = x . (R^T W)^T (AutoRound page,
    section 1.1: R1 fused into the outputs of o_proj / down_proj when
    online_r1_rotation is False, and R2 on the v_proj output per head of
    head_dim rows). R = rotation_matrix(out_features, block)."""
    w64 = _as_f64(w)
    if w64.ndim != 2 or w64.shape[0] != out_features:
        raise ValueError("w must be [out_features, in_features]")
    return rotation_matrix(out_features, block).T @ w64


def _as_f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)
