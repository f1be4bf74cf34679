"""Pins for the oracle's Hadamard constructions and rotation (CPU only).

Each check ties the oracle to something other than itself: the hand-worked
cases in tests/golden/hand_cases.json, closed forms (popcount entries,
H H^T = n I), invariants (orthogonality, norm preservation, the weight
pairing x R R^T W^T = x W^T from the AutoRound "Rotation Transform"
introduction), and an independent fast Walsh-Hadamard transform written here.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import hadamard as H

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def fwht_reference(x):
    """Independent in-place iterative FWHT (natural order), unnormalised,
    float64, along the last axis."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(*y.shape[:-1], n // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(*y.shape[:-3], n)
        h *= 2
    return y


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_sylvester_orthogonal_exact(n):
    h = H.sylvester(n)
    assert h.dtype == np.int64
    assert set(np.unique(h)) <= {-1, 1}
    # float64 BLAS product: every partial sum is an integer of magnitude <= n,
    # so it is exact
    hf = h.astype(np.float64)
    assert np.array_equal(hf @ hf.T, n * np.eye(n))
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("n", [2, 8, 64, 256])
def test_sylvester_popcount_closed_form(n):
    h = H.sylvester(n)
    for i in range(n):
        for j in range(n):
            assert h[i, j] == (-1) ** bin(i & j).count("1")


@pytest.mark.parametrize("n", [4, 128, 4096])
def test_normalised_involutory(n):
    r = oracle.rotation_matrix(n)
    assert np.allclose(r @ r, np.eye(n), atol=1e-12)


def test_one_hot_and_constant_vectors():
    n = 256
    r = oracle.rotation_matrix(n)
    for i in (0, 1, 37, 255):
        e = np.zeros(n)
        e[i] = 1.0
        assert np.allclose(e @ r, H.sylvester(n)[i] / math.sqrt(n), atol=0)
    y = np.ones(n) @ r
    expect = np.zeros(n)
    expect[0] = math.sqrt(n)
    assert np.allclose(y, expect, atol=1e-12)


def test_hand_cases_h2_h4():
    for key, n in (("h2", 2), ("h4", 4)):
        c = GOLDEN[key]
        y = oracle.rotate(np.array([c["x"]]), n)
        assert np.allclose(y[0], c["y"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("n", [2, 16, 128, 1024, 4096])
def test_dense_product_matches_independent_fwht(n):
    rng = np.random.default_rng(100 + n)
    x = rng.standard_normal((5, n))
    y = oracle.rotate(x, n)
    ref = fwht_reference(x) / math.sqrt(n)
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("n,block", [(14336, 2048), (256, 32), (96, 32), (4096, 4096), (64, 2)])
def test_block_diagonal_matches_per_block_fwht(n, block):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, n))
    y = oracle.rotate(x, n, block)
    ref = fwht_reference(x.reshape(3, n // block, block)).reshape(3, n) / math.sqrt(block)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.abs(ref).max()
    # the dense block-diagonal matrix gives the same product
    if n <= 4096:
        assert np.allclose(x @ oracle.rotation_matrix(n, block), y, rtol=0, atol=1e-12)


def test_block_equal_to_width_is_full_width():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 512))
    assert np.array_equal(oracle.rotate(x, 512, 512), oracle.rotate(x, 512, 0))
    assert np.array_equal(oracle.rotate(x, 512, -1), oracle.rotate(x, 512, 0))


@pytest.mark.parametrize("n,block", [(4096, 0), (14336, 2048), (14336, 0), (128, 0), (96, 0)])
def test_norm_preservation_and_weight_pairing(n, block):
    """||x R|| = ||x|| and (x R)(W R)^T = x W^T within 1e-10 relative."""
    rng = np.random.default_rng(n + max(block, 0))
    x = rng.standard_normal((3, n))
    w = rng.standard_normal((5, n))
    xr = oracle.rotate(x, n, block)
    wr = oracle.rotate(w, n, block)
    assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    ref = x @ w.T
    got = xr @ wr.T
    assert np.max(np.abs(got - ref)) <= 1e-10 * np.abs(ref).max()


def test_kronecker_with_two_is_sylvester():
    """K-outer Kronecker convention: H_2 (x) H_n equals H_2n."""
    for n in (1, 4, 64):
        assert np.array_equal(np.kron(H.sylvester(2), H.sylvester(n)), H.sylvester(2 * n))


@pytest.mark.parametrize("k", [4, 8, 12, 20, 24, 28, 32, 44, 48, 60, 68, 72, 80, 84, 104, 108, 132, 140])
def test_paley_hadamard(k):
    h = H.paley_hadamard(k)
    assert set(np.unique(h)) <= {-1, 1}
    assert np.array_equal(h @ h.T, k * np.eye(k, dtype=np.int64))


@pytest.mark.parametrize("k", [12, 20, 24, 44, 48, 60, 68, 72, 80, 84, 104, 108, 132, 140])
def test_paley_prime_closed_form(k):
    """For prime q = k - 1 the Paley I matrix of AutoRound "Rotation
    Transform", section 1.5's base orders has the textbook closed form:
    row 0 all +1, column 0 -1 below it, +1 on the diagonal, and
    H[1 + a][1 + b] = Legendre(a - b | q) elsewhere.  The Legendre symbol is
    taken from Euler's criterion (a^((q-1)/2) mod q), not from the oracle's
    table of squares."""
    q = k - 1
    if any(q % d == 0 for d in range(2, int(q ** 0.5) + 1)):
        pytest.skip("q = %d is not prime" % q)
    want = np.ones((k, k), dtype=np.int64)
    want[1:, 0] = -1
    for a in range(q):
        for b in range(q):
            if a != b:
                e = pow((a - b) % q, (q - 1) // 2, q)
                want[1 + a, 1 + b] = 1 if e == 1 else -1
    assert np.array_equal(H.paley_hadamard(k), want)


def test_gf27_modulus_and_squares():
    # x^3 + 2x + 1 is the first monic irreducible cubic over GF(3) in the
    # enumeration order (worked by hand: codes 0..6 all have a root in GF(3)).
    assert H._field_modulus(3, 3) == [1, 2, 0, 1]
    _, chi, _ = H._quadratic_character(27)
    assert chi[0] == 0
    assert int((chi == 1).sum()) == 13 and int((chi == -1).sum()) == 13
    # GF(11): squares of 1..10 are {1, 3, 4, 5, 9}
    _, chi11, _ = H._quadratic_character(11)
    assert [i for i in range(11) if chi11[i] == 1] == [1, 3, 4, 5, 9]


def test_paley_unsupported_orders():
    for k in (36, 52, 56):  # q = 35, 51, 55 are not prime powers
        with pytest.raises(ValueError):
            H.paley_hadamard(k)


@pytest.mark.parametrize("n,expect", [
    (14336, (28, 512)), (12, (12, 1)), (96, (12, 8)), (20, (20, 1)), (5120, (20, 256)),
    (11008, (344, 32)), (144, (72, 2)), (28 * 4, (28, 4)), (3 * 2 ** 10, (12, 256)),
])
def test_kron_factor(n, expect):
    assert H.kron_factor(n) == expect


@pytest.mark.parametrize("n", [18, 7, 4096])
def test_kron_factor_rejects(n):
    with pytest.raises(ValueError):
        H.kron_factor(n)


@pytest.mark.parametrize("n", [14336, 96, 20 * 16])
def test_kronecker_rotation_two_step(n):
    """x (H_K (x) H_M) / sqrt(n) equals: FWHT each contiguous length-M piece,
    then mix the K pieces with H_K^T (the K-outer Kronecker identity)."""
    k, m = H.kron_factor(n)
    rng = np.random.default_rng(n)
    x = rng.standard_normal((2, n))
    y = oracle.rotate(x, n)
    z = fwht_reference(x.reshape(2, k, m))
    hk = H.paley_hadamard(k).astype(np.float64)
    ref = np.einsum("ak,rkm->ram", hk.T, z).reshape(2, n) / math.sqrt(n)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.abs(ref).max()
    r = oracle.rotation_matrix(n) if n <= 4096 else None
    if r is not None:
        assert np.allclose(r @ r.T, np.eye(n), atol=1e-12)


def test_incoherence_drops_under_rotation():
    """QuIP note, 'Incoherence' section: a matrix with planted outliers has a
    large mu (max entry / rms entry); a Hadamard rotation brings it near the
    Gaussian level sqrt(2 ln(mn)).  Sanity check, not a parity pin."""
    import synth
    x = synth.r1_activations(seed=2, tokens=256, hidden=1024).float().numpy().astype(np.float64)
    mu = lambda a: np.abs(a).max() / np.sqrt(np.mean(a * a))
    y = oracle.rotate(x, 1024)
    assert mu(x) > 50
    assert mu(y) < 2.5 * math.sqrt(2 * math.log(x.size))


# ------------------------------------------------ randomised rotations (f2)

@pytest.mark.parametrize("case", ["mixed_h2_rpbh", "mixed_h2_random", "mixed_h4_all"])
def test_mixed_hand_cases(case):
    c = GOLDEN[case]
    n = len(c["x"])
    y = oracle.rotate_mixed(np.array([c["x"]]), n, 0, c.get("perm"), c.get("in_signs"), c.get("out_signs"))
    assert np.allclose(y[0], c["y"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("n,block", [(64, 0), (64, 16), (48, 0), (256, 32)])
def test_mixed_identity_reduces_to_plain(n, block):
    x = np.random.default_rng(n + block).standard_normal((5, n))
    y = oracle.rotate_mixed(x, n, block, np.arange(n), np.ones(n, np.int8), np.ones(n, np.int8))
    assert np.allclose(y, oracle.rotate(x, n, block), rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,block", [(64, 0), (128, 32), (48, 0), (1024, 64)])
def test_mixed_orthogonal_and_inverse(n, block):
    rng = np.random.default_rng(7 * n + block)
    x = rng.standard_normal((6, n))
    perm = rng.permutation(n)
    si = rng.choice([-1, 1], n).astype(np.int8)
    so = rng.choice([-1, 1], n).astype(np.int8)
    y = oracle.rotate_mixed(x, n, block, perm, si, so)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # undo step by step with elementwise operations: out signs, R^T, in signs, scatter
    z = y * so
    z = z @ oracle.rotation_matrix(n, block).T
    z = z * si
    back = np.empty_like(z)
    back[:, perm] = z
    assert np.allclose(back, x, rtol=0, atol=1e-12)


def test_mixed_brute_force_tiny():
    """n = 8, block 4, every factor present: explicit sums over the entries."""
    rng = np.random.default_rng(3)
    n, b = 8, 4
    x = rng.standard_normal(n)
    perm = rng.permutation(n)
    si = rng.choice([-1, 1], n)
    so = rng.choice([-1, 1], n)
    want = np.zeros(n)
    for k in range(n):
        acc = 0.0
        for j in range(n):
            if j // b == k // b:
                acc += si[j] * x[perm[j]] * (-1) ** bin((j % b) & (k % b)).count("1") / 2.0
        want[k] = so[k] * acc
    got = oracle.rotate_mixed(x[None], n, b, perm, si, so)[0]
    assert np.allclose(got, want, rtol=0, atol=1e-14)


def test_mixed_rejects_non_permutation():
    with pytest.raises(ValueError):
        oracle.rotate_mixed(np.zeros((1, 4)), 4, 0, [0, 1, 1, 3])


# ------------------------------------------------ output-side weight fusion (f3)

def test_out_fusion_hand_case():
    c = GOLDEN["out_fusion_h2"]
    assert np.allclose(oracle.rotate_out(np.array(c["w"]), 2), c["w_rot"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("out_f,in_f,block", [(64, 24, 0), (256, 40, 32), (128, 16, 128), (48, 8, 0)])
def test_out_fusion_layer_equivalence(out_f, in_f, block):
    """For y = x . W^T, the fused weight gives the rotated output:
    x . (R^T W)^T = (x . W^T) . R, and the rotation of the row side is
    unchanged by it."""
    rng = np.random.default_rng(out_f + in_f + block)
    w = rng.standard_normal((out_f, in_f))
    x = rng.standard_normal((7, in_f))
    wr = oracle.rotate_out(w, out_f, block)
    want = oracle.rotate(x @ w.T, out_f, block)
    assert np.allclose(x @ wr.T, want, rtol=0, atol=1e-12)
    # columns keep their norms (orthogonal R)
    assert np.allclose(np.linalg.norm(wr, axis=0), np.linalg.norm(w, axis=0), rtol=1e-13)


def test_out_fusion_brute_force_tiny():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((8, 3))
    got = oracle.rotate_out(w, 8, 4)
    want = np.zeros_like(w)
    for o in range(8):
        for i in range(3):
            want[o, i] = sum(w[r, i] * (-1) ** bin((r % 4) & (o % 4)).count("1") / 2.0
                             for r in range(8) if r // 4 == o // 4)
    assert np.allclose(got, want, rtol=0, atol=1e-14)
