"""Pins of the oracle's Walsh-Hadamard rotation (UltraQuant article, technology section: an orthogonal
Walsh-Hadamard transform evens out the value distribution before 4-bit compression). The pins are
closed forms of the Hadamard matrix, not the oracle's own butterflies."""
import numpy as np
import pytest

SIZES = [2, 4, 8, 16, 32, 64, 128, 256]


def popcount_sign_matrix(n):
    i = np.arange(n)
    m = np.bitwise_and.outer(i, i)
    pc = np.array([[bin(int(x)).count("1") for x in row] for row in m])
    return np.where(pc % 2 == 0, 1.0, -1.0)


@pytest.mark.parametrize("n", SIZES)
def test_columns_are_sylvester_hadamard(orc, n):
    # FWHT(e_j) must be column j of H with H[i][j] = (-1)^popcount(i & j) (natural / Sylvester order).
    H = np.stack([orc.fwht_f32(np.eye(n, dtype=np.float32)[j]) for j in range(n)], axis=1)
    assert np.array_equal(H, popcount_sign_matrix(n))


@pytest.mark.parametrize("n", SIZES)
def test_h_ht_is_n_identity(orc, n):
    # H H^T = n I, the defining property of a Hadamard matrix.
    H = np.stack([orc.fwht_f32(np.eye(n, dtype=np.float32)[j]) for j in range(n)], axis=1).astype(np.float64)
    assert np.array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", [64, 128, 256])
def test_involution_exact_on_small_integers(orc, n):
    # H (H x) = n x, exact in fp32 while every partial sum stays an integer below 2^24.
    rng = np.random.default_rng(1)
    x = rng.integers(-50, 51, n).astype(np.float32)
    y = orc.fwht_f32(orc.fwht_f32(x))
    assert np.array_equal(y, n * x)


@pytest.mark.parametrize("n", [64, 128, 256])
def test_matches_fp64_matrix_product(orc, n):
    # Random fp32 input: each output is a sum of n terms, error <= log2(n) roundings of the running sums.
    rng = np.random.default_rng(2)
    x = rng.standard_normal(n).astype(np.float32)
    y = orc.fwht_f32(x).astype(np.float64)
    ref = popcount_sign_matrix(n) @ x.astype(np.float64)
    bound = np.log2(n) * np.abs(x).sum() * 2.0 ** -24
    assert np.max(np.abs(y - ref)) <= bound


@pytest.mark.parametrize("n", [64, 128, 256])
def test_rotation_scale_and_orthogonality(orc, n):
    c = orc.rot_scale(n)
    assert c == float(np.float32(1.0 / np.sqrt(n)))          # fp32(1/sqrt(n)), correctly rounded
    assert abs(c * c * n - 1.0) < 2 * 2.0 ** -23              # c H is orthogonal up to the rounding of c
    rng = np.random.default_rng(3)
    x = rng.standard_normal(n).astype(np.float32)
    once = orc.fwht_f32(x) * np.float32(c)
    twice = orc.fwht_f32(once) * np.float32(c)
    assert np.max(np.abs(twice - x)) < 1e-5
