"""Pins of the query-preparation oracle (oracle/prep.py) against closed forms,
invariants and a hand-worked example.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import prep as P


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_sylvester_closed_form():
    # H[i, j] = (-1) ** popcount(i & j), written independently of the recursion
    for d in (1, 2, 4, 8, 128):
        h = P.sylvester(d)
        ref = np.array([[(-1) ** bin(i & j).count("1") for j in range(d)] for i in range(d)], dtype=np.float64)
        assert np.array_equal(h, ref)
        assert np.array_equal(h @ h.T, d * np.eye(d))


def test_hand_example_d4():
    # q = [1, 2, 3, 4], rope_dim = 2 half-split with angle pi/2 (cos 0, sin 1):
    # pair (0, 1): (1, 2) -> (1*0 - 2*1, 1*1 + 2*0) = (-2, 1); x = [-2, 1, 3, 4]
    # H4 x / 2 = [(-2+1+3+4), (-2-1+3-4), (-2+1-3-4), (-2-1-3+4)] / 2 = [3, -2, -4, -1]
    q = bf16_bits([[[1, 2, 3, 4]]])
    out = P.prep_query(q, np.array([[0.0]]), np.array([[1.0]]), rope_dim=2)
    assert np.array_equal(out[0, 0], [3.0, -2.0, -4.0, -1.0])
    # interleaved pairs (0, 1) too at rope_dim 2: the same result
    assert np.array_equal(P.prep_query(q, np.array([[0.0]]), np.array([[1.0]]), 2, True)[0, 0], [3.0, -2.0, -4.0, -1.0])
    # rope_dim 4 half-split pairs (0, 2), (1, 3), both by pi/2: [-3, -4, 1, 2] -> H/2
    out4 = P.prep_query(q, np.array([[0.0, 0.0]]), np.array([[1.0, 1.0]]), rope_dim=4)
    assert np.array_equal(out4[0, 0], [(-3 - 4 + 1 + 2) / 2, (-3 + 4 + 1 - 2) / 2, (-3 - 4 - 1 - 2) / 2,
                                       (-3 + 4 - 1 + 2) / 2])


def test_identity_rotation_and_involution():
    rng = np.random.default_rng(3)
    q = bf16_bits(rng.standard_normal((3, 5, 128)))
    x = P.decode_bf16(q)
    ones, zeros = np.ones((3, 64)), np.zeros((3, 64))
    # cos 1, sin 0 rotates nothing; the transform is its own inverse
    y = P.prep_query(q, ones, zeros, rope_dim=128)
    assert np.allclose(P.hadamard(y), x, rtol=0, atol=1e-12)
    assert np.allclose(P.prep_query(q, zeros[:, :0], zeros[:, :0], rope_dim=0), y, rtol=0, atol=0)
    # orthonormal: norms are preserved, with any rotation
    ang = rng.uniform(-np.pi, np.pi, (3, 64))
    z = P.prep_query(q, np.cos(ang), np.sin(ang), rope_dim=128)
    assert np.allclose(np.linalg.norm(z, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_unit_vectors_give_hadamard_columns():
    d = 128
    e = np.zeros((1, d, d), dtype=np.float32)
    e[0, np.arange(d), np.arange(d)] = 1.0
    y = P.prep_query(bf16_bits(e), np.zeros((1, 0)), np.zeros((1, 0)), rope_dim=0)
    col = np.array([[(-1) ** bin(i & j).count("1") for i in range(d)] for j in range(d)]) / np.sqrt(d)
    assert np.allclose(y[0], col, rtol=0, atol=1e-15)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_composes(interleaved):
    # rotating by a, then by b, equals rotating by a + b (cos / sin of the sum)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 128))
    a, b = rng.uniform(-3, 3, (2, 32)), rng.uniform(-3, 3, (2, 32))
    r1 = P.rope(P.rope(x, np.cos(a), np.sin(a), 64, interleaved), np.cos(b), np.sin(b), 64, interleaved)
    r2 = P.rope(x, np.cos(a + b), np.sin(a + b), 64, interleaved)
    assert np.allclose(r1, r2, rtol=0, atol=1e-12)
    assert np.array_equal(r1[..., 64:], x[..., 64:])          # dims past rope_dim pass through


def test_pairing_layouts():
    # half-split pairs (i, i + 32); interleaved pairs (2i, 2i + 1), with one rotated pair
    x = np.arange(128, dtype=np.float64).reshape(1, 1, 128)
    c, s = np.ones((1, 32)), np.zeros((1, 32))
    c[0, 5], s[0, 5] = 0.0, 1.0
    h = P.rope(x, c, s, 64, False)[0, 0]
    assert (h[5], h[37]) == (-37.0, 5.0) and np.array_equal(np.delete(h, [5, 37]), np.delete(x[0, 0], [5, 37]))
    i = P.rope(x, c, s, 64, True)[0, 0]
    assert (i[10], i[11]) == (-11.0, 10.0) and np.array_equal(np.delete(i, [10, 11]), np.delete(x[0, 0], [10, 11]))


def test_bf16_ulp():
    assert P.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert P.bf16_ulp(np.array([1.99]))[0] == 2.0 ** -7
    assert P.bf16_ulp(np.array([2.0]))[0] == 2.0 ** -6
    assert P.bf16_ulp(np.array([-0.3]))[0] == 2.0 ** -9
