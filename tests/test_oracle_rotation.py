"""Pins of the oracle's rotation R = U · Hadamard · bit-reversal against closed forms, a library
Hadamard, an independent fast Walsh-Hadamard transform and the roles the pages give each factor
("超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化", section OSCAR 的设计: U aligns the
attention-relevant directions, the Hadamard spreads outlier energy, the bit-reversal balances the
INT2 groups)."""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_library_sylvester(d):
    assert np.array_equal(oracle.hadamard(d), scipy.linalg.hadamard(d).astype(np.float64))


@pytest.mark.parametrize("d", [2, 8, 128])
def test_hadamard_orthogonal(d):
    h = oracle.hadamard(d)
    assert np.array_equal(h @ h.T, d * np.eye(d))


def test_bit_reverse_closed_form_values():
    # 7-bit reversal: 0000001 -> 1000000, 0000011 -> 1100000, 1111111 -> 1111111
    assert oracle.bit_reverse(1, 128) == 64
    assert oracle.bit_reverse(3, 128) == 96
    assert oracle.bit_reverse(127, 128) == 127
    assert oracle.bit_reverse(0, 128) == 0
    assert oracle.bit_reverse(6, 8) == 3      # 110 -> 011
    assert oracle.bit_reverse(1, 8) == 4      # 001 -> 100


@pytest.mark.parametrize("d", [2, 4, 8, 64, 128, 256])
def test_bit_reversal_is_involution(d):
    j = np.arange(d)
    r = oracle.bit_reverse(j, d)
    assert np.array_equal(np.sort(r), j)            # a permutation
    assert np.array_equal(oracle.bit_reverse(r, d), j)
    p = oracle.bit_reversal_matrix(d)
    assert np.array_equal(p, p.T)
    assert np.array_equal(p @ p, np.eye(d))


def _fwht(x):
    """Iterative in-place butterflies (a different algorithm from the oracle's dense product)."""
    y = np.array(x, dtype=np.float64)
    d = y.shape[-1]
    h = 1
    while h < d:
        for i in range(0, d, 2 * h):
            a = y[..., i:i + h].copy()
            b = y[..., i + h:i + 2 * h].copy()
            y[..., i:i + h] = a + b
            y[..., i + h:i + 2 * h] = a - b
        h *= 2
    return y


def test_fwht_path_equals_dense_rotation():
    uk, _ = workloads.rotation_bases(workloads.get("tiny_gqa4_1k"), 0)
    u = uk[0].numpy()
    rng = np.random.default_rng(0)
    x = rng.standard_normal((16, 128))
    y = _fwht(x @ u.astype(np.float64)) / math.sqrt(128)
    perm = np.array([int("{:07b}".format(j)[::-1], 2) for j in range(128)])
    fast = y[:, perm]
    dense = oracle.rotate(x, u)
    assert np.max(np.abs(fast - dense)) < 1e-12


def test_rotation_orthogonal_with_fp32_u():
    wl = workloads.get("qwen3_8b_100k")
    uk, uv = workloads.rotation_bases(wl, 0)
    for u in (uk[0], uk[7], uv[3]):
        r = oracle.rotation_matrix(u.numpy())
        assert np.max(np.abs(r @ r.T - np.eye(128))) <= 1e-6


def test_u_first_then_spread():
    # x along U's first column: x U = e_0, the Hadamard turns e_0 into a flat vector and the
    # permutation keeps it flat.  Multiplying on the other side (x R^T) or placing U last breaks it.
    uk, _ = workloads.rotation_bases(workloads.get("tiny_gqa4_1k"), 0)
    u = uk[0].numpy().astype(np.float64)
    x = u[:, 0]
    xr = oracle.rotate(x, u)
    assert np.max(np.abs(xr - 1 / math.sqrt(128))) < 1e-6
    # U's second column: e_1 H = (+,-,+,-,...); after the bit reversal the first 64 channels are
    # positive and the last 64 negative, so the two channel halves (two groups of 64) each hold a
    # constant vector.
    xr1 = oracle.rotate(u[:, 1], u)
    assert np.max(np.abs(xr1[:64] - 1 / math.sqrt(128))) < 1e-6
    assert np.max(np.abs(xr1[64:] + 1 / math.sqrt(128))) < 1e-6


def test_unrotate_inverts_rotate():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 128))
    # an exactly representable orthogonal U (fp64 QR): R R^T = I to rounding
    u64, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    assert np.max(np.abs(oracle.unrotate(oracle.rotate(x, u64), u64) - x)) < 1e-12
    # the fp32 U the kernels receive is orthogonal only to ~1e-7
    uk, _ = workloads.rotation_bases(workloads.get("tiny_gqa4_1k"), 0)
    u32 = uk[0].numpy()
    assert np.max(np.abs(oracle.unrotate(oracle.rotate(x, u32), u32) - x)) < 1e-5


def test_outlier_energy_spread():
    # A single outlier channel (x = 16 e_k) is spread evenly: every rotated channel with U = I has
    # magnitude 16 / sqrt(d).
    x = np.zeros(128)
    x[17] = 16.0
    xr = oracle.rotate(x, np.eye(128, dtype=np.float32))
    assert np.allclose(np.abs(xr), 16 / math.sqrt(128), atol=1e-12)
