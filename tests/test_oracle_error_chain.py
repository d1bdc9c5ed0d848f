"""Pins of the oracle's error-chain metrics (the comparison of the OSCAR write-up's figure 1:
attention-score KL and attention-output MSE of naive INT2, Hadamard-only, clip-only and OSCAR).

The metric functions are pinned by closed forms (an exact cache gives zero error; a constant
value shift d gives output MSE d^2 and KL 0; a key change along a direction orthogonal to every
query changes nothing), by Gibbs' inequality (KL >= 0) and by brute force on a tiny case; the
quantise-roundtrip by its bound (|error| <= s/2 in the frame, where the frame is orthogonal).
The variant comparison on a small synthetic layer checks only what the arithmetic of these
inputs fixes: with channel outliers of gain 16, quantising without a rotation (naive,
clip-only) gives far larger errors than either rotated variant."""
import math

import numpy as np
import pytest

import oracle
import workloads
from oracle import error_chain


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_exact_cache_has_zero_error():
    r = _rng(1)
    q, k, v = r.standard_normal((5, 16)), r.standard_normal((40, 16)), r.standard_normal((40, 16))
    kl, mse, ke, ve = oracle.attention_error_metrics(q, k, v, k, v, 0.25)
    assert kl == 0.0 and mse == 0.0 and ke == 0.0 and ve == 0.0


def test_value_shift_closed_form():
    # every output is a convex combination of the values: shifting all values by delta shifts
    # every output by delta exactly, and the score distribution is unchanged
    r = _rng(2)
    q, k, v = r.standard_normal((3, 8)), r.standard_normal((20, 8)), r.standard_normal((20, 8))
    kl, mse, ke, ve = oracle.attention_error_metrics(q, k, v, k, v + 0.125, 0.5)
    assert kl == pytest.approx(0.0, abs=1e-15)
    assert mse == pytest.approx(0.125 ** 2, rel=1e-12)
    assert ve == pytest.approx(0.125 ** 2, rel=1e-12) and ke == 0.0


def test_key_change_orthogonal_to_the_queries_changes_nothing():
    r = _rng(3)
    q = np.zeros((4, 6))
    q[:, :3] = r.standard_normal((4, 3))
    k, v = r.standard_normal((30, 6)), r.standard_normal((30, 6))
    k_hat = k.copy()
    k_hat[:, 3:] += r.standard_normal((30, 3))
    kl, mse, ke, _ = oracle.attention_error_metrics(q, k, v, k_hat, v, 1.0)
    assert kl == pytest.approx(0.0, abs=1e-13) and mse == pytest.approx(0.0, abs=1e-26)
    assert ke > 0.1


def test_kl_brute_force_and_gibbs():
    r = _rng(4)
    q, k, v = r.standard_normal((2, 4)), r.standard_normal((7, 4)), r.standard_normal((7, 4))
    k_hat = k + 0.3 * r.standard_normal((7, 4))
    kl, mse, _, _ = oracle.attention_error_metrics(q, k, v, k_hat, v, 0.7)
    tot_kl, tot_se = 0.0, 0.0
    for i in range(2):
        s = [0.7 * sum(q[i, c] * k[t, c] for c in range(4)) for t in range(7)]
        sh = [0.7 * sum(q[i, c] * k_hat[t, c] for c in range(4)) for t in range(7)]
        z, zh = sum(math.exp(x) for x in s), sum(math.exp(x) for x in sh)
        p = [math.exp(x) / z for x in s]
        ph = [math.exp(x) / zh for x in sh]
        tot_kl += sum(a * math.log(a / b) for a, b in zip(p, ph))
        for c in range(4):
            o = sum(p[t] * v[t, c] for t in range(7))
            oh = sum(ph[t] * v[t, c] for t in range(7))
            tot_se += (o - oh) ** 2
    assert kl == pytest.approx(tot_kl / 2, rel=1e-10)
    assert mse == pytest.approx(tot_se / 8, rel=1e-10)
    assert kl > 0


@pytest.mark.parametrize("frame", ["identity", "hadamard", "random"])
def test_roundtrip_error_bound_in_the_frame(frame):
    d, g = 128, 64
    r = _rng(5)
    x = r.standard_normal((50, d)) * 2
    u = None if frame == "identity" else (np.eye(d) if frame == "hadamard" else
                                          np.linalg.qr(r.standard_normal((d, d)))[0])
    rm = oracle.frame_matrix(u, d)
    assert np.allclose(rm @ rm.T, np.eye(d), atol=1e-12)
    xh = oracle.quantize_roundtrip(x, rm, np.inf, g)
    # back in the frame the error of each element is at most half a (fp16) step of its group,
    # plus the fp32 rounding of the rotated value and the fp16 rounding of the zero point
    xr = (x @ rm).astype(np.float32).astype(np.float64)
    er = (xh @ rm) - xr
    xg = xr.reshape(50, d // g, g)
    step = (xg.max(-1) - xg.min(-1)) / 3
    bound = np.repeat(step / 2 * (1 + 2e-3) + 1e-3 * np.abs(xg).max(-1), g, axis=-1)
    assert np.all(np.abs(er) <= bound.reshape(50, d))


def test_unrotated_variants_lose_to_the_rotated_ones_on_outlier_channels():
    wl = workloads.scaled(workloads.get("qwen3_4b_32k"), context=2048)
    res = error_chain.layer_errors(wl, kv=0, n_calib=128, n_eval=8)
    for bad in ("naive", "clip_only"):
        for good in ("hadamard_only", "oscar"):
            assert res[bad][0] > 3 * res[good][0], (bad, good)   # score KL
            assert res[bad][1] > 3 * res[good][1], (bad, good)   # output MSE
            assert res[bad][2] > 3 * res[good][2], (bad, good)   # key MSE
    for name in error_chain.VARIANTS:
        assert all(np.isfinite(res[name])) and res[name][0] >= 0
