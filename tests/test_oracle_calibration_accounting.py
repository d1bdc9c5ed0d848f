"""Pins of the oracle's offline calibration ("超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
section OSCAR 的设计: key rotation from the query covariance Q^T Q, value rotation from the
score-weighted value covariance V^T S^T S V) and of the storage accounting against the figures the
pages print (tests/golden/bits_per_element.txt)."""
import math
import os

import numpy as np
import pytest

import oracle
import workloads


def test_key_rotation_is_eigenbasis():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((3000, 32)) * np.linspace(3, 0.1, 32)
    u = oracle.key_rotation(q)
    c = q.T @ q
    lam = np.diag(u.T @ c @ u)
    assert np.max(np.abs(c @ u - u * lam)) <= 1e-9 * np.abs(c).max()
    assert np.max(np.abs(u.T @ u - np.eye(32))) < 1e-12
    assert np.all(np.diff(lam) <= 0)
    pick = np.argmax(np.abs(u), axis=0)
    assert np.all(u[pick, np.arange(32)] > 0)


def test_key_rotation_recovers_population_basis():
    # Queries drawn from N(0, O diag(lambda) O^T) with well separated eigenvalues: the leading
    # calibrated directions match O's leading columns up to sign.
    d = 16
    rng = np.random.default_rng(1)
    o = np.linalg.qr(rng.standard_normal((d, d)))[0]
    lam = 4.0 ** -np.arange(d)
    q = (rng.standard_normal((20000, d)) * np.sqrt(lam)) @ o.T
    u = oracle.key_rotation(q)
    for i in range(4):
        assert abs(abs(u[:, i] @ o[:, i]) - 1) < 1e-3


def test_value_rotation_uniform_scores_special_case():
    # identical keys -> every score row is uniform, so S V is the mean value for every query and
    # (S V)^T (S V) is rank one along that mean
    rng = np.random.default_rng(2)
    k = np.tile(rng.standard_normal(16), (50, 1))
    v = rng.standard_normal((50, 16)) + 2.0
    q = rng.standard_normal((30, 16))
    c = oracle.value_covariance(q, k, v, 0.25, chunk=7)
    mean = v.mean(0)
    assert np.max(np.abs(c - 30 * np.outer(mean, mean))) < 1e-9 * np.abs(c).max()
    u = oracle.value_rotation(q, k, v, 0.25)
    assert abs(abs(u[:, 0] @ mean / np.linalg.norm(mean)) - 1) < 1e-9


def test_value_covariance_matches_explicit_softmax():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((40, 8))
    v = rng.standard_normal((40, 8))
    q = rng.standard_normal((9, 8))
    c = oracle.value_covariance(q, k, v, 0.5, chunk=4)
    ref = np.zeros((8, 8))
    for qi in q:
        s = np.array([math.exp(0.5 * (qi @ kk)) for kk in k])
        s /= s.sum()
        sv = s @ v
        ref += np.outer(sv, sv)
    assert np.max(np.abs(c - ref)) < 1e-12


def test_clip_threshold_percentile():
    x = np.zeros((1000, 4))
    x[:, 0] = np.arange(1000)
    u = np.eye(4)
    # with U = I the rotated vectors are x H / 2 permuted, so every |x'_j| = x_0 / 2
    assert oracle.clip_threshold(x, u, 100.0) == pytest.approx(999 / 2)
    assert oracle.clip_threshold(x, u, 50.0) == pytest.approx(np.percentile(np.arange(1000) / 2, 50))


def _golden():
    rows = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "bits_per_element.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            key, _, ctx, grp, exp = [c.strip() for c in line.split("|")]
            rows[key] = (ctx, int(grp), float(exp))
    return rows


def test_bits_per_element_against_pages():
    g = _golden()
    _, grp, exp = g["fig3_int2_baselines"]
    assert oracle.history_bytes_per_token_head(128, grp) == 72
    assert oracle.history_bytes_per_token_head(128, grp) * 8 / 256 == exp
    ctx, grp, exp = g["fig4_aime25_32k"]
    assert round(oracle.effective_bits_per_element(int(ctx), 128, grp), 3) == exp
    _, _, exp = g["fig5_memory"]
    assert 16 / 2 == exp
    assert oracle.history_bytes_per_token_head(128, 64) == 80
    assert oracle.Geometry().block_bytes == 64 * 72 and oracle.Geometry(group=64).block_bytes == 64 * 80


def test_workload_queries_have_the_stated_spectrum():
    wl = workloads.get("qwen3_4b_32k")
    q = workloads.calibration_queries(wl, 0, n=4000).double().numpy()
    o = workloads.query_covariance_bases(wl, 0)
    lam = workloads.query_spectrum(128)
    assert abs(lam.sum() - 128) < 1e-9 and abs(lam[0] / lam[3] - 4 ** 1.5) < 1e-9
    proj = q[:, 0, :] @ o[0]
    var = proj.var(0)
    assert abs(var[0] / lam[0] - 1) < 0.1 and abs(var[10] / lam[10] - 1) < 0.1
