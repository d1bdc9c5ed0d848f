"""Pins of the oracle's Lloyd-Max codebook (reading R19: four levels in the group's normalised
coordinate, fitted by Lloyd's algorithm, with the uniform INT2 scale and zero point kept).

Lloyd's algorithm is pinned by textbook results it must reproduce: the 4-level Lloyd-Max quantiser
of a unit Gaussian (J. Max, "Quantizing for minimum distortion", IRE Trans. Inf. Theory, 1960:
levels +-0.4528 and +-1.510, thresholds 0 and +-0.9816, mean squared error 0.1175) and of a
uniform density (the uniform mid-rise quantiser, error step^2 / 12); by the two optimality
conditions at its fixed point; by its non-increasing distortion; and by brute force on four and
on seven points.  The codebook quantiser is pinned by the special case that reduces it to the uniform INT2
quantiser (levels 0, 1, 2, 3) and by the nearest-level property."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import error_chain


def test_unit_gaussian_matches_max_1960():
    x = np.linspace(-8.0, 8.0, 400001)
    lv, thr, hist = oracle.lloyd_max(x, np.exp(-x * x / 2), levels=(-1.5, -0.5, 0.5, 1.5),
                                     iters=300)
    assert np.allclose(lv, [-1.510, -0.4528, 0.4528, 1.510], atol=6e-4)
    assert np.allclose(thr, [-0.9816, 0.0, 0.9816], atol=2e-4)
    assert hist[-1] == pytest.approx(0.1175, abs=1e-4)


def test_uniform_density_gives_the_uniform_mid_rise_quantiser():
    x = np.linspace(0.0, 3.0, 300001)
    lv, thr, hist = oracle.lloyd_max(x, levels=(0, 1, 2, 3), iters=300)
    assert np.allclose(lv, [0.375, 1.125, 1.875, 2.625], atol=1e-4)
    assert np.allclose(thr, [0.75, 1.5, 2.25], atol=1e-4)
    assert hist[-1] == pytest.approx(0.75 ** 2 / 12, rel=1e-4)


def test_four_points_four_levels_brute_force():
    pts = np.array([0.1, 0.9, 2.2, 2.95])
    lv, _, hist = oracle.lloyd_max(pts, levels=(0, 1, 2, 3), iters=3)
    assert np.allclose(lv, pts) and hist[-1] == 0.0
    # brute force over every split of 7 sorted points into 4 contiguous cells: the optimal
    # split's centroids satisfy both conditions, so Lloyd's algorithm started there stays there
    for seed in range(5):
        r = np.sort(np.random.default_rng(seed).uniform(0, 3, 7))
        splits = [(a, b, e) for a in range(1, 5) for b in range(a + 1, 6) for e in range(b + 1, 7)]
        cost = [sum(((c - c.mean()) ** 2).sum() for c in np.split(r, s)) / 7 for s in splits]
        best = splits[int(np.argmin(cost))]
        cent = [c.mean() for c in np.split(r, best)]
        lv, _, h = oracle.lloyd_max(r, levels=cent, iters=5)
        assert np.allclose(lv, cent, rtol=0, atol=1e-15)
        assert h[-1] == pytest.approx(min(cost), rel=1e-12)


def test_fixed_point_conditions_and_monotone_distortion():
    r = np.random.default_rng(1)
    t = np.clip(r.normal(1.5, 0.6, 20000), 0, 3)
    lv, thr, hist = oracle.lloyd_max(t, iters=200)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))
    assert np.allclose(thr, (lv[:-1] + lv[1:]) / 2)
    cell = np.searchsorted(thr, t, side="left")
    for i in range(4):
        assert lv[i] == pytest.approx(t[cell == i].mean(), abs=1e-9)
    # a bell-shaped density pulls the outer levels inwards from the grid's end points
    assert 0 < lv[0] and lv[3] < 3


@pytest.mark.parametrize("group", [32, 128])
def test_uniform_levels_reduce_to_the_int2_quantiser(group):
    r = np.random.default_rng(2)
    xr = (r.standard_normal((64, 128)) * 3).astype(np.float32)
    codes, s, z, pre = oracle.quantize(xr, 4.0, group)
    cb, cs, cz = oracle.quantize_codebook(xr, 4.0, group, (0, 1, 2, 3))
    assert np.array_equal(s.view(np.uint16), cs.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), cz.view(np.uint16))
    frac = pre["t"] - np.floor(pre["t"])
    tie = frac == 0.5
    assert not tie.any()   # halfway values would round to even in one and down in the other
    assert np.array_equal(codes, cb)
    assert np.array_equal(oracle.dequantize(codes, s, z, group),
                          oracle.dequantize_codebook(cb, cs, cz, group, (0, 1, 2, 3)))


def test_codebook_codes_name_the_nearest_level():
    r = np.random.default_rng(3)
    xr = r.standard_normal((32, 128)).astype(np.float32)
    levels = (0.2, 0.9, 2.05, 2.8)
    codes, s, z = oracle.quantize_codebook(xr, np.inf, 64, levels)
    t = oracle.codebook_coordinates(xr, np.inf, 64)
    dist = np.abs(t[..., None] - np.asarray(levels))
    assert np.all(dist[np.arange(32)[:, None], np.arange(128), codes] <= dist.min(-1) + 1e-12)
    # reconstruction is s * level + z group by group
    sf = np.repeat(s.astype(np.float64), 64, -1)
    zf = np.repeat(z.astype(np.float64), 64, -1)
    assert np.allclose(oracle.dequantize_codebook(codes, s, z, 64, levels),
                       sf * np.asarray(levels)[codes] + zf, rtol=0, atol=1e-12)


def test_fitted_codebooks_do_not_lose_on_their_calibration_data():
    # Lloyd's iterations start from the uniform grid and never increase the distortion, so on the
    # calibration coordinates the fitted levels do at least as well as the INT2 grid
    wl = workloads.scaled(workloads.get("qwen3_4b_32k"), context=2048)
    d = wl.head_dim
    r = oracle.frame_matrix(np.eye(d), d)
    k_cal, _ = workloads.kv_tokens(wl, 0, 1, 0, 1024)
    t = oracle.codebook_coordinates((k_cal[:, 0].double().numpy() @ r).astype(np.float32),
                                    np.inf, wl.group_size)
    lv, _, hist = oracle.lloyd_max(t, iters=50)
    assert hist[-1] <= hist[0]
    grid = np.clip(np.rint(t), 0, 3)
    assert hist[0] == pytest.approx(np.mean((t - grid) ** 2), rel=1e-12)
    levels = error_chain.codebooks(wl, 0, (r, np.inf, r, np.inf), n_tokens=1024, iters=50)
    assert np.allclose(levels[0], lv)
    # the equally spaced fit likewise starts from the plain grid (lo 0, step 1) and cannot lose
    lo, step, hist_u = oracle.lloyd_max_uniform(t, iters=50)
    assert hist_u[-1] <= hist_u[0] and hist_u[0] == pytest.approx(hist[0], rel=1e-12)
    # equally spaced levels are a special case of free ones, so on these data the free fit (a
    # local optimum from the same start) is not beaten beyond a small margin
    assert hist_u[-1] >= hist[-1] - 1e-3
    spaced = error_chain.codebooks(wl, 0, (r, np.inf, r, np.inf), n_tokens=1024, iters=50,
                                   uniform=True)
    assert spaced[0] == (np.float32(lo), np.float32(step))


# ---- the equally spaced codebook that the GPU encoder runs (reading R20)

def test_optimum_uniform_quantiser_of_a_unit_gaussian_matches_max_1960():
    # Max's table of optimum uniform quantisers: 4 levels, step 0.9957, mean squared error 0.1188
    x = np.linspace(-8.0, 8.0, 400001)
    lo, step, hist = oracle.lloyd_max_uniform(x, np.exp(-x * x / 2), lo=-1.5, step=1.0, iters=300)
    assert step == pytest.approx(0.9957, abs=2e-4)
    assert lo == pytest.approx(-1.5 * step, abs=1e-4)
    assert hist[-1] == pytest.approx(0.1188, abs=1e-4)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))
    # and it cannot beat the unconstrained Lloyd-Max quantiser (0.1175)
    assert hist[-1] > 0.1175


def test_optimum_uniform_quantiser_of_a_uniform_density():
    x = np.linspace(0.0, 3.0, 300001)
    lo, step, hist = oracle.lloyd_max_uniform(x, iters=300)
    assert lo == pytest.approx(0.375, abs=1e-4) and step == pytest.approx(0.75, abs=1e-4)
    assert hist[-1] == pytest.approx(0.75 ** 2 / 12, rel=1e-4)


def test_equally_spaced_levels_hand_worked():
    # groups of 4: [0, 1, 2, 3] and [-2, -1, 0.5, 4] with (lo, step) = (0.5, 2/3):
    #   group 0: r = 1, scale = fp16(2/3) = 0x3955, zero = fp16(0 + 0.5) = 0x3800;
    #            t = (x - 0.5) / 0.66650390625 = -0.75, 0.75, 2.25, 3.75 -> codes 0, 1, 2, 3
    #   group 1: r = 2, scale = fp16(4/3) = 0x3D55, zero = fp16(-2 + 1) = 0xBC00;
    #            t = -0.75, 0, 1.125, 3.75 -> codes 0, 0, 1, 3
    x = np.array([[0, 1, 2, 3, -2, -1, 0.5, 4]], np.float32)
    codes, s, z, _ = oracle.quantize(x, np.inf, 4, (0.5, np.float32(2 / 3)))
    assert codes.tolist() == [[0, 1, 2, 3, 0, 0, 1, 3]]
    assert s.view(np.uint16).tolist() == [[0x3955, 0x3D55]]
    assert z.view(np.uint16).tolist() == [[0x3800, 0xBC00]]


@pytest.mark.parametrize("group", [64, 128])
def test_plain_levels_are_the_int2_grid(group):
    r = np.random.default_rng(7)
    xr = (r.standard_normal((40, 128)) * 2).astype(np.float32)
    a = oracle.quantize(xr, 3.0, group)
    b = oracle.quantize(xr, 3.0, group, (0.0, 1.0))
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_equally_spaced_levels_are_a_codebook_on_the_same_coordinate():
    # with (lo, step) the stored values are zero' + scale' * c; away from rounding boundaries the
    # codes are those of the R19 codebook quantiser with levels lo + step * c
    r = np.random.default_rng(8)
    xr = r.standard_normal((64, 128)).astype(np.float32)
    lo, step = 0.55, 0.63
    codes, s, z, pre = oracle.quantize(xr, np.inf, 64, (lo, np.float32(step)))
    cb, _, _ = oracle.quantize_codebook(xr, np.inf, 64, lo + step * np.arange(4))
    far = np.abs(pre["t"] - np.floor(pre["t"]) - 0.5) > 1e-2
    assert np.array_equal(codes[far], cb[far])
    assert (codes != cb).mean() < 1e-2


# ---- the codebook symmetric about 1.5 that the GPU attention runs (reading R21)

def test_symmetric_fit_of_a_centred_gaussian_matches_max_1960():
    # t ~ N(1.5, 0.5^2): the 4-level Lloyd-Max quantiser of a Gaussian is symmetric, so the
    # restricted fit reaches Max's levels 1.5 +- 0.5 {0.4528, 1.510} and error 0.25 * 0.1175
    x = np.linspace(1.5 - 4.0, 1.5 + 4.0, 400001)
    wgt = np.exp(-(x - 1.5) ** 2 / (2 * 0.25))
    lv, thr, hist = oracle.lloyd_max_symmetric(x, wgt, l0=0.0, l1=1.0, iters=300)
    assert np.allclose(lv, 1.5 + 0.5 * np.array([-1.510, -0.4528, 0.4528, 1.510]), atol=4e-4)
    assert np.allclose(thr, 1.5 + 0.5 * np.array([-0.9816, 0.0, 0.9816]), atol=2e-4)
    assert hist[-1] == pytest.approx(0.25 * 0.1175, abs=1e-4)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))


def test_symmetric_fit_of_a_uniform_density():
    x = np.linspace(0.0, 3.0, 300001)
    lv, thr, hist = oracle.lloyd_max_symmetric(x, iters=300)
    assert np.allclose(lv, [0.375, 1.125, 1.875, 2.625], atol=1e-4)
    assert hist[-1] == pytest.approx(0.75 ** 2 / 12, rel=1e-4)


def test_symmetric_fit_agrees_with_the_free_fit_on_mirrored_data():
    # on a sample closed under t -> 3 - t the free Lloyd iteration started from a symmetric
    # codebook stays symmetric, so both algorithms walk the same levels
    # (no sample sits on the middle threshold 1.5, where a tie takes the lower code and would
    # break the mirror symmetry of the free iteration)
    r = np.random.default_rng(11)
    half = r.gamma(2.0, 0.4, 5000)
    half = half[half < 1.45]
    t = np.concatenate([half, 3.0 - half])
    lv_f, _, hist_f = oracle.lloyd_max(t, levels=(0.1, 1.0, 2.0, 2.9), iters=60)
    lv_s, _, hist_s = oracle.lloyd_max_symmetric(t, l0=0.1, l1=1.0, iters=60)
    assert np.allclose(lv_f, lv_s, rtol=0, atol=1e-12)
    assert np.allclose(hist_f, hist_s, rtol=1e-12, atol=0)


def test_symmetric_fit_brute_force_on_a_small_mirrored_set():
    # six points and their mirrors: every symmetric split into four contiguous cells, scored by
    # the symmetric least-squares levels, has its optimum as a fixed point of the iteration
    r = np.sort(np.random.default_rng(12).uniform(0, 1.5, 6))
    t = np.sort(np.concatenate([r, 3.0 - r]))
    best = None
    for a in range(1, 6):   # cell 0 = first a points (mirror: cell 3), cell 1 = the rest below 1.5
        c0, c1 = r[:a], r[a:]
        l0, l1 = c0.mean(), c1.mean()
        cost = 2 * (((c0 - l0) ** 2).sum() + ((c1 - l1) ** 2).sum()) / 12
        if best is None or cost < best[0]:
            best = (cost, l0, l1)
    lv, _, hist = oracle.lloyd_max_symmetric(t, l0=best[1], l1=best[2], iters=5)
    assert np.allclose(lv, oracle.symmetric_levels(best[1], best[2]), rtol=0, atol=1e-15)
    assert hist[-1] == pytest.approx(best[0], rel=1e-12)


def test_symmetric_levels_write_the_codebook_as_bit_planes():
    # (l0, l1, 3 - l1, 3 - l0) = a + b c + d b1 with a = l0, b = l1 - l0, d = 3 + l0 - 3 l1 and
    # b1 = c >> 1: the form in which the attention kernel applies the codebook
    l0, l1 = 0.37, 1.21
    lv = oracle.symmetric_levels(l0, l1)
    c = np.arange(4)
    a, b, d = l0, l1 - l0, 3 + l0 - 3 * l1
    assert np.allclose(lv, a + b * c + d * (c >> 1), rtol=0, atol=1e-15)


def test_grid_codebook_through_demote_and_attention_is_the_plain_path():
    # the codebook (0, 1, 2, 3) is the uniform grid: demotion writes the same bytes and attention
    # returns the same outputs as without a codebook (away from halfway points, where the grid
    # rounds to even and the codebook takes the lower code)
    g = oracle.Geometry(group=64)
    rng = np.random.default_rng(5)
    hkv, n = 2, 150
    u = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(hkv)])
    k = rng.standard_normal((1, n, hkv, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, hkv, 128)).astype(np.float32)
    table = np.array([[2, 0, 1]], np.int32)
    clip = np.full(hkv, 3.5)
    grid = np.tile(np.arange(4.0), (hkv, 1))
    p0, p1 = oracle.new_pool(3, hkv, g), oracle.new_pool(3, hkv, g)
    oracle.demote(p0, table, u, u, clip, clip, k, v, [0], g)
    oracle.demote(p1, table, u, u, clip, clip, k, v, [0], g, codebook_k=grid, codebook_v=grid)
    assert np.array_equal(p0, p1)
    L = n + 320
    sink = rng.standard_normal((1, hkv, 64, 128)).astype(np.float32)
    rec = rng.standard_normal((1, hkv, 256, 128)).astype(np.float32)
    q = rng.standard_normal((1, 4, 128))
    a = oracle.decode_attention(p0, table, sink, sink, rec, rec, [0], [L], q, u, u, g)
    b = oracle.decode_attention(p0, table, sink, sink, rec, rec, [0], [L], q, u, u, g,
                                codebook_k=grid, codebook_v=grid)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)
