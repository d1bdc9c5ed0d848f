"""Pins of the oracle's clip / asymmetric INT2 group quantisation and of the 2-bit packing
("超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化", section OSCAR 的设计: clip, scale /
zero-point quantisation, four 2-bit codes per byte)."""
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_cases.txt")


def _golden_cases():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        clip, vals, codes, s, z = [c.strip() for c in line.split("|")]
        rows.append((float(clip), [float(v) for v in vals.split(",")],
                     [int(c) for c in codes.split(",")], float(s), float(z)))
    return rows


@pytest.mark.parametrize("case", _golden_cases())
def test_hand_worked_groups(case):
    clip, vals, codes, s, z = case
    c, sc, zc, _ = oracle.quantize(np.array([vals], np.float32), clip, 4)
    assert c[0].tolist() == codes
    assert float(sc[0, 0]) == s and float(zc[0, 0]) == z


def test_fp16_rounding_of_scale():
    # range 1 -> (1/3) in fp32 is 0.3333333432674408; the nearest fp16 is 0x3555 = 0.333251953125
    _, sc, zc, _ = oracle.quantize(np.array([[0.0, 0.2, 0.7, 1.0]], np.float32), 100.0, 4)
    assert sc.view(np.uint16)[0, 0] == 0x3555
    assert float(zc[0, 0]) == 0.0


def _random_rotated(n=400, seed=0, scale=2.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)) * scale
    x[:, 5] *= 8
    return x.astype(np.float32)


@pytest.mark.parametrize("group", [128, 64])
def test_codes_are_nearest_level_brute_force(group):
    # Independent check in fp64: each code must be the nearest of the four levels s*k + z
    # (ties to the even code), except where the fp64 distances of the two best levels differ by
    # less than 1e-5 of the scale (there the fp32 decision may legitimately go either way).
    xr = _random_rotated()
    clip = 4.0
    codes, s16, z16, _ = oracle.quantize(xr, clip, group)
    xc = np.clip(xr.astype(np.float64), -clip, clip)
    ng = 128 // group
    s = np.repeat(s16.astype(np.float64), group, axis=1)
    z = np.repeat(z16.astype(np.float64), group, axis=1)
    levels = s[..., None] * np.arange(4)[None, None, :] + z[..., None]
    dist = np.abs(xc[..., None] - levels)
    # ties: prefer the even code -> add a tiny bias to odd codes
    best = np.argmin(dist + np.array([0, 1e-300, 0, 1e-300]), axis=-1)
    srt = np.sort(dist, axis=-1)
    ambiguous = (srt[..., 1] - srt[..., 0]) <= 1e-5 * np.maximum(s, 1e-30)
    ok = (best == codes) | ambiguous | (s == 0)
    assert ok.all()
    assert ambiguous.mean() < 1e-3
    assert set(np.unique(codes)) <= {0, 1, 2, 3}
    assert ng * group == 128


@pytest.mark.parametrize("group", [128, 64, 32])
def test_reconstruction_error_bound(group):
    xr = _random_rotated(seed=3)
    clip = 4.0
    codes, s16, z16, pre = oracle.quantize(xr, clip, group)
    xc = np.clip(xr.astype(np.float64), -clip, clip)
    rec = oracle.dequantize(codes, s16, z16, group)
    s = np.repeat(s16.astype(np.float64), group, axis=1)
    z = np.repeat(z16.astype(np.float64), group, axis=1)
    mn = np.repeat(pre["z"].astype(np.float64), group, axis=1)
    s_exact = np.repeat(pre["s"].astype(np.float64), group, axis=1)
    bound = 0.5 * s + np.abs(z - mn) + 3 * np.abs(s - s_exact) + 1e-6
    assert (np.abs(rec - xc) <= bound).all()


def test_group_extremes_map_to_end_codes():
    xr = _random_rotated(seed=4)
    codes, _, _, _ = oracle.quantize(xr, 100.0, 64)
    g = xr.reshape(-1, 2, 64)
    c = codes.reshape(-1, 2, 64)
    lo = np.take_along_axis(c, g.argmin(-1)[..., None], -1)
    hi = np.take_along_axis(c, g.argmax(-1)[..., None], -1)
    assert (lo == 0).all() and (hi == 3).all()


def test_constant_group_is_degenerate():
    xr = np.full((1, 128), 0.37, np.float32)
    codes, s16, z16, _ = oracle.quantize(xr, 4.0, 128)
    assert float(s16[0, 0]) == 0.0 and (codes == 0).all()
    assert float(z16[0, 0]) == float(np.float16(0.37))


def test_clip_is_symmetric_and_applied_after_rotation():
    xr = np.array([[-9.0, -1.0, 0.5, 9.0]], np.float32)
    codes, s16, z16, _ = oracle.quantize(xr, 2.0, 4)
    rec = oracle.dequantize(codes, s16, z16, 4)[0]
    assert rec[0] == -2.0 and abs(rec[3] - 2.0) < 2e-3


def test_pack_exhaustive_roundtrip():
    allbytes = np.arange(256, dtype=np.uint8)[:, None]
    codes = oracle.unpack_codes(allbytes)
    assert codes.shape == (256, 4)
    assert np.array_equal(oracle.pack_codes(codes), allbytes)
    # byte b, code i in bits [2i, 2i+1]
    for b in range(256):
        assert codes[b].tolist() == [(b >> (2 * i)) & 3 for i in range(4)]


def test_pack_known_bytes():
    assert oracle.pack_codes(np.array([1, 2, 3, 0], np.uint8)).tolist() == [0x39]
    assert oracle.pack_codes(np.array([3, 3, 3, 3, 0, 0, 0, 1], np.uint8)).tolist() == [0xFF, 0x40]


def test_pack_random_roundtrip():
    rng = np.random.default_rng(9)
    c = rng.integers(0, 4, size=(37, 128), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(c)), c)


def test_encode_on_workload_tokens():
    wl = workloads.get("tiny_gqa4_1k")
    k, _ = workloads.kv_tokens(wl, 0, 0, 64, 32)
    uk, _ = workloads.rotation_bases(wl, 0)
    codes, s16, z16, pre = oracle.encode(k[:, 0].float().numpy(), uk[0].numpy(), 4.0, 128)
    assert codes.shape == (32, 128) and s16.shape == (32, 1)
    # the clip at 4 bounds the group range, so the scale is at most 8/3 (up to fp16 rounding)
    assert (s16.astype(np.float64) <= 8 / 3 * (1 + 2 ** -10)).all()
