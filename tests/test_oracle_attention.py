"""Pins of the oracle's decode attention: textbook softmax attention (a library routine), the
online-softmax merge of segments ("超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
section OSCAR 的设计: BF16 and INT2 parts combined by an online-softmax merge), and a tiny case
worked in explicit Python loops."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle


def _sdpa(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q)[:, :, None], t(k), t(v), scale=scale)
    return o[0, 0, 0].numpy()


def test_attend_equals_library_attention():
    rng = np.random.default_rng(0)
    for n in (1, 7, 500):
        q = rng.standard_normal(128)
        k = rng.standard_normal((n, 128)) * 2
        v = rng.standard_normal((n, 128))
        o, lse = oracle.attend(q, k, v, 1 / math.sqrt(128))
        assert np.max(np.abs(o - _sdpa(q, k, v, 1 / math.sqrt(128)))) < 1e-12
        s = k @ q / math.sqrt(128)
        assert abs(lse - np.log(np.exp(s - s.max()).sum()) - s.max()) < 1e-12


def test_merge_equals_single_softmax_any_split_and_order():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(64)
    k = rng.standard_normal((300, 64)) * 3
    v = rng.standard_normal((300, 64))
    ref, _ = oracle.attend(q, k, v, 0.125)
    for cuts in ([0, 300], [0, 1, 300], [0, 64, 65, 299, 300], [0, 100, 100, 200, 300]):
        parts = [oracle.softmax_partial(q, k[a:b], v[a:b], 0.125) for a, b in zip(cuts, cuts[1:])]
        for perm in itertools.islice(itertools.permutations(parts), 6):
            m, l, acc = oracle.merge_partials(list(perm))
            assert np.max(np.abs(acc / l - ref)) < 1e-12
    # an empty segment (m = -inf, l = 0) is neutral
    m0 = oracle.softmax_partial(q, k[:0], v[:0], 0.125)
    assert m0[0] == -np.inf and m0[1] == 0.0
    m, l, acc = oracle.merge_partials([m0, oracle.softmax_partial(q, k, v, 0.125)])
    assert np.max(np.abs(acc / l - ref)) < 1e-12


def _tiny_state(seed, length, hq=2):
    g = oracle.Geometry(head_dim=8, group=4, page=4, sink=2, recent=3)
    rng = np.random.default_rng(seed)
    uk = np.linalg.qr(rng.standard_normal((8, 8)))[0].astype(np.float32)[None]
    uv = np.linalg.qr(rng.standard_normal((8, 8)))[0].astype(np.float32)[None]
    ck, cv = 1.5, 1.2
    xk = rng.standard_normal((length, 8)).astype(np.float32)
    xv = rng.standard_normal((length, 8)).astype(np.float32)
    npages = 3
    table = np.array([[2, 0, 1]], np.int32)
    pool = oracle.new_pool(npages, 1, g)
    sk = np.zeros((1, 1, 2, 8), np.float32)
    sv = np.zeros_like(sk)
    rk = np.zeros((1, 1, 3, 8), np.float32)
    rv = np.zeros_like(rk)
    for pos in range(length):
        oracle.append(pool, table, sk, sv, rk, rv, uk, uv, [ck], [cv], xk[pos][None, None],
                      xv[pos][None, None], [0], [pos], g)
    q = rng.standard_normal((1, hq, 8))
    return g, (pool, table, sk, sv, rk, rv, uk, uv, q), (xk, xv, ck, cv)


def _loops_reference(xk, xv, uk, uv, ck, cv, q, length):
    """Everything in explicit loops, fp64, with the quantiser written as 'nearest of four levels'."""
    d, grp, sink, recent = 8, 4, 2, 3

    def had(i, j):
        return -1.0 if bin(i & j).count("1") % 2 else 1.0

    def rev(j):
        return int("{:03b}".format(j)[::-1], 2)

    def rot(u):
        return [[sum(float(u[i][k]) * had(k, rev(j)) for k in range(d)) / math.sqrt(d)
                 for j in range(d)] for i in range(d)]

    def quant_dequant(x, r, c):
        xr = [sum(x[i] * r[i][j] for i in range(d)) for j in range(d)]
        xr = [min(max(v, -c), c) for v in xr]
        out = [0.0] * d
        for m in range(d // grp):
            grp_vals = xr[m * grp:(m + 1) * grp]
            lo, hi = min(grp_vals), max(grp_vals)
            s = float(np.float16((hi - lo) / 3))
            z = float(np.float16(lo))
            for jj in range(grp):
                x_ = grp_vals[jj]
                if s == 0:
                    code = 0
                else:
                    dists = [abs(x_ - (s * k + z)) for k in range(4)]
                    code = min(range(4), key=lambda k: (dists[k], k % 2))
                out[m * grp + jj] = s * code + z
        return [sum(out[j] * r[i][j] for j in range(d)) for i in range(d)]   # x = x' R^T

    rk, rv = rot(uk[0]), rot(uv[0])
    keys, vals = [], []
    for pos in range(length):
        in_hist = sink <= pos < length - recent
        kx = [float(a) for a in xk[pos]]
        vx = [float(a) for a in xv[pos]]
        if in_hist:
            kx = quant_dequant(kx, rk, ck)
            vx = quant_dequant(vx, rv, cv)
        keys.append(kx)
        vals.append(vx)
    outs = []
    for h in range(q.shape[1]):
        s = [sum(q[0, h, j] * kk[j] for j in range(d)) / math.sqrt(d) for kk in keys]
        mx = max(s)
        w = [math.exp(a - mx) for a in s]
        tot = sum(w)
        outs.append([sum(w[t] * vals[t][j] for t in range(length)) / tot for j in range(d)])
    return np.array(outs)


@pytest.mark.parametrize("length", [1, 2, 4, 5, 6, 9, 12])
def test_tiny_brute_force(length):
    g, (pool, table, sk, sv, rk, rv, uk, uv, q), (xk, xv, ck, cv) = _tiny_state(7, length)
    out, _ = oracle.decode_attention(pool, table, sk, sv, rk, rv, [0], [length], q, uk, uv, g)
    ref = _loops_reference(xk, xv, uk, uv, ck, cv, q, length)
    assert np.max(np.abs(out[0] - ref)) < 1e-9


def test_rotation_only_equals_textbook():
    # Quantisation off: store the exact rotated history and un-rotate it; the cache must give the
    # same attention as the raw keys and values (this fixes R versus R^T).
    rng = np.random.default_rng(3)
    u64 = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    k = rng.standard_normal((200, 128))
    v = rng.standard_normal((200, 128))
    q = rng.standard_normal(128)
    kr = oracle.unrotate(oracle.rotate(k, u64), u64)
    vr = oracle.unrotate(oracle.rotate(v, u64), u64)
    o1, _ = oracle.attend(q, kr, vr, 1 / math.sqrt(128))
    assert np.max(np.abs(o1 - _sdpa(q, k, v, 1 / math.sqrt(128)))) < 1e-12
    # and in the rotated frame: (q R) . k' = q . k
    qr = oracle.rotate(q, u64)
    assert np.max(np.abs(oracle.rotate(k, u64) @ qr - k @ q)) < 1e-10


def test_gqa_head_mapping():
    # query heads 0..G-1 read KV head 0, G..2G-1 read KV head 1
    g = oracle.Geometry(head_dim=8, group=8, page=4, sink=2, recent=3)
    rng = np.random.default_rng(11)
    sk = rng.standard_normal((1, 2, 2, 8)).astype(np.float32)
    sv = rng.standard_normal((1, 2, 2, 8)).astype(np.float32)
    rk = np.zeros((1, 2, 3, 8), np.float32)
    rv = np.zeros_like(rk)
    u = np.stack([np.eye(8, dtype=np.float32)] * 2)
    q = rng.standard_normal((1, 4, 8))
    out, _ = oracle.decode_attention(oracle.new_pool(1, 2, g), np.zeros((1, 1), np.int32), sk, sv,
                                     rk, rv, [0], [2], q, u, u, g)
    for h in range(4):
        kv = h // 2
        ref, _ = oracle.attend(q[0, h], sk[0, kv], sv[0, kv], 1 / math.sqrt(8))
        assert np.max(np.abs(out[0, h] - ref)) < 1e-12
