"""Pins of the oracle's paged pool layout and of the decode-step write order.

The pages require a paged KV pool ("超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
section OSCAR 的设计: compatible with paged KV and a radix prefix cache) and say that a new token
first enters the recent window and that the oldest recent token is then demoted; the byte layout
inside a page is this library's own (documented in include/oscar.h) and is pinned here by a
hand-worked example."""
import numpy as np

import oracle


def test_hand_worked_block_layout():
    g = oracle.Geometry(head_dim=8, group=4, page=4, sink=2, recent=3)
    assert (g.k_codes_off, g.v_codes_off, g.meta_off, g.block_bytes) == (0, 8, 16, 80)
    assert not g.tiled
    pool = oracle.new_pool(2, 1, g)
    table = np.array([1, 0], np.int32)             # logical page 1 -> physical page 0
    kc = np.array([[1, 2, 3, 0, 0, 0, 0, 1]], np.uint8)
    vc = np.array([[3, 0, 1, 2, 0, 0, 0, 0]], np.uint8)
    ks = np.array([[1.0, 0.5]], np.float16)
    kz = np.array([[-1.0, 2.0]], np.float16)
    vs = np.array([[0.25, 0.0]], np.float16)
    vz = np.array([[0.0, -2.0]], np.float16)
    oracle.store_history(pool, table, [6], 0, (kc, ks, kz), (vc, vs, vz), g)
    blk = pool[0, 0]
    assert not pool[1].any()
    # history index 6 -> logical page 1 (physical 0), slot 2
    assert blk[4:6].tolist() == [0x39, 0x40]                      # key codes, 2 bytes per token
    assert blk[8:16].tolist() == [0x30, 0, 0x10, 0x20, 0, 0, 0, 0]  # value codes, shift 4 = slot 2
    # meta of slot 2 at 16 + 2 * 16: key (scale, zero) per group, then value
    assert blk[48:56].tolist() == [0x00, 0x3C, 0x00, 0xBC, 0x00, 0x38, 0x00, 0x40]
    assert blk[56:64].tolist() == [0x00, 0x34, 0x00, 0x00, 0x00, 0x00, 0x00, 0xC0]
    touched = np.zeros(80, bool)
    touched[[4, 5, 8, 10, 11]] = True
    touched[48:64] = True
    assert not blk[~touched].any()


def test_hand_worked_tiled_order():
    # Full geometry: words of 16 codes in the tiled order.  Key code 2 at token 37, channel 103:
    # 37 = 16*2 + 5 (st 2, n 5); 103 = 16*6 + 4*1 + 3 (word 6 = 4*1 + 2, byte 1, bits 6..7)
    # -> chunk row 1, lane 16*2 + 5 = 37, entry 2*0 + 1 = 1: word 4*(64 + 37) + 1 = 405,
    # byte 4*405 + 1 = 1621, value 2 << 6.
    # Value code 3 at token 50, channel 77: 50 = 16*3 + 4*0 + 2 (tile s 3, group u 0, j 2) sits
    # at code position 8*1 + 2*3 + 0 = 14 of word (77, u 0), i.e. byte 3, bits 4..5;
    # 77 = 16*4 + 13 (nt 4, n 13) -> chunk row 1, lane 16*0 + 13 = 13, entry 0: word
    # 4*(64 + 13) = 308, byte 2048 + 4*308 + 3 = 3283, value 3 << 4.
    g = oracle.Geometry()
    assert g.tiled and (g.v_codes_off, g.meta_off, g.block_bytes) == (2048, 4096, 4608)
    assert oracle.k_word_index(37, 6) == 405 and oracle.v_word_index(77, 3) == 500
    pool = oracle.new_pool(1, 1, g)
    kc = np.zeros((2, 128), np.uint8)
    vc = np.zeros((2, 128), np.uint8)
    kc[0, 103] = 2
    vc[1, 77] = 3
    one = np.ones((2, 1), np.float16)
    zero = np.zeros((2, 1), np.float16)
    oracle.store_history(pool, np.array([0], np.int32), [37, 50], 0, (kc, zero, zero),
                         (vc, zero, zero), g)
    blk = pool[0, 0]
    nz = np.nonzero(blk)[0].tolist()
    assert oracle.v_word_index(77, 0) == 308 and oracle.v_code_pos(50) == (0, 14)
    assert nz == [1621, 3283]
    assert blk[1621] == 2 << 6 and blk[3283] == 3 << 4
    # the word orders are permutations of all 512 words of each region
    t, w = np.meshgrid(np.arange(64), np.arange(8), indexing="ij")
    assert sorted(oracle.k_word_index(t, w).ravel().tolist()) == list(range(512))
    c, u = np.meshgrid(np.arange(128), np.arange(4), indexing="ij")
    assert sorted(oracle.v_word_index(c, u).ravel().tolist()) == list(range(512))
    # the value-code positions of a page's 64 tokens fill the 16 positions of each of 4 words
    assert sorted(oracle.v_code_pos(t) for t in range(64)) == [(u, p) for u in range(4)
                                                                for p in range(16)]
    # meta of token 50: key pair at 4096 + 50 * 8, value pair right after
    oracle.store_history(pool, np.array([0], np.int32), [50], 0, (kc[:1], one[:1], zero[:1]),
                         (vc[:1], zero[:1], one[:1]), g)
    assert blk[4096 + 400: 4096 + 408].tolist() == [0x00, 0x3C, 0, 0, 0, 0, 0x00, 0x3C]


def test_store_load_roundtrip_random():
    rng = np.random.default_rng(2)
    for group in (128, 64):
        g = oracle.Geometry(group=group)
        table = rng.permutation(6).astype(np.int32)
        pool = oracle.new_pool(6, 2, g)
        n = 6 * 64 - 5
        kc = rng.integers(0, 4, (n, 128), dtype=np.uint8)
        vc = rng.integers(0, 4, (n, 128), dtype=np.uint8)
        m = [rng.standard_normal((n, 128 // group)).astype(np.float16) for _ in range(4)]
        order = rng.permutation(n)                 # any store order gives the same bytes
        oracle.store_history(pool, table, order, 1, (kc[order], m[0][order], m[1][order]),
                             (vc[order], m[2][order], m[3][order]), g)
        (kc2, ks2, kz2), (vc2, vs2, vz2) = oracle.load_history(pool, table, n, 1, g)
        assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)
        for a, b in zip((ks2, kz2, vs2, vz2), m):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
        assert not pool[:, 0].any()


def test_segment_lengths_closed_form():
    g = oracle.Geometry()
    assert oracle.segment_lengths(1, g) == (1, 0, 0)
    assert oracle.segment_lengths(64, g) == (64, 0, 0)
    assert oracle.segment_lengths(65, g) == (64, 0, 1)
    assert oracle.segment_lengths(320, g) == (64, 0, 256)
    assert oracle.segment_lengths(321, g) == (64, 1, 256)
    assert oracle.segment_lengths(1024, g) == (64, 704, 256)
    assert oracle.segment_lengths(100000, g) == (64, 99680, 256)


def test_recent_slots_ring():
    g = oracle.Geometry()
    s = oracle.recent_slots(300, g)
    assert s.tolist() == list(range(64, 256)) + list(range(0, 44))
    s = oracle.recent_slots(1000, g)                # positions 744..999
    assert sorted(s.tolist()) == list(range(256))
    assert s[0] == 744 % 256


def test_append_demotes_the_overwritten_token():
    g = oracle.Geometry(head_dim=8, group=8, page=4, sink=2, recent=3)
    rng = np.random.default_rng(5)
    u = np.linalg.qr(rng.standard_normal((8, 8)))[0].astype(np.float32)[None]
    toks_k = rng.standard_normal((12, 1, 8)).astype(np.float32)
    toks_v = rng.standard_normal((12, 1, 8)).astype(np.float32)
    pool = oracle.new_pool(3, 1, g)
    table = np.array([[2, 0, 1]], np.int32)
    sk = np.zeros((1, 1, 2, 8), np.float32)
    sv = np.zeros_like(sk)
    rk = np.zeros((1, 1, 3, 8), np.float32)
    rv = np.zeros_like(rk)
    for pos in range(12):
        oracle.append(pool, table, sk, sv, rk, rv, u, u, [9.0], [9.0], toks_k[pos][None],
                      toks_v[pos][None], [0], [pos], g)
    assert np.array_equal(sk[0, 0], toks_k[:2, 0])
    assert np.array_equal(rk[0, 0, [9 % 3, 10 % 3, 11 % 3]], toks_k[9:12, 0])
    # positions 2..8 are history 0..6, each encoded exactly like a direct encode
    (kc, ks, kz), _ = oracle.load_history(pool, table[0], 7, 0, g)
    ekc, eks, ekz, _ = oracle.encode(toks_k[2:9, 0], u[0], 9.0, 8)
    assert np.array_equal(kc, ekc) and np.array_equal(ks, eks) and np.array_equal(kz, ekz)
