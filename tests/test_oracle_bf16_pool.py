"""Pins of the oracle's paged BF16 baseline layout (CPU only).

The pages measure the INT2 history against a history kept in BF16 (the OSCAR write-up's
evaluation part; the paper page's Abstract).  The BF16 page layout is this project's own, so it is
pinned by hand-worked element positions, round trips and the bf16 bit conversion; the attention
over the gathered cache is the oracle's ``attend``, pinned elsewhere against textbook softmax
attention."""
import math

import numpy as np
import torch

import oracle


def test_hand_worked_positions():
    # token 70 of a sequence whose page table row is [5, 2]: page 2, slot 6.  Key channel 3 sits
    # at element 6 * 128 + 3 = 771 of the block; value channel 3 at 64 * 128 + 3 * 64 + 6 = 8390.
    pool = oracle.bf16_new_pool(6, 2)
    k = np.zeros(128, np.uint16)
    v = np.zeros(128, np.uint16)
    k[3] = 0x1234
    v[3] = 0xABCD
    oracle.bf16_store(pool, [5, 2], 70, 1, k, v)
    assert pool[2, 1, 771] == 0x1234
    assert pool[2, 1, 8390] == 0xABCD
    assert np.count_nonzero(pool) == 2
    # token 0 of the same row: page 5, slot 0 -> key element c, value element 8192 + 64 c
    k[:] = np.arange(128)
    v[:] = np.arange(128) + 1000
    oracle.bf16_store(pool, [5, 2], 0, 0, k, v)
    assert np.array_equal(pool[5, 0, :128], np.arange(128))
    assert np.array_equal(pool[5, 0, 8192 + 64 * np.arange(128)], np.arange(128) + 1000)


def test_store_gather_round_trip_on_shuffled_pages():
    rng = np.random.default_rng(7)
    length, hkv = 3 * 64 + 17, 2
    row = rng.permutation(8)[:4]
    pool = oracle.bf16_new_pool(8, hkv, fill=0x7FC0)
    keys = rng.integers(0, 1 << 16, size=(length, hkv, 128), dtype=np.uint16)
    values = rng.integers(0, 1 << 16, size=(length, hkv, 128), dtype=np.uint16)
    for t in range(length):
        for h in range(hkv):
            oracle.bf16_store(pool, row, t, h, keys[t, h], values[t, h])
    for h in range(hkv):
        k, v = oracle.bf16_gather(pool, row, length, h)
        assert np.array_equal(k, keys[:, h]) and np.array_equal(v, values[:, h])
    # slots past the length and pages not in the row keep the fill
    blk = pool[row[3], 0]
    slot = length % 64
    assert np.all(blk[slot * 128:64 * 128] == 0x7FC0)
    for pg in set(range(8)) - set(row.tolist()):
        assert np.all(pool[pg] == 0x7FC0)
    # every element of a stored token is written exactly once: the pages used hold
    # length x hkv x 2 x 128 non-fill elements at most
    assert np.count_nonzero(pool != 0x7FC0) <= length * hkv * 256


def test_bf16_bits_match_torch():
    x = torch.randn(1000, dtype=torch.float32) * 100
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_float(bits), b.double().numpy())
    assert oracle.bf16_bits_to_float(np.array([0x3F80, 0xC000], np.uint16)).tolist() == [1.0, -2.0]


def test_attention_over_the_gathered_cache_is_textbook():
    rng = np.random.default_rng(3)
    length = 150
    row = [3, 0, 1]
    pool = oracle.bf16_new_pool(4, 1)
    kf = torch.randn(length, 128).to(torch.bfloat16)
    vf = torch.randn(length, 128).to(torch.bfloat16)
    kb = kf.view(torch.int16).numpy().view(np.uint16)
    vb = vf.view(torch.int16).numpy().view(np.uint16)
    for t in range(length):
        oracle.bf16_store(pool, row, t, 0, kb[t], vb[t])
    k, v = oracle.bf16_gather(pool, row, length, 0)
    q = rng.standard_normal(128)
    out, lse = oracle.attend(q, oracle.bf16_bits_to_float(k), oracle.bf16_bits_to_float(v),
                             1 / math.sqrt(128))
    s = kf.double().numpy() @ q / math.sqrt(128)
    w = np.exp(s - s.max())
    ref = (w / w.sum()) @ vf.double().numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
    assert abs(lse - (s.max() + math.log(w.sum()))) < 1e-12
