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
    # token 70 of a sequence whose page table row is [5, 2]: page 2, slot 6.  Key channel 3:
    # row 0, chunk 6 (key octet 0, token 6 of its 16), element 3 -> 0 * 512 + 6 * 8 + 3 = 51.
    # Value channel 3: row 8 (value tile 0), chunk 3 (token octet 0, channel 3), element 6
    # -> 8 * 512 + 3 * 8 + 6 = 4126.
    pool = oracle.bf16_new_pool(6, 2)
    k = np.zeros(128, np.uint16)
    v = np.zeros(128, np.uint16)
    k[3] = 0x1234
    v[3] = 0xABCD
    oracle.bf16_store(pool, [5, 2], 70, 1, k, v)
    assert pool[2, 1, 51] == 0x1234
    assert pool[2, 1, 4126] == 0xABCD
    assert np.count_nonzero(pool) == 2
    # slot 53 (second half of the page, second 16-token tile, token 5 of it), channel 77:
    # key row 16 + 4 + 2 = 22, chunk 16 * 1 + 5 = 21, element 5 -> 11437;
    # value row 16 + 8 + 4 = 28, chunk 16 * 2 + 13 = 45, element 5 -> 14701
    assert oracle.bf16_key_index(53, 77) == 11437
    assert oracle.bf16_value_index(53, 77) == 14701
    # one lane's 16-byte chunk holds 8 consecutive key channels of one token, or one value
    # channel of 8 consecutive tokens
    assert [oracle.bf16_key_index(0, c) for c in range(10)] == [0, 1, 2, 3, 4, 5, 6, 7, 128, 129]
    assert [oracle.bf16_value_index(t, 0) for t in range(10)] == \
        [4096, 4097, 4098, 4099, 4100, 4101, 4102, 4103, 4096 + 128, 4096 + 129]


def test_block_indices_are_a_bijection():
    idx = [oracle.bf16_key_index(t, c) for t in range(64) for c in range(128)]
    idx += [oracle.bf16_value_index(t, c) for t in range(64) for c in range(128)]
    assert sorted(idx) == list(range(2 * 64 * 128))


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
    c = np.arange(128)
    for slot in range(length % 64, 64):
        assert np.all(blk[oracle.bf16_key_index(slot, c)] == 0x7FC0)
        assert np.all(blk[oracle.bf16_value_index(slot, c)] == 0x7FC0)
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
