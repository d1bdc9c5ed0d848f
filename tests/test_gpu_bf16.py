"""GPU parity of the paged BF16 baseline (oscar_bf16_store, oscar_bf16_decode_attn) against the
CPU oracle, called through the C ABI.

Pool bytes after the GPU store are compared bit-exactly with the oracle's layout; attention must
match the oracle's fp64 softmax attention over the same bf16 keys and values within 2e-3 max row
error (the bound used for the INT2 path).  Pools start filled with NaN bit patterns, so a kernel
that let a slot past a sequence's length (or an unwritten page) reach a result would fail."""

import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import workloads
from bf16_cases import Bf16Case, check_bf16 as _check

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2)])
def test_bf16_store_and_attention_ragged(hq, hkv):
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=hq, num_kv_heads=hkv)
    lengths = [1, 63, 64, 65, 700, 3001]
    _note(f"bf16 ragged hq={hq} hkv={hkv} lengths={lengths}")
    case = Bf16Case(wl, lengths)
    case.store_all()
    torch.cuda.synchronize()
    got = case.pool.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got.reshape(case.num_pages, hkv, -1), case.oracle_pool())
    q = workloads.queries(wl, 0, device="cuda", batch=len(lengths))
    _check(case, q)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 2)])
def test_bf16_single_sequence_every_gqa(hq, hkv):
    # one sequence per launch selects the non-temporal page loads
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=hq, num_kv_heads=hkv)
    case = Bf16Case(wl, [2345])
    case.store_all()
    q = workloads.queries(wl, 0, device="cuda", batch=1)
    _check(case, q)


def test_bf16_page_table_shuffle_gives_identical_output():
    wl = workloads.get("tiny_gqa4_1k")
    lengths = [2000, 777]
    case = Bf16Case(wl, lengths)
    case.store_all()
    q = workloads.queries(wl, 0, device="cuda", batch=2)
    out1 = _check(case, q)
    # the same tokens through another shuffle of physical pages
    case2 = Bf16Case(wl, lengths, layer=1)
    case2.kv = case.kv
    assert not np.array_equal(case2.table, case.table)
    case2.store_all()
    out2 = torch.empty_like(out1)
    case2.attend(q, out2, None)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_bf16_decode_step_appends_then_attends():
    wl = workloads.get("tiny_gqa4_1k")
    lengths = [191, 64]
    case = Bf16Case(wl, lengths, spare=8)
    # store all but the last 3 tokens, then append them one decode step at a time
    full = case.kv
    case.kv = [(k[:L - 3], v[:L - 3]) for (k, v), L in zip(full, lengths)]
    case.store_all()
    for step in range(3):
        pos = [L - 3 + step for L in lengths]
        k_new = torch.stack([k[p] for (k, _), p in zip(full, pos)]).unsqueeze(1)
        v_new = torch.stack([v[p] for (_, v), p in zip(full, pos)]).unsqueeze(1)
        ok.bf16_store(case.lay, case.pool, case.table_dev, k_new, v_new,
                      torch.tensor(pos, dtype=torch.int32, device="cuda"))
        q = workloads.queries(wl, 0, step=step, device="cuda", batch=2)
        _check(case, q, lengths=[p + 1 for p in pos], kv=full)


def test_bf16_full_size_qwen3_8b_100k():
    # the benchmark's layer shape: batch 1, 32 query / 8 KV heads, 100,000 tokens, one plan
    wl = workloads.get("qwen3_8b_100k")
    case = Bf16Case(wl, [100000])
    _note(f"bf16 full size: pages={case.num_pages}")
    case.store_all()
    torch.cuda.synchronize()
    # sampled pages bit-exact: the first, a middle one and the partly filled last one
    row = case.table[0]
    sample = {int(row[0]), int(row[700]), int(row[1562])}
    got = case.pool.view(torch.int16).cpu().numpy().view(np.uint16).reshape(case.num_pages, 8, -1)
    ref = case.oracle_pool(pages=sample)
    for pg in sample:
        assert np.array_equal(got[pg], ref[pg]), pg
    q = workloads.queries(wl, 0, device="cuda")
    _check(case, q, rows=[(0, h) for h in range(0, 32, 3)])


def test_bf16_shared_prefix_batch():
    # sequences share their first 32,768 tokens through the page table (prefix-cache hit)
    wl = workloads.scaled(workloads.get("qwen3_8b_b64_prefix"), batch=3, ragged=(33000, 40000))
    lengths = workloads.context_lengths(wl)
    case = Bf16Case(wl, lengths)
    assert np.array_equal(case.table[0, :512], case.table[1, :512])
    case.store_all()
    q = workloads.queries(wl, 0, device="cuda")
    _check(case, q, rows=[(b, h) for b in range(3) for h in (0, 13, 31)])


def test_bf16_full_size_qwen3_32b_131k_gqa8():
    # batch 16 at 131,072 tokens, 64 query / 8 KV heads (G = 8): the shape bench.py times for
    # this workload's BF16 baseline; sampled rows of the first and last sequence
    wl = workloads.get("qwen3_32b_131k")
    case = Bf16Case(wl, workloads.context_lengths(wl))
    _note(f"bf16 full size 32b: pages={case.num_pages}")
    case.store_all()
    q = workloads.queries(wl, 0, device="cuda")
    _check(case, q, rows=[(b, h) for b in (0, 15) for h in (0, 33, 63)])


def test_bf16_full_size_qwen3_8b_b64_shared_prefix():
    # batch 64, ragged 8k..128k, 32k shared prefix: the batched workload's BF16 baseline shape
    wl = workloads.get("qwen3_8b_b64_prefix")
    lengths = workloads.context_lengths(wl)
    case = Bf16Case(wl, lengths)
    _note(f"bf16 full size b64: pages={case.num_pages}, lengths {min(lengths)}..{max(lengths)}")
    case.store_all()
    q = workloads.queries(wl, 0, device="cuda")
    longest, shortest = int(np.argmax(lengths)), int(np.argmin(lengths))
    _check(case, q, rows=[(b, h) for b in (longest, shortest, 7) for h in (2, 29)])
