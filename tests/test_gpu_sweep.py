"""Seeded sweep over shapes, GPU against the CPU oracle through the C ABI.

Each draw picks a batch (1-4), a GQA width (1, 2, 4, 8), a group size (64, 128), the number of
KV heads (1-2) and per-sequence lengths clustered around the places where the work changes shape
(the sink and recent boundaries at 64 and 320, page boundaries, 16-slot word boundaries); the
INT2 path (the GPU reads the oracle's pool bytes; attention within 2e-3 max row error, LSE within
1e-3) and the BF16 baseline (GPU store and attention) are both checked on the same draws.  Odd
draws also give every KV head an equally spaced codebook (lo, step) and check the GPU's own
demotion against the oracle's pool bytes."""
import numpy as np
import pytest
import torch

import workloads
from oscar_cases import ATTN_TOL, Case, attention_error, compare_pool_blocks
from bf16_cases import Bf16Case, check_bf16

pytestmark = pytest.mark.gpu

ANCHORS = [1, 63, 64, 65, 319, 320, 321, 335, 336, 383, 384, 385, 1024, 1345]


def _draw(seed):
    rng = np.random.default_rng(seed)
    gqa = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 3))
    group = int(rng.choice([64, 128]))
    batch = int(rng.integers(1, 5))
    lengths = []
    for _ in range(batch):
        base = int(rng.choice(ANCHORS))
        lengths.append(max(1, base + int(rng.integers(-2, 3)) + 64 * int(rng.integers(0, 20))))
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=gqa * hkv,
                          num_kv_heads=hkv, group_size=group, seed=100 + seed)
    levels = None
    if seed % 2:
        levels = tuple(np.stack([rng.uniform(0.2, 0.8, hkv), rng.uniform(0.5, 1.0, hkv)],
                                -1).astype(np.float32) for _ in range(2))
    return wl, lengths, levels


@pytest.mark.parametrize("seed", range(16))
def test_sweep_int2_and_bf16(seed):
    wl, lengths, levels = _draw(seed)
    print(f"sweep {seed}: G={wl.gqa} Hkv={wl.num_kv_heads} g={wl.group_size} lengths={lengths} "
          f"levels={None if levels is None else [lv.tolist() for lv in levels]}", flush=True)
    case = Case(wl, lengths, levels=levels)
    pool = case.oracle_pool()
    g = case.gpu_inputs()
    if levels is not None:
        own = case.gpu_cache(g)
        torch.cuda.synchronize()
        compare_pool_blocks(own.pool.cpu().numpy(), pool, case)
    cache = case.gpu_cache(g, pool_from_oracle=pool)
    out, lse = case.gpu_attention(g, cache)
    ref, ref_lse = case.oracle_attention(pool)
    err = attention_error(out, ref)
    assert err <= ATTN_TOL, err
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3
    bcase = Bf16Case(wl, lengths)
    bcase.store_all()
    q = workloads.queries(wl, 0, device="cuda", batch=len(lengths))
    check_bf16(bcase, q)
