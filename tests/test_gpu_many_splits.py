"""The per-GPU share of a tensor-parallel layer (one or two KV heads at 100k tokens), where the
split plan meets the merge's limit.

The merge kernel loads the partials of the first 96 splits of a row up front and takes any
further splits in a second loop.  On the four-head single-group pass the plan gives a row at
most 96 splits (longer items instead); the int8 / bf16 pass (eight heads, or two groups) can
still plan more, and takes the second loop.  Every row is compared with the oracle's softmax
attention (2e-3) and its log-sum-exp (1e-3).
"""
import numpy as np
import pytest

import bit_rotated_kv_decode_amd as ok
import workloads
from oscar_cases import ATTN_TOL, Case, attention_error

pytestmark = pytest.mark.gpu


CASES = {   # (workload changes, lengths, whether the plan passes the merge's 96 splits)
    "hkv2_gqa4_100k": dict(wl=dict(num_q_heads=8, num_kv_heads=2), lengths=[100000], more=False),
    "hkv1_gqa4_100k": dict(wl=dict(num_q_heads=4, num_kv_heads=1), lengths=[100000], more=False),
    "hkv1_gqa8_g64_100k": dict(wl=dict(num_q_heads=8, num_kv_heads=1, group_size=64),
                               lengths=[100000], more=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_attention_beyond_merge_prefetch(name):
    spec = CASES[name]
    wl = workloads.scaled(workloads.get("qwen3_8b_100k"), num_layers=1, **spec["wl"])
    lengths = spec["lengths"]
    case = Case(wl, lengths)
    splits, _ = ok.decode_splits(case.layout, len(lengths), max(lengths))
    assert (splits > 96) == spec["more"]
    print(f"many splits {name}: lengths {lengths}, {splits} splits per row", flush=True)
    pool = case.oracle_pool()
    g = case.gpu_inputs()
    cache = case.gpu_cache(g, pool_from_oracle=pool)
    out, lse = case.gpu_attention(g, cache)
    ref, ref_lse = case.oracle_attention(pool)
    err = attention_error(out, ref)
    lse_err = float(np.max(np.abs(lse - ref_lse)))
    print(f"max row error {err:.3e}, lse error {lse_err:.3e}", flush=True)
    assert err <= ATTN_TOL
    assert lse_err <= 1e-3
