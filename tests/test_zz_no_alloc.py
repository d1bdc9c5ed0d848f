"""oscar_decode_step_noalloc (the decode step for callers that cannot allocate device memory)
against oscar_decode_step on the same inputs: outputs, log-sum-exp and every cache byte must be
identical, on two calls in a row, the second with a smaller batch and shorter contexts (the
scratch array keeps the first call's contents, which the second call must not depend on)."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import workloads
from oscar_cases import ATTN_TOL, Case, attention_error

pytestmark = pytest.mark.gpu


def _clone(cache):
    return ok.Cache(cache.layout, cache.pool.clone(), cache.sink_k.clone(), cache.sink_v.clone(),
                    cache.recent_k.clone(), cache.recent_v.clone())


def _step(case, g, cache, lengths, noalloc, mx=None):
    b = len(lengths)
    hq = case.wl.num_q_heads
    pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    slots = torch.arange(b, dtype=torch.int32, device="cuda")
    kn, vn = zip(*[workloads.kv_tokens(case.wl, 0, i, L, 1, "cuda") for i, L in enumerate(lengths)])
    kn, vn = torch.cat(kn).contiguous(), torch.cat(vn).contiguous()
    q = workloads.queries(case.wl, 0, step=7, device="cuda", batch=b).contiguous()
    out = torch.full((b, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((b, hq), float("nan"), dtype=torch.float32, device="cuda")
    mx = max(lengths) + 1 if mx is None else mx
    table = g["table"][:b].contiguous()
    args = (case.layout, cache.pool, table, cache.sink_k, cache.sink_v, cache.recent_k,
            cache.recent_v, g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], kn, vn, slots, pos, q,
            out)
    if noalloc:
        ok.decode_step_noalloc(*args, mx, lse=lse)
    else:
        ws = torch.zeros(ok.decode_workspace_bytes(case.layout, b, mx), dtype=torch.uint8,
                         device="cuda")
        ok.decode_step(*args, ws, mx, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_noalloc_step_matches_workspace_step_twice():
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=8, num_kv_heads=2)
    lengths = [3000, 1500, 321, 700]
    case = Case(wl, lengths, spare=8)
    print(f"no-alloc step: lengths {lengths}", flush=True)
    g = case.gpu_inputs()
    base = case.gpu_cache(g, pool_from_oracle=case.oracle_pool())
    for call, lens in enumerate((lengths, [2000, 900])):
        # the second call: fewer sequences, shorter contexts, and a smaller plan
        a, b = _clone(base), _clone(base)
        out_ws, lse_ws = _step(case, g, a, lens, noalloc=False)
        out_na, lse_na = _step(case, g, b, lens, noalloc=True)
        print(f"call {call}: batch {len(lens)}, max row error between the two "
              f"{attention_error(out_na, out_ws):.3e}", flush=True)
        assert np.isfinite(out_na).all() and np.isfinite(lse_na).all()
        assert np.array_equal(out_na, out_ws)
        assert np.array_equal(lse_na, lse_ws)
        for name in ("pool", "sink_k", "sink_v", "recent_k", "recent_v"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
        assert attention_error(out_na, out_ws) <= ATTN_TOL


def test_noalloc_fused_step_matches_workspace_step_twice():
    # the same with plans whose segment launch appends and rotates the query (long max_seq_len:
    # INT2 blocks of at least 32 pages, all at once); the flag words of the scratch array start
    # zero and each call leaves them zero
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=8, num_kv_heads=2)
    lengths, mx = [3000, 1500, 321, 700], 100000
    case = Case(wl, lengths, spare=mx)
    print(f"no-alloc fused step: lengths {lengths}, max_seq_len {mx}", flush=True)
    g = case.gpu_inputs()
    base = case.gpu_cache(g, pool_from_oracle=case.oracle_pool())
    for call, lens in enumerate((lengths, [2000, 900])):
        assert ok.decode_step_launches(case.layout, len(lens), mx) == 2
        a, b = _clone(base), _clone(base)
        out_ws, lse_ws = _step(case, g, a, lens, noalloc=False, mx=mx)
        out_na, lse_na = _step(case, g, b, lens, noalloc=True, mx=mx)
        print(f"call {call}: batch {len(lens)}, max row error between the two "
              f"{attention_error(out_na, out_ws):.3e}", flush=True)
        assert np.isfinite(out_na).all() and np.isfinite(lse_na).all()
        assert np.array_equal(out_na, out_ws)
        assert np.array_equal(lse_na, lse_ws)
        for name in ("pool", "sink_k", "sink_v", "recent_k", "recent_v"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
