"""GPU parity of the equally spaced codebook (reading R20: levels lo + step * c in units of the
group's (max - min) / 3 above its minimum, given per KV head for keys and values) against the CPU
oracle, called through the C ABI: bulk demotion and decode-step writes bit-exact under the
acceptance rule of oscar_cases, attention over the resulting cache within 2e-3, and the plain
grid (0, 1) identical to passing no levels."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import oracle
import workloads
from oscar_cases import ATTN_TOL, Case, attention_error, compare_pool_blocks

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _levels(hkv, seed):
    """(lo, step) per KV head for keys and values: symmetric codebooks around the group's middle
    (lo in [0.3, 0.7], step = (3 - 2 lo) / 3), on the last head an asymmetric one, and with two
    or more heads one that changes only the step (keys) or only the offset (values)."""
    rng = np.random.default_rng(seed)
    out = []
    for t in range(2):
        lo = rng.uniform(0.3, 0.7, hkv)
        lv = np.stack([lo, (3 - 2 * lo) / 3], -1).astype(np.float32)
        lv[-1] = (0.25, 0.8)
        if hkv > 1:
            lv[0] = (0.0, 0.7) if t == 0 else (0.3, 1.0)
        out.append(lv)
    return out


@pytest.mark.parametrize("group,hq,hkv", [(128, 8, 2), (64, 8, 2), (64, 4, 1)])
def test_demote_and_attend_with_levels(group, hq, hkv):
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), group_size=group, num_q_heads=hq,
                          num_kv_heads=hkv)
    lengths = [321, 1000, 385 + 64 * 5 + 3, 64]
    case = Case(wl, lengths, levels=_levels(hkv, group + hkv))
    _note(f"levels demote g={group} hq={hq} hkv={hkv} lengths={lengths} "
          f"levels_k={case.levels_k.tolist()}")
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    torch.cuda.synchronize()
    pool = case.oracle_pool()
    flips = compare_pool_blocks(cache.pool.cpu().numpy(), pool, case)
    _note(f"code flips: {flips}")
    # the codebook changes the bytes: the plain grid's pool differs
    plain = Case(wl, lengths).oracle_pool()
    assert not np.array_equal(plain, pool)
    out, lse = case.gpu_attention(g, cache)
    ref, ref_lse = case.oracle_attention(pool)
    err = attention_error(out, ref)
    _note(f"max row error {err:.3e}")
    assert err <= ATTN_TOL
    assert np.max(np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse))) <= 1e-3


def test_plain_levels_equal_no_levels():
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=8, num_kv_heads=2)
    lengths = [900, 2000]
    plain = np.tile(np.array([[0.0, 1.0]], np.float32), (2, 1))
    a = Case(wl, lengths)
    b = Case(wl, lengths, levels=(plain, plain))
    ga, gb = a.gpu_inputs(), b.gpu_inputs()
    ca, cb = a.gpu_cache(ga), b.gpu_cache(gb)
    torch.cuda.synchronize()
    assert torch.equal(ca.pool, cb.pool)


def test_append_and_decode_step_with_levels():
    # decode-step writes with codebook levels across the full-ring threshold and page
    # boundaries: append against the oracle's append, decode_step against append + decode_attn,
    # and the final attention against the oracle
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=8, num_kv_heads=2)
    start, steps = [318, 1011], 24
    lk, lv = _levels(2, 5)
    case = Case(wl, [s + steps for s in start], levels=(lk, lv))
    final = list(case.lengths)
    case.lengths = list(start)
    g = case.gpu_inputs()
    lay = case.layout
    ca, cb = case.gpu_cache(g), case.gpu_cache(g)
    sk, sv, rk, rv = case.oracle_segments()
    pool = case.oracle_pool()
    mx = max(final)
    ws_a = torch.zeros(ok.decode_workspace_bytes(lay, 2, mx), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty_like(ws_a)
    out_a = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    for s in range(steps):
        pos = [p + s for p in start]
        _note(f"levels step {s}: positions {pos}")
        k_new = torch.stack([case.k[b][pos[b]] for b in range(2)])
        v_new = torch.stack([case.v[b][pos[b]] for b in range(2)])
        pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
        ok.decode_step(lay, ca.pool, g["table"], ca.sink_k, ca.sink_v, ca.recent_k, ca.recent_v,
                       g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new.to("cuda"),
                       v_new.to("cuda"), g["slots"], pos_t, g["q"], out_a, ws_a, mx,
                       levels_k=g["levels_k"], levels_v=g["levels_v"])
        ok.append(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k, cb.recent_v,
                  g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new.to("cuda"),
                  v_new.to("cuda"), g["slots"], pos_t, levels_k=g["levels_k"],
                  levels_v=g["levels_v"])
        ok.decode_attn(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k, cb.recent_v,
                       g["slots"], pos_t + 1, g["q"], g["u_k"], g["u_v"], out_b, ws_b, mx)
        oracle.append(pool, case.table, sk, sv, rk, rv, case.u_k.numpy(), case.u_v.numpy(),
                      case.clip_k, case.clip_v, k_new.float().numpy(), v_new.float().numpy(),
                      [0, 1], pos, case.geom, lk, lv)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), s
    assert torch.equal(ca.pool, cb.pool)
    case.lengths = final
    compare_pool_blocks(ca.pool.cpu().numpy(), pool, case)
    # the pool the oracle built by appending equals the one it builds in bulk
    assert np.array_equal(pool, case.oracle_pool())
    ref, _ = case.oracle_attention(pool)
    err = attention_error(out_a.cpu().numpy(), ref)
    _note(f"levels decode_step final max row error {err:.3e}")
    assert err <= ATTN_TOL
