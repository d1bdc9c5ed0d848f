"""GPU parity of symmetric Lloyd-Max codebooks (reading R21: per KV head and tensor, levels
(l0, l1, 3 - l1, 3 - l0) in t = (x - z) / s with the plain grid's fp16 scale and zero point, the
code naming the nearest level, ties to the lower one) against the CPU oracle, called through the
C ABI: bulk demotion and decode-step writes bit-exact under the acceptance rule of oscar_cases
(rounding windows at the codebook's midpoints), attention over the resulting cache within 2e-3,
and the codebook (0, 1) giving the plain grid's attention."""
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


def _codebooks(hkv, seed):
    """(l0, l1) per KV head for keys and values: l0 in [0.15, 0.6], l1 in [1.0, 1.35] (the
    shapes a Lloyd-Max fit gives for a peaked distribution), on the last head the plain grid
    (0, 1), and with two or more heads one whose inner levels sit below the plain grid's."""
    rng = np.random.default_rng(seed)
    out = []
    for t in range(2):
        cb = np.stack([rng.uniform(0.15, 0.6, hkv), rng.uniform(1.0, 1.35, hkv)],
                      -1).astype(np.float32)
        cb[-1] = (0.0, 1.0)
        if hkv > 1:
            cb[0] = (0.35, 0.9) if t == 0 else (0.5, 1.2)
        out.append(cb)
    return out


@pytest.mark.parametrize("hq,hkv,lengths", [
    (8, 2, [321, 1000, 385 + 64 * 5 + 3, 64]),
    (4, 1, [4099]),
    (4, 4, [700, 2600]),
])
def test_demote_and_attend_with_codebook(hq, hkv, lengths):
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=hq, num_kv_heads=hkv)
    case = Case(wl, lengths, codebook=_codebooks(hkv, 11 * hq + hkv))
    _note(f"codebook demote hq={hq} hkv={hkv} lengths={lengths} cb_k={case.cb_k.tolist()} "
          f"cb_v={case.cb_v.tolist()}")
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    torch.cuda.synchronize()
    pool = case.oracle_pool()
    flips = compare_pool_blocks(cache.pool.cpu().numpy(), pool, case)
    _note(f"code flips: {flips}")
    out, lse = case.gpu_attention(g, cache)
    ref, ref_lse = case.oracle_attention(pool)
    err = attention_error(out, ref)
    _note(f"max row error {err:.3e}")
    assert err <= ATTN_TOL
    assert np.max(np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse))) <= 1e-3


def test_demote_with_codebook_group64():
    # the encoder takes a codebook at any group size; attention over it needs group 128
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), group_size=64, num_q_heads=8,
                          num_kv_heads=2)
    lengths = [1000, 400]
    case = Case(wl, lengths, codebook=_codebooks(2, 3))
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    torch.cuda.synchronize()
    flips = compare_pool_blocks(cache.pool.cpu().numpy(), case.oracle_pool(), case)
    _note(f"group-64 codebook code flips: {flips}")
    with pytest.raises(ok.OscarError):
        case.gpu_attention(g, cache)


def test_plain_codebook_matches_plain_grid():
    # levels (0, 1, 2, 3) are the plain grid: the codebook encoder writes the plain encoder's
    # bytes except on exact half-way ties (lower code against round-half-even), and the codebook
    # attention over the plain pool gives the plain attention
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=8, num_kv_heads=2)
    lengths = [900, 2000]
    plain = np.tile(np.array([[0.0, 1.0]], np.float32), (2, 1))
    a = Case(wl, lengths)
    b = Case(wl, lengths, codebook=(plain, plain))
    ga, gb = a.gpu_inputs(), b.gpu_inputs()
    ca, cb = a.gpu_cache(ga), b.gpu_cache(gb)
    torch.cuda.synchronize()
    diff = (ca.pool != cb.pool).sum().item()
    _note(f"plain codebook: {diff} differing pool bytes")
    assert diff <= 1e-5 * ca.pool.numel()
    oa, la = a.gpu_attention(ga, ca)
    ob, lb = b.gpu_attention(gb, ca)
    rel = np.max(np.abs(oa - ob)) / np.max(np.abs(oa))
    _note(f"plain codebook attention vs plain: {rel:.3e}")
    assert rel <= 1e-5
    assert np.max(np.abs(la - lb)) <= 1e-5


def test_plain_attention_refuses_codebook_layout():
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=8, num_kv_heads=2)
    case = Case(wl, [700], codebook=_codebooks(2, 1))
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    out = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(ok.decode_workspace_bytes(case.layout, 1, 700), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(ok.OscarError):
        ok.decode_attn(case.layout, cache.pool, g["table"], cache.sink_k, cache.sink_v,
                       cache.recent_k, cache.recent_v, g["slots"], g["lens"], g["q"], g["u_k"],
                       g["u_v"], out, ws, 700)


def test_append_and_decode_step_with_codebook():
    # decode-step writes under codebooks across the full-ring threshold and page boundaries:
    # append against the oracle's append, decode_step against append + decode_attn_codebook,
    # and the final attention against the oracle
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=8, num_kv_heads=2)
    start, steps = [318, 1011], 24
    ck, cv = _codebooks(2, 5)
    case = Case(wl, [s + steps for s in start], codebook=(ck, cv))
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
        _note(f"codebook step {s}: positions {pos}")
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
        ok.decode_attn_codebook(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k,
                                cb.recent_v, g["slots"], pos_t + 1, g["q"], g["u_k"], g["u_v"],
                                g["levels_k"], g["levels_v"], out_b, ws_b, mx)
        oracle.append(pool, case.table, sk, sv, rk, rv, case.u_k.numpy(), case.u_v.numpy(),
                      case.clip_k, case.clip_v, k_new.float().numpy(), v_new.float().numpy(),
                      [0, 1], pos, case.geom, codebook_k=case.codebooks("k"),
                      codebook_v=case.codebooks("v"))
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), s
    assert torch.equal(ca.pool, cb.pool)
    case.lengths = final
    compare_pool_blocks(ca.pool.cpu().numpy(), pool, case)
    # the pool the oracle built by appending equals the one it builds in bulk
    assert np.array_equal(pool, case.oracle_pool())
    ref, _ = case.oracle_attention(pool)
    err = attention_error(out_a.cpu().numpy(), ref)
    _note(f"codebook decode_step final max row error {err:.3e}")
    assert err <= ATTN_TOL
