"""oscar_decode_step where the segment launch appends the new token and rotates the query itself
(the fp8 pass -- at most four query heads per KV head, one group -- with its INT2 blocks all
running at once on at least 32 pages each: the plan of a long max_seq_len, here 100k or 200k
tokens over short sequences, whose split blocks past a sequence's pages return at once), against
the two-launch path (oscar_append, then oscar_decode_attn over the appended cache): outputs,
log-sum-exp and every cache byte equal at each step, and the final attention against the oracle.

The steps cross the sink's end (position 64), the full-ring threshold (320, where the appended
token first displaces a ring row into the history), a value-word group (16) and a history page
boundary (64); batch 1 runs the non-temporal page loads, larger batches the cached ones."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import workloads
from oscar_cases import ATTN_TOL, Case, attention_error

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _levels(hkv):
    """Equally spaced codebooks (lo, step) per KV head for keys and values, one per head."""
    lo = np.linspace(0.3, 0.6, hkv, dtype=np.float32)
    lv = np.stack([lo, (3 - 2 * lo) / 3], -1).astype(np.float32)
    return lv, lv[::-1].copy()


@pytest.mark.parametrize("hq,hkv,start,steps,mx,levels", [
    (8, 2, [315], 8, 200000, False),                  # four heads per KV head, one sequence
    (8, 2, [58, 317, 1019, 700], 9, 100000, False),   # ragged batch
    (8, 4, [60, 318, 1020], 7, 100000, False),        # two heads per KV head
    (4, 4, [62, 316], 6, 100000, False),              # one head per KV head
    (4, 4, [1021], 5, 100000, False),
    (8, 2, [317, 1020], 6, 100000, True),             # equally spaced codebook levels
    (4, 4, [1300, 2250], 4, 100000, False),           # the page read by waves 1 and 2
])
def test_fused_step_matches_two_launches(hq, hkv, start, steps, mx, levels):
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=hq, num_kv_heads=hkv)
    case = Case(wl, [s + steps for s in start], spare=mx,
                levels=_levels(hkv) if levels else None)
    final = list(case.lengths)
    case.lengths = list(start)
    g = case.gpu_inputs()
    lay = case.layout
    B = len(start)
    ca, cb = case.gpu_cache(g), case.gpu_cache(g)
    assert ok.decode_step_launches(lay, B, mx) == 2
    ws_a = torch.zeros(ok.decode_workspace_bytes(lay, B, mx), dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    out_a = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    lse_a = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    gen = torch.Generator().manual_seed(hq * 7 + hkv + B)
    for s in range(steps):
        pos = [p + s for p in start]
        _note(f"fused step hq={hq} hkv={hkv} step {s}: positions {pos}")
        k_new = torch.stack([case.k[b][pos[b]] for b in range(B)]).to("cuda")
        v_new = torch.stack([case.v[b][pos[b]] for b in range(B)]).to("cuda")
        pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
        q_s = torch.randn(g["q"].shape, generator=gen).to(torch.bfloat16).to("cuda")
        ok.decode_step(lay, ca.pool, g["table"], ca.sink_k, ca.sink_v, ca.recent_k, ca.recent_v,
                       g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new, v_new, g["slots"],
                       pos_t, q_s, out_a, ws_a, mx, lse=lse_a, levels_k=g["levels_k"],
                       levels_v=g["levels_v"])
        ok.append(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k, cb.recent_v,
                  g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new, v_new, g["slots"], pos_t,
                  levels_k=g["levels_k"], levels_v=g["levels_v"])
        ok.decode_attn(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k, cb.recent_v,
                       g["slots"], pos_t + 1, q_s, g["u_k"], g["u_v"], out_b, ws_b, mx,
                       lse=lse_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), s
        assert torch.equal(lse_a, lse_b), s
        assert torch.equal(ca.pool, cb.pool), s
        assert torch.equal(ca.sink_k, cb.sink_k) and torch.equal(ca.sink_v, cb.sink_v), s
        assert torch.equal(ca.recent_k, cb.recent_k) and torch.equal(ca.recent_v, cb.recent_v), s
    case.lengths = final
    case.q = q_s.cpu()
    ref, ref_lse = case.oracle_attention(case.oracle_pool())
    err = attention_error(out_a.cpu().numpy(), ref)
    _note(f"fused step final max row error {err:.3e}")
    assert err <= ATTN_TOL
    assert np.allclose(lse_a.cpu().numpy(), ref_lse, rtol=0, atol=1e-3)


def _draw(seed):
    """A seeded shape for the two-launch step: batch 1-4, one, two or four query heads per KV
    head, positions from the sink to a few thousand, some exactly at a boundary."""
    rng = np.random.default_rng(1000 + seed)
    gqa = int(rng.choice([1, 2, 4]))
    hkv = int(rng.choice([1, 2, 4])) if gqa < 4 else int(rng.choice([1, 2]))
    batch = int(rng.integers(1, 5))
    edges = [63, 64, 319, 320, 383, 384, 399, 400, 447, 448]
    start = [int(rng.choice(edges)) - 1 if rng.random() < 0.4 else int(rng.integers(0, 3000))
             for _ in range(batch)]
    return gqa * hkv, hkv, [max(0, s) for s in start]


@pytest.mark.parametrize("seed", range(8))
def test_fused_step_sweep(seed):
    hq, hkv, start = _draw(seed)
    B, steps = len(start), 3
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=hq, num_kv_heads=hkv)
    # the shortest max_seq_len from 100k up whose plan fuses the step
    mx = next(m for m in range(100000, 400001, 20000)
              if ok.decode_step_launches(ok.make_layout(hq, hkv, 10, B, (m + 63) // 64, 128),
                                         B, m) == 2)
    case = Case(wl, [s + steps for s in start], spare=mx)
    final = list(case.lengths)
    case.lengths = list(start)
    g = case.gpu_inputs()
    lay = case.layout
    assert ok.decode_step_launches(lay, B, mx) == 2
    _note(f"fused sweep {seed}: hq={hq} hkv={hkv} start={start} max_seq_len={mx}")
    ca, cb = case.gpu_cache(g), case.gpu_cache(g)
    ws_a = torch.zeros(ok.decode_workspace_bytes(lay, B, mx), dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    out_a = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    gen = torch.Generator().manual_seed(seed)
    for s in range(steps):
        pos = [p + s for p in start]
        k_new = torch.stack([case.k[b][pos[b]] for b in range(B)]).to("cuda")
        v_new = torch.stack([case.v[b][pos[b]] for b in range(B)]).to("cuda")
        pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
        q_s = torch.randn(g["q"].shape, generator=gen).to(torch.bfloat16).to("cuda")
        ok.decode_step(lay, ca.pool, g["table"], ca.sink_k, ca.sink_v, ca.recent_k, ca.recent_v,
                       g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new, v_new, g["slots"],
                       pos_t, q_s, out_a, ws_a, mx)
        ok.append(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k, cb.recent_v,
                  g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new, v_new, g["slots"], pos_t)
        ok.decode_attn(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k, cb.recent_v,
                       g["slots"], pos_t + 1, q_s, g["u_k"], g["u_v"], out_b, ws_b, mx)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), s
        assert torch.equal(ca.pool, cb.pool), s
        assert torch.equal(ca.sink_k, cb.sink_k) and torch.equal(ca.sink_v, cb.sink_v), s
        assert torch.equal(ca.recent_k, cb.recent_k) and torch.equal(ca.recent_v, cb.recent_v), s
    case.lengths = final
    case.q = q_s.cpu()
    ref, _ = case.oracle_attention(case.oracle_pool())
    assert attention_error(out_a.cpu().numpy(), ref) <= ATTN_TOL
