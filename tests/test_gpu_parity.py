"""GPU parity of liboscar against the CPU oracle, called through the C ABI.

Demotion: pool bytes bit-exact under the acceptance rule of oscar_cases.  Attention: the GPU reads
pool bytes written by the oracle (so the attention comparison does not depend on demotion) and
must match the oracle's softmax attention within 2e-3 max row error; an end-to-end case uses the
GPU's own demotion."""
import math

import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import oracle
import workloads
from oscar_cases import ATTN_TOL, Case, attention_error, compare_pool_blocks

pytestmark = pytest.mark.gpu


def _tiny(**kw):
    return workloads.scaled(workloads.get("tiny_gqa4_1k"), **kw)


def _note(msg):
    print(msg, flush=True)


def test_demote_tiny_two_calls_bit_exact():
    # 704 history tokens written by two calls: 448 tokens, then 256 tokens
    case = Case(_tiny())
    _note(f"demote tiny: lengths={case.lengths} pages={case.num_pages}")
    g = case.gpu_inputs()
    cache = case.gpu_cache(g, pool_from_oracle=oracle.new_pool(case.num_pages, 1, case.geom))
    k = case.k[0].to("cuda")[64:768].unsqueeze(0)
    v = case.v[0].to("cuda")[64:768].unsqueeze(0)
    ok.demote(case.layout, cache.pool, g["table"], g["u_k"], g["u_v"], g["clip_k"], g["clip_v"],
              k[:, :448], v[:, :448], torch.zeros(1, dtype=torch.int32, device="cuda"))
    ok.demote(case.layout, cache.pool, g["table"], g["u_k"], g["u_v"], g["clip_k"], g["clip_v"],
              k[:, 448:], v[:, 448:], torch.full((1,), 448, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ref = case.oracle_pool()
    flips = compare_pool_blocks(cache.pool.cpu().numpy(), ref, case)
    _note(f"code flips: {flips}")


@pytest.mark.parametrize("group,hq,hkv", [(128, 8, 2), (64, 8, 1), (64, 16, 2)])
def test_demote_ragged_unaligned(group, hq, hkv):
    wl = _tiny(group_size=group, num_q_heads=hq, num_kv_heads=hkv)
    lengths = [321, 400, 1000, 385 + 64 * 5 + 3]
    case = Case(wl, lengths)
    _note(f"demote ragged g={group} hq={hq} hkv={hkv} lengths={lengths}")
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)                           # GPU demotion, one call per sequence
    torch.cuda.synchronize()
    compare_pool_blocks(cache.pool.cpu().numpy(), case.oracle_pool(), case)
    # unaligned starts: rewrite each sequence's history in pieces of 7, 13 and the rest
    cache2 = case.gpu_cache(g, pool_from_oracle=oracle.new_pool(case.num_pages, hkv, case.geom))
    for b, L in enumerate(lengths):
        n = L - 320
        k = case.k[b].to("cuda")[64:64 + n].unsqueeze(0)
        v = case.v[b].to("cuda")[64:64 + n].unsqueeze(0)
        for lo, hi in ((0, 7), (7, 20), (20, n)):
            ok.demote(case.layout, cache2.pool, g["table"][b:b + 1], g["u_k"], g["u_v"],
                      g["clip_k"], g["clip_v"], k[:, lo:hi], v[:, lo:hi],
                      torch.full((1,), lo, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(cache2.pool, cache.pool)


ATTN_CASES = {
    "tiny_1k": dict(wl=dict(), lengths=None),
    "edges_g4": dict(wl=dict(num_q_heads=8, num_kv_heads=2),
                     lengths=[1, 63, 64, 65, 300, 320, 321, 385, 1000, 1024 + 64 * 3 + 7]),
    "gqa1": dict(wl=dict(num_q_heads=2, num_kv_heads=2), lengths=[700, 2000]),
    "gqa2": dict(wl=dict(num_q_heads=4, num_kv_heads=2), lengths=[2500, 333]),
    "gqa8_g64": dict(wl=dict(num_q_heads=16, num_kv_heads=2, group_size=64),
                     lengths=[3000, 1500, 321]),
    "g64_gqa4": dict(wl=dict(num_q_heads=8, num_kv_heads=2, group_size=64), lengths=[4100]),
    # one sequence per launch selects the kernels' non-temporal page loads: every GQA width
    "gqa1_b1": dict(wl=dict(num_q_heads=2, num_kv_heads=2), lengths=[1700]),
    "gqa2_b1_g64": dict(wl=dict(num_q_heads=4, num_kv_heads=2, group_size=64), lengths=[2222]),
    "gqa8_b1": dict(wl=dict(num_q_heads=16, num_kv_heads=2), lengths=[2600]),
    "gqa8_b1_g64": dict(wl=dict(num_q_heads=16, num_kv_heads=2, group_size=64), lengths=[1901]),
}


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_attention_on_oracle_pool(name):
    spec = ATTN_CASES[name]
    case = Case(_tiny(**spec["wl"]), spec["lengths"])
    _note(f"attention {name}: lengths={case.lengths}")
    pool = case.oracle_pool()
    g = case.gpu_inputs()
    cache = case.gpu_cache(g, pool_from_oracle=pool)
    out, lse = case.gpu_attention(g, cache)
    ref, ref_lse = case.oracle_attention(pool)
    err = attention_error(out, ref)
    _note(f"max row error {err:.3e}")
    assert err <= ATTN_TOL
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3


def test_attention_many_rows_one_merge_block_per_row():
    # 64 sequences x 8 query heads = 512 rows: the merge takes one block per row (all four
    # output quarters) instead of one block per quarter; ragged lengths, some with no history
    wl = _tiny(num_q_heads=8, num_kv_heads=2)
    lengths = [int(x) for x in np.random.default_rng(3).integers(1, 1400, 64)]
    lengths[:4] = [1, 320, 321, 1399]
    case = Case(wl, lengths)
    _note(f"attention 512 rows: lengths {min(lengths)}..{max(lengths)}")
    pool = case.oracle_pool()
    g = case.gpu_inputs()
    cache = case.gpu_cache(g, pool_from_oracle=pool)
    out, lse = case.gpu_attention(g, cache)
    ref, ref_lse = case.oracle_attention(pool)
    err = attention_error(out, ref)
    _note(f"max row error {err:.3e}")
    assert err <= ATTN_TOL
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3


def test_attention_end_to_end_tiny():
    case = Case(_tiny())
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)                           # GPU demotion
    out, _ = case.gpu_attention(g, cache)
    ref, _ = case.oracle_attention(case.oracle_pool())  # oracle demotion
    err = attention_error(out, ref)
    _note(f"end-to-end max row error {err:.3e}")
    assert err <= ATTN_TOL


def test_hadamard_only_variant_end_to_end():
    # the Hadamard-only variant of the error chain (U = I, no clip: the largest finite clip):
    # GPU demotion and attention against the oracle's, through the same kernels
    wl = _tiny(num_q_heads=8, num_kv_heads=2)
    eye = torch.eye(128, dtype=torch.float32).expand(2, 128, 128).contiguous()
    no_clip = np.full(2, 65504.0, np.float32)
    case = Case(wl, [1500, 777], u=(eye, eye.clone()), clip=(no_clip, no_clip))
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    out, _ = case.gpu_attention(g, cache)
    ref, _ = case.oracle_attention(case.oracle_pool())
    err = attention_error(out, ref)
    _note(f"hadamard-only end-to-end max row error {err:.3e}")
    assert err <= ATTN_TOL


def test_page_shuffle_and_split_invariance():
    wl = _tiny(num_q_heads=8, num_kv_heads=2)
    case = Case(wl, [5000, 2222], spare=150000)   # room for a larger planning bound
    pool = case.oracle_pool()
    g = case.gpu_inputs()
    cache = case.gpu_cache(g, pool_from_oracle=pool)
    out1, _ = case.gpu_attention(g, cache)
    # a different physical placement of the same pages
    perm = np.random.default_rng(0).permutation(case.num_pages)
    pool2 = np.zeros_like(pool)
    pool2[perm] = pool
    table2 = case.table.copy()
    for b, L in enumerate(case.lengths):
        n = workloads.history_pages(L)
        table2[b, :n] = perm[case.table[b, :n]]
    g2 = dict(g)
    g2["table"] = torch.from_numpy(table2).to("cuda")
    cache2 = case.gpu_cache(g2, pool_from_oracle=pool2)
    out2, _ = case.gpu_attention(g2, cache2)
    assert np.array_equal(out1, out2)
    # a larger max_seq_len changes the split plan; the result changes only by rounding
    out3, _ = case.gpu_attention(g, cache, max_seq_len=150000)
    assert attention_error(out3, out1) < 1e-4


def test_softmax_reference_fallback():
    # A wave takes its softmax reference from its first page.  Here wave 0 of split 0 (pages 0
    # and 4 at 7 pages per split) sees small keys on page 0 and, on page 4, one key aligned with
    # query head 0 whose logit passes the reference by far more than 2^64: the wave must redo its
    # pages against its exact maxima (without that the output would overflow).
    wl = _tiny(num_q_heads=8, num_kv_heads=2)
    hkv = wl.num_kv_heads
    big = np.full(hkv, 1e4, np.float32)
    case = Case(wl, [5000, 700], spare=150000, clip=(big, big))
    for b in range(case.batch):
        k = case.k[b].float()
        k[64:64 + 7 * 64] *= 0.01                      # pages 0..6: small keys
        if b == 0:
            k[64 + 4 * 64 + 5, 0] = 10.0 * case.q[0, 0].float()   # page 4, KV head 0
        case.k[b] = k.to(torch.bfloat16)
    pool = case.oracle_pool()
    g = case.gpu_inputs()
    cache = case.gpu_cache(g, pool_from_oracle=pool)
    out, lse = case.gpu_attention(g, cache, max_seq_len=150000)
    ref, ref_lse = case.oracle_attention(pool)
    err = attention_error(out, ref)
    _note(f"reference fallback: max row error {err:.3e}, lse head 0 {lse[0, 0]:.2f} "
          f"(oracle {ref_lse[0, 0]:.2f})")
    assert np.isfinite(out).all()
    assert err <= ATTN_TOL
    assert np.max(np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse))) <= 1e-3


def test_append_steps_match_oracle():
    # decode-step writes from an empty cache across the sink / recent / history boundaries
    wl = _tiny(num_q_heads=4, num_kv_heads=2)
    steps = 400
    case = Case(wl, [steps + 5, steps + 40], spare=64)
    g = case.gpu_inputs()
    lay = case.layout
    cache = ok.Cache.allocate(lay)
    start = [5, 0]            # sequence 1 starts empty, sequence 0 five tokens behind
    hk = np.zeros((2, 2, 64, 128), np.float32)
    hv = np.zeros_like(hk)
    rk = np.zeros((2, 2, 256, 128), np.float32)
    rv = np.zeros_like(rk)
    pool = oracle.new_pool(case.num_pages, 2, case.geom)
    lens = [0, 0]
    for s in range(steps + 40):
        active = [b for b in range(2) if s >= start[b] and lens[b] < case.lengths[b]]
        if not active:
            continue
        idx = torch.tensor(active)
        k_new = torch.stack([case.k[b][lens[b]] for b in active])
        v_new = torch.stack([case.v[b][lens[b]] for b in active])
        tab = g["table"][idx.to("cuda")].contiguous()
        ok.append(lay, cache.pool, tab, cache.sink_k, cache.sink_v, cache.recent_k, cache.recent_v,
                  g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new.to("cuda"),
                  v_new.to("cuda"), torch.tensor(active, dtype=torch.int32, device="cuda"),
                  torch.tensor([lens[b] for b in active], dtype=torch.int32, device="cuda"))
        oracle.append(pool, case.table[active], hk, hv, rk, rv, case.u_k.numpy(),
                      case.u_v.numpy(), case.clip_k, case.clip_v, k_new.float().numpy(),
                      v_new.float().numpy(), active, [lens[b] for b in active], case.geom)
        for b in active:
            lens[b] += 1
    torch.cuda.synchronize()
    assert np.array_equal(cache.sink_k.float().cpu().numpy(), hk)
    assert np.array_equal(cache.recent_v.float().cpu().numpy(), rv)
    assert np.array_equal(cache.recent_k.float().cpu().numpy(), rk)
    case.lengths = lens
    compare_pool_blocks(cache.pool.cpu().numpy(), pool, case)


def test_decode_step_matches_append_then_attend():
    # oscar_decode_step (append + query rotation in one launch, then attention) against
    # oscar_append followed by oscar_decode_attn: identical outputs and cache bytes every step;
    # the sequences cross the full-ring threshold (320), value-word (16) and page (64) boundaries.
    wl = _tiny(num_q_heads=8, num_kv_heads=2)
    start, steps = [318, 1011], 30
    case = Case(wl, [s + steps for s in start])
    final = list(case.lengths)
    case.lengths = list(start)
    g = case.gpu_inputs()
    lay = case.layout
    ca, cb = case.gpu_cache(g), case.gpu_cache(g)
    mx = max(final)
    ws_a = torch.zeros(ok.decode_workspace_bytes(lay, 2, mx), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty_like(ws_a)
    gen = torch.Generator().manual_seed(11)   # a different query every step
    out_a = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    for s in range(steps):
        pos = [p + s for p in start]
        _note(f"decode step {s}: positions {pos}")
        k_new = torch.stack([case.k[b][pos[b]] for b in range(2)]).to("cuda")
        v_new = torch.stack([case.v[b][pos[b]] for b in range(2)]).to("cuda")
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
    assert torch.equal(ca.pool, cb.pool) and torch.equal(ca.sink_v, cb.sink_v)
    assert torch.equal(ca.recent_k, cb.recent_k) and torch.equal(ca.recent_v, cb.recent_v)
    case.lengths = final
    case.q = q_s.cpu()
    ref, _ = case.oracle_attention(case.oracle_pool())
    err = attention_error(out_a.cpu().numpy(), ref)
    _note(f"decode_step final max row error {err:.3e}")
    assert err <= ATTN_TOL
