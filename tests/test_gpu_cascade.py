"""GPU parity of the shared-prefix cascade (oscar_decode_attn_prefix, oscar_decode_step_prefix)
through the C ABI.  The cascade changes only who reads the prefix pages (a cascade block stages a
chunk of 12 shared pages of a KV head once for up to 16 sequences), not what is computed: every
case is checked against the oracle's attention over the same cache bytes (max row error 2e-3,
LSE 1e-3) and against the plain oscar_decode_attn on the same inputs.  The two GPU paths run the
same per-page-pair arithmetic; they differ in where pairs of pages start (a cascade chunk's
pairs start at its first page, a split's after the chunks it skips), so the probabilities of a
pair are split into fp8 parts against another pair maximum, and in how the fp32 partials are
grouped before the merge.  Both move a row by a few 1e-6 of its largest output (about 2^-20 per
element, the parts' resolution); the paths must agree to 1e-4, twenty times inside the oracle
tolerance, while a mistake in the cascade's bookkeeping (a chunk counted twice or dropped, a
wrong slot, a sequence given another's pages) moves rows by percents.

Workloads: the tiny GQA workload scaled to several head shapes, with a shared prefix of 8192
tokens (127 history pages: ten whole chunks and seven pages more) and ragged lengths from 1 token
to well past the prefix, so that sequences hold no chunk, part of the chunks, or all of them, and
groups of 16 end ragged."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import workloads
from oscar_cases import ATTN_TOL, Case, attention_error

pytestmark = pytest.mark.gpu

PREFIX = 8192
# 1 token (no history), inside the prefix (no whole chunk, one chunk, chunks and a partial page),
# exactly at chunk ends, past the prefix by a little and by a lot
LENGTHS = [9000, 1, 700, 320 + 12 * 64, 320 + 12 * 64 - 1, 320 + 24 * 64 + 5, 3000, 8191 + 320,
           12000, 5000, 8192, 320 + 120 * 64, 8500, 2048, 321, 15000,
           10000, 7000, 320 + 127 * 64, 4400]
PAIR_TOL = 1e-4


def _note(msg):
    print(msg, flush=True)


def _case(hq, hkv, lengths, group=128, spare=0):
    wl = workloads.scaled(workloads.get("tiny_gqa4_1k"), num_q_heads=hq, num_kv_heads=hkv,
                          group_size=group, shared_prefix=PREFIX, batch=len(lengths))
    return Case(wl, lengths, spare=spare)


def _prefix_inputs(case, spare=0, cut=None):
    ids, shared = workloads.shared_prefix(case.wl, case.table, case.lengths, spare_tokens=spare)
    if cut is not None:
        shared = np.minimum(shared, cut).astype(np.int32)
    ok.check_shared_prefix(case.layout, case.table, ids, shared)
    return (torch.from_numpy(np.ascontiguousarray(ids)).cuda(),
            torch.from_numpy(np.ascontiguousarray(shared)).cuda())


def _attend_prefix(case, g, cache, ids, shared, mx=None, stages=None):
    mx = max(case.lengths) if mx is None else mx
    out = torch.full((case.batch, case.wl.num_q_heads, 128), float("nan"), dtype=torch.float32,
                     device="cuda")
    lse = torch.full((case.batch, case.wl.num_q_heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    nbytes = ok.decode_workspace_bytes_prefix(case.layout, case.batch, mx, ids.numel())
    # NaN bytes in the workspace: a slot read before it is written poisons the row
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    for st in ([ok.STAGE_ALL] if stages is None else stages):
        ok.decode_attn_prefix(case.layout, cache.pool, g["table"], cache.sink_k, cache.sink_v,
                              cache.recent_k, cache.recent_v, g["slots"], g["lens"], g["q"],
                              g["u_k"], g["u_v"], ids, shared, out, ws, mx, lse=lse, stages=st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _blocks(case, pool):
    """The GPU pool's bytes as the oracle's [page][KV head][block] array."""
    return pool.cpu().numpy().reshape(case.num_pages, case.wl.num_kv_heads, -1)


def _rel(a, b):
    scale = np.maximum(np.abs(b).max(axis=-1, keepdims=True), 1e-30)
    return float(np.max(np.abs(a - b) / scale))


def _check(case, g, cache, out, lse, plain=None):
    ref, ref_lse = case.oracle_attention(_blocks(case, cache.pool))
    err = attention_error(out, ref)
    lerr = float(np.max(np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse))))
    _note(f"  vs oracle: max row error {err:.3e}, lse {lerr:.2e}")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert err <= ATTN_TOL
    assert lerr <= 1e-3
    if plain is None:
        plain = case.gpu_attention(g, cache)
    d, dl = _rel(out, plain[0]), float(np.max(np.abs(lse - plain[1])))
    _note(f"  vs plain decode_attn: {d:.2e}, lse {dl:.2e}")
    assert d <= PAIR_TOL and dl <= PAIR_TOL


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 4)])
def test_cascade_matches_oracle_and_plain_path(hq, hkv):
    case = _case(hq, hkv, LENGTHS)
    ids, shared = _prefix_inputs(case)
    _note(f"cascade hq={hq} hkv={hkv}: {len(LENGTHS)} sequences, prefix {ids.numel()} pages, "
          f"shared {shared.tolist()}")
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    out, lse = _attend_prefix(case, g, cache, ids, shared)
    _check(case, g, cache, out, lse)


def test_cascade_stage_by_stage_and_larger_plans():
    # the stages run one call at a time give the one-call result bit for bit; a max_seq_len
    # beyond the longest sequence (more splits, a different pages-per-split) changes nothing
    case = _case(8, 2, LENGTHS)
    # page-table rows long enough for 131072-token plans
    case.table = np.pad(case.table, ((0, 0), (0, 2100 - case.table.shape[1])))
    case.layout = ok.make_layout(8, 2, case.num_pages, case.batch, 2100, 128)
    ids, shared = _prefix_inputs(case)
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    out, lse = _attend_prefix(case, g, cache, ids, shared)
    staged = _attend_prefix(case, g, cache, ids, shared,
                            stages=[ok.STAGE_QUERY, ok.STAGE_BF16, ok.STAGE_INT2, ok.STAGE_MERGE])
    assert np.array_equal(out, staged[0]) and np.array_equal(lse, staged[1])
    plain = case.gpu_attention(g, cache)
    for mx in (20000, 131072):
        _note(f"max_seq_len {mx}: splits {ok.decode_splits(case.layout, case.batch, mx)}")
        big = _attend_prefix(case, g, cache, ids, shared, mx=mx)
        assert _rel(big[0], plain[0]) <= PAIR_TOL
        assert float(np.max(np.abs(big[1] - plain[1]))) <= PAIR_TOL


@pytest.mark.parametrize("cut", [0, 5, 30, 200])
def test_cascade_with_fewer_shared_pages_declared(cut):
    # a row may declare fewer shared pages than its table aliases (down to none): the cascade
    # then takes fewer chunks for it and its split items the rest
    case = _case(8, 2, LENGTHS)
    ids, shared = _prefix_inputs(case, cut=cut)
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    out, lse = _attend_prefix(case, g, cache, ids, shared)
    plain = case.gpu_attention(g, cache)
    d = _rel(out, plain[0])
    _note(f"shared pages cut to {cut}: vs plain {d:.2e}")
    assert d <= PAIR_TOL
    assert float(np.max(np.abs(lse - plain[1]))) <= PAIR_TOL


def test_cascade_many_groups():
    # 40 sequences: groups of 16, 16 and 8; every sequence past the prefix
    rng = np.random.default_rng(7)
    lengths = [int(x) for x in rng.integers(PREFIX + 400, PREFIX + 4000, size=40)]
    lengths[5] = 1500   # one inside the prefix
    case = _case(8, 2, lengths)
    ids, shared = _prefix_inputs(case)
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    out, lse = _attend_prefix(case, g, cache, ids, shared)
    _check(case, g, cache, out, lse)


@pytest.mark.parametrize("hq,hkv,group", [(16, 2, 128), (8, 2, 64)])
def test_prefix_call_on_layouts_without_cascade(hq, hkv, group):
    # eight query heads per KV head, or group_size 64: the split items take every page
    case = _case(hq, hkv, LENGTHS[:6], group=group)
    ids, shared = _prefix_inputs(case)
    assert (ok.decode_workspace_bytes_prefix(case.layout, case.batch, max(case.lengths),
                                             ids.numel()) ==
            ok.decode_workspace_bytes(case.layout, case.batch, max(case.lengths)))
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)
    out, lse = _attend_prefix(case, g, cache, ids, shared)
    plain = case.gpu_attention(g, cache)
    assert np.array_equal(out, plain[0]) and np.array_equal(lse, plain[1])


def test_decode_step_prefix_matches_decode_step():
    # decode steps over a shared prefix: sequences past the prefix cross page boundaries, one
    # inside it writes into private copies (the table gives it those); the prefix step and the
    # plain step write the same pool bytes and agree on attention every step
    steps = 40
    start = [PREFIX + 300, PREFIX + 1000 - 20, 2500, PREFIX + 64 * 30 + 320 - 7]
    case = _case(8, 2, [s + steps for s in start])
    final = list(case.lengths)
    # the table of the starting lengths with room for the steps: a page a step writes into is
    # private to its sequence (copy-on-write)
    case.lengths = list(start)
    case.table, case.num_pages = workloads.page_tables(case.wl, start, 0, spare_tokens=steps)
    case.layout = ok.make_layout(8, 2, case.num_pages, 4, case.table.shape[1], 128)
    ids, shared = _prefix_inputs(case, spare=steps)
    ok.check_page_table(case.layout, case.table, start, extra_tokens=steps)
    g = case.gpu_inputs()
    lay = case.layout
    ca, cb = case.gpu_cache(g), case.gpu_cache(g)
    mx = max(final)
    ws_a = torch.zeros(ok.decode_workspace_bytes_prefix(lay, 4, mx, ids.numel()),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros(ok.decode_workspace_bytes(lay, 4, mx), dtype=torch.uint8, device="cuda")
    out_a = torch.empty((4, 8, 128), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    worst = 0.0
    for s in range(steps):
        pos = [p + s for p in start]
        k_new = torch.stack([case.k[b][pos[b]] for b in range(4)]).cuda()
        v_new = torch.stack([case.v[b][pos[b]] for b in range(4)]).cuda()
        pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
        ok.decode_step_prefix(lay, ca.pool, g["table"], ca.sink_k, ca.sink_v, ca.recent_k,
                              ca.recent_v, g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new,
                              v_new, g["slots"], pos_t, g["q"], ids, shared, out_a, ws_a, mx)
        ok.decode_step(lay, cb.pool, g["table"], cb.sink_k, cb.sink_v, cb.recent_k, cb.recent_v,
                       g["u_k"], g["u_v"], g["clip_k"], g["clip_v"], k_new, v_new, g["slots"],
                       pos_t, g["q"], out_b, ws_b, mx)
        torch.cuda.synchronize()
        worst = max(worst, _rel(out_a.cpu().numpy(), out_b.cpu().numpy()))
    _note(f"decode_step_prefix vs decode_step over {steps} steps: {worst:.2e}")
    assert worst <= PAIR_TOL
    assert torch.equal(ca.pool, cb.pool)
    assert torch.equal(ca.recent_k, cb.recent_k) and torch.equal(ca.recent_v, cb.recent_v)
    # the last step's attention against the oracle
    case.lengths = final
    ref, _ = case.oracle_attention(_blocks(case, ca.pool))
    err = attention_error(out_a.cpu().numpy(), ref)
    _note(f"final step vs oracle: {err:.3e}")
    assert err <= ATTN_TOL
