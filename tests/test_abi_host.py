"""Host-side tests of the C ABI: the library loads, exports every function include/oscar.h
declares, answers size queries, and rejects bad arguments before any HIP call (no GPU needed:
every call here fails validation or is a pure host function)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import bit_rotated_kv_decode_amd as ok

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(oscar_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 14
    lib = ok.lib()
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", ok.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\b(oscar_\w+)\b", dyn))
    assert set(names) <= exported
    # the binding declares a signature for each one
    assert set(names) == set(ok._SIGNATURES)


def test_version_and_status_strings():
    lib = ok.lib()
    assert lib.oscar_abi_version() == 8
    for s in (0, -1, -2, -3, -4, -5, -6, -99):
        assert lib.oscar_status_string(s)


def _lay(**kw):
    base = dict(head_dim=128, group_size=128, num_q_heads=32, num_kv_heads=8, page_tokens=64,
                sink_tokens=64, recent_tokens=256, num_pages=10, max_seqs=2, max_pages_per_seq=5,
                levels_kind=0)
    base.update(kw)
    return ok.Layout(*[base[n] for n, _ in ok.Layout._fields_])


@pytest.mark.parametrize("bad", [dict(head_dim=64), dict(group_size=32), dict(num_q_heads=30),
                                 dict(num_q_heads=128, num_kv_heads=8), dict(page_tokens=32),
                                 dict(sink_tokens=0), dict(recent_tokens=128), dict(num_pages=-1),
                                 dict(levels_kind=2)])
def test_layout_rejects_unsupported(bad):
    lay = _lay(**bad)
    assert ok.lib().oscar_layout_check(ctypes.byref(lay)) == -2
    assert ok.page_block_bytes(lay) == 0 and ok.pool_bytes(lay) == 0
    assert ok.lib().oscar_last_error()


def test_layout_null():
    assert ok.lib().oscar_layout_check(None) == -1


def test_size_queries():
    lay = _lay()
    assert ok.page_block_bytes(lay) == 4608
    assert ok.page_bytes(lay) == 8 * 4608
    assert ok.pool_bytes(lay) == 10 * 8 * 4608
    assert ok.sink_bytes(lay) == 2 * 8 * 64 * 128 * 2
    assert ok.recent_bytes(lay) == 2 * 8 * 256 * 128 * 2
    lay64 = _lay(group_size=64)
    assert ok.page_block_bytes(lay64) == 5120
    w1 = ok.decode_workspace_bytes(lay, 1, 1024)
    w2 = ok.decode_workspace_bytes(lay, 4, 100000)
    assert 0 < w1 < w2 and w1 % 256 == 0
    assert ok.decode_workspace_bytes(lay, -1, 10) == 0


def test_bf16_size_queries():
    lay = _lay()
    assert ok.bf16_page_block_bytes(lay) == 32768      # 64 tokens x 128 channels x (K, V) x 2 B
    assert ok.bf16_page_bytes(lay) == 8 * 32768
    assert ok.bf16_pool_bytes(lay) == 10 * 8 * 32768
    big = _lay(max_pages_per_seq=2000)
    # 100,000 tokens, batch 1, 8 KV heads: 1,563 pages in splits of 25 -> 63 splits; 32 rows of
    # (m, l) pairs (16,128 B) then 32 x 63 accumulators of 512 B
    assert ok.bf16_decode_workspace_bytes(big, 1, 100000) == 16128 + 32 * 63 * 512
    assert ok.bf16_decode_workspace_bytes(big, -1, 10) == 0
    assert ok.bf16_page_block_bytes(_lay(head_dim=64)) == 0


def _call_bf16_decode(lay, **over):
    a = dict(pool=4096, pt=4096, lens=4096, q=4096, out=4096, lse=None, ws=4096, wsb=1 << 30,
             batch=1, maxlen=300)
    a.update(over)
    return ok.lib().oscar_bf16_decode_attn(ctypes.byref(lay), a["pool"], a["pt"], a["lens"],
                                           a["q"], 0.0, a["out"], a["lse"], a["ws"], a["wsb"],
                                           a["batch"], a["maxlen"], None)


def _call_bf16_store(lay, **over):
    a = dict(pool=4096, pt=4096, k=4096, v=4096, sb=0, st=0, sh=0, start=4096, batch=1, n=1)
    a.update(over)
    return ok.lib().oscar_bf16_store(ctypes.byref(lay), a["pool"], a["pt"], a["k"], a["v"],
                                     a["sb"], a["st"], a["sh"], a["start"], a["batch"], a["n"],
                                     None)


def test_bf16_validation_happens_before_launch():
    lay = _lay()
    assert _call_bf16_decode(lay, q=None) == -1
    assert _call_bf16_decode(lay, pool=None) == -1
    assert _call_bf16_decode(lay, ws=None) == -5
    assert _call_bf16_decode(lay, wsb=16) == -5
    assert _call_bf16_decode(lay, q=4096 + 8) == -3      # operands are read 16 bytes at a time
    assert _call_bf16_decode(lay, ws=4096 + 64) == -3
    assert _call_bf16_decode(lay, maxlen=0) == -4
    assert _call_bf16_decode(lay, maxlen=5 * 64 + 1) == -4   # 6 pages > max_pages_per_seq 5
    assert _call_bf16_decode(lay, batch=-1) == -4
    assert _call_bf16_decode(lay, batch=0, q=None) == 0
    assert _call_bf16_decode(_lay(num_q_heads=24)) == -2
    assert _call_bf16_store(lay, pool=None) == -1
    assert _call_bf16_store(lay, start=4098) == -3
    assert _call_bf16_store(lay, pool=4100) == -3
    assert _call_bf16_store(lay, n=-1) == -4
    assert _call_bf16_store(lay, sh=-1) == -4
    assert _call_bf16_store(lay, n=0, pool=None) == 0


def _call_demote(lay, **over):
    a = dict(pool=4096, page_table=4096, u_k=4096, u_v=4096, clip_k=4096, clip_v=4096,
             lv_k=None, lv_v=None, k_src=4096, v_src=4096, sb=0, st=0, sh=0, hist=4096, batch=1,
             n=1)
    a.update(over)
    return ok.lib().oscar_demote(ctypes.byref(lay), a["pool"], a["page_table"], a["u_k"],
                                 a["u_v"], a["clip_k"], a["clip_v"], a["lv_k"], a["lv_v"],
                                 a["k_src"], a["v_src"], a["sb"], a["st"], a["sh"], a["hist"],
                                 a["batch"], a["n"], None)


def test_demote_validation_happens_before_launch():
    lay = _lay()
    assert _call_demote(lay, pool=None) == -1
    assert _call_demote(lay, hist=None) == -1
    assert _call_demote(lay, pool=4097) == -3
    assert _call_demote(lay, k_src=4097) == -3
    assert _call_demote(lay, batch=-1) == -4
    assert _call_demote(lay, st=-2) == -4
    assert _call_demote(_lay(group_size=16)) == -2
    # the codebook levels are optional; given, they must be 4-byte aligned
    assert _call_demote(lay, lv_k=4098, pool=None) == -1
    assert _call_demote(lay, lv_k=4098) == -3
    assert _call_demote(lay, lv_v=4097) == -3
    # nothing to do: OK without touching any pointer
    assert _call_demote(lay, pool=None, n=0) == 0
    assert _call_demote(lay, pool=None, batch=0) == 0


def _call_decode(lay, **over):
    a = dict(pool=4096, pt=4096, sk=4096, sv=4096, rk=4096, rv=4096, slot=4096, lens=4096,
             q=4096, uk=4096, uv=4096, out=4096, lse=None, ws=4096, wsb=1 << 30, batch=1,
             maxlen=600)
    a.update(over)
    return ok.lib().oscar_decode_attn(
        ctypes.byref(lay), a["pool"], a["pt"], a["sk"], a["sv"], a["rk"], a["rv"], a["slot"],
        a["lens"], a["q"], a["uk"], a["uv"], 0.0, a["out"], a["lse"], a["ws"], a["wsb"],
        a["batch"], a["maxlen"], None)


def test_decode_validation_happens_before_launch():
    lay = _lay()
    assert _call_decode(lay, q=None) == -1
    assert _call_decode(lay, out=None) == -1
    assert _call_decode(lay, ws=None) == -5
    assert _call_decode(lay, wsb=16) == -5
    assert _call_decode(lay, ws=4096 + 64) == -3
    assert _call_decode(lay, sk=4096 + 8) == -3
    assert _call_decode(lay, maxlen=0) == -4
    # 100000 tokens need 1558 pages > max_pages_per_seq 5
    assert _call_decode(lay, maxlen=100000) == -4
    assert _call_decode(lay, batch=-3) == -4
    assert _call_decode(lay, batch=0, q=None) == 0
    assert _call_decode(lay, wsb=16) == -5
    assert "workspace" in ok.lib().oscar_last_error().decode()
    # a split covers at most 256 pages and a head at most 1024 splits: 64 * 256 * 1024 history
    # tokens plus the 320 BF16 ones is the longest context the plan accepts
    big = _lay(max_pages_per_seq=300000)
    assert _call_decode(big, maxlen=64 * 256 * 1024 + 320 + 1) == -4
    assert "work items" in ok.lib().oscar_last_error().decode()


def _call_decode_cb(lay, **over):
    a = dict(pool=4096, pt=4096, sk=4096, sv=4096, rk=4096, rv=4096, slot=4096, lens=4096,
             q=4096, uk=4096, uv=4096, lk=4096, lv=4096, out=4096, lse=None, ws=4096,
             wsb=1 << 30, batch=1, maxlen=600, stages=ok.STAGE_ALL)
    a.update(over)
    return ok.lib().oscar_decode_attn_codebook(
        ctypes.byref(lay), a["pool"], a["pt"], a["sk"], a["sv"], a["rk"], a["rv"], a["slot"],
        a["lens"], a["q"], a["uk"], a["uv"], a["lk"], a["lv"], 0.0, a["out"], a["lse"], a["ws"],
        a["wsb"], a["batch"], a["maxlen"], a["stages"], None)


def test_codebook_attention_validation_happens_before_launch():
    # a history encoded with symmetric codebooks needs their levels, and runs on the fp8 pass only
    sym = _lay(levels_kind=1)
    assert _call_decode(sym) == -2                       # the plain entry point refuses it
    assert "codebook" in ok.lib().oscar_last_error().decode()
    assert _call_decode_cb(sym, lk=None) == -1
    assert _call_decode_cb(sym, lv=4096 + 2) == -3
    assert _call_decode_cb(_lay(levels_kind=1, num_q_heads=64), ) == -2   # 8 heads per KV head
    assert _call_decode_cb(_lay(levels_kind=1, group_size=64)) == -2
    assert _call_decode_cb(sym, q=None) == -1            # the usual checks still run
    assert _call_decode_cb(sym, maxlen=100000) == -4
    assert _call_decode_cb(sym, batch=0, q=None) == 0


def test_append_validation_happens_before_launch():
    lay = _lay()
    f = ok.lib().oscar_append
    args = [4096] * 16
    args[10] = args[11] = None   # levels_k, levels_v: optional
    assert f(ctypes.byref(lay), *([None] + args[1:]), 1, None) == -1
    assert f(ctypes.byref(lay), *([4096 + 4] + args[1:]), 1, None) == -3
    assert f(ctypes.byref(_lay(max_seqs=0)), *args, 1, None) == -2
    assert f(ctypes.byref(lay), *args, -1, None) == -4
    bad = list(args)
    bad[11] = 4096 + 2
    assert f(ctypes.byref(lay), *bad, 1, None) == -3


def _call_step(lay, **over):
    a = dict(pool=4096, pt=4096, sk=4096, sv=4096, rk=4096, rv=4096, uk=4096, uv=4096, ck=4096,
             cv=4096, lk=None, lv=None, kn=4096, vn=4096, slot=4096, pos=4096, q=4096, out=4096,
             lse=None, ws=4096, wsb=1 << 30, batch=1, maxlen=600)
    a.update(over)
    return ok.lib().oscar_decode_step(
        ctypes.byref(lay), a["pool"], a["pt"], a["sk"], a["sv"], a["rk"], a["rv"], a["uk"],
        a["uv"], a["ck"], a["cv"], a["lk"], a["lv"], a["kn"], a["vn"], a["slot"], a["pos"],
        a["q"], 0.0, a["out"], a["lse"], a["ws"], a["wsb"], a["batch"], a["maxlen"], None)


def test_step_validation_happens_before_launch():
    lay = _lay()
    # an append argument or a decode argument may fail; either way nothing is launched
    assert _call_step(lay, kn=None) == -1
    assert _call_step(lay, ck=4096 + 2) == -3
    assert _call_step(lay, lk=4096 + 2) == -3
    assert _call_step(_lay(max_seqs=0)) == -2
    assert _call_step(lay, q=None) == -1
    assert _call_step(lay, ws=None) == -5
    assert _call_step(lay, maxlen=100000) == -4
    assert _call_step(lay, batch=-1) == -4
    assert _call_step(lay, batch=0, q=None, kn=None) == 0


def test_check_page_table():
    lay = _lay(num_pages=8, max_pages_per_seq=4)
    # 320 + 3*64 tokens -> 3 pages each
    lens = [320 + 3 * 64, 320 + 2 * 64 + 1]
    good = np.array([[5, 1, 7, 0], [2, 3, 6, 0]], np.int32)
    ok.check_page_table(lay, good, lens)
    with pytest.raises(ok.OscarError):
        ok.check_page_table(lay, np.array([[5, 1, 8, 0], [2, 3, 6, 0]], np.int32), lens)
    with pytest.raises(ok.OscarError):          # page 1 used twice by sequence 0
        ok.check_page_table(lay, np.array([[5, 1, 1, 0], [2, 3, 6, 0]], np.int32), lens)
    with pytest.raises(ok.OscarError):          # shared page at different logical positions
        ok.check_page_table(lay, np.array([[5, 1, 7, 0], [1, 3, 6, 0]], np.int32), lens)
    # a shared prefix of two pages is fine, a shared page after a private one is not
    ok.check_page_table(lay, np.array([[5, 1, 7, 0], [5, 1, 6, 0]], np.int32), lens)
    with pytest.raises(ok.OscarError):
        ok.check_page_table(lay, np.array([[5, 1, 7, 0], [2, 1, 6, 0]], np.int32), lens)
    with pytest.raises(ok.OscarError):          # 5 pages needed > 4
        ok.check_page_table(lay, good, [320 + 4 * 64 + 1, 10])
    ok.check_page_table(lay, good, [320 + 3 * 64, 10], extra_tokens=64)   # 4 pages fit
    with pytest.raises(ok.OscarError):
        ok.check_page_table(lay, good, [320 + 3 * 64, 10], extra_tokens=65)
    with pytest.raises(ok.OscarError):
        ok.check_page_table(lay, good, [-1, 10])


def test_workload_page_tables_pass_the_checker():
    import workloads
    wl = workloads.scaled(workloads.get("qwen3_8b_b64_prefix"), batch=8)
    lens = workloads.context_lengths(wl)
    table, num_pages = workloads.page_tables(wl, lens, spare_tokens=10)
    lay = _lay(num_pages=num_pages, max_pages_per_seq=table.shape[1], max_seqs=8)
    ok.check_page_table(lay, table, lens, extra_tokens=10)
    # every sequence shares the prefix pages below the page its next write falls in
    shared = (32768 - 64) // 64
    for b, L in enumerate(lens):
        n0 = min(shared, (L - 320) // 64)
        assert workloads.shared_pages(wl, L, 10) == n0
        assert (table[b, :n0] == table[0, :n0]).all()
        # from there on the sequence's pages are its own
        own = table[b, n0:workloads.history_pages(L + 10)]
        others = np.concatenate([table[c, :workloads.history_pages(lens[c] + 10)]
                                 for c in range(len(lens)) if c != b])
        assert not np.isin(own, others).any()
    # without private copies, a sequence inside the prefix would demote into a shared page
    short = int(np.argmin(lens))
    assert lens[short] - 320 < shared * 64
    aliased = table.copy()
    n_short = workloads.history_pages(lens[short] + 10)
    longest = int(np.argmax(lens))
    aliased[short, :n_short] = table[longest, :n_short]
    ok.check_page_table(lay, aliased, lens)                    # reading shared pages is fine
    with pytest.raises(ok.OscarError, match="share"):
        ok.check_page_table(lay, aliased, lens, extra_tokens=10)


def test_check_page_table_rejects_writes_into_shared_pages():
    lay = _lay(num_pages=8, max_pages_per_seq=4)
    # sequence 1 holds 1.5 pages of history, both its pages are aliased from sequence 0
    lens = [320 + 3 * 64, 320 + 64 + 32]
    table = np.array([[5, 1, 7, 0], [5, 1, 0, 0]], np.int32)
    ok.check_page_table(lay, table, lens)
    with pytest.raises(ok.OscarError, match="share"):    # next write: slot 32 of page 1
        ok.check_page_table(lay, table, lens, extra_tokens=1)
    # a private copy of the written page makes the table valid
    ok.check_page_table(lay, np.array([[5, 1, 7, 0], [5, 2, 0, 0]], np.int32), lens,
                        extra_tokens=1)
    # a write range that reaches into the next page needs that page private too
    ok.check_page_table(lay, np.array([[5, 1, 7, 0], [5, 2, 3, 0]], np.int32), lens,
                        extra_tokens=33)
    with pytest.raises(ok.OscarError, match="share"):
        ok.check_page_table(lay, np.array([[5, 1, 7, 0], [5, 2, 7, 0]], np.int32),
                            [320 + 3 * 64, 320 + 64 + 32], extra_tokens=33)
    # contexts without history yet: the first demotion writes history index 0
    with pytest.raises(ok.OscarError, match="share"):
        ok.check_page_table(lay, np.array([[5, 1, 7, 0], [5, 0, 0, 0]], np.int32),
                            [320 + 3 * 64, 320], extra_tokens=1)
    ok.check_page_table(lay, np.array([[5, 1, 7, 0], [4, 0, 0, 0]], np.int32),
                        [320 + 3 * 64, 320], extra_tokens=1)


def test_levels_marshalling_checks_shape_and_device():
    # the binding accepts None (plain grid) or an fp32 [Hkv, 2] device tensor for levels_k /
    # levels_v; anything else raises before the library is called
    import torch
    lay = _lay()
    assert ok._levels(None, "levels_k", lay) is None
    with pytest.raises(TypeError, match="Hkv, 2"):
        ok._levels(torch.zeros(lay.num_kv_heads + 1, 2), "levels_k", lay)
    with pytest.raises(TypeError, match="GPU"):
        ok._levels(torch.zeros(lay.num_kv_heads, 2), "levels_k", lay)


def _int2_buffers(lay, bsz, **wrong):
    """Host tensors of the sizes the INT2 entry points need; ``wrong`` replaces some of them."""
    import torch
    hkv, hq = lay.num_kv_heads, lay.num_q_heads
    t = dict(pool=torch.zeros(ok.pool_bytes(lay), dtype=torch.uint8),
             table=torch.zeros(bsz, lay.max_pages_per_seq, dtype=torch.int32),
             sink_k=torch.zeros(lay.max_seqs, hkv, 64, 128, dtype=torch.bfloat16),
             recent_k=torch.zeros(lay.max_seqs, hkv, 256, 128, dtype=torch.bfloat16),
             u=torch.zeros(hkv, 128, 128), clip=torch.ones(hkv),
             rows=torch.zeros(bsz, dtype=torch.int32),
             q=torch.zeros(bsz, hq, 128, dtype=torch.bfloat16),
             out=torch.zeros(bsz, hq, 128), lse=torch.zeros(bsz, hq),
             kn=torch.zeros(bsz, hkv, 128, dtype=torch.bfloat16),
             ws=torch.zeros(1 << 20, dtype=torch.uint8))
    t.update(wrong)
    return t


@pytest.mark.parametrize("wrong, name", [
    (dict(pool="short"), "pool"), (dict(table="cols"), "page_table"),
    (dict(table="rows"), "page_table"), (dict(u="heads"), "u_k"), (dict(clip="heads"), "clip_k"),
    (dict(sink_k="slots"), "sink_k"), (dict(recent_k="slots"), "recent_k"),
    (dict(rows="short"), "seq_slot"), (dict(lse="shape"), "lse")])
def test_binding_rejects_undersized_buffers(wrong, name):
    # the C ABI cannot see allocation sizes, so the binding checks every buffer against the
    # layout before the call; a wrong size raises TypeError naming the buffer
    import torch
    lay = _lay(num_pages=6, max_seqs=3, max_pages_per_seq=4)
    bsz = 2
    good = _int2_buffers(lay, bsz)
    bad = {"short": lambda t: t[:-1] if t.dim() == 1 else t[:, :-1],
           "cols": lambda t: t[:, :-1], "rows": lambda t: t[:1],
           "heads": lambda t: t[:-1], "slots": lambda t: t[:-1],
           "shape": lambda t: t[:, :-1]}
    key = next(iter(wrong))
    t = dict(good)
    t[key] = bad[wrong[key]](good[key]).contiguous()
    calls = {
        "append": lambda: ok.append(lay, t["pool"], t["table"], t["sink_k"], t["sink_k"],
                                    t["recent_k"], t["recent_k"], t["u"], t["u"], t["clip"],
                                    t["clip"], t["kn"], t["kn"], t["rows"], good["rows"]),
        "decode_attn": lambda: ok.decode_attn(lay, t["pool"], t["table"], t["sink_k"],
                                              t["sink_k"], t["recent_k"], t["recent_k"],
                                              t["rows"], good["rows"], t["q"], t["u"], t["u"],
                                              t["out"], t["ws"], 1000, lse=t["lse"]),
        "decode_step": lambda: ok.decode_step(lay, t["pool"], t["table"], t["sink_k"],
                                              t["sink_k"], t["recent_k"], t["recent_k"], t["u"],
                                              t["u"], t["clip"], t["clip"], t["kn"], t["kn"],
                                              t["rows"], good["rows"], t["q"], t["out"],
                                              t["ws"], 1000, lse=t["lse"]),
    }
    uses = {"append": {"pool", "table", "sink_k", "recent_k", "u", "clip", "rows"},
            "decode_attn": {"pool", "table", "sink_k", "recent_k", "u", "rows", "lse"},
            "decode_step": {"pool", "table", "sink_k", "recent_k", "u", "clip", "rows", "lse"}}
    for fn, call in calls.items():
        if key not in uses[fn]:
            continue
        with pytest.raises(TypeError, match=name):
            call()
    # with every size right, the call gets as far as the device check (host tensors here)
    t = dict(good)
    for call in calls.values():
        with pytest.raises(TypeError, match="GPU"):
            call()
    # demote: pool, table, rotation, clip and hist_start against the layout
    src = torch.zeros(bsz, 3, lay.num_kv_heads, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="hist_start"):
        ok.demote(lay, good["pool"], good["table"], good["u"], good["u"], good["clip"],
                  good["clip"], src, src, good["rows"][:1])
    with pytest.raises(TypeError, match="pool"):
        ok.demote(lay, good["pool"][:-1], good["table"], good["u"], good["u"], good["clip"],
                  good["clip"], src, src, good["rows"])
    # BF16 baseline entry points
    bpool = torch.zeros(ok.bf16_pool_bytes(lay), dtype=torch.uint8)
    with pytest.raises(TypeError, match="pool"):
        ok.bf16_store(lay, bpool[:-1], good["table"], src, src, good["rows"])
    with pytest.raises(TypeError, match="start_pos"):
        ok.bf16_store(lay, bpool, good["table"], src, src, good["rows"][:1])
    with pytest.raises(TypeError, match="page_table"):
        ok.bf16_decode_attn(lay, bpool, good["table"][:, :-1].contiguous(), good["rows"],
                            good["q"], good["out"], good["ws"], 1000)


def test_decode_splits_query():
    # the plan aims at one round of two blocks per compute unit (512 blocks with the BF16 chunk
    # blocks), at least 4 pages per split; on the four-head single-group pass, whole page pairs
    # per wave (multiples of 8 pages while the grid keeps 3/4 of its blocks), then one block per
    # compute unit (256) when that gives a wave four pairs or more, or two per unit give it less
    # than one
    lay = _lay(num_kv_heads=8, num_q_heads=32, max_pages_per_seq=2000)
    # 1558 pages x 8 heads: 27 -> 32 pages (392 blocks), then 49 -> 56 pages: 224 blocks
    assert ok.decode_splits(lay, 1, 100000) == (28, 56)
    # 507 x 8: 9 pages (16 would leave 254 of 456 blocks; one per unit would give 2 pairs)
    assert ok.decode_splits(lay, 1, 32768) == (57, 9)
    assert ok.decode_splits(lay, 1, 320) == (0, 4)
    # at most 96 splits per row (what the merge loads at once): 1558 / 96 -> 17 -> 24 pages
    one = _lay(num_kv_heads=1, num_q_heads=4, max_pages_per_seq=2000)
    assert ok.decode_splits(one, 1, 100000) == (65, 24)
    two = _lay(num_kv_heads=2, num_q_heads=8, max_pages_per_seq=2000)
    assert ok.decode_splits(two, 1, 100000) == (65, 24)
    gqa8 = _lay(num_kv_heads=8, num_q_heads=64, max_pages_per_seq=2000)
    assert ok.decode_splits(gqa8, 1, 100000) == (58, 27)      # the int8 / bf16 pass: as planned
    sym = _lay(num_kv_heads=8, num_q_heads=32, max_pages_per_seq=2000, levels_kind=1)
    assert ok.decode_splits(sym, 1, 100000) == (58, 27)       # symmetric codebooks: as planned
    big = _lay(num_kv_heads=8, num_q_heads=32, max_pages_per_seq=2100, max_seqs=64)
    assert ok.decode_splits(big, 64, 130009) == (8, 256)      # the per-item page limit
    with pytest.raises(ok.OscarError):
        ok.decode_splits(lay, -1, 10)


def test_probe_validation_happens_before_launch():
    lib = ok.lib()
    lay = _lay()
    buf, sink = 4096, 8192            # fake, aligned addresses: every call below is rejected
    assert lib.oscar_probe_read(None, 64, sink, 16, 16, None) == -1
    assert lib.oscar_probe_read(buf + 8, 64, sink, 16, 16, None) == -3
    assert lib.oscar_probe_read(buf, 72, sink, 16, 16, None) == -3
    assert lib.oscar_probe_read(buf, 64, sink, 16, 0, None) == -4
    assert lib.oscar_probe_read(buf, 64, sink, 15, 16, None) == -2
    assert lib.oscar_probe_read(buf, 0, sink, 16, 16, None) == 0      # nothing to read
    L = ctypes.byref(lay)
    assert lib.oscar_probe_gather(L, None, buf, 4, 2, 2, 0, sink, 64, None) == -1
    assert lib.oscar_probe_gather(L, buf, buf, 11, 2, 2, 0, sink, 64, None) == -4   # > num_pages
    assert lib.oscar_probe_gather(L, buf, buf, 4, 0, 2, 0, sink, 64, None) == -4
    assert lib.oscar_probe_gather(L, buf, buf, 4, 257, 2, 0, sink, 64, None) == -4
    assert lib.oscar_probe_gather(L, buf, buf, 4, 2, 5, 0, sink, 64, None) == -4
    assert lib.oscar_probe_gather(L, buf, buf, 4, 2, 0, 0, sink, 64, None) == -4
    assert lib.oscar_probe_gather(L, buf, buf, 4, 2, 2, -1, sink, 64, None) == -4
    # 2 splits x 8 heads x 4 waves = 64 sink words needed
    assert lib.oscar_probe_gather(L, buf, buf, 4, 2, 2, 0, sink, 63, None) == -2
    assert lib.oscar_probe_gather(L, buf, buf, 0, 2, 2, 0, sink, 0, None) == 0


def _call_step_noalloc(lay, **over):
    a = dict(pool=4096, pt=4096, sk=4096, sv=4096, rk=4096, rv=4096, uk=4096, uv=4096, ck=4096,
             cv=4096, lk=None, lv=None, kn=4096, vn=4096, slot=4096, pos=4096, q=4096, out=4096,
             lse=None, batch=1, maxlen=600)
    a.update(over)
    return ok.lib().oscar_decode_step_noalloc(
        ctypes.byref(lay), a["pool"], a["pt"], a["sk"], a["sv"], a["rk"], a["rv"], a["uk"],
        a["uv"], a["ck"], a["cv"], a["lk"], a["lv"], a["kn"], a["vn"], a["slot"], a["pos"],
        a["q"], 0.0, a["out"], a["lse"], a["batch"], a["maxlen"], None)


def _call_decode_prefix(lay, **over):
    a = dict(pool=4096, pt=4096, sk=4096, sv=4096, rk=4096, rv=4096, slot=4096, lens=4096,
             q=4096, uk=4096, uv=4096, ids=4096, shared=4096, npre=3, out=4096, lse=None,
             ws=4096, wsb=1 << 30, batch=1, maxlen=600, stages=ok.STAGE_ALL)
    a.update(over)
    return ok.lib().oscar_decode_attn_prefix(
        ctypes.byref(lay), a["pool"], a["pt"], a["sk"], a["sv"], a["rk"], a["rv"], a["slot"],
        a["lens"], a["q"], a["uk"], a["uv"], a["ids"], a["shared"], a["npre"], 0.0, a["out"],
        a["lse"], a["ws"], a["wsb"], a["batch"], a["maxlen"], a["stages"], None)


def _call_step_prefix(lay, **over):
    a = dict(pool=4096, pt=4096, sk=4096, sv=4096, rk=4096, rv=4096, uk=4096, uv=4096, ck=4096,
             cv=4096, kn=4096, vn=4096, slot=4096, pos=4096, q=4096, ids=4096, shared=4096,
             npre=3, out=4096, lse=None, ws=4096, wsb=1 << 30, batch=1, maxlen=600)
    a.update(over)
    return ok.lib().oscar_decode_step_prefix(
        ctypes.byref(lay), a["pool"], a["pt"], a["sk"], a["sv"], a["rk"], a["rv"], a["uk"],
        a["uv"], a["ck"], a["cv"], a["kn"], a["vn"], a["slot"], a["pos"], a["q"], a["ids"],
        a["shared"], a["npre"], 0.0, a["out"], a["lse"], a["ws"], a["wsb"], a["batch"],
        a["maxlen"], None)


def test_prefix_validation_happens_before_launch():
    lay = _lay()
    for call in (_call_decode_prefix, _call_step_prefix):
        assert call(lay, ids=None) == -1                  # a prefix needs its page ids
        assert call(lay, shared=None) == -1
        assert call(lay, ids=4098) == -3
        assert call(lay, shared=4097) == -3
        assert call(lay, npre=-1) == -4
        assert call(lay, npre=11) == -4                   # more pages than the pool holds
        assert call(lay, npre=6) == -4                    # longer than a page-table row
        assert call(_lay(levels_kind=1)) == -2            # no cascade over symmetric codebooks
        assert "levels_kind" in ok.lib().oscar_last_error().decode()
        assert call(lay, q=None) == -1                    # the checks of the plain call still run
        assert call(lay, ws=None) == -5
        assert call(lay, maxlen=100000) == -4
        # without a prefix the arrays are not needed, and nothing to do is OK
        assert call(lay, npre=0, ids=None, shared=None, q=None) == -1
        assert call(lay, batch=0, q=None, ids=None, shared=None, npre=0) == 0
    assert _call_step_prefix(lay, kn=None) == -1
    assert _call_step_prefix(lay, ck=4096 + 2) == -3
    assert _call_decode_prefix(lay, stages=0) == -4


def test_prefix_workspace_grows_by_the_cascade_slots():
    big = _lay(num_pages=4000, max_pages_per_seq=2100, max_seqs=64)
    for batch, maxlen in ((64, 131072), (1, 100000), (3, 40000)):
        base = ok.decode_workspace_bytes(big, batch, maxlen)
        assert ok.decode_workspace_bytes_prefix(big, batch, maxlen, 0) == base
        w = ok.decode_workspace_bytes_prefix(big, batch, maxlen, 511)
        # 42 whole chunks of 12 pages: 42 more partial slots of (m, l) and 128 accumulators per
        # (sequence, query head) row, each region rounded up to 256 bytes
        rows = batch * 32
        extra = w - base
        assert rows * 42 * (128 + 2) * 4 <= extra <= rows * 42 * (128 + 2) * 4 + 512
        # a prefix shorter than one chunk adds nothing
        assert ok.decode_workspace_bytes_prefix(big, batch, maxlen, 11) == base
    # layouts on the int8 / bf16 pass take no cascade: the plan is the plain one
    gqa8 = _lay(num_q_heads=64, num_pages=4000, max_pages_per_seq=2100, max_seqs=64)
    assert (ok.decode_workspace_bytes_prefix(gqa8, 64, 131072, 511) ==
            ok.decode_workspace_bytes(gqa8, 64, 131072))
    assert ok.decode_workspace_bytes_prefix(big, 64, 131072, -1) == 0


def test_check_shared_prefix():
    import workloads
    wl = workloads.scaled(workloads.get("qwen3_8b_b64_prefix"), batch=8)
    lens = workloads.context_lengths(wl)
    table, num_pages = workloads.page_tables(wl, lens, spare_tokens=10)
    lay = _lay(num_pages=num_pages, max_pages_per_seq=table.shape[1], max_seqs=8)
    ids, shared = workloads.shared_prefix(wl, table, lens, spare_tokens=10)
    assert len(ids) == max(shared) and len(ids) <= 511
    ok.check_shared_prefix(lay, table, ids, shared)
    # the description may claim fewer shared pages than the table has, never more
    ok.check_shared_prefix(lay, table, ids, [max(0, n - 5) for n in shared])
    with pytest.raises(ok.OscarError, match="shared prefix"):
        bad = list(shared)
        bad[int(np.argmin(shared))] += 1
        ok.check_shared_prefix(lay, table, ids, bad)
    with pytest.raises(ok.OscarError, match="outside"):
        ok.check_shared_prefix(lay, table, ids, [len(ids) + 1] * len(shared))
    with pytest.raises(ok.OscarError, match="outside"):
        bad_ids = np.array(ids, np.int32)
        bad_ids[3] = num_pages
        ok.check_shared_prefix(lay, table, bad_ids, shared)
    ok.check_shared_prefix(lay, table, [], [0] * len(shared))


def test_step_noalloc_validation_happens_before_launch():
    # the no-allocation step checks what oscar_decode_step checks, plus its scratch limit, all
    # before it looks up the scratch array or launches anything
    lay = _lay()
    assert _call_step_noalloc(lay, kn=None) == -1
    assert _call_step_noalloc(lay, q=None) == -1
    assert _call_step_noalloc(lay, ck=4096 + 2) == -3
    assert _call_step_noalloc(lay, maxlen=100000) == -4
    assert _call_step_noalloc(lay, batch=-1) == -4
    assert _call_step_noalloc(lay, batch=0, q=None, kn=None) == 0
    # a plan larger than the 16 MiB scratch array is refused with a message that says so
    big = _lay(num_q_heads=64, num_kv_heads=8, max_seqs=512, max_pages_per_seq=2100)
    need = ok.decode_workspace_bytes(big, 512, 131072)
    assert need > (16 << 20)
    assert _call_step_noalloc(big, batch=512, maxlen=131072) == -5
    assert "scratch" in ok.lib().oscar_last_error().decode()
    # the same plan with a caller workspace gets past that check (and fails on the fake pool)
    assert ok.decode_workspace_bytes(_lay(), 1, 600) <= (16 << 20)


def _call_step_stages(lay, **over):
    a = dict(pool=4096, pt=4096, sk=4096, sv=4096, rk=4096, rv=4096, uk=4096, uv=4096, ck=4096,
             cv=4096, lk=None, lv=None, kn=4096, vn=4096, slot=4096, pos=4096, q=4096, out=4096,
             lse=None, ws=4096, wsb=1 << 30, batch=1, maxlen=600, stages=ok.STAGE_ALL)
    a.update(over)
    return ok.lib().oscar_decode_step_stages(
        ctypes.byref(lay), a["pool"], a["pt"], a["sk"], a["sv"], a["rk"], a["rv"], a["uk"],
        a["uv"], a["ck"], a["cv"], a["lk"], a["lv"], a["kn"], a["vn"], a["slot"], a["pos"],
        a["q"], 0.0, a["out"], a["lse"], a["ws"], a["wsb"], a["batch"], a["maxlen"],
        a["stages"], None)


def test_step_stages_validation_happens_before_launch():
    lay = _lay(max_pages_per_seq=1600)
    long = dict(maxlen=100000)    # 224 INT2 blocks of 56 pages: the segment launch appends
    assert ok.decode_step_launches(lay, 1, 100000) == 2
    assert _call_step_stages(lay, stages=0, **long) == -4
    assert _call_step_stages(lay, stages=16, **long) == -4
    for part in (ok.STAGE_INT2, ok.STAGE_BF16, ok.STAGE_QUERY | ok.STAGE_BF16 | ok.STAGE_MERGE):
        assert _call_step_stages(lay, stages=part, **long) == -4
        assert "together" in ok.lib().oscar_last_error().decode()
    assert _call_step_stages(lay, q=None, **long) == -1    # the plain call's checks still run
    assert _call_step_stages(lay, wsb=16, **long) == -5


def test_step_launch_count():
    # the segment launch appends and rotates the query on the fp8 pass (at most four query heads
    # per KV head, one group per vector) without codebooks, when its INT2 blocks all run at once
    # with at least 32 pages each; otherwise a preparation launch first
    assert ok.decode_splits(_lay(), 1, 100000) == (28, 56)
    assert ok.decode_step_launches(_lay(), 1, 100000) == 2                   # 224 blocks
    assert ok.decode_step_launches(_lay(num_q_heads=8, num_kv_heads=2), 4, 100000) == 2
    assert ok.decode_step_launches(_lay(num_q_heads=4, num_kv_heads=4), 2, 100000) == 2
    assert ok.decode_step_launches(_lay(), 1, 600) == 3                      # 4 pages per block
    assert ok.decode_step_launches(_lay(num_q_heads=4, num_kv_heads=1), 1, 100000) == 3
    assert ok.decode_step_launches(_lay(), 64, 32768) == 3                   # > one block per unit
    assert ok.decode_step_launches(_lay(num_q_heads=64), 1, 100000) == 3     # eight per KV head
    assert ok.decode_step_launches(_lay(group_size=64), 1, 100000) == 3      # two groups
    assert ok.decode_step_launches(_lay(levels_kind=1), 1, 100000) == 3      # symmetric levels
    assert ok.decode_step_launches(_lay(), 0, 600) == 0
    assert ok.decode_step_launches(_lay(head_dim=64), 1, 600) == 0
