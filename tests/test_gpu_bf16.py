"""GPU parity of the paged BF16 baseline (oscar_bf16_store, oscar_bf16_decode_attn) against the
CPU oracle, called through the C ABI.

Pool bytes after the GPU store are compared bit-exactly with the oracle's layout; attention must
match the oracle's fp64 softmax attention over the same bf16 keys and values within 2e-3 max row
error (the bound used for the INT2 path).  Pools start filled with NaN bit patterns, so a kernel
that let a slot past a sequence's length (or an unwritten page) reach a result would fail."""
import math

import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import oracle
import workloads
from oscar_cases import ATTN_TOL, attention_error

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0
LSE_TOL = 1e-3


def _note(msg):
    print(msg, flush=True)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Bf16Case:
    """One layer of the BF16 baseline: tokens of every sequence stored from position 0."""

    def __init__(self, wl, lengths, layer=0, spare=0):
        self.wl, self.lengths, self.layer = wl, list(lengths), layer
        self.batch = len(self.lengths)
        self.table, self.num_pages = workloads.page_tables(wl, self.lengths, layer,
                                                           spare_tokens=spare, sink=0, recent=0)
        self.lay = ok.make_layout(wl.num_q_heads, wl.num_kv_heads, self.num_pages, self.batch,
                                  self.table.shape[1], group_size=wl.group_size)
        self.table_dev = torch.from_numpy(self.table).to("cuda")
        nbytes = ok.bf16_pool_bytes(self.lay)
        self.pool = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.pool.view(torch.int16).fill_(NAN_BITS)
        self.kv = [workloads.kv_tokens(wl, layer, b, 0, L, device="cuda")
                   for b, L in enumerate(self.lengths)]

    def store_all(self):
        for b, (k, v) in enumerate(self.kv):
            ok.bf16_store(self.lay, self.pool, self.table_dev[b:b + 1].contiguous(),
                          k.unsqueeze(0), v.unsqueeze(0),
                          torch.zeros(1, dtype=torch.int32, device="cuda"))

    def oracle_pool(self, pages=None):
        """The oracle's pool (uint16 [num_pages, Hkv, 16384]) for the stored tokens; ``pages``
        restricts the work to a set of physical pages."""
        pool = oracle.bf16_new_pool(self.num_pages, self.wl.num_kv_heads, fill=NAN_BITS)
        for b, (k, v) in enumerate(self.kv):
            kb, vb = _bits(k), _bits(v)
            row = self.table[b]
            for t in range(self.lengths[b]):
                if pages is not None and int(row[t // 64]) not in pages:
                    continue
                for h in range(self.wl.num_kv_heads):
                    oracle.bf16_store(pool, row, t, h, kb[t, h], vb[t, h])
        return pool

    def attend(self, q, out, lse, lengths=None, max_seq_len=None):
        lengths = self.lengths if lengths is None else lengths
        max_seq_len = max(lengths) if max_seq_len is None else max_seq_len
        ws = torch.empty(ok.bf16_decode_workspace_bytes(self.lay, self.batch, max_seq_len),
                         dtype=torch.uint8, device="cuda")
        lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        ok.bf16_decode_attn(self.lay, self.pool, self.table_dev, lens, q, out, ws, max_seq_len,
                            lse=lse)

    def reference(self, q, rows, lengths=None, kv=None):
        lengths = self.lengths if lengths is None else lengths
        kv = self.kv if kv is None else kv
        qn = q.double().cpu().numpy()
        ref = np.full(q.shape, np.nan)
        lse = np.full(q.shape[:2], np.nan)
        g = self.wl.gqa
        cache = {}
        for b, h in rows:
            key = (b, h // g)
            if key not in cache:
                k, v = kv[b]
                L = lengths[b]
                cache = {key: (k[:L, h // g].double().cpu().numpy(),
                               v[:L, h // g].double().cpu().numpy())}
            ref[b, h], lse[b, h] = oracle.attend(qn[b, h], *cache[key], 1 / math.sqrt(128))
        return ref, lse


def _check(case, q, rows=None, lengths=None, kv=None):
    bsz, hq = q.shape[0], q.shape[1]
    out = torch.empty(bsz, hq, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(bsz, hq, dtype=torch.float32, device="cuda")
    case.attend(q, out, lse, lengths=lengths)
    torch.cuda.synchronize()
    rows = rows or [(b, h) for b in range(bsz) for h in range(hq)]
    ref, ref_lse = case.reference(q, rows, lengths=lengths, kv=kv)
    o = out.double().cpu().numpy()
    err = attention_error(o, ref, rows)
    lse_err = max(abs(float(lse[b, h]) - ref_lse[b, h]) for b, h in rows)
    _note(f"max row error {err:.3e}, lse error {lse_err:.3e}")
    assert np.all(np.isfinite(o[[b for b, _ in rows], [h for _, h in rows]]))
    assert err <= ATTN_TOL
    assert lse_err <= LSE_TOL
    return out


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
