"""Test support for the paged BF16 baseline: one layer's tokens stored from position 0, the
oracle's pool for the same tokens, and the comparison of attention rows (2e-3 max row error, the
bound of the INT2 path; LSE within 1e-3)."""
import math

import numpy as np
import torch

import bit_rotated_kv_decode_amd as ok
import oracle
import workloads
from oscar_cases import ATTN_TOL, attention_error

NAN_BITS = 0x7FC0
LSE_TOL = 1e-3


def bits(t: torch.Tensor) -> np.ndarray:
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
            kb, vb = bits(k), bits(v)
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


def check_bf16(case, q, rows=None, lengths=None, kv=None):
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
    print(f"max row error {err:.3e}, lse error {lse_err:.3e}", flush=True)
    assert np.all(np.isfinite(o[[b for b, _ in rows], [h for _, h in rows]]))
    assert err <= ATTN_TOL
    assert lse_err <= LSE_TOL
    return out
