"""Test support: one layer's cache state built twice from the same seeded inputs, on the GPU
through liboscar and on the host through the oracle, plus the comparison rules.

Acceptance rules (north of the kernels, fixed here):
  * demotion bytes are bit-exact, except a code whose oracle pre-rounding value t lies within
    1e-5 relative of a rounding boundary (k + 1/2), or fp16 meta whose pre-rounding value lies
    within 1e-5 relative of an fp16 midpoint (the codes of such a group are then checked to be
    the nearest level under the GPU's meta); at most 1e-4 of all codes may differ;
  * attention outputs: max over (sequence, query head) rows of |o_gpu - o_ref|_inf / |o_ref|_inf
    at most 2e-3.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import bit_rotated_kv_decode_amd as ok
import oracle
import workloads

ATTN_TOL = 2e-3
WINDOW = 1e-5
MAX_FLIP_FRACTION = 1e-4


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


class Case:
    """Inputs of one layer: token K/V per sequence (bf16, host), queries, U, clip, page table."""

    def __init__(self, wl, lengths=None, layer=0, spare=0, u=None, clip=None, device_tokens=None,
                 levels=None, codebook=None):
        self.wl = wl
        self.lengths = list(workloads.context_lengths(wl) if lengths is None else lengths)
        self.batch = len(self.lengths)
        self.layer = layer
        self.table, self.num_pages = workloads.page_tables(wl, self.lengths, layer,
                                                           spare_tokens=spare)
        if u is None:
            u = workloads.rotation_bases(wl, layer)
        self.u_k, self.u_v = u                          # torch fp32 [Hkv, d, d] host
        hkv = wl.num_kv_heads
        if clip is None:
            clip = (np.full(hkv, wl.clip, np.float32), np.full(hkv, wl.clip, np.float32))
        self.clip_k, self.clip_v = (np.asarray(c, np.float32) for c in clip)
        # optional equally spaced codebooks: (lo, step) per KV head for keys and for values
        self.levels_k, self.levels_v = ((None, None) if levels is None else
                                        (np.asarray(lv, np.float32) for lv in levels))
        # optional symmetric Lloyd-Max codebooks (reading R21): (l0, l1) per KV head for keys and
        # values, levels (l0, l1, 3 - l1, 3 - l0)
        assert levels is None or codebook is None
        self.cb_k, self.cb_v = ((None, None) if codebook is None else
                                (np.asarray(c, np.float32) for c in codebook))
        dev = device_tokens or "cpu"
        self.k, self.v = [], []
        for b, L in enumerate(self.lengths):
            k, v = workloads.kv_tokens(wl, layer, b, 0, L, dev)
            self.k.append(k)
            self.v.append(v)
        self.q = workloads.queries(wl, layer, 0, "cpu", batch=self.batch)
        self.geom = oracle.Geometry(group=wl.group_size)
        self.layout = ok.make_layout(wl.num_q_heads, wl.num_kv_heads, self.num_pages, self.batch,
                                     self.table.shape[1], wl.group_size,
                                     levels_kind=0 if codebook is None else ok.LEVELS_SYMMETRIC)

    # -------------------------------------------------------------------------------- oracle
    def oracle_segments(self):
        hkv, d = self.wl.num_kv_heads, self.wl.head_dim
        sk = np.zeros((self.batch, hkv, 64, d), np.float32)
        sv = np.zeros_like(sk)
        rk = np.zeros((self.batch, hkv, 256, d), np.float32)
        rv = np.zeros_like(rk)
        for b, L in enumerate(self.lengths):
            k, v = bf16_np(self.k[b]), bf16_np(self.v[b])
            ns = min(L, 64)
            sk[b, :, :ns] = k[:ns].transpose(1, 0, 2)
            sv[b, :, :ns] = v[:ns].transpose(1, 0, 2)
            pos = np.arange(max(64, L - 256), L)
            rk[b][:, pos % 256] = k[pos].transpose(1, 0, 2)
            rv[b][:, pos % 256] = v[pos].transpose(1, 0, 2)
        return sk, sv, rk, rv

    def oracle_pool(self, heads=None):
        pool = oracle.new_pool(self.num_pages, self.wl.num_kv_heads, self.geom)
        for b, L in enumerate(self.lengths):
            n = max(0, L - 320)
            if n == 0:
                continue
            k = bf16_np(self.k[b][64:64 + n])[None]
            v = bf16_np(self.v[b][64:64 + n])[None]
            if heads is not None:
                for h in heads:
                    kq = self.encode(k[0, :, h], "k", h)
                    vq = self.encode(v[0, :, h], "v", h)
                    oracle.store_history(pool, self.table[b], np.arange(n), h, kq, vq, self.geom)
            else:
                oracle.demote(pool, self.table[b:b + 1], self.u_k.numpy(), self.u_v.numpy(),
                              self.clip_k, self.clip_v, k, v, [0], self.geom, self.levels_k,
                              self.levels_v, self.codebooks("k"), self.codebooks("v"))
        return pool

    def head_levels(self, tensor, h):
        lv = self.levels_k if tensor == "k" else self.levels_v
        return None if lv is None else lv[h]

    def codebooks(self, tensor):
        """Four levels per KV head of the symmetric codebooks, or None."""
        cb = self.cb_k if tensor == "k" else self.cb_v
        return None if cb is None else np.stack([oracle.symmetric_levels(float(a), float(b))
                                                 for a, b in cb])

    def head_codebook(self, tensor, h):
        cb = self.codebooks(tensor)
        return None if cb is None else cb[h]

    def encode(self, x, tensor, h):
        """The oracle's (codes, scale, zero) of tokens x (fp32 [n, d]) for KV head h."""
        u = (self.u_k if tensor == "k" else self.u_v)[h].numpy()
        c = (self.clip_k if tensor == "k" else self.clip_v)[h]
        cb = self.head_codebook(tensor, h)
        if cb is not None:
            return oracle.quantize_codebook(oracle.rotate_to_fp32(x, u), c, self.geom.group, cb)
        return oracle.encode(x, u, c, self.geom.group, self.head_levels(tensor, h))[:3]

    def oracle_attention(self, pool, heads=None):
        sk, sv, rk, rv = self.oracle_segments()
        return oracle.decode_attention(pool, self.table, sk, sv, rk, rv, np.arange(self.batch),
                                       self.lengths, bf16_np(self.q), self.u_k.numpy(),
                                       self.u_v.numpy(), self.geom, heads=heads,
                                       codebook_k=self.codebooks("k"),
                                       codebook_v=self.codebooks("v"))

    # -------------------------------------------------------------------------------- GPU
    def gpu_inputs(self):
        dev = "cuda"
        g = dict(table=torch.from_numpy(self.table).to(dev),
                 u_k=self.u_k.to(dev).contiguous(), u_v=self.u_v.to(dev).contiguous(),
                 clip_k=torch.from_numpy(self.clip_k).to(dev),
                 clip_v=torch.from_numpy(self.clip_v).to(dev),
                 q=self.q.to(dev).contiguous(),
                 lens=torch.tensor(self.lengths, dtype=torch.int32, device=dev),
                 slots=torch.arange(self.batch, dtype=torch.int32, device=dev),
                 levels_k=None if self.levels_k is None else torch.from_numpy(self.levels_k).to(dev),
                 levels_v=None if self.levels_v is None else torch.from_numpy(self.levels_v).to(dev))
        if self.cb_k is not None:
            g["levels_k"] = torch.from_numpy(self.cb_k).to(dev)
            g["levels_v"] = torch.from_numpy(self.cb_v).to(dev)
        return g

    def gpu_cache(self, g, pool_from_oracle=None):
        cache = ok.Cache.allocate(self.layout)
        for b, L in enumerate(self.lengths):
            k = self.k[b].to("cuda")
            v = self.v[b].to("cuda")
            ns = min(L, 64)
            cache.sink_k[b, :, :ns] = k[:ns].transpose(0, 1)
            cache.sink_v[b, :, :ns] = v[:ns].transpose(0, 1)
            if L > 64:
                pos = torch.arange(max(64, L - 256), L, device="cuda")
                cache.recent_k[b][:, pos % 256] = k[pos].transpose(0, 1)
                cache.recent_v[b][:, pos % 256] = v[pos].transpose(0, 1)
        if pool_from_oracle is not None:
            cache.pool.copy_(torch.from_numpy(pool_from_oracle.reshape(cache.pool.shape)))
        else:
            zero = torch.zeros(1, dtype=torch.int32, device="cuda")
            for b, L in enumerate(self.lengths):
                n = max(0, L - 320)
                if n == 0:
                    continue
                k = self.k[b].to("cuda")[64:64 + n].unsqueeze(0)
                v = self.v[b].to("cuda")[64:64 + n].unsqueeze(0)
                ok.demote(self.layout, cache.pool, g["table"][b:b + 1], g["u_k"], g["u_v"],
                          g["clip_k"], g["clip_v"], k, v, zero, levels_k=g["levels_k"],
                          levels_v=g["levels_v"])
        return cache

    def gpu_attention(self, g, cache, max_seq_len=None, with_lse=True):
        mx = max(self.lengths) if max_seq_len is None else max_seq_len
        out = torch.empty((self.batch, self.wl.num_q_heads, 128), dtype=torch.float32,
                          device="cuda")
        lse = torch.empty((self.batch, self.wl.num_q_heads), dtype=torch.float32,
                          device="cuda") if with_lse else None
        ws = torch.empty(ok.decode_workspace_bytes(self.layout, self.batch, mx),
                         dtype=torch.uint8, device="cuda")
        if self.cb_k is not None:
            ok.decode_attn_codebook(self.layout, cache.pool, g["table"], cache.sink_k,
                                    cache.sink_v, cache.recent_k, cache.recent_v, g["slots"],
                                    g["lens"], g["q"], g["u_k"], g["u_v"], g["levels_k"],
                                    g["levels_v"], out, ws, mx, lse=lse)
        else:
            ok.decode_attn(self.layout, cache.pool, g["table"], cache.sink_k, cache.sink_v,
                           cache.recent_k, cache.recent_v, g["slots"], g["lens"], g["q"],
                           g["u_k"], g["u_v"], out, ws, mx, lse=lse)
        torch.cuda.synchronize()
        return out.cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


# ------------------------------------------------------------------------------------ checks

def attention_error(out, ref, rows=None) -> float:
    """max over rows of |out - ref|_inf / |ref|_inf."""
    if rows is None:
        rows = [(b, h) for b in range(ref.shape[0]) for h in range(ref.shape[1])]
    worst = 0.0
    for b, h in rows:
        den = np.max(np.abs(ref[b, h]))
        worst = max(worst, float(np.max(np.abs(out[b, h] - ref[b, h])) / den))
    return worst


def _near_half(t, window=WINDOW):
    t = np.asarray(t, np.float64)
    return np.abs(t - (np.floor(t) + 0.5)) <= window * np.maximum(np.abs(t), 1.0)


def _near_fp16_midpoint(x, window=WINDOW):
    x = np.float64(x)
    h = np.float16(x)
    lo, hi = sorted([float(h), float(np.nextafter(h, np.float16(np.inf if x > float(h) else -np.inf)))])
    mid = 0.5 * (lo + hi)
    return abs(x - mid) <= window * max(abs(x), 1e-30)


def compare_pool_blocks(gpu: np.ndarray, ref: np.ndarray, case: Case, heads=None):
    """Compare GPU pool bytes with the oracle's under the acceptance rule.  Returns the number of
    differing codes (0 when the bytes are identical)."""
    hkv = case.wl.num_kv_heads
    g = case.geom
    gpu = gpu.reshape(case.num_pages, hkv, g.block_bytes)
    ref = ref.reshape(case.num_pages, hkv, g.block_bytes)
    if heads is not None:
        gpu = gpu[:, heads]
        ref = ref[:, heads]
    if np.array_equal(gpu, ref):
        return 0
    # locate every differing (sequence, history index, head, tensor) from the documented layout
    owner = {}
    for b, L in enumerate(case.lengths):
        for p in range(workloads.history_pages(L)):
            owner.setdefault(int(case.table[b, p]), (b, p))
    head_ids = list(range(hkv)) if heads is None else list(heads)
    bad_tokens = set()
    pages, hh, offs = np.nonzero(gpu != ref)
    byte_owner = _byte_owners(g)
    for pg, hi, off in zip(pages, hh, offs):
        b, p = owner[int(pg)]
        h = head_ids[hi]
        slots, tensor = byte_owner[int(off)]
        for s in slots:
            bad_tokens.add((b, p * g.page + s, h, tensor))
    flips = 0
    total_codes = sum(max(0, L - 320) for L in case.lengths) * 2 * len(head_ids) * g.head_dim
    for b, t, h, tensor in sorted(bad_tokens):
        src = case.k[b] if tensor == "k" else case.v[b]
        x = bf16_np(src[64 + t, h])[None]
        u = (case.u_k if tensor == "k" else case.u_v)[h].numpy()
        c = (case.clip_k if tensor == "k" else case.clip_v)[h]
        page = int(case.table[b, t // g.page])
        blk_g = gpu[page][head_ids.index(h)]
        blk_r = ref[page][head_ids.index(h)]
        lv = case.head_levels(tensor, h)
        cb = case.head_codebook(tensor, h)
        rc, _, _ = _token(blk_r, t % g.page, tensor, g)
        assert np.array_equal(rc, case.encode(x, tensor, h)[0][0]), \
            "oracle pool and oracle encode disagree"
        flips += check_token(blk_g, t % g.page, tensor, x, u, c, g, (b, t, h, tensor), lv, cb)
    assert flips <= MAX_FLIP_FRACTION * total_codes, (flips, total_codes)
    return flips


def check_token(blk, slot, tensor, x, u, c, g, where=None, levels=None, codebook=None):
    """Check one token's bytes in a GPU-written block against the oracle's encoding of x (fp32
    [1, d] of the bf16 token; ``levels`` the head's (lo, step) or None; ``codebook`` its four
    levels or None) under the acceptance rule; returns the number of codes that differ (all of
    them inside the rounding window, which for a codebook is around the midpoints of its
    levels)."""
    codes, s16, z16, pre = oracle.encode(x, u, c, g.group, levels)
    if codebook is not None:
        codes = oracle.quantize_codebook(oracle.rotate_to_fp32(x, u), c, g.group, codebook)[0]
        mids = (np.asarray(codebook)[:-1] + np.asarray(codebook)[1:]) / 2
        near = lambda t: np.any(np.abs(np.asarray(t, np.float64)[:, None] - mids) <=
                                WINDOW * np.maximum(np.abs(np.asarray(t))[:, None], 1.0), axis=1)
    else:
        near = _near_half
    gc, gs, gz = _token(blk, slot, tensor, g)
    flips = 0
    for m in range(g.n_groups):
        sl = slice(m * g.group, (m + 1) * g.group)
        same_s = gs[m].view(np.uint16) == s16[0, m].view(np.uint16)
        same_z = gz[m].view(np.uint16) == z16[0, m].view(np.uint16)
        if not same_s:
            assert _near_fp16_midpoint(pre["s"][0, m]), (where, "scale")
        if not same_z:
            assert _near_fp16_midpoint(pre["z"][0, m]), (where, "zero")
        if same_s and same_z:
            diff = gc[sl] != codes[0, sl]
            assert near(pre["t"][0, sl][diff]).all(), (where, "code")
            flips += int(diff.sum())
        else:
            # legitimate meta difference: the GPU codes must be nearest levels under its meta
            xr = np.clip(oracle.rotate(x, u)[0, sl], -c, c)
            grid = np.arange(4) if codebook is None else np.asarray(codebook)
            lv = float(gs[m]) * grid[None, :] + float(gz[m])
            dist = np.abs(xr[:, None] - lv)
            best = np.sort(dist, axis=1)
            chosen = dist[np.arange(g.group), gc[sl]]
            assert (chosen <= best[:, 0] + WINDOW * max(float(gs[m]), 1e-30)).all(), where
            flips += int((gc[sl] != codes[0, sl]).sum())
    return flips


def _byte_owners(g):
    """Block byte offset -> (history slots whose data it holds, tensor), from the oracle's
    layout functions."""
    own = {}
    ng4 = 4 * g.n_groups
    for s in range(g.page):
        for off in oracle.k_code_bytes(s, g):
            own[int(off)] = ([s], "k")
        for off in oracle.v_code_bytes(s, g):
            own.setdefault(int(off), ([], "v"))[0].append(s)
        m0 = g.meta_off + s * g.meta_bytes_per_token
        for off in range(m0, m0 + ng4):
            own[off] = ([s], "k")
        for off in range(m0 + ng4, m0 + 2 * ng4):
            own[off] = ([s], "v")
    return own


def _token(blk, slot, tensor, g):
    ng = g.n_groups
    m0 = g.meta_off + slot * g.meta_bytes_per_token + (0 if tensor == "k" else 4 * ng)
    if tensor == "k":
        row = blk[oracle.k_code_bytes(slot, g)]
        codes = np.stack([(row >> (2 * i)) & 3 for i in range(4)], -1).reshape(-1)
    else:
        byte = blk[oracle.v_code_bytes(slot, g)]
        codes = (byte >> oracle.v_code_shift(slot, g)) & 3
    meta = blk[m0: m0 + 4 * ng]
    m = np.frombuffer(meta.tobytes(), dtype="<f2").reshape(ng, 2)
    return codes.astype(np.uint8), m[:, 0].copy(), m[:, 1].copy()
