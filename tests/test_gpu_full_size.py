"""Full-size GPU parity on sampled outputs, through the C ABI.

Each workload's layer is built at its full size by the library's own bulk demotion, then one
oscar_decode_step (append, demotion of the displaced token, attention) runs in the launch
configuration the benchmark uses.  The oracle then checks, on samples it can compute one by one:
  * demotion: sampled history tokens (and the token demoted by the step) re-encoded by the oracle
    against the GPU's page bytes, under the acceptance rule of oscar_cases;
  * attention: sampled (sequence, KV head) pairs, the oracle's softmax attention over the same
    cache bytes (the GPU-written pool and BF16 segments after the step) against the GPU rows,
    within 2e-3 max row error.
"""
import math

import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import oracle
import workloads
from oscar_cases import ATTN_TOL, MAX_FLIP_FRACTION, attention_error, bf16_np, check_token

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


class FullLayer:
    """One layer of a workload at full size on the GPU after one decode step."""

    def __init__(self, wl, layer=0, u=None, clip=None, lengths=None, levels=None, codebook=None,
                 prefix=False):
        self.wl, self.layer = wl, layer
        self.lengths = list(workloads.context_lengths(wl) if lengths is None else lengths)
        self.B = len(self.lengths)
        hkv = wl.num_kv_heads
        self.table, self.num_pages = workloads.page_tables(wl, self.lengths, layer, spare_tokens=1)
        self.u_k, self.u_v = workloads.rotation_bases(wl, layer) if u is None else u
        if clip is None:
            clip = (np.full(hkv, wl.clip, np.float32), np.full(hkv, wl.clip, np.float32))
        self.clip_k, self.clip_v = (np.asarray(c, np.float32) for c in clip)
        # optional equally spaced codebooks, (lo, step) per KV head for keys and for values
        self.levels = None if levels is None else tuple(np.asarray(x, np.float32) for x in levels)
        # optional symmetric Lloyd-Max codebooks, (l0, l1) per KV head for keys and for values
        # (reading R21); the oracle takes their four levels from the same fp32 values
        assert levels is None or codebook is None
        self.cb = None if codebook is None else tuple(np.asarray(x, np.float32) for x in codebook)
        self.cb4 = None if codebook is None else tuple(
            np.stack([oracle.symmetric_levels(float(a), float(c)) for a, c in x]) for x in self.cb)
        self.geom = oracle.Geometry(group=wl.group_size)
        self.lay = ok.make_layout(wl.num_q_heads, hkv, self.num_pages, self.B,
                                  self.table.shape[1], wl.group_size,
                                  levels_kind=0 if codebook is None else ok.LEVELS_SYMMETRIC)
        dev = "cuda"
        cache = ok.Cache.allocate(self.lay, zero=False)
        table = torch.from_numpy(self.table).to(dev)
        uk, uv = self.u_k.to(dev).contiguous(), self.u_v.to(dev).contiguous()
        ck, cv = torch.from_numpy(self.clip_k).to(dev), torch.from_numpy(self.clip_v).to(dev)
        given = self.levels if self.levels is not None else self.cb
        lk, lv = ((None, None) if given is None else
                  (torch.from_numpy(given[0]).to(dev), torch.from_numpy(given[1]).to(dev)))
        # history: shared-prefix pages once (from the longest sequence), private pages per
        # sequence (including the copies of prefix pages a short sequence will write into)
        n_hist = [max(0, L - 320) for L in self.lengths]
        longest = int(np.argmax(self.lengths))
        for b in range(self.B):
            lo0 = 0 if b == longest else 64 * workloads.shared_pages(wl, self.lengths[b], 1)
            for lo in range(lo0, n_hist[b], 16384):
                n = min(16384, n_hist[b] - lo)
                k, v = workloads.kv_tokens(wl, layer, b, 64 + lo, n, dev)
                ok.demote(self.lay, cache.pool, table[b:b + 1], uk, uv, ck, cv, k.unsqueeze(0),
                          v.unsqueeze(0), torch.full((1,), lo, dtype=torch.int32, device=dev),
                          levels_k=lk, levels_v=lv)
            L = self.lengths[b]
            k, v = workloads.kv_tokens(wl, layer, b, 0, min(L, 64), dev)
            cache.sink_k[b, :, :k.shape[0]] = k.transpose(0, 1)
            cache.sink_v[b, :, :k.shape[0]] = v.transpose(0, 1)
            if L > 64:
                pos = torch.arange(max(64, L - 256), L, device=dev)
                k, v = workloads.kv_tokens(wl, layer, b, int(pos[0]), len(pos), dev)
                cache.recent_k[b][:, pos % 256] = k.transpose(0, 1)
                cache.recent_v[b][:, pos % 256] = v.transpose(0, 1)
        # one decode step: the new token at position L, attention over L + 1 tokens
        kn, vn = zip(*[workloads.kv_tokens(wl, layer, b, L, 1, dev)
                       for b, L in enumerate(self.lengths)])
        self.k_new = torch.cat(kn).contiguous()
        self.v_new = torch.cat(vn).contiguous()
        self.q = workloads.queries(wl, layer, 0, dev, batch=self.B).contiguous()
        pos = torch.tensor(self.lengths, dtype=torch.int32, device=dev)
        slots = torch.arange(self.B, dtype=torch.int32, device=dev)
        mx = max(self.lengths) + 1
        out = torch.empty((self.B, wl.num_q_heads, 128), dtype=torch.float32, device=dev)
        if prefix:
            # the shared prefix handed to the cascade, as the benchmark hands it
            ids, shared = workloads.shared_prefix(wl, self.table, self.lengths, spare_tokens=1)
            ok.check_shared_prefix(self.lay, self.table, ids, shared)
            self.prefix = (torch.from_numpy(ids).to(dev), torch.from_numpy(shared).to(dev))
            ws = torch.zeros(ok.decode_workspace_bytes_prefix(self.lay, self.B, mx, len(ids)),
                             dtype=torch.uint8, device=dev)
            ok.decode_step_prefix(self.lay, cache.pool, table, cache.sink_k, cache.sink_v,
                                  cache.recent_k, cache.recent_v, uk, uv, ck, cv, self.k_new,
                                  self.v_new, slots, pos, self.q, *self.prefix, out, ws, mx)
        else:
            ws = torch.zeros(ok.decode_workspace_bytes(self.lay, self.B, mx), dtype=torch.uint8,
                             device=dev)
            ok.decode_step(self.lay, cache.pool, table, cache.sink_k, cache.sink_v,
                           cache.recent_k, cache.recent_v, uk, uv, ck, cv, self.k_new, self.v_new,
                           slots, pos, self.q, out, ws, mx, levels_k=lk, levels_v=lv)
        torch.cuda.synchronize()
        self.gpu = dict(table=table, uk=uk, uv=uv, slots=slots, mx=mx)
        self.cache = cache
        self.out = out.cpu().numpy()
        self.blocks = cache.pool.view(self.num_pages, hkv, self.geom.block_bytes)

    def token(self, b, position):
        """(k, v) fp32 [Hkv, d] of one position, drawn on the device the layer was built from."""
        k, v = workloads.kv_tokens(self.wl, self.layer, b, position, 1, "cuda")
        return bf16_np(k[0]), bf16_np(v[0])

    def check_demotion(self, samples):
        """samples: (b, history index, kv head) triples; both K and V of each are checked."""
        flips = 0
        for b, t, h in samples:
            k, v = self.token(b, 64 + t)
            blk = self.blocks[int(self.table[b, t // 64]), h].cpu().numpy()
            for i, (tensor, x, u, c) in enumerate((("k", k, self.u_k, self.clip_k),
                                                   ("v", v, self.u_v, self.clip_v))):
                lv = None if self.levels is None else self.levels[i][h]
                cb = None if self.cb4 is None else self.cb4[i][h]
                flips += check_token(blk, t % 64, tensor, x[h][None], u[h].numpy(), c[h],
                                     self.geom, (b, t, h, tensor), lv, cb)
        assert flips <= MAX_FLIP_FRACTION * len(samples) * 2 * 128 + 1, flips
        return flips

    def check_attention(self, b, kv):
        """Oracle attention of sequence b, KV head kv's query heads on the GPU's cache bytes."""
        wl, g = self.wl, self.geom
        L = self.lengths[b] + 1
        n_pages = workloads.history_pages(L)
        ids = torch.from_numpy(self.table[b, :n_pages].astype(np.int64)).cuda()
        pool = self.blocks.index_select(0, ids).cpu().numpy() if n_pages else \
            np.zeros((1, wl.num_kv_heads, g.block_bytes), np.uint8)
        table = np.arange(max(n_pages, 1), dtype=np.int32)[None]
        seg = [bf16_np(t[b:b + 1]) for t in (self.cache.sink_k, self.cache.sink_v,
                                             self.cache.recent_k, self.cache.recent_v)]
        heads = [(0, kv * wl.gqa + i) for i in range(wl.gqa)]
        ref, _ = oracle.decode_attention(pool, table, *seg, [0], [L],
                                         bf16_np(self.q[b:b + 1]), self.u_k.numpy(),
                                         self.u_v.numpy(), g, heads=heads,
                                         codebook_k=None if self.cb4 is None else self.cb4[0],
                                         codebook_v=None if self.cb4 is None else self.cb4[1])
        rows = [(0, h) for _, h in heads]
        err = attention_error(self.out[b:b + 1], ref, rows)
        _note(f"  attention b={b} kv={kv} L={L}: max row error {err:.2e}")
        assert err <= ATTN_TOL
        return err


    def check_head_bytes(self, b, h):
        """Every history token of sequence b and KV head h after the step: the oracle encodes
        them all and writes its own blocks; GPU blocks must match them byte for byte except in
        tokens whose own fields differ, and those must pass the acceptance rule one by one.
        Returns (tokens checked, tokens whose bytes differ)."""
        g, wl = self.geom, self.wl
        n = max(0, self.lengths[b] + 1 - 320)
        n_pages = (n + 63) // 64
        k, v = workloads.kv_tokens(wl, self.layer, b, 64, n, "cuda")
        k, v = bf16_np(k[:, h]), bf16_np(v[:, h])
        enc = []
        for i, (x, u, c) in enumerate(((k, self.u_k, self.clip_k), (v, self.u_v, self.clip_v))):
            cb = None if self.cb4 is None else self.cb4[i][h]
            lv = None if self.levels is None else self.levels[i][h]
            if cb is not None:
                enc.append(oracle.quantize_codebook(oracle.rotate_to_fp32(x, u[h].numpy()), c[h],
                                                    g.group, cb))
            else:
                enc.append(oracle.encode(x, u[h].numpy(), c[h], g.group, lv)[:3])
        row = np.arange(n_pages, dtype=np.int64)
        ref = oracle.new_pool(n_pages, 1, g)
        oracle.store_history(ref, row, np.arange(n), 0, enc[0], enc[1], g)
        ids = torch.from_numpy(self.table[b, :n_pages].astype(np.int64)).cuda()
        got = self.blocks[:, h].index_select(0, ids).cpu().numpy()
        ref = ref[:, 0]
        differ = 0
        for p in np.nonzero((got != ref).any(axis=1))[0]:
            for slot in range(min(64, n - 64 * p)):
                t = 64 * int(p) + slot
                m0 = g.meta_off + slot * g.meta_bytes_per_token
                kb = oracle.k_code_bytes(slot, g)
                vb, vs = oracle.v_code_bytes(slot, g), oracle.v_code_shift(slot, g)
                own = (np.array_equal(got[p, kb], ref[p, kb]) and
                       np.array_equal(got[p, m0:m0 + g.meta_bytes_per_token],
                                      ref[p, m0:m0 + g.meta_bytes_per_token]) and
                       np.array_equal((got[p, vb] >> vs) & 3, (ref[p, vb] >> vs) & 3))
                if own:
                    continue
                differ += 1
                for i, (tensor, x, u, c) in enumerate((("k", k, self.u_k, self.clip_k),
                                                       ("v", v, self.u_v, self.clip_v))):
                    check_token(got[p], slot, tensor, x[t][None], u[h].numpy(), c[h], g,
                                (b, t, h, tensor),
                                None if self.levels is None else self.levels[i][h],
                                None if self.cb4 is None else self.cb4[i][h])
        assert differ <= MAX_FLIP_FRACTION * n * 2 * 128 + 1, differ
        return n, differ


def _samples(rng, layer, count, heads=None):
    """Random (b, history index, kv) triples over the layer's history before the step, plus the
    token each sampled sequence demoted during the step."""
    out = []
    hkv = layer.wl.num_kv_heads
    seqs = [b for b, L in enumerate(layer.lengths) if L > 320]
    for _ in range(count):
        b = int(rng.choice(seqs))
        out.append((b, int(rng.integers(0, layer.lengths[b] - 320)),
                    int(rng.integers(0, hkv)) if heads is None else int(rng.choice(heads))))
    for b in sorted({s[0] for s in out})[:4]:
        out.append((b, layer.lengths[b] - 320, int(rng.integers(0, hkv))))
    return out


def test_full_size_qwen3_8b_100k():
    wl = workloads.get("qwen3_8b_100k")
    _note("qwen3_8b_100k layer 0: building 99,681 history tokens x 8 KV heads")
    layer = FullLayer(wl, layer=0)
    rng = np.random.default_rng(31)
    _note(f"  demotion flips: {layer.check_demotion(_samples(rng, layer, 96))}")
    n, differ = layer.check_head_bytes(0, 2)
    _note(f"  KV head 2: all {n} history tokens' bytes, {differ} tokens inside rounding windows")
    for kv in range(wl.num_kv_heads):     # all 32 query rows
        layer.check_attention(0, kv)


def test_full_size_qwen3_8b_100k_equally_spaced_codebook():
    # layer 1 of the benchmark workload with an equally spaced Lloyd-Max codebook per KV head,
    # fitted by the oracle on the coordinates of the layer's first 2,048 history tokens
    wl = workloads.get("qwen3_8b_100k")
    u_k, u_v = workloads.rotation_bases(wl, 1)
    k, v = workloads.kv_tokens(wl, 1, 0, 64, 2048, "cuda")
    k, v = bf16_np(k), bf16_np(v)
    levels = []
    for x, u in ((k, u_k), (v, u_v)):
        lv = []
        for h in range(wl.num_kv_heads):
            xr = oracle.rotate_to_fp32(x[:, h], u[h].numpy())
            lo, step, _ = oracle.lloyd_max_uniform(
                oracle.codebook_coordinates(xr, wl.clip, wl.group_size), iters=30)
            lv.append((lo, step))
        levels.append(np.array(lv, np.float32))
    _note(f"qwen3_8b_100k layer 1 with codebooks: keys {levels[0][:2].round(3).tolist()}, "
          f"values {levels[1][:2].round(3).tolist()}")
    layer = FullLayer(wl, layer=1, levels=levels)
    rng = np.random.default_rng(35)
    _note(f"  demotion flips: {layer.check_demotion(_samples(rng, layer, 96))}")
    for kv in (1, 6):
        layer.check_attention(0, kv)


def test_full_size_qwen3_8b_100k_symmetric_codebook():
    # layer 2 of the benchmark workload with symmetric Lloyd-Max codebooks per KV head (reading
    # R21), fitted by the oracle on the coordinates of the layer's first 2,048 history tokens;
    # attention through the codebook decode (decode_step on a levels_kind 1 layout)
    wl = workloads.get("qwen3_8b_100k")
    u_k, u_v = workloads.rotation_bases(wl, 2)
    k, v = workloads.kv_tokens(wl, 2, 0, 64, 2048, "cuda")
    k, v = bf16_np(k), bf16_np(v)
    cbs = []
    for x, u in ((k, u_k), (v, u_v)):
        cb = []
        for h in range(wl.num_kv_heads):
            xr = oracle.rotate_to_fp32(x[:, h], u[h].numpy())
            lv = oracle.lloyd_max_symmetric(
                oracle.codebook_coordinates(xr, wl.clip, wl.group_size), iters=30)[0]
            cb.append((lv[0], lv[1]))
        cbs.append(np.array(cb, np.float32))
    _note(f"qwen3_8b_100k layer 2 with symmetric codebooks: keys {cbs[0][:2].round(3).tolist()}, "
          f"values {cbs[1][:2].round(3).tolist()}")
    layer = FullLayer(wl, layer=2, codebook=cbs)
    rng = np.random.default_rng(36)
    _note(f"  demotion flips: {layer.check_demotion(_samples(rng, layer, 96))}")
    n, differ = layer.check_head_bytes(0, 4)
    _note(f"  KV head 4: all {n} history tokens' bytes, {differ} tokens inside rounding windows")
    for kv in range(wl.num_kv_heads):
        layer.check_attention(0, kv)


def test_full_size_qwen3_8b_b64_shared_prefix():
    # the step runs with the shared-prefix cascade (the benchmark times it beside the plain
    # step); the plain attention over the cache the step left must agree with it to the fp8
    # parts' resolution and fp32 summation order (1e-4 of each row's largest output: pages pair
    # up from other starting pages in the two paths), and sampled rows must agree with the oracle
    wl = workloads.get("qwen3_8b_b64_prefix")
    layer = FullLayer(wl, layer=0, prefix=True)
    lens = layer.lengths
    _note(f"qwen3_8b_b64_prefix: 64 sequences, lengths {min(lens)}..{max(lens)}, prefix "
          f"{layer.prefix[0].numel()} pages")
    rng = np.random.default_rng(32)
    _note(f"  demotion flips: {layer.check_demotion(_samples(rng, layer, 96))}")
    c, gi = layer.cache, layer.gpu
    plain = torch.empty((layer.B, wl.num_q_heads, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(ok.decode_workspace_bytes(layer.lay, layer.B, gi["mx"]), dtype=torch.uint8,
                     device="cuda")
    lens1 = torch.tensor(lens, dtype=torch.int32, device="cuda") + 1
    ok.decode_attn(layer.lay, c.pool, gi["table"], c.sink_k, c.sink_v, c.recent_k, c.recent_v,
                   gi["slots"], lens1, layer.q, gi["uk"], gi["uv"], plain, ws, gi["mx"])
    torch.cuda.synchronize()
    plain = plain.cpu().numpy()
    scale = np.maximum(np.abs(plain).max(axis=-1, keepdims=True), 1e-30)
    d = float(np.max(np.abs(layer.out - plain) / scale))
    _note(f"  cascade step vs plain attention: {d:.2e}")
    assert d <= 1e-4
    order = np.argsort(lens)
    for b, kv in ((int(order[-1]), 3), (int(order[0]), 6), (int(order[32]), 0)):
        layer.check_attention(b, kv)


def test_full_size_qwen3_32b_131k_gqa8_group64():
    wl = workloads.get("qwen3_32b_131k")
    u = workloads.rotation_bases(wl, 0)
    # calibrated clip: 99.9th percentile of |x R| over the first clip_calib_tokens positions
    k, v = workloads.kv_tokens(wl, 0, 0, 0, wl.clip_calib_tokens, "cuda")
    k, v = bf16_np(k), bf16_np(v)
    clip_k = np.array([oracle.clip_threshold(k[:, h], u[0][h].numpy())
                       for h in range(wl.num_kv_heads)], np.float32)
    clip_v = np.array([oracle.clip_threshold(v[:, h], u[1][h].numpy())
                       for h in range(wl.num_kv_heads)], np.float32)
    _note(f"qwen3_32b_131k: 16 x 130,752 history tokens, clip_k {clip_k.round(2).tolist()}")
    layer = FullLayer(wl, layer=0, u=u, clip=(clip_k, clip_v))
    rng = np.random.default_rng(33)
    _note(f"  demotion flips: {layer.check_demotion(_samples(rng, layer, 96))}")
    for b, kv in ((0, 2), (15, 7)):
        layer.check_attention(b, kv)


def test_full_size_qwen3_4b_32k_calibrated():
    # KV head 0 is calibrated by the oracle (U_k, U_v from the calibration queries of its query
    # heads over the layer's own context, clip = 99.9th percentile); the other heads keep seeded
    # orthogonal bases and clip 4.0 (they only fill the launch).
    wl = workloads.get("qwen3_4b_32k")
    hkv, gq = wl.num_kv_heads, wl.gqa
    qr = workloads.rotation_bases(workloads.scaled(wl, rotation="qr"), 0)
    u_k, u_v = qr[0].clone(), qr[1].clone()
    clip_k = np.full(hkv, 4.0, np.float32)
    clip_v = np.full(hkv, 4.0, np.float32)
    q_cal = workloads.calibration_queries(wl, 0).double().numpy()[:, :gq].reshape(-1, 128)
    k, v = workloads.kv_tokens(wl, 0, 0, 0, wl.context, "cuda")
    k0, v0 = bf16_np(k[:, 0]), bf16_np(v[:, 0])
    uk0 = oracle.key_rotation(q_cal)
    uv0 = oracle.value_rotation(q_cal, k0, v0, 1.0 / math.sqrt(128))
    u_k[0] = torch.from_numpy(uk0.astype(np.float32))
    u_v[0] = torch.from_numpy(uv0.astype(np.float32))
    clip_k[0] = oracle.clip_threshold(k0, u_k[0].numpy())
    clip_v[0] = oracle.clip_threshold(v0, u_v[0].numpy())
    _note(f"qwen3_4b_32k: calibrated KV head 0, clip ({clip_k[0]:.3f}, {clip_v[0]:.3f})")
    layer = FullLayer(wl, layer=0, u=(u_k, u_v), clip=(clip_k, clip_v))
    rng = np.random.default_rng(34)
    _note(f"  demotion flips: {layer.check_demotion(_samples(rng, layer, 96, heads=[0]))}")
    for kv in (0, 5):
        layer.check_attention(0, kv)
