"""Plain CPU reference ("oracle") for the OSCAR INT2-history decode path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this module.  The HIP library never does, and this module imports nothing
from it: the two share no code.  Every function here is slow, vectorised numpy written to be
checked against the pages by eye; floating point is fp64 except where a float decides an integer
code (see ``quantize``), where the oracle takes the decision in the precision the kernels use
(fp32), on values first computed in fp64.

Sources (web pages on OSCAR; cited by the short keys below):
  [W1] "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化" (66bd.net, article 13430)
  [W3] the repost of the same write-up on m.kljzs.com (untitled page; it keeps the evaluation part)
  [P]  "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization",
       ModelScope paper page of arXiv 2605.17757 (Chinese summary "摘要" and "Abstract")

What the path computes, in the pages' terms:
  * the KV pool of a sequence has three segments: a BF16 attention sink of 64 tokens, a rotated
    INT2 history, and a BF16 window of the 256 most recent tokens ([W1] §OSCAR 的设计);
  * a history key or value x is stored as the codes of x' = x R with R = U · Hadamard ·
    bit-reversal, one R per layer and head for keys and one for values ([W1] §OSCAR 的设计), after
    clipping to a calibrated threshold and asymmetric INT2 quantisation with a scale and a zero
    point, four 2-bit codes to a byte ([W1] §OSCAR 的设计; [P] 摘要);
  * a new token goes into the recent window; the oldest recent token is then rotated, clipped,
    quantised, packed and moved into the history ([W1] §OSCAR 的设计);
  * decode attention treats the BF16 segments and the INT2 segment separately and combines the two
    with an online-softmax merge; the result is ordinary softmax attention over the whole cache
    ([W1] §OSCAR 的设计).

Readings taken where the pages are silent:
  R1  x' = x R for a row vector x (U first, then the Hadamard, then the permutation).
  R2  Hadamard in Sylvester order, scaled by 1/sqrt(d); bit-reversal reverses the log2(d)-bit
      channel index, P[i, j] = 1 iff i = rev(j).
  R3  clip is symmetric, |x'| <= c, per (layer, KV head, K|V), applied after rotation.
  R4  groups run along the rotated channels of one token: channels [m g, (m+1) g).
  R5  zero point = group minimum, scale = (max - min) / 3; both stored as fp16 (round to nearest
      even); codes use the stored fp16 values: code = clamp(rint((x'' - z) / s), 0, 3) with ties to
      even; a group whose fp16 scale is 0 stores all-zero codes.
  R6  the float steps that decide codes (rotated value to fp32, clip, min/max, range, /3, fp16
      rounding, (x - z)/s) run in IEEE fp32, the kernels' precision; the rotation itself is fp64.
  R7  pack order: code of element 4b+i sits in bits [2i, 2i+1] of byte b (LSB first).
  R8  page layout (one block per page and KV head, 64 tokens): key codes packed along channels,
      value codes packed along tokens, then per token the fp16 (scale, zero) pairs of its key
      groups followed by those of its value groups.  At the kernels' geometry (128 channels,
      64-token pages) the 4-byte words of 16 codes are stored in a tiled order, one 16-byte chunk
      per lane of a 64-lane wave (see ``k_word_index`` / ``v_word_index``); smaller test
      geometries keep plain row order.
  R9  order within a decode step: append the new token, demote the token that leaves the recent
      window, then attend; the recent window holds the last min(256, L-64) tokens.
  R10 attention: scores scaled by 1/sqrt(d), no mask, query head i uses KV head i // G.
  R11 calibration: U_k = eigenvectors of the summed Q^T Q of the KV head's query heads; U_v =
      eigenvectors of (S V)^T (S V) with S = softmax(Q K^T / sqrt(d)) ([W1] §OSCAR 的设计 names the
      two covariances); eigenvectors in descending eigenvalue order, each column's largest-magnitude
      entry made positive; clip = a percentile of |x R|.
  R19 a Lloyd-Max codebook keeps R5's scale and zero and replaces the grid {0, 1, 2, 3} by four
      levels fitted by Lloyd's algorithm (``lloyd_max``); codes name the nearest level (a value
      halfway takes the lower code) and decode to s * level + z (``quantize_codebook``,
      ``dequantize_codebook``; ``demote`` / ``append`` / ``decode_attention`` take per-KV-head
      levels as ``codebook_k`` / ``codebook_v``).
  R20 the Lloyd-Max codebook restricted to equally spaced levels lo + step * c in the same
      coordinate (``lloyd_max_uniform``): the same as storing scale' = s * step and zero' =
      z + s * lo with R5's codes, so it runs on the GPU path unchanged past the encoder
      (``quantize(..., levels=(lo, step))``).
  R21 the Lloyd-Max codebook restricted to levels symmetric about 1.5, (l0, l1, 3 - l1, 3 - l0)
      (``lloyd_max_symmetric``, ``symmetric_levels``): the codebooks the GPU path decodes, since
      such levels are a + b c + d (c >> 1) in the code's bits.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# ----------------------------------------------------------------------------------------------
# geometry

@dataclasses.dataclass(frozen=True)
class Geometry:
    """Cache geometry.  The pages fix sink = 64 and recent = 256 ([W1] §OSCAR 的设计); page = 64
    tokens is the library's paged-KV block.  Smaller values serve brute-force tests."""

    head_dim: int = 128
    group: int = 128
    page: int = 64
    sink: int = 64
    recent: int = 256

    @property
    def n_groups(self) -> int:
        return self.head_dim // self.group

    # byte offsets inside one (page, KV head) block (reading R8)
    @property
    def k_codes_off(self) -> int:
        return 0

    @property
    def v_codes_off(self) -> int:
        return self.page * self.head_dim // 4

    @property
    def meta_off(self) -> int:
        return self.v_codes_off + self.head_dim * self.page // 4

    @property
    def meta_bytes_per_token(self) -> int:
        return 2 * self.n_groups * 4

    @property
    def block_bytes(self) -> int:
        return self.meta_off + self.page * self.meta_bytes_per_token

    @property
    def tiled(self) -> bool:
        return self.head_dim == 128 and self.page == 64


# ----------------------------------------------------------------------------------------------
# rotation R = U · Hadamard · bit-reversal   ([W1] §OSCAR 的设计; [W3] same design paragraph)

def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two): H[i, j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("order must be a power of two")
    idx = np.arange(d)
    both = np.bitwise_and.outer(idx, idx)
    parity = np.zeros_like(both)
    while both.any():
        parity ^= both & 1
        both = both >> 1
    return np.where(parity == 0, 1.0, -1.0)


def bit_reverse(j, d: int):
    """Reverse the log2(d) low bits of channel index j (reading R2)."""
    nbits = int(round(math.log2(d)))
    j = np.asarray(j)
    out = np.zeros_like(j)
    for b in range(nbits):
        out = out | (((j >> b) & 1) << (nbits - 1 - b))
    return out


def bit_reversal_matrix(d: int) -> np.ndarray:
    """Permutation matrix P with P[i, j] = 1 iff i = rev(j), so (x P)_j = x_rev(j)."""
    p = np.zeros((d, d))
    j = np.arange(d)
    p[bit_reverse(j, d), j] = 1.0
    return p


def rotation_matrix(u) -> np.ndarray:
    """R = U (H / sqrt(d)) P in fp64, from the fp32 U the kernels receive (reading R1, R2)."""
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    return u @ (hadamard(d) / math.sqrt(d)) @ bit_reversal_matrix(d)


# ----------------------------------------------------------------------------------------------
# quantisation ([W1] §OSCAR 的设计: clip, asymmetric scale / zero point, 4 codes per byte)

def rotate(x, u) -> np.ndarray:
    """x' = x R in fp64 (reading R1).  x: (..., d)."""
    return np.asarray(x, dtype=np.float64) @ rotation_matrix(u)


def unrotate(xr, u) -> np.ndarray:
    """x = x' R^T in fp64: R is orthogonal, so this undoes ``rotate``."""
    return np.asarray(xr, dtype=np.float64) @ rotation_matrix(u).T


def rotate_to_fp32(x, u) -> np.ndarray:
    """x' = x R computed in fp64 and rounded once to fp32 (reading R6).  x: (..., d)."""
    return rotate(x, u).astype(np.float32)


def quantize(xr, clip, group: int, levels=None):
    """Clip and quantise rotated vectors xr (..., d) (fp32) group by group (readings R3-R6).

    ``levels`` = (lo, step) selects an equally spaced codebook (reading R20): the stored scale
    and zero point become fp16((max-min)/3 * step) and fp16(min + (max-min)/3 * lo), each product
    and sum rounded to fp32 on its own; None, or (0, 1), is the uniform grid of R5.
    Returns (codes uint8 (..., d), scale fp16 (..., d/g), zero fp16 (..., d/g), pre) where
    ``pre`` holds the values just before each rounding step, for acceptance windows:
    pre["t"] fp32 (..., d) is (x'' - z) / s before rint, pre["s"] fp32 is the scale before the
    fp16 rounding ((max-min)/3 on the uniform grid) and pre["z"] fp32 the zero point before it
    (the group minimum on the uniform grid).
    """
    x = np.asarray(xr, dtype=np.float32)
    c = np.float32(clip)
    xc = np.minimum(np.maximum(x, -c), c)
    d = x.shape[-1]
    xg = xc.reshape(x.shape[:-1] + (d // group, group))
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    s32 = (mx - mn) / np.float32(3.0)
    lo, step = (0.0, 1.0) if levels is None else (float(levels[0]), float(levels[1]))
    z32 = mn if lo == 0.0 else mn + s32 * np.float32(lo)
    if step != 1.0:
        s32 = s32 * np.float32(step)
    s16 = s32.astype(np.float16)
    z16 = z32.astype(np.float16)
    sf = s16.astype(np.float32)[..., None]
    zf = z16.astype(np.float32)[..., None]
    safe = np.where(sf == 0, np.float32(1.0), sf)
    t = (xg - zf) / safe
    codes = np.clip(np.rint(t), 0, 3)
    codes = np.where(sf == 0, 0, codes).astype(np.uint8).reshape(x.shape)
    pre = {"t": np.where(sf == 0, np.float32(0), t).reshape(x.shape), "s": s32, "z": z32}
    return codes, s16, z16, pre


def dequantize(codes, scale, zero, group: int) -> np.ndarray:
    """Rotated-space values s * code + z in fp64, (..., d)."""
    c = np.asarray(codes, dtype=np.float64)
    d = c.shape[-1]
    cg = c.reshape(c.shape[:-1] + (d // group, group))
    s = np.asarray(scale, dtype=np.float64)[..., None]
    z = np.asarray(zero, dtype=np.float64)[..., None]
    return (s * cg + z).reshape(c.shape)


def encode(x, u, clip, group: int, levels=None):
    """Rotate, clip and quantise vectors x (..., d): the demotion step on values."""
    return quantize(rotate_to_fp32(x, u), clip, group, levels)


# ----------------------------------------------------------------------------------------------
# packing (4 codes per byte; reading R7)

def pack_codes(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    n = c.shape[-1]
    c4 = c.reshape(c.shape[:-1] + (n // 4, 4))
    return (c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    parts = [(p >> (2 * i)) & 3 for i in range(4)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 4,)).astype(np.uint8)


# ----------------------------------------------------------------------------------------------
# paged pool (reading R8)

def new_pool(num_pages: int, num_kv_heads: int, geom: Geometry) -> np.ndarray:
    return np.zeros((num_pages, num_kv_heads, geom.block_bytes), dtype=np.uint8)


def k_word_index(t, w):
    """Word position of key codes (token t, channels 16w .. 16w+15) in the tiled order of a
    64-token, 128-channel block (reading R8).  With t = 16 st + n and w = 4 hf + q, the word is
    entry 2 (st mod 2) + hf of the 16-byte chunk of lane 16 q + n in 1 KiB chunk row st // 2."""
    t = np.asarray(t)
    w = np.asarray(w)
    st, n = t // 16, t % 16
    hf, q = w // 4, w % 4
    return ((st // 2) * 64 + 16 * q + n) * 4 + (st % 2) * 2 + hf


def v_word_index(c, u):
    """Word position of the value-code word (channel c, token group u) in the tiled order (reading
    R8).  With c = 16 nt + n, the word is entry nt mod 4 of the 16-byte chunk of lane 16 u + n in
    1 KiB chunk row nt // 4."""
    c = np.asarray(c)
    u = np.asarray(u)
    nt, n = c // 16, c % 16
    return ((nt // 4) * 64 + 16 * u + n) * 4 + nt % 4


def v_code_pos(slot: int):
    """(token group u, code position 0..15 in the word) of token `slot`'s value codes in the tiled
    order (reading R8).  With slot = 16 s + 4 u + j, the word of group u holds the 16 tokens
    16 s' + 4 u + j' (every 16-token tile s', four consecutive tokens of each), the code of
    (s, j) at position 8 (j // 2) + 2 s + (j mod 2)."""
    s, n = slot // 16, slot % 16
    u, j = n // 4, n % 4
    return u, 8 * (j // 2) + 2 * s + (j % 2)


def k_code_bytes(slot: int, geom: Geometry) -> np.ndarray:
    """Byte offsets (within the block) of the d/4 packed key-code bytes of one token, in channel
    order: byte j holds channels 4j .. 4j+3."""
    j = np.arange(geom.head_dim // 4)
    if geom.tiled:
        return geom.k_codes_off + 4 * k_word_index(slot, j // 4) + j % 4
    return geom.k_codes_off + slot * geom.head_dim // 4 + j


def v_code_bytes(slot: int, geom: Geometry) -> np.ndarray:
    """Byte offset, per channel, of the packed value-code byte that holds token `slot`'s code (at
    bits v_code_shift(slot))."""
    c = np.arange(geom.head_dim)
    if geom.tiled:
        u, pos = v_code_pos(slot)
        return geom.v_codes_off + 4 * v_word_index(c, u) + pos // 4
    return geom.v_codes_off + c * (geom.page // 4) + slot // 4


def v_code_shift(slot: int, geom: Geometry) -> int:
    """Bit offset of token `slot`'s value code inside its byte (see v_code_bytes)."""
    if geom.tiled:
        return 2 * (v_code_pos(slot)[1] % 4)
    return 2 * (slot % 4)


def _meta_bytes(scale16, zero16) -> np.ndarray:
    """(n, G) fp16 scale and zero -> (n, G*4) bytes: per group the scale's two bytes, then the
    zero's, little endian."""
    s = np.asarray(scale16, dtype=np.float16).view(np.uint16)
    z = np.asarray(zero16, dtype=np.float16).view(np.uint16)
    pair = np.stack([s, z], axis=-1).astype("<u2")
    return pair.reshape(pair.shape[0], -1).view(np.uint8).reshape(pair.shape[0], -1)


def store_history(pool, table_row, hist_idx, head, kq, vq, geom: Geometry):
    """Write encoded tokens into the pool.

    hist_idx (n,) history indices; kq / vq = (codes (n,d), scale (n,G), zero (n,G)).  Token with
    history index t lives in page table_row[t // page], slot t % page.
    """
    hist_idx = np.asarray(hist_idx)
    kc, ks, kz = kq
    vc, vs, vz = vq
    pg = geom.page
    kmeta = _meta_bytes(ks, kz)
    vmeta = _meta_bytes(vs, vz)
    kpacked = pack_codes(kc)
    msz = geom.n_groups * 4
    for n, t in enumerate(hist_idx):
        blk = pool[table_row[t // pg], head]
        slot = int(t % pg)
        blk[k_code_bytes(slot, geom)] = kpacked[n]
        # value codes: channel j's codes for the page's tokens are packed along tokens
        byte = v_code_bytes(slot, geom)
        shift = v_code_shift(slot, geom)
        blk[byte] = (blk[byte] & np.uint8(~(3 << shift) & 0xFF)) | (vc[n].astype(np.uint8) << shift)
        m0 = geom.meta_off + slot * geom.meta_bytes_per_token
        blk[m0: m0 + msz] = kmeta[n]
        blk[m0 + msz: m0 + 2 * msz] = vmeta[n]


def load_history(pool, table_row, n_hist: int, head, geom: Geometry):
    """Read history tokens [0, n_hist) of one sequence and KV head back from the pool.

    Returns ((k codes, k scale, k zero), (v codes, v scale, v zero)) with codes (n, d) and
    scale / zero fp16 (n, G)."""
    d, pg, ng = geom.head_dim, geom.page, geom.n_groups
    kc = np.zeros((n_hist, d), np.uint8)
    vc = np.zeros((n_hist, d), np.uint8)
    ks = np.zeros((n_hist, ng), np.float16)
    kz = np.zeros_like(ks)
    vs = np.zeros_like(ks)
    vz = np.zeros_like(ks)
    msz = ng * 4
    for t in range(n_hist):
        blk = pool[table_row[t // pg], head]
        slot = t % pg
        kc[t] = unpack_codes(blk[k_code_bytes(slot, geom)])
        vc[t] = (blk[v_code_bytes(slot, geom)] >> v_code_shift(slot, geom)) & 3
        m0 = geom.meta_off + slot * geom.meta_bytes_per_token
        km = blk[m0: m0 + msz].view("<f2").reshape(ng, 2)
        vm = blk[m0 + msz: m0 + 2 * msz].view("<f2").reshape(ng, 2)
        ks[t], kz[t] = km[:, 0], km[:, 1]
        vs[t], vz[t] = vm[:, 0], vm[:, 1]
    return (kc, ks, kz), (vc, vs, vz)


# ----------------------------------------------------------------------------------------------
# the demotion step and the decode-step write ([W1] §OSCAR 的设计; reading R9)

def demote(pool, page_table, u_k, u_v, clip_k, clip_v, k_src, v_src, hist_start,
           geom: Geometry, levels_k=None, levels_v=None, codebook_k=None, codebook_v=None):
    """Encode tokens k_src / v_src (B, n, Hkv, d) and store them at history indices
    hist_start[b] + i.  levels_k / levels_v: None (uniform grid) or (lo, step) per KV head
    (reading R20); codebook_k / codebook_v: None or four sorted levels per KV head (reading R19),
    exclusive with levels.  Modifies ``pool`` in place."""
    k_src = np.asarray(k_src, dtype=np.float64)
    v_src = np.asarray(v_src, dtype=np.float64)
    bsz, n, hkv, _ = k_src.shape

    def enc(x, u, clip, lv, cb):
        if cb is not None:
            return quantize_codebook(rotate_to_fp32(x, u), clip, geom.group, cb)
        return encode(x, u, clip, geom.group, lv)[:3]

    for b in range(bsz):
        idx = int(hist_start[b]) + np.arange(n)
        for h in range(hkv):
            kq = enc(k_src[b, :, h], u_k[h], clip_k[h], None if levels_k is None else levels_k[h],
                     None if codebook_k is None else codebook_k[h])
            vq = enc(v_src[b, :, h], u_v[h], clip_v[h], None if levels_v is None else levels_v[h],
                     None if codebook_v is None else codebook_v[h])
            store_history(pool, page_table[b], idx, h, kq, vq, geom)


def append(pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k, u_v, clip_k, clip_v,
           k_new, v_new, seq_slot, seq_lens, geom: Geometry, levels_k=None, levels_v=None,
           codebook_k=None, codebook_v=None):
    """One decode-step write (reading R9).  seq_lens[b] is the length before the append, i.e. the
    position P of the new token.  P < sink: the token goes to the sink.  Otherwise it goes to
    recent-window ring slot P % recent, and when P >= sink + recent the token it replaces
    (position P - recent) is first demoted to history index P - sink - recent.  Modifies the
    arrays in place."""
    for b in range(len(seq_lens)):
        pos = int(seq_lens[b])
        slot = int(seq_slot[b])
        if pos < geom.sink:
            sink_k[slot, :, pos] = k_new[b]
            sink_v[slot, :, pos] = v_new[b]
            continue
        r = pos % geom.recent
        if pos >= geom.sink + geom.recent:
            old_k = np.asarray(recent_k[slot, :, r], dtype=np.float64)[None, None]
            old_v = np.asarray(recent_v[slot, :, r], dtype=np.float64)[None, None]
            demote(pool, page_table[b:b + 1], u_k, u_v, clip_k, clip_v, old_k, old_v,
                   [pos - geom.sink - geom.recent], geom, levels_k, levels_v, codebook_k,
                   codebook_v)
        recent_k[slot, :, r] = k_new[b]
        recent_v[slot, :, r] = v_new[b]


# ----------------------------------------------------------------------------------------------
# decode attention ([W1] §OSCAR 的设计; readings R9, R10)

def segment_lengths(length: int, geom: Geometry):
    """(sink tokens, history tokens, recent tokens) of a context of ``length`` tokens."""
    n_sink = min(length, geom.sink)
    n_recent = min(geom.recent, max(0, length - geom.sink))
    n_hist = max(0, length - geom.sink - geom.recent)
    return n_sink, n_hist, n_recent


def recent_slots(length: int, geom: Geometry) -> np.ndarray:
    """Ring slots of the recent window: positions max(sink, L - recent) .. L-1, modulo recent."""
    start = max(geom.sink, length - geom.recent)
    return np.arange(start, length) % geom.recent


def gather_cache(pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k, u_v, slot, b, kv,
                 length: int, geom: Geometry, codebook_k=None, codebook_v=None):
    """All cached keys and values of one (sequence, KV head) in fp64, unrotated: sink tokens,
    then history tokens dequantised in rotated space and mapped back by R^T, then recent tokens.
    codebook_k / codebook_v: None (codes are the uniform grid) or four levels per KV head (R19)."""
    n_sink, n_hist, _ = segment_lengths(length, geom)
    ks = [np.asarray(sink_k[slot, kv, :n_sink], dtype=np.float64)]
    vs = [np.asarray(sink_v[slot, kv, :n_sink], dtype=np.float64)]
    if n_hist:
        (kc, kS, kZ), (vc, vS, vZ) = load_history(pool, page_table[b], n_hist, kv, geom)

        def deq(c, sc, z, cb):
            if cb is None:
                return dequantize(c, sc, z, geom.group)
            return dequantize_codebook(c, sc, z, geom.group, cb[kv])

        ks.append(unrotate(deq(kc, kS, kZ, codebook_k), u_k[kv]))
        vs.append(unrotate(deq(vc, vS, vZ, codebook_v), u_v[kv]))
    rs = recent_slots(length, geom)
    ks.append(np.asarray(recent_k[slot, kv, rs], dtype=np.float64))
    vs.append(np.asarray(recent_v[slot, kv, rs], dtype=np.float64))
    return np.concatenate(ks, 0), np.concatenate(vs, 0)


def attend(q, keys, values, sm_scale: float):
    """Softmax attention of one query over keys/values (n, d), fp64.  Returns (out (d,), lse)."""
    s = (np.asarray(keys, np.float64) @ np.asarray(q, np.float64)) * sm_scale
    m = s.max()
    w = np.exp(s - m)
    tot = w.sum()
    return (w @ np.asarray(values, np.float64)) / tot, m + math.log(tot)


def decode_attention(pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot, seq_lens,
                     q, u_k, u_v, geom: Geometry, sm_scale=None, heads=None, codebook_k=None,
                     codebook_v=None):
    """Decode attention of q (B, Hq, d) over each sequence's three-segment cache.

    Returns (out fp64 (B, Hq, d), lse fp64 (B, Hq)); ``heads`` optionally restricts the work to a
    list of (b, q_head) pairs (other rows stay NaN); codebook_k / codebook_v as for
    ``gather_cache``."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = np.asarray(u_k).shape[0]
    gqa = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    out = np.full((bsz, hq, d), np.nan)
    lse = np.full((bsz, hq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(bsz) for h in range(hq)]
    cache = {}
    for b, h in todo:
        kv = h // gqa
        if (b, kv) not in cache:
            cache = {(b, kv): gather_cache(pool, page_table, sink_k, sink_v, recent_k, recent_v,
                                           u_k, u_v, int(seq_slot[b]), b, kv, int(seq_lens[b]),
                                           geom, codebook_k, codebook_v)}
        keys, values = cache[(b, kv)]
        out[b, h], lse[b, h] = attend(q[b, h], keys, values, sm_scale)
    return out, lse


# ----------------------------------------------------------------------------------------------
# online-softmax partials and their merge ([W1] §OSCAR 的设计: BF16 and INT2 parts are combined by
# an online-softmax merge)

def softmax_partial(q, keys, values, sm_scale: float):
    """(m, l, acc) of one segment: m = max score, l = sum exp(s - m), acc = sum exp(s - m) v."""
    s = (np.asarray(keys, np.float64) @ np.asarray(q, np.float64)) * sm_scale
    if s.size == 0:
        return -np.inf, 0.0, np.zeros(np.asarray(values).shape[-1])
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ np.asarray(values, np.float64)


def merge_partials(parts):
    """Merge (m, l, acc) partials of disjoint segments into one (m, l, acc)."""
    m = max(p[0] for p in parts)
    if m == -np.inf:
        return m, 0.0, np.zeros_like(parts[0][2])
    l = sum(p[1] * math.exp(p[0] - m) for p in parts if p[1] > 0)
    acc = sum(p[2] * math.exp(p[0] - m) for p in parts if p[1] > 0)
    return m, l, acc


# ----------------------------------------------------------------------------------------------
# paged BF16 baseline ([W1] and [W3], evaluation part, and [P] Abstract state the INT2 history's
# memory and decode-speed gains against a history kept in BF16).  The layout is this project's
# own (include/oscar.h): one block per (page, KV head) of 64 tokens holds every key and value
# element of those tokens, 32 rows of 64 chunks of 8 bf16 elements; the token at position t of a
# sequence lives in page table_row[t // 64], slot t % 64.  Values are bf16 bit patterns.

def bf16_key_index(slot, c):
    """Element index (in bf16 units) of key channel c of page slot ``slot`` inside a block."""
    row = 16 * (slot // 32) + 4 * ((slot // 16) % 2) + c // 32
    chunk = 16 * ((c % 32) // 8) + slot % 16
    return row * 512 + chunk * 8 + c % 8


def bf16_value_index(slot, c):
    """Element index (in bf16 units) of value channel c of page slot ``slot`` inside a block."""
    row = 16 * (slot // 32) + 8 + c // 16
    chunk = 16 * ((slot % 32) // 8) + c % 16
    return row * 512 + chunk * 8 + slot % 8


def bf16_new_pool(num_pages: int, num_kv_heads: int, d: int = 128, page: int = 64,
                  fill: int = 0) -> np.ndarray:
    """uint16 [num_pages, num_kv_heads, 2 * page * d], every element set to ``fill``."""
    return np.full((num_pages, num_kv_heads, 2 * page * d), fill, dtype=np.uint16)


def bf16_store(pool, table_row, pos: int, head: int, k_bits, v_bits, page: int = 64) -> None:
    """Write one token's key and value (uint16 bit patterns, length 128) at position ``pos``."""
    c = np.arange(len(k_bits))
    blk = pool[int(table_row[pos // page]), head]
    slot = pos % page
    blk[bf16_key_index(slot, c)] = k_bits
    blk[bf16_value_index(slot, c)] = v_bits


def bf16_gather(pool, table_row, length: int, head: int, d: int = 128, page: int = 64):
    """Keys and values (length, d) of positions 0 .. length-1, as uint16 bit patterns."""
    keys = np.empty((length, d), dtype=np.uint16)
    values = np.empty((length, d), dtype=np.uint16)
    c = np.arange(d)
    for t in range(length):
        blk = pool[int(table_row[t // page]), head]
        keys[t] = blk[bf16_key_index(t % page, c)]
        values[t] = blk[bf16_value_index(t % page, c)]
    return keys, values


def bf16_bits_to_float(bits) -> np.ndarray:
    """bf16 bit patterns -> fp64 values (a bf16 is the upper half of an IEEE binary32)."""
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# offline calibration ([W1] §OSCAR 的设计 and figure 2, left side; [P] 摘要; reading R11)

def _sorted_eigenvectors(c: np.ndarray) -> np.ndarray:
    w, v = np.linalg.eigh(c)
    order = np.argsort(w)[::-1]
    v = v[:, order]
    pick = np.argmax(np.abs(v), axis=0)
    sign = np.sign(v[pick, np.arange(v.shape[1])])
    return v * sign[None, :]


def key_covariance(q_cal) -> np.ndarray:
    """Q^T Q over calibration queries q_cal (n, d) (all query heads of one KV head stacked)."""
    q = np.asarray(q_cal, dtype=np.float64)
    return q.T @ q


def value_covariance(q_cal, keys, values, sm_scale: float, chunk: int = 512) -> np.ndarray:
    """(S V)^T (S V) with S = softmax(Q K^T * sm_scale) row-wise, over calibration queries."""
    q = np.asarray(q_cal, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    c = np.zeros((v.shape[1], v.shape[1]))
    for i in range(0, q.shape[0], chunk):
        s = (q[i:i + chunk] @ k.T) * sm_scale
        s = np.exp(s - s.max(axis=1, keepdims=True))
        s /= s.sum(axis=1, keepdims=True)
        sv = s @ v
        c += sv.T @ sv
    return c


def key_rotation(q_cal) -> np.ndarray:
    return _sorted_eigenvectors(key_covariance(q_cal))


def value_rotation(q_cal, keys, values, sm_scale: float) -> np.ndarray:
    return _sorted_eigenvectors(value_covariance(q_cal, keys, values, sm_scale))


def clip_threshold(x, u, percentile: float = 99.9) -> float:
    """Percentile (linear interpolation) of |x R| over all tokens and channels of x (n, d)."""
    return float(np.percentile(np.abs(rotate(x, u)), percentile))


# ----------------------------------------------------------------------------------------------
# the error chain of the rotation choices ([W1] figure 1, section OSCAR 的动机: naive INT2,
# Hadamard-only, clip-only and OSCAR compared by the attention-score KL and the attention-output
# MSE their quantisation noise causes, not only by K/V reconstruction error).  The frame of each
# variant is an orthogonal R: identity (naive, clip-only), H P / sqrt(d) (Hadamard-only, U = I)
# or U H P / sqrt(d) (OSCAR); no clip is an infinite threshold.

def frame_matrix(u=None, d: int = 128) -> np.ndarray:
    """Orthogonal frame of a variant: U H P / sqrt(d) for a basis U, the identity for None."""
    return np.eye(d) if u is None else rotation_matrix(u)


def quantize_roundtrip(x, r, clip, group: int, levels=None) -> np.ndarray:
    """Vectors x (n, d) quantised in the frame R (x' = x R, rounded to fp32, clipped to |x'| <=
    clip, group INT2 codes with fp16 scale and zero point, optionally on the equally spaced
    codebook ``levels`` = (lo, step)) and mapped back: (s c + z) R^T, fp64."""
    xr = (np.asarray(x, dtype=np.float64) @ r).astype(np.float32)
    codes, scale, zero, _ = quantize(xr, clip, group, levels)
    return dequantize(codes, scale, zero, group) @ np.asarray(r, dtype=np.float64).T


# ----------------------------------------------------------------------------------------------
# a Lloyd-Max codebook in place of the uniform INT2 grid ([W3], the closing comparison with
# TurboQuant: OSCAR's newer code pairs the attention-aware rotation with a Lloyd-Max codebook;
# the page gives no further detail).  Reading R19: the group's fp16 scale and zero point stay as
# in R5 and map the clipped group onto t = (x'' - z) / s in [0, 3]; a code names one of four
# levels l_0 < l_1 < l_2 < l_3 in that coordinate (the nearest; a value halfway between two
# levels takes the lower code), and the stored value is s * l_code + z.  The levels are fitted
# per (layer, KV head, K|V) on calibration data by Lloyd's algorithm.  {0, 1, 2, 3} is the
# uniform grid of R5.

def lloyd_max(values, weights=None, levels=(0.0, 1.0, 2.0, 3.0), iters: int = 100):
    """Lloyd's algorithm for a scalar quantiser with len(levels) reconstruction levels.

    Alternates the two conditions a Lloyd-Max quantiser satisfies: each decision threshold lies
    halfway between the two levels around it (nearest-neighbour condition), and each level is the
    (weighted) mean of the values in its cell (centroid condition).  A cell with no weight keeps
    its level.  ``values`` are samples (or grid points of a density, with ``weights``).
    Returns (levels, thresholds, distortion before each update and after the last one), the
    distortion being the weighted mean squared error.
    """
    x = np.asarray(values, dtype=np.float64).ravel()
    w = np.ones_like(x) if weights is None else np.asarray(weights, dtype=np.float64).ravel()
    lv = np.sort(np.asarray(levels, dtype=np.float64))
    history = []
    for _ in range(iters + 1):
        thr = (lv[:-1] + lv[1:]) / 2
        cell = np.searchsorted(thr, x, side="left")
        history.append(float(np.sum(w * (x - lv[cell]) ** 2) / np.sum(w)))
        if len(history) == iters + 1:
            break
        new = lv.copy()
        for i in range(len(lv)):
            wi = w[cell == i]
            if wi.sum() > 0:
                new[i] = float(np.sum(wi * x[cell == i]) / wi.sum())
        lv = new
    return lv, (lv[:-1] + lv[1:]) / 2, history


def lloyd_max_uniform(values, weights=None, lo: float = 0.0, step: float = 1.0,
                      iters: int = 100):
    """The optimum equally spaced 4-level quantiser (levels lo + step * c, c = 0..3; reading R20)
    by alternating its two conditions: each value takes the nearest level, code
    clamp(rint((t - lo) / step), 0, 3); (lo, step) is the (weighted) least-squares line of the
    values on their codes.  Neither step increases the distortion.  Returns (lo, step,
    distortion before each update and after the last one)."""
    x = np.asarray(values, dtype=np.float64).ravel()
    w = np.ones_like(x) if weights is None else np.asarray(weights, dtype=np.float64).ravel()
    wt = w.sum()
    history = []
    for it in range(iters + 1):
        c = np.clip(np.rint((x - lo) / step), 0, 3)
        history.append(float(np.sum(w * (x - lo - step * c) ** 2) / wt))
        if it == iters:
            break
        mc, mx = np.sum(w * c) / wt, np.sum(w * x) / wt
        var = np.sum(w * (c - mc) ** 2) / wt
        if var > 0:
            step = float(np.sum(w * (c - mc) * (x - mx)) / wt / var)
            lo = float(mx - step * mc)
    return lo, step, history


def symmetric_levels(l0: float, l1: float) -> np.ndarray:
    """The four levels (l0, l1, 3 - l1, 3 - l0) of a codebook symmetric about 1.5 (reading R21)."""
    return np.array([l0, l1, 3.0 - l1, 3.0 - l0], dtype=np.float64)


def lloyd_max_symmetric(values, weights=None, l0: float = 0.0, l1: float = 1.0,
                        iters: int = 100):
    """Lloyd's algorithm restricted to codebooks symmetric about 1.5 (reading R21): levels
    (l0, l1, 3 - l1, 3 - l0).  Each step applies the two conditions within that family: every
    value takes the nearest level (thresholds (l0 + l1) / 2, 1.5 and their mirror; a value halfway
    takes the lower code), then l0 (l1) is the least-squares level of cell 0 (1) together with the
    mirror images 3 - t of cell 3 (2) -- the centroid of the pair of cells that share it.  A pair
    with no weight keeps its level.  Returns (levels (4,), thresholds (3,), distortion before each
    update and after the last one)."""
    x = np.asarray(values, dtype=np.float64).ravel()
    w = np.ones_like(x) if weights is None else np.asarray(weights, dtype=np.float64).ravel()
    history = []
    for it in range(iters + 1):
        lv = symmetric_levels(l0, l1)
        thr = (lv[:-1] + lv[1:]) / 2
        cell = np.searchsorted(thr, x, side="left")
        history.append(float(np.sum(w * (x - lv[cell]) ** 2) / np.sum(w)))
        if it == iters:
            break
        new = []
        for lo_c, hi_c, cur in ((0, 3, l0), (1, 2, l1)):
            wl, wh = w[cell == lo_c], w[cell == hi_c]
            tot = wl.sum() + wh.sum()
            new.append(cur if tot == 0 else
                       float((np.sum(wl * x[cell == lo_c]) + np.sum(wh * (3.0 - x[cell == hi_c])))
                             / tot))
        l0, l1 = new
    lv = symmetric_levels(l0, l1)
    return lv, (lv[:-1] + lv[1:]) / 2, history


def codebook_coordinates(xr, clip, group: int) -> np.ndarray:
    """t = (x'' - z) / s of every element of rotated fp32 vectors xr (..., d), with the group's
    fp16 scale and zero (R5): the coordinate a codebook is fitted in and applied to."""
    return quantize(xr, clip, group)[3]["t"].astype(np.float64)


def quantize_codebook(xr, clip, group: int, levels):
    """Codes (..., d) of rotated vectors under a codebook (R19), with the fp16 scale and zero of
    R5 (returned as in ``quantize``)."""
    _, s16, z16, pre = quantize(xr, clip, group)
    lv = np.sort(np.asarray(levels, dtype=np.float64))
    codes = np.searchsorted((lv[:-1] + lv[1:]) / 2, pre["t"].astype(np.float64), side="left")
    return codes.astype(np.uint8), s16, z16


def dequantize_codebook(codes, scale, zero, group: int, levels) -> np.ndarray:
    """Rotated-space values s * l_code + z in fp64, (..., d)."""
    lv = np.sort(np.asarray(levels, dtype=np.float64))
    return dequantize(lv[np.asarray(codes, dtype=np.int64)], scale, zero, group)


def quantize_roundtrip_codebook(x, r, clip, group: int, levels) -> np.ndarray:
    """``quantize_roundtrip`` with the codebook levels in place of the uniform grid."""
    xr = (np.asarray(x, dtype=np.float64) @ r).astype(np.float32)
    codes, scale, zero = quantize_codebook(xr, clip, group, levels)
    return dequantize_codebook(codes, scale, zero, group, levels) @ np.asarray(r, np.float64).T


def attention_error_metrics(q, keys, values, keys_hat, values_hat, sm_scale: float):
    """Errors that replacing (keys, values) (n, d) by (keys_hat, values_hat) causes for queries
    q (m, d): mean over queries of KL(p || p_hat) of the softmax score distributions, mean squared
    error of the attention outputs per element, and mean squared K and V reconstruction errors."""
    q = np.asarray(q, dtype=np.float64)
    s = (q @ np.asarray(keys, np.float64).T) * sm_scale
    sh = (q @ np.asarray(keys_hat, np.float64).T) * sm_scale
    ls = s - s.max(axis=1, keepdims=True)
    ls -= np.log(np.exp(ls).sum(axis=1, keepdims=True))
    lsh = sh - sh.max(axis=1, keepdims=True)
    lsh -= np.log(np.exp(lsh).sum(axis=1, keepdims=True))
    p = np.exp(ls)
    kl = float(np.mean(np.sum(p * (ls - lsh), axis=1)))
    o = p @ np.asarray(values, np.float64)
    oh = np.exp(lsh) @ np.asarray(values_hat, np.float64)
    mse = float(np.mean((o - oh) ** 2))
    k_err = float(np.mean((np.asarray(keys, np.float64) - keys_hat) ** 2))
    v_err = float(np.mean((np.asarray(values, np.float64) - values_hat) ** 2))
    return kl, mse, k_err, v_err


# ----------------------------------------------------------------------------------------------
# byte accounting ([W3] evaluation: effective bits per KV element and the ~8x memory claim)

def history_bytes_per_token_head(head_dim: int, group: int) -> int:
    """Key codes + value codes + fp16 (scale, zero) per group for keys and values."""
    return 2 * head_dim // 4 + 2 * (head_dim // group) * 4


def effective_bits_per_element(length: int, head_dim: int, group: int, sink: int = 64,
                               recent: int = 256) -> float:
    """Average stored bits per K/V element of a context: BF16 sink and recent, INT2 history."""
    bf16 = min(length, sink + recent)
    hist = max(0, length - sink - recent)
    bits = bf16 * 16.0 + hist * history_bytes_per_token_head(head_dim, group) * 8 / (2 * head_dim)
    return bits / length
