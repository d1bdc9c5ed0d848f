"""Seeded synthetic inputs for the OSCAR INT2-history decode path.

This module only draws random numbers: keys, values, queries, rotation bases, context lengths and
page tables.  It holds none of the method's arithmetic (no rotation, clipping, quantisation,
packing or attention), so both the HIP path and the CPU oracle take their inputs from it.

Every draw is keyed by (workload seed, layer, stream, chunk), so any sub-range of any sequence can
be regenerated on its own, on the device where it is needed.  Keys and values are generated in
chunks of ``CHUNK`` positions; a chunk that lies inside a shared prefix is drawn once for all
sequences.  Draws on different device types use different torch generators, so a run keeps all
draws of one tensor on one device and copies slices to the host for the oracle.

The workloads stand in for the system measurements on the pages (no model weights or datasets are
used): 100k-context batch-1 decode with a full prefix hit and large-batch decode with a shared
prefix (the repost of the OSCAR write-up on m.kljzs.com, figures 5 and 6), at Qwen3-shaped head
counts.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Sequence

import numpy as np
import torch

CHUNK = 4096

# tensor ids used in seed derivation
_K, _V, _Q, _UK, _UV, _OUT_K, _OUT_V, _QCAL, _SIGMA, _PAGES, _LENS = range(11)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic decode workload."""

    name: str
    seed: int
    num_layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    group_size: int
    context: Optional[int]          # fixed context length, or None for ragged lengths
    ragged: Optional[tuple] = None  # (lo, hi) inclusive bounds of ragged context lengths
    shared_prefix: int = 0          # tokens shared by every sequence through the page table
    kv_dist: str = "normal"         # "normal" | "student_t3"
    outliers: str = "none"          # "fixed4" | "one_per_head" | "none"
    outlier_gain: float = 16.0
    query_dist: str = "normal"      # "normal" | "aniso"
    rotation: str = "qr"            # "qr" | "cov_eig" | "calibrated"
    clip: Optional[float] = 4.0     # None: calibrated per head
    calib_queries: int = 0          # calibration query positions (rotation == "calibrated")
    clip_calib_tokens: int = 0      # tokens used for a calibrated clip

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads


FIXED_OUTLIER_CHANNELS = (3, 17, 64, 101)

WORKLOADS = {
    # tiny single layer, GQA 4, context 1024 = 64 + 704 + 256
    "tiny_gqa4_1k": Workload(
        name="tiny_gqa4_1k", seed=1, num_layers=1, batch=1, num_q_heads=4, num_kv_heads=1,
        head_dim=128, group_size=128, context=1024, outliers="fixed4", rotation="qr", clip=4.0),
    # Qwen3-4B-shaped layer with CPU calibration, context 32768
    "qwen3_4b_32k": Workload(
        name="qwen3_4b_32k", seed=2, num_layers=1, batch=1, num_q_heads=32, num_kv_heads=8,
        head_dim=128, group_size=128, context=32768, outliers="fixed4", query_dist="aniso",
        rotation="calibrated", clip=None, calib_queries=4096, clip_calib_tokens=32768),
    # Qwen3-8B-shaped batch-1 decode at 100k context, 36 layers
    "qwen3_8b_100k": Workload(
        name="qwen3_8b_100k", seed=3, num_layers=36, batch=1, num_q_heads=32, num_kv_heads=8,
        head_dim=128, group_size=128, context=100000, outliers="one_per_head", rotation="qr",
        clip=4.0),
    # one GPU's share of the same layers under 8-way tensor parallelism (one KV head per GPU)
    "qwen3_8b_100k_kv1": Workload(
        name="qwen3_8b_100k_kv1", seed=3, num_layers=36, batch=1, num_q_heads=4, num_kv_heads=1,
        head_dim=128, group_size=128, context=100000, outliers="one_per_head", rotation="qr",
        clip=4.0),
    # Qwen3-8B-shaped batch 64, ragged 8k..128k contexts, 32768-token shared prefix
    "qwen3_8b_b64_prefix": Workload(
        name="qwen3_8b_b64_prefix", seed=4, num_layers=36, batch=64, num_q_heads=32,
        num_kv_heads=8, head_dim=128, group_size=128, context=None, ragged=(8192, 131072),
        shared_prefix=32768, outliers="one_per_head", rotation="qr", clip=4.0),
    # Qwen3-32B-shaped long context, GQA 8, group 64, heavy-tailed K/V
    "qwen3_32b_131k": Workload(
        name="qwen3_32b_131k", seed=5, num_layers=1, batch=16, num_q_heads=64, num_kv_heads=8,
        head_dim=128, group_size=64, context=131072, kv_dist="student_t3", query_dist="aniso",
        rotation="cov_eig", clip=None, clip_calib_tokens=4096),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of ``wl`` with some fields replaced (smaller contexts or batches for fast tests)."""
    return dataclasses.replace(wl, **changes)


# ----------------------------------------------------------------------------------------------
# seed derivation

def _seed(*key) -> int:
    h = hashlib.blake2b(repr(key).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(*key))
    return g


def _np_rng(*key) -> np.random.Generator:
    return np.random.default_rng(_seed(*key))


# ----------------------------------------------------------------------------------------------
# context lengths and page tables

def context_lengths(wl: Workload) -> list:
    if wl.context is not None:
        return [int(wl.context)] * wl.batch
    lo, hi = wl.ragged
    rng = _np_rng(wl.seed, _LENS)
    return [int(x) for x in rng.integers(lo, hi + 1, size=wl.batch)]


def history_pages(length: int, sink: int = 64, recent: int = 256, page: int = 64) -> int:
    """Pages a context of ``length`` tokens occupies in the INT2 history (plain page arithmetic)."""
    return max(0, -(-(length - sink - recent) // page))


def shared_pages(wl: Workload, length: int, spare_tokens: int = 0, sink: int = 64,
                 recent: int = 256, page: int = 64) -> int:
    """Logical pages of a sequence of ``length`` tokens that alias the shared prefix's physical
    pages.  Pages inside ``wl.shared_prefix`` are shared, except from the page that the
    sequence's next write (history index length - sink - recent, when ``spare_tokens`` > 0) falls
    in: a sequence still inside the prefix gets private copies of the pages it will write
    (copy-on-write), so that its own new tokens never land in a page other sequences read."""
    if not wl.shared_prefix:
        return 0
    n = min((wl.shared_prefix - sink) // page, history_pages(length + spare_tokens, sink, recent,
                                                             page))
    if spare_tokens > 0:
        n = min(n, max(0, length - sink - recent) // page)
    return n


def page_tables(wl: Workload, lengths: Sequence[int], layer: int = 0, spare_tokens: int = 0,
                sink: int = 64, recent: int = 256, page: int = 64):
    """Shuffled page tables.

    Every sequence gets room for ``spare_tokens`` more history tokens than its context holds.
    Logical pages that fall inside ``wl.shared_prefix`` map to the same physical pages in every
    sequence (a full prefix-cache hit), up to the page a sequence will write next (see
    ``shared_pages``); all other pages are private.  Physical page ids are a seeded permutation
    of ``range(num_pages)``.  Returns (table int32 [B, max_pages], num_pages); entries past a
    sequence's last page are 0 and are never read.
    """
    need = [history_pages(L + spare_tokens, sink, recent, page) for L in lengths]
    share = [shared_pages(wl, L, spare_tokens, sink, recent, page) for L in lengths]
    shared_used = max(share) if share else 0
    num_pages = shared_used + sum(n - s for n, s in zip(need, share))
    max_pages = max(1, max(need) if need else 1)
    perm = _np_rng(wl.seed, _PAGES, layer).permutation(max(num_pages, 1)).astype(np.int32)
    table = np.zeros((len(lengths), max_pages), dtype=np.int32)
    nxt = shared_used
    for b, (n, s) in enumerate(zip(need, share)):
        table[b, :s] = perm[:s]
        table[b, s:n] = perm[nxt:nxt + (n - s)]
        nxt += n - s
    return table, max(num_pages, 1)


def shared_prefix(wl: Workload, table: np.ndarray, lengths: Sequence[int], spare_tokens: int = 0,
                  sink: int = 64, recent: int = 256, page: int = 64):
    """The shared prefix of ``page_tables``' table as the cascade takes it: (physical page ids of
    the prefix, int32 [P]; per sequence, how many leading pages of its row are those)."""
    share = [shared_pages(wl, L, spare_tokens, sink, recent, page) for L in lengths]
    n = max(share) if share else 0
    ids = table[int(np.argmax(share)), :n].astype(np.int32) if n else np.zeros(0, np.int32)
    return ids, np.asarray(share, np.int32)


# ----------------------------------------------------------------------------------------------
# keys and values

def outlier_gains(wl: Workload, layer: int, tensor: str) -> torch.Tensor:
    """Per-channel multipliers [Hkv, d] (fp32) applied to a fresh draw before bf16 rounding."""
    gains = torch.ones(wl.num_kv_heads, wl.head_dim, dtype=torch.float32)
    if wl.outliers == "fixed4":
        gains[:, list(FIXED_OUTLIER_CHANNELS)] = wl.outlier_gain
    elif wl.outliers == "one_per_head":
        n_out = max(1, round(0.01 * wl.head_dim))
        rng = _np_rng(wl.seed, _OUT_K if tensor == "k" else _OUT_V, layer)
        for h in range(wl.num_kv_heads):
            gains[h, rng.choice(wl.head_dim, size=n_out, replace=False)] = wl.outlier_gain
    return gains


def _draw_chunk(wl: Workload, layer: int, source: int, chunk: int, tensor_id: int, device):
    g = _gen(device, wl.seed, tensor_id, layer, source, chunk)
    shape = (CHUNK, wl.num_kv_heads, wl.head_dim)
    if wl.kv_dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if wl.kv_dist == "student_t3":
        z = torch.randn((4,) + shape, generator=g, device=device, dtype=torch.float32)
        chi2 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
        return z[0] / torch.sqrt(chi2 / 3.0)
    raise ValueError(wl.kv_dist)


def kv_tokens(wl: Workload, layer: int, seq: int, start: int, count: int, device="cpu"):
    """Keys and values of positions [start, start+count) of sequence ``seq``: bf16 [count, Hkv, d]."""
    out = []
    gk = outlier_gains(wl, layer, "k").to(device)
    gv = outlier_gains(wl, layer, "v").to(device)
    for tensor_id, gains, dst in ((_K, gk, "k"), (_V, gv, "v")):
        parts = []
        pos = start
        end = start + count
        while pos < end:
            c = pos // CHUNK
            lo = pos - c * CHUNK
            hi = min(CHUNK, end - c * CHUNK)
            source = -1 if (c + 1) * CHUNK <= wl.shared_prefix else seq
            x = _draw_chunk(wl, layer, source, c, tensor_id, device)[lo:hi]
            parts.append((x * gains).to(torch.bfloat16))
            pos = c * CHUNK + hi
        if parts:
            out.append(torch.cat(parts, 0))
        else:
            out.append(torch.empty((0, wl.num_kv_heads, wl.head_dim), dtype=torch.bfloat16,
                                   device=device))
    return out[0], out[1]


# ----------------------------------------------------------------------------------------------
# queries and rotation bases

def _haar(rng: np.random.Generator, d: int) -> np.ndarray:
    """Orthogonal matrix from the QR factorisation of a Gaussian draw, column signs fixed by diag(R)."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def query_spectrum(d: int) -> np.ndarray:
    """Eigenvalues proportional to i^-1.5 (i = 1..d), normalised to trace d (fp64)."""
    lam = np.arange(1, d + 1, dtype=np.float64) ** -1.5
    return lam * (d / lam.sum())


def query_covariance_bases(wl: Workload, layer: int) -> np.ndarray:
    """Seeded orthogonal bases O_h [Hkv, d, d] (fp64) of the per-KV-head query covariance
    Sigma_h = O_h diag(lambda) O_h^T used by anisotropic queries."""
    rng = _np_rng(wl.seed, _SIGMA, layer)
    return np.stack([_haar(rng, wl.head_dim) for _ in range(wl.num_kv_heads)])


def rotation_bases(wl: Workload, layer: int):
    """U_k, U_v as fp32 [Hkv, d, d] for workloads whose U is drawn (not calibrated)."""
    if wl.rotation == "qr":
        rk = _np_rng(wl.seed, _UK, layer)
        rv = _np_rng(wl.seed, _UV, layer)
        uk = np.stack([_haar(rk, wl.head_dim) for _ in range(wl.num_kv_heads)])
        uv = np.stack([_haar(rv, wl.head_dim) for _ in range(wl.num_kv_heads)])
    elif wl.rotation == "cov_eig":
        # Sigma_h is built from O_h with descending eigenvalues, so O_h's columns are its
        # eigenvectors in descending order; K and V share it.
        o = query_covariance_bases(wl, layer)
        uk, uv = o, o.copy()
    else:
        raise ValueError("calibrated rotations come from the calibration step")
    return (torch.from_numpy(uk.astype(np.float32)), torch.from_numpy(uv.astype(np.float32)))


def _queries_from_normal(wl: Workload, layer: int, z: torch.Tensor) -> torch.Tensor:
    """Map standard normal draws [..., Hq, d] to the workload's query distribution (fp32)."""
    if wl.query_dist == "normal":
        return z
    o = torch.from_numpy(query_covariance_bases(wl, layer)).to(z.device, torch.float64)
    sq = torch.from_numpy(np.sqrt(query_spectrum(wl.head_dim))).to(z.device, torch.float64)
    hkv = torch.arange(wl.num_q_heads, device=z.device) // wl.gqa
    # q = (z * sqrt(lambda)) O^T  per KV head
    y = (z.to(torch.float64) * sq).unsqueeze(-2)           # [..., Hq, 1, d]
    ot = o[hkv].transpose(-1, -2).contiguous()             # [Hq, d, d], ot[h, j, i] = O_h[i, j]
    return torch.matmul(y, ot).squeeze(-2).to(torch.float32)


def queries(wl: Workload, layer: int, step: int = 0, device="cpu", batch: Optional[int] = None):
    """Decode queries, bf16 [B, Hq, d]."""
    b = wl.batch if batch is None else batch
    g = _gen(device, wl.seed, _Q, layer, step)
    z = torch.randn((b, wl.num_q_heads, wl.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    return _queries_from_normal(wl, layer, z).to(torch.bfloat16)


def calibration_queries(wl: Workload, layer: int, n: Optional[int] = None) -> torch.Tensor:
    """Calibration query positions, fp32 [n, Hq, d] on the host."""
    n = wl.calib_queries if n is None else n
    g = _gen("cpu", wl.seed, _QCAL, layer)
    z = torch.randn((n, wl.num_q_heads, wl.head_dim), generator=g, dtype=torch.float32)
    return _queries_from_normal(wl, layer, z)
