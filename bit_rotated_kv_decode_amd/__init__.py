"""OSCAR INT2-history decode path for AMD Instinct MI355X (gfx950).

Thin Python binding of ``liboscar.so`` (C ABI declared in ``include/oscar.h``): this module only
marshals arguments; every step of the path runs in the library's HIP kernels.  PyTorch supplies
device memory and the current stream.  There is no CPU fallback: if the library is not built or
a call fails, an ``OscarError`` is raised.

The entry points follow the OSCAR write-up "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化"
(section OSCAR 的设计): ``append`` writes a decode step's new token into the BF16 recent window
and demotes the token it displaces into the rotated INT2 history, ``demote`` encodes a run of
tokens into the history, and ``decode_attn`` runs decode attention over the BF16 sink, the INT2
history and the BF16 recent window with an online-softmax merge.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

__all__ = [
    "OscarError", "Layout", "LIB_PATH", "lib", "make_layout", "page_block_bytes", "page_bytes",
    "pool_bytes", "sink_bytes", "recent_bytes", "decode_workspace_bytes", "decode_splits",
    "check_page_table", "decode_workspace_bytes_prefix", "check_shared_prefix",
    "decode_step_launches",
    "demote", "append", "decode_attn", "decode_attn_codebook", "decode_attn_prefix",
    "decode_step", "decode_step_prefix", "decode_step_noalloc", "Cache",
    "STAGE_QUERY", "STAGE_INT2", "STAGE_BF16", "STAGE_MERGE", "STAGE_ALL", "HEAD_DIM", "PAGE_TOKENS", "SINK_TOKENS",
    "RECENT_TOKENS", "bf16_page_block_bytes", "bf16_page_bytes", "bf16_pool_bytes",
    "bf16_decode_workspace_bytes", "bf16_store", "bf16_decode_attn", "probe_read",
    "probe_gather",
]

HEAD_DIM = 128
PAGE_TOKENS = 64
SINK_TOKENS = 64
RECENT_TOKENS = 256

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "liboscar.so")


class OscarError(RuntimeError):
    """A liboscar call returned an error status, or the library is missing."""


class Layout(ctypes.Structure):
    """Mirror of ``oscar_layout`` (include/oscar.h)."""

    _fields_ = [(name, ctypes.c_int32) for name in (
        "head_dim", "group_size", "num_q_heads", "num_kv_heads", "page_tokens", "sink_tokens",
        "recent_tokens", "num_pages", "max_seqs", "max_pages_per_seq", "levels_kind")]

    def __repr__(self):
        return "Layout(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_c_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_LP = ctypes.POINTER(Layout)

_SIGNATURES = {
    "oscar_abi_version": (ctypes.c_uint32, []),
    "oscar_status_string": (ctypes.c_char_p, [_i32]),
    "oscar_last_error": (ctypes.c_char_p, []),
    "oscar_layout_check": (_i32, [_LP]),
    "oscar_page_block_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_page_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_pool_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_sink_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_recent_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_decode_workspace_bytes": (ctypes.c_size_t, [_LP, _i32, _i32]),
    "oscar_decode_splits": (_i32, [_LP, _i32, _i32, _vp]),
    "oscar_check_page_table": (_i32, [_LP, _vp, _vp, _i32, _i32]),
    "oscar_demote": (_i32, [_LP] + [_vp] * 10 + [_i64, _i64, _i64, _vp, _i32, _i32, _vp]),
    "oscar_append": (_i32, [_LP] + [_vp] * 16 + [_i32, _vp]),
    "oscar_decode_attn": (_i32, [_LP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _i32, _i32,
                                 _vp]),
    "oscar_decode_attn_stages": (_i32, [_LP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t,
                                        _i32, _i32, ctypes.c_uint32, _vp]),
    "oscar_decode_attn_codebook": (_i32, [_LP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                          ctypes.c_size_t, _i32, _i32, ctypes.c_uint32, _vp]),
    "oscar_decode_step": (_i32, [_LP] + [_vp] * 17 + [ctypes.c_float, _vp, _vp, _vp,
                                                       ctypes.c_size_t, _i32, _i32, _vp]),
    "oscar_decode_step_noalloc": (_i32, [_LP] + [_vp] * 17 + [ctypes.c_float, _vp, _vp, _i32,
                                                               _i32, _vp]),
    "oscar_decode_step_launches": (_i32, [_LP, _i32, _i32]),
    "oscar_decode_step_stages": (_i32, [_LP] + [_vp] * 17 + [ctypes.c_float, _vp, _vp, _vp,
                                                              ctypes.c_size_t, _i32, _i32,
                                                              ctypes.c_uint32, _vp]),
    "oscar_decode_workspace_bytes_prefix": (ctypes.c_size_t, [_LP, _i32, _i32, _i32]),
    "oscar_check_shared_prefix": (_i32, [_LP, _vp, _i32, _vp, _vp, _i32]),
    "oscar_decode_attn_prefix": (_i32, [_LP] + [_vp] * 13 + [_i32, ctypes.c_float, _vp, _vp,
                                                              _vp, ctypes.c_size_t, _i32, _i32,
                                                              ctypes.c_uint32, _vp]),
    "oscar_decode_step_prefix": (_i32, [_LP] + [_vp] * 17 + [_i32, ctypes.c_float, _vp, _vp,
                                                              _vp, ctypes.c_size_t, _i32, _i32,
                                                              _vp]),
    "oscar_bf16_page_block_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_bf16_page_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_bf16_pool_bytes": (ctypes.c_size_t, [_LP]),
    "oscar_bf16_decode_workspace_bytes": (ctypes.c_size_t, [_LP, _i32, _i32]),
    "oscar_bf16_store": (_i32, [_LP, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _i32, _vp]),
    "oscar_bf16_decode_attn": (_i32, [_LP, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                      ctypes.c_size_t, _i32, _i32, _vp]),
    "oscar_probe_read": (_i32, [_vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _i32, _vp]),
    "oscar_probe_gather": (_i32, [_LP, _vp, _vp, _i32, _i32, _i32, _i32, _vp, ctypes.c_size_t,
                                   _vp]),
}

STAGE_QUERY, STAGE_INT2, STAGE_BF16, STAGE_MERGE, STAGE_ALL = 1, 2, 4, 8, 15
LEVELS_SPACED, LEVELS_SYMMETRIC = 0, 1

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load liboscar.so from this package directory (raises OscarError if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OscarError(f"{LIB_PATH} is not built: run bit_rotated_kv_decode_amd.build.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise OscarError(f"{what}: {L.oscar_status_string(status).decode()} ({status}): "
                         f"{L.oscar_last_error().decode()}")


def make_layout(num_q_heads: int, num_kv_heads: int, num_pages: int, max_seqs: int,
                max_pages_per_seq: int, group_size: int = 128, head_dim: int = HEAD_DIM,
                levels_kind: int = 0) -> Layout:
    """levels_kind: what levels_k / levels_v hold -- 0: (lo, step) of equally spaced codebooks;
    1: (l0, l1) of Lloyd-Max codebooks symmetric about 1.5 (LEVELS_SYMMETRIC)."""
    lay = Layout(head_dim, group_size, num_q_heads, num_kv_heads, PAGE_TOKENS, SINK_TOKENS,
                 RECENT_TOKENS, num_pages, max_seqs, max_pages_per_seq, levels_kind)
    _check(lib().oscar_layout_check(ctypes.byref(lay)), "layout")
    return lay


def page_block_bytes(lay: Layout) -> int:
    return lib().oscar_page_block_bytes(ctypes.byref(lay))


def page_bytes(lay: Layout) -> int:
    return lib().oscar_page_bytes(ctypes.byref(lay))


def pool_bytes(lay: Layout) -> int:
    return lib().oscar_pool_bytes(ctypes.byref(lay))


def sink_bytes(lay: Layout) -> int:
    return lib().oscar_sink_bytes(ctypes.byref(lay))


def recent_bytes(lay: Layout) -> int:
    return lib().oscar_recent_bytes(ctypes.byref(lay))


def decode_workspace_bytes(lay: Layout, batch: int, max_seq_len: int) -> int:
    return lib().oscar_decode_workspace_bytes(ctypes.byref(lay), batch, max_seq_len)


def decode_workspace_bytes_prefix(lay: Layout, batch: int, max_seq_len: int,
                                  prefix_pages: int) -> int:
    return lib().oscar_decode_workspace_bytes_prefix(ctypes.byref(lay), batch, max_seq_len,
                                                     prefix_pages)


def decode_step_launches(lay: Layout, batch: int, max_seq_len: int) -> int:
    """Launches of one oscar_decode_step: 2 when the segment launch appends and rotates the query
    itself, else 3 (0: invalid layout or shape)."""
    return lib().oscar_decode_step_launches(ctypes.byref(lay), batch, max_seq_len)


def decode_splits(lay: Layout, batch: int, max_seq_len: int):
    """(splits per (sequence, KV head), history pages per split) of the decode work plan."""
    pps = ctypes.c_int32(0)
    n = lib().oscar_decode_splits(ctypes.byref(lay), batch, max_seq_len, ctypes.byref(pps))
    if n < 0:
        raise OscarError("decode_splits: invalid arguments")
    return n, pps.value


def check_page_table(lay: Layout, page_table, seq_lens, extra_tokens: int = 0) -> None:
    """Validate a host copy of a page table (int32 [B, max_pages_per_seq]) and lengths."""
    pt = torch.as_tensor(page_table, dtype=torch.int32).cpu().contiguous()
    sl = torch.as_tensor(seq_lens, dtype=torch.int32).cpu().contiguous()
    if pt.dim() != 2 or pt.shape[1] != lay.max_pages_per_seq or pt.shape[0] != sl.numel():
        raise OscarError("page table must be [batch, max_pages_per_seq] with one length per row")
    _check(lib().oscar_check_page_table(ctypes.byref(lay), pt.data_ptr(), sl.data_ptr(),
                                        sl.numel(), extra_tokens), "check_page_table")


def check_shared_prefix(lay: Layout, page_table, prefix_ids, shared_pages) -> None:
    """Validate host copies of a shared-prefix description (oscar_check_shared_prefix): page ids
    in range and, per sequence b, its first shared_pages[b] page-table entries equal to
    prefix_ids[0 ..)."""
    pt = torch.as_tensor(page_table, dtype=torch.int32).cpu().contiguous()
    ids = torch.as_tensor(prefix_ids, dtype=torch.int32).cpu().contiguous().reshape(-1)
    sh = torch.as_tensor(shared_pages, dtype=torch.int32).cpu().contiguous().reshape(-1)
    if pt.dim() != 2 or pt.shape[1] != lay.max_pages_per_seq or pt.shape[0] != sh.numel():
        raise OscarError("page table must be [batch, max_pages_per_seq] with one shared_pages "
                         "entry per row")
    _check(lib().oscar_check_shared_prefix(ctypes.byref(lay), pt.data_ptr(), sh.numel(),
                                           ids.data_ptr(), sh.data_ptr(), ids.numel()),
           "check_shared_prefix")


# ----------------------------------------------------------------------------------------------
# argument marshalling helpers

def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be on a GPU device")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _contig(t: torch.Tensor, name: str, dtype) -> int:
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    return _dev(t, name, dtype)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


# Size checks of device buffers.  The C ABI takes bare pointers and cannot see allocation sizes,
# and the kernels index these buffers from the layout without bounds checks, so a buffer that is
# too small must be caught here, before the library is called.

def _min_bytes(t: torch.Tensor, name: str, nbytes: int) -> None:
    if t.numel() * t.element_size() < nbytes:
        raise TypeError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise TypeError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows(t: torch.Tensor, name: str, n: int) -> None:
    if t.numel() != n:
        raise TypeError(f"{name} must hold {n} entries (one per sequence), got {t.numel()}")


def _table(t: torch.Tensor, lay: Layout, batch: int) -> None:
    if t.dim() != 2 or t.shape[1] != lay.max_pages_per_seq or t.shape[0] < batch:
        raise TypeError(f"page_table must be [>= {batch}, {lay.max_pages_per_seq}] "
                        f"(max_pages_per_seq), got {tuple(t.shape)}")


def _rotation(lay: Layout, u_k, u_v, clip_k=None, clip_v=None) -> None:
    for name, u in (("u_k", u_k), ("u_v", u_v)):
        _shape(u, name, (lay.num_kv_heads, HEAD_DIM, HEAD_DIM))
    for name, c in (("clip_k", clip_k), ("clip_v", clip_v)):
        if c is not None:
            _shape(c, name, (lay.num_kv_heads,))


def _segments(lay: Layout, sink_k, sink_v, recent_k, recent_v) -> None:
    for name, t, n in (("sink_k", sink_k, SINK_TOKENS), ("sink_v", sink_v, SINK_TOKENS),
                       ("recent_k", recent_k, RECENT_TOKENS),
                       ("recent_v", recent_v, RECENT_TOKENS)):
        _min_bytes(t, name, lay.max_seqs * lay.num_kv_heads * n * HEAD_DIM * 2)


def _levels(t: Optional[torch.Tensor], name: str, lay: Layout):
    if t is None:
        return None
    if tuple(t.shape) != (lay.num_kv_heads, 2):
        raise TypeError(f"{name} must be [Hkv, 2] (lo, step) per KV head")
    return _contig(t, name, torch.float32)


def demote(lay: Layout, pool: torch.Tensor, page_table: torch.Tensor, u_k: torch.Tensor,
           u_v: torch.Tensor, clip_k: torch.Tensor, clip_v: torch.Tensor, k_src: torch.Tensor,
           v_src: torch.Tensor, hist_start: torch.Tensor,
           levels_k: Optional[torch.Tensor] = None,
           levels_v: Optional[torch.Tensor] = None) -> None:
    """Encode k_src / v_src (bf16 [B, n, Hkv, 128], unit stride on the last axis, the same
    strides for both) into history indices hist_start[b] + i (oscar_demote).  levels_k /
    levels_v: optional fp32 [Hkv, 2] (lo, step) of an equally spaced codebook per KV head."""
    if k_src.dim() != 4 or k_src.shape != v_src.shape or k_src.stride() != v_src.stride():
        raise TypeError("k_src / v_src must be [B, n, Hkv, 128] with identical strides")
    if k_src.stride(3) != 1 or k_src.shape[3] != HEAD_DIM or k_src.shape[2] != lay.num_kv_heads:
        raise TypeError("k_src last axis must be contiguous head_dim; axis 2 the KV heads")
    bsz, n = k_src.shape[0], k_src.shape[1]
    _min_bytes(pool, "pool", pool_bytes(lay))
    _table(page_table, lay, bsz)
    _rotation(lay, u_k, u_v, clip_k, clip_v)
    _rows(hist_start, "hist_start", bsz)
    _check(lib().oscar_demote(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(u_k, "u_k", torch.float32),
        _contig(u_v, "u_v", torch.float32), _contig(clip_k, "clip_k", torch.float32),
        _contig(clip_v, "clip_v", torch.float32), _levels(levels_k, "levels_k", lay),
        _levels(levels_v, "levels_v", lay), _dev(k_src, "k_src", torch.bfloat16),
        _dev(v_src, "v_src", torch.bfloat16), k_src.stride(0), k_src.stride(1), k_src.stride(2),
        _contig(hist_start, "hist_start", torch.int32), bsz, n, _stream()), "demote")


def append(lay: Layout, pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k, u_v, clip_k,
           clip_v, k_new: torch.Tensor, v_new: torch.Tensor, seq_slot: torch.Tensor,
           seq_lens: torch.Tensor, levels_k: Optional[torch.Tensor] = None,
           levels_v: Optional[torch.Tensor] = None) -> None:
    """Decode-step write of k_new / v_new (bf16 [B, Hkv, 128]) at positions seq_lens[b]
    (oscar_append); the caller advances seq_lens afterwards."""
    bsz = seq_lens.numel()
    if tuple(k_new.shape) != (bsz, lay.num_kv_heads, HEAD_DIM) or k_new.shape != v_new.shape:
        raise TypeError("k_new / v_new must be [batch, Hkv, 128]")
    _min_bytes(pool, "pool", pool_bytes(lay))
    _table(page_table, lay, bsz)
    _segments(lay, sink_k, sink_v, recent_k, recent_v)
    _rotation(lay, u_k, u_v, clip_k, clip_v)
    _rows(seq_slot, "seq_slot", bsz)
    _check(lib().oscar_append(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(sink_k, "sink_k", torch.bfloat16),
        _contig(sink_v, "sink_v", torch.bfloat16), _contig(recent_k, "recent_k", torch.bfloat16),
        _contig(recent_v, "recent_v", torch.bfloat16), _contig(u_k, "u_k", torch.float32),
        _contig(u_v, "u_v", torch.float32), _contig(clip_k, "clip_k", torch.float32),
        _contig(clip_v, "clip_v", torch.float32), _levels(levels_k, "levels_k", lay),
        _levels(levels_v, "levels_v", lay), _contig(k_new, "k_new", torch.bfloat16),
        _contig(v_new, "v_new", torch.bfloat16), _contig(seq_slot, "seq_slot", torch.int32),
        _contig(seq_lens, "seq_lens", torch.int32), bsz, _stream()), "append")


def _int2_attn_sizes(lay, bsz, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                     u_k, u_v, lse):
    _min_bytes(pool, "pool", pool_bytes(lay))
    _table(page_table, lay, bsz)
    _segments(lay, sink_k, sink_v, recent_k, recent_v)
    _rotation(lay, u_k, u_v)
    _rows(seq_slot, "seq_slot", bsz)
    if lse is not None:
        _shape(lse, "lse", (bsz, lay.num_q_heads))


def decode_attn(lay: Layout, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                seq_lens, q: torch.Tensor, u_k, u_v, out: torch.Tensor, workspace: torch.Tensor,
                max_seq_len: int, lse: Optional[torch.Tensor] = None,
                sm_scale: float = 0.0, stages: int = STAGE_ALL) -> None:
    """Decode attention of q (bf16 [B, Hq, 128]) into out (fp32 [B, Hq, 128]) and optionally
    lse (fp32 [B, Hq]) (oscar_decode_attn_stages; ``stages`` selects a subset of the stages).
    workspace: uint8 tensor of at least decode_workspace_bytes(lay, B, max_seq_len) bytes."""
    bsz = seq_lens.numel()
    if tuple(q.shape) != (bsz, lay.num_q_heads, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise TypeError("q / out must be [batch, Hq, 128]")
    _int2_attn_sizes(lay, bsz, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                     u_k, u_v, lse)
    _check(lib().oscar_decode_attn_stages(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(sink_k, "sink_k", torch.bfloat16),
        _contig(sink_v, "sink_v", torch.bfloat16), _contig(recent_k, "recent_k", torch.bfloat16),
        _contig(recent_v, "recent_v", torch.bfloat16), _contig(seq_slot, "seq_slot", torch.int32),
        _contig(seq_lens, "seq_lens", torch.int32), _contig(q, "q", torch.bfloat16),
        _contig(u_k, "u_k", torch.float32), _contig(u_v, "u_v", torch.float32), float(sm_scale),
        _contig(out, "out", torch.float32),
        None if lse is None else _contig(lse, "lse", torch.float32),
        _contig(workspace, "workspace", torch.uint8), workspace.numel(), bsz, int(max_seq_len),
        int(stages), _stream()), "decode_attn")


def decode_attn_codebook(lay: Layout, pool, page_table, sink_k, sink_v, recent_k, recent_v,
                         seq_slot, seq_lens, q: torch.Tensor, u_k, u_v, levels_k: torch.Tensor,
                         levels_v: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                         max_seq_len: int, lse: Optional[torch.Tensor] = None,
                         sm_scale: float = 0.0, stages: int = STAGE_ALL) -> None:
    """decode_attn over a history encoded with symmetric codebooks (lay.levels_kind 1):
    levels_k / levels_v fp32 [Hkv, 2] = (l0, l1) per KV head (oscar_decode_attn_codebook)."""
    bsz = seq_lens.numel()
    if tuple(q.shape) != (bsz, lay.num_q_heads, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise TypeError("q / out must be [batch, Hq, 128]")
    _int2_attn_sizes(lay, bsz, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                     u_k, u_v, lse)
    _check(lib().oscar_decode_attn_codebook(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(sink_k, "sink_k", torch.bfloat16),
        _contig(sink_v, "sink_v", torch.bfloat16), _contig(recent_k, "recent_k", torch.bfloat16),
        _contig(recent_v, "recent_v", torch.bfloat16), _contig(seq_slot, "seq_slot", torch.int32),
        _contig(seq_lens, "seq_lens", torch.int32), _contig(q, "q", torch.bfloat16),
        _contig(u_k, "u_k", torch.float32), _contig(u_v, "u_v", torch.float32),
        _levels(levels_k, "levels_k", lay), _levels(levels_v, "levels_v", lay), float(sm_scale),
        _contig(out, "out", torch.float32),
        None if lse is None else _contig(lse, "lse", torch.float32),
        _contig(workspace, "workspace", torch.uint8), workspace.numel(), bsz, int(max_seq_len),
        int(stages), _stream()), "decode_attn_codebook")


def _prefix(prefix_ids: torch.Tensor, shared_pages: torch.Tensor, bsz: int):
    if prefix_ids.dim() != 1:
        raise TypeError("prefix_ids must be int32 [prefix_pages]")
    _rows(shared_pages, "shared_pages", bsz)
    n = prefix_ids.numel()
    if n == 0:
        return None, None, 0
    return (_contig(prefix_ids, "prefix_ids", torch.int32),
            _contig(shared_pages, "shared_pages", torch.int32), n)


def decode_attn_prefix(lay: Layout, pool, page_table, sink_k, sink_v, recent_k, recent_v,
                       seq_slot, seq_lens, q: torch.Tensor, u_k, u_v, prefix_ids: torch.Tensor,
                       shared_pages: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                       max_seq_len: int, lse: Optional[torch.Tensor] = None,
                       sm_scale: float = 0.0, stages: int = STAGE_ALL) -> None:
    """decode_attn for sequences that share a prefix through the page table
    (oscar_decode_attn_prefix): prefix_ids int32 [P] = the prefix's page ids, shared_pages int32
    [B] = leading pages of each row that are those.  The same result as decode_attn; whole chunks
    of shared pages are read once per group of sequences.  workspace: at least
    decode_workspace_bytes_prefix(lay, B, max_seq_len, P) bytes."""
    bsz = seq_lens.numel()
    if tuple(q.shape) != (bsz, lay.num_q_heads, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise TypeError("q / out must be [batch, Hq, 128]")
    _int2_attn_sizes(lay, bsz, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                     u_k, u_v, lse)
    ids, shared, n = _prefix(prefix_ids, shared_pages, bsz)
    _check(lib().oscar_decode_attn_prefix(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(sink_k, "sink_k", torch.bfloat16),
        _contig(sink_v, "sink_v", torch.bfloat16), _contig(recent_k, "recent_k", torch.bfloat16),
        _contig(recent_v, "recent_v", torch.bfloat16), _contig(seq_slot, "seq_slot", torch.int32),
        _contig(seq_lens, "seq_lens", torch.int32), _contig(q, "q", torch.bfloat16),
        _contig(u_k, "u_k", torch.float32), _contig(u_v, "u_v", torch.float32), ids, shared, n,
        float(sm_scale), _contig(out, "out", torch.float32),
        None if lse is None else _contig(lse, "lse", torch.float32),
        _contig(workspace, "workspace", torch.uint8), workspace.numel(), bsz, int(max_seq_len),
        int(stages), _stream()), "decode_attn_prefix")


def decode_step(lay: Layout, pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k, u_v,
                clip_k, clip_v, k_new: torch.Tensor, v_new: torch.Tensor, seq_slot, seq_pos,
                q: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor, max_seq_len: int,
                lse: Optional[torch.Tensor] = None, sm_scale: float = 0.0,
                levels_k: Optional[torch.Tensor] = None,
                levels_v: Optional[torch.Tensor] = None, stages: Optional[int] = None) -> None:
    """append(k_new, v_new at seq_pos) then decode_attn(q) over seq_pos + 1 tokens
    (oscar_decode_step, or oscar_decode_step_stages with the launches `stages` selects); the
    caller advances seq_pos afterwards.  The workspace must be zero-filled before its first use."""
    bsz = seq_pos.numel()
    if tuple(k_new.shape) != (bsz, lay.num_kv_heads, HEAD_DIM) or k_new.shape != v_new.shape:
        raise TypeError("k_new / v_new must be [batch, Hkv, 128]")
    if tuple(q.shape) != (bsz, lay.num_q_heads, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise TypeError("q / out must be [batch, Hq, 128]")
    _int2_attn_sizes(lay, bsz, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                     u_k, u_v, lse)
    _shape(clip_k, "clip_k", (lay.num_kv_heads,))
    _shape(clip_v, "clip_v", (lay.num_kv_heads,))
    fn = lib().oscar_decode_step if stages is None else lib().oscar_decode_step_stages
    _check(fn(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(sink_k, "sink_k", torch.bfloat16),
        _contig(sink_v, "sink_v", torch.bfloat16), _contig(recent_k, "recent_k", torch.bfloat16),
        _contig(recent_v, "recent_v", torch.bfloat16), _contig(u_k, "u_k", torch.float32),
        _contig(u_v, "u_v", torch.float32), _contig(clip_k, "clip_k", torch.float32),
        _contig(clip_v, "clip_v", torch.float32), _levels(levels_k, "levels_k", lay),
        _levels(levels_v, "levels_v", lay), _contig(k_new, "k_new", torch.bfloat16),
        _contig(v_new, "v_new", torch.bfloat16), _contig(seq_slot, "seq_slot", torch.int32),
        _contig(seq_pos, "seq_pos", torch.int32), _contig(q, "q", torch.bfloat16),
        float(sm_scale), _contig(out, "out", torch.float32),
        None if lse is None else _contig(lse, "lse", torch.float32),
        _contig(workspace, "workspace", torch.uint8), workspace.numel(), bsz, int(max_seq_len),
        *(() if stages is None else (ctypes.c_uint32(stages),)), _stream()), "decode_step")


def decode_step_prefix(lay: Layout, pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k,
                       u_v, clip_k, clip_v, k_new: torch.Tensor, v_new: torch.Tensor, seq_slot,
                       seq_pos, q: torch.Tensor, prefix_ids: torch.Tensor,
                       shared_pages: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                       max_seq_len: int, lse: Optional[torch.Tensor] = None,
                       sm_scale: float = 0.0) -> None:
    """decode_step over a shared prefix (oscar_decode_step_prefix): append, then
    decode_attn_prefix over seq_pos + 1 tokens."""
    bsz = seq_pos.numel()
    if tuple(k_new.shape) != (bsz, lay.num_kv_heads, HEAD_DIM) or k_new.shape != v_new.shape:
        raise TypeError("k_new / v_new must be [batch, Hkv, 128]")
    if tuple(q.shape) != (bsz, lay.num_q_heads, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise TypeError("q / out must be [batch, Hq, 128]")
    _int2_attn_sizes(lay, bsz, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                     u_k, u_v, lse)
    _shape(clip_k, "clip_k", (lay.num_kv_heads,))
    _shape(clip_v, "clip_v", (lay.num_kv_heads,))
    ids, shared, n = _prefix(prefix_ids, shared_pages, bsz)
    _check(lib().oscar_decode_step_prefix(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(sink_k, "sink_k", torch.bfloat16),
        _contig(sink_v, "sink_v", torch.bfloat16), _contig(recent_k, "recent_k", torch.bfloat16),
        _contig(recent_v, "recent_v", torch.bfloat16), _contig(u_k, "u_k", torch.float32),
        _contig(u_v, "u_v", torch.float32), _contig(clip_k, "clip_k", torch.float32),
        _contig(clip_v, "clip_v", torch.float32), _contig(k_new, "k_new", torch.bfloat16),
        _contig(v_new, "v_new", torch.bfloat16), _contig(seq_slot, "seq_slot", torch.int32),
        _contig(seq_pos, "seq_pos", torch.int32), _contig(q, "q", torch.bfloat16), ids, shared,
        n, float(sm_scale), _contig(out, "out", torch.float32),
        None if lse is None else _contig(lse, "lse", torch.float32),
        _contig(workspace, "workspace", torch.uint8), workspace.numel(), bsz, int(max_seq_len),
        _stream()), "decode_step_prefix")


def decode_step_noalloc(lay: Layout, pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k,
                        u_v, clip_k, clip_v, k_new: torch.Tensor, v_new: torch.Tensor, seq_slot,
                        seq_pos, q: torch.Tensor, out: torch.Tensor, max_seq_len: int,
                        lse: Optional[torch.Tensor] = None, sm_scale: float = 0.0,
                        levels_k: Optional[torch.Tensor] = None,
                        levels_v: Optional[torch.Tensor] = None) -> None:
    """decode_step with the library's own per-GPU scratch array as workspace
    (oscar_decode_step_noalloc): nothing is allocated; calls that overlap on one GPU race."""
    bsz = seq_pos.numel()
    if tuple(k_new.shape) != (bsz, lay.num_kv_heads, HEAD_DIM) or k_new.shape != v_new.shape:
        raise TypeError("k_new / v_new must be [batch, Hkv, 128]")
    if tuple(q.shape) != (bsz, lay.num_q_heads, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise TypeError("q / out must be [batch, Hq, 128]")
    _int2_attn_sizes(lay, bsz, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                     u_k, u_v, lse)
    _shape(clip_k, "clip_k", (lay.num_kv_heads,))
    _shape(clip_v, "clip_v", (lay.num_kv_heads,))
    _check(lib().oscar_decode_step_noalloc(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(sink_k, "sink_k", torch.bfloat16),
        _contig(sink_v, "sink_v", torch.bfloat16), _contig(recent_k, "recent_k", torch.bfloat16),
        _contig(recent_v, "recent_v", torch.bfloat16), _contig(u_k, "u_k", torch.float32),
        _contig(u_v, "u_v", torch.float32), _contig(clip_k, "clip_k", torch.float32),
        _contig(clip_v, "clip_v", torch.float32), _levels(levels_k, "levels_k", lay),
        _levels(levels_v, "levels_v", lay), _contig(k_new, "k_new", torch.bfloat16),
        _contig(v_new, "v_new", torch.bfloat16), _contig(seq_slot, "seq_slot", torch.int32),
        _contig(seq_pos, "seq_pos", torch.int32), _contig(q, "q", torch.bfloat16),
        float(sm_scale), _contig(out, "out", torch.float32),
        None if lse is None else _contig(lse, "lse", torch.float32), bsz, int(max_seq_len),
        _stream()), "decode_step_noalloc")


# ----------------------------------------------------------------------------------------------
# paged BF16 baseline (every cached token in BF16 pages of 64 tokens; include/oscar.h)

def bf16_page_block_bytes(lay: Layout) -> int:
    return lib().oscar_bf16_page_block_bytes(ctypes.byref(lay))


def bf16_page_bytes(lay: Layout) -> int:
    return lib().oscar_bf16_page_bytes(ctypes.byref(lay))


def bf16_pool_bytes(lay: Layout) -> int:
    return lib().oscar_bf16_pool_bytes(ctypes.byref(lay))


def bf16_decode_workspace_bytes(lay: Layout, batch: int, max_seq_len: int) -> int:
    return lib().oscar_bf16_decode_workspace_bytes(ctypes.byref(lay), batch, max_seq_len)


def bf16_store(lay: Layout, pool: torch.Tensor, page_table: torch.Tensor, k_src: torch.Tensor,
               v_src: torch.Tensor, start_pos: torch.Tensor) -> None:
    """Write k_src / v_src (bf16 [B, n, Hkv, 128], unit stride on the last axis, the same strides
    for both) to positions start_pos[b] + i of the BF16 pool (oscar_bf16_store)."""
    if k_src.dim() != 4 or k_src.shape != v_src.shape or k_src.stride() != v_src.stride():
        raise TypeError("k_src / v_src must be [B, n, Hkv, 128] with identical strides")
    if k_src.stride(3) != 1 or k_src.shape[3] != HEAD_DIM or k_src.shape[2] != lay.num_kv_heads:
        raise TypeError("k_src last axis must be contiguous head_dim; axis 2 the KV heads")
    bsz, n = k_src.shape[0], k_src.shape[1]
    _min_bytes(pool, "pool", bf16_pool_bytes(lay))
    _table(page_table, lay, bsz)
    _rows(start_pos, "start_pos", bsz)
    _check(lib().oscar_bf16_store(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _dev(k_src, "k_src", torch.bfloat16),
        _dev(v_src, "v_src", torch.bfloat16), k_src.stride(0), k_src.stride(1), k_src.stride(2),
        _contig(start_pos, "start_pos", torch.int32), bsz, n, _stream()), "bf16_store")


def bf16_decode_attn(lay: Layout, pool: torch.Tensor, page_table: torch.Tensor,
                     seq_lens: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                     workspace: torch.Tensor, max_seq_len: int,
                     lse: Optional[torch.Tensor] = None, sm_scale: float = 0.0) -> None:
    """Decode attention of q (bf16 [B, Hq, 128]) over the BF16 pool into out (fp32
    [B, Hq, 128]) and optionally lse (fp32 [B, Hq]) (oscar_bf16_decode_attn)."""
    bsz = seq_lens.numel()
    if tuple(q.shape) != (bsz, lay.num_q_heads, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise TypeError("q / out must be [batch, Hq, 128]")
    _min_bytes(pool, "pool", bf16_pool_bytes(lay))
    _table(page_table, lay, bsz)
    if lse is not None:
        _shape(lse, "lse", (bsz, lay.num_q_heads))
    _check(lib().oscar_bf16_decode_attn(
        ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
        _contig(page_table, "page_table", torch.int32), _contig(seq_lens, "seq_lens", torch.int32),
        _contig(q, "q", torch.bfloat16), float(sm_scale), _contig(out, "out", torch.float32),
        None if lse is None else _contig(lse, "lse", torch.float32),
        _contig(workspace, "workspace", torch.uint8), workspace.numel(), bsz, int(max_seq_len),
        _stream()), "bf16_decode_attn")


@dataclasses.dataclass
class Cache:
    """Device buffers of one layer's three-segment cache, allocated with torch."""

    layout: Layout
    pool: torch.Tensor       # uint8 [num_pages, page_bytes]
    sink_k: torch.Tensor     # bf16 [max_seqs, Hkv, 64, 128]
    sink_v: torch.Tensor
    recent_k: torch.Tensor   # bf16 [max_seqs, Hkv, 256, 128]
    recent_v: torch.Tensor

    @classmethod
    def allocate(cls, lay: Layout, device="cuda", zero: bool = True) -> "Cache":
        mk = torch.zeros if zero else torch.empty
        pool = mk((max(lay.num_pages, 1), page_bytes(lay)), dtype=torch.uint8, device=device)
        seg = lambda n: mk((max(lay.max_seqs, 1), lay.num_kv_heads, n, HEAD_DIM),
                           dtype=torch.bfloat16, device=device)
        return cls(lay, pool, seg(SINK_TOKENS), seg(SINK_TOKENS), seg(RECENT_TOKENS),
                   seg(RECENT_TOKENS))


# ----------------------------------------------------------------------------------------------
# memory probes (measurement only: plain reads for the practical HBM ceilings; include/oscar.h)

def probe_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int = 2048) -> None:
    """Stream every byte of ``buf`` once (oscar_probe_read); ``sink``: int32 device tensor of at
    least ``blocks`` entries."""
    _check(lib().oscar_probe_read(_contig(buf, "buf", buf.dtype),
                                  buf.numel() * buf.element_size(),
                                  _contig(sink, "sink", torch.int32), sink.numel(), blocks,
                                  _stream()), "probe_read")


def probe_gather(lay: Layout, pool: torch.Tensor, table_row: torch.Tensor, n_pages: int,
                 pages_per_split: int, sets: int, sink: torch.Tensor, work: int = 0) -> None:
    """Read the INT2 pool blocks of ``n_pages`` pages of one page-table row in the decode kernel's
    order, ``sets`` register sets of page pairs per wave and ``work`` fp32 multiply-adds per pair
    (oscar_probe_gather)."""
    _min_bytes(pool, "pool", pool_bytes(lay))
    if table_row.numel() < n_pages:
        raise TypeError(f"table_row holds {table_row.numel()} entries, needs {n_pages}")
    _check(lib().oscar_probe_gather(ctypes.byref(lay), _contig(pool, "pool", torch.uint8),
                                    _contig(table_row, "table_row", torch.int32), n_pages,
                                    pages_per_split, sets, work,
                                    _contig(sink, "sink", torch.int32),
                                    sink.numel(), _stream()), "probe_gather")
