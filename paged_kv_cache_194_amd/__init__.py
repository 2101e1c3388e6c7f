"""Python binding of libpagedkv.so: argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks that
their dtypes, shapes and contiguity match what the C ABI expects, and calls the
entry point of the same name on the current HIP stream.  All computation runs
in the library's HIP kernels; if the library is missing this module raises
instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PagedKVError", "BLOCK_SIZE", "lib", "library_path", "kv_append", "paged_decode_attn",
    "varlen_attn", "prefix_import", "prefix_export", "column_copy", "BatchControl",
    "attn_workspace_bytes", "attn_num_splits", "status_string", "last_error", "EXPORTED_SYMBOLS",
    "paged_decode_attn_noalloc", "NOALLOC_SCRATCH_BYTES",
]

BLOCK_SIZE = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libpagedkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP = range(5)
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}

EXPORTED_SYMBOLS = (
    "pkv_kv_append", "pkv_paged_decode_attn", "pkv_varlen_attn", "pkv_prefix_import",
    "pkv_prefix_export", "pkv_attn_workspace_bytes", "pkv_attn_num_splits", "pkv_status_string",
    "pkv_last_error", "pkv_batch_create", "pkv_batch_destroy", "pkv_batch_max_seqs", "pkv_batch_cols",
    "pkv_batch_rows", "pkv_batch_rows_needed", "pkv_batch_seq_new", "pkv_batch_seq_rm",
    "pkv_batch_seq_clone", "pkv_batch_rewind", "pkv_batch_pos", "pkv_batch_floor",
    "pkv_batch_declare_step", "pkv_batch_prepare_step", "pkv_batch_commit_step", "pkv_column_copy",
    "pkv_paged_decode_attn_noalloc",
)

# Bytes of the static split-K scratch behind paged_decode_attn_noalloc (the
# header's PKV_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20


class PagedKVError(ValueError):
    """A non-OK status from libpagedkv.so."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


def _status_name(s: int) -> str:
    return {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE",
            4: "PKV_EHIP"}.get(s, f"status {s}")


_LIB: Optional[ctypes.CDLL] = None

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "pkv_kv_append": (_i32, [_vp, _vp, _i64, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _vp]),
    "pkv_paged_decode_attn": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32,
                                     _vp, _vp, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _i32, _vp,
                                     _sz, _i32, _vp]),
    "pkv_paged_decode_attn_noalloc": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32,
                                             _i32, _vp, _vp, _i32, _i32, _i32, _f32, _i32, _i32, _vp,
                                             _i32, _i32, _vp]),
    "pkv_varlen_attn": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                               _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                               _i32, _vp, _i32, _vp, _sz, _i32, _vp]),
    "pkv_prefix_import": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp,
                                 _i32, _i32, _i32, _vp]),
    "pkv_prefix_export": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _i32, _i32,
                                 _i32, _vp]),
    "pkv_batch_create": (_vp, [_i32, _i32, _i32, _i32]),
    "pkv_batch_destroy": (None, [_vp]),
    "pkv_batch_max_seqs": (_i32, [_vp]),
    "pkv_batch_cols": (_i32, [_vp]),
    "pkv_batch_rows": (_i32, [_vp]),
    "pkv_batch_rows_needed": (_i32, [_vp, _i32, _i32]),
    "pkv_batch_seq_new": (_i32, [_vp, _vp]),
    "pkv_batch_seq_rm": (_i32, [_vp, _i32]),
    "pkv_batch_seq_clone": (_i32, [_vp, _i32, _vp, _vp]),
    "pkv_batch_rewind": (_i32, [_vp, _i32, _i32]),
    "pkv_batch_pos": (_i32, [_vp, _i32, _vp]),
    "pkv_batch_floor": (_i32, [_vp, _i32]),
    "pkv_batch_declare_step": (_i32, [_vp, _vp, _vp, _i32, _i32]),
    "pkv_batch_prepare_step": (_i32, [_vp, _vp, _i32, _vp, _vp]),
    "pkv_batch_commit_step": (_i32, [_vp]),
    "pkv_column_copy": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_attn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_attn_num_splits": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_status_string": (ctypes.c_char_p, [_i32]),
    "pkv_last_error": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        handle = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def status_string(s: int) -> str:
    return lib().pkv_status_string(s).decode()


def last_error() -> str:
    return lib().pkv_last_error().decode()


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PagedKVError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise PagedKVError(PKV_EINVAL, f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise PagedKVError(PKV_EINVAL, msg)


def _dev(*ts) -> None:
    for t in ts:
        if t is not None:
            _need(t.is_cuda, "tensors must be on the GPU")
            _need(t.is_contiguous(), "tensors must be contiguous")


def kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Write ``k_new``/``v_new`` ``[T, Hkv, D]`` into the flat slot view of the caches."""
    _dev(k_cache, v_cache, k_new, v_new, slot_mapping)
    _need(k_new.dim() == 3 and k_new.shape == v_new.shape, "k_new/v_new must be [T, Hkv, D]")
    _need(k_cache.shape == v_cache.shape, "k_cache and v_cache differ in shape")
    _need(k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype, "dtypes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == k_new.shape[0],
          "slot_mapping must be int64 [T]")
    T, H, D = k_new.shape
    _need(tuple(k_cache.shape[-2:]) == (H, D), "cache trailing dims must be (Hkv, D)")
    num_slots = k_cache.numel() // (H * D)
    _check(lib().pkv_kv_append(_ptr(k_cache), _ptr(v_cache), num_slots, _ptr(k_new), _ptr(v_new),
                               T, _ptr(slot_mapping), H, D, _dtype(k_new), _stream(k_new)))


def _paged_cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _need(k_cache.dim() == 4 and k_cache.shape[1] == BLOCK_SIZE,
          "paged caches must be [num_blocks, 16, Hkv, D]")
    _need(k_cache.shape == v_cache.shape and k_cache.dtype == v_cache.dtype,
          "k_cache and v_cache differ in shape or dtype")
    return k_cache.shape[0], k_cache.shape[2], k_cache.shape[3]


def prefix_import(k_cache: torch.Tensor, v_cache: torch.Tensor, k_src: torch.Tensor,
                  v_src: torch.Tensor, block_table: torch.Tensor, n: Optional[int] = None,
                  seqused_k: Optional[torch.Tensor] = None) -> None:
    """Copy positions ``[:n]`` (default: all) of a dense prefill cache
    ``[B, Hkv, S, D]`` into the paged caches through ``block_table`` ``[B, M]``;
    when ``seqused_k`` ``[B]`` is given it is set to ``n`` by the same launch."""
    _dev(k_cache, v_cache, k_src, v_src, block_table, seqused_k)
    nb, H, D = _paged_cache_dims(k_cache, v_cache)
    _need(k_src.dim() == 4 and k_src.shape == v_src.shape, "k_src/v_src must be [B, Hkv, S, D]")
    _need(k_src.dtype == v_src.dtype == k_cache.dtype, "dtypes differ")
    B, Hs, S, Ds = k_src.shape
    _need((Hs, Ds) == (H, D), "source heads / head_dim differ from the cache")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B,
          "block_table must be int32 [B, max_blocks]")
    if seqused_k is not None:
        _need(seqused_k.dtype == torch.int32 and seqused_k.numel() == B, "seqused_k must be int32 [B]")
    n = S if n is None else int(n)
    _check(lib().pkv_prefix_import(_ptr(k_cache), _ptr(v_cache), nb, BLOCK_SIZE, _ptr(k_src),
                                   _ptr(v_src), B, S, n, _ptr(block_table), block_table.shape[1],
                                   _ptr(seqused_k), H, D, _dtype(k_cache), _stream(k_cache)))


def prefix_export(k_dst: torch.Tensor, v_dst: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, block_table: torch.Tensor) -> None:
    """Copy the first ``n`` positions of each sequence out of the paged caches
    into dense ``k_dst``/``v_dst`` ``[B, Hkv, n, D]``."""
    _dev(k_dst, v_dst, k_cache, v_cache, block_table)
    nb, H, D = _paged_cache_dims(k_cache, v_cache)
    _need(k_dst.dim() == 4 and k_dst.shape == v_dst.shape, "k_dst/v_dst must be [B, Hkv, n, D]")
    _need(k_dst.dtype == v_dst.dtype == k_cache.dtype, "dtypes differ")
    B, Hd, n, Dd = k_dst.shape
    _need((Hd, Dd) == (H, D), "destination heads / head_dim differ from the cache")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B,
          "block_table must be int32 [B, max_blocks]")
    _check(lib().pkv_prefix_export(_ptr(k_dst), _ptr(v_dst), _ptr(k_cache), _ptr(v_cache), nb,
                                   BLOCK_SIZE, B, n, _ptr(block_table), block_table.shape[1], H, D,
                                   _dtype(k_cache), _stream(k_cache)))


def column_copy(k_store: torch.Tensor, v_store: torch.Tensor, src_col: int, dst_col: int,
                n_rows: int) -> None:
    """Copy store rows ``[:n_rows]`` of column ``src_col`` to ``dst_col`` in
    ``[rows, cols, Hkv, D]`` K and V stores."""
    _dev(k_store, v_store)
    _need(k_store.dim() == 4 and k_store.shape == v_store.shape and k_store.dtype == v_store.dtype,
          "stores must be equal [rows, cols, Hkv, D]")
    rows, cols, H, D = k_store.shape
    _check(lib().pkv_column_copy(_ptr(k_store), _ptr(v_store), rows, cols, H, D, int(src_col),
                                 int(dst_col), int(n_rows), _dtype(k_store), _stream(k_store)))


class BatchControl:
    """Host bookkeeping of a batched-sequence column store (one column per
    sequence, the last one scratch); see ``pkv_batch_*`` in the C header.

    ``prepare_step`` returns ``(seq_info, slots, num_segments)`` as host
    tensors (int32 ``[2 * max_seqs, 4]``, int64 ``[width]``) ready to be moved
    to the device for ``kv_append`` and ``varlen_attn``."""

    def __init__(self, max_seqs: int, capacity: int, window: int = 0, max_write: int = 1):
        h = lib().pkv_batch_create(max_seqs, capacity, window, max_write)
        if not h:
            raise PagedKVError(PKV_EINVAL, last_error())
        self._h = ctypes.c_void_p(h)
        self.max_seqs = int(lib().pkv_batch_max_seqs(self._h))
        self.cols = int(lib().pkv_batch_cols(self._h))
        self.rows = int(lib().pkv_batch_rows(self._h))
        self.max_segments = 2 * self.max_seqs

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _LIB is not None:
            _LIB.pkv_batch_destroy(h)
            self._h = None

    def _out(self, fn, *args) -> int:
        v = ctypes.c_int32(0)
        _check(fn(self._h, *args, ctypes.byref(v)))
        return int(v.value)

    def seq_new(self) -> int:
        return self._out(lib().pkv_batch_seq_new)

    def seq_rm(self, seq: int) -> None:
        _check(lib().pkv_batch_seq_rm(self._h, int(seq)))

    def seq_clone(self, src: int, stores=()) -> int:
        """A new sequence at ``src``'s position; ``stores`` lists the
        ``(k_store, v_store)`` of every layer whose column is copied."""
        dst, rows = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pkv_batch_seq_clone(self._h, int(src), ctypes.byref(dst), ctypes.byref(rows)))
        for k, v in stores:
            column_copy(k, v, src, dst.value, rows.value)
        return int(dst.value)

    def rewind(self, seq: int, pos: int) -> None:
        _check(lib().pkv_batch_rewind(self._h, int(seq), int(pos)))

    def pos(self, seq: int) -> int:
        return self._out(lib().pkv_batch_pos, int(seq))

    def floor(self, seq: int) -> int:
        return int(lib().pkv_batch_floor(self._h, int(seq)))

    def rows_needed(self, step_width: int, row_step: int = 256) -> int:
        return int(lib().pkv_batch_rows_needed(self._h, int(step_width), int(row_step)))

    def declare_step(self, seqs, n_tokens, width: Optional[int] = None) -> None:
        seqs = [int(x) for x in seqs]
        n_tokens = [int(x) for x in n_tokens]
        _need(len(seqs) == len(n_tokens), "one token count per sequence")
        width = sum(n_tokens) if width is None else int(width)
        a = (ctypes.c_int32 * max(1, len(seqs)))(*seqs)
        b = (ctypes.c_int32 * max(1, len(n_tokens)))(*n_tokens)
        _check(lib().pkv_batch_declare_step(self._h, a, b, len(seqs), width))
        self._width = width

    def prepare_step(self):
        info = torch.zeros((self.max_segments, 4), dtype=torch.int32)
        slots = torch.zeros((max(1, self._width),), dtype=torch.int64)[:self._width]
        n = ctypes.c_int32(0)
        _check(lib().pkv_batch_prepare_step(self._h, ctypes.c_void_p(info.data_ptr()), self.max_segments,
                                            ctypes.c_void_p(slots.data_ptr()), ctypes.byref(n)))
        return info, slots, int(n.value)

    def commit_step(self) -> None:
        _check(lib().pkv_batch_commit_step(self._h))


def attn_workspace_bytes(units: int, max_seqlen_q: int, max_seqlen_k: int, q_heads: int,
                         kv_heads: int, head_dim: int, num_splits: int = 0) -> int:
    return int(lib().pkv_attn_workspace_bytes(units, max_seqlen_q, max_seqlen_k, q_heads,
                                              kv_heads, head_dim, num_splits))


def attn_num_splits(units: int, max_seqlen_q: int, max_seqlen_k: int, q_heads: int,
                    kv_heads: int, head_dim: int, num_splits: int = 0) -> int:
    return int(lib().pkv_attn_num_splits(units, max_seqlen_q, max_seqlen_k, q_heads, kv_heads,
                                         head_dim, num_splits))


def _workspace(ws: Optional[torch.Tensor], need: int, like: torch.Tensor):
    if need == 0:
        return ws, 0 if ws is None else ws.numel() * ws.element_size()
    if ws is None:
        ws = torch.zeros(need, dtype=torch.uint8, device=like.device)   # counters start at 0
    _dev(ws)
    return ws, ws.numel() * ws.element_size()


def paged_decode_attn(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, block_table: torch.Tensor, seqused_k: torch.Tensor,
                      max_seqlen_k: int, softmax_scale: Optional[float] = None,
                      causal: bool = False, window: int = 0, num_splits: int = 0,
                      workspace: Optional[torch.Tensor] = None,
                      k_new: Optional[torch.Tensor] = None,
                      v_new: Optional[torch.Tensor] = None,
                      kv_start: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One query per sequence: ``q``/``out`` ``[B, Hq, D]`` over ``[NB, 16, Hkv, D]`` caches.
    With ``k_new``/``v_new`` ``[B, Hkv, D]`` the token is appended at position
    ``seqused_k[b] - 1`` first.  ``kv_start`` int32 ``[B]``: left-padding bounds."""
    _dev(out, q, k_cache, v_cache, block_table, seqused_k, k_new, v_new, kv_start)
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [B, Hq, D]")
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "caches must be [NB, 16, Hkv, D]")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2, "block_table must be int32 [B, W]")
    _need(seqused_k.dtype == torch.int32, "seqused_k must be int32")
    B, Hq, D = q.shape
    NB, BS, Hkv, Dk = k_cache.shape
    _need(Dk == D and block_table.shape[0] == B and seqused_k.numel() == B, "shape mismatch")
    _need(q.dtype == k_cache.dtype == v_cache.dtype == out.dtype, "dtypes differ")
    if k_new is not None or v_new is not None:
        _need(k_new is not None and v_new is not None, "give both k_new and v_new")
        _need(tuple(k_new.shape) == (B, Hkv, D) and k_new.shape == v_new.shape, "k_new/v_new must be [B, Hkv, D]")
        _need(k_new.dtype == v_new.dtype == q.dtype, "dtypes differ")
    if kv_start is not None:
        _need(kv_start.dtype == torch.int32 and kv_start.numel() == B, "kv_start must be int32 [B]")
    scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    need = attn_workspace_bytes(B, 1, max_seqlen_k, Hq, Hkv, D, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q)
    _check(lib().pkv_paged_decode_attn(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), NB, BS, _ptr(block_table),
        block_table.shape[1], _ptr(seqused_k), B, int(max_seqlen_k), _ptr(k_new), _ptr(v_new),
        Hq, Hkv, D, scale, int(bool(causal)), int(window), _ptr(kv_start), int(num_splits),
        _ptr(workspace), ws_bytes, _dtype(q), _stream(q)))
    return out


def paged_decode_attn_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                              v_cache: torch.Tensor, block_table: torch.Tensor, seqused_k: torch.Tensor,
                              max_seqlen_k: int, softmax_scale: Optional[float] = None,
                              causal: bool = False, window: int = 0, num_splits: int = 0,
                              k_new: Optional[torch.Tensor] = None,
                              v_new: Optional[torch.Tensor] = None,
                              kv_start: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``paged_decode_attn`` without a workspace: the library's static device
    scratch (``NOALLOC_SCRATCH_BYTES`` per GPU) holds the split-K partials, so
    nothing is allocated.  Calls that overlap in time on one GPU race."""
    _dev(out, q, k_cache, v_cache, block_table, seqused_k, k_new, v_new, kv_start)
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [B, Hq, D]")
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "caches must be [NB, 16, Hkv, D]")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2, "block_table must be int32 [B, W]")
    _need(seqused_k.dtype == torch.int32, "seqused_k must be int32")
    B, Hq, D = q.shape
    NB, BS, Hkv, Dk = k_cache.shape
    _need(Dk == D and block_table.shape[0] == B and seqused_k.numel() == B, "shape mismatch")
    _need(q.dtype == k_cache.dtype == v_cache.dtype == out.dtype, "dtypes differ")
    if k_new is not None or v_new is not None:
        _need(k_new is not None and v_new is not None, "give both k_new and v_new")
        _need(tuple(k_new.shape) == (B, Hkv, D) and k_new.shape == v_new.shape, "k_new/v_new must be [B, Hkv, D]")
        _need(k_new.dtype == v_new.dtype == q.dtype, "dtypes differ")
    if kv_start is not None:
        _need(kv_start.dtype == torch.int32 and kv_start.numel() == B, "kv_start must be int32 [B]")
    scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    _check(lib().pkv_paged_decode_attn_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), NB, BS, _ptr(block_table),
        block_table.shape[1], _ptr(seqused_k), B, int(max_seqlen_k), _ptr(k_new), _ptr(v_new),
        Hq, Hkv, D, scale, int(bool(causal)), int(window), _ptr(kv_start), int(num_splits),
        _dtype(q), _stream(q)))
    return out


def varlen_attn(out: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                max_seqlen_q: int, max_seqlen_k: int,
                cu_seqlens_q: Optional[torch.Tensor] = None,
                seqused_k: Optional[torch.Tensor] = None,
                block_table: Optional[torch.Tensor] = None,
                seq_info: Optional[torch.Tensor] = None,
                softmax_scale: Optional[float] = None, causal: bool = False, window: int = 0,
                num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                kv_start: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed rows ``q``/``out`` ``[total_q, Hq, D]`` over a paged cache
    (``cu_seqlens_q``, ``seqused_k``, ``block_table``; ``k``/``v`` ``[NB, 16, Hkv, D]``)
    or a column store (``seq_info`` ``[S, 4]``; ``k``/``v`` ``[rows, cols, Hkv, D]``).
    ``kv_start`` int32, one per sequence or segment: left-padding bounds."""
    _dev(out, q, k, v, cu_seqlens_q, seqused_k, block_table, seq_info, kv_start)
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [total_q, Hq, D]")
    _need(k.dim() == 4 and k.shape == v.shape, "k/v must be 4-d and equal in shape")
    _need(q.dtype == k.dtype == v.dtype == out.dtype, "dtypes differ")
    total_q, Hq, D = q.shape
    _need(k.shape[3] == D, "head_dim mismatch")
    Hkv = k.shape[2]
    scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    nb = bs = mb = rows = cols = 0
    num_seqs = num_segments = 0
    if block_table is not None:
        _need(seq_info is None, "give block_table or seq_info, not both")
        _need(cu_seqlens_q is not None and seqused_k is not None, "paged mode needs cu_seqlens_q and seqused_k")
        _need(block_table.dtype == cu_seqlens_q.dtype == seqused_k.dtype == torch.int32, "index tensors must be int32")
        num_seqs = seqused_k.numel()
        _need(cu_seqlens_q.numel() == num_seqs + 1 and block_table.shape[0] == num_seqs, "shape mismatch")
        nb, bs = k.shape[0], k.shape[1]
        mb = block_table.shape[1]
        units = num_seqs
    else:
        _need(seq_info is not None, "give block_table or seq_info")
        _need(seq_info.dtype == torch.int32 and seq_info.dim() == 2 and seq_info.shape[1] == 4,
              "seq_info must be int32 [S, 4]")
        num_segments = seq_info.shape[0]
        rows, cols = k.shape[0], k.shape[1]
        units = num_segments
    if kv_start is not None:
        _need(kv_start.dtype == torch.int32 and kv_start.numel() == units,
              "kv_start must be int32, one per sequence or segment")
    need = attn_workspace_bytes(units, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q)
    _check(lib().pkv_varlen_attn(
        _ptr(out), _ptr(q), total_q, _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(seqused_k),
        num_seqs, _ptr(block_table), mb, nb, bs, _ptr(seq_info), num_segments, rows, cols,
        int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D, scale, int(bool(causal)), int(window),
        _ptr(kv_start), int(num_splits), _ptr(workspace), ws_bytes, _dtype(q), _stream(q)))
    return out
