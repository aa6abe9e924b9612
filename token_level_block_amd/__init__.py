"""Python binding of libuniprefill, the UniPrefill token-selection hot path
for MI355X (gfx950).

Argument marshalling only: every function below forwards to the C ABI declared
in include/uniprefill.h (same names without the `up_` prefix); all of the
path's work runs in the library's HIP kernels.  Buffers may be passed as
torch tensors (their data_ptr() is used) or as raw integer device addresses.
PyTorch supplies device memory and streams and nothing else.

The library is built in-tree by token_level_block_amd/build.py.  If it is
missing, importing this package raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuniprefill.so")

# One HIP runtime per process: torch ships its own libamdhip64.so.7 and HSA
# runtime, with the same sonames as the ROCm install this library links
# against.  Loading torch first makes libuniprefill bind to the runtime torch
# already uses; loading it first would put two runtimes in the process.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing; build it with `python token_level_block_amd/build.py` "
        "(hipcc, gfx950).  There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

UP_OK = 0
UP_ERR_NULL = -1
UP_ERR_SHAPE = -2
UP_ERR_PARAM = -3
UP_ERR_WORKSPACE = -4
UP_ERR_ALIGN = -5
UP_ERR_HIP = -6
UP_SCORES_IN = 1

EXPORTED = ("up_max_blocks", "up_select_workspace_bytes", "up_select_blocks", "up_select_blocks_profiled",
            "up_compact_workspace_bytes", "up_compact", "up_compact_noalloc", "up_scatter_back",
            "up_update_metadata", "up_slot_mapping", "up_write_kv_cache",
            "up_ffn_workspace_bytes", "up_ffn_forward", "up_status_string")


class SelectParams(ctypes.Structure):
    """Mirror of up_select_params."""
    _fields_ = [
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_sink", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("top_p", ctypes.c_double),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class UniPrefillError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_vp = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

_lib.up_max_blocks.restype = _i64
_lib.up_max_blocks.argtypes = [_i32, _i32, _i64]
_lib.up_select_workspace_bytes.restype = _sz
_lib.up_select_workspace_bytes.argtypes = [ctypes.POINTER(SelectParams), _i32, _i64]
_lib.up_select_blocks.restype = ctypes.c_int
_lib.up_select_blocks.argtypes = [ctypes.POINTER(SelectParams), _vp, _i64, _vp, _i64, _vp, _i32, _i64,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.up_select_blocks_profiled.restype = ctypes.c_int
_lib.up_select_blocks_profiled.argtypes = _lib.up_select_blocks.argtypes + [_vp, _vp]
_lib.up_compact_workspace_bytes.restype = _sz
_lib.up_compact_workspace_bytes.argtypes = [_i32, _i64]
_lib.up_compact.restype = ctypes.c_int
_lib.up_compact.argtypes = [_vp, _vp, _i32, _i64, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                            ctypes.POINTER(_i64), _vp, _vp, _vp, _vp, _sz, _vp]
_lib.up_compact_noalloc.restype = ctypes.c_int
_lib.up_compact_noalloc.argtypes = [_vp, _vp, _i32, _i64, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                    ctypes.POINTER(_i64), _vp, _vp, _vp, _vp]
_lib.up_scatter_back.restype = ctypes.c_int
_lib.up_scatter_back.argtypes = [_vp, _i64, _vp, _vp, _i32, _i64, _vp, _i64, _vp]
_lib.up_update_metadata.restype = ctypes.c_int
_lib.up_update_metadata.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp]
_lib.up_slot_mapping.restype = ctypes.c_int
_lib.up_slot_mapping.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i32, _i64, _vp, _vp]
_lib.up_write_kv_cache.restype = ctypes.c_int
_lib.up_write_kv_cache.argtypes = [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _vp, _i64, _vp]
_lib.up_ffn_workspace_bytes.restype = _sz
_lib.up_ffn_workspace_bytes.argtypes = [_i32, _i32, _i64]
_lib.up_ffn_forward.restype = ctypes.c_int
_lib.up_ffn_forward.argtypes = [_i32, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.up_status_string.restype = ctypes.c_char_p
_lib.up_status_string.argtypes = [ctypes.c_int]


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str, raise_on_error: bool):
    if status != UP_OK and raise_on_error:
        raise UniPrefillError(status, where)
    return status


def status_string(status: int) -> str:
    return _lib.up_status_string(int(status)).decode()


def make_params(num_heads_q, num_heads_kv, head_dim, block_size=64, num_sink=128, window=128,
                top_p=0.99, softmax_scale=0.0, scores_in=False) -> SelectParams:
    return SelectParams(num_heads_q, num_heads_kv, head_dim, block_size, num_sink, window,
                        float(top_p), float(softmax_scale), UP_SCORES_IN if scores_in else 0)


def max_blocks(block_size: int, num_reqs: int, max_tokens: int) -> int:
    return int(_lib.up_max_blocks(block_size, num_reqs, max_tokens))


def select_workspace_bytes(params: SelectParams, num_reqs: int, max_tokens: int) -> int:
    return int(_lib.up_select_workspace_bytes(ctypes.byref(params), num_reqs, max_tokens))


def select_blocks(params: SelectParams, q, q_row_stride, k, k_row_stride, cu_seqlens, num_reqs,
                  max_tokens, scores_in, block_scores, block_offsets, keep_block, keep_mask,
                  kept_per_req, workspace, workspace_bytes=None, stream=None, raise_on_error=True):
    """up_select_blocks.  q/k strides are in elements between consecutive tokens."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    pp = ctypes.byref(params) if params is not None else None
    st = _lib.up_select_blocks(pp, _ptr(q), q_row_stride, _ptr(k), k_row_stride,
                               _ptr(cu_seqlens), num_reqs, max_tokens, _ptr(scores_in),
                               _ptr(block_scores), _ptr(block_offsets), _ptr(keep_block),
                               _ptr(keep_mask), _ptr(kept_per_req), _ptr(workspace),
                               workspace_bytes, _stream(stream))
    return _check(st, "up_select_blocks", raise_on_error)


def select_blocks_profiled(params: SelectParams, q, q_row_stride, k, k_row_stride, cu_seqlens, num_reqs,
                           max_tokens, scores_in, block_scores, block_offsets, keep_block, keep_mask,
                           kept_per_req, workspace, score_begin, score_end, workspace_bytes=None, stream=None,
                           raise_on_error=True):
    """up_select_blocks_profiled (include/uniprefill_prof.h): up_select_blocks plus
    two hipEvent_t handles recorded right around the score kernel."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    pp = ctypes.byref(params) if params is not None else None
    st = _lib.up_select_blocks_profiled(pp, _ptr(q), q_row_stride, _ptr(k), k_row_stride,
                                        _ptr(cu_seqlens), num_reqs, max_tokens, _ptr(scores_in),
                                        _ptr(block_scores), _ptr(block_offsets), _ptr(keep_block),
                                        _ptr(keep_mask), _ptr(kept_per_req), _ptr(workspace),
                                        workspace_bytes, _stream(stream), score_begin, score_end)
    return _check(st, "up_select_blocks_profiled", raise_on_error)


def compact_workspace_bytes(num_reqs: int, max_tokens: int) -> int:
    return int(_lib.up_compact_workspace_bytes(num_reqs, max_tokens))


def compact(keep_mask, cu_seqlens, num_reqs, max_tokens, src, dst, row_bytes, index_in, index_out,
            cu_seqlens_out, workspace, workspace_bytes=None, stream=None, raise_on_error=True):
    """up_compact.  src, dst and row_bytes are sequences (one entry per buffer)."""
    nb = len(src)
    if len(dst) != nb or len(row_bytes) != nb:
        raise ValueError("src, dst and row_bytes must have one entry per buffer")
    src_arr = (_vp * max(nb, 1))(*[_ptr(x) for x in src])
    dst_arr = (_vp * max(nb, 1))(*[_ptr(x) for x in dst])
    rb_arr = (_i64 * max(nb, 1))(*[int(x) for x in row_bytes])
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.up_compact(_ptr(keep_mask), _ptr(cu_seqlens), num_reqs, max_tokens, nb, src_arr, dst_arr,
                         rb_arr, _ptr(index_in), _ptr(index_out), _ptr(cu_seqlens_out), _ptr(workspace),
                         workspace_bytes, _stream(stream))
    return _check(st, "up_compact", raise_on_error)


COMPACT_NOALLOC_MAX_TOKENS = 4000000   # UP_COMPACT_NOALLOC_MAX_TOKENS


def compact_noalloc(keep_mask, cu_seqlens, num_reqs, max_tokens, src, dst, row_bytes, index_in, index_out,
                    cu_seqlens_out, stream=None, raise_on_error=True):
    """up_compact_noalloc: up_compact without a workspace (the library's
    per-GPU scratch; at most COMPACT_NOALLOC_MAX_TOKENS tokens)."""
    nb = len(src)
    if len(dst) != nb or len(row_bytes) != nb:
        raise ValueError("src, dst and row_bytes must have one entry per buffer")
    src_arr = (_vp * max(nb, 1))(*[_ptr(x) for x in src])
    dst_arr = (_vp * max(nb, 1))(*[_ptr(x) for x in dst])
    rb_arr = (_i64 * max(nb, 1))(*[int(x) for x in row_bytes])
    st = _lib.up_compact_noalloc(_ptr(keep_mask), _ptr(cu_seqlens), num_reqs, max_tokens, nb, src_arr, dst_arr,
                                 rb_arr, _ptr(index_in), _ptr(index_out), _ptr(cu_seqlens_out), _stream(stream))
    return _check(st, "up_compact_noalloc", raise_on_error)


def scatter_back(compacted, row_bytes, index_map, cu_seqlens_out, num_reqs, max_tokens, full,
                 full_rows, stream=None, raise_on_error=True):
    """up_scatter_back (Eq. 8 carry-forward)."""
    st = _lib.up_scatter_back(_ptr(compacted), row_bytes, _ptr(index_map), _ptr(cu_seqlens_out),
                              num_reqs, max_tokens, _ptr(full), full_rows, _stream(stream))
    return _check(st, "up_scatter_back", raise_on_error)


def update_metadata(layer, num_layers, num_reqs, cu_seqlens_old, cu_seqlens_new, seq_lens,
                    num_actual_tokens, drop_count, drop_layer, drop_len, max_drops, seqused_base,
                    stream=None, raise_on_error=True):
    """up_update_metadata (seq_lens, num_actual_tokens, drop history, Eq. 17 table)."""
    st = _lib.up_update_metadata(layer, num_layers, num_reqs, _ptr(cu_seqlens_old), _ptr(cu_seqlens_new),
                                 _ptr(seq_lens), _ptr(num_actual_tokens), _ptr(drop_count),
                                 _ptr(drop_layer), _ptr(drop_len), max_drops, _ptr(seqused_base),
                                 _stream(stream))
    return _check(st, "up_update_metadata", raise_on_error)


def slot_mapping(block_table, block_table_stride, max_blocks_per_req, kv_block_size, cu_seqlens, seq_lens,
                 num_reqs, max_tokens, slots, stream=None, raise_on_error=True):
    """up_slot_mapping (Eq. 16 per-layer KV cache slots, int64 out)."""
    st = _lib.up_slot_mapping(_ptr(block_table), block_table_stride, max_blocks_per_req, kv_block_size,
                              _ptr(cu_seqlens), _ptr(seq_lens), num_reqs, max_tokens, _ptr(slots),
                              _stream(stream))
    return _check(st, "up_slot_mapping", raise_on_error)


def write_kv_cache(key, key_row_stride, value, value_row_stride, row_bytes, slots, cu_seqlens, num_reqs,
                   max_tokens, key_cache, value_cache, cache_slots, stream=None, raise_on_error=True):
    """up_write_kv_cache (retained rows into the paged cache; strides in bytes)."""
    st = _lib.up_write_kv_cache(_ptr(key), key_row_stride, _ptr(value), value_row_stride, row_bytes,
                                _ptr(slots), _ptr(cu_seqlens), num_reqs, max_tokens, _ptr(key_cache),
                                _ptr(value_cache), cache_slots, _stream(stream))
    return _check(st, "up_write_kv_cache", raise_on_error)


def ffn_workspace_bytes(hidden: int, intermediate: int, rows: int) -> int:
    return int(_lib.up_ffn_workspace_bytes(hidden, intermediate, rows))


def ffn_forward(hidden, intermediate, x, rows, w_gate_up, w_down, y, workspace, workspace_bytes=None,
                stream=None, raise_on_error=True):
    """up_ffn_forward: the gated FFN sublayer on `rows` rows (allocation-free)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.up_ffn_forward(hidden, intermediate, _ptr(x), rows, _ptr(w_gate_up), _ptr(w_down), _ptr(y),
                             _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(st, "up_ffn_forward", raise_on_error)


class FFN:
    """The gated FFN sublayer (hidden D, intermediate F) that runs on the
    retained rows after a drop: holds the two widths and forwards to
    up_ffn_workspace_bytes / up_ffn_forward."""

    def __init__(self, hidden: int, intermediate: int):
        if _lib.up_ffn_workspace_bytes(hidden, intermediate, 0) == 0:
            raise UniPrefillError(UP_ERR_PARAM, "FFN widths")
        self.hidden, self.intermediate = hidden, intermediate

    def workspace_bytes(self, rows: int) -> int:
        return ffn_workspace_bytes(self.hidden, self.intermediate, rows)

    def forward(self, x, rows, w_gate_up, w_down, y, workspace, workspace_bytes=None, stream=None,
                raise_on_error=True):
        return ffn_forward(self.hidden, self.intermediate, x, rows, w_gate_up, w_down, y, workspace,
                           workspace_bytes, stream, raise_on_error)

    def close(self):
        pass
