"""Python binding of libloopvq.so: the LoopVQ decode-attention / encode library for MI355X.

Thin ctypes layer over the C ABI in include/loopvq.h: every function here has the
name of the C entry point it calls and only marshals arguments (tensor data
pointers, the current HIP stream).  All computation runs in the library's HIP
kernels; torch is used for device memory and streams only.  If the shared
library is missing the import of the entry points fails loudly: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libloopvq.so")

LOOPVQ_OK = 0
LOOPVQ_ERR_INVALID_ARG = -1
LOOPVQ_ERR_UNSUPPORTED = -2
LOOPVQ_ERR_MISALIGNED = -3
LOOPVQ_ERR_WORKSPACE = -4
LOOPVQ_ERR_HIP = -5

_I32, _I64, _F32, _F64, _P = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p


class loopvq_config(ctypes.Structure):
    _fields_ = [(n, _I32) for n in (
        "num_layers", "num_loops", "loop_group", "num_q_heads", "num_kv_heads", "head_dim",
        "chans_per_group", "index_bits", "prefix_tokens", "recent_tokens", "page_tokens",
        "codebook_per_loop_group")]


class loopvq_layout(ctypes.Structure):
    _fields_ = [("tile_bytes", _I64), ("kind_bytes", _I64), ("page_bytes", _I64),
                ("pool_head_stride_bytes", _I64), ("pool_bytes", _I64), ("codebook_elems", _I64),
                ("norms_elems", _I64), ("prefix_elems", _I64), ("recent_elems", _I64),
                ("bits_per_elem", _F64)]


class loopvq_encode_args(ctypes.Structure):
    _fields_ = [("layer", _I32), ("loop_group", _I32), ("kind", _I32), ("n_tokens", _I32),
                ("src", _P), ("stride_loop", _I64), ("stride_token", _I64), ("stride_head", _I64),
                ("seq_id", _P), ("vq_pos", _P), ("block_table", _P), ("batch", _I32),
                ("max_pages_per_seq", _I32), ("num_pages", _I64), ("cb", _P), ("cb_norms", _P),
                ("pool", _P), ("out_idx", _P), ("rerank_count", _P)]


class loopvq_evict_args(ctypes.Structure):
    _fields_ = [("batch", _I32), ("max_pages_per_seq", _I32), ("num_pages", _I64), ("k_ring", _P), ("v_ring", _P),
                ("ring_slot", _P), ("vq_pos", _P), ("block_table", _P), ("cb_k", _P), ("cb_v", _P),
                ("norms_k", _P), ("norms_v", _P), ("pool", _P), ("out_idx", _P), ("rerank_count", _P)]


class loopvq_lloyd_args(ctypes.Structure):
    _fields_ = [("layer", _I32), ("cb_set", _I32), ("n_samples", _I32), ("src", _P), ("stride_loop", _I64),
                ("stride_token", _I64), ("stride_head", _I64), ("weight", _P), ("cb", _P), ("cb_norms", _P),
                ("assign", _P), ("cluster_weight", _P), ("distortion", _P), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t), ("rerank_count", _P)]


class loopvq_decode_args(ctypes.Structure):
    _fields_ = [("layer", _I32), ("loop", _I32), ("batch", _I32), ("max_pages_per_seq", _I32),
                ("max_seq_len", _I32), ("num_splits", _I32), ("num_pages", _I64),
                ("q", _P), ("seq_lens", _P), ("block_table", _P), ("pool", _P),
                ("cb_k_prep", _P), ("cb_v_prep", _P), ("k_prefix", _P), ("v_prefix", _P),
                ("k_recent", _P), ("v_recent", _P), ("rot", _P), ("softmax_scale", _F32),
                ("out", _P), ("lse", _P)]


class loopvq_extend_args(ctypes.Structure):
    _fields_ = [("layer", _I32), ("loop", _I32), ("batch", _I32), ("chunk", _I32), ("max_pages_per_seq", _I32),
                ("max_seq_len", _I32), ("num_pages", _I64), ("q", _P), ("k_new", _P), ("v_new", _P),
                ("seq_lens", _P), ("chunk_lens", _P), ("block_table", _P), ("pool", _P), ("cb_k_grp", _P),
                ("cb_v_grp", _P), ("k_prefix", _P), ("v_prefix", _P), ("k_recent", _P), ("v_recent", _P),
                ("rot", _P), ("softmax_scale", _F32), ("out", _P), ("lse", _P)]


EXPORTS = ("loopvq_config_check", "loopvq_bits_per_elem", "loopvq_layout_query", "loopvq_codebook_prepare",
           "loopvq_codebook_prepare_groups",
           "loopvq_encode", "loopvq_evict", "loopvq_lloyd_workspace", "loopvq_lloyd_step",
           "loopvq_lloyd_update",
           "loopvq_decode_attn_workspace", "loopvq_decode_attn", "loopvq_decode_attn_noalloc",
           "loopvq_extend_attn", "loopvq_status_string", "loopvq_last_error")

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with sub_bit_loop_loopvq_amd/build_lib.py "
                               "(or __graft_entry__.build()); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        cfgp = ctypes.POINTER(loopvq_config)
        L.loopvq_config_check.argtypes, L.loopvq_config_check.restype = [cfgp], _I32
        L.loopvq_bits_per_elem.argtypes, L.loopvq_bits_per_elem.restype = [cfgp], _F64
        L.loopvq_layout_query.argtypes = [cfgp, _I32, _I64, ctypes.POINTER(loopvq_layout)]
        L.loopvq_layout_query.restype = _I32
        L.loopvq_codebook_prepare.argtypes, L.loopvq_codebook_prepare.restype = [cfgp, _P, _P, _P, _P], _I32
        L.loopvq_codebook_prepare_groups.argtypes = [cfgp, _P, _P, _P]
        L.loopvq_codebook_prepare_groups.restype = _I32
        L.loopvq_encode.argtypes = [cfgp, ctypes.POINTER(loopvq_encode_args), _P]
        L.loopvq_encode.restype = _I32
        L.loopvq_evict.argtypes = [cfgp, ctypes.POINTER(loopvq_evict_args), _P]
        L.loopvq_evict.restype = _I32
        L.loopvq_lloyd_workspace.argtypes = [cfgp, _I32, ctypes.POINTER(ctypes.c_size_t)]
        L.loopvq_lloyd_workspace.restype = _I32
        L.loopvq_lloyd_step.argtypes = [cfgp, ctypes.POINTER(loopvq_lloyd_args), _P]
        L.loopvq_lloyd_step.restype = _I32
        L.loopvq_lloyd_update.argtypes = [cfgp, ctypes.POINTER(loopvq_lloyd_args), _P]
        L.loopvq_lloyd_update.restype = _I32
        L.loopvq_decode_attn_workspace.argtypes = [cfgp, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]
        L.loopvq_decode_attn_workspace.restype = _I32
        L.loopvq_decode_attn.argtypes = [cfgp, ctypes.POINTER(loopvq_decode_args), _P, ctypes.c_size_t, _P]
        L.loopvq_decode_attn.restype = _I32
        L.loopvq_decode_attn_noalloc.argtypes = [cfgp, ctypes.POINTER(loopvq_decode_args), _P]
        L.loopvq_decode_attn_noalloc.restype = _I32
        L.loopvq_extend_attn.argtypes = [cfgp, ctypes.POINTER(loopvq_extend_args), _P]
        L.loopvq_extend_attn.restype = _I32
        L.loopvq_status_string.argtypes, L.loopvq_status_string.restype = [_I32], ctypes.c_char_p
        L.loopvq_last_error.argtypes, L.loopvq_last_error.restype = [], ctypes.c_char_p
        _lib = L
    return _lib


class LoopVQError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"loopvq status {status} ({loopvq_status_string(status)}): {detail}")
        self.status = status


def _check(status: int) -> None:
    if status != LOOPVQ_OK:
        raise LoopVQError(status, loopvq_last_error())


def _ptr(x) -> int | None:
    """Device (or host) address of a tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(wl=None, **kw) -> loopvq_config:
    """Build a loopvq_config from keyword fields, or from a workload description's sizes."""
    if wl is not None:
        kw = dict(num_layers=wl.layers, num_loops=wl.loops, loop_group=wl.loop_group, num_q_heads=wl.q_heads,
                  num_kv_heads=wl.kv_heads, head_dim=wl.head_dim, chans_per_group=wl.chans,
                  index_bits=wl.index_bits, prefix_tokens=wl.prefix, recent_tokens=wl.recent,
                  page_tokens=wl.page_tokens, codebook_per_loop_group=int(wl.codebook_per_loop_group), **kw)
    return loopvq_config(**kw)


# ----------------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ----------------------------------------------------------------------------------
def loopvq_status_string(status: int) -> str:
    return lib().loopvq_status_string(status).decode()


def loopvq_last_error() -> str:
    return lib().loopvq_last_error().decode()


def loopvq_config_check(cfg: loopvq_config) -> int:
    """Returns the status code (0 = valid) without raising."""
    return lib().loopvq_config_check(ctypes.byref(cfg))


def loopvq_bits_per_elem(cfg: loopvq_config) -> float:
    return lib().loopvq_bits_per_elem(ctypes.byref(cfg))


def loopvq_layout_query(cfg: loopvq_config, batch: int, num_pages: int) -> loopvq_layout:
    out = loopvq_layout()
    _check(lib().loopvq_layout_query(ctypes.byref(cfg), batch, num_pages, ctypes.byref(out)))
    return out


def loopvq_codebook_prepare(cfg, cb, cb_prep, cb_norms=None, stream=None) -> None:
    _check(lib().loopvq_codebook_prepare(ctypes.byref(cfg), _ptr(cb), _ptr(cb_prep), _ptr(cb_norms),
                                         _stream(stream)))


def loopvq_codebook_prepare_groups(cfg, cb, cb_grp, stream=None) -> None:
    _check(lib().loopvq_codebook_prepare_groups(ctypes.byref(cfg), _ptr(cb), _ptr(cb_grp), _stream(stream)))


def loopvq_encode(cfg, *, layer, loop_group, kind, n_tokens, src, stride_loop, stride_token, stride_head,
                  seq_id, vq_pos, block_table, batch, max_pages_per_seq, num_pages, cb, cb_norms, pool,
                  out_idx=None, rerank_count=None, stream=None) -> None:
    a = loopvq_encode_args(layer=layer, loop_group=loop_group, kind=kind, n_tokens=n_tokens, src=_ptr(src),
                           stride_loop=stride_loop, stride_token=stride_token, stride_head=stride_head,
                           seq_id=_ptr(seq_id), vq_pos=_ptr(vq_pos), block_table=_ptr(block_table), batch=batch,
                           max_pages_per_seq=max_pages_per_seq, num_pages=num_pages, cb=_ptr(cb),
                           cb_norms=_ptr(cb_norms), pool=_ptr(pool), out_idx=_ptr(out_idx),
                           rerank_count=_ptr(rerank_count))
    _check(lib().loopvq_encode(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))


def loopvq_evict(cfg, *, batch, max_pages_per_seq, num_pages, k_ring, v_ring, ring_slot, vq_pos, block_table, cb_k,
                 cb_v, norms_k, norms_v, pool, out_idx=None, rerank_count=None, stream=None) -> None:
    a = loopvq_evict_args(batch=batch, max_pages_per_seq=max_pages_per_seq, num_pages=num_pages,
                          k_ring=_ptr(k_ring), v_ring=_ptr(v_ring), ring_slot=_ptr(ring_slot), vq_pos=_ptr(vq_pos),
                          block_table=_ptr(block_table), cb_k=_ptr(cb_k), cb_v=_ptr(cb_v), norms_k=_ptr(norms_k),
                          norms_v=_ptr(norms_v), pool=_ptr(pool), out_idx=_ptr(out_idx),
                          rerank_count=_ptr(rerank_count))
    _check(lib().loopvq_evict(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))


def loopvq_lloyd_workspace(cfg, n_samples: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().loopvq_lloyd_workspace(ctypes.byref(cfg), n_samples, ctypes.byref(n)))
    return n.value


def _lloyd_args(layer, cb_set, n_samples, src, stride_loop, stride_token, stride_head, weight, cb, cb_norms, assign,
                workspace, workspace_bytes, cluster_weight, distortion, rerank_count):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return loopvq_lloyd_args(layer=layer, cb_set=cb_set, n_samples=n_samples, src=_ptr(src), stride_loop=stride_loop,
                             stride_token=stride_token, stride_head=stride_head, weight=_ptr(weight), cb=_ptr(cb),
                             cb_norms=_ptr(cb_norms), assign=_ptr(assign), cluster_weight=_ptr(cluster_weight),
                             distortion=_ptr(distortion), workspace=_ptr(workspace), workspace_bytes=workspace_bytes,
                             rerank_count=_ptr(rerank_count))


def loopvq_lloyd_step(cfg, *, layer, cb_set, n_samples, src, stride_loop, stride_token, stride_head, weight, cb,
                      cb_norms, assign, workspace, workspace_bytes=None, cluster_weight=None, distortion=None,
                      rerank_count=None, stream=None) -> None:
    a = _lloyd_args(layer, cb_set, n_samples, src, stride_loop, stride_token, stride_head, weight, cb, cb_norms,
                    assign, workspace, workspace_bytes, cluster_weight, distortion, rerank_count)
    _check(lib().loopvq_lloyd_step(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))


def loopvq_lloyd_update(cfg, *, layer, cb_set, n_samples, src, stride_loop, stride_token, stride_head, weight, cb,
                        cb_norms, assign, workspace, workspace_bytes=None, cluster_weight=None, distortion=None,
                        stream=None) -> None:
    a = _lloyd_args(layer, cb_set, n_samples, src, stride_loop, stride_token, stride_head, weight, cb, cb_norms,
                    assign, workspace, workspace_bytes, cluster_weight, distortion, None)
    _check(lib().loopvq_lloyd_update(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))


def loopvq_decode_attn_workspace(cfg, batch: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().loopvq_decode_attn_workspace(ctypes.byref(cfg), batch, max_seq_len, ctypes.byref(n)))
    return n.value


def _decode_args(layer, loop, batch, q, seq_lens, max_seq_len, out, block_table, pool, max_pages_per_seq,
                 num_pages, cb_k_prep, cb_v_prep, k_prefix, v_prefix, k_recent, v_recent, rot, softmax_scale, lse,
                 num_splits):
    return loopvq_decode_args(layer=layer, loop=loop, batch=batch, max_pages_per_seq=max_pages_per_seq,
                              max_seq_len=max_seq_len, num_splits=num_splits, num_pages=num_pages, q=_ptr(q),
                              seq_lens=_ptr(seq_lens), block_table=_ptr(block_table), pool=_ptr(pool),
                              cb_k_prep=_ptr(cb_k_prep), cb_v_prep=_ptr(cb_v_prep), k_prefix=_ptr(k_prefix),
                              v_prefix=_ptr(v_prefix), k_recent=_ptr(k_recent), v_recent=_ptr(v_recent),
                              rot=_ptr(rot), softmax_scale=softmax_scale, out=_ptr(out), lse=_ptr(lse))


def loopvq_decode_attn(cfg, *, layer, loop, batch, q, seq_lens, max_seq_len, out, block_table=None, pool=None,
                       max_pages_per_seq=0, num_pages=0, cb_k_prep=None, cb_v_prep=None, k_prefix=None,
                       v_prefix=None, k_recent=None, v_recent=None, rot=None, softmax_scale=0.0, lse=None,
                       num_splits=0, workspace=None, workspace_bytes=None, stream=None) -> None:
    a = _decode_args(layer, loop, batch, q, seq_lens, max_seq_len, out, block_table, pool, max_pages_per_seq,
                     num_pages, cb_k_prep, cb_v_prep, k_prefix, v_prefix, k_recent, v_recent, rot, softmax_scale, lse,
                     num_splits)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().loopvq_decode_attn(ctypes.byref(cfg), ctypes.byref(a), _ptr(workspace), workspace_bytes,
                                    _stream(stream)))


def loopvq_decode_attn_noalloc(cfg, *, layer, loop, batch, q, seq_lens, max_seq_len, out, block_table=None,
                               pool=None, max_pages_per_seq=0, num_pages=0, cb_k_prep=None, cb_v_prep=None,
                               k_prefix=None, v_prefix=None, k_recent=None, v_recent=None, rot=None,
                               softmax_scale=0.0, lse=None, num_splits=0, stream=None) -> None:
    a = _decode_args(layer, loop, batch, q, seq_lens, max_seq_len, out, block_table, pool, max_pages_per_seq,
                     num_pages, cb_k_prep, cb_v_prep, k_prefix, v_prefix, k_recent, v_recent, rot, softmax_scale, lse,
                     num_splits)
    _check(lib().loopvq_decode_attn_noalloc(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))


def loopvq_extend_attn(cfg, *, layer, loop, batch, chunk, q, k_new, v_new, seq_lens, max_seq_len, out,
                       chunk_lens=None, block_table=None, pool=None, max_pages_per_seq=0, num_pages=0,
                       cb_k_grp=None, cb_v_grp=None, k_prefix=None, v_prefix=None, k_recent=None, v_recent=None,
                       rot=None, softmax_scale=0.0, lse=None, stream=None) -> None:
    a = loopvq_extend_args(layer=layer, loop=loop, batch=batch, chunk=chunk, max_pages_per_seq=max_pages_per_seq,
                           max_seq_len=max_seq_len, num_pages=num_pages, q=_ptr(q), k_new=_ptr(k_new),
                           v_new=_ptr(v_new), seq_lens=_ptr(seq_lens), chunk_lens=_ptr(chunk_lens),
                           block_table=_ptr(block_table), pool=_ptr(pool), cb_k_grp=_ptr(cb_k_grp),
                           cb_v_grp=_ptr(cb_v_grp), k_prefix=_ptr(k_prefix), v_prefix=_ptr(v_prefix),
                           k_recent=_ptr(k_recent), v_recent=_ptr(v_recent), rot=_ptr(rot),
                           softmax_scale=softmax_scale, out=_ptr(out), lse=_ptr(lse))
    _check(lib().loopvq_extend_attn(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))

