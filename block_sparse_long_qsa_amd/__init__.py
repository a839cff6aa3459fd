"""Python binding of the MI355X QSA library (libqsa.so, C ABI in include/qsa.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors supply device pointers; the current torch stream supplies the
HIP stream.  Each function has the name of the C entry point it calls and
raises QSAError on a non-OK status.  If libqsa.so has not been built this
module raises at first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# QSA_LIB_PATH names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree libqsa.so.
LIB_PATH = os.environ.get("QSA_LIB_PATH") or os.path.join(_PKG, "libqsa.so")

(QSA_OP_APPEND, QSA_OP_INDEX, QSA_OP_SELECT, QSA_OP_ATTEND, QSA_OP_FORWARD, QSA_OP_DECODE, QSA_OP_INDEX_SELECT,
 QSA_OP_INDEX_DECODE, QSA_OP_TOKEN_INDEX_SELECT, QSA_OP_TOKEN_INDEX_DECODE, QSA_OP_TRAIN_FORWARD,
 QSA_OP_TRAIN_BACKWARD) = range(12)

STATUS = {0: "QSA_OK", 1: "QSA_ERR_NULL", 2: "QSA_ERR_SHAPE", 3: "QSA_ERR_UNSUPPORTED", 4: "QSA_ERR_ALIGN",
          5: "QSA_ERR_CAPACITY", 6: "QSA_ERR_WORKSPACE", 7: "QSA_ERR_HIP"}

# The C entry points (kept in step with include/qsa.h).
EXPORTS = ["qsa_default_params", "qsa_create", "qsa_destroy", "qsa_get_params", "qsa_workspace_size",
           "qsa_append", "qsa_index", "qsa_select", "qsa_index_select", "qsa_attend", "qsa_dense_attend", "qsa_forward",
           "qsa_decode",
           "qsa_decode_noalloc", "qsa_decode_reuse", "qsa_index_decode", "qsa_token_index_select", "qsa_token_index_decode",
           "qsa_train_forward", "qsa_train_backward_indexer", "qsa_train_backward_attention",
           "qsa_gdn_workspace_size", "qsa_gdn_chunk_prefill", "qsa_gdn_prep", "qsa_gdn_scan",
           "qsa_status_string", "qsa_last_hip_error"]


class QSAError(RuntimeError):
    def __init__(self, status: int, where: str, hip: int = 0):
        self.status = status
        msg = "%s failed: %s" % (where, STATUS.get(status, status))
        if status == 7:
            msg += " (hip error %d)" % hip
        super().__init__(msg)


class Params(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("n_idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("idx_rope_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("budget_blocks", ctypes.c_int32),
                ("topk_cap", ctypes.c_int32), ("max_ctx", ctypes.c_int64), ("rope_theta", ctypes.c_double),
                ("yarn_factor", ctypes.c_double), ("yarn_orig_ctx", ctypes.c_int64)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libqsa.so; raise if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libqsa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.qsa_default_params.argtypes = [ctypes.POINTER(Params)]
    L.qsa_default_params.restype = None
    L.qsa_create.argtypes = [ctypes.POINTER(Params), ctypes.c_int, ctypes.POINTER(vp)]
    L.qsa_create.restype = ctypes.c_int
    L.qsa_destroy.argtypes = [vp]
    L.qsa_destroy.restype = None
    L.qsa_get_params.argtypes = [vp, ctypes.POINTER(Params)]
    L.qsa_get_params.restype = ctypes.c_int
    L.qsa_workspace_size.argtypes = [vp, ctypes.c_int, i32, i64, i64]
    L.qsa_workspace_size.restype = sz
    L.qsa_append.argtypes = [vp, vp, i32, i64, i64] + [vp] * 7
    L.qsa_append.restype = ctypes.c_int
    L.qsa_index.argtypes = [vp, vp, i32, i64, i64] + [vp] * 4 + [sz]
    L.qsa_index.restype = ctypes.c_int
    L.qsa_select.argtypes = [vp, vp, i32, i64, i64, vp, vp]
    L.qsa_select.restype = ctypes.c_int
    L.qsa_index_select.argtypes = [vp, vp, i32, i64, i64] + [vp] * 4 + [sz]
    L.qsa_index_select.restype = ctypes.c_int
    L.qsa_attend.argtypes = [vp, vp, i32, i64, i64] + [vp] * 5
    L.qsa_attend.restype = ctypes.c_int
    L.qsa_dense_attend.argtypes = [vp, vp, i32, i64, i64] + [vp] * 4
    L.qsa_dense_attend.restype = ctypes.c_int
    L.qsa_forward.argtypes = [vp, vp, i32, i64, i64] + [vp] * 12 + [sz]
    L.qsa_forward.restype = ctypes.c_int
    L.qsa_decode.argtypes = [vp, vp, i32, vp, i64] + [vp] * 12 + [sz]
    L.qsa_decode.restype = ctypes.c_int
    L.qsa_decode_noalloc.argtypes = [vp, vp, i32, vp, i64] + [vp] * 11
    L.qsa_decode_noalloc.restype = ctypes.c_int
    L.qsa_decode_reuse.argtypes = [vp, vp, i32, vp, vp, i64] + [vp] * 11 + [sz]
    L.qsa_decode_reuse.restype = ctypes.c_int
    L.qsa_index_decode.argtypes = [vp, vp, i32, vp, i64] + [vp] * 6 + [sz]
    L.qsa_index_decode.restype = ctypes.c_int
    L.qsa_token_index_select.argtypes = [vp, vp, i32, i64, i64] + [vp] * 5 + [sz]
    L.qsa_token_index_select.restype = ctypes.c_int
    L.qsa_token_index_decode.argtypes = [vp, vp, i32, vp, i64] + [vp] * 5 + [sz]
    L.qsa_token_index_decode.restype = ctypes.c_int
    L.qsa_train_forward.argtypes = [vp, vp, i32, i64] + [vp] * 10 + [sz]
    L.qsa_train_forward.restype = ctypes.c_int
    L.qsa_train_backward_indexer.argtypes = [vp, vp, i32, i64] + [vp] * 10 + [sz]
    L.qsa_train_backward_indexer.restype = ctypes.c_int
    L.qsa_train_backward_attention.argtypes = [vp, vp, i32, i64] + [vp] * 10
    L.qsa_train_backward_attention.restype = ctypes.c_int
    L.qsa_gdn_workspace_size.argtypes = [i32, i64, i32, i32]
    L.qsa_gdn_workspace_size.restype = sz
    L.qsa_gdn_chunk_prefill.argtypes = [vp, i32, vp, i64, i64, i32, i32, ctypes.c_float] + [vp] * 9 + [sz]
    L.qsa_gdn_chunk_prefill.restype = ctypes.c_int
    L.qsa_gdn_prep.argtypes = [vp, i32, vp, i64, i64, i32, i32, ctypes.c_float] + [vp] * 5 + [sz]
    L.qsa_gdn_prep.restype = ctypes.c_int
    L.qsa_gdn_scan.argtypes = [vp, i32, vp, i64, i64, i32, i32, ctypes.c_float] + [vp] * 8 + [sz]
    L.qsa_gdn_scan.restype = ctypes.c_int
    L.qsa_status_string.argtypes = [ctypes.c_int]
    L.qsa_status_string.restype = ctypes.c_char_p
    L.qsa_last_hip_error.argtypes = []
    L.qsa_last_hip_error.restype = ctypes.c_int
    _lib_handle = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise QSAError(status, where, lib().qsa_last_hip_error())


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor", numel: Optional[int] = None):
    """Device address of t after checking what the kernels assume of it: a
    contiguous device tensor of the given dtype holding at least `numel`
    elements (the library sees only the pointer, so a host tensor or a short
    buffer would otherwise reach a kernel)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor, got one on %s" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, the call needs %d" % (name, t.numel(), numel))
    return t.data_ptr()


def _bf(t, name, numel: Optional[int] = None):
    return _ptr(t, torch.bfloat16, name, numel)


# Elements per token / per sequence of the layouts in include/qsa.h.
_Q, _KV, _QI, _KI, _ST = 24 * 256, 2 * 256, 4 * 128, 128, 32


def _caches(h, B, k_cache=None, v_cache=None, kbar_cache=None, kpend=None):
    """Pointers of the caches a call passes, each checked against B sequences of
    the handle's capacity (absent ones are None)."""
    n = h.max_ctx
    return (_bf(k_cache, "k_cache", B * 2 * n * 256) if k_cache is not None else None,
            _bf(v_cache, "v_cache", B * 2 * n * 256) if v_cache is not None else None,
            _bf(kbar_cache, "kbar_cache", B * (n // 4) * 128) if kbar_cache is not None else None,
            _bf(kpend, "kpend", B * 4 * 128) if kpend is not None else None)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def default_params(**overrides) -> Params:
    p = Params()
    lib().qsa_default_params(ctypes.byref(p))
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


class Handle:
    """Owns a qsa_handle (the layer parameters and device rotary tables)."""

    def __init__(self, params: Optional[Params] = None, device: int = 0, **overrides):
        if params is None:
            params = default_params(**overrides)
        self.params = params
        self.device = device
        h = ctypes.c_void_p()
        _check(lib().qsa_create(ctypes.byref(params), device, ctypes.byref(h)), "qsa_create")
        self._h = h

    @property
    def ptr(self):
        return self._h

    @property
    def budget(self) -> int:
        return self.params.budget_blocks

    @property
    def max_ctx(self) -> int:
        return self.params.max_ctx

    def close(self):
        if self._h is not None and self._h.value:
            lib().qsa_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qsa_create(params: Optional[Params] = None, device: int = 0, **overrides) -> Handle:
    return Handle(params, device, **overrides)


def qsa_destroy(h: Handle):
    h.close()


def qsa_workspace_size(h: Handle, op: int, batch: int, length: int, q_offset: int) -> int:
    return int(lib().qsa_workspace_size(h.ptr, op, batch, length, q_offset))


def workspace(h: Handle, op: int, batch: int, length: int, q_offset: int, device="cuda") -> torch.Tensor:
    n = qsa_workspace_size(h, op, batch, length, q_offset)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def alloc_caches(h: Handle, batch: int, device="cuda"):
    """Caller-owned caches in the library's layouts (see include/qsa.h)."""
    nb = h.max_ctx // 4
    bf = torch.bfloat16
    return {
        "k_cache": torch.empty((batch, 2, nb, 8, 4, 32), dtype=bf, device=device),
        "v_cache": torch.empty((batch, 2, nb, 256, 4), dtype=bf, device=device),
        "kbar_cache": torch.empty((batch, nb, 128), dtype=bf, device=device),
        "kpend": torch.zeros((batch, 4, 128), dtype=bf, device=device),
    }


def qsa_append(h, B, L, q_offset, k, v, k_idx, k_cache, v_cache, kbar_cache, kpend, stream=None):
    n = B * L
    kc, vc, kb, kp = _caches(h, B, k_cache, v_cache, kbar_cache, kpend)
    _check(lib().qsa_append(h.ptr, _stream(stream), B, L, q_offset, _bf(k, "k", n * _KV), _bf(v, "v", n * _KV),
                            _bf(k_idx, "k_idx", n * _KI), kc, vc, kb, kp), "qsa_append")


def qsa_index(h, B, L, q_offset, q_idx, kbar_cache, scores, ws, stream=None):
    ncol = (q_offset + L + 3) // 4
    _, _, kb, _ = _caches(h, B, kbar_cache=kbar_cache)
    _check(lib().qsa_index(h.ptr, _stream(stream), B, L, q_offset, _bf(q_idx, "q_idx", B * L * _QI), kb,
                           _ptr(scores, torch.float32, "scores", B * L * ncol), _ptr(ws, None, "ws"), _nbytes(ws)),
           "qsa_index")


def qsa_select(h, B, L, q_offset, scores, block_idx, stream=None):
    ncol = (q_offset + L + 3) // 4
    _check(lib().qsa_select(h.ptr, _stream(stream), B, L, q_offset, _ptr(scores, torch.float32, "scores", B * L * ncol),
                            _ptr(block_idx, torch.int32, "block_idx", B * L * h.budget)), "qsa_select")


def qsa_index_select(h, B, L, q_offset, q_idx, kbar_cache, block_idx, ws, stream=None):
    _, _, kb, _ = _caches(h, B, kbar_cache=kbar_cache)
    _check(lib().qsa_index_select(h.ptr, _stream(stream), B, L, q_offset, _bf(q_idx, "q_idx", B * L * _QI), kb,
                                  _ptr(block_idx, torch.int32, "block_idx", B * L * h.budget),
                                  _ptr(ws, None, "ws"), _nbytes(ws)), "qsa_index_select")


def qsa_attend(h, B, L, q_offset, q, k_cache, v_cache, block_idx, out, stream=None):
    kc, vc, _, _ = _caches(h, B, k_cache, v_cache)
    _check(lib().qsa_attend(h.ptr, _stream(stream), B, L, q_offset, _bf(q, "q", B * L * _Q), kc, vc,
                            _ptr(block_idx, torch.int32, "block_idx", B * L * h.budget), _bf(out, "out", B * L * _Q)),
           "qsa_attend")


def qsa_dense_attend(h, B, L, q_offset, q, k_cache, v_cache, out, stream=None):
    kc, vc, _, _ = _caches(h, B, k_cache, v_cache)
    _check(lib().qsa_dense_attend(h.ptr, _stream(stream), B, L, q_offset, _bf(q, "q", B * L * _Q), kc, vc,
                                  _bf(out, "out", B * L * _Q)), "qsa_dense_attend")


def qsa_forward(h, B, L, q_offset, q, k, v, q_idx, k_idx, k_cache, v_cache, kbar_cache, kpend, out, block_idx, ws,
                stream=None):
    n = B * L
    kc, vc, kb, kp = _caches(h, B, k_cache, v_cache, kbar_cache, kpend)
    _check(lib().qsa_forward(h.ptr, _stream(stream), B, L, q_offset, _bf(q, "q", n * _Q), _bf(k, "k", n * _KV),
                             _bf(v, "v", n * _KV), _bf(q_idx, "q_idx", n * _QI), _bf(k_idx, "k_idx", n * _KI),
                             kc, vc, kb, kp, _bf(out, "out", n * _Q),
                             _ptr(block_idx, torch.int32, "block_idx", n * h.budget), _ptr(ws, None, "ws"),
                             _nbytes(ws)), "qsa_forward")


def qsa_decode(h, B, cache_len, ctx_bound, q, k, v, q_idx, k_idx, k_cache, v_cache, kbar_cache, kpend, out,
               block_idx, ws, stream=None):
    kc, vc, kb, kp = _caches(h, B, k_cache, v_cache, kbar_cache, kpend)
    _check(lib().qsa_decode(h.ptr, _stream(stream), B, _ptr(cache_len, torch.int32, "cache_len", B), ctx_bound,
                            _bf(q, "q", B * _Q), _bf(k, "k", B * _KV), _bf(v, "v", B * _KV),
                            _bf(q_idx, "q_idx", B * _QI), _bf(k_idx, "k_idx", B * _KI), kc, vc, kb, kp,
                            _bf(out, "out", B * _Q), _ptr(block_idx, torch.int32, "block_idx", B * h.budget),
                            _ptr(ws, None, "ws"), _nbytes(ws)), "qsa_decode")


# Bytes of the library's per-GPU scratch array behind qsa_decode_noalloc.
NOALLOC_SCRATCH_BYTES = 32 << 20


def qsa_decode_noalloc(h, B, cache_len, ctx_bound, q, k, v, q_idx, k_idx, k_cache, v_cache, kbar_cache, kpend, out,
                       block_idx=None, stream=None):
    kc, vc, kb, kp = _caches(h, B, k_cache, v_cache, kbar_cache, kpend)
    _check(lib().qsa_decode_noalloc(h.ptr, _stream(stream), B, _ptr(cache_len, torch.int32, "cache_len", B),
                                    ctx_bound, _bf(q, "q", B * _Q), _bf(k, "k", B * _KV), _bf(v, "v", B * _KV),
                                    _bf(q_idx, "q_idx", B * _QI), _bf(k_idx, "k_idx", B * _KI), kc, vc, kb, kp,
                                    _bf(out, "out", B * _Q),
                                    _ptr(block_idx, torch.int32, "block_idx", B * h.budget)), "qsa_decode_noalloc")


def qsa_decode_reuse(h, B, cache_len, sel_pos, ctx_bound, q, k, v, k_idx, k_cache, v_cache, kbar_cache, kpend,
                     block_idx, out, ws, stream=None):
    kc, vc, kb, kp = _caches(h, B, k_cache, v_cache, kbar_cache, kpend)
    _check(lib().qsa_decode_reuse(h.ptr, _stream(stream), B, _ptr(cache_len, torch.int32, "cache_len", B),
                                  _ptr(sel_pos, torch.int32, "sel_pos", B), ctx_bound, _bf(q, "q", B * _Q),
                                  _bf(k, "k", B * _KV), _bf(v, "v", B * _KV), _bf(k_idx, "k_idx", B * _KI),
                                  kc, vc, kb, kp, _ptr(block_idx, torch.int32, "block_idx", B * h.budget),
                                  _bf(out, "out", B * _Q), _ptr(ws, None, "ws"), _nbytes(ws)), "qsa_decode_reuse")


def qsa_index_decode(h, B, cache_len, ctx_bound, q_idx, k_idx, kbar_cache, kpend, block_idx, ws, stream=None):
    _, _, kb, kp = _caches(h, B, kbar_cache=kbar_cache, kpend=kpend)
    _check(lib().qsa_index_decode(h.ptr, _stream(stream), B, _ptr(cache_len, torch.int32, "cache_len", B), ctx_bound,
                                  _bf(q_idx, "q_idx", B * _QI), _bf(k_idx, "k_idx", B * _KI), kb, kp,
                                  _ptr(block_idx, torch.int32, "block_idx", B * h.budget), _ptr(ws, None, "ws"),
                                  _nbytes(ws)), "qsa_index_decode")


def alloc_token_keys(h: Handle, batch: int, device="cuda") -> torch.Tensor:
    """Caller-owned token-level indexer key cache [B][max_ctx][128] bf16."""
    return torch.empty((batch, h.max_ctx, 128), dtype=torch.bfloat16, device=device)


def qsa_token_index_select(h, B, L, q_offset, q_idx, k_idx, ktok_cache, token_idx, ws, stream=None):
    _check(lib().qsa_token_index_select(h.ptr, _stream(stream), B, L, q_offset, _bf(q_idx, "q_idx", B * L * _QI),
                                        _bf(k_idx, "k_idx", B * L * _KI),
                                        _bf(ktok_cache, "ktok_cache", B * h.max_ctx * 128),
                                        _ptr(token_idx, torch.int32, "token_idx", B * L * h.budget),
                                        _ptr(ws, None, "ws"), _nbytes(ws)), "qsa_token_index_select")


def qsa_token_index_decode(h, B, cache_len, ctx_bound, q_idx, k_idx, ktok_cache, token_idx, ws, stream=None):
    _check(lib().qsa_token_index_decode(h.ptr, _stream(stream), B, _ptr(cache_len, torch.int32, "cache_len", B),
                                        ctx_bound, _bf(q_idx, "q_idx", B * _QI), _bf(k_idx, "k_idx", B * _KI),
                                        _bf(ktok_cache, "ktok_cache", B * h.max_ctx * 128),
                                        _ptr(token_idx, torch.int32, "token_idx", B * h.budget),
                                        _ptr(ws, None, "ws"), _nbytes(ws)), "qsa_token_index_decode")


def qsa_train_forward(h, B, L, q, q_idx, k_cache, v_cache, kbar_cache, block_idx, out, stats, kl, ws, stream=None):
    n = B * L
    kc, vc, kb, _ = _caches(h, B, k_cache, v_cache, kbar_cache)
    _check(lib().qsa_train_forward(h.ptr, _stream(stream), B, L, _bf(q, "q", n * _Q), _bf(q_idx, "q_idx", n * _QI),
                                   kc, vc, kb, _ptr(block_idx, torch.int32, "block_idx", n * h.budget),
                                   _bf(out, "out", n * _Q), _ptr(stats, torch.float32, "stats", n * _ST),
                                   _ptr(kl, torch.float32, "kl", n), _ptr(ws, None, "ws"), _nbytes(ws)),
           "qsa_train_forward")


def qsa_train_backward_indexer(h, B, L, q, q_idx, k_cache, kbar_cache, block_idx, stats, dkl, dq_idx, dk_idx, ws,
                               stream=None):
    n = B * L
    kc, _, kb, _ = _caches(h, B, k_cache, kbar_cache=kbar_cache)
    _check(lib().qsa_train_backward_indexer(h.ptr, _stream(stream), B, L, _bf(q, "q", n * _Q),
                                            _bf(q_idx, "q_idx", n * _QI), kc, kb,
                                            _ptr(block_idx, torch.int32, "block_idx", n * h.budget),
                                            _ptr(stats, torch.float32, "stats", n * _ST),
                                            _ptr(dkl, torch.float32, "dkl", n),
                                            _ptr(dq_idx, torch.float32, "dq_idx", n * _QI),
                                            _ptr(dk_idx, torch.float32, "dk_idx", n * _KI),
                                            _ptr(ws, None, "ws"), _nbytes(ws)), "qsa_train_backward_indexer")


def qsa_train_backward_attention(h, B, L, q, k_cache, v_cache, block_idx, out, dout, stats, dq, dk, dv,
                                 stream=None):
    n = B * L
    kc, vc, _, _ = _caches(h, B, k_cache, v_cache)
    _check(lib().qsa_train_backward_attention(h.ptr, _stream(stream), B, L, _bf(q, "q", n * _Q), kc, vc,
                                              _ptr(block_idx, torch.int32, "block_idx", n * h.budget),
                                              _bf(out, "out", n * _Q), _bf(dout, "dout", n * _Q),
                                              _ptr(stats, torch.float32, "stats", n * _ST),
                                              _ptr(dq, torch.float32, "dq", n * _Q), _ptr(dk, torch.float32, "dk", n * _KV),
                                              _ptr(dv, torch.float32, "dv", n * _KV)), "qsa_train_backward_attention")


def qsa_gdn_workspace_size(nseq, max_len, hq_heads, hv_heads) -> int:
    return int(lib().qsa_gdn_workspace_size(nseq, max_len, hq_heads, hv_heads))


def _gdn_shapes(q, k, v, g, beta, o):
    n_tok, hq = q.shape[0], q.shape[1]
    hv = v.shape[1]
    checks = [("k", k, q.shape), ("g", g, (n_tok, hv)), ("beta", beta, (n_tok, hv))]
    if o is not None:
        checks.append(("o", o, v.shape))
    for name, t, shape in checks:
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if v.shape[0] != n_tok or q.shape[2] != 128 or v.shape[2] != 128:
        raise ValueError("q, k, v must be [n_tokens][heads][128] with one n_tokens")
    return n_tok, hq, hv


def qsa_gdn_chunk_prefill(nseq, cu_seqlens, max_len, q, k, v, g, beta, scale, initial_state, o, final_state, ws,
                          stream=None):
    """Gated DeltaNet chunked prefill over packed sequences (argument marshalling
    only).  q, k [n_tokens][Hq][128] bf16, v and o [n_tokens][Hv][128] bf16, g and
    beta [n_tokens][Hv] fp32, cu_seqlens int32 [nseq + 1] on the device, states
    [nseq][Hv][128][128] fp32 or None."""
    n_tok, hq, hv = _gdn_shapes(q, k, v, g, beta, o)
    ns = max(nseq, 0) * hv * 128 * 128
    _check(lib().qsa_gdn_chunk_prefill(_stream(stream), nseq,
                                       _ptr(cu_seqlens, torch.int32, "cu_seqlens", max(nseq, 0) + 1), n_tok,
                                       max_len, hq, hv, float(scale), _bf(q, "q"), _bf(k, "k"), _bf(v, "v"),
                                       _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
                                       _ptr(initial_state, torch.float32, "initial_state", ns), _bf(o, "o"),
                                       _ptr(final_state, torch.float32, "final_state", ns), _ptr(ws, None, "ws"),
                                       _nbytes(ws)), "qsa_gdn_chunk_prefill")


def qsa_gdn_prep(nseq, cu_seqlens, max_len, q, k, hv, g, beta, scale, ws, stream=None):
    n_tok, hq = q.shape[0], q.shape[1]
    if tuple(k.shape) != tuple(q.shape) or q.dim() != 3 or q.shape[2] != 128:
        raise ValueError("q, k must be [n_tokens][heads][128] of one shape")
    _check(lib().qsa_gdn_prep(_stream(stream), nseq, _ptr(cu_seqlens, torch.int32, "cu_seqlens", max(nseq, 0) + 1),
                              n_tok, max_len, hq, hv, float(scale), _bf(q, "q"), _bf(k, "k"),
                              _ptr(g, torch.float32, "g", n_tok * hv), _ptr(beta, torch.float32, "beta", n_tok * hv),
                              _ptr(ws, None, "ws"), _nbytes(ws)), "qsa_gdn_prep")


def qsa_gdn_scan(nseq, cu_seqlens, max_len, q, k, v, g, scale, initial_state, o, final_state, ws, stream=None):
    n_tok, hq, hv = _gdn_shapes(q, k, v, g, None, o)
    ns = max(nseq, 0) * hv * 128 * 128
    _check(lib().qsa_gdn_scan(_stream(stream), nseq, _ptr(cu_seqlens, torch.int32, "cu_seqlens", max(nseq, 0) + 1),
                              n_tok, max_len, hq, hv, float(scale), _bf(q, "q"), _bf(k, "k"), _bf(v, "v"),
                              _ptr(g, torch.float32, "g"), _ptr(initial_state, torch.float32, "initial_state", ns),
                              _bf(o, "o"), _ptr(final_state, torch.float32, "final_state", ns), _ptr(ws, None, "ws"),
                              _nbytes(ws)), "qsa_gdn_scan")


def qsa_status_string(status: int) -> str:
    return lib().qsa_status_string(status).decode()


def qsa_last_hip_error() -> int:
    return int(lib().qsa_last_hip_error())
