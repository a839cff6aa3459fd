"""Binding of the benchmark's gather-rate probe (libqsa_probe.so).

Not part of the QSA boundary: bench.py uses it to measure, in the same run and
on the same GPU, how fast 2 KiB micro-blocks can be gathered (from a region
that fits in the L2, uniformly at random from a cache of the workload's size,
and along the attention's own selection lists with no arithmetic).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqsa_probe.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqsa_probe.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.qsa_probe_gather.argtypes = [vp, vp, vp, i64, i64, vp, i64, i32, i64, i32, i32, vp]
        L.qsa_probe_gather.restype = ctypes.c_int
        _lib = L
    return _lib


def gather(k_cache: torch.Tensor, v_cache: torch.Tensor, idx: torch.Tensor, sink: torch.Tensor,
           launch_rows: int = 4096, step: int = 8, pad_kib: int = 96) -> None:
    """Gather, for both KV groups, the blocks that each row of idx names
    (int32 [rows][list_len]) from blocked caches of one sequence
    ([1][2][nblk][...], 2 KiB per block and group).  Asynchronous on the
    current stream."""
    assert k_cache.is_cuda and v_cache.is_cuda and idx.is_cuda and sink.is_cuda
    assert k_cache.dtype == v_cache.dtype == torch.bfloat16 and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert k_cache.shape[0] == 1 and k_cache.shape[1] == 2 and v_cache.shape[:3] == k_cache.shape[:3]
    nblk = k_cache.shape[2]
    assert k_cache.numel() == v_cache.numel() == 2 * nblk * 1024
    assert idx.dtype == torch.int32 and idx.is_contiguous() and idx.dim() == 2
    assert sink.dtype == torch.int32 and sink.numel() >= 65536
    rows, ll = idx.shape
    rc = lib().qsa_probe_gather(torch.cuda.current_stream().cuda_stream, k_cache.data_ptr(), v_cache.data_ptr(),
                                nblk * 2048, nblk, idx.data_ptr(), rows, ll, launch_rows, step, pad_kib,
                                sink.data_ptr())
    if rc != 0:
        raise RuntimeError("qsa_probe_gather failed: hip error %d" % rc)
