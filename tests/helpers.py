"""Shared helpers of the parity tests: running the library, calling the oracle
on the same seeded inputs, and the acceptance rules.

Acceptance (stated once, used everywhere):
  * rotated operands (K~ cache, k̄ cache, pending raw keys): bit-exact;
  * scores: |gpu - oracle| <= 1e-4 * max(1, |oracle|) (fp32 MFMA accumulation of
    128 exact bf16 products against an fp64 sum);
  * selections: same count min(budget, o), ascending, -1 padded, all < o; every
    block in the symmetric difference with the oracle's set has an oracle
    score within 1e-3 of the oracle's budget-th score (near-ties may go either
    way under fp32 vs fp64 accumulation);
  * outputs: |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| element-wise, and the
    normwise error ||gpu - oracle|| / ||oracle|| <= 1e-2 per row.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth

SCORE_RTOL = 1e-4
TIE_TOL = 1e-3
OUT_ATOL = 2e-2
OUT_RTOL = 1e-2
OUT_NORMWISE = 1e-2


def bits(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits(t)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def params_for(h_budget: int, yarn: float = 1.0) -> O.Params:
    return O.Params(budget=h_budget, yarn_factor=yarn)


def kcache_tokens(k_cache: torch.Tensor) -> torch.Tensor:
    """Blocked K~ cache [B][2][nb][8][4][32] -> token-major [B][2][nb*4][256]."""
    B, G, nb = k_cache.shape[:3]
    return k_cache.permute(0, 1, 2, 4, 3, 5).reshape(B, G, nb * 4, 256)


def vcache_tokens(v_cache: torch.Tensor) -> torch.Tensor:
    """Blocked V cache [B][2][nb][256][4] -> token-major [B][2][nb*4][256]."""
    B, G, nb = v_cache.shape[:3]
    return v_cache.permute(0, 1, 2, 4, 3).reshape(B, G, nb * 4, 256)


def check_scores(gpu_row: np.ndarray, ora_row: np.ndarray, where=""):
    assert gpu_row.shape == ora_row.shape, where
    err = np.abs(gpu_row.astype(np.float64) - ora_row)
    tol = SCORE_RTOL * np.maximum(1.0, np.abs(ora_row))
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, "%s: %d score(s) off, first block %d gpu %r oracle %r" % (
        where, bad.size, bad[0], gpu_row[bad[0]], ora_row[bad[0]])


def check_selection(gpu_sel: np.ndarray, ora_sel: np.ndarray, ora_scores: np.ndarray, budget: int, o: int,
                    where=""):
    n = min(budget, o)
    g = gpu_sel[:n]
    assert np.all(gpu_sel[n:] == -1), "%s: padding" % where
    assert np.all(g >= 0) and np.all(g < o), "%s: out of range" % where
    assert np.all(np.diff(g) > 0), "%s: not ascending/unique" % where
    a, b = set(g.tolist()), set(ora_sel[:n].tolist())
    if a == b:
        return 0
    kth = np.sort(ora_scores)[::-1][budget - 1]
    for blk in a ^ b:
        assert abs(ora_scores[blk] - kth) <= TIE_TOL, "%s: block %d score %r vs K-th %r" % (
            where, blk, ora_scores[blk], kth)
    return len(a ^ b) // 2


def check_out(gpu: np.ndarray, ref: np.ndarray, where=""):
    gpu = gpu.astype(np.float64)
    err = np.abs(gpu - ref)
    tol = OUT_ATOL + OUT_RTOL * np.abs(ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, "%s: %d element(s) off, first %s gpu %r ref %r" % (
        where, len(bad), tuple(bad[0]), gpu[tuple(bad[0])], ref[tuple(bad[0])])
    nw = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    assert nw <= OUT_NORMWISE, "%s: normwise error %g" % (where, nw)
    return float(err.max()), float(nw)


def oracle_layer(x: dict, seq: int, p: O.Params, n_keys: int = None) -> O.LayerOracle:
    k, v, ki = (bits(x[n][seq]) for n in ("k", "v", "k_idx"))
    if n_keys is not None:
        k, v, ki = k[:n_keys], v[:n_keys], ki[:n_keys]
    return O.LayerOracle(k, v, ki, p)
