"""CPU oracle for one Qwen Sparse Attention (QSA) layer -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import, call or link anything under ``oracle/``.  The HIP
library never touches it, and it shares no code with the HIP library.

This is a plain, slow, step-by-step implementation of what the layer computes,
in fp64 wherever the pages leave the precision open.  Sources (web pages on the
Qwen3.8-Flash-Next release):

  [PKR] discuss.pytorch.kr, "Qwen3.8-Flash-Next, 1/9의 학습 비용으로
        Qwen3.7-Plus(397B-A17B) 수준에 도달한 125B-A6B 모델"
          - spec table under "모델 전체 구조: 네 층 중 셋은 GDN, 하나는 QSA"
            (rows Qwen Sparse Attention / QSA 인덱서 / QSA 예산 / 컨텍스트 길이)
          - section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션"
            (mean-pooled micro-blocks, compression before RoPE, score I_ib,
            block-causal scoring, K = 2048 / r = 4 / 512 blocks, tail included)
          - section "100만 토큰까지 늘리기" (rope_parameters block)
  [LMF] llmfeed.kr, "Qwen 팀, 새 구조를 적용한 Qwen3.8-Flash-Next 공개 가중치로
        출시", section "규모와 구조" (QSA bullet)
  [YaRN] Peng et al., "YaRN: Efficient Context Window Extension of Large
        Language Models" (2023): NTK-by-parts ramp and attention temperature.

Readings of points the pages leave open are listed in the repository's design
notes; each function names the one it applies.

Parity status: every function below is pinned by the non-GPU tests (closed
forms, brute force on tiny inputs, a library routine on special cases, planted
needles); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_SO = os.path.join(_BUILD, "liboracle_rope.so")
_lock = threading.Lock()
_lib_handle = None


def build_helper(force: bool = False) -> str:
    """Compile the libm table helper (plain C, gcc)."""
    os.makedirs(_BUILD, exist_ok=True)
    src = os.path.join(_HERE, "rope_tables.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-builtin", "-ffp-contract=off", "-fPIC", "-shared",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    with _lock:
        if _lib_handle is None:
            lib = ctypes.CDLL(build_helper())
            lib.oracle_rope_table.restype = None
            lib.oracle_rope_table.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
            _lib_handle = lib
    return _lib_handle


# ----------------------------------------------------------------------------
# Layer parameters  ([PKR] spec table; [LMF] "규모와 구조"; [PKR] "100만 토큰까지 늘리기")
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Params:
    n_q_heads: int = 24
    n_kv_heads: int = 2
    head_dim: int = 256
    rope_dim: int = 64            # rotary dims of the core heads (partial factor 0.25 of 256)
    n_idx_heads: int = 4
    idx_dim: int = 128
    idx_rope_dim: int = 64        # reading: the indexer rotates its first 64 dims too
    block: int = 4                # micro-block size r
    budget: int = 512             # K / r = 2048 / 4 blocks
    rope_theta: float = 1e7
    yarn_factor: float = 1.0      # 1 = native context, 4 = YaRN to 1M
    yarn_orig_ctx: int = 262144
    yarn_beta_fast: float = 32.0  # [YaRN] ramp bounds (alpha = 1, beta = 32)
    yarn_beta_slow: float = 1.0


# ----------------------------------------------------------------------------
# bf16 <-> fp32
# ----------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (RNE), returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# Rotary tables  ([PKR] "100만 토큰까지 늘리기": theta 1e7, partial 0.25,
# mrope sections [11, 11, 10]; for text all three sections share one position,
# so the rotation is plain 1-D RoPE over 32 frequencies)
# ----------------------------------------------------------------------------
def inv_freq(p: Params) -> np.ndarray:
    """Per-pair angular frequencies (fp64), YaRN-adjusted when yarn_factor > 1.

    omega_j = theta^(-2j/64).  Under YaRN ([YaRN] NTK-by-parts) each pair is
    blended between interpolation (omega/s) and extrapolation (omega) by a ramp
    over r_j = L_orig / lambda_j, lambda_j = 2*pi / omega_j.
    """
    n = p.rope_dim // 2
    out = np.empty(n, dtype=np.float64)
    for j in range(n):
        w = math.pow(p.rope_theta, -(2.0 * j) / float(p.rope_dim))
        if p.yarn_factor > 1.0:
            wavelength = 2.0 * math.pi / w
            r = float(p.yarn_orig_ctx) / wavelength
            g = (r - p.yarn_beta_slow) / (p.yarn_beta_fast - p.yarn_beta_slow)
            g = min(max(g, 0.0), 1.0)
            w = (1.0 - g) * w / p.yarn_factor + g * w
        out[j] = w
    return out


def rope_table(positions: np.ndarray, p: Params):
    """fp32 cos/sin of position * omega_j, each evaluated in fp64 by host libm."""
    f = np.ascontiguousarray(inv_freq(p))
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    n = f.shape[0]
    c = np.empty((pos.shape[0], n), dtype=np.float32)
    s = np.empty((pos.shape[0], n), dtype=np.float32)
    _lib().oracle_rope_table(f.ctypes.data, n, pos.ctypes.data, pos.shape[0], c.ctypes.data, s.ctypes.data)
    return c, s


def rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the first 2*n dims of the last axis, in fp32.

    x: fp32 [..., D]; cos/sin: fp32 [..., n] broadcastable to x[..., :n].
    Pairs are (j, j+n).  Every product and sum is a separately rounded fp32
    operation: x'_j = a*c - b*s, x'_{j+n} = b*c + a*s with a = x_j, b = x_{j+n}.
    Remaining dims pass through.  Returns fp32 (not yet rounded to bf16).
    """
    n = cos.shape[-1]
    x = np.asarray(x, dtype=np.float32)
    out = x.copy()
    a = x[..., :n]
    b = x[..., n:2 * n]
    ac = (a * cos).astype(np.float32)
    bs = (b * sin).astype(np.float32)
    bc = (b * cos).astype(np.float32)
    as_ = (a * sin).astype(np.float32)
    out[..., :n] = (ac - bs).astype(np.float32)
    out[..., n:2 * n] = (bc + as_).astype(np.float32)
    return out


def softmax_scale(p: Params) -> float:
    """1/sqrt(head_dim), times the YaRN temperature (0.1 ln s + 1)^2 when s > 1."""
    sigma = 1.0 / math.sqrt(p.head_dim)
    if p.yarn_factor > 1.0:
        m = 0.1 * math.log(p.yarn_factor) + 1.0
        sigma *= m * m
    return sigma


# ----------------------------------------------------------------------------
# Indexer operands  ([PKR] "QSA: ..." section: keys are split into
# non-overlapping micro-blocks of r tokens and mean-pooled; compression comes
# before the positional encoding, the pooled key takes the block-start position)
# ----------------------------------------------------------------------------
def pool_block_keys(k_idx: np.ndarray, block: int = 4) -> np.ndarray:
    """Mean of each complete micro-block of raw indexer keys, fp32.

    k_idx: fp32 [n_tok][128].  The sum runs in token order with fp32 rounding at
    each step, then is scaled by 1/r.  Tokens of an incomplete last block are
    dropped (only fully observed blocks are scored).
    """
    nb = k_idx.shape[0] // block
    acc = k_idx[0:nb * block:block].astype(np.float32).copy()
    for t in range(1, block):
        acc = (acc + k_idx[t:nb * block:block]).astype(np.float32)
    return (acc * np.float32(1.0 / block)).astype(np.float32)


def indexer_keys(k_idx_bits: np.ndarray, p: Params) -> np.ndarray:
    """Pooled, rotated, bf16-rounded indexer keys k̄[b] for every complete block.

    k_idx_bits: uint16 [n_tok][128].  Returns fp32 (bf16 values) [n_tok//4][128].
    """
    raw = bf16_bits_to_f32(k_idx_bits)
    pooled = pool_block_keys(raw, p.block)
    nb = pooled.shape[0]
    c, s = rope_table(np.arange(nb, dtype=np.int64) * p.block, p)
    return bf16_round(rotate(pooled, c, s))


def indexer_queries(q_idx_bits: np.ndarray, positions: np.ndarray, p: Params) -> np.ndarray:
    """Rotated, bf16-rounded indexer queries. q_idx_bits: uint16 [n][4][128]."""
    c, s = rope_table(positions, p)
    return bf16_round(rotate(bf16_bits_to_f32(q_idx_bits), c[:, None, :], s[:, None, :]))


def core_rotate(x_bits: np.ndarray, positions: np.ndarray, p: Params) -> np.ndarray:
    """Rotated, bf16-rounded core q or k heads. x_bits: uint16 [n][H][256]."""
    c, s = rope_table(positions, p)
    return bf16_round(rotate(bf16_bits_to_f32(x_bits), c[:, None, :], s[:, None, :]))


# ----------------------------------------------------------------------------
# Score and selection  ([PKR] "QSA: ..." section, equation I_ib; budget and
# always-included tail of the last incomplete block)
# ----------------------------------------------------------------------------
def own_block(pos: int, p: Params) -> int:
    return pos // p.block


def block_scores(qt_idx: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """I[b] = sum_h ReLU(<q~_h, k̄_b>) in fp64.  qt_idx [4][128], kbar [o][128]."""
    logits = qt_idx.astype(np.float64) @ kbar.astype(np.float64).T      # [4][o]
    return np.maximum(logits, 0.0).sum(axis=0)


def select_blocks(scores: np.ndarray, budget: int) -> np.ndarray:
    """Top-min(budget, o) candidates under (score desc, block desc), ascending, -1 padded."""
    o = scores.shape[0]
    out = np.full(budget, -1, dtype=np.int32)
    if o <= budget:
        out[:o] = np.arange(o, dtype=np.int32)
        return out
    blocks = np.arange(o)
    order = np.lexsort((-blocks, -scores))   # primary: score desc; secondary: block desc
    out[:] = np.sort(order[:budget]).astype(np.int32)
    return out


def token_set(sel: np.ndarray, pos: int, p: Params) -> np.ndarray:
    """Tokens attended by query `pos`: the selected blocks' tokens, then 4*o(pos)..pos."""
    sel = sel[sel >= 0].astype(np.int64)
    blk = (sel[:, None] * p.block + np.arange(p.block)[None, :]).reshape(-1)
    own = np.arange(own_block(pos, p) * p.block, pos + 1, dtype=np.int64)
    return np.concatenate([blk, own])


def token_set_reused(sel: np.ndarray, sel_pos: int, pos: int, p: Params) -> np.ndarray:
    """Tokens attended by query `pos` that reuses the selection made for an
    earlier query at `sel_pos` <= pos ([PKR] section on the MTP module: top-k
    indices reused across speculative decoding steps).  Reading: the reused
    blocks (those before sel_pos's own block) keep their meaning, and the query
    attends every token from the start of sel_pos's own block up to itself --
    the own-block rule widened to cover the blocks completed since the
    selection.  With sel_pos = pos this is token_set."""
    o0 = own_block(sel_pos, p)
    sel = sel[(sel >= 0) & (sel < o0)].astype(np.int64)
    blk = (sel[:, None] * p.block + np.arange(p.block)[None, :]).reshape(-1)
    tail = np.arange(o0 * p.block, pos + 1, dtype=np.int64)
    return np.concatenate([blk, tail])


def attend(qt: np.ndarray, kt: np.ndarray, v: np.ndarray, sigma: float, p: Params) -> np.ndarray:
    """Softmax attention of each query head over the given tokens, fp64.

    qt [24][256] rotated queries; kt, v [T][2][256] rotated keys and values.
    Query head h reads KV head h // (24 / 2).
    """
    grp = p.n_q_heads // p.n_kv_heads
    out = np.empty((p.n_q_heads, p.head_dim), dtype=np.float64)
    for g in range(p.n_kv_heads):
        q = qt[g * grp:(g + 1) * grp].astype(np.float64)        # [12][256]
        k = kt[:, g].astype(np.float64)                         # [T][256]
        vv = v[:, g].astype(np.float64)
        z = sigma * (q @ k.T)                                   # [12][T]
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z)
        out[g * grp:(g + 1) * grp] = (e @ vv) / e.sum(axis=1, keepdims=True)
    return out


def token_index_keys(k_idx_bits: np.ndarray, p: Params) -> np.ndarray:
    """Token-level indexer keys: each raw indexer key rotated at its own position
    and rounded to bf16 (indexer_keys with one-token blocks).  fp32 [n_tok][128]."""
    return indexer_keys(k_idx_bits, dataclasses.replace(p, block=1))


def token_index_rows(q_idx_bits: np.ndarray, k_idx_bits: np.ndarray, positions, p: Params):
    """Token-level indexer, compression ratio r = 1 ([PKR] "QSA: ..." section: the
    per-token indexer of DeepSeek-V3.2's DSA, O(n^2), that pooling r tokens per
    key replaces).  Reading: the same score and selection rules with every token
    its own block -- keys rotated at their own positions (pooling of one token is
    the identity), query p scores every t < p, keeps the top min(budget, p)
    under (score desc, t desc), ascending, -1 padded.

    q_idx_bits: uint16 [n][4][128] for the given positions; k_idx_bits: uint16
    [n_tok][128] for positions 0..n_tok-1.  Returns (sel int32 [n][budget],
    list of fp64 score arrays)."""
    pt = dataclasses.replace(p, block=1)
    keys = token_index_keys(k_idx_bits, p)
    sels, scs = [], []
    for pos, qb in zip(positions, q_idx_bits):
        pos = int(pos)
        qt = indexer_queries(np.asarray(qb)[None], np.array([pos]), pt)[0]
        sc = block_scores(qt, keys[:pos])
        sels.append(select_blocks(sc, pt.budget))
        scs.append(sc)
    return np.stack(sels), scs


# ----------------------------------------------------------------------------
# Whole layer, row by row
# ----------------------------------------------------------------------------
class LayerOracle:
    """QSA rows for one sequence.

    k_bits, v_bits: uint16 [n_keys][2][256]; k_idx_bits: uint16 [n_keys][128]
    hold the keys of positions 0..n_keys-1.  A query at position p uses keys
    0..p only.  Queries are given per row.
    """

    def __init__(self, k_bits, v_bits, k_idx_bits, p: Params):
        self.p = p
        self.k_bits = k_bits
        self.v = bf16_bits_to_f32(v_bits)
        self.n_keys = k_bits.shape[0]
        self.kbar = indexer_keys(k_idx_bits, p)
        self.sigma = softmax_scale(p)

    def row(self, pos: int, q_bits: np.ndarray, q_idx_bits: np.ndarray):
        """(out fp64 [24][256], selected blocks int32 [budget], scores fp64 [o])."""
        p = self.p
        assert 0 <= pos < self.n_keys
        o = own_block(pos, p)
        qt_idx = indexer_queries(q_idx_bits[None], np.array([pos]), p)[0]
        scores = block_scores(qt_idx, self.kbar[:o])
        sel = select_blocks(scores, p.budget)
        toks = token_set(sel, pos, p)
        kt = core_rotate(self.k_bits[toks], toks, p)
        qt = core_rotate(q_bits[None], np.array([pos]), p)[0]
        out = attend(qt, kt, self.v[toks], self.sigma, p)
        return out, sel, scores

    def row_reused(self, pos: int, q_bits: np.ndarray, sel: np.ndarray, sel_pos: int):
        """Output fp64 [24][256] of query `pos` attending with the selection
        `sel` that was made for position sel_pos (token_set_reused)."""
        p = self.p
        assert 0 <= sel_pos <= pos < self.n_keys
        toks = token_set_reused(np.asarray(sel), sel_pos, pos, p)
        kt = core_rotate(self.k_bits[toks], toks, p)
        qt = core_rotate(q_bits[None], np.array([pos]), p)[0]
        return attend(qt, kt, self.v[toks], self.sigma, p)


def prefill_rows(q_bits, k_bits, v_bits, q_idx_bits, k_idx_bits, rows, p: Params, q_offset: int = 0):
    """Oracle rows of a prefill over one sequence.

    Keys cover positions 0..n_keys-1; q_bits/q_idx_bits cover positions
    q_offset..q_offset+Lq-1; `rows` are indices into the query arrays.
    Returns (out fp64 [n][24][256], sel int32 [n][budget], list of score arrays).
    """
    lay = LayerOracle(k_bits, v_bits, k_idx_bits, p)
    outs, sels, scs = [], [], []
    for r in rows:
        o, s, sc = lay.row(q_offset + int(r), q_bits[int(r)], q_idx_bits[int(r)])
        outs.append(o)
        sels.append(s)
        scs.append(sc)
    return np.stack(outs), np.stack(sels), scs
