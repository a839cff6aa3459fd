"""Training-side oracle of the QSA layer -- TEST INFRASTRUCTURE.

Same rules as the package: only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it; it shares no code with the
HIP library.  fp64 throughout; gradients by torch autograd on the CPU.

Source: [PKR] (see the package docstring), section "QSA: 인덱서 자체의 비용을
줄이는 희소 어텐션": the indexer is trained against the backbone's attention
distribution matched per micro-block with MAX pooling (stage 1, dense
distillation), then jointly with the backbone under a fused kernel that
computes the sparse attention output and the indexer's KL-divergence loss in
one pass without materialising intermediates (stage 2).

Readings (the pages give no formula for the loss):
  * teacher of query p over its selected blocks S(p) (the valid entries of its
    selection): a_t = mean over the 24 query heads of the attention probability
    of token t (softmax over the whole token set T(p)); A_b = max of a_t over
    the block's 4 tokens; pi_b = A_b / sum_{b' in S(p)} A_b'.  The own block
    is not scored by the indexer and takes no part.  With every block selected
    (budget >= floor(p/4)) T(p) is the whole causal context and this is the
    dense, max-pooled teacher of stage 1.
  * student: s_b = softmax over S(p) of I_pb = sum_h ReLU(<q~_h(p), k̄_b>).
  * loss of query p: KL(pi || s) = sum_b pi_b (ln pi_b - ln s_b); 0 when
    |S(p)| <= 1.
  * gradient: the teacher is a constant (stop-gradient, the backbone is not
    trained by this loss); dKL/dI_pb = s_b - pi_b; ReLU' = [logit > 0]; the
    rotations pass gradients by their transpose, the mean pooling gives 1/4
    to each of the block's raw keys, and the bf16 roundings of the rotated
    operands pass gradients unchanged.

The attention's own gradient (the backbone's, attention_grads) is torch
autograd through the same token sets: softmax over T(p), dout contracted
with the output, rotations passing their transposes.

Parity status: pinned by tests/test_oracle_train_pins.py (closed forms of the
KL, finite differences of the losses and of the whole gradient chains, max
pooling of a planted token, the dense special case against the plain
attention and against torch's SDPA backward).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (LayerOracle, Params, bf16_bits_to_f32, core_rotate, indexer_keys, indexer_queries, own_block,
               rope_table, token_set)
from . import softmax_scale as softmax_scale_of


def teacher_row(lay: LayerOracle, pos: int, q_bits: np.ndarray, sel: np.ndarray):
    """Teacher of query `pos`: (A [n] fp64 over the valid selected blocks in
    selection order, their block ids [n], lse [24] fp64 natural-log
    log-sum-exp of the scaled logits over T(pos))."""
    p = lay.p
    o = own_block(pos, p)
    blocks = np.asarray(sel)[(np.asarray(sel) >= 0) & (np.asarray(sel) < o)].astype(np.int64)
    toks = token_set(blocks, pos, p)
    kt = core_rotate(lay.k_bits[toks], toks, p).astype(np.float64)      # [T][2][256]
    qt = core_rotate(q_bits[None], np.array([pos]), p)[0].astype(np.float64)
    grp = p.n_q_heads // p.n_kv_heads
    probs = np.empty((p.n_q_heads, toks.shape[0]))
    lse = np.empty(p.n_q_heads)
    for g in range(p.n_kv_heads):
        z = lay.sigma * (qt[g * grp:(g + 1) * grp] @ kt[:, g].T)          # [12][T]
        m = z.max(axis=1, keepdims=True)
        l = np.log(np.exp(z - m).sum(axis=1, keepdims=True)) + m
        probs[g * grp:(g + 1) * grp] = np.exp(z - l)
        lse[g * grp:(g + 1) * grp] = l[:, 0]
    a = probs.mean(axis=0)                                                # [T]
    A = a[:4 * blocks.shape[0]].reshape(-1, 4).max(axis=1) if blocks.size else np.zeros(0)
    return A, blocks, lse


def kl_of(A: np.ndarray, I: np.ndarray):
    """(KL(pi || softmax(I)), ln sum A, logsumexp I) with pi = A / sum A."""
    if A.shape[0] <= 1:
        return 0.0, (float(np.log(A.sum())) if A.shape[0] else 0.0), (float(I[0]) if I.shape[0] else 0.0)
    Z = A.sum()
    pi = A / Z
    m = I.max()
    lse_i = m + np.log(np.exp(I - m).sum())
    logpi = np.where(pi > 0, np.log(np.where(pi > 0, pi, 1.0)), 0.0)
    kl = float(np.sum(pi * (logpi - (I - lse_i))))
    return kl, float(np.log(Z)), float(lse_i)


def train_rows(lay: LayerOracle, rows, q_bits, q_idx_bits, sel, q_offset: int = 0):
    """Per row r (query position q_offset + r): dict with out [24][256], lse
    [24], kl, lnZ, lse_i, A (teacher weights) and I (student scores) over the
    selected blocks."""
    p = lay.p
    res = []
    for r in rows:
        pos = q_offset + int(r)
        out = lay.row_reused(pos, q_bits[int(r)], sel[int(r)], pos)       # attention over T(pos) of `sel`
        A, blocks, lse = teacher_row(lay, pos, q_bits[int(r)], sel[int(r)])
        qt = indexer_queries(q_idx_bits[int(r)][None], np.array([pos]), p)[0].astype(np.float64)
        I = np.maximum(qt @ lay.kbar[blocks].astype(np.float64).T, 0.0).sum(axis=0) if blocks.size else np.zeros(0)
        kl, lnz, lse_i = kl_of(A, I)
        res.append(dict(out=out, lse=lse, kl=kl, lnZ=lnz, lse_i=lse_i, A=A, I=I, blocks=blocks))
    return res


def _rot_t(x: torch.Tensor, c: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    n = c.shape[-1]
    a, b = x[..., :n], x[..., n:2 * n]
    return torch.cat([a * c - b * s, b * c + a * s, x[..., 2 * n:]], dim=-1)


def indexer_loss(q_idx: torch.Tensor, k_idx: torch.Tensor, teach, dkl: np.ndarray, p: Params,
                 q_offset: int = 0, rounded=None):
    """sum_r dkl[r] * KL_r as a differentiable function of the raw indexer
    queries q_idx [Lq][4][128] (positions q_offset + r) and raw indexer keys
    k_idx [n_tok][128] (positions 0..n_tok-1), fp64 torch tensors.  teach[r] =
    (A, blocks) of row r.  `rounded` = (q~ values [Lq][4][128], k̄ values
    [nb][128]) replaces the forward values of the rotated operands (their bf16
    roundings) while the gradient passes unchanged; None keeps exact fp64."""
    Lq = q_idx.shape[0]
    n_tok = k_idx.shape[0]
    c, s = rope_table(np.arange(q_offset, q_offset + Lq), p)
    qt = _rot_t(q_idx, torch.from_numpy(c.astype(np.float64))[:, None, :],
                torch.from_numpy(s.astype(np.float64))[:, None, :])
    nb = n_tok // p.block
    pooled = k_idx[:nb * p.block].reshape(nb, p.block, -1).mean(dim=1)
    cb, sb = rope_table(np.arange(nb) * p.block, p)
    kb = _rot_t(pooled, torch.from_numpy(cb.astype(np.float64)), torch.from_numpy(sb.astype(np.float64)))
    if rounded is not None:
        qt = qt + (torch.from_numpy(rounded[0]) - qt).detach()
        kb = kb + (torch.from_numpy(rounded[1]) - kb).detach()
    loss = torch.zeros((), dtype=torch.float64)
    for r in range(Lq):
        A, blocks = teach[r]
        if blocks.shape[0] <= 1 or dkl[r] == 0.0:
            continue
        I = torch.relu(qt[r] @ kb[torch.from_numpy(blocks)].T).sum(dim=0)
        pi = torch.from_numpy(A / A.sum())
        logpi = torch.where(pi > 0, torch.log(torch.where(pi > 0, pi, torch.ones_like(pi))), torch.zeros_like(pi))
        loss = loss + float(dkl[r]) * torch.sum(pi * (logpi - torch.log_softmax(I, dim=0)))
    return loss


def indexer_grads(q_idx_bits: np.ndarray, k_idx_bits: np.ndarray, teach, dkl: np.ndarray, p: Params,
                  q_offset: int = 0):
    """Gradients of sum_r dkl[r] * KL_r with respect to the raw indexer queries
    (fp64 [Lq][4][128]) and raw indexer keys (fp64 [n_tok][128]), at the bf16
    values the forward uses."""
    qi = torch.tensor(bf16_bits_to_f32(q_idx_bits), dtype=torch.float64, requires_grad=True)
    ki = torch.tensor(bf16_bits_to_f32(k_idx_bits), dtype=torch.float64, requires_grad=True)
    Lq = q_idx_bits.shape[0]
    rq = indexer_queries(q_idx_bits, np.arange(q_offset, q_offset + Lq), p).astype(np.float64)
    rk = indexer_keys(k_idx_bits, p).astype(np.float64)
    loss = indexer_loss(qi, ki, teach, dkl, p, q_offset, rounded=(rq, rk))
    if loss.requires_grad:
        loss.backward()
    gq = qi.grad.numpy() if qi.grad is not None else np.zeros(qi.shape)
    gk = ki.grad.numpy() if ki.grad is not None else np.zeros(ki.shape)
    return gq, gk


def attention_loss(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: np.ndarray, dout: torch.Tensor, p: Params,
                   rounded=None):
    """sum_p <dout_p, out_p> of the sparse attention (the token sets of `sel`,
    queries at positions 0..L-1) as a differentiable function of the raw q
    [L][24][256], k [L][2][256] and v [L][2][256] (fp64 torch tensors).
    `rounded` = (q~ values, k~ values) replaces the forward values of the
    rotated operands (their bf16 roundings) with the gradient passing
    unchanged; None keeps exact fp64."""
    L = q.shape[0]
    c, s = rope_table(np.arange(L), p)
    ct = torch.from_numpy(c.astype(np.float64))[:, None, :]
    st = torch.from_numpy(s.astype(np.float64))[:, None, :]
    qt = _rot_t(q, ct, st)
    kt = _rot_t(k, ct, st)
    if rounded is not None:
        qt = qt + (torch.from_numpy(rounded[0]) - qt).detach()
        kt = kt + (torch.from_numpy(rounded[1]) - kt).detach()
    sigma = softmax_scale_of(p)
    grp = p.n_q_heads // p.n_kv_heads
    loss = torch.zeros((), dtype=torch.float64)
    for pos in range(L):
        toks = torch.from_numpy(token_set(sel[pos], pos, p))
        for g in range(p.n_kv_heads):
            z = sigma * (qt[pos, g * grp:(g + 1) * grp] @ kt[toks, g].T)
            out = torch.softmax(z, dim=1) @ v[toks, g]
            loss = loss + torch.sum(dout[pos, g * grp:(g + 1) * grp] * out)
    return loss


def attention_grads(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, sel: np.ndarray, dout: np.ndarray,
                    p: Params):
    """Gradients of sum_p <dout_p, out_p> with respect to the raw q, k, v (fp64),
    at the bf16 values the forward uses.  Returns (dq, dk, dv)."""
    q = torch.tensor(bf16_bits_to_f32(q_bits), dtype=torch.float64, requires_grad=True)
    k = torch.tensor(bf16_bits_to_f32(k_bits), dtype=torch.float64, requires_grad=True)
    v = torch.tensor(bf16_bits_to_f32(v_bits), dtype=torch.float64, requires_grad=True)
    L = q_bits.shape[0]
    pos = np.arange(L)
    rq = core_rotate(q_bits, pos, p).astype(np.float64)
    rk = core_rotate(k_bits, pos, p).astype(np.float64)
    loss = attention_loss(q, k, v, sel, torch.tensor(dout, dtype=torch.float64), p, rounded=(rq, rk))
    loss.backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def attention_grads_rows(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, sel: np.ndarray,
                         dout: np.ndarray, rows, p: Params):
    """attention_grads when only the query rows `rows` carry an upstream
    gradient (dout [n][24][256] for those rows), for long sequences: the graph
    holds those rows and the tokens they attend.  Returns (dq [n][24][256],
    tokens [m] (positions), dk [m][2][256], dv [m][2][256]); every other
    token's gradient is zero."""
    rows = np.asarray(list(rows), dtype=np.int64)
    tsets = [token_set(sel[r], int(r), p) for r in rows]
    toks = np.unique(np.concatenate(tsets))
    where = {int(t): i for i, t in enumerate(toks)}
    q = torch.tensor(bf16_bits_to_f32(q_bits[rows]), dtype=torch.float64, requires_grad=True)
    k = torch.tensor(bf16_bits_to_f32(k_bits[toks]), dtype=torch.float64, requires_grad=True)
    v = torch.tensor(bf16_bits_to_f32(v_bits[toks]), dtype=torch.float64, requires_grad=True)
    cq, sq = rope_table(rows, p)
    ck, sk = rope_table(toks, p)
    qt = _rot_t(q, torch.from_numpy(cq.astype(np.float64))[:, None, :], torch.from_numpy(sq.astype(np.float64))[:, None, :])
    kt = _rot_t(k, torch.from_numpy(ck.astype(np.float64))[:, None, :], torch.from_numpy(sk.astype(np.float64))[:, None, :])
    qt = qt + (torch.from_numpy(core_rotate(q_bits[rows], rows, p).astype(np.float64)) - qt).detach()
    kt = kt + (torch.from_numpy(core_rotate(k_bits[toks], toks, p).astype(np.float64)) - kt).detach()
    sigma = softmax_scale_of(p)
    grp = p.n_q_heads // p.n_kv_heads
    d = torch.tensor(dout, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for i, ts in enumerate(tsets):
        ix = torch.tensor([where[int(t)] for t in ts])
        for g in range(p.n_kv_heads):
            z = sigma * (qt[i, g * grp:(g + 1) * grp] @ kt[ix, g].T)
            loss = loss + torch.sum(d[i, g * grp:(g + 1) * grp] * (torch.softmax(z, dim=1) @ v[ix, g]))
    loss.backward()
    return q.grad.numpy(), toks, k.grad.numpy(), v.grad.numpy()


def indexer_grads_rows(q_idx_bits: np.ndarray, k_idx_bits: np.ndarray, teach, dkl: np.ndarray, rows, p: Params):
    """indexer_grads when only the query rows `rows` carry an upstream gradient
    (q_idx_bits [n][4][128] and teach / dkl for those rows; k_idx_bits [n_tok][128]
    for the whole sequence).  Returns (dq_idx [n][4][128], dk_idx [n_tok][128])."""
    rows = np.asarray(list(rows), dtype=np.int64)
    used = np.unique(np.concatenate([bl for _, bl in teach] + [np.zeros(0, np.int64)])).astype(np.int64)
    where = {int(b): i for i, b in enumerate(used)}
    qi = torch.tensor(bf16_bits_to_f32(q_idx_bits), dtype=torch.float64, requires_grad=True)
    tok = (used[:, None] * p.block + np.arange(p.block)[None, :]).reshape(-1)
    ki = torch.tensor(bf16_bits_to_f32(k_idx_bits[tok]), dtype=torch.float64, requires_grad=True)
    cq, sq = rope_table(rows, p)
    qt = _rot_t(qi, torch.from_numpy(cq.astype(np.float64))[:, None, :], torch.from_numpy(sq.astype(np.float64))[:, None, :])
    qt = qt + (torch.from_numpy(indexer_queries(q_idx_bits, rows, p).astype(np.float64)) - qt).detach()
    pooled = ki.reshape(used.shape[0], p.block, -1).mean(dim=1)
    cb, sb = rope_table(used * p.block, p)
    kb = _rot_t(pooled, torch.from_numpy(cb.astype(np.float64)), torch.from_numpy(sb.astype(np.float64)))
    kb = kb + (torch.from_numpy(indexer_keys(k_idx_bits, p)[used].astype(np.float64)) - kb).detach()
    loss = torch.zeros((), dtype=torch.float64)
    for i, (A, blocks) in enumerate(teach):
        if blocks.shape[0] <= 1 or dkl[i] == 0.0:
            continue
        I = torch.relu(qt[i] @ kb[torch.tensor([where[int(b)] for b in blocks])].T).sum(dim=0)
        pi = torch.from_numpy(A / A.sum())
        logpi = torch.where(pi > 0, torch.log(torch.where(pi > 0, pi, torch.ones_like(pi))), torch.zeros_like(pi))
        loss = loss + float(dkl[i]) * torch.sum(pi * (logpi - torch.log_softmax(I, dim=0)))
    gk = np.zeros((k_idx_bits.shape[0], k_idx_bits.shape[1]))
    gq = np.zeros(qi.shape)
    if loss.requires_grad:
        loss.backward()
        gq = qi.grad.numpy()
        gk[tok] = ki.grad.numpy()
    return gq, gk
