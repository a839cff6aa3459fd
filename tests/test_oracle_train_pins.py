"""Pins of the training-side oracle (oracle/train.py) against facts it does not
compute itself: closed forms of the KL divergence, finite differences of the
loss and of the whole indexer gradient chain, max pooling of a planted token,
and the dense special case.  CPU only."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import train as T


def _logsumexp(x):
    m = x.max()
    return m + np.log(np.exp(x - m).sum())


def test_kl_closed_forms():
    rng = np.random.default_rng(5)
    n = 7
    I = rng.standard_normal(n) * 3
    ls = I - _logsumexp(I)
    # uniform teacher: KL = -ln n - mean(ln s)
    kl, lnz, lse_i = T.kl_of(np.full(n, 0.2), I)
    assert abs(kl - (-np.log(n) - ls.mean())) < 1e-12
    assert abs(lnz - np.log(1.4)) < 1e-12 and abs(lse_i - _logsumexp(I)) < 1e-12
    # student equal to the teacher: KL = 0
    A = rng.random(n) + 0.1
    kl, _, _ = T.kl_of(A, np.log(A) + 3.7)
    assert abs(kl) < 1e-12
    # non-negative, and zero for fewer than two blocks
    for _ in range(20):
        assert T.kl_of(rng.random(n) + 1e-3, rng.standard_normal(n) * 5)[0] >= -1e-12
    assert T.kl_of(np.array([0.3]), np.array([2.0]))[0] == 0.0
    assert T.kl_of(np.zeros(0), np.zeros(0))[0] == 0.0


def test_kl_gradient_is_student_minus_teacher():
    """dKL/dI_b = s_b - pi_b, by central differences of kl_of."""
    rng = np.random.default_rng(6)
    A = rng.random(6) + 0.05
    I = rng.standard_normal(6) * 2
    s = np.exp(I - _logsumexp(I))
    pi = A / A.sum()
    h = 1e-6
    for b in range(6):
        e = np.zeros(6)
        e[b] = h
        fd = (T.kl_of(A, I + e)[0] - T.kl_of(A, I - e)[0]) / (2 * h)
        assert abs(fd - (s[b] - pi[b])) < 1e-7


def test_indexer_gradient_chain_finite_differences():
    """Gradients of sum_r dkl_r KL_r with respect to the raw indexer queries and
    keys (through the rotation, the ReLU and the mean pooling) equal central
    differences of the loss, on rotary and non-rotary dims, queries and keys."""
    rng = np.random.default_rng(7)
    p = O.Params(budget=3)
    L = 24
    qi = torch.tensor(rng.standard_normal((L, 4, 128)), dtype=torch.float64, requires_grad=True)
    ki = torch.tensor(rng.standard_normal((L, 128)), dtype=torch.float64, requires_grad=True)
    teach = []
    for r in range(L):
        o = r // 4
        blocks = np.sort(rng.choice(o, size=min(3, o), replace=False)) if o else np.zeros(0, np.int64)
        teach.append((rng.random(blocks.shape[0]) + 0.05, blocks.astype(np.int64)))
    dkl = rng.random(L) + 0.5
    loss = T.indexer_loss(qi, ki, teach, dkl, p)
    loss.backward()
    h = 1e-6
    for (r, hd, d) in [(23, 0, 3), (23, 2, 40), (17, 1, 100), (9, 3, 31), (22, 0, 63)]:
        with torch.no_grad():
            e = torch.zeros_like(qi)
            e[r, hd, d] = h
            fd = (T.indexer_loss(qi + e, ki, teach, dkl, p) - T.indexer_loss(qi - e, ki, teach, dkl, p)) / (2 * h)
        assert abs(float(fd) - float(qi.grad[r, hd, d])) < 1e-6 * max(1.0, abs(float(fd)))
    for (t, d) in [(0, 5), (3, 37), (9, 64), (13, 127), (18, 10)]:
        with torch.no_grad():
            e = torch.zeros_like(ki)
            e[t, d] = h
            fd = (T.indexer_loss(qi, ki + e, teach, dkl, p) - T.indexer_loss(qi, ki - e, teach, dkl, p)) / (2 * h)
        assert abs(float(fd) - float(ki.grad[t, d])) < 1e-6 * max(1.0, abs(float(fd)))
    # keys of the last, incomplete block and of never-selected blocks get nothing
    assert float(ki.grad[20:].abs().sum()) == 0.0 or L % 4 == 0
    used = set(int(b) for _, bl in teach for b in bl)
    for b in range(L // 4):
        if b not in used:
            assert float(ki.grad[4 * b:4 * b + 4].abs().sum()) == 0.0


def _layer(rng, n, p):
    bf = lambda a: O.f32_to_bf16_bits(a.astype(np.float32))
    k = bf(rng.standard_normal((n, 2, 256)))
    v = bf(rng.standard_normal((n, 2, 256)))
    ki = bf(rng.standard_normal((n, 128)))
    return O.LayerOracle(k, v, ki, p), k, v, ki


def test_teacher_max_pools_a_planted_token():
    """One token whose key aligns with every query head takes almost all the
    attention: its block dominates the max-pooled teacher."""
    rng = np.random.default_rng(8)
    p = O.Params(budget=6)
    n = 80
    pos = 79
    lay, k, v, ki = _layer(rng, n, p)
    q = rng.standard_normal((24, 256)).astype(np.float32)
    q[:, 64:] = np.abs(q[:, 64:])
    kk = O.bf16_bits_to_f32(k)
    kk[41, :, 64:] = 6.0                      # token 41, block 10, non-rotary dims
    lay = O.LayerOracle(O.f32_to_bf16_bits(kk), v, ki, p)
    sel = np.array([2, 5, 10, 11, 15, 17], dtype=np.int32)
    A, blocks, lse = T.teacher_row(lay, pos, O.f32_to_bf16_bits(q), sel)
    assert list(blocks) == list(sel)
    pi = A / A.sum()
    assert pi[2] > 0.95
    # a block's weight is the max over its tokens (the planted token's mass, ~1),
    # not their mean (~1/4)
    assert A[2] > 0.99


def test_teacher_dense_case_is_the_attention_distribution():
    """With every block selected, the head-mean probabilities over T(p) sum to 1,
    the per-head log-sum-exp matches torch's logsumexp of the scaled logits of
    the whole causal context, and the output equals the plain row."""
    rng = np.random.default_rng(9)
    p = O.Params(budget=64)
    n = 90
    pos = 86
    lay, k, v, ki = _layer(rng, n, p)
    q = O.f32_to_bf16_bits(rng.standard_normal((24, 256)).astype(np.float32))
    qi = O.f32_to_bf16_bits(rng.standard_normal((4, 128)).astype(np.float32))
    sel = O.select_blocks(np.zeros(pos // 4), p.budget)
    A, blocks, lse = T.teacher_row(lay, pos, q, sel)
    assert blocks.shape[0] == pos // 4
    toks = np.arange(pos + 1)
    kt = torch.tensor(O.core_rotate(k[toks], toks, p), dtype=torch.float64)
    qt = torch.tensor(O.core_rotate(q[None], np.array([pos]), p)[0], dtype=torch.float64)
    z = lay.sigma * torch.einsum("hd,tgd->hgt", qt, kt)
    ref = torch.stack([torch.logsumexp(z[h, h // 12], dim=0) for h in range(24)]).numpy()
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)
    rows = T.train_rows(lay, [pos], q[None].repeat(pos + 1, 0), qi[None].repeat(pos + 1, 0),
                        np.stack([sel] * (pos + 1)))
    out_plain, _, _ = lay.row(pos, q, qi)
    np.testing.assert_allclose(rows[0]["out"], out_plain, rtol=0, atol=1e-12)
    assert rows[0]["kl"] >= 0.0


def test_indexer_loss_forward_matches_the_pinned_scores():
    """The differentiable loss's forward (fp64 rotation of raw keys mean-pooled
    per block and rotated at the block start) equals sum_r dkl_r KL(pi_r ||
    softmax(I_r)) with I from the pinned fp32 pooling, rotation and scoring."""
    rng = np.random.default_rng(10)
    p = O.Params(budget=4)
    L = 40
    q = rng.standard_normal((L, 4, 128)).astype(np.float32)
    k = rng.standard_normal((L, 128)).astype(np.float32)
    teach = []
    for r in range(L):
        o = r // 4
        blocks = np.sort(rng.choice(o, size=min(4, o), replace=False)).astype(np.int64) if o else np.zeros(0, np.int64)
        teach.append((rng.random(blocks.shape[0]) + 0.05, blocks))
    dkl = rng.random(L) + 0.5
    got = float(T.indexer_loss(torch.tensor(q, dtype=torch.float64), torch.tensor(k, dtype=torch.float64),
                               teach, dkl, p))
    pooled = O.pool_block_keys(k, 4)
    c, s = O.rope_table(np.arange(pooled.shape[0]) * 4, p)
    kbar = O.rotate(pooled, c, s)
    ref = 0.0
    for r in range(L):
        A, blocks = teach[r]
        cq, sq = O.rope_table(np.array([r]), p)
        qt = O.rotate(q[r], cq, sq)
        I = O.block_scores(qt, kbar)[blocks] if blocks.size else np.zeros(0)
        ref += dkl[r] * T.kl_of(A, I)[0]
    assert abs(got - ref) < 1e-4 * max(1.0, abs(ref))


def test_attention_gradients_finite_differences():
    """Gradients of sum_p <dout_p, out_p> with respect to the raw q, k, v (through
    the rotations and the token sets) equal central differences of the loss."""
    rng = np.random.default_rng(12)
    p = O.Params(budget=2)
    L = 18
    q = torch.tensor(rng.standard_normal((L, 24, 256)) * 0.5, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(rng.standard_normal((L, 2, 256)) * 0.5, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(rng.standard_normal((L, 2, 256)), dtype=torch.float64, requires_grad=True)
    sel = np.full((L, 2), -1, dtype=np.int32)
    for r in range(L):
        o = r // 4
        c = np.sort(rng.choice(o, size=min(2, o), replace=False)) if o else np.zeros(0, np.int64)
        sel[r, :c.shape[0]] = c
    dout = torch.tensor(rng.standard_normal((L, 24, 256)), dtype=torch.float64)
    loss = T.attention_loss(q, k, v, sel, dout, p)
    loss.backward()
    h = 1e-6
    for (t, idx) in [(q, (17, 3, 5)), (q, (9, 20, 40)), (q, (12, 13, 200)), (k, (2, 0, 10)), (k, (14, 1, 50)),
                     (k, (5, 1, 130)), (v, (0, 1, 7)), (v, (16, 0, 255))]:
        with torch.no_grad():
            e = torch.zeros_like(t)
            e[idx] = h
            args = [q, k, v]
            ip = [a + e if a is t else a for a in args]
            im = [a - e if a is t else a for a in args]
            fd = (T.attention_loss(*ip, sel, dout, p) - T.attention_loss(*im, sel, dout, p)) / (2 * h)
        assert abs(float(fd) - float(t.grad[idx])) < 1e-6 * max(1.0, abs(float(fd))), idx


def test_attention_gradients_dense_case_match_sdpa_backward():
    """With every block selected, the gradients equal torch's SDPA backward
    (causal, GQA 12:1, fp64) on the rotated operands, with dq and dk rotated
    back by the transposed rotation (rotation by minus the angle)."""
    rng = np.random.default_rng(13)
    p = O.Params(budget=64)
    L = 37
    bf = lambda a: O.f32_to_bf16_bits(a.astype(np.float32))
    qb, kb, vb = bf(rng.standard_normal((L, 24, 256))), bf(rng.standard_normal((L, 2, 256))), bf(
        rng.standard_normal((L, 2, 256)))
    sel = np.stack([O.select_blocks(np.zeros(r // 4), p.budget) for r in range(L)])
    dout = rng.standard_normal((L, 24, 256))
    dq, dk, dv = T.attention_grads(qb, kb, vb, sel, dout, p)
    pos = np.arange(L)
    qt = torch.tensor(O.core_rotate(qb, pos, p), dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(O.core_rotate(kb, pos, p), dtype=torch.float64, requires_grad=True)
    v = torch.tensor(O.bf16_bits_to_f32(vb), dtype=torch.float64, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2)[None], kt.permute(1, 0, 2)[None], v.permute(1, 0, 2)[None], is_causal=True,
        scale=O.softmax_scale(p), enable_gqa=True)
    (o[0].permute(1, 0, 2) * torch.tensor(dout)).sum().backward()
    c, s = O.rope_table(pos, p)
    back = lambda g: O.rotate(g.astype(np.float32), c[:, None, :], -s[:, None, :])   # R^T
    np.testing.assert_allclose(dv, v.grad.numpy(), rtol=0, atol=1e-9)
    np.testing.assert_allclose(dq, back(qt.grad.numpy()), rtol=0, atol=2e-5 * np.abs(dq).max())
    np.testing.assert_allclose(dk, back(kt.grad.numpy()), rtol=0, atol=2e-5 * np.abs(dk).max())


def test_row_subset_gradients_equal_the_full_ones():
    """The row-subset forms (for long sequences) give the full forms' gradients
    when only those rows carry an upstream gradient."""
    rng = np.random.default_rng(14)
    p = O.Params(budget=3)
    L = 30
    bf = lambda a: O.f32_to_bf16_bits(a.astype(np.float32))
    qb, kb, vb = bf(rng.standard_normal((L, 24, 256))), bf(rng.standard_normal((L, 2, 256))), bf(
        rng.standard_normal((L, 2, 256)))
    qib, kib = bf(rng.standard_normal((L, 4, 128))), bf(rng.standard_normal((L, 128)))
    sel = np.full((L, 3), -1, dtype=np.int32)
    for r in range(L):
        o = r // 4
        c = np.sort(rng.choice(o, size=min(3, o), replace=False)) if o else np.zeros(0, np.int64)
        sel[r, :c.shape[0]] = c
    rows = [5, 17, 29]
    dout = np.zeros((L, 24, 256))
    dout[rows] = rng.standard_normal((3, 24, 256))
    dq, dk, dv = T.attention_grads(qb, kb, vb, sel, dout, p)
    sq, toks, sk, sv = T.attention_grads_rows(qb, kb, vb, sel, dout[rows], rows, p)
    np.testing.assert_allclose(sq, dq[rows], rtol=0, atol=1e-12)
    fk, fv = np.zeros_like(dk), np.zeros_like(dv)
    fk[toks], fv[toks] = sk, sv
    np.testing.assert_allclose(fk, dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fv, dv, rtol=0, atol=1e-12)
    teach = []
    for r in range(L):
        o = r // 4
        bl = sel[r][(sel[r] >= 0) & (sel[r] < o)].astype(np.int64)
        teach.append((rng.random(bl.shape[0]) + 0.05, bl))
    dkl = np.zeros(L)
    dkl[rows] = [0.7, 1.3, 0.4]
    gq, gk = T.indexer_grads(qib, kib, teach, dkl, p)
    hq, hk = T.indexer_grads_rows(qib[rows], kib, [teach[r] for r in rows], dkl[rows], rows, p)
    np.testing.assert_allclose(hq, gq[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(hk, gk, rtol=0, atol=1e-12)
