"""Parity of the training path (qsa_train_forward, qsa_train_backward_indexer)
with the training oracle (oracle/train.py), through the C ABI, on seeded
synthetic sequences.  The selection fed to both sides is the oracle's.

Acceptance (derived from the arithmetic):
  * out: as every attention output (2e-2 + 1e-2|ref| element-wise, 1e-2 normwise);
  * per-head log-sum-exp: |d| <= 3e-3 -- the attention kernel sums its
    probabilities after rounding each to bf16 (relative 2^-9), so ln(l) moves by
    at most 2^-9 ~ 2e-3, plus fp32 logits;
  * ln Z: |d| <= 1e-2 and kl: |d| <= 1e-2 + 1e-2 |kl| -- the teacher's
    probabilities inherit the per-head log-sum-exp error (<= 2e-3 relative per
    head) through a max over tokens and a sum over blocks;
  * log-sum-exp of the indexer scores: |d| <= 1e-3 max(1, |ref|) (fp32 MFMA
    scores, relative 1e-4);
  * kl also moves with the scores: dKL/dI_b = s_b - pi_b, so |d| <= 2 max|dI|
    (about 1e-4 |I| <= 5e-3 here); a per-head error of the log-sum-exp scales
    all of that head's probabilities alike and cancels in pi = A / Z;
  * attention gradients (dq, dk, dv): normwise and max-element errors <= 1e-2
    relative to the oracle's norm / largest element -- P and dS enter the
    MFMAs rounded to bf16 (2^-9 relative each) and D = <dout, out> uses the
    bf16 output;
  * indexer gradients: normwise ||gpu - ref|| / ||ref|| <= 5e-3 and element-wise
    |d| <= 5e-3 max|ref| per tensor -- the coefficients s - pi carry the scores'
    relative error (1e-4 |I| <= 5e-3 in s); a ReLU mask flips only for a logit
    within fp32 rounding of 0.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_qsa_amd as Q
import oracle as O
import synth
from oracle import train as T
from helpers import bits, check_out, f32, oracle_layer

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.lib()
    yield
    torch.cuda.synchronize()


def _oracle_selection(x, b, p, L):
    kbar = O.indexer_keys(bits(x["k_idx"][b]), p)
    qt = O.indexer_queries(bits(x["q_idx"][b]), np.arange(L), p)
    return np.stack([O.select_blocks(O.block_scores(qt[i], kbar[:i // 4]), p.budget) for i in range(L)])


def _run(B, L, budget, seed, needles=6):
    w = synth.Workload("t", "prefill", B, L, budget, needles, "random", seed)
    x = synth.prefill_inputs(w, "cpu")
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    p = O.Params(budget=budget)
    h = Q.Handle(max_ctx=(L + 3) // 4 * 4, budget_blocks=budget)
    c = Q.alloc_caches(h, B)
    Q.qsa_append(h, B, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    sel = np.stack([_oracle_selection(x, b, p, L) for b in range(B)]).astype(np.int32)
    bidx = torch.from_numpy(sel).to(DEV)
    out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    stats = torch.empty((B, L, 32), dtype=torch.float32, device=DEV)
    kl = torch.empty((B, L), dtype=torch.float32, device=DEV)
    ws = Q.workspace(h, Q.QSA_OP_TRAIN_FORWARD, B, L, 0)
    Q.qsa_train_forward(h, B, L, xd["q"], xd["q_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], bidx, out,
                        stats, kl, ws)
    g = np.random.default_rng(seed + 1000)
    dkl_np = (g.random((B, L)) + 0.5).astype(np.float32)
    dkl = torch.from_numpy(dkl_np).to(DEV)
    dq = torch.empty((B, L, 4, 128), dtype=torch.float32, device=DEV)
    dk = torch.empty((B, L, 128), dtype=torch.float32, device=DEV)
    wsb = Q.workspace(h, Q.QSA_OP_TRAIN_BACKWARD, B, L, 0)
    Q.qsa_train_backward_indexer(h, B, L, xd["q"], xd["q_idx"], c["k_cache"], c["kbar_cache"], bidx, stats, dkl,
                                 dq, dk, wsb)
    torch.cuda.synchronize()
    return x, p, sel, dkl_np, f32(out), stats.cpu().numpy(), kl.cpu().numpy(), dq.cpu().numpy(), dk.cpu().numpy()


def _check(B, L, budget, seed):
    x, p, sel, dkl, out, stats, kl, dq, dk = _run(B, L, budget, seed)
    worst = {"kl": 0.0, "lse": 0.0}
    for b in range(B):
        lay = oracle_layer(x, b, p)
        rows = T.train_rows(lay, range(L), bits(x["q"][b]), bits(x["q_idx"][b]), sel[b])
        for i, r in enumerate(rows):
            check_out(out[b, i], r["out"], "seq %d row %d" % (b, i))
            d_lse = np.abs(stats[b, i, :24] - r["lse"]).max()
            assert d_lse <= 3e-3, (b, i, d_lse)
            assert abs(kl[b, i] - r["kl"]) <= 1e-2 + 1e-2 * abs(r["kl"]), (b, i, kl[b, i], r["kl"])
            if r["blocks"].shape[0] >= 1:
                assert abs(stats[b, i, 24] - r["lnZ"]) <= 1e-2, (b, i)
                assert abs(stats[b, i, 25] - r["lse_i"]) <= 1e-3 * max(1.0, abs(r["lse_i"])), (b, i)
            assert np.all(stats[b, i, 26:] == 0)
            worst["kl"] = max(worst["kl"], abs(kl[b, i] - r["kl"]))
            worst["lse"] = max(worst["lse"], d_lse)
        teach = [(r["A"], r["blocks"]) for r in rows]
        gq, gk = T.indexer_grads(bits(x["q_idx"][b]), bits(x["k_idx"][b]), teach, dkl[b].astype(np.float64), p)
        for name, got, ref in (("dq_idx", dq[b], gq), ("dk_idx", dk[b], gk)):
            scale = max(np.abs(ref).max(), 1e-30)
            worst[name] = max(worst.get(name, 0.0), np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
            assert np.abs(got - ref).max() <= 5e-3 * scale, (name, b, np.abs(got - ref).max(), scale)
            assert np.linalg.norm(got - ref) <= 5e-3 * np.linalg.norm(ref), (name, b)
        # tokens of a trailing partial block get no gradient
        assert np.all(dk[b, (L // 4) * 4:] == 0)
    return worst


def test_train_sparse_rows():
    """Stage-2 reading: budget 16 over 300 tokens, so most rows select a subset."""
    print("worst deviations", _check(2, 300, 16, 71))


def test_train_dense_teacher():
    """Stage-1 reading: the budget covers every block, so the teacher is the
    dense max-pooled attention distribution over all complete blocks."""
    print("worst deviations", _check(1, 203, 64, 72))


def test_train_attention_backward():
    """qsa_train_backward_attention against the oracle's autograd gradients of
    sum_p <dout_p, out_p> with respect to the raw q, k, v."""
    B, L, budget = 2, 150, 16
    w = synth.Workload("t", "prefill", B, L, budget, 6, "random", 73)
    x = synth.prefill_inputs(w, "cpu")
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    p = O.Params(budget=budget)
    h = Q.Handle(max_ctx=(L + 3) // 4 * 4, budget_blocks=budget)
    c = Q.alloc_caches(h, B)
    Q.qsa_append(h, B, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    sel = np.stack([_oracle_selection(x, b, p, L) for b in range(B)]).astype(np.int32)
    bidx = torch.from_numpy(sel).to(DEV)
    out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    stats = torch.empty((B, L, 32), dtype=torch.float32, device=DEV)
    kl = torch.empty((B, L), dtype=torch.float32, device=DEV)
    Q.qsa_train_forward(h, B, L, xd["q"], xd["q_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], bidx, out, stats,
                        kl, Q.workspace(h, Q.QSA_OP_TRAIN_FORWARD, B, L, 0))
    g = torch.Generator().manual_seed(74)
    dout = torch.randn((B, L, 24, 256), generator=g).to(torch.bfloat16)
    dq = torch.empty((B, L, 24, 256), dtype=torch.float32, device=DEV)
    dk = torch.empty((B, L, 2, 256), dtype=torch.float32, device=DEV)
    dv = torch.empty((B, L, 2, 256), dtype=torch.float32, device=DEV)
    Q.qsa_train_backward_attention(h, B, L, xd["q"], c["k_cache"], c["v_cache"], bidx, out, dout.to(DEV), stats, dq,
                                   dk, dv)
    torch.cuda.synchronize()
    worst = {}
    for b in range(B):
        rq, rk, rv = T.attention_grads(bits(x["q"][b]), bits(x["k"][b]), bits(x["v"][b]), sel[b],
                                       dout[b].float().numpy().astype(np.float64), p)
        for name, got, ref in (("dq", dq[b].cpu().numpy(), rq), ("dk", dk[b].cpu().numpy(), rk),
                               ("dv", dv[b].cpu().numpy(), rv)):
            nw = np.linalg.norm(got - ref) / np.linalg.norm(ref)
            mx = np.abs(got - ref).max() / np.abs(ref).max()
            worst[name] = max(worst.get(name, 0.0), nw)
            worst[name + "_max"] = max(worst.get(name + "_max", 0.0), mx)
            assert nw <= 1e-2 and mx <= 1e-2, (name, b, nw, mx)
    print("worst deviations", worst)


def test_train_fullsize_32k_sampled_rows():
    """The 32,768-token workload at budget 512: every kernel of the training
    step runs over all rows; sampled rows carry the upstream gradients (dkl and
    dout zero elsewhere), so the oracle checks those rows' outputs, KL and
    query gradients and every token's key and value gradients.  The sampled
    rows use the oracle's selection; the other rows the most recent blocks."""
    w = synth.WORKLOADS["prefill_32k"]
    L, budget = w.seq_len, w.budget
    x = synth.prefill_inputs(w, "cpu")
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    p = O.Params(budget=budget)
    rows = [3, 517, 2051, 8190, 16385, 24576, 32766, 32767]
    sel = np.full((L, budget), -1, dtype=np.int32)
    for i in range(L):
        o = i // 4
        n = min(o, budget)
        sel[i, :n] = np.arange(o - n, o)
    kbar = O.indexer_keys(bits(x["k_idx"][0]), p)
    for i in rows:
        qt = O.indexer_queries(bits(x["q_idx"][0, i:i + 1]), np.array([i]), p)[0]
        sel[i] = O.select_blocks(O.block_scores(qt, kbar[:i // 4]), budget)
    h = Q.Handle(max_ctx=L, budget_blocks=budget)
    c = Q.alloc_caches(h, 1)
    Q.qsa_append(h, 1, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    bidx = torch.from_numpy(sel[None]).to(DEV)
    out = torch.empty((1, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    stats = torch.empty((1, L, 32), dtype=torch.float32, device=DEV)
    kl = torch.empty((1, L), dtype=torch.float32, device=DEV)
    Q.qsa_train_forward(h, 1, L, xd["q"], xd["q_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], bidx, out, stats,
                        kl, Q.workspace(h, Q.QSA_OP_TRAIN_FORWARD, 1, L, 0))
    g = np.random.default_rng(75)
    dkl = np.zeros((1, L), dtype=np.float32)
    dkl[0, rows] = g.random(len(rows)) + 0.5
    dout = torch.zeros((1, L, 24, 256), dtype=torch.bfloat16)
    dout[0, rows] = torch.from_numpy(g.standard_normal((len(rows), 24, 256)).astype(np.float32)).to(torch.bfloat16)
    dq_idx = torch.empty((1, L, 4, 128), dtype=torch.float32, device=DEV)
    dk_idx = torch.empty((1, L, 128), dtype=torch.float32, device=DEV)
    Q.qsa_train_backward_indexer(h, 1, L, xd["q"], xd["q_idx"], c["k_cache"], c["kbar_cache"], bidx, stats,
                                 torch.from_numpy(dkl).to(DEV), dq_idx, dk_idx,
                                 Q.workspace(h, Q.QSA_OP_TRAIN_BACKWARD, 1, L, 0))
    dq = torch.empty((1, L, 24, 256), dtype=torch.float32, device=DEV)
    dk = torch.empty((1, L, 2, 256), dtype=torch.float32, device=DEV)
    dv = torch.empty((1, L, 2, 256), dtype=torch.float32, device=DEV)
    Q.qsa_train_backward_attention(h, 1, L, xd["q"], c["k_cache"], c["v_cache"], bidx, out, dout.to(DEV), stats, dq,
                                   dk, dv)
    torch.cuda.synchronize()
    lay = oracle_layer(x, 0, p)
    res = T.train_rows(lay, rows, bits(x["q"][0]), bits(x["q_idx"][0]), sel)
    o_np, st_np, kl_np = f32(out[0]), stats[0].cpu().numpy(), kl[0].cpu().numpy()
    for i, r in zip(rows, res):
        check_out(o_np[i], r["out"], "row %d" % i)
        assert np.abs(st_np[i, :24] - r["lse"]).max() <= 3e-3, i
        assert abs(kl_np[i] - r["kl"]) <= 1e-2 + 1e-2 * abs(r["kl"]), (i, kl_np[i], r["kl"])
    teach = [(r["A"], r["blocks"]) for r in res]
    gq, gk = T.indexer_grads_rows(bits(x["q_idx"][0, rows]), bits(x["k_idx"][0]), teach, dkl[0, rows].astype(np.float64),
                                  rows, p)
    dqi, dki = dq_idx[0].cpu().numpy(), dk_idx[0].cpu().numpy()
    others = np.setdiff1d(np.arange(L), rows)
    assert np.all(dqi[others] == 0)
    for name, got, ref in (("dq_idx", dqi[rows], gq), ("dk_idx", dki, gk)):
        assert np.linalg.norm(got - ref) <= 5e-3 * np.linalg.norm(ref), name
        assert np.abs(got - ref).max() <= 5e-3 * np.abs(ref).max(), name
    aq, toks, ak, av = T.attention_grads_rows(bits(x["q"][0]), bits(x["k"][0]), bits(x["v"][0]), sel,
                                              dout[0, rows].float().numpy().astype(np.float64), rows, p)
    dq_np, dk_np, dv_np = dq[0].cpu().numpy(), dk[0].cpu().numpy(), dv[0].cpu().numpy()
    assert np.all(dq_np[others] == 0)
    fk, fv = np.zeros_like(dk_np), np.zeros_like(dv_np)
    fk[toks], fv[toks] = ak, av
    for name, got, ref in (("dq", dq_np[rows], aq), ("dk", dk_np, fk), ("dv", dv_np, fv)):
        assert np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref), name
        assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max(), name


def test_train_attention_backward_262k_bench_config():
    """The attention backward on the 262,144-token workload at budget 512 (the
    size bench.py --train times).  Call 1: only sampled rows carry an upstream
    gradient, so the oracle gives those rows' dq and every token's dk, dv.
    Call 2: every row carries a random dout; checked on every token through
    two identities of the softmax backward that hold at any size: the
    probabilities of a (row, head) sum to one, so summed over tokens dv of a
    KV group equals the sum of dout over rows and the group's heads; and the
    dS of a (row, head) sum to zero (sum_t P_t (dP_t - D) with
    D = <dout, out>), so dk summed over tokens vanishes on the dims RoPE
    leaves alone (64..255), up to the bf16 rounding of out (about 2e-3 of the
    norm of dk there)."""
    w = synth.WORKLOADS["prefill_256k"]
    L, budget = w.seq_len, w.budget
    x = synth.prefill_inputs(w, DEV)
    p = O.Params(budget=budget)
    rows = [5, 4099, 65537, 131070, 196611, 262143]
    sel = np.full((L, budget), -1, dtype=np.int32)
    o = np.arange(L) // 4
    n = np.minimum(o, budget)
    col = np.arange(budget)[None, :]
    np.copyto(sel, (o - n)[:, None] + col, where=col < n[:, None])
    kbar = O.indexer_keys(bits(x["k_idx"][0]), p)
    for i in rows:
        qt = O.indexer_queries(bits(x["q_idx"][0, i:i + 1]), np.array([i]), p)[0]
        sel[i] = O.select_blocks(O.block_scores(qt, kbar[:i // 4]), budget)
    del kbar
    h = Q.Handle(max_ctx=L, budget_blocks=budget)
    c = Q.alloc_caches(h, 1)
    Q.qsa_append(h, 1, L, 0, x["k"], x["v"], x["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    bidx = torch.from_numpy(sel[None]).to(DEV)
    out = torch.empty((1, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    stats = torch.empty((1, L, 32), dtype=torch.float32, device=DEV)
    kl = torch.empty((1, L), dtype=torch.float32, device=DEV)
    Q.qsa_train_forward(h, 1, L, x["q"], x["q_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], bidx, out, stats,
                        kl, Q.workspace(h, Q.QSA_OP_TRAIN_FORWARD, 1, L, 0))
    dq = torch.empty((1, L, 24, 256), dtype=torch.float32, device=DEV)
    dk = torch.empty((1, L, 2, 256), dtype=torch.float32, device=DEV)
    dv = torch.empty((1, L, 2, 256), dtype=torch.float32, device=DEV)

    # call 1: sampled rows
    g = np.random.default_rng(76)
    d_rows = torch.from_numpy(g.standard_normal((len(rows), 24, 256)).astype(np.float32)).to(torch.bfloat16)
    dout = torch.zeros((1, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    dout[0, rows] = d_rows.to(DEV)
    Q.qsa_train_backward_attention(h, 1, L, x["q"], c["k_cache"], c["v_cache"], bidx, out, dout, stats, dq, dk, dv)
    torch.cuda.synchronize()
    print("262k backward, sampled rows: launched", flush=True)
    q_rows = bits(x["q"][0, rows])
    k_all, v_all = bits(x["k"][0]), bits(x["v"][0])
    full_q = np.zeros((L, 24, 256), dtype=np.uint16)
    full_q[rows] = q_rows
    aq, toks, ak, av = T.attention_grads_rows(full_q, k_all, v_all, sel, d_rows.float().numpy().astype(np.float64),
                                              rows, p)
    del full_q
    dq_rows = dq[0, rows].cpu().numpy()
    dk_np, dv_np = dk[0].cpu().numpy(), dv[0].cpu().numpy()
    assert int(torch.count_nonzero(dq[0])) == int(torch.count_nonzero(dq[0, rows]))   # other rows: exact zeros
    fk, fv = np.zeros_like(dk_np), np.zeros_like(dv_np)
    fk[toks], fv[toks] = ak, av
    for name, got, ref in (("dq", dq_rows, aq), ("dk", dk_np, fk), ("dv", dv_np, fv)):
        assert np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref), name
        assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max(), name
    del dk_np, dv_np, fk, fv

    # call 2: every row, identities on every token
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    dout = torch.randn((1, L, 24, 256), device=DEV, generator=gen).to(torch.bfloat16)
    Q.qsa_train_backward_attention(h, 1, L, x["q"], c["k_cache"], c["v_cache"], bidx, out, dout, stats, dq, dk, dv)
    torch.cuda.synchronize()
    print("262k backward, every row: launched", flush=True)
    for grp in range(2):
        ref = dout[0, :, 12 * grp:12 * (grp + 1)].double().sum(dim=(0, 1)).cpu().numpy()
        got = dv[0, :, grp].double().sum(dim=0).cpu().numpy()
        assert np.linalg.norm(got - ref) <= 1e-3 * np.linalg.norm(ref), ("dv sum", grp)
        ksum = dk[0, :, grp, 64:].double().sum(dim=0).cpu().numpy()
        knorm = float(dk[0, :, grp, 64:].double().norm())
        assert knorm > 0 and np.linalg.norm(ksum) <= 2e-2 * knorm, ("dk sum", grp, np.linalg.norm(ksum), knorm)
        print("group %d: |sum dv - sum dout| / |sum dout| = %.3g, |sum dk[64:]| / |dk[64:]| = %.3g"
              % (grp, np.linalg.norm(got - ref) / np.linalg.norm(ref), np.linalg.norm(ksum) / knorm), flush=True)
