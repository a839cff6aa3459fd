"""Parity of the dense causal GQA kernel (qsa_dense_attend, the dense baseline
of the pages' module speed-ups) with the CPU oracle's dense rows: QSA rows
with a budget that covers every block before the query's own, which the
oracle pins already tie to causal SDPA.  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import block_sparse_long_qsa_amd as Q
import oracle as O
import synth
from helpers import bits, check_out, f32, oracle_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.lib()
    yield
    torch.cuda.synchronize()


def _setup(w, max_ctx, yarn=1.0, poison=False):
    x = synth.prefill_inputs(w, "cpu")
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    h = Q.Handle(max_ctx=max_ctx, budget_blocks=16, yarn_factor=yarn)
    c = Q.alloc_caches(h, w.batch)
    for t in c.values():              # unwritten slots: NaN (poison) or zeros
        t.view(torch.int16).fill_(0x7FC0 if poison else 0)
    Q.qsa_append(h, w.batch, w.seq_len, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"],
                 c["kbar_cache"], c["kpend"])
    return x, xd, h, c


def _dense_p(yarn=1.0):
    return O.Params(budget=1 << 20, yarn_factor=yarn)      # every block before the own one is selected


@pytest.mark.parametrize("yarn", [1.0, 4.0])
def test_dense_attend_every_row(yarn):
    """Every row of two ragged sequences (700 tokens: 43 full query tiles and a
    tail of 12) against the oracle's dense rows; YaRN changes the rotation and
    the logit scale."""
    B, L = 2, 700
    w = synth.Workload("t", "prefill", B, L, 16, 6, "random", 51)
    x, xd, h, c = _setup(w, 1024, yarn)
    out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    Q.qsa_dense_attend(h, B, L, 0, xd["q"], c["k_cache"], c["v_cache"], out)
    torch.cuda.synchronize()
    o = f32(out)
    p = _dense_p(yarn)
    for b in range(B):
        lay = oracle_layer(x, b, p)
        for i in range(b, L, 1 + b):
            ref, _, _ = lay.row(i, bits(x["q"][b, i]), bits(x["q_idx"][b, i]))
            check_out(o[b, i], ref, "seq %d row %d" % (b, i))


def test_dense_attend_chunk_at_offset_and_unwritten_slots():
    """Queries 516 .. 1099 in one call at q_offset 516 (keys 0 .. 1099 in the
    caches): rows match the oracle; with every unwritten cache slot NaN the
    output is bitwise that of zero-filled caches."""
    B, n_keys, q0 = 1, 1100, 516
    w = synth.Workload("t", "prefill", B, n_keys, 16, 4, "random", 52)
    res = {}
    for poison in (False, True):
        x, xd, h, c = _setup(w, 2048, poison=poison)
        n = n_keys - q0
        out = torch.empty((B, n, 24, 256), dtype=torch.bfloat16, device=DEV)
        Q.qsa_dense_attend(h, B, n, q0, xd["q"][:, q0:].contiguous(), c["k_cache"], c["v_cache"], out)
        torch.cuda.synchronize()
        res[poison] = out
    assert torch.equal(res[False].view(torch.int16), res[True].view(torch.int16))
    o = f32(res[False])
    lay = oracle_layer(x, 0, _dense_p())
    for i in list(range(0, n, 7)) + [n - 1]:
        ref, _, _ = lay.row(q0 + i, bits(x["q"][0, q0 + i]), bits(x["q_idx"][0, q0 + i]))
        check_out(o[0, i], ref, "row %d" % (q0 + i))


def test_dense_attend_equals_sparse_with_every_block():
    """qsa_attend with every block before the own one in block_idx computes the
    same attention; the two kernels agree within the output tolerance."""
    B, L = 1, 600
    w = synth.Workload("t", "prefill", B, L, 16, 4, "random", 53)
    x, xd, h0, c = _setup(w, 1024)
    h = Q.Handle(max_ctx=1024, budget_blocks=150)          # 150 >= floor(599 / 4)
    sel = torch.full((B, L, 150), -1, dtype=torch.int32)
    for i in range(L):
        o = i // 4
        sel[0, i, :o] = torch.arange(o, dtype=torch.int32)
    out_s = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    out_d = torch.empty_like(out_s)
    Q.qsa_attend(h, B, L, 0, xd["q"], c["k_cache"], c["v_cache"], sel.to(DEV), out_s)
    Q.qsa_dense_attend(h, B, L, 0, xd["q"], c["k_cache"], c["v_cache"], out_d)
    torch.cuda.synchronize()
    check_out(f32(out_d[0]), f32(out_s[0]).astype(np.float64), "dense vs sparse")


def test_dense_attend_logits_beyond_the_headroom():
    """A block whose keys give later queries logits far above every logit of
    the first 32 keys (so the kernel's fixed reference maximum would overflow):
    the exact two-pass walk takes over, and the rows still match the oracle."""
    B, L = 1, 260
    w = synth.Workload("t", "prefill", B, L, 16, 0, "random", 54)
    x = synth.prefill_inputs(w, "cpu")
    rng = np.random.default_rng(54)
    u = np.zeros(256)
    u[64:] = rng.standard_normal(192)
    u /= np.linalg.norm(u)
    for g in range(2):
        x["k"][0, 160:164, g] = torch.from_numpy(60.0 * u).to(torch.bfloat16)
    x["q"][0, 170:] = torch.from_numpy(16.0 * u).to(torch.bfloat16)     # raw q.k ~ 960 on those keys
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    h = Q.Handle(max_ctx=512, budget_blocks=16)
    c = Q.alloc_caches(h, B)
    Q.qsa_append(h, B, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    Q.qsa_dense_attend(h, B, L, 0, xd["q"], c["k_cache"], c["v_cache"], out)
    torch.cuda.synchronize()
    o = f32(out[0])
    assert np.isfinite(o).all()
    lay = oracle_layer(x, 0, _dense_p())
    for i in (0, 31, 100, 159, 163, 169, 170, 200, 255, 259):
        ref, _, _ = lay.row(i, bits(x["q"][0, i]), bits(x["q_idx"][0, i]))
        check_out(o[i], ref, "row %d" % i)


def test_dense_attend_262k_sampled_rows():
    """The 262,144-token workload in the launch configuration bench.py's
    ratio leg times: sampled rows against the oracle's dense rows."""
    w = synth.WORKLOADS["prefill_256k"]
    L = w.seq_len
    x = synth.prefill_inputs(w, DEV)
    h = Q.Handle(max_ctx=L, budget_blocks=w.budget)
    c = Q.alloc_caches(h, 1)
    Q.qsa_append(h, 1, L, 0, x["k"], x["v"], x["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    out = torch.empty((1, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    Q.qsa_dense_attend(h, 1, L, 0, x["q"], c["k_cache"], c["v_cache"], out)
    torch.cuda.synchronize()
    lay = O.LayerOracle(bits(x["k"][0]), bits(x["v"][0]), bits(x["k_idx"][0]), O.Params(budget=1 << 20))
    for r in (0, 15, 16, 4095, 65536, 131071, 200003, L - 1):
        ref, _, _ = lay.row(r, bits(x["q"][0, r]), bits(x["q_idx"][0, r]))
        check_out(out[0, r].float().cpu().numpy(), ref, "row %d" % r)
