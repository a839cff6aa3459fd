"""Parity at the workloads' full sizes, in the launch configuration bench.py
times: sampled rows the oracle computes one by one (every 1,024th row and the
last 24 at 262,144 tokens; every 16,384th row and the chunk boundaries at
1,048,576; 8 of the 64 decode sequences at 131,072 and 3 of 8 at 1,048,576;
4 rows of a 32-row ragged decode whose longest row holds 80,000 tokens),
the selection invariants on every row and every sequence, checked on the
device (count min(budget, floor(p/4)), strictly ascending, every id in
[0, floor(p/4)), -1 padding after the ids), and every needle probe's needle.

Large inputs are drawn on the GPU by the seeded generator (a GPU and a CPU
generator give different streams); the oracle reads host copies of those
inputs -- never anything the library wrote.
"""
import gc

import numpy as np
import pytest
import torch

import block_sparse_long_qsa_amd as Q
import oracle as O
import synth
from helpers import bits, check_out, check_selection

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _free():
    assert torch.cuda.is_available()
    Q.lib()
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _say(*a):
    print(*a, flush=True)


def _prefill_run(w, x, chunk=None):
    """Prefill of one sequence: chunks via qsa_forward, or the bench's stage calls."""
    L = w.seq_len
    h = Q.Handle(max_ctx=L, budget_blocks=w.budget, yarn_factor=w.yarn_factor)
    c = Q.alloc_caches(h, 1)
    bidx = torch.empty((1, L, w.budget), dtype=torch.int32, device=DEV)
    out = torch.empty((1, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    if chunk is None:
        ws = Q.workspace(h, Q.QSA_OP_INDEX_SELECT, 1, L, 0)
        Q.qsa_append(h, 1, L, 0, x["k"], x["v"], x["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
        Q.qsa_index_select(h, 1, L, 0, x["q_idx"], c["kbar_cache"], bidx, ws)
        Q.qsa_attend(h, 1, L, 0, x["q"], c["k_cache"], c["v_cache"], bidx, out)
    else:
        for s0 in range(0, L, chunk):
            n = min(chunk, L - s0)
            ws = Q.workspace(h, Q.QSA_OP_FORWARD, 1, n, s0)
            sl = lambda t: t[:, s0:s0 + n]
            Q.qsa_forward(h, 1, n, s0, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["q_idx"]), sl(x["k_idx"]),
                          c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], sl(out), sl(bidx), ws)
            del ws
            torch.cuda.synchronize()
            _say("  chunk at %d done" % s0)
    torch.cuda.synchronize()
    return out, bidx


def _check_needles_prefill(plan, bidx):
    rows = np.concatenate(plan.probes)
    owners = np.concatenate([[b] * len(p) for b, p in zip(plan.blocks, plan.probes)])
    got = bidx[0, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    miss = [(int(r), int(b)) for r, b, g in zip(rows, owners, got) if b not in g]
    assert not miss, "needle blocks not selected by their probes: %s" % miss[:5]
    return len(rows)


def _check_rows(x, out, bidx, p, rows):
    lay = O.LayerOracle(bits(x["k"][0]), bits(x["v"][0]), bits(x["k_idx"][0]), p)
    o = out[0, torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    bi = bidx[0, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    worst = 0.0
    for j, r in enumerate(rows):
        ref, sel, sc = lay.row(int(r), bits(x["q"][0, r]), bits(x["q_idx"][0, r]))
        check_selection(bi[j], sel, sc, p.budget, int(r) // 4, "row %d" % r)
        err, _ = check_out(o[j], ref, "row %d" % r)
        worst = max(worst, err)
    return worst


def _check_invariants(bidx, budget, q_offset=0, pos=None):
    """Selection invariants of every row, on the device, in row slices: row i
    (query position q_offset + i, or pos[i]) holds min(budget, floor(p/4))
    strictly ascending ids in [0, floor(p/4)) followed by -1."""
    sel_all = bidx.reshape(-1, budget)
    n_rows = sel_all.shape[0]
    col = torch.arange(budget, device=DEV)
    for r0 in range(0, n_rows, 65536):
        sel = sel_all[r0:r0 + 65536]
        if pos is None:
            p = torch.arange(r0, r0 + sel.shape[0], device=DEV, dtype=torch.int64) + q_offset
        else:
            p = pos[r0:r0 + sel.shape[0]].to(torch.int64)
        o = p // 4
        n = torch.clamp(o, max=budget)
        valid = col[None, :] < n[:, None]
        s64 = sel.to(torch.int64)
        assert torch.equal(sel >= 0, valid), "rows %d..: ids / padding layout" % r0
        assert bool(((s64 < o[:, None]) | ~valid).all()), "rows %d..: id past floor(p/4)" % r0
        asc = (s64[:, 1:] > s64[:, :-1]) | ~valid[:, 1:]
        assert bool(asc.all()), "rows %d..: not strictly ascending" % r0
    return n_rows


def _sample_rows(L, stride, tail, extra=()):
    rows = set(range(stride - 1, L, stride)) | set(range(L - tail, L)) | set(int(e) for e in extra if 0 <= e < L)
    return np.array(sorted(rows), dtype=np.int64)


def test_prefill_32k_sampled():
    w = synth.WORKLOADS["prefill_32k"]
    x = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in synth.prefill_inputs(w, "cpu").items()}
    out, bidx = _prefill_run(w, x)
    _check_invariants(bidx, w.budget)
    n = _check_needles_prefill(x["needles"][0], bidx)
    plan = x["needles"][0]
    rows = _sample_rows(w.seq_len, 512, 16, [p[0] for p in plan.probes[::8]] + [2044, 2047, 2048, 2051, 2052])
    worst = _check_rows(x, out, bidx, O.Params(budget=w.budget), rows)
    _say("prefill 32k: %d rows vs oracle (max abs err %.4g), %d needle probes" % (len(rows), worst, n))


def test_prefill_256k_sampled_bench_config():
    w = synth.WORKLOADS["prefill_256k"]
    x = synth.prefill_inputs(w, DEV)
    out, bidx = _prefill_run(w, x)
    _check_invariants(bidx, w.budget)
    n = _check_needles_prefill(x["needles"][0], bidx)
    plan = x["needles"][0]
    # every 1024th row, the recency-scaled tail, and one probe of every 16th needle
    rows = _sample_rows(w.seq_len, 1024, 24, [p[0] for p in plan.probes[::16]] + [262144 - 257, 262144 - 256])
    worst = _check_rows(x, out, bidx, O.Params(budget=w.budget), rows)
    _say("prefill 256k: %d rows vs oracle (max abs err %.4g), %d needle probes" % (len(rows), worst, n))


def _decode_run(w):
    B, ctx = w.batch, w.seq_len
    x = synth.decode_inputs(w, DEV)
    h = Q.Handle(max_ctx=ctx + 4, budget_blocks=w.budget, yarn_factor=w.yarn_factor)
    c = Q.alloc_caches(h, B)
    for b in range(B):
        cs = {k: v[b:b + 1] for k, v in c.items()}
        Q.qsa_append(h, 1, ctx, 0, x["k"][b:b + 1, :ctx], x["v"][b:b + 1, :ctx], x["k_idx"][b:b + 1, :ctx],
                     cs["k_cache"], cs["v_cache"], cs["kbar_cache"], cs["kpend"])
    new = {n: x[n][:, ctx:ctx + 1].contiguous() for n in ("k", "v", "k_idx")}
    cache_len = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    ws = Q.workspace(h, Q.QSA_OP_DECODE, B, 1, ctx)
    out = torch.empty((B, 1, 24, 256), dtype=torch.bfloat16, device=DEV)
    bidx = torch.empty((B, 1, w.budget), dtype=torch.int32, device=DEV)
    Q.qsa_decode(h, B, cache_len, ctx, x["q"], new["k"], new["v"], x["q_idx"], new["k_idx"], c["k_cache"],
                 c["v_cache"], c["kbar_cache"], c["kpend"], out, bidx, ws)
    torch.cuda.synchronize()
    return x, out, bidx


def _check_decode(w, x, out, bidx, seqs):
    p = O.Params(budget=w.budget, yarn_factor=w.yarn_factor)
    _check_invariants(bidx, w.budget, pos=torch.full((w.batch,), w.seq_len, device=DEV))
    bi = bidx.cpu().numpy()
    for b in range(w.batch):                      # needles of every sequence
        for blk in x["needles"][b].blocks:
            assert blk in bi[b, 0], "sequence %d misses needle block %d" % (b, blk)
    worst = 0.0
    for b in seqs:
        lay = O.LayerOracle(bits(x["k"][b]), bits(x["v"][b]), bits(x["k_idx"][b]), p)
        ref, sel, sc = lay.row(w.seq_len, bits(x["q"][b, 0]), bits(x["q_idx"][b, 0]))
        check_selection(bi[b, 0], sel, sc, w.budget, w.seq_len // 4, "seq %d" % b)
        err, _ = check_out(out[b, 0].float().cpu().numpy(), ref, "seq %d" % b)
        worst = max(worst, err)
        del lay
    return worst


def test_decode_128k_sampled_bench_config():
    w = synth.WORKLOADS["decode_128k"]
    x, out, bidx = _decode_run(w)
    seqs = tuple(range(0, 64, 9))
    worst = _check_decode(w, x, out, bidx, seqs=seqs)
    _say("decode 128k: %d sequences vs oracle (max abs err %.4g), invariants and needles of 64 sequences" % (
        len(seqs), worst))


def test_decode_long_rows_candidate_lists():
    """One call of 32 ragged rows whose longest row (80,000 cached tokens,
    20,000 candidate blocks) the scan covers with 8 work-groups, so the
    selection reads the scan's candidate lists.  Row 0 has a zero indexer
    query: every score is 0, every score is a candidate -- more than the list
    selection holds in registers -- and the exact radix path takes it (ties go
    to the later block: its last 512 blocks).  Row 1 (60,000 tokens) takes the
    list path over 6 work-groups; rows 2.. are short.  Invariants on every
    row, rows 0, 1, 2 and 31 against the oracle."""
    budget, B = 512, 32
    lens = [80000, 60000] + [300 + 97 * b for b in range(2, B)]
    w = synth.Workload("t", "decode", B, max(lens), budget, 4, "random", 47)
    x = synth.decode_inputs(w, DEV, ctx=max(lens), batch=B)
    x["q_idx"][0] = 0
    h = Q.Handle(max_ctx=max(lens) + 4, budget_blocks=budget)
    c = Q.alloc_caches(h, B)
    for b, n in enumerate(lens):
        cs = {k: v[b:b + 1] for k, v in c.items()}
        Q.qsa_append(h, 1, n, 0, x["k"][b:b + 1, :n].contiguous(), x["v"][b:b + 1, :n].contiguous(),
                     x["k_idx"][b:b + 1, :n].contiguous(), cs["k_cache"], cs["v_cache"], cs["kbar_cache"],
                     cs["kpend"])
    new = {n: torch.stack([x[n][b, lens[b]] for b in range(B)])[:, None].contiguous() for n in ("k", "v", "k_idx")}
    cache_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = Q.workspace(h, Q.QSA_OP_DECODE, B, 1, max(lens))
    out = torch.empty((B, 1, 24, 256), dtype=torch.bfloat16, device=DEV)
    bidx = torch.empty((B, 1, budget), dtype=torch.int32, device=DEV)
    Q.qsa_decode(h, B, cache_len, max(lens), x["q"], new["k"], new["v"], x["q_idx"], new["k_idx"], c["k_cache"],
                 c["v_cache"], c["kbar_cache"], c["kpend"], out, bidx, ws)
    torch.cuda.synchronize()
    _check_invariants(bidx, budget, pos=cache_len)
    bi = bidx.cpu().numpy()
    assert np.array_equal(bi[0, 0], np.arange(lens[0] // 4 - budget, lens[0] // 4)), "row 0: not its last blocks"
    p = O.Params(budget=budget)
    worst = 0.0
    for b in (0, 1, 2, B - 1):
        n = lens[b]
        lay = O.LayerOracle(bits(x["k"][b, :n + 1]), bits(x["v"][b, :n + 1]), bits(x["k_idx"][b, :n + 1]), p)
        ref, sel, sc = lay.row(n, bits(x["q"][b, 0]), bits(x["q_idx"][b, 0]))
        check_selection(bi[b, 0], sel, sc, budget, n // 4, "row %d" % b)
        err, _ = check_out(out[b, 0].float().cpu().numpy(), ref, "row %d" % b)
        worst = max(worst, err)
        del lay
    _say("decode long rows: invariants of %d rows, 4 vs oracle (max abs err %.4g)" % (B, worst))


def test_decode_1m_yarn_sampled():
    w = synth.WORKLOADS["decode_1m"]
    x, out, bidx = _decode_run(w)
    worst = _check_decode(w, x, out, bidx, seqs=(0, 3, 7))
    _say("decode 1M yarn: 3 sequences vs oracle (max abs err %.4g), invariants and needles of 8 sequences" % worst)


def test_prefill_1m_yarn_chunked_sampled():
    w = synth.WORKLOADS["prefill_1m"]
    x = synth.prefill_inputs(w, DEV)
    out, bidx = _prefill_run(w, x, chunk=w.chunk)
    _check_invariants(bidx, w.budget)
    n = _check_needles_prefill(x["needles"][0], bidx)
    bounds = [c + d for c in range(w.chunk, w.seq_len, w.chunk) for d in (-1, 0, 1)]
    rows = _sample_rows(w.seq_len, 16384, 4, bounds[::2])
    worst = _check_rows(x, out, bidx, O.Params(budget=w.budget, yarn_factor=w.yarn_factor), rows)
    _say("prefill 1M chunked yarn: %d rows vs oracle (max abs err %.4g), %d needle probes" % (len(rows), worst, n))
