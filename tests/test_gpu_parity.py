"""Parity of the HIP library against the CPU oracle, element by element, on
seeded synthetic inputs small enough for the oracle to finish in seconds but
spanning several tiles of every kernel and a ragged tail.  All calls go
through the C ABI (ctypes binding)."""
import numpy as np
import pytest
import torch

import block_sparse_long_qsa_amd as Q
import oracle as O
import synth
from helpers import (bits, check_out, check_scores, check_selection, f32, kcache_tokens, oracle_layer,
                     vcache_tokens)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _to(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _prefill(w, L=None, B=None):
    x = synth.prefill_inputs(w, "cpu", seq_len=L, batch=B)
    return x, _to(x)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.lib()          # fails loudly if libqsa.so is missing
    yield
    torch.cuda.synchronize()


def _forward(h, xd, B, L, q_offset=0, caches=None, chunks=None):
    c = caches if caches is not None else Q.alloc_caches(h, B)
    out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    bidx = torch.empty((B, L, h.budget), dtype=torch.int32, device=DEV)
    spans = chunks or [(0, L)]
    for s0, s1 in spans:
        n = s1 - s0
        ws = Q.workspace(h, Q.QSA_OP_FORWARD, B, n, q_offset + s0)
        sl = lambda t: t[:, s0:s1].contiguous()
        o = torch.empty((B, n, 24, 256), dtype=torch.bfloat16, device=DEV)
        bi = torch.empty((B, n, h.budget), dtype=torch.int32, device=DEV)
        Q.qsa_forward(h, B, n, q_offset + s0, sl(xd["q"]), sl(xd["k"]), sl(xd["v"]), sl(xd["q_idx"]),
                      sl(xd["k_idx"]), c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], o, bi, ws)
        out[:, s0:s1] = o
        bidx[:, s0:s1] = bi
    torch.cuda.synchronize()
    return out, bidx, c


# ---------------------------------------------------------------- prologue
@pytest.mark.parametrize("yarn", [1.0, 4.0])
def test_append_caches_bit_exact(yarn):
    """Rotated K~, transposed V, pooled k̄ and pending raw keys, appended in
    three calls at unaligned offsets, equal the oracle's bf16 values bit for bit."""
    B, L = 2, 203
    w = synth.Workload("t", "prefill", B, L, 64, 4, "random", 21)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=256, budget_blocks=64, yarn_factor=yarn)
    c = Q.alloc_caches(h, B)
    for s0, s1 in [(0, 33), (33, 34), (34, 203)]:
        sl = lambda t: t[:, s0:s1].contiguous()
        Q.qsa_append(h, B, s1 - s0, s0, sl(xd["k"]), sl(xd["v"]), sl(xd["k_idx"]), c["k_cache"], c["v_cache"],
                     c["kbar_cache"], c["kpend"])
    torch.cuda.synchronize()
    p = O.Params(yarn_factor=yarn)
    kt = kcache_tokens(c["k_cache"])
    vt = vcache_tokens(c["v_cache"])
    pos = np.arange(L)
    for b in range(B):
        ref_k = O.f32_to_bf16_bits(O.core_rotate(bits(x["k"][b]), pos, p))          # [L][2][256]
        got_k = bits(kt[b, :, :L].permute(1, 0, 2))
        assert np.array_equal(got_k, ref_k)
        assert np.array_equal(bits(vt[b, :, :L].permute(1, 0, 2)), bits(x["v"][b]))
        ref_kbar = O.f32_to_bf16_bits(O.indexer_keys(bits(x["k_idx"][b]), p))      # [50][128]
        assert np.array_equal(bits(c["kbar_cache"][b, :L // 4]), ref_kbar)
        assert np.array_equal(bits(c["kpend"][b, :L % 4]), bits(x["k_idx"][b, (L // 4) * 4:]))


# ---------------------------------------------------------------- indexer
@pytest.mark.parametrize("B,L,q_offset", [(1, 2500, 0), (2, 333, 0), (1, 640, 1024)])
def test_index_scores(B, L, q_offset):
    """qsa_index scores vs the oracle's fp64 scores; -1 on every non-candidate."""
    w = synth.Workload("t", "prefill", B, q_offset + L, 64, 6, "random", 22)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=4096, budget_blocks=64)
    c = Q.alloc_caches(h, B)
    Q.qsa_append(h, B, q_offset + L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"],
                 c["kpend"])
    ncol = (q_offset + L + 3) // 4
    scores = torch.empty((B, L, ncol), dtype=torch.float32, device=DEV)
    ws = Q.workspace(h, Q.QSA_OP_INDEX, B, L, q_offset)
    sl = lambda t: t[:, q_offset:q_offset + L].contiguous()
    Q.qsa_index(h, B, L, q_offset, sl(xd["q_idx"]), c["kbar_cache"], scores, ws)
    # the fused index + select stage selects what select(scores) selects
    bidx_a = torch.empty((B, L, h.budget), dtype=torch.int32, device=DEV)
    bidx_b = torch.empty_like(bidx_a)
    Q.qsa_select(h, B, L, q_offset, scores, bidx_a)
    ws2 = Q.workspace(h, Q.QSA_OP_INDEX_SELECT, B, L, q_offset)
    Q.qsa_index_select(h, B, L, q_offset, sl(xd["q_idx"]), c["kbar_cache"], bidx_b, ws2)
    torch.cuda.synchronize()
    s = f32(scores)
    p = O.Params()
    for b in range(B):
        kbar = O.indexer_keys(bits(x["k_idx"][b]), p)
        qt = O.indexer_queries(bits(x["q_idx"][b, q_offset:]), np.arange(q_offset, q_offset + L), p)
        for i in range(L):
            o = (q_offset + i) // 4
            check_scores(s[b, i, :o], O.block_scores(qt[i], kbar[:o]), "b%d row %d" % (b, i))
            assert np.all(s[b, i, o:] == -1.0)
    assert torch.equal(bidx_a, bidx_b)


# ---------------------------------------------------------------- fused index + select
def _index_paths(h, x, xd, B, L):
    c = Q.alloc_caches(h, B)
    Q.qsa_append(h, B, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    ncol = (L + 3) // 4
    scores = torch.empty((B, L, ncol), dtype=torch.float32, device=DEV)
    Q.qsa_index(h, B, L, 0, xd["q_idx"], c["kbar_cache"], scores, Q.workspace(h, Q.QSA_OP_INDEX, B, L, 0))
    a = torch.empty((B, L, h.budget), dtype=torch.int32, device=DEV)
    Q.qsa_select(h, B, L, 0, scores, a)
    f = torch.empty_like(a)
    Q.qsa_index_select(h, B, L, 0, xd["q_idx"], c["kbar_cache"], f, Q.workspace(h, Q.QSA_OP_INDEX_SELECT, B, L, 0))
    torch.cuda.synchronize()
    return a, f


@pytest.mark.parametrize("budget", [17, 64, 512])
def test_index_select_fused_equals_score_matrix_path(budget):
    """The fused streaming kernel selects exactly what select(score matrix) selects."""
    B, L = 2, 6000
    w = synth.Workload("t", "prefill", B, L, budget, 8, "random", 40 + budget)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=6144, budget_blocks=budget)
    a, f = _index_paths(h, x, xd, B, L)
    assert torch.equal(a, f)


@pytest.mark.parametrize("kind", ["zero_blocks", "large_scores"])
def test_index_select_fused_end_bins(kind):
    """Boundaries in the two clamped end bins of the fused kernel's histogram:
    half the pooled keys zero (many exact 0 scores, ties broken by block), or
    keys scaled by 16 (budget-th score above the histogram's top edge)."""
    B, L, budget = 1, 6000, 512
    w = synth.Workload("t", "prefill", B, L, budget, 8, "random", 43)
    x = synth.prefill_inputs(w, "cpu")
    if kind == "zero_blocks":
        g = np.random.default_rng(44)
        dead = np.nonzero(g.random(L // 4) < 0.5)[0]
        tok = (dead[:, None] * 4 + np.arange(4)[None, :]).reshape(-1)
        x["k_idx"][:, torch.from_numpy(tok)] = 0
    else:
        x["k_idx"] = x["k_idx"] * 16
    xd = _to(x)
    h = Q.Handle(max_ctx=6144, budget_blocks=budget)
    a, f = _index_paths(h, x, xd, B, L)
    assert torch.equal(a, f)
    p = O.Params(budget=budget)
    lay = oracle_layer(x, 0, p)
    fb = f.cpu().numpy()
    for i in [2051, 2400, 3000, 4095, 4099, 5999]:
        _, sel, sc = lay.row(i, bits(x["q"][0, i]), bits(x["q_idx"][0, i]))
        check_selection(fb[0, i], sel, sc, budget, i // 4, "row %d" % i)


def test_index_select_overflow_fallback():
    """With a candidate list far shorter than needed every long row overflows and
    is recomputed exactly: the result still meets the oracle."""
    B, L, budget = 1, 5000, 64
    w = synth.Workload("t", "prefill", B, L, budget, 8, "random", 41)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=5120, budget_blocks=budget, topk_cap=64)
    a, f = _index_paths(h, x, xd, B, L)
    p = O.Params(budget=budget)
    lay = oracle_layer(x, 0, p)
    fb = f.cpu().numpy()
    for i in list(range(250, 270)) + list(range(4990, 5000)) + [1234, 3000]:
        _, sel, sc = lay.row(i, bits(x["q"][0, i]), bits(x["q_idx"][0, i]))
        check_selection(fb[0, i], sel, sc, budget, i // 4, "row %d" % i)


# ---------------------------------------------------------------- select
@pytest.mark.parametrize("mode", ["float", "coarse", "zeros", "mixed"])
@pytest.mark.parametrize("budget", [1, 7, 64, 512])
def test_select_bit_exact(mode, budget):
    """qsa_select on seeded score rows (with many exact ties) equals the oracle's
    (score desc, block desc) top-k exactly."""
    B, L, q_offset = 2, 300, 2400
    s = synth.score_rows(31 + budget, B, L, q_offset, mode)
    h = Q.Handle(max_ctx=4096, budget_blocks=budget)
    bidx = torch.empty((B, L, budget), dtype=torch.int32, device=DEV)
    Q.qsa_select(h, B, L, q_offset, torch.from_numpy(s).to(DEV), bidx)
    torch.cuda.synchronize()
    got = bidx.cpu().numpy()
    for b in range(B):
        for i in range(L):
            o = (q_offset + i) // 4
            ref = O.select_blocks(s[b, i, :o].astype(np.float64), budget)
            assert np.array_equal(got[b, i], ref), (mode, budget, b, i)


def test_select_small_rows():
    """Rows with fewer candidates than the budget (including none) take them all."""
    B, L = 1, 40
    s = synth.score_rows(5, B, L, 0, "coarse")
    h = Q.Handle(max_ctx=64, budget_blocks=8)
    bidx = torch.empty((B, L, 8), dtype=torch.int32, device=DEV)
    Q.qsa_select(h, B, L, 0, torch.from_numpy(s).to(DEV), bidx)
    torch.cuda.synchronize()
    got = bidx.cpu().numpy()
    for i in range(L):
        assert np.array_equal(got[0, i], O.select_blocks(s[0, i, :i // 4].astype(np.float64), 8))


# ---------------------------------------------------------------- attention
def test_attend_with_oracle_selection():
    """qsa_attend over the oracle's own selection vs the oracle's output rows."""
    B, L, budget = 1, 700, 16
    w = synth.Workload("t", "prefill", B, L, budget, 4, "random", 23)
    x, xd = _prefill(w)
    p = O.Params(budget=budget)
    rows = np.arange(L)
    ref, sel, _ = O.prefill_rows(*(bits(x[n][0]) for n in ("q", "k", "v", "q_idx", "k_idx")), rows, p)
    h = Q.Handle(max_ctx=1024, budget_blocks=budget)
    c = Q.alloc_caches(h, B)
    Q.qsa_append(h, B, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    Q.qsa_attend(h, B, L, 0, xd["q"], c["k_cache"], c["v_cache"], torch.from_numpy(sel[None]).to(DEV), out)
    torch.cuda.synchronize()
    check_out(f32(out[0]), ref, "attend")


def test_attend_skips_leading_invalid_entries():
    """qsa_attend skips block_idx entries outside [0, floor(p/4)), also when
    they fill the whole first chunks of a row's walk (12 leading entries of -1
    or ids >= floor(p/4)); the rest of the list and the own block are attended
    as the oracle attends them.  Rows whose every entry is invalid attend their
    own block alone."""
    B, L, budget = 1, 600, 32
    w = synth.Workload("t", "prefill", B, L, budget, 4, "random", 41)
    x, xd = _prefill(w)
    rng = np.random.default_rng(41)
    sel = np.full((L, budget), -1, dtype=np.int32)
    for i in range(L):
        o = i // 4
        bad = np.where(rng.random(12) < 0.5, -1, o + rng.integers(0, 50, 12)).astype(np.int32)
        if i % 7 == 0:                                   # nothing valid at all
            sel[i] = np.where(rng.random(budget) < 0.5, -1, o + rng.integers(0, 9, budget))
            continue
        n_ok = min(o, budget - 12)
        ok = np.sort(rng.choice(o, n_ok, replace=False)).astype(np.int32) if n_ok > 0 else np.zeros(0, np.int32)
        row = np.concatenate([bad, ok])
        sel[i, :row.size] = row[:budget]
    h = Q.Handle(max_ctx=1024, budget_blocks=budget)
    c = Q.alloc_caches(h, B)
    Q.qsa_append(h, B, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    Q.qsa_attend(h, B, L, 0, xd["q"], c["k_cache"], c["v_cache"], torch.from_numpy(sel[None]).to(DEV), out)
    torch.cuda.synchronize()
    o = f32(out[0])
    assert np.isfinite(o).all()
    p = O.Params(budget=budget)
    lay = oracle_layer(x, 0, p)
    for i in range(0, L, 3):
        # the entries the walk reads are the first min(floor(p/4), budget); only ids in [0, floor(p/4)) count
        n_read = min(i // 4, budget)
        ref = lay.row_reused(i, bits(x["q"][0, i]), sel[i, :n_read], i)
        check_out(o[i], ref, "row %d" % i)


# ---------------------------------------------------------------- forward
def _check_forward(x, out, bidx, p, rows, seqs=(0,), q_offset=0):
    n_swapped = 0
    for b in seqs:
        lay = oracle_layer(x, b, p)
        for i in rows:
            pos = q_offset + int(i)
            ref, sel, sc = lay.row(pos, bits(x["q"][b, i]), bits(x["q_idx"][b, i]))
            n_swapped += check_selection(bidx[b, i], sel, sc, p.budget, pos // 4, "b%d row %d" % (b, i))
            check_out(out[b, i], ref, "b%d row %d" % (b, i))
    return n_swapped


def test_forward_prefill_1k_all_rows():
    """The small prefill workload (L=1024, budget 64, 8 needles): every row."""
    w = synth.WORKLOADS["prefill_1k"]
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=1024, budget_blocks=w.budget)
    out, bidx, _ = _forward(h, xd, 1, w.seq_len)
    _check_forward(x, f32(out), bidx.cpu().numpy(), O.Params(budget=w.budget), range(w.seq_len))
    # planted needles are selected by their probes
    plan = x["needles"][0]
    bi = bidx.cpu().numpy()[0]
    for n, blk in enumerate(plan.blocks):
        for pr in plan.probes[n]:
            assert blk in bi[pr]


def test_forward_ragged_batch2():
    B, L, budget = 2, 1027, 40
    w = synth.Workload("t", "prefill", B, L, budget, 5, "random", 24)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    out, bidx, c = _forward(h, xd, B, L)
    rows = list(range(0, 12)) + list(range(150, 170)) + list(range(L - 40, L))
    _check_forward(x, f32(out), bidx.cpu().numpy(), O.Params(budget=budget), rows, seqs=(0, 1))
    # the trailing incomplete block's raw keys are pending
    assert np.array_equal(bits(c["kpend"][:, :L % 4]), bits(x["k_idx"][:, (L // 4) * 4:]))


def test_forward_chunked_equals_one_shot():
    """Chunked prefill (chunk starts multiple of 4) is bit-identical to one shot."""
    B, L, budget = 1, 2048, 64
    w = synth.Workload("t", "prefill", B, L, budget, 8, "even", 25)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    o1, b1, _ = _forward(h, xd, B, L)
    o2, b2, _ = _forward(h, xd, B, L, chunks=[(0, 512), (512, 1300), (1300, 2048)])
    assert torch.equal(b1, b2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    _check_forward(x, f32(o2), b2.cpu().numpy(), O.Params(budget=budget), [511, 512, 513, 1299, 1300, 2047])


def test_forward_deterministic():
    B, L, budget = 1, 1500, 100
    w = synth.Workload("t", "prefill", B, L, budget, 4, "random", 26)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=1536, budget_blocks=budget)
    o1, b1, _ = _forward(h, xd, B, L)
    o2, b2, _ = _forward(h, xd, B, L)
    assert torch.equal(b1, b2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_forward_yarn_small():
    B, L, budget = 1, 900, 32
    w = synth.Workload("t", "prefill", B, L, budget, 4, "random", 27, yarn_factor=4.0)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=1024, budget_blocks=budget, yarn_factor=4.0)
    out, bidx, _ = _forward(h, xd, B, L)
    _check_forward(x, f32(out), bidx.cpu().numpy(), O.Params(budget=budget, yarn_factor=4.0),
                   list(range(0, 8)) + list(range(800, 900)))


# ---------------------------------------------------------------- decode
def _decode_setup(w, ctx_per_seq, h, edit=None):
    """Caches filled by qsa_append to each sequence's own length, then one
    decode step; edit(x) may change the host inputs first."""
    B = len(ctx_per_seq)
    x = synth.decode_inputs(w, "cpu", ctx=max(ctx_per_seq), batch=B)
    if edit is not None:
        edit(x)
    xd = _to(x)
    c = Q.alloc_caches(h, B)
    for b, n in enumerate(ctx_per_seq):
        if n == 0:
            continue
        sl = lambda t: t[b:b + 1, :n].contiguous()
        cs = {k: v[b:b + 1] for k, v in c.items()}
        Q.qsa_append(h, 1, n, 0, sl(xd["k"]), sl(xd["v"]), sl(xd["k_idx"]), cs["k_cache"], cs["v_cache"],
                     cs["kbar_cache"], cs["kpend"])
    # the new token of sequence b sits at position n_b: take its k/v/k_idx from that row
    new = {n: torch.stack([xd[n][b, ctx_per_seq[b]] for b in range(B)])[:, None].contiguous()
           for n in ("k", "v", "k_idx")}
    cache_len = torch.tensor(ctx_per_seq, dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, 24, 256), dtype=torch.bfloat16, device=DEV)
    bidx = torch.empty((B, 1, h.budget), dtype=torch.int32, device=DEV)
    bound = max(ctx_per_seq)
    ws = Q.workspace(h, Q.QSA_OP_DECODE, B, 1, bound)
    Q.qsa_decode(h, B, cache_len, bound, xd["q"], new["k"], new["v"], xd["q_idx"], new["k_idx"], c["k_cache"],
                 c["v_cache"], c["kbar_cache"], c["kpend"], out, bidx, ws)
    torch.cuda.synchronize()
    return x, out, bidx, c


def test_decode_small_ragged_lengths():
    budget = 48
    lens = [1500, 3, 0, 1201, 1202, 1203, 700, 257]
    w = synth.Workload("t", "decode", len(lens), max(lens), budget, 6, "random", 28)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    x, out, bidx, c = _decode_setup(w, lens, h)
    p = O.Params(budget=budget)
    o = f32(out)
    bi = bidx.cpu().numpy()
    for b, n in enumerate(lens):
        lay = oracle_layer(x, b, p, n_keys=n + 1)
        ref, sel, sc = lay.row(n, bits(x["q"][b, 0]), bits(x["q_idx"][b, 0]))
        check_selection(bi[b, 0], sel, sc, budget, n // 4, "seq %d" % b)
        check_out(o[b, 0], ref, "seq %d" % b)
        # the appended token and, for completed blocks, its pooled key are in the caches
        if n % 4 == 3:
            ref_kbar = O.f32_to_bf16_bits(O.indexer_keys(bits(x["k_idx"][b, :n + 1]), p))
            assert np.array_equal(bits(c["kbar_cache"][b, n // 4]), ref_kbar[n // 4])


def test_decode_long_ragged_rows_many_scan_workgroups():
    """Rows of 16,383 / 10,000 / 2,047 / 75 candidate blocks in one call: the
    scan splits each row over up to 16 work-groups (256 keys per wave at this
    batch), rows leave different numbers of histogram summaries, one row keeps
    all its candidates; selections and outputs against the oracle's rows."""
    budget = 512
    lens = [65535, 40003, 8190, 300]
    w = synth.Workload("t", "decode", len(lens), max(lens), budget, 8, "random", 31)
    h = Q.Handle(max_ctx=65540, budget_blocks=budget)
    x, out, bidx, _ = _decode_setup(w, lens, h)
    p = O.Params(budget=budget)
    o = f32(out)
    bi = bidx.cpu().numpy()
    for b, n in enumerate(lens):
        lay = oracle_layer(x, b, p, n_keys=n + 1)
        ref, sel, sc = lay.row(n, bits(x["q"][b, 0]), bits(x["q_idx"][b, 0]))
        check_selection(bi[b, 0], sel, sc, budget, n // 4, "seq %d" % b)
        check_out(o[b, 0], ref, "seq %d" % b)


@pytest.mark.parametrize("B", [130, 256])
def test_decode_large_batch_few_splits(B):
    """Batches whose split attention has two splits per (sequence, KV group)
    (B = 130) or one (B = 256, the merge of a single partial), ragged lengths
    from 0 to 700 tokens: every sequence's selection and output against the
    oracle's row."""
    budget = 32
    rng = np.random.default_rng(40 + B)
    lens = [int(v) for v in rng.integers(0, 701, size=B)]
    lens[:6] = [0, 1, 3, 4, 127, 700]
    w = synth.Workload("t", "decode", B, max(lens), budget, 4, "random", 41 + B)
    h = Q.Handle(max_ctx=1024, budget_blocks=budget)
    x, out, bidx, _ = _decode_setup(w, lens, h)
    p = O.Params(budget=budget)
    o = f32(out)
    bi = bidx.cpu().numpy()
    for b, n in enumerate(lens):
        lay = oracle_layer(x, b, p, n_keys=n + 1)
        ref, sel, sc = lay.row(n, bits(x["q"][b, 0]), bits(x["q_idx"][b, 0]))
        check_selection(bi[b, 0], sel, sc, budget, n // 4, "seq %d" % b)
        check_out(o[b, 0], ref, "seq %d" % b)


def test_decode_crowded_boundary_digits():
    """Ties at the selection boundary: sequence 0 has a zero indexer query (every
    score is 0, so the boundary digit holds all 1,250 candidates, more than the
    digit's fast path ranks), sequence 1 zero keys for 400 of its 750 blocks
    (fewer than 512 positive scores, then a boundary digit of about 420 tied
    zeros), sequence 2 no ties.  Ties go to the later block; selections and
    outputs against the oracle's rows."""
    budget = 512
    lens = [5000, 3000, 4500]

    def edit(x):
        x["q_idx"][0] = 0
        x["k_idx"][1, 4 * 100:4 * 500] = 0

    w = synth.Workload("t", "decode", len(lens), max(lens), budget, 4, "random", 36)
    h = Q.Handle(max_ctx=8192, budget_blocks=budget)
    x, out, bidx, _ = _decode_setup(w, lens, h, edit)
    p = O.Params(budget=budget)
    o = f32(out)
    bi = bidx.cpu().numpy()
    for b, n in enumerate(lens):
        lay = oracle_layer(x, b, p, n_keys=n + 1)
        ref, sel, sc = lay.row(n, bits(x["q"][b, 0]), bits(x["q_idx"][b, 0]))
        check_selection(bi[b, 0], sel, sc, budget, n // 4, "seq %d" % b)
        check_out(o[b, 0], ref, "seq %d" % b)
    # all scores tie in sequence 0: the selection is the last 512 blocks
    assert np.array_equal(bi[0, 0], np.arange(lens[0] // 4 - budget, lens[0] // 4))


def test_decode_matches_prefill_row():
    """Decode at p and prefill row p (same n+1 tokens, same query) both meet the
    oracle's row p, and agree with each other."""
    budget, n = 64, 1403
    w = synth.Workload("t", "decode", 1, n, budget, 6, "random", 29)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    x, out_d, bidx_d, _ = _decode_setup(w, [n], h)
    xp = {k: x[k][:, :n + 1].clone() for k in ("k", "v", "k_idx")}
    xp["q"] = torch.zeros((1, n + 1, 24, 256), dtype=torch.bfloat16)
    xp["q_idx"] = torch.zeros((1, n + 1, 4, 128), dtype=torch.bfloat16)
    xp["q"][:, n] = x["q"][:, 0]
    xp["q_idx"][:, n] = x["q_idx"][:, 0]
    out_p, bidx_p, _ = _forward(h, _to(xp), 1, n + 1)
    p = O.Params(budget=budget)
    ref, sel, sc = oracle_layer(x, 0, p, n_keys=n + 1).row(n, bits(x["q"][0, 0]), bits(x["q_idx"][0, 0]))
    for name, o, bi in (("decode", out_d[0, 0], bidx_d[0, 0]), ("prefill", out_p[0, n], bidx_p[0, n])):
        check_selection(bi.cpu().numpy(), sel, sc, budget, n // 4, name)
        check_out(f32(o), ref, name)
    check_out(f32(out_d[0, 0]), f32(out_p[0, n]).astype(np.float64), "decode vs prefill")


def test_decode_reuse_speculative_steps():
    """A full decode step at p0, then draft steps p0+1 .. p0+4 (crossing a block
    boundary) that reuse its selection: reuse at p0 itself reproduces the full
    step bit for bit, and every draft step meets the oracle's reused-selection
    row; the appended tokens keep the caches exact."""
    budget, p0s = 48, [1202, 999]
    B, L = len(p0s), max(p0s) + 6
    w = synth.Workload("t", "prefill", B, L, budget, 6, "random", 30)
    x = synth.prefill_inputs(w, "cpu")
    xd = _to(x)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    c = Q.alloc_caches(h, B)
    for b, n in enumerate(p0s):
        sl = lambda t: t[b:b + 1, :n].contiguous()
        cs = {k: v[b:b + 1] for k, v in c.items()}
        Q.qsa_append(h, 1, n, 0, sl(xd["k"]), sl(xd["v"]), sl(xd["k_idx"]), cs["k_cache"], cs["v_cache"],
                     cs["kbar_cache"], cs["kpend"])

    def tok(name, pos):
        return torch.stack([xd[name][b, pos[b]] for b in range(B)])[:, None].contiguous()

    bound = max(p0s) + 4
    ws = Q.workspace(h, Q.QSA_OP_DECODE, B, 1, bound)
    sel_pos = torch.tensor(p0s, dtype=torch.int32, device=DEV)
    out0 = torch.empty((B, 1, 24, 256), dtype=torch.bfloat16, device=DEV)
    bidx0 = torch.empty((B, 1, budget), dtype=torch.int32, device=DEV)
    Q.qsa_decode(h, B, sel_pos, bound, tok("q", p0s), tok("k", p0s), tok("v", p0s), tok("q_idx", p0s),
                 tok("k_idx", p0s), c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], out0, bidx0, ws)
    sel_gpu = bidx0.view(B, budget).contiguous()
    out_r = torch.empty_like(out0)
    Q.qsa_decode_reuse(h, B, sel_pos, sel_pos, bound, tok("q", p0s), tok("k", p0s), tok("v", p0s),
                       tok("k_idx", p0s), c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], sel_gpu, out_r, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out0)
    p = O.Params(budget=budget)
    lays = [oracle_layer(x, b, p) for b in range(B)]
    sels = []
    for b, n in enumerate(p0s):
        _, sel, sc = lays[b].row(n, bits(x["q"][b, n]), bits(x["q_idx"][b, n]))
        got = sel_gpu[b].cpu().numpy()
        assert sorted(got[got >= 0].tolist()) == sorted(sel[sel >= 0].tolist()), "seq %d selection" % b
        sels.append(sel)
    for i in range(1, 5):
        pos = [n + i for n in p0s]
        cache_len = torch.tensor(pos, dtype=torch.int32, device=DEV)
        out = torch.empty_like(out0)
        Q.qsa_decode_reuse(h, B, cache_len, sel_pos, bound, tok("q", pos), tok("k", pos), tok("v", pos),
                           tok("k_idx", pos), c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], sel_gpu, out,
                           ws)
        torch.cuda.synchronize()
        o = f32(out)
        for b in range(B):
            ref = lays[b].row_reused(pos[b], bits(x["q"][b, pos[b]]), sels[b], p0s[b])
            check_out(o[b, 0], ref, "seq %d step %d" % (b, i))
            if pos[b] % 4 == 3:
                ref_kbar = O.f32_to_bf16_bits(O.indexer_keys(bits(x["k_idx"][b, :pos[b] + 1]), p))
                assert np.array_equal(bits(c["kbar_cache"][b, pos[b] // 4]), ref_kbar[pos[b] // 4])


def test_decode_reuse_selection_position_bounds():
    """sel_pos is clamped to [0, p]: past p it is the plain decode step (bit for
    bit); below 0 it is 0, so the query attends every token 0..p (its reused
    list names no block before block 0).  Bad sizes are rejected on the host."""
    budget, n, B = 32, 777, 1
    w = synth.Workload("t", "decode", B, n, budget, 4, "random", 31)
    h = Q.Handle(max_ctx=1024, budget_blocks=budget)
    x, out0, bidx0, c = _decode_setup(w, [n], h)
    xd = _to(x)
    new = {k: xd[k][:, n:n + 1].contiguous() for k in ("k", "v", "k_idx")}
    cache_len = torch.tensor([n], dtype=torch.int32, device=DEV)
    ws = Q.workspace(h, Q.QSA_OP_DECODE, B, 1, n)
    sel = bidx0.view(B, budget).contiguous()
    outs = {}
    for name, sp in (("past", n + 50), ("neg", -7)):
        o = torch.empty_like(out0)
        Q.qsa_decode_reuse(h, B, cache_len, torch.tensor([sp], dtype=torch.int32, device=DEV), n, xd["q"], new["k"],
                           new["v"], new["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], sel, o, ws)
        outs[name] = o
    torch.cuda.synchronize()
    assert torch.equal(outs["past"], out0)
    p = O.Params(budget=budget)
    lay = oracle_layer(x, 0, p, n_keys=n + 1)
    ref = lay.row_reused(n, bits(x["q"][0, 0]), np.full(budget, -1), 0)
    check_out(f32(outs["neg"][0, 0]), ref, "sel_pos < 0")
    with pytest.raises(Q.QSAError) as e:
        Q.qsa_decode_reuse(h, B, cache_len, cache_len, n, xd["q"], new["k"], new["v"], new["k_idx"], c["k_cache"],
                           c["v_cache"], c["kbar_cache"], c["kpend"], sel, outs["neg"], ws[:16])
    assert e.value.status == 6
    with pytest.raises(Q.QSAError) as e:
        Q.qsa_decode_reuse(h, B, cache_len, cache_len, 1024, xd["q"], new["k"], new["v"], new["k_idx"],
                           c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], sel, outs["neg"], ws)
    assert e.value.status == 5


def test_decode_reuse_selection_position_below_every_id():
    """A reused selection whose ids all lie at or past the block of sel_pos: the
    first chunks of every split's walk are wholly masked, and the step attends
    only the tail from sel_pos's own block to p, as the oracle's reused row."""
    budget, n, B = 32, 1200, 1
    w = synth.Workload("t", "decode", B, n, budget, 4, "random", 43)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    x, out0, bidx0, c = _decode_setup(w, [n], h)
    xd = _to(x)
    new = {k: xd[k][:, n:n + 1].contiguous() for k in ("k", "v", "k_idx")}
    cache_len = torch.tensor([n], dtype=torch.int32, device=DEV)
    ws = Q.workspace(h, Q.QSA_OP_DECODE, B, 1, n)
    rng = np.random.default_rng(43)
    sel_np = np.sort(rng.choice(np.arange(200, 300), budget, replace=False)).astype(np.int32)[None]
    sel = torch.from_numpy(sel_np).to(DEV)
    p = O.Params(budget=budget)
    lay = oracle_layer(x, 0, p, n_keys=n + 1)
    for sp in (4 * 200, 4 * 100 + 3, 4 * 40 + 2):
        assert sp // 4 <= sel_np.min()
        o = torch.empty_like(out0)
        Q.qsa_decode_reuse(h, B, cache_len, torch.tensor([sp], dtype=torch.int32, device=DEV), n, xd["q"],
                           new["k"], new["v"], new["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"],
                           c["kpend"], sel, o, ws)
        torch.cuda.synchronize()
        got = f32(o[0, 0])
        assert np.isfinite(got).all(), "sel_pos %d" % sp
        ref = lay.row_reused(n, bits(x["q"][0, 0]), sel_np[0], sp)
        check_out(got, ref, "sel_pos %d" % sp)


# ---------------------------------------------------------------- token-level indexer (r = 1)
def _token_prefill(h, xd, B, L, spans):
    ktok = Q.alloc_token_keys(h, B)
    tidx = torch.empty((B, L, h.budget), dtype=torch.int32, device=DEV)
    for s0, s1 in spans:
        n = s1 - s0
        ws = Q.workspace(h, Q.QSA_OP_TOKEN_INDEX_SELECT, B, n, s0)
        ti = torch.empty((B, n, h.budget), dtype=torch.int32, device=DEV)
        Q.qsa_token_index_select(h, B, n, s0, xd["q_idx"][:, s0:s1].contiguous(), xd["k_idx"][:, s0:s1].contiguous(),
                                 ktok, ti, ws)
        tidx[:, s0:s1] = ti
    torch.cuda.synchronize()
    return tidx, ktok


def test_token_index_select_every_row():
    """r = 1 in two chunks at an unaligned offset: token keys rotated at their own
    positions bit for bit, and every row's top tokens meet the oracle."""
    B, L, budget = 2, 700, 48
    w = synth.Workload("t", "prefill", B, L, budget, 6, "random", 61)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=768, budget_blocks=budget)
    tidx, ktok = _token_prefill(h, xd, B, L, [(0, 301), (301, 700)])
    p = O.Params(budget=budget)
    got = tidx.cpu().numpy()
    for b in range(B):
        ref_k = O.f32_to_bf16_bits(O.token_index_keys(bits(x["k_idx"][b]), p))
        assert np.array_equal(bits(ktok[b, :L]), ref_k)
        sel, scs = O.token_index_rows(bits(x["q_idx"][b]), bits(x["k_idx"][b]), range(L), p)
        for i in range(L):
            check_selection(got[b, i], sel[i], scs[i], budget, i, "seq %d row %d" % (b, i))


@pytest.mark.parametrize("cap", [0, 64])
def test_token_index_select_long_rows(cap):
    """r = 1 over 6,000 tokens (the streaming threshold, candidate lists and the
    in-kernel final selection on long rows); with a 64-entry list every long
    row overflows and is recomputed by the fixup kernel."""
    B, L, budget = 1, 6000, 64
    w = synth.Workload("t", "prefill", B, L, budget, 8, "random", 62)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=6144, budget_blocks=budget, topk_cap=cap)
    tidx, _ = _token_prefill(h, xd, B, L, [(0, L)])
    got = tidx.cpu().numpy()
    rows = [0, 1, 63, 64, 65, 500, 2047, 4096, 5000, 5998, 5999]
    sel, scs = O.token_index_rows(bits(x["q_idx"][0, rows]), bits(x["k_idx"][0]), rows, O.Params(budget=budget))
    for j, i in enumerate(rows):
        check_selection(got[0, i], sel[j], scs[j], budget, i, "row %d" % i)


def test_token_index_decode_ragged():
    """One decode step of the token-level indexer per sequence (lengths 0 .. 900)
    equals the oracle's row p over the prefilled keys."""
    budget, lens = 32, [900, 3, 0, 513, 64]
    B, L = len(lens), max(lens) + 1
    w = synth.Workload("t", "prefill", B, L, budget, 6, "random", 63)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=1024, budget_blocks=budget)
    _, ktok = _token_prefill(h, xd, B, L, [(0, L)])
    new_q = torch.stack([xd["q_idx"][b, n] for b, n in enumerate(lens)])[:, None].contiguous()
    new_k = torch.stack([xd["k_idx"][b, n] for b, n in enumerate(lens)])[:, None].contiguous()
    cache_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    bound = max(lens)
    ws = Q.workspace(h, Q.QSA_OP_TOKEN_INDEX_DECODE, B, 1, bound)
    tidx = torch.empty((B, budget), dtype=torch.int32, device=DEV)
    Q.qsa_token_index_decode(h, B, cache_len, bound, new_q, new_k, ktok, tidx, ws)
    torch.cuda.synchronize()
    got = tidx.cpu().numpy()
    p = O.Params(budget=budget)
    for b, n in enumerate(lens):
        sel, scs = O.token_index_rows(bits(x["q_idx"][b, n:n + 1]), bits(x["k_idx"][b, :n + 1]), [n], p)
        check_selection(got[b], sel[0], scs[0], budget, n, "seq %d" % b)


def test_index_decode_equals_decode_selection():
    """qsa_index_decode selects what qsa_decode selects (and the oracle), and
    appends the new token's indexer key the same way."""
    budget = 48
    lens = [1500, 3, 0, 1203, 700]
    w = synth.Workload("t", "decode", len(lens), max(lens), budget, 6, "random", 64)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    x, _, bidx, c = _decode_setup(w, lens, h)
    B = len(lens)
    xd = _to(x)
    c2 = Q.alloc_caches(h, B)
    for b, n in enumerate(lens):
        if n:
            sl = lambda t: t[b:b + 1, :n].contiguous()
            cs = {k: v[b:b + 1] for k, v in c2.items()}
            Q.qsa_append(h, 1, n, 0, sl(xd["k"]), sl(xd["v"]), sl(xd["k_idx"]), cs["k_cache"], cs["v_cache"],
                         cs["kbar_cache"], cs["kpend"])
    new_k = torch.stack([xd["k_idx"][b, n] for b, n in enumerate(lens)])[:, None].contiguous()
    cache_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = Q.workspace(h, Q.QSA_OP_INDEX_DECODE, B, 1, max(lens))
    sel = torch.empty((B, budget), dtype=torch.int32, device=DEV)
    Q.qsa_index_decode(h, B, cache_len, max(lens), xd["q_idx"], new_k, c2["kbar_cache"], c2["kpend"], sel, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel, bidx[:, 0])
    for b, n in enumerate(lens):
        nb = (n + 1) // 4
        assert torch.equal(c2["kbar_cache"][b, :nb], c["kbar_cache"][b, :nb])
        assert torch.equal(c2["kpend"][b, :(n % 4) + 1], c["kpend"][b, :(n % 4) + 1])


def test_binding_checks_buffers_before_launch():
    """A short or host buffer is refused by the binding before anything is
    enqueued (the library sees only its address)."""
    B, L = 1, 64
    h = Q.Handle(max_ctx=L, budget_blocks=16)
    c = Q.alloc_caches(h, B)
    q = torch.zeros((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    bidx = torch.full((B, L, 16), -1, dtype=torch.int32, device=DEV)
    short = torch.empty((B, L - 1, 24, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="needs"):
        Q.qsa_attend(h, B, L, 0, q, c["k_cache"], c["v_cache"], bidx, short)
    with pytest.raises(ValueError, match="device tensor"):
        Q.qsa_attend(h, B, L, 0, q.cpu(), c["k_cache"], c["v_cache"], bidx, torch.empty_like(q))
    small = Q.alloc_caches(Q.Handle(max_ctx=L // 2, budget_blocks=16), B)
    with pytest.raises(ValueError, match="k_cache"):
        Q.qsa_attend(h, B, L, 0, q, small["k_cache"], c["v_cache"], bidx, torch.empty_like(q))
    torch.cuda.synchronize()


def test_batch_beyond_grid_limit_is_a_shape_error():
    """B is a grid dimension of the kernels: B > 65535 is refused on the host
    (QSA_ERR_SHAPE) before any pointer is looked at."""
    h = Q.Handle(max_ctx=64, budget_blocks=16)
    lib = Q.lib()
    assert lib.qsa_attend(h.ptr, None, 65536, 4, 0, None, None, None, None, None) == 2
    assert lib.qsa_append(h.ptr, None, 65536, 4, 0, None, None, None, None, None, None, None) == 2
    assert lib.qsa_decode(h.ptr, None, 65536, None, 64, *([None] * 12), 0) == 2
    assert lib.qsa_attend(h.ptr, None, 0, 4, 0, None, None, None, None, None) == 2


@pytest.mark.parametrize("L", [1, 2, 3, 5, 8, 13])
def test_forward_tiny_prefills(L):
    """Whole calls of a few tokens (B = 2, budget 2): rows before the first
    complete block have no candidate and attend their own tokens only; rows
    with fewer complete blocks than the budget take them all.  Every row vs
    the oracle."""
    B, budget = 2, 2
    w = synth.Workload("t", "prefill", B, L, budget, 0, "random", 40 + L)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=16, budget_blocks=budget)
    out, bidx, _ = _forward(h, xd, B, L)
    _check_forward(x, f32(out), bidx.cpu().numpy(), O.Params(budget=budget), range(L), seqs=(0, 1))


def test_forward_chunks_of_one_block_equal_one_shot():
    """Chunks of 4 tokens (one micro-block each; every chunk but the first
    attends only cached blocks plus its own) are bit-identical to one shot."""
    B, L, budget = 2, 96, 8
    w = synth.Workload("t", "prefill", B, L, budget, 2, "random", 47)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=96, budget_blocks=budget)
    o1, b1, _ = _forward(h, xd, B, L)
    o2, b2, _ = _forward(h, xd, B, L, chunks=[(s, s + 4) for s in range(0, L, 4)])
    assert torch.equal(b1, b2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    _check_forward(x, f32(o2), b2.cpu().numpy(), O.Params(budget=budget), [0, 3, 4, 35, 36, 95], seqs=(0, 1))


def test_empty_calls_touch_nothing():
    """L = 0 is a no-op that succeeds: caches and outputs keep their bytes."""
    B = 2
    h = Q.Handle(max_ctx=64, budget_blocks=4)
    c = Q.alloc_caches(h, B)
    for t in c.values():
        t.view(torch.int16).fill_(0x1234)
    before = {k: v.clone() for k, v in c.items()}
    e = lambda *s, dt=torch.bfloat16: torch.empty(s, dtype=dt, device=DEV)
    q, kv, qi, ki = e(B, 0, 24, 256), e(B, 0, 2, 256), e(B, 0, 4, 128), e(B, 0, 128)
    out, bidx = e(B, 0, 24, 256), e(B, 0, 4, dt=torch.int32)
    ws = Q.workspace(h, Q.QSA_OP_FORWARD, B, 0, 16)
    Q.qsa_forward(h, B, 0, 16, q, kv, kv, qi, ki, c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], out, bidx,
                  ws)
    Q.qsa_append(h, B, 0, 16, kv, kv, ki, c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    Q.qsa_attend(h, B, 0, 16, q, c["k_cache"], c["v_cache"], bidx, out)
    Q.qsa_index_select(h, B, 0, 16, qi, c["kbar_cache"], bidx, Q.workspace(h, Q.QSA_OP_INDEX_SELECT, B, 0, 16))
    torch.cuda.synchronize()
    for k in c:
        assert torch.equal(c[k], before[k]), k


def _poison(caches, ws, on):
    """Fill the caches and the workspace: zeros, or bit patterns no valid slot
    holds (NaN in K~, -NaN in V, +Inf in k̄ and the pending keys, 0xFF bytes in
    the workspace)."""
    pats = {"k_cache": 0x7FC0, "v_cache": -64, "kbar_cache": 0x7F80, "kpend": 0x7F80}   # -64 = 0xFFC0
    for name, t in caches.items():
        t.view(torch.int16).fill_(pats[name] if on else 0)
    ws.fill_(0xFF if on else 0)


def test_poisoned_caches_and_workspace_leave_results_unchanged():
    """Cache slots the call does not write (past each sequence's length, the
    partial own block, k̄ of incomplete blocks) and every workspace byte are
    filled with NaN / Inf / 0xFF patterns before qsa_forward (two chunks) and
    qsa_decode (ragged lengths): outputs and selections are bitwise those of
    zero-filled buffers, and finite."""
    budget = 32
    B, L = 2, 1001
    w = synth.Workload("t", "prefill", B, L, budget, 4, "random", 47)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=2048, budget_blocks=budget)
    res = {}
    for on in (False, True):
        c = Q.alloc_caches(h, B)
        out = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
        bidx = torch.empty((B, L, budget), dtype=torch.int32, device=DEV)
        ws = Q.workspace(h, Q.QSA_OP_FORWARD, B, 512, 0)
        _poison(c, ws, on)
        for s0, s1 in ((0, 512), (512, L)):
            ws.fill_(0xFF if on else 0)
            sl = lambda t: t[:, s0:s1].contiguous()
            o = torch.empty((B, s1 - s0, 24, 256), dtype=torch.bfloat16, device=DEV)
            bi = torch.empty((B, s1 - s0, budget), dtype=torch.int32, device=DEV)
            Q.qsa_forward(h, B, s1 - s0, s0, sl(xd["q"]), sl(xd["k"]), sl(xd["v"]), sl(xd["q_idx"]),
                          sl(xd["k_idx"]), c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], o, bi, ws)
            out[:, s0:s1] = o
            bidx[:, s0:s1] = bi
        torch.cuda.synchronize()
        res[on] = (out, bidx)
    assert torch.equal(res[False][1], res[True][1])
    assert torch.equal(res[False][0].view(torch.int16), res[True][0].view(torch.int16))
    assert torch.isfinite(res[True][0].float()).all()

    lens = [1500, 3, 0, 701, 1202, 255]
    wd = synth.Workload("t", "decode", len(lens), max(lens), budget, 4, "random", 48)
    xdc = _to(synth.decode_inputs(wd, "cpu", ctx=max(lens), batch=len(lens)))
    dres = {}
    for on in (False, True):
        c = Q.alloc_caches(h, len(lens))
        ws = Q.workspace(h, Q.QSA_OP_DECODE, len(lens), 1, max(lens))
        _poison(c, ws, on)
        for b, n in enumerate(lens):
            if n:
                sl = lambda t: t[b:b + 1, :n].contiguous()
                cs = {k: v[b:b + 1] for k, v in c.items()}
                Q.qsa_append(h, 1, n, 0, sl(xdc["k"]), sl(xdc["v"]), sl(xdc["k_idx"]), cs["k_cache"],
                             cs["v_cache"], cs["kbar_cache"], cs["kpend"])
        new = {n: torch.stack([xdc[n][b, lens[b]] for b in range(len(lens))])[:, None].contiguous()
               for n in ("k", "v", "k_idx")}
        cache_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
        out = torch.empty((len(lens), 1, 24, 256), dtype=torch.bfloat16, device=DEV)
        bidx = torch.empty((len(lens), 1, budget), dtype=torch.int32, device=DEV)
        Q.qsa_decode(h, len(lens), cache_len, max(lens), xdc["q"], new["k"], new["v"], xdc["q_idx"], new["k_idx"],
                     c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], out, bidx, ws)
        torch.cuda.synchronize()
        dres[on] = (out, bidx)
    assert torch.equal(dres[False][1], dres[True][1])
    assert torch.equal(dres[False][0].view(torch.int16), dres[True][0].view(torch.int16))
    assert torch.isfinite(dres[True][0].float()).all()


def test_forward_long_equals_staged_calls():
    """A 140,000-row prefill with B = 2 (the attention in 2,048-row launches,
    the last one ragged; index + select in launches of 131,072 rows, the
    16 GiB of candidate lists they may hold, then 8,928), in one qsa_forward
    call and as two chunks (65,536 rows, then 74,464 at q_offset 65,536), is
    bit-identical to qsa_append + qsa_index_select + qsa_attend over all rows,
    and sampled rows match the oracle."""
    B, L, budget = 2, 140000, 64
    w = synth.Workload("t", "prefill", B, L, budget, 8, "random", 48)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=L, budget_blocks=budget)
    c = Q.alloc_caches(h, B)
    o2 = torch.empty((B, L, 24, 256), dtype=torch.bfloat16, device=DEV)
    b2 = torch.empty((B, L, budget), dtype=torch.int32, device=DEV)
    Q.qsa_append(h, B, L, 0, xd["k"], xd["v"], xd["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    Q.qsa_index_select(h, B, L, 0, xd["q_idx"], c["kbar_cache"], b2, Q.workspace(h, Q.QSA_OP_INDEX_SELECT, B, L, 0))
    Q.qsa_attend(h, B, L, 0, xd["q"], c["k_cache"], c["v_cache"], b2, o2)
    torch.cuda.synchronize()
    del c
    for chunks in (None, [(0, 65536), (65536, L)]):
        o1, b1, _ = _forward(h, xd, B, L, chunks=chunks)
        assert torch.equal(b1, b2), chunks
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), chunks
        del o1, b1
    rows = [0, 8191, 8192, 32767, 32768, 65535, 65536, 131071, 131072, 131073, 137215, 137216, 139999]
    _check_forward(x, f32(o2), b2.cpu().numpy(), O.Params(budget=budget), rows, seqs=(0, 1))


def test_forward_attention_launch_boundaries_and_lone_rows():
    """The prefill attention takes two neighbouring rows per wave in launches
    of 2,048 rows: rows on both sides of each launch boundary, a last launch of
    three rows (the pair 4,096-4,097, then row 4,098 alone), and, as chunks of
    2,052 and 2,047 rows (the second an odd count at q_offset 2,052, whose last
    row is alone in its wave), bitwise the one-shot result; rows against the
    oracle."""
    B, L, budget = 2, 4099, 64
    w = synth.Workload("t", "prefill", B, L, budget, 8, "random", 52)
    x, xd = _prefill(w)
    h = Q.Handle(max_ctx=4100, budget_blocks=budget)       # a whole number of blocks
    o1, b1, _ = _forward(h, xd, B, L)
    o2, b2, _ = _forward(h, xd, B, L, chunks=[(0, 2052), (2052, L)])
    assert torch.equal(b1, b2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    rows = [0, 1, 2, 2045, 2046, 2047, 2048, 2049, 2050, 2051, 2052, 2053, 4094, 4095, 4096, 4097, 4098]
    _check_forward(x, f32(o1), b1.cpu().numpy(), O.Params(budget=budget), rows, seqs=(0, 1))
