"""Pins of the CPU oracle against facts it does not compute itself.

Every test here runs on the CPU.  Each pin is chosen so that a plausible slip in
the oracle (a dropped term, a wrong sign or pairing, a wrong pooling position, a
transposed operand, an off-by-one in the causal boundary) fails at least one:

* constants: the values the pages print (tests/golden/qsa_spec.json);
* bf16 rounding: hand-worked bit patterns and torch's own cast;
* rotary tables and rotation: complex exponentials (numpy), norm preservation,
  identity at position 0, relative-position invariance, YaRN bands derived by
  hand from the YaRN paper;
* pooled scoring: the per-token identity (mean of logits of tokens rotated at
  the block start), computed in fp64 through complex arithmetic;
* selection: brute-force subset enumeration on tiny inputs;
* attention: torch's scaled_dot_product_attention in fp64 (dense when the
  budget covers every block; with an explicit mask built from the selection);
* needles: planted blocks are always selected by their probes;
* causality: a row never depends on keys after its position.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bits(t):
    return synth.bf16_bits(t)


# ---------------------------------------------------------------- constants
def test_spec_constants_match_pages():
    g = _gold("qsa_spec.json")
    p = O.Params()
    assert p.n_q_heads == g["n_q_heads"]["value"]
    assert p.n_kv_heads == g["n_kv_heads"]["value"]
    assert p.head_dim == g["head_dim"]["value"]
    assert p.rope_dim == g["rope_dim"]["value"]
    assert p.rope_dim == int(g["partial_rotary_factor"]["value"] * p.head_dim)
    assert p.rope_dim // 2 == sum(g["mrope_section"]["value"])
    assert p.n_idx_heads == g["n_idx_heads"]["value"]
    assert p.idx_dim == g["idx_dim"]["value"]
    assert p.block == g["block"]["value"]
    assert p.budget == g["budget"]["value"] == g["budget_tokens"]["value"] // p.block
    assert p.rope_theta == g["rope_theta"]["value"]
    assert p.yarn_orig_ctx == g["yarn_orig_ctx"]["value"]


# ---------------------------------------------------------------- bf16
def test_bf16_rne_hand_cases():
    for c in _gold("bf16_rne.json")["cases"]:
        x = np.array([int(c["f32_hex"], 16)], dtype=np.uint32).view(np.float32)
        got = int(O.f32_to_bf16_bits(x)[0])
        assert got == int(c["bf16_hex"], 16), c["note"]


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 200000),
                        (rng.integers(0, 2 ** 16, 100000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), ref)


# ---------------------------------------------------------------- rotary
def test_inv_freq_closed_form():
    p = O.Params()
    w = O.inv_freq(p)
    assert w.shape == (32,)
    assert w[0] == 1.0
    j = np.arange(32)
    np.testing.assert_allclose(w, 10.0 ** (-7.0 * j / 32.0), rtol=1e-14)
    # a plain context (factor 1) ignores the YaRN fields
    assert np.array_equal(O.inv_freq(O.Params(yarn_factor=1.0, yarn_orig_ctx=123)), w)


def test_yarn_bands_from_hand_derivation():
    g = _gold("yarn_bands.json")
    base = O.inv_freq(O.Params())
    y = O.inv_freq(O.Params(yarn_factor=4.0))
    for j in g["extrapolated_pairs"]:
        assert y[j] == base[j]
    for j in g["interpolated_pairs"]:
        assert y[j] == base[j] / 4.0
    ramp = np.array(g["ramp_pairs"])
    frac = (y[ramp] - base[ramp] / 4) / (base[ramp] - base[ramp] / 4)   # = gamma_j in (0,1)
    assert np.all((frac > 0) & (frac < 1))
    assert np.all(np.diff(frac) < 0), "gamma must fall as the wavelength grows"
    r15 = 262144 * base[15] / (2 * math.pi)
    assert abs(r15 - g["r_15"]["value"]) < g["r_15"]["tol"]
    np.testing.assert_allclose(frac[0], (r15 - 1) / 31, rtol=1e-12)
    t = g["attention_temperature_factor"]
    assert abs(O.softmax_scale(O.Params(yarn_factor=4.0)) * 16 - t["value"]) < t["tol"]
    assert O.softmax_scale(O.Params()) == 1.0 / 16


def test_rope_table_is_libm_cos_sin():
    p = O.Params(yarn_factor=4.0)
    pos = np.array([0, 1, 2, 3, 1000, 262143, 1048575], dtype=np.int64)
    c, s = O.rope_table(pos, p)
    w = O.inv_freq(p)
    for i, q in enumerate(pos):
        for j in range(32):
            a = float(q) * float(w[j])
            assert c[i, j] == np.float32(math.cos(a)) and s[i, j] == np.float32(math.sin(a))
    # and against complex exponentials (numpy) to within an fp32 rounding
    pos = np.arange(0, 300000, 7, dtype=np.int64)
    c, s = O.rope_table(pos, O.Params())
    e = np.exp(1j * pos[:, None].astype(np.float64) * O.inv_freq(O.Params())[None, :])
    np.testing.assert_allclose(c, e.real, atol=6e-8, rtol=0)
    np.testing.assert_allclose(s, e.imag, atol=6e-8, rtol=0)


def _rot_complex(x64, pos, w, n=32):
    """Reference rotation through complex multiplication, fp64."""
    z = (x64[..., :n] + 1j * x64[..., n:2 * n]) * np.exp(1j * pos * w)
    out = x64.copy()
    out[..., :n] = z.real
    out[..., n:2 * n] = z.imag
    return out


def test_rotate_is_complex_multiplication():
    rng = np.random.default_rng(1)
    p = O.Params()
    w = O.inv_freq(p)
    for pos in [0, 1, 5, 4096, 262143]:
        x = rng.standard_normal((3, 256)).astype(np.float32)
        c, s = O.rope_table(np.array([pos]), p)
        r = O.rotate(x, c, s)
        ref = _rot_complex(x.astype(np.float64), pos, w)
        np.testing.assert_allclose(r, ref, atol=2e-6, rtol=0)
        assert np.array_equal(r[:, 64:], x[:, 64:])
        if pos == 0:
            assert np.array_equal(r, x)


def test_rotation_relative_position_and_norm():
    rng = np.random.default_rng(2)
    p = O.Params()
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)

    def dot(pq, pk):
        cq, sq = O.rope_table(np.array([pq]), p)
        ck, sk = O.rope_table(np.array([pk]), p)
        rq = O.rotate(q[None], cq, sq)[0].astype(np.float64)
        rk = O.rotate(k[None], ck, sk)[0].astype(np.float64)
        return rq @ rk, np.linalg.norm(rq)

    d0, n0 = dot(100, 37)
    for shift in [1, 1000, 50000]:
        d1, n1 = dot(100 + shift, 37 + shift)
        assert abs(d0 - d1) < 1e-3
        assert abs(n1 - np.linalg.norm(q)) < 1e-4


# ---------------------------------------------------------------- pooled scoring
def test_pooled_score_equals_mean_of_token_logits():
    """Compression before RoPE: the score against k̄_b equals, per head, the mean
    of the logits of the block's raw keys each rotated at the block start 4b,
    then ReLU and a sum over heads (fp64 complex arithmetic, no bf16 rounding)."""
    rng = np.random.default_rng(3)
    p = O.Params()
    w = O.inv_freq(p)
    n_tok = 64
    kraw = rng.standard_normal((n_tok, 128)).astype(np.float32)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    pos_q = 61
    pooled = O.pool_block_keys(kraw, 4)
    c, s = O.rope_table(np.arange(pooled.shape[0]) * 4, p)
    kbar = O.rotate(pooled, c, s)                      # fp32, unrounded
    cq, sq = O.rope_table(np.array([pos_q]), p)
    qt = O.rotate(q, cq, sq)
    got = O.block_scores(qt, kbar)
    qt64 = _rot_complex(q.astype(np.float64), pos_q, w)
    for b in range(pooled.shape[0]):
        toks = _rot_complex(kraw[4 * b:4 * b + 4].astype(np.float64), 4 * b, w)   # all at 4b
        logit = (qt64 @ toks.T).mean(axis=1)                                        # [4 heads]
        ref = np.sum((np.abs(logit) + logit) / 2)
        assert abs(got[b] - ref) < 2e-4 * max(1.0, abs(ref))
        # rotating each token at its own position instead gives a different score
    wrong = _rot_complex(kraw[4:8].astype(np.float64), np.arange(4, 8)[:, None], w)
    assert abs(((qt64 @ wrong.T).mean(axis=1)).sum() - (qt64 @ _rot_complex(
        kraw[4:8].astype(np.float64), 4, w).T).mean(axis=1).sum()) > 1e-3


def _bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significand bits), floored at 2^-16."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -8)))
    return 2.0 ** (e - 7)


def _kbar_reference(kraw_bits, key_pos, w):
    """Independent fp64 pooled key: the fp32 token-order mean of each complete
    block's four raw bf16 keys (written out here, not the oracle's pooling),
    rotated through complex multiplication at key_pos(b)."""
    raw = (kraw_bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    nb = raw.shape[0] // 4
    acc = raw[0:4 * nb:4].copy()
    for t in (1, 2, 3):
        acc = np.float32(acc + raw[t:4 * nb:4])
    mean = np.float32(acc * np.float32(0.25)).astype(np.float64)
    pos = key_pos(np.arange(nb))[:, None].astype(np.float64)
    return _rot_complex(mean, pos, w[None, :])


def _within_one_ulp(got, ref):
    return bool(np.all(np.abs(got.astype(np.float64) - ref) <= _bf16_ulp(ref)))


@pytest.mark.parametrize("yarn", [1.0, 4.0])
def test_indexer_keys_pooled_then_rotated_at_block_start(yarn):
    """oracle.indexer_keys itself: every k̄[b] is within one bf16 ulp of the
    fp64 rotation, at the block-start position 4b, of the fp32 token-order mean
    of the block's four raw keys ([PKR] "QSA: ...": compression before the
    positional encoding, one block-start position per pooled key).  A ragged
    tail of 3 tokens yields no key.  The same check fails for the plausible
    slips: rotating at b, at the block's last token 4b+3, or not at all."""
    rng = np.random.default_rng(21)
    p = O.Params(yarn_factor=yarn)
    if yarn == 1.0:   # closed form, independent of the oracle's frequency code
        w = np.array([p.rope_theta ** (-2.0 * j / 64.0) for j in range(32)])
    else:             # the YaRN frequencies are pinned by their hand-derived bands
        w = O.inv_freq(p)
    n_blocks = 700
    kb = O.f32_to_bf16_bits(rng.standard_normal((4 * n_blocks + 3, 128)).astype(np.float32))
    got = O.indexer_keys(kb, p)
    assert got.shape == (n_blocks, 128)
    assert np.array_equal(O.bf16_round(got), got)          # bf16 values
    assert _within_one_ulp(got, _kbar_reference(kb, lambda b: 4 * b, w))
    # non-rotary dims are the plain mean, rounded once
    assert _within_one_ulp(got[:, 64:], _kbar_reference(kb, lambda b: 4 * b, w)[:, 64:])
    for wrong in (lambda b: b, lambda b: 4 * b + 3, lambda b: 0 * b):
        assert not _within_one_ulp(got, _kbar_reference(kb, wrong, w))


def test_token_level_indexer_brute_force():
    """r = 1: every key rotated at its own position (fp64 complex arithmetic on
    the bf16 inputs), logits against the query rotated at p, ReLU, sum over
    heads, candidates t < p only; the selection is the brute-force top-k of
    those scores up to near-ties (bf16 rounding of the rotated operands)."""
    rng = np.random.default_rng(11)
    p = O.Params(budget=5)
    w = O.inv_freq(p)
    n_tok = 40
    kb = O.f32_to_bf16_bits(rng.standard_normal((n_tok, 128)).astype(np.float32))
    qb = O.f32_to_bf16_bits(rng.standard_normal((n_tok, 4, 128)).astype(np.float32))
    pos = [0, 1, 4, 5, 17, 39]
    sel, scs = O.token_index_rows(qb[pos], kb, pos, p)
    kf = O.bf16_bits_to_f32(kb).astype(np.float64)
    for i, pq in enumerate(pos):
        assert scs[i].shape == (pq,)
        qt = _rot_complex(O.bf16_bits_to_f32(qb[pq]).astype(np.float64), pq, w)
        ref = np.zeros(pq)
        for t in range(pq):
            kt = _rot_complex(kf[t:t + 1], t, w)[0]
            ref[t] = sum(max(0.0, float(qt[h] @ kt)) for h in range(4))
        np.testing.assert_allclose(scs[i], ref, rtol=2e-2, atol=0.1)
        n = min(p.budget, pq)
        assert np.all(sel[i, n:] == -1) and np.all(np.diff(sel[i, :n]) > 0)
        order = sorted(range(pq), key=lambda t: (-ref[t], -t))[:n]
        kth = sorted(ref, reverse=True)[n - 1] if n else 0.0
        for t in set(order) ^ set(sel[i, :n].tolist()):
            assert abs(ref[t] - kth) < 0.5, (pq, t)


def test_pooling_is_token_order_fp32_mean():
    x = np.array([[1.0], [2.0 ** -24], [2.0 ** -24], [-1.0]], dtype=np.float32)
    # ((1 + 2^-24) + 2^-24) - 1 in fp32: each 2^-24 is lost against 1 (ties to even)
    assert O.pool_block_keys(x, 4)[0, 0] == 0.0
    x = np.arange(16, dtype=np.float32).reshape(8, 2)
    np.testing.assert_array_equal(O.pool_block_keys(x, 4), [[3.0, 4.0], [11.0, 12.0]])
    assert O.pool_block_keys(np.ones((7, 3), np.float32), 4).shape == (1, 3)


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("seed", range(40))
def test_select_brute_force(seed):
    rng = np.random.default_rng(seed)
    o = int(rng.integers(0, 9))
    budget = int(rng.integers(1, 4))
    scores = rng.integers(0, 4, o).astype(np.float64)       # many exact ties
    sel = O.select_blocks(scores, budget)
    k = min(budget, o)
    chosen = sel[sel >= 0]
    assert len(chosen) == k and np.all(sel[k:] == -1)
    assert np.all(np.diff(chosen) > 0)
    best = max((sum(scores[list(c)]) for c in itertools.combinations(range(o), k)), default=0.0)
    assert sum(scores[chosen]) == best
    # the tie rule: every chosen block precedes every other under (score desc, block desc)
    rest = [b for b in range(o) if b not in set(chosen.tolist())]
    for a in chosen:
        for b in rest:
            assert (scores[a], a) > (scores[b], b)


def test_select_fewer_candidates_than_budget_takes_all():
    sel = O.select_blocks(np.zeros(5), 8)
    assert sel.tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert O.select_blocks(np.zeros(0), 3).tolist() == [-1, -1, -1]


def test_token_set_own_block_tail():
    p = O.Params()
    assert O.token_set(np.array([-1, -1]), 2, p).tolist() == [0, 1, 2]
    assert O.token_set(np.array([0, -1]), 7, p).tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    assert O.token_set(np.array([1, 3]), 17, p).tolist() == [4, 5, 6, 7, 12, 13, 14, 15, 16, 17]


def test_token_set_reused_widens_the_own_block_tail():
    p = O.Params()
    sel = np.array([1, 3, 5, -1])
    # reuse at the selecting position itself is the plain rule (candidates of
    # position 21..23 are blocks 0..4)
    for pos in (21, 22, 23):
        assert O.token_set_reused(sel, pos, pos, p).tolist() == O.token_set(sel[sel < 5], pos, p).tolist()
    # selection made at 21 (own block 5): block 5 is no longer a selected block
    # but part of the tail, which now runs from token 20 to the query
    assert O.token_set_reused(sel, 21, 26, p).tolist() == [4, 5, 6, 7, 12, 13, 14, 15] + list(range(20, 27))
    # blocks at or after the selecting position's own block are never read from the list
    assert O.token_set_reused(np.array([6, 7]), 21, 30, p).tolist() == list(range(20, 31))


# ---------------------------------------------------------------- attention
def _small(L, budget, seed=0, needles=0):
    w = synth.Workload("t", "prefill", 1, L, budget, needles, "random", seed)
    x = synth.prefill_inputs(w)
    return w, x


def _sdpa_rows(x, p, mask_fn):
    """Causal GQA attention via torch SDPA (fp64) on the oracle's rotated operands."""
    L = x["q"].shape[1]
    pos = np.arange(L)
    qt = O.core_rotate(_bits(x["q"][0]), pos, p).astype(np.float64)      # [L][24][256]
    kt = O.core_rotate(_bits(x["k"][0]), pos, p).astype(np.float64)      # [L][2][256]
    v = O.bf16_bits_to_f32(_bits(x["v"][0])).astype(np.float64)
    q_t = torch.from_numpy(qt).permute(1, 0, 2)                          # [24][L][256]
    k_t = torch.from_numpy(kt).permute(1, 0, 2).repeat_interleave(12, 0).contiguous()
    v_t = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(12, 0).contiguous()
    mask = torch.from_numpy(mask_fn(L))
    out = torch.nn.functional.scaled_dot_product_attention(q_t[None], k_t[None], v_t[None],
                                                           attn_mask=mask[None, None], scale=1.0 / 16)
    return out[0].permute(1, 0, 2).numpy()                               # [L][24][256]


def test_dense_equivalence_when_budget_covers_everything():
    L = 96
    w, x = _small(L, budget=64, seed=5)
    p = O.Params(budget=64)
    assert (L - 1) // 4 <= p.budget
    rows = np.arange(L)
    out, sel, _ = O.prefill_rows(_bits(x["q"][0]), _bits(x["k"][0]), _bits(x["v"][0]),
                                 _bits(x["q_idx"][0]), _bits(x["k_idx"][0]), rows, p)
    ref = _sdpa_rows(x, p, lambda n: np.tril(np.ones((n, n), dtype=bool)))
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=1e-10)


def test_reused_selection_dense_and_masked_equivalence():
    """A query reusing an earlier query's selection equals SDPA over exactly
    the reused blocks and the widened tail; with a budget covering every block
    before the selecting position it is dense causal attention."""
    L = 120
    w, x = _small(L, budget=40, seed=8)
    for budget in (40, 3):
        p = O.Params(budget=budget)
        lay = O.LayerOracle(_bits(x["k"][0]), _bits(x["v"][0]), _bits(x["k_idx"][0]), p)
        pairs = [(101, 101), (101, 103), (101, 107), (99, 116), (3, 9)]
        sels = {sp: lay.row(sp, _bits(x["q"][0, sp]), _bits(x["q_idx"][0, sp]))[1] for sp, _ in pairs}

        def mask_fn(n):
            m = np.zeros((n, n), dtype=bool)
            for sp, pos in pairs:
                for b in sels[sp]:
                    if 0 <= b < sp // 4:
                        m[pos, 4 * b:4 * b + 4] = True
                m[pos, 4 * (sp // 4):pos + 1] = True
            return m

        ref = _sdpa_rows(x, p, mask_fn)
        for sp, pos in pairs:
            out = lay.row_reused(pos, _bits(x["q"][0, pos]), sels[sp], sp)
            np.testing.assert_allclose(out, ref[pos], atol=1e-12, rtol=1e-10)
            if budget >= sp // 4:
                dense = _sdpa_rows(x, p, lambda n: np.tril(np.ones((n, n), dtype=bool)))
                np.testing.assert_allclose(out, dense[pos], atol=1e-12, rtol=1e-10)


def test_masked_equivalence_small_budget():
    L = 160
    w, x = _small(L, budget=3, seed=6)
    p = O.Params(budget=3)
    rows = np.arange(L)
    out, sel, _ = O.prefill_rows(_bits(x["q"][0]), _bits(x["k"][0]), _bits(x["v"][0]),
                                 _bits(x["q_idx"][0]), _bits(x["k_idx"][0]), rows, p)

    def mask_fn(n):
        m = np.zeros((n, n), dtype=bool)
        for i in range(n):
            for b in sel[i]:
                if b >= 0:
                    assert b < i // 4
                    m[i, 4 * b:4 * b + 4] = True
            m[i, 4 * (i // 4):i + 1] = True
        return m

    ref = _sdpa_rows(x, p, mask_fn)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=1e-10)
    # softmax rows are convex combinations of V
    v = O.bf16_bits_to_f32(_bits(x["v"][0]))
    assert np.all(out[:, :12] <= v[:, 0].max(0) + 1e-12) and np.all(out[:, :12] >= v[:, 0].min(0) - 1e-12)


# ---------------------------------------------------------------- needles
def test_planted_needles_always_selected():
    w = synth.Workload("t", "prefill", 1, 2048, 64, 8, "random", 11)
    x = synth.prefill_inputs(w)
    p = O.Params(budget=64)
    plan = x["needles"][0]
    rows = np.concatenate(plan.probes)
    _, sel, scores = O.prefill_rows(_bits(x["q"][0]), _bits(x["k"][0]), _bits(x["v"][0]),
                                    _bits(x["q_idx"][0]), _bits(x["k_idx"][0]), rows, p)
    i = 0
    checked = 0
    for n, b in enumerate(plan.blocks):
        for _ in plan.probes[n]:
            assert b in sel[i]
            sc = scores[i]
            if sc.shape[0] > p.budget:
                kth = np.sort(np.delete(sc, b))[::-1][p.budget - 1]
                assert sc[b] >= 2 * kth
                checked += 1
            i += 1
    assert checked >= 40


def test_needles_decode_probe():
    w = synth.Workload("t", "decode", 2, 4096, 64, 16, "random", 12)
    x = synth.decode_inputs(w)
    p = O.Params(budget=64)
    for s in range(2):
        lay = O.LayerOracle(_bits(x["k"][s]), _bits(x["v"][s]), _bits(x["k_idx"][s]), p)
        _, sel, sc = lay.row(4096, _bits(x["q"][s, 0]), _bits(x["q_idx"][s, 0]))
        for b in x["needles"][s].blocks:
            assert b in sel


# ---------------------------------------------------------------- causality
def test_rows_never_read_future_keys():
    L = 200
    w, x = _small(L, budget=5, seed=7)
    p = O.Params(budget=5)
    q, k, v, qi, ki = (_bits(x[n][0]) for n in ("q", "k", "v", "q_idx", "k_idx"))
    full = O.LayerOracle(k, v, ki, p)
    for pos in [0, 3, 4, 7, 8, 99, 150, 199]:
        trunc = O.LayerOracle(k[:pos + 1], v[:pos + 1], ki[:pos + 1], p)
        a = full.row(pos, q[pos], qi[pos])
        b = trunc.row(pos, q[pos], qi[pos])
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert a[2].shape == (pos // 4,)


def test_yarn_changes_only_long_wavelengths():
    L = 64
    w, x = _small(L, budget=64, seed=8)
    pa = O.Params(budget=64)
    pb = O.Params(budget=64, yarn_factor=4.0)
    ka = O.indexer_keys(_bits(x["k_idx"][0]), pa)
    kb = O.indexer_keys(_bits(x["k_idx"][0]), pb)
    # pairs 0..14 keep their frequency, so dims j and j+32 of those pairs agree
    keep = list(range(15)) + list(range(32, 47)) + list(range(64, 128))
    assert np.array_equal(ka[:, keep], kb[:, keep])
    assert not np.array_equal(ka, kb)
