"""Parity of the Gated DeltaNet chunked prefill (HIP) with the token-by-token
oracle (oracle/gdn.py), through the C ABI.

Tolerance.  The kernels round to bf16 every matrix-core operand that is not
an input: the chunk matrices Tb and P, the state S each time it multiplies
K and Q, and the intermediates X = V - diag(gamma) K S and U.  Each rounding
is a relative perturbation of at most 2^-9 of one operand of one product, and
the products are sums of terms no larger than the output's own scale, so
|o - o_ref| stays within a few times 2^-8 of the scale of o (the state's
columns decay and are rewritten, so earlier roundings do not pile up).  The
bound used is 8 * 2^-8 * max(|o_ref| over the head) per element, and the
same for the final state against its own scale.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_qsa_amd as Q
import synth
from oracle import gdn as OG

pytestmark = pytest.mark.gpu

TOL = 8 * 2.0 ** -8


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gdn(x, scale, with_final=True, max_len=None):
    cu = x["cu_seqlens"]
    lens = x["lens"]
    nseq = len(lens)
    hv = x["v"].shape[1]
    max_len = max(lens) if max_len is None else max_len
    o = torch.empty_like(x["v"])
    fs = torch.empty(nseq, hv, 128, 128, device="cuda") if with_final else None
    ws = torch.empty(max(Q.qsa_gdn_workspace_size(nseq, max_len, x["q"].shape[1], hv), 16), dtype=torch.uint8, device="cuda")
    Q.qsa_gdn_chunk_prefill(nseq, cu, max_len, x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["s0"], o, fs, ws)
    torch.cuda.synchronize()
    return o, fs


def oracle_seq(x, s, scale):
    a, b = int(x["cu_seqlens"][s]), int(x["cu_seqlens"][s + 1])
    s0 = None if x["s0"] is None else _np(x["s0"][s])
    return OG.gdn_recurrent(_np(x["q"][a:b]), _np(x["k"][a:b]), _np(x["v"][a:b]), _np(x["g"][a:b]),
                            _np(x["beta"][a:b]), scale, s0)


def check(got, ref, where):
    scale = max(np.abs(ref).max(), 1e-6)
    err = np.abs(got - ref).max()
    print("%s: max|err| %.3e  scale %.3e  ratio %.4f" % (where, err, scale, err / scale), flush=True)
    assert err <= TOL * scale, where


@pytest.mark.parametrize("lens,hq,hv,init", [
    ([1, 64, 200, 129], 2, 6, True),     # one token, one exact chunk, ragged tails
    ([300], 16, 48, False),              # the pages' head counts
    ([65, 3, 192], 4, 4, True),          # one V head per QK head
])
def test_gdn_matches_oracle(lens, hq, hv, init):
    x = synth.gdn_inputs(5, lens, hq, hv, "cuda", init_state=init)
    scale = 128 ** -0.5
    print("gdn lens=%s hq=%d hv=%d init=%s" % (lens, hq, hv, init), flush=True)
    o, fs = run_gdn(x, scale)
    for s in range(len(lens)):
        ro, rs = oracle_seq(x, s, scale)
        a, b = int(x["cu_seqlens"][s]), int(x["cu_seqlens"][s + 1])
        for h in range(hv):
            check(_np(o[a:b, h]), ro[:, h], "seq %d head %d out" % (s, h))
            check(_np(fs[s, h]), rs[h], "seq %d head %d state" % (s, h))


def test_gdn_state_chaining():
    """Prefill of [0, T) equals prefill of [0, T1) then [T1, T) from its final state."""
    T, T1 = 333, 137
    x = synth.gdn_inputs(6, [T], 2, 6, "cuda", init_state=True)
    scale = 128 ** -0.5
    o_all, s_all = run_gdn(x, scale)
    first = {key: (val[:T1] if key in ("q", "k", "v", "g", "beta") else val) for key, val in x.items()}
    first["lens"] = [T1]
    first["cu_seqlens"] = torch.tensor([0, T1], dtype=torch.int32, device="cuda")
    o1, s1 = run_gdn(first, scale)
    second = {key: (val[T1:].contiguous() if key in ("q", "k", "v", "g", "beta") else val) for key, val in x.items()}
    second["lens"] = [T - T1]
    second["cu_seqlens"] = torch.tensor([0, T - T1], dtype=torch.int32, device="cuda")
    second["s0"] = s1
    o2, s2 = run_gdn(second, scale)
    ro, rs = oracle_seq(x, 0, scale)
    for h in range(6):
        check(_np(torch.cat([o1, o2])[:, h]), ro[:, h], "chained head %d out" % h)
        check(_np(s2[0, h]), rs[h], "chained head %d state" % h)
        check(_np(o_all[:, h]), ro[:, h], "whole head %d out" % h)


def test_gdn_empty_sequences_keep_their_state():
    x = synth.gdn_inputs(7, [0, 70, 0], 2, 6, "cuda", init_state=True)
    o, fs = run_gdn(x, 0.1)
    assert torch.equal(fs[0], x["s0"][0]) and torch.equal(fs[2], x["s0"][2])
    ro, rs = oracle_seq(x, 1, 0.1)
    for h in range(6):
        check(_np(o[:, h]), ro[:, h], "head %d out" % h)
        check(_np(fs[1, h]), rs[h], "head %d state" % h)


def test_gdn_no_initial_state_and_no_final_state():
    x = synth.gdn_inputs(8, [97], 2, 2, "cuda", init_state=False)
    o, _ = run_gdn(x, 0.2, with_final=False)
    ro, _ = oracle_seq(x, 0, 0.2)
    for h in range(2):
        check(_np(o[:, h]), ro[:, h], "head %d out" % h)


def _bench_config_run(lens):
    """The bench's launch configuration: qsa_gdn_prep then qsa_gdn_scan, 16 QK
    heads, 48 V heads, no initial state."""
    x = synth.gdn_inputs(21, lens, 16, 48, "cuda")
    nseq, max_len = len(lens), max(lens)
    o = torch.empty_like(x["v"])
    fs = torch.empty(nseq, 48, 128, 128, device="cuda")
    ws = torch.empty(Q.qsa_gdn_workspace_size(nseq, max_len, 16, 48), dtype=torch.uint8, device="cuda")
    scale = 128 ** -0.5
    Q.qsa_gdn_prep(nseq, x["cu_seqlens"], max_len, x["q"], x["k"], 48, x["g"], x["beta"], scale, ws)
    Q.qsa_gdn_scan(nseq, x["cu_seqlens"], max_len, x["q"], x["k"], x["v"], x["g"], scale, None, o, fs, ws)
    torch.cuda.synchronize()
    del ws
    return x, o, fs, scale


def _oracle_one_head(x, s, hv, scale, upto=None):
    a, b = int(x["cu_seqlens"][s]), int(x["cu_seqlens"][s + 1])
    b = b if upto is None else a + upto
    hq = hv // 3
    sl = lambda t, h: _np(t[a:b, h:h + 1])
    return OG.gdn_recurrent(sl(x["q"], hq), sl(x["k"], hq), sl(x["v"], hv), sl(x["g"], hv), sl(x["beta"], hv), scale)


def test_gdn_full_size_262144_bench_config():
    """One 262,144-token sequence: V head 47 (QK head 15) checked over every
    token and its final state; V head 0 over the first 4,096 tokens."""
    print("gdn full size: T=262144, hq=16, hv=48", flush=True)
    x, o, fs, scale = _bench_config_run([262144])
    ro, rs = _oracle_one_head(x, 0, 47, scale)
    check(_np(o[:, 47]), ro[:, 0], "head 47 out")
    check(_np(fs[0, 47]), rs[0], "head 47 state")
    ro, _ = _oracle_one_head(x, 0, 0, scale, upto=4096)
    check(_np(o[:4096, 0]), ro[:, 0], "head 0 out, first 4096 tokens")


def test_gdn_full_size_8x32768_bench_config():
    """Eight packed 32,768-token sequences: sequence 7, V head 23 over every
    token and its final state; sequence 0, V head 5 over its first 4,096."""
    print("gdn full size: 8 x 32768, hq=16, hv=48", flush=True)
    x, o, fs, scale = _bench_config_run([32768] * 8)
    ro, rs = _oracle_one_head(x, 7, 23, scale)
    a = 7 * 32768
    check(_np(o[a:a + 32768, 23]), ro[:, 0], "seq 7 head 23 out")
    check(_np(fs[7, 23]), rs[0], "seq 7 head 23 state")
    ro, _ = _oracle_one_head(x, 0, 5, scale, upto=4096)
    check(_np(o[:4096, 5]), ro[:, 0], "seq 0 head 5 out, first 4096 tokens")
