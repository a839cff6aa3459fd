#!/usr/bin/env python3
"""Benchmark of the MI355X QSA layer on one GPU.

One step = one pass of the whole hot path:
  * prefill of one 262,144-token sequence, budget 512 blocks (the stages
    qsa_append -> qsa_index_select -> qsa_attend, exactly the kernels
    qsa_forward launches), and
  * one decode step for 64 sequences with 131,072 cached tokens each.
Inputs are seeded synthetic tensors already resident in HBM when timing starts.

Printed: ONE JSON line.  `value` is prefill tokens/s at 262,144 tokens; decode
tokens/s sits beside it.  `roofline` covers the dominant kernel, the sparse
attention (attend_prefill_kernel), with its duration from HIP events recorded
on the stream the kernel runs on: its algorithmic FLOP/s against the bf16 MFMA
peak, and beside it the rate of its gathers against gather ceilings measured in
the same run (libqsa_probe.so) and its compulsory HBM bytes against the HBM
peak.  `cpu_baseline` times the CPU oracle on a bounded sample of the same
prefill rows (all threads and one thread), and `decode.cpu_baseline` on the
decode query of two of the 64 sequences (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_long_qsa_amd as Q  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16, TFLOP/s

# HBM-side bytes of the attention over the 262,144-token workload (128 launches
# of attend_prefill_kernel, 2,048 rows each), read by rocprofv3 --pmc
# (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000 KiB per launch, mean of the 384
# launches of three passes; the factors are what the counters read for a plain
# 1 GiB copy).  The counter summary is
# profiles/attend_prefill_kernel_L262144__hbm_counters.md.  The figure is
# reported only while the kernel's sources hash to these digests (sources whose
# attend_prefill_kernel compiles to the same instructions as the build the
# counters were taken with).
ATTEND_TRAFFIC_BYTES = (1809886.1 * 2.000 + 26109.4 * 1.000) * 1024 * 128
ATTEND_TRAFFIC_SOURCES = {
    "k_attend.hip": "bc30d8cfe032675f6ab2ee4a2c5b4ba106d1456b11c4725e88382c6761329cc4",
    "attend_parts.h": "25edb0e75d70d3aa067623febdd54d9bef69310f4a4340d74e159cf22e4f59a5",
    "qsa_common.h": "e68f00491eca878a52d16e3650d7ec7653f15dcb5c7fc4ff03e9c640f02d6a24",
}


def attend_traffic_bytes():
    """Counter-measured HBM-side bytes of the attention over the workload (all
    its launches), or None if the kernel changed since."""
    import hashlib
    for name, digest in ATTEND_TRAFFIC_SOURCES.items():
        with open(os.path.join(ROOT, "block_sparse_long_qsa_amd", "csrc", name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return ATTEND_TRAFFIC_BYTES


def _progress(msg):
    print(msg, file=sys.stderr, flush=True)


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def setup_prefill(w):
    x = synth.prefill_inputs(w, "cuda")
    L = w.seq_len
    h = Q.Handle(max_ctx=L, budget_blocks=w.budget, yarn_factor=w.yarn_factor)
    c = Q.alloc_caches(h, 1)
    ws = Q.workspace(h, Q.QSA_OP_FORWARD, 1, L, 0)      # also large enough for qsa_index_select
    bidx = torch.empty((1, L, w.budget), dtype=torch.int32, device="cuda")
    out = torch.empty((1, L, 24, 256), dtype=torch.bfloat16, device="cuda")
    return dict(x=x, h=h, c=c, ws=ws, bidx=bidx, out=out, L=L)


def prefill_forward(s, ev):
    """One prefill as the library runs it: qsa_forward (append, fused index +
    select, then the attention in launches of 4,096 rows)."""
    x, h, c, L = s["x"], s["h"], s["c"], s["L"]
    ev[0].record()
    Q.qsa_forward(h, 1, L, 0, x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], c["k_cache"], c["v_cache"],
                  c["kbar_cache"], c["kpend"], s["out"], s["bidx"], s["ws"])
    ev[1].record()


def prefill_stages(s, ev):
    """The same work as three calls on one stream, with events between them:
    the per-stage times and the attention kernel's own duration."""
    x, h, c, L = s["x"], s["h"], s["c"], s["L"]
    ev[0].record()
    Q.qsa_append(h, 1, L, 0, x["k"], x["v"], x["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"])
    ev[1].record()
    Q.qsa_index_select(h, 1, L, 0, x["q_idx"], c["kbar_cache"], s["bidx"], s["ws"])
    ev[2].record()
    Q.qsa_attend(h, 1, L, 0, x["q"], c["k_cache"], c["v_cache"], s["bidx"], s["out"])
    ev[3].record()


def setup_decode(w):
    B, ctx = w.batch, w.seq_len
    x = synth.decode_inputs(w, "cuda")
    h = Q.Handle(max_ctx=ctx + 4, budget_blocks=w.budget, yarn_factor=w.yarn_factor)
    c = Q.alloc_caches(h, B)
    for b in range(B):                           # cached context, sequence by sequence
        cs = {k: v[b:b + 1] for k, v in c.items()}
        Q.qsa_append(h, 1, ctx, 0, x["k"][b:b + 1, :ctx], x["v"][b:b + 1, :ctx], x["k_idx"][b:b + 1, :ctx],
                     cs["k_cache"], cs["v_cache"], cs["kbar_cache"], cs["kpend"])
    new = {n: x[n][:, ctx:ctx + 1].contiguous() for n in ("k", "v", "k_idx")}
    x_keep = {"q": x["q"], "q_idx": x["q_idx"], **new}
    del x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    cache_len = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    ws = Q.workspace(h, Q.QSA_OP_DECODE, B, 1, ctx)
    out = torch.empty((B, 1, 24, 256), dtype=torch.bfloat16, device="cuda")
    bidx = torch.empty((B, 1, w.budget), dtype=torch.int32, device="cuda")
    return dict(x=x_keep, h=h, c=c, ws=ws, out=out, bidx=bidx, cache_len=cache_len, B=B, ctx=ctx)


def decode_step(s):
    x, c = s["x"], s["c"]
    Q.qsa_decode(s["h"], s["B"], s["cache_len"], s["ctx"], x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"],
                 c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], s["out"], s["bidx"], s["ws"])


def attention_bytes(L, budget):
    """Algorithmic bytes of one sparse-attention launch over queries 0..L-1.

    Per query p: the gathered K~ and V of |T(p)| tokens for both KV heads
    (|T(p)| * 2 heads * 256 dims * 2 B * 2 tensors = 2048 B per token), its q
    row (24 * 256 * 2 B), its output row (same) and its selection (4 B per
    budget slot).  |T(p)| = min(budget, floor(p/4)) * 4 + (p mod 4) + 1.
    """
    p = np.arange(L, dtype=np.int64)
    T = np.minimum(budget, p // 4) * 4 + (p % 4) + 1
    return int(T.sum() * 2048 + L * (2 * 24 * 256 * 2 + 4 * budget)), int(T.sum())


def indexer_flops(L):
    p = np.arange(L, dtype=np.int64)
    return int(2 * 4 * 128 * (p // 4).sum())


def decode_bytes(B, ctx, budget):
    """Algorithmic HBM bytes of one decode step: per sequence the pooled keys of
    every candidate block (floor(p/4) * 256 B), the gathered K~/V of
    |T(p)| tokens (2048 B each), the new token's inputs and caches writes and
    the output row (small, counted as q 12 KiB + k,v 2 KiB + out 12 KiB)."""
    p = ctx
    T = min(budget, p // 4) * 4 + (p % 4) + 1
    per = (p // 4) * 256 + T * 2048 + 12288 + 2048 + 1024 + 12288
    return B * per


def measured_ceilings():
    """Rates this GPU reaches with plain library operations, beside the
    datasheet peaks: a 4 GiB device-to-device copy (bytes read + written per
    second) and a 8192^3 bf16 GEMM (torch.matmul)."""
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm_tfs = 20 * 2 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_GBs": copy_gbs, "gemm_bf16_TFs": gemm_tfs,
            "how": "4 GiB device copy (read + write bytes) and 8192^3 bf16 torch.matmul"}


def gather_ceilings(sp, reps=3):
    """Rates at which this GPU gathers 2 KiB micro-blocks, measured in this run
    with the benchmark's probe (libqsa_probe.so: the attention walk's loads with
    no arithmetic, both KV groups, 8 list entries per step):
      * l2_resident: every id in the first 128 blocks (1 MiB of K~/V), at the
        probe's full occupancy -- the ceiling of any gather;
      * no_reuse: ids uniform over the workload's whole cache, at the
        attention's occupancy (one wave per SIMD) -- random gathers that the
        L2 cannot serve;
      * attention_stream: the attention's own selection lists in its own
        launch shape (4,096 rows, group-major) -- its access stream alone.
    Returns {name: {"ms", "GBs"}} with GB/s of gathered bytes."""
    from block_sparse_long_qsa_amd import probe
    kc, vc = sp["c"]["k_cache"], sp["c"]["v_cache"]
    nblk = kc.shape[2]
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")

    def timed(idx, **kw):
        probe.gather(kc, vc, idx, sink, **kw)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e = _events(2)
            e[0].record()
            probe.gather(kc, vc, idx, sink, **kw)
            e[1].record()
            torch.cuda.synchronize()
            ts.append(e[0].elapsed_time(e[1]))
        ms = float(np.median(ts))
        nbytes = idx.shape[0] * 2 * (idx.shape[1] // 8 * 8) * 4096
        return {"ms": ms, "GBs": nbytes / (ms * 1e-3) / 1e9}

    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    res = {}
    idx = torch.randint(0, 128, (65536, 512), generator=g, dtype=torch.int32, device="cuda")
    res["l2_resident"] = timed(idx, pad_kib=0)
    idx = torch.randint(0, nblk, (65536, 512), generator=g, dtype=torch.int32, device="cuda")
    res["no_reuse"] = timed(idx, pad_kib=96)
    del idx
    res["attention_stream"] = timed(sp["bidx"][0], pad_kib=96, launch_rows=4096)
    torch.cuda.empty_cache()
    res["how"] = ("probe gathers (libqsa_probe.so), 16-byte loads, 8 list entries per step, K~ and V of both "
                  "groups; GB/s of gathered bytes")
    return res


def _cpu_info():
    """The host CPU's model name and the threads this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(s_pref, w, n_rows=None, budget_s=20.0):
    """Time the oracle on an evenly spaced sample of the prefill's rows (all the
    threads BLAS uses), then on a fixed 8-row sample with one thread."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    x = s_pref["x"]
    L = w.seq_len
    t0 = time.time()
    host = {n: synth.bf16_bits(x[n][0]) for n in ("k", "v", "k_idx")}
    p = O.Params(budget=w.budget, yarn_factor=w.yarn_factor)
    t_copy = time.time() - t0
    # rows: evenly spaced over the sequence (every stride-th row), so the sample
    # has the causal cost profile of the full run
    stride = L // (n_rows or 256)
    rows = np.arange(stride - 1, L, stride)
    t0 = time.time()
    lay = O.LayerOracle(host["k"], host["v"], host["k_idx"], p)
    t_pool = time.time() - t0
    done = []
    outs, sels = [], []
    for r in rows:
        o, sel, _ = lay.row(int(r), synth.bf16_bits(x["q"][0, r]), synth.bf16_bits(x["q_idx"][0, r]))
        done.append(int(r))
        outs.append(o)
        sels.append(sel)
        if time.time() - t0 > budget_s:
            break
    dt = time.time() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    # the same oracle rows with one thread: every 32,768-th row (8 rows)
    fixed = np.arange(L // 8 - 1, L, L // 8)
    with threadpool_limits(limits=1):
        t1 = time.time()
        for r in fixed:
            lay.row(int(r), synth.bf16_bits(x["q"][0, r]), synth.bf16_bits(x["q_idx"][0, r]))
        dt1 = time.time() - t1
    # parity of the GPU rows against the oracle rows just computed
    gpu_out = s_pref["out"][0, done].float().cpu().numpy()
    gpu_sel = s_pref["bidx"][0, done].cpu().numpy()
    max_err = float(np.max(np.abs(gpu_out - np.stack(outs))))
    sel_diff = int(sum(len(set(a[a >= 0].tolist()) ^ set(b[b >= 0].tolist())) for a, b in zip(gpu_sel, sels)))
    return {
        "value": len(done) / dt, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
        "sample": "%d prefill rows of the L=%d sequence, every %d-th row (rows %d..%d), incl. pooling all %d "
                  "blocks (%.1f s); host copy of inputs %.1f s not counted" % (
                      len(done), L, stride, done[0], done[-1], L // 4, t_pool, t_copy),
        "one_core": {"value": len(fixed) / dt1, "unit": "tok/s", "threads": 1,
                     "sample": "prefill rows %s (every %d-th row), pooling not counted" % (
                         ",".join(str(int(r)) for r in fixed), L // 8)},
        **_cpu_info(),
        "parity_on_sample": {"rows": len(done), "max_abs_err": max_err, "selection_sym_diff": sel_diff},
    }


def cpu_baseline_decode(sd, wd, n_seq=2):
    """The oracle's decode rows for the first n_seq sequences of the decode
    workload (inputs regenerated from the same seeds), timed per query with all
    BLAS threads (pooling the cached keys is a per-sequence set-up, timed
    apart), and their parity with the GPU's decode step."""
    import oracle as O
    from threadpoolctl import threadpool_info
    x = synth.decode_inputs(wd, "cuda", batch=n_seq)
    p = O.Params(budget=wd.budget, yarn_factor=wd.yarn_factor)
    ctx = wd.seq_len
    t_pool = t_row = 0.0
    max_err, sel_diff = 0.0, 0
    for b in range(n_seq):
        host = {n: synth.bf16_bits(x[n][b]) for n in ("k", "v", "k_idx")}
        t0 = time.time()
        lay = O.LayerOracle(host["k"], host["v"], host["k_idx"], p)
        t1 = time.time()
        o, sel, _ = lay.row(ctx, synth.bf16_bits(x["q"][b, 0]), synth.bf16_bits(x["q_idx"][b, 0]))
        t2 = time.time()
        t_pool += t1 - t0
        t_row += t2 - t1
        g = sd["out"][b, 0].float().cpu().numpy()
        gs = sd["bidx"][b, 0].cpu().numpy()
        max_err = max(max_err, float(np.max(np.abs(g - o))))
        sel_diff += len(set(gs[gs >= 0].tolist()) ^ set(sel[sel >= 0].tolist()))
    del x
    torch.cuda.empty_cache()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": n_seq / t_row, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "sample": "the decode query of sequences 0..%d of %d (context %d each); pooling their cached keys "
                      "%.1f s not counted" % (n_seq - 1, wd.batch, ctx, t_pool),
            "parity_on_sample": {"seqs": n_seq, "max_abs_err": max_err, "selection_sym_diff": sel_diff}}


def prefill_1m_state():
    """Inputs, handle, caches and buffers of the 1,048,576-token chunked prefill (YaRN 4)."""
    wp = synth.WORKLOADS["prefill_1m"]
    L, C = wp.seq_len, wp.chunk
    x = synth.prefill_inputs(wp, "cuda")
    h = Q.Handle(max_ctx=L, budget_blocks=wp.budget, yarn_factor=wp.yarn_factor)
    c = Q.alloc_caches(h, 1)
    ws = Q.workspace(h, Q.QSA_OP_FORWARD, 1, C, L - C)
    out = torch.empty((1, L, 24, 256), dtype=torch.bfloat16, device="cuda")
    bidx = torch.empty((1, L, wp.budget), dtype=torch.int32, device="cuda")
    return dict(w=wp, x=x, h=h, c=c, ws=ws, out=out, bidx=bidx, L=L, C=C)


def qsa_prefill_1m_ms(steps, st=None):
    """QSA chunked prefill of 1,048,576 tokens (YaRN 4) in 65,536-token
    qsa_forward calls: one warm-up pass, then the mean of `steps` passes (ms)."""
    own = st is None
    if own:
        st = prefill_1m_state()
    x, h, c, ws, out, bidx, L, C = (st[k] for k in ("x", "h", "c", "ws", "out", "bidx", "L", "C"))

    def prefill():
        for s0 in range(0, L, C):
            sl = lambda t: t[:, s0:s0 + C]
            Q.qsa_forward(h, 1, C, s0, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["q_idx"]), sl(x["k_idx"]),
                          c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], sl(out), sl(bidx), ws)

    prefill()
    torch.cuda.synchronize()
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        prefill()
    ev[1].record()
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) / steps
    if own:
        del st, x, c, ws, out, bidx, h
        torch.cuda.empty_cache()
    return t


def dense_attend_ms(h, c, x, out, L, reps=1):
    """This library's dense causal GQA kernel (qsa_dense_attend) over every
    query of an L-token prefill whose K~/V caches are already filled: one
    warm-up call on the last 16 rows, then the mean of `reps` full calls (ms)."""
    Q.qsa_dense_attend(h, 1, 16, L - 16, x["q"][:, L - 16:], c["k_cache"], c["v_cache"], out[:, L - 16:])
    torch.cuda.synchronize()
    ev = _events(2)
    ev[0].record()
    for _ in range(reps):
        Q.qsa_dense_attend(h, 1, L, 0, x["q"], c["k_cache"], c["v_cache"], out)
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def dense_flops(L):
    """Algorithmic FLOPs of dense causal attention over L queries: 2 products x
    2 FLOP x 24 heads x 256 dims per (query, key <= query) pair."""
    return 4 * 24 * 256 * L * (L + 1) // 2


def run_c5(steps):
    """The 1M-token configuration (YaRN factor 4): a chunked prefill of
    1,048,576 tokens in 65,536-token qsa_forward calls, and decode steps of
    8 sequences with 1,048,576 cached tokens each.  One JSON line."""
    wp, wd = synth.WORKLOADS["prefill_1m"], synth.WORKLOADS["decode_1m"]
    L = wp.seq_len
    t_pre = qsa_prefill_1m_ms(steps)
    _progress("c5 prefill done")
    ev = _events(2)
    sd = setup_decode(wd)
    for _ in range(3):
        decode_step(sd)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(10 * steps):
        decode_step(sd)
    ev[1].record()
    torch.cuda.synchronize()
    t_dec = ev[0].elapsed_time(ev[1]) / (10 * steps)
    ab, _ = attention_bytes(L, wp.budget)
    db = decode_bytes(wd.batch, wd.seq_len, wd.budget)
    res = {
        "c5": {
            "prefill": {"workload": wp.name, "ms": t_pre, "tok_s": L / (t_pre * 1e-3),
                        "indexer_tflop": indexer_flops(L) / 1e12, "attention_gathered_TB": ab / 1e12},
            "decode": {"workload": wd.name, "ms": t_dec, "tok_s": wd.batch / (t_dec * 1e-3),
                       "roofline": {"bound": "hbm", "achieved": db / (t_dec * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": db / (t_dec * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "algorithmic_bytes": db}},
            "steps": steps, "dtype": "bf16", "data": "synthetic",
        }
    }
    print(json.dumps(res), flush=True)


def dense_prefill_ms(L, reps=1):
    """Dense causal GQA attention over L tokens (24 query heads, 2 KV heads, head
    dim 256, bf16) with PyTorch's flash / memory-efficient SDPA kernels: the
    dense baseline of the pages' speed-up figures.  Timing only (random
    operands of the layer's shapes)."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    q = torch.randn(1, 24, L, 256, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(1, 2, L, 256, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(1, 2, L, 256, device="cuda", generator=g).to(torch.bfloat16)
    f = torch.nn.functional.scaled_dot_product_attention
    with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
        o = f(q, k, v, is_causal=True, scale=1.0 / 16, enable_gqa=True)
        torch.cuda.synchronize()
        ev = _events(2)
        ev[0].record()
        for _ in range(reps):
            o = f(q, k, v, is_causal=True, scale=1.0 / 16, enable_gqa=True)
        ev[1].record()
        torch.cuda.synchronize()
    del q, k, v, o
    torch.cuda.empty_cache()
    return ev[0].elapsed_time(ev[1]) / reps


def indexer_ratio_prefill(w, steps):
    """The indexer alone at compression ratio 4 against ratio 1 on prefill
    workload w (in w.chunk-token calls when it is chunked): qsa_index_select over
    the pooled keys (built beforehand by qsa_append) against
    qsa_token_index_select over every token's key (its per-call key rotation
    included), both selecting the budget's 512 entries per query.  ms per pass."""
    L = w.seq_len
    C = w.chunk or L
    x = synth.prefill_inputs(w, "cuda")
    h = Q.Handle(max_ctx=L, budget_blocks=w.budget, yarn_factor=w.yarn_factor)
    c = Q.alloc_caches(h, 1)
    for s0 in range(0, L, C):
        sl = lambda t: t[:, s0:s0 + C]
        Q.qsa_append(h, 1, C, s0, sl(x["k"]), sl(x["v"]), sl(x["k_idx"]), c["k_cache"], c["v_cache"],
                     c["kbar_cache"], c["kpend"])
    for n in ("q", "k", "v"):
        del x[n]
    torch.cuda.empty_cache()
    ktok = Q.alloc_token_keys(h, 1)
    sel = torch.empty((1, C, w.budget), dtype=torch.int32, device="cuda")
    ws4 = Q.workspace(h, Q.QSA_OP_INDEX_SELECT, 1, C, L - C)
    ws1 = Q.workspace(h, Q.QSA_OP_TOKEN_INDEX_SELECT, 1, C, L - C)

    def r4():
        for s0 in range(0, L, C):
            Q.qsa_index_select(h, 1, C, s0, x["q_idx"][:, s0:s0 + C], c["kbar_cache"], sel, ws4)

    def r1():
        for s0 in range(0, L, C):
            Q.qsa_token_index_select(h, 1, C, s0, x["q_idx"][:, s0:s0 + C], x["k_idx"][:, s0:s0 + C], ktok, sel,
                                     ws1)

    t = {}
    for name, fn in (("r4", r4), ("r1", r1)):
        fn()
        torch.cuda.synchronize()
        e = _events(2)
        e[0].record()
        for _ in range(steps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        t[name] = e[0].elapsed_time(e[1]) / steps
    del x, c, ktok, sel, ws4, ws1, h
    torch.cuda.empty_cache()
    return t


def indexer_ratio_decode(wd, steps):
    """One decode step's indexer alone at ratio 4 (qsa_index_decode over the pooled
    cache) against ratio 1 (qsa_token_index_decode over a token-key cache of
    random bf16 keys: timing only) for wd.batch sequences of wd.seq_len tokens."""
    sd = setup_decode(wd)
    h, B, ctx, x, c = sd["h"], sd["B"], sd["ctx"], sd["x"], sd["c"]
    for n in ("k_cache", "v_cache"):
        del c[n]
    torch.cuda.empty_cache()
    ktok = Q.alloc_token_keys(h, B)
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    for b in range(B):
        ktok[b].copy_(torch.randn(ktok.shape[1:], device="cuda", generator=g).to(torch.bfloat16))
    sel = torch.empty((B, wd.budget), dtype=torch.int32, device="cuda")
    ws4 = Q.workspace(h, Q.QSA_OP_INDEX_DECODE, B, 1, ctx)
    ws1 = Q.workspace(h, Q.QSA_OP_TOKEN_INDEX_DECODE, B, 1, ctx)
    fns = {"r4": lambda: Q.qsa_index_decode(h, B, sd["cache_len"], ctx, x["q_idx"], x["k_idx"], c["kbar_cache"],
                                            c["kpend"], sel, ws4),
           "r1": lambda: Q.qsa_token_index_decode(h, B, sd["cache_len"], ctx, x["q_idx"], x["k_idx"], ktok, sel,
                                                  ws1)}
    t = {}
    for name, fn in fns.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e = _events(2)
        e[0].record()
        for _ in range(10 * steps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        t[name] = e[0].elapsed_time(e[1]) / (10 * steps)
    del sd, ktok, sel, ws4, ws1
    torch.cuda.empty_cache()
    return t


def run_ratios(steps):
    """QSA against dense attention on this GPU, as in the pages' module
    speed-ups (prefill and decode at 1M tokens): QSA prefill (append + fused
    index/select + sparse attention) against this library's dense causal GQA
    kernel over the same caches (qsa_dense_attend; PyTorch's SDPA beside it for
    reference) at 262,144 and 1,048,576 tokens, and QSA decode of 8 x 1,048,576
    against the same split-K
    decode kernel over every cached token (qsa_decode_reuse with a selection
    made at position 0: no selected block, the tail is the whole context).
    Then the indexer alone at compression ratio 4 against ratio 1 (the pages'
    indexer speed-ups), at 262,144 and 1,048,576 prefill tokens and for the
    8 x 1,048,576 decode step."""
    res = {}
    wp = synth.WORKLOADS["prefill_256k"]
    sp = setup_prefill(wp)
    for _ in range(2):
        prefill_forward(sp, _events(2))
    ev = [_events(2) for _ in range(steps)]
    for e in ev:
        prefill_forward(sp, e)
    torch.cuda.synchronize()
    t_qsa = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_dense = dense_attend_ms(sp["h"], sp["c"], sp["x"], sp["out"], wp.seq_len, reps=2)
    del sp
    torch.cuda.empty_cache()
    t_sdpa = dense_prefill_ms(wp.seq_len, reps=2)
    _progress("ratios: prefill 262144 done")
    res["prefill_262144"] = {"qsa_ms": t_qsa, "dense_ms": t_dense, "speedup": t_dense / t_qsa,
                             "dense_tflops": dense_flops(wp.seq_len) / (t_dense * 1e-3) / 1e12,
                             "dense_kernel": "qsa_dense_attend (this library)",
                             "torch_sdpa_ms": t_sdpa}
    wp_1m = synth.WORKLOADS["prefill_1m"]
    st = prefill_1m_state()
    t_qsa_1m = qsa_prefill_1m_ms(1, st)
    t_dense_1m = dense_attend_ms(st["h"], st["c"], st["x"], st["out"], st["L"], reps=1)
    del st
    torch.cuda.empty_cache()
    t_sdpa_1m = dense_prefill_ms(1 << 20, reps=1)
    _progress("ratios: prefill 1048576 done")
    res["prefill_1048576"] = {"qsa_ms": t_qsa_1m, "dense_ms": t_dense_1m, "speedup": t_dense_1m / t_qsa_1m,
                              "dense_tflops": dense_flops(1 << 20) / (t_dense_1m * 1e-3) / 1e12,
                              "dense_kernel": "qsa_dense_attend (this library)",
                              "torch_sdpa_ms": t_sdpa_1m,
                              "torch_sdpa_tflops": dense_flops(1 << 20) / (t_sdpa_1m * 1e-3) / 1e12}
    wd = synth.WORKLOADS["decode_1m"]
    sd = setup_decode(wd)
    x, c = sd["x"], sd["c"]
    zero = torch.zeros_like(sd["cache_len"])
    sel = sd["bidx"].view(sd["B"], -1).contiguous()

    def dense_step():
        Q.qsa_decode_reuse(sd["h"], sd["B"], sd["cache_len"], zero, sd["ctx"], x["q"], x["k"], x["v"], x["k_idx"],
                           c["k_cache"], c["v_cache"], c["kbar_cache"], c["kpend"], sel, sd["out"], sd["ws"])

    times = {}
    for name, fn in (("qsa", lambda: decode_step(sd)), ("dense", dense_step)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e = _events(2)
        e[0].record()
        for _ in range(5 * steps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        times[name] = e[0].elapsed_time(e[1]) / (5 * steps)
    res["decode_B8_ctx1048576"] = {"qsa_ms": times["qsa"], "dense_split_k_ms": times["dense"],
                                   "speedup": times["dense"] / times["qsa"]}
    res["pages_module_speedups_at_1M"] = {"prefill": 7.6, "decode": 4.9,
                                          "note": "other hardware, dense baseline a paged GQA library"}
    del sd, x, c, sel
    torch.cuda.empty_cache()
    idx = {}
    for key, w in (("prefill_262144", synth.WORKLOADS["prefill_256k"]), ("prefill_1048576", wp_1m)):
        t = indexer_ratio_prefill(w, steps)
        _progress("ratios: indexer " + key + " done")
        idx[key] = {"r4_ms": t["r4"], "r1_ms": t["r1"], "speedup": t["r1"] / t["r4"]}
    t = indexer_ratio_decode(wd, steps)
    idx["decode_B8_ctx1048576"] = {"r4_ms": t["r4"], "r1_ms": t["r1"], "speedup": t["r1"] / t["r4"]}
    idx["pages_indexer_speedups_r4"] = {"prefill": 3.8, "decode": 4.4, "note": "other hardware"}
    res["indexer_r4_vs_r1"] = idx
    print(json.dumps({"ratios": res}), flush=True)


def train_bytes(L, budget):
    """Algorithmic bytes of one indexer-loss pass (teacher + student) over L
    query rows: per selected block 2 x 2,048 B of K~ (both KV groups) and 256 B
    of k̄, per query its q (12,288 B), q_idx (1,024 B) and stats (128 B)."""
    o = np.arange(L, dtype=np.int64) // 4
    nsel = np.minimum(o, budget).sum()
    return int(nsel) * (2 * 2048 + 256) + L * (12288 + 1024 + 128)


def run_train(steps):
    """One training step of the layer on the 32,768- and 262,144-token prefill
    workloads: forward = qsa_append + qsa_index_select (the top-k, not
    differentiated) + qsa_train_forward (sparse attention with log-sum-exp, then
    the indexer KL loss); backward = qsa_train_backward_indexer (gradients to the
    raw indexer queries and keys) + qsa_train_backward_attention (gradients to
    q, k, v).  HIP events between the stages; one JSON line."""
    res = {}
    for key in ("prefill_32k", "prefill_256k"):
        w = synth.WORKLOADS[key]
        L, budget = w.seq_len, w.budget
        x = synth.prefill_inputs(w, "cuda")
        h = Q.Handle(max_ctx=L, budget_blocks=budget)
        c = Q.alloc_caches(h, 1)
        bidx = torch.empty((1, L, budget), dtype=torch.int32, device="cuda")
        out = torch.empty((1, L, 24, 256), dtype=torch.bfloat16, device="cuda")
        stats = torch.empty((1, L, 32), dtype=torch.float32, device="cuda")
        kl = torch.empty((1, L), dtype=torch.float32, device="cuda")
        dkl = torch.full((1, L), 1.0 / L, dtype=torch.float32, device="cuda")
        dq = torch.empty((1, L, 4, 128), dtype=torch.float32, device="cuda")
        dk = torch.empty((1, L, 128), dtype=torch.float32, device="cuda")
        g = torch.Generator(device="cuda")
        g.manual_seed(11)
        dout = torch.randn((1, L, 24, 256), device="cuda", generator=g).to(torch.bfloat16)
        dqa = torch.empty((1, L, 24, 256), dtype=torch.float32, device="cuda")
        dka = torch.empty((1, L, 2, 256), dtype=torch.float32, device="cuda")
        dva = torch.empty((1, L, 2, 256), dtype=torch.float32, device="cuda")
        ws_is = Q.workspace(h, Q.QSA_OP_INDEX_SELECT, 1, L, 0)
        ws_f = Q.workspace(h, Q.QSA_OP_TRAIN_FORWARD, 1, L, 0)
        ws_b = Q.workspace(h, Q.QSA_OP_TRAIN_BACKWARD, 1, L, 0)

        def step(ev):
            ev[0].record()
            Q.qsa_append(h, 1, L, 0, x["k"], x["v"], x["k_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"],
                         c["kpend"])
            Q.qsa_index_select(h, 1, L, 0, x["q_idx"], c["kbar_cache"], bidx, ws_is)
            ev[1].record()
            Q.qsa_train_forward(h, 1, L, x["q"], x["q_idx"], c["k_cache"], c["v_cache"], c["kbar_cache"], bidx, out,
                                stats, kl, ws_f)
            ev[2].record()
            Q.qsa_train_backward_indexer(h, 1, L, x["q"], x["q_idx"], c["k_cache"], c["kbar_cache"], bidx, stats, dkl,
                                         dq, dk, ws_b)
            ev[3].record()
            Q.qsa_train_backward_attention(h, 1, L, x["q"], c["k_cache"], c["v_cache"], bidx, out, dout, stats,
                                           dqa, dka, dva)
            ev[4].record()

        step(_events(5))
        torch.cuda.synchronize()
        evs = [_events(5) for _ in range(steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        fwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
        att_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in evs]))
        tot = sel_ms + fwd_ms + bwd_ms + att_ms
        _progress("train: " + w.name + " done")
        res[w.name] = {"ms": tot, "tok_s": L / (tot * 1e-3),
                       "stage_ms": {"append_index_select": sel_ms, "train_forward": fwd_ms, "backward_indexer": bwd_ms,
                                    "backward_attention": att_ms},
                       "mean_kl": float(kl.mean()), "indexer_loss_bytes_per_pass": train_bytes(L, budget)}
        del x, c, bidx, out, stats, kl, dkl, dq, dk, ws_is, ws_f, ws_b, h, dout, dqa, dka, dva
        torch.cuda.empty_cache()
    print(json.dumps({"train": res, "steps": steps, "dtype": "bf16", "data": "synthetic"}), flush=True)


GDN_HQ, GDN_HV = 16, 48      # QK and V heads of the pages' GDN layers (head dim 128)


def gdn_counts(lens, hq=GDN_HQ, hv=GDN_HV):
    """Algorithmic work of the two GDN kernels over packed sequences `lens`
    (chunks of 64; the last chunk of a sequence counts as a whole chunk, as the
    kernels compute it).  Scan, per (chunk, V head): [K; Q] S, Tb X, P U and
    K^T U = 8,388,608 flops; bytes: q, k once per QK head (32 KiB per chunk), v
    and o (16 KiB each), g (256 B), Tb and P (16 KiB).  Prep, per (chunk, QK
    head): the 10 causal 16 x 16 tiles of K K^T and Q K^T = 1,310,720 flops;
    bytes: q, k (32 KiB), g and beta (512 B per V head), Tb and P written
    (16 KiB per V head)."""
    nck = sum((n + 63) // 64 for n in lens)
    ntok = sum(lens)
    scan_flops = nck * hv * 8388608
    prep_flops = nck * hq * 1310720
    qk_bytes = ntok * hq * 128 * 2 * 2
    scan_bytes = qk_bytes + ntok * hv * (128 * 2 * 2 + 4) + nck * hv * 16384
    prep_bytes = qk_bytes + ntok * hv * 8 + nck * hv * 16384
    return {"scan_flops": scan_flops, "prep_flops": prep_flops, "scan_bytes": scan_bytes, "prep_bytes": prep_bytes}


def gdn_cpu_baseline(x, n_tok=512):
    """The oracle (token-by-token fp64 recurrence, all 48 V heads) on the first
    n_tok tokens of the workload."""
    from oracle import gdn as OG
    f = lambda t: t[:n_tok].float().cpu().numpy().astype(np.float64)
    q, k, v, g, b = f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"])
    t0 = time.perf_counter()
    OG.gdn_recurrent(q, k, v, g, b, 128 ** -0.5)
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tok/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": "first %d tokens of the 262,144-token sequence, all 48 V heads" % n_tok}


def run_gdn(steps, cpu=True):
    """Gated DeltaNet chunked prefill (the hybrid's other token mixer) on one
    262,144-token sequence and on 8 packed sequences of 32,768 tokens; 16 QK
    heads, 48 V heads, head dim 128.  HIP events around qsa_gdn_prep and
    qsa_gdn_scan (the two kernels qsa_gdn_chunk_prefill launches) on the
    current stream; one JSON line."""
    res = {}
    base = None
    for name, lens in (("gdn_T262144_x1", [262144]), ("gdn_T32768_x8", [32768] * 8)):
        x = synth.gdn_inputs(21, lens, GDN_HQ, GDN_HV, "cuda")
        nseq, max_len = len(lens), max(lens)
        o = torch.empty_like(x["v"])
        fs = torch.empty(nseq, GDN_HV, 128, 128, device="cuda")
        ws = torch.empty(Q.qsa_gdn_workspace_size(nseq, max_len, GDN_HQ, GDN_HV), dtype=torch.uint8, device="cuda")
        scale = 128 ** -0.5

        def step(ev):
            ev[0].record()
            Q.qsa_gdn_prep(nseq, x["cu_seqlens"], max_len, x["q"], x["k"], GDN_HV, x["g"], x["beta"], scale, ws)
            ev[1].record()
            Q.qsa_gdn_scan(nseq, x["cu_seqlens"], max_len, x["q"], x["k"], x["v"], x["g"], scale, None, o, fs, ws)
            ev[2].record()

        step(_events(3))
        torch.cuda.synchronize()
        evs = [_events(3) for _ in range(steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        c = gdn_counts(lens)
        ntok = sum(lens)

        def roof(flops, nbytes, ms):
            tfs = flops / (ms * 1e-3) / 1e12
            gbs = nbytes / (ms * 1e-3) / 1e9
            out = {"tflops": tfs, "mfma_frac": tfs / MFMA_BF16_PEAK_TFS, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                   "algorithmic_flops": flops, "algorithmic_bytes": nbytes, "avg_ms": ms}
            return out

        res[name] = {"ms": prep_ms + scan_ms, "tok_s": ntok / ((prep_ms + scan_ms) * 1e-3),
                     "gdn_prep_kernel": roof(c["prep_flops"], c["prep_bytes"], prep_ms),
                     "gdn_scan_kernel": roof(c["scan_flops"], c["scan_bytes"], scan_ms)}
        if base is None:
            base = x if cpu else None
        else:
            del x
        del o, fs, ws
        torch.cuda.empty_cache()
    line = {"gdn": res, "steps": steps, "dtype": "bf16", "data": "synthetic",
            "config": {"hq_heads": GDN_HQ, "hv_heads": GDN_HV, "head_dim": 128, "chunk": 64}}
    if base is not None:
        line["cpu_baseline"] = gdn_cpu_baseline(base)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="decode step only (profiling)")
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured copy / GEMM ceilings")
    ap.add_argument("--ratios", action="store_true",
                    help="measure QSA against dense attention (the pages' module speed-ups) instead")
    ap.add_argument("--c5", action="store_true",
                    help="measure the 1M-token configuration instead (chunked prefill, B=8 decode)")
    ap.add_argument("--train", action="store_true",
                    help="measure a training step (indexer loss forward and backward) instead")
    ap.add_argument("--gdn", action="store_true",
                    help="measure the Gated DeltaNet chunked prefill instead")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    torch.cuda.init()
    if args.c5:
        run_c5(max(1, min(args.steps, 3)))
        return
    if args.ratios:
        run_ratios(max(1, min(args.steps, 3)))
        return
    if args.train:
        run_train(max(1, min(args.steps, 5)))
        return
    if args.gdn:
        run_gdn(max(1, min(args.steps, 10)), cpu=not args.no_cpu_baseline)
        return
    if args.calib_copy:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wp = synth.WORKLOADS["prefill_256k"]
    wd = synth.WORKLOADS["decode_128k"]
    sp = None if args.no_prefill else setup_prefill(wp)
    sd = None if args.no_decode else setup_decode(wd)
    torch.cuda.synchronize()
    print("setup done", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        if sp:
            prefill_forward(sp, _events(2))
        if sd:
            decode_step(sd)
    torch.cuda.synchronize()
    print("warmup done", file=sys.stderr, flush=True)

    ev_f = [_events(2) for _ in range(args.steps)]
    ev_d = [_events(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if sp:
            prefill_forward(sp, ev_f[i])
        if sd:
            ev_d[i][0].record()
            decode_step(sd)
            ev_d[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_p = []
    if sp:                  # per-stage times: the staged calls, after the timed region
        n_st = max(1, min(args.steps, 5))
        prefill_stages(sp, _events(4))
        ev_p = [_events(4) for _ in range(n_st)]
        for e in ev_p:
            prefill_stages(sp, e)
        torch.cuda.synchronize()

    if sp is None:
        t_dec = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_d]))
        print(json.dumps({"decode_only": True, "ms": t_dec, "tok_s": wd.batch / (t_dec * 1e-3),
                          "hbm_frac": decode_bytes(wd.batch, wd.seq_len, wd.budget) / (t_dec * 1e-3) / 1e9 /
                          HBM_PEAK_GBS}))
        return
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev_p])   # ms
    t_append, t_isel, t_attn = st.mean(axis=0)
    t_prefill = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_f]))
    t_staged = float(st.sum(axis=1).mean())
    t_dec = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_d])) if sd else None

    L = wp.seq_len
    attn_bytes, sum_T = attention_bytes(L, wp.budget)
    attn_flops = 24576 * sum_T                 # 2 FLOP x 2 products x 24 heads x 256 dims per gathered token
    attn_tfs = attn_flops / (t_attn * 1e-3) / 1e12
    gath_bytes = 2048 * sum_T                  # K~ and V of both KV groups per gathered token
    gath_gbs = gath_bytes / (t_attn * 1e-3) / 1e9
    # compulsory HBM bytes of the attention pass: the K~/V caches once, q read,
    # output written and the selection read once
    comp_bytes = L * (2048 + 2 * 24 * 256 * 2 + 4 * wp.budget)
    tr_bytes = attend_traffic_bytes()
    idx_tfs = indexer_flops(L) / (t_isel * 1e-3) / 1e12
    res = {
        "metric": "QSA prefill tok/s @256K + decode tok/s @128K ctx; % of MFMA/HBM peak",
        "value": L / (t_prefill * 1e-3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 with planted needles; no datasets or weights)",
        "config": {
            "workload": "%s + %s" % (wp.name, wd.name),
            "prefill": {"batch": 1, "seq_len": L, "budget_blocks": wp.budget, "needles": wp.n_needles,
                        "recency_blocks_x1.5": wp.recency_blocks},
            "decode": {"batch": wd.batch, "ctx": wd.seq_len, "budget_blocks": wd.budget},
        },
        "prefill": {
            "ms": t_prefill, "tok_s": L / (t_prefill * 1e-3), "call": "qsa_forward",
            "staged_ms": t_staged,
            "stage_ms": {"append": float(t_append), "index_select": float(t_isel), "attend": float(t_attn)},
            "index_select_tflops_equiv": idx_tfs,
            "index_select_mfma_frac": idx_tfs / MFMA_BF16_PEAK_TFS,
        },
        "roofline": {
            "kernel": "attend_prefill_kernel (qsa_attend: %d launches of up to 2,048 rows, two queries per wave)"
                      % ((L + 2047) // 2048),
            "bound": "mfma", "achieved": attn_tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": attn_tfs / MFMA_BF16_PEAK_TFS,
            "traffic": None if tr_bytes is None else tr_bytes / (t_attn * 1e-3) / 1e9,
            "traffic_unit": "GB/s, HBM side (rocprofv3 FETCH_SIZE/WRITE_SIZE scaled by a copy kernel's reading)",
            "traffic_bytes_per_pass": tr_bytes,
            "algorithmic_flops": attn_flops, "gathered_tokens": sum_T, "avg_ms": float(t_attn),
            "gather": {"achieved_GBs": gath_gbs, "gathered_bytes": gath_bytes},
            "compulsory_hbm": {"bytes": comp_bytes, "GBs": comp_bytes / (t_attn * 1e-3) / 1e9,
                               "frac_of_hbm_peak": comp_bytes / (t_attn * 1e-3) / 1e9 / HBM_PEAK_GBS},
        },
    }
    if sd:
        db = decode_bytes(wd.batch, wd.seq_len, wd.budget)
        dgbs = db / (t_dec * 1e-3) / 1e9
        res["decode"] = {"ms": t_dec, "tok_s": wd.batch / (t_dec * 1e-3),
                         "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": dgbs / HBM_PEAK_GBS, "algorithmic_bytes": db}}
    if not args.no_ceilings:
        ceil = measured_ceilings()
        res["measured_ceilings"] = ceil
        gc = gather_ceilings(sp)
        ceil["gather"] = gc
        gr = res["roofline"]["gather"]
        gr["l2_resident_ceiling_GBs"] = gc["l2_resident"]["GBs"]
        gr["frac_of_l2_resident_ceiling"] = gath_gbs / gc["l2_resident"]["GBs"]
        gr["no_reuse_GBs"] = gc["no_reuse"]["GBs"]
        gr["own_stream_without_arithmetic_ms"] = gc["attention_stream"]["ms"]
        gr["kernel_ms_over_own_stream_ms"] = float(t_attn) / gc["attention_stream"]["ms"]
        res["prefill"]["index_select_frac_of_measured_gemm"] = idx_tfs / ceil["gemm_bf16_TFs"]
        if sd:
            res["decode"]["roofline"]["frac_of_measured_copy"] = res["decode"]["roofline"]["achieved"] / ceil["copy_GBs"]
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        res["cpu_baseline"] = cpu_baseline(sp, wp, n_rows=args.cpu_rows)
        if sd:
            res["decode"]["cpu_baseline"] = cpu_baseline_decode(sd, wd)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
