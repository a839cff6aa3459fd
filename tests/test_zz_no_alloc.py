"""qsa_decode_noalloc -- the decode step with no workspace argument, its
scratch in the library's fixed per-GPU array -- against qsa_decode with a
caller workspace: two calls in a row, the second with a smaller batch and
context, give bitwise the outputs and selections qsa_decode gives; a size whose
scratch exceeds the array is refused before anything is enqueued."""
import ctypes

import pytest
import torch

import block_sparse_long_qsa_amd as Q
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(h, lens, seed):
    B = len(lens)
    w = synth.Workload("t", "decode", B, max(lens), h.budget, 4, "random", seed)
    x = synth.decode_inputs(w, "cpu", ctx=max(lens), batch=B)
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _decode(h, lens, x, noalloc):
    """Fresh caches holding each sequence's context, then one decode step."""
    B = len(lens)
    c = Q.alloc_caches(h, B)
    for t in c.values():          # slots no call writes compare equal
        t.zero_()
    for b, n in enumerate(lens):
        if n:
            sl = lambda t: t[b:b + 1, :n].contiguous()
            cs = {k: v[b:b + 1] for k, v in c.items()}
            Q.qsa_append(h, 1, n, 0, sl(x["k"]), sl(x["v"]), sl(x["k_idx"]), cs["k_cache"], cs["v_cache"],
                         cs["kbar_cache"], cs["kpend"])
    new = {n: torch.stack([x[n][b, lens[b]] for b in range(B)])[:, None].contiguous() for n in ("k", "v", "k_idx")}
    cache_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, 24, 256), dtype=torch.bfloat16, device=DEV)
    bidx = torch.empty((B, 1, h.budget), dtype=torch.int32, device=DEV)
    args = (h, B, cache_len, max(lens), x["q"], new["k"], new["v"], x["q_idx"], new["k_idx"], c["k_cache"],
            c["v_cache"], c["kbar_cache"], c["kpend"], out, bidx)
    if noalloc:
        Q.qsa_decode_noalloc(*args)
    else:
        Q.qsa_decode(*args, Q.workspace(h, Q.QSA_OP_DECODE, B, 1, max(lens)))
    torch.cuda.synchronize()
    return out, bidx, c


def test_noalloc_decode_equals_decode_with_workspace():
    h = Q.Handle(max_ctx=8192, budget_blocks=64)
    cases = [([6000, 3, 0, 4097, 5999, 1200, 777, 6001, 255, 4096, 2, 5000], 61), ([900, 17, 400], 62)]
    xs = [_inputs(h, lens, seed) for lens, seed in cases]
    ref = [_decode(h, lens, x, noalloc=False) for (lens, _), x in zip(cases, xs)]
    got = [_decode(h, lens, x, noalloc=True) for (lens, _), x in zip(cases, xs)]    # two calls in a row
    for (lens, _), r, g in zip(cases, ref, got):
        assert torch.equal(r[1], g[1]), "selection, batch %d" % len(lens)
        assert torch.equal(r[0].view(torch.int16), g[0].view(torch.int16)), "output, batch %d" % len(lens)
        for name in ("k_cache", "v_cache", "kbar_cache", "kpend"):
            assert torch.equal(r[2][name].view(torch.int16), g[2][name].view(torch.int16)), name


def test_noalloc_decode_refuses_sizes_beyond_its_scratch():
    """B = 64 at a 262,140-token context needs about 38 MiB of scratch: refused
    with QSA_ERR_WORKSPACE on the host (the pointers are never dereferenced:
    the size check comes first), while the 32 MiB array covers B = 64 at
    131,072 (sized, not run)."""
    h = Q.Handle(max_ctx=262144, budget_blocks=512)
    need = Q.qsa_workspace_size(h, Q.QSA_OP_DECODE, 64, 1, 262140)
    assert need > Q.NOALLOC_SCRATCH_BYTES
    assert Q.qsa_workspace_size(h, Q.QSA_OP_DECODE, 64, 1, 131072) <= Q.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)
    st = Q.lib().qsa_decode_noalloc(h.ptr, None, 64, fake, 262140, *([fake] * 10), None)
    assert st == 6
