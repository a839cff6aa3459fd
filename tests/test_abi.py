"""The C-ABI library without a GPU: it loads, exports every entry point that
include/qsa.h declares, and rejects bad arguments on the host before any HIP
call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import block_sparse_long_qsa_amd as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(Q.EXPORTS)


def _param_counts():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(qsa_[a-z_]+)\s*\(([^;{]*?)\)\s*;", src):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_header():
    lib = Q.lib()
    counts = _param_counts()
    assert counts, "no declarations parsed"
    for name, n in counts.items():
        argtypes = getattr(lib, name).argtypes
        assert argtypes is not None and len(argtypes) == n, (name, n, argtypes)


def test_library_exports_every_declared_symbol():
    lib = Q.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_default_params_are_the_layer_shapes():
    p = Q.default_params()
    assert (p.n_q_heads, p.n_kv_heads, p.head_dim, p.rope_dim) == (24, 2, 256, 64)
    assert (p.n_idx_heads, p.idx_dim, p.idx_rope_dim, p.block) == (4, 128, 64, 4)
    assert p.budget_blocks == 512 and p.rope_theta == 1e7 and p.yarn_orig_ctx == 262144


@pytest.mark.parametrize("field,value,status", [
    ("n_q_heads", 32, 3), ("head_dim", 128, 3), ("block", 8, 3), ("topk_cap", 1, 2), ("topk_cap", 9000, 2),
    ("budget_blocks", 0, 2), ("budget_blocks", 513, 2), ("max_ctx", 6, 2), ("max_ctx", 0, 2),
    ("yarn_factor", 0.5, 2), ("rope_theta", 0.0, 2)])
def test_create_rejects_bad_params_on_host(field, value, status):
    p = Q.default_params(**{field: value})
    h = ctypes.c_void_p(123)
    assert Q.lib().qsa_create(ctypes.byref(p), 0, ctypes.byref(h)) == status
    assert h.value is None


def test_null_handle_and_status_strings():
    lib = Q.lib()
    assert lib.qsa_create(None, 0, None) == 1
    assert lib.qsa_workspace_size(None, 4, 1, 10, 0) == 0
    assert lib.qsa_append(None, None, 1, 4, 0, *([None] * 7)) == 1
    assert lib.qsa_forward(None, None, 1, 4, 0, *([None] * 12), 0) == 1
    assert lib.qsa_index_select(None, None, 1, 4, 0, None, None, None, None, 0) == 1
    assert lib.qsa_attend(None, None, 1, 4, 0, None, None, None, None, None) == 1
    assert lib.qsa_decode(None, None, 1, None, 0, *([None] * 12), 0) == 1
    assert lib.qsa_decode_reuse(None, None, 1, None, None, 0, *([None] * 11), 0) == 1
    for s in range(8):
        assert Q.qsa_status_string(s)
    assert Q.qsa_last_hip_error() == 0
    lib.qsa_destroy(None)


def test_no_cpu_fallback_in_binding():
    src = open(os.path.join(ROOT, "block_sparse_long_qsa_amd", "__init__.py")).read()
    assert "oracle" not in src and "import synth" not in src


def test_gdn_workspace_size():
    # Tb and P per (sequence, V head, chunk of 64) and K^T per (sequence, QK head, chunk): 16 KiB each.
    assert Q.qsa_gdn_workspace_size(1, 64, 16, 48) == (48 + 16) * 16384
    assert Q.qsa_gdn_workspace_size(2, 65, 16, 48) == 2 * 2 * (48 + 16) * 16384
    assert Q.qsa_gdn_workspace_size(1, 0, 16, 48) == 0
    assert Q.qsa_gdn_workspace_size(0, 64, 16, 48) == 0


def _gdn_call(nseq=1, cu=16, n_tok=64, max_len=64, hq=2, hv=6, q=16, k=16, v=16, g=16, beta=16, o=16, ws=16,
              ws_bytes=None):
    lib = Q.lib()
    if ws_bytes is None:
        ws_bytes = lib.qsa_gdn_workspace_size(nseq, max_len, hq, hv)
    # Pointer values are never dereferenced: every case fails a host check first.
    return lib.qsa_gdn_chunk_prefill(None, nseq, cu, n_tok, max_len, hq, hv, 0.1, q, k, v, g, beta, None, o, None,
                                     ws, ws_bytes)


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), 1), (dict(q=None), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(ws=None), 1),
    (dict(nseq=0), 2), (dict(nseq=70000), 2), (dict(n_tok=-1), 2), (dict(max_len=-1), 2), (dict(hq=0), 2),
    (dict(hv=5), 2), (dict(hv=1), 2), (dict(q=24), 4), (dict(k=8), 4), (dict(ws=8), 4), (dict(ws_bytes=100), 6),
])
def test_gdn_rejects_bad_arguments_on_the_host(kw, status):
    assert _gdn_call(**kw) == status


def test_binding_rejects_host_tensors():
    """The binding hands only addresses to the library, so it refuses a host
    tensor (its address is not a device address) before any call."""
    import torch
    with pytest.raises(ValueError, match="device tensor"):
        Q._ptr(torch.zeros(16, dtype=torch.float32), torch.float32, "x")
    with pytest.raises(ValueError, match="device tensor"):
        Q._bf(torch.zeros(16, dtype=torch.bfloat16), "q")
    assert Q._ptr(None) is None


def test_probe_library_exports_its_header_and_checks_arguments():
    """The benchmark's gather probe (include/qsa_probe.h, libqsa_probe.so):
    every declared symbol is exported, the binding passes the declared number
    of arguments, and bad arguments are refused before any HIP call."""
    from block_sparse_long_qsa_amd import probe
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qsa_probe.h")).read(), flags=re.S)
    decls = re.findall(r"\b(qsa_[a-z_]+)\s*\(([^;{]*?)\)\s*;", src)
    assert [d[0] for d in decls] == ["qsa_probe_gather"]
    lib = probe.lib()
    assert len(lib.qsa_probe_gather.argtypes) == decls[0][1].count(",") + 1
    ok = dict(stream=None, k=16, v=16, gs=2048, nb=1, idx=16, rows=1, ll=8, lr=4096, step=8, pad=0, sink=16)
    def call(**kw):
        a = {**ok, **kw}
        return lib.qsa_probe_gather(a["stream"], a["k"], a["v"], a["gs"], a["nb"], a["idx"], a["rows"], a["ll"],
                                    a["lr"], a["step"], a["pad"], a["sink"])
    for kw in (dict(k=None), dict(v=None), dict(idx=None), dict(sink=None), dict(rows=-1), dict(ll=-1),
               dict(lr=0), dict(nb=0), dict(step=3), dict(step=16), dict(pad=32)):
        assert call(**kw) == 1, kw


def test_create_without_a_gpu_builds_tables_then_reports_hip():
    """Valid parameters on a machine with no usable GPU: the host rotary tables
    are built (1,048,576 positions, YaRN 4), then the device step fails with
    QSA_ERR_HIP and a recorded HIP code, and no handle is returned."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    p = Q.default_params(max_ctx=1 << 20, yarn_factor=4.0)
    h = ctypes.c_void_p(123)
    assert Q.lib().qsa_create(ctypes.byref(p), 0, ctypes.byref(h)) == 7
    assert h.value is None and Q.qsa_last_hip_error() != 0
