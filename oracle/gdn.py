"""Gated DeltaNet oracle -- TEST INFRASTRUCTURE.

Same rules as the package: only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it; it shares no code with the
HIP library.  fp64, one token at a time.

Source: [PKR] (see the package docstring):
  * section "어텐션: GDN이 기억하고 QSA가 찾아낸다": the gated delta rule
        S_t = (alpha_t I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
    alpha_t in (0, 1) a decay gate, beta_t in (0, 1) the strength of the delta
    write (the value stored under k_t is estimated first and only the error is
    written);
  * spec table: 48 V heads, 16 QK heads, head dim 128;
  * section on FlashQLA: the chunked-prefill interface -- q, k [B, T, H_q, K],
    v [B, T, H_v, V], g and beta [B, T, H_v], a scale, an optional initial
    state [B, H_v, K, V], the final state returned.

Readings (not fixed by the pages): alpha_t = exp(g_t) (g is the gate in log
space, as the interface's name suggests); V head h reads QK head
h // (H_v / H_q); the output of token t is scale * S_t^T q_t (the read-out after
the update); q and k arrive already normalised (the model's short convolution
and L2 norm precede the kernel).

Parity status: pinned by tests/test_oracle_gdn_pins.py (closed forms with no
write, with orthonormal keys and with a rewritten key; linearity).
"""
from __future__ import annotations

import numpy as np


def gdn_recurrent(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray, scale: float,
                  s0: np.ndarray = None):
    """One sequence.  q, k [T][Hq][K]; v [T][Hv][V]; g, beta [T][Hv]; s0
    [Hv][K][V] or None (zeros).  Returns (o [T][Hv][V], S_T [Hv][K][V]),
    fp64."""
    T, Hq, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    rep = Hv // Hq
    heads = np.arange(Hv) // rep
    S = np.zeros((Hv, K, V)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.empty((T, Hv, V))
    for t in range(T):
        kt = k[t][heads].astype(np.float64)                  # [Hv][K]
        qt = q[t][heads].astype(np.float64)
        a = np.exp(g[t].astype(np.float64))[:, None, None]
        b = beta[t].astype(np.float64)[:, None, None]
        ks = np.einsum("hk,hkv->hv", kt, S)                  # value stored under k_t
        S = a * S - b * kt[:, :, None] * ks[:, None, :] + b * kt[:, :, None] * v[t].astype(np.float64)[:, None, :]
        o[t] = scale * np.einsum("hk,hkv->hv", qt, S)
    return o, S
