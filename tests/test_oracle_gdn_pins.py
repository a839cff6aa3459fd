"""Pins of the Gated DeltaNet oracle (oracle/gdn.py) against closed forms it
does not compute itself.  CPU only."""
import numpy as np

from oracle import gdn as G


def test_no_write_is_pure_decay():
    """beta = 0: the state only decays, o_t = scale * (prod_{i<=t} alpha_i) S0^T q_t."""
    rng = np.random.default_rng(1)
    T, Hq, Hv, K, V = 7, 2, 4, 5, 3
    q, k = rng.standard_normal((T, Hq, K)), rng.standard_normal((T, Hq, K))
    v = rng.standard_normal((T, Hv, V))
    g = -rng.random((T, Hv))
    s0 = rng.standard_normal((Hv, K, V))
    o, S = G.gdn_recurrent(q, k, v, g, np.zeros((T, Hv)), 0.5, s0)
    dec = np.exp(np.cumsum(g, axis=0))                       # [T][Hv]
    for t in range(T):
        for h in range(Hv):
            ref = 0.5 * dec[t, h] * s0[h].T @ q[t, h // 2]
            assert np.allclose(o[t, h], ref, atol=1e-12)
    assert np.allclose(S, dec[-1][:, None, None] * s0, atol=1e-12)


def test_orthonormal_keys_store_every_value():
    """alpha = 1, beta = 1, keys e_0, e_1, ...: each step writes v_t under e_t
    exactly, so o_t = scale * sum_{j<=t} q_t[j] v_j."""
    rng = np.random.default_rng(2)
    T, K, V = 6, 8, 4
    k = np.zeros((T, 1, K))
    for t in range(T):
        k[t, 0, t] = 1.0
    q = rng.standard_normal((T, 1, K))
    v = rng.standard_normal((T, 1, V))
    o, S = G.gdn_recurrent(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), 1.0)
    for t in range(T):
        ref = sum(q[t, 0, j] * v[j, 0] for j in range(t + 1))
        assert np.allclose(o[t, 0], ref, atol=1e-12)
    assert np.allclose(S[0][:T], v[:, 0], atol=1e-12) and np.allclose(S[0][T:], 0.0)


def test_rewriting_a_key_replaces_its_value():
    """alpha = 1, beta = 1, a unit key written twice: the second write replaces
    the first (the delta rule erases before it writes); with beta = 1/2 the
    stored value moves halfway."""
    K, V = 4, 3
    e = np.zeros(K)
    e[2] = 1.0
    k = np.stack([e, e])[:, None, :]
    q = np.stack([e, e])[:, None, :]
    v = np.array([[[1.0, 2.0, 3.0]], [[-4.0, 0.5, 7.0]]])
    o, S = G.gdn_recurrent(q, k, v, np.zeros((2, 1)), np.ones((2, 1)), 1.0)
    assert np.allclose(o[1, 0], v[1, 0]) and np.allclose(S[0][2], v[1, 0])
    o, S = G.gdn_recurrent(q, k, v, np.zeros((2, 1)), np.full((2, 1), 0.5), 1.0)
    assert np.allclose(S[0][2], 0.5 * (0.5 * v[0, 0]) + 0.5 * v[1, 0])


def test_linear_in_values_and_initial_state():
    """For fixed q, k, gates: (v, S0) -> (o, S_T) is linear."""
    rng = np.random.default_rng(3)
    T, Hq, Hv, K, V = 9, 1, 3, 6, 5
    q, k = rng.standard_normal((T, Hq, K)), rng.standard_normal((T, Hq, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g, beta = -rng.random((T, Hv)), rng.random((T, Hv))
    v1, v2 = rng.standard_normal((T, Hv, V)), rng.standard_normal((T, Hv, V))
    s1, s2 = rng.standard_normal((Hv, K, V)), rng.standard_normal((Hv, K, V))
    o1, S1 = G.gdn_recurrent(q, k, v1, g, beta, 0.3, s1)
    o2, S2 = G.gdn_recurrent(q, k, v2, g, beta, 0.3, s2)
    o3, S3 = G.gdn_recurrent(q, k, 2 * v1 - v2, g, beta, 0.3, 2 * s1 - s2)
    assert np.allclose(o3, 2 * o1 - o2, atol=1e-10) and np.allclose(S3, 2 * S1 - S2, atol=1e-10)
