"""The chunked (WY / UT transform) form of the gated delta rule, in plain numpy fp64,
against the token-by-token oracle.

This is the algorithm the GPU kernels implement (not their code: this file shares
nothing with them).  For a chunk of n rows entering with state S_0 (d_v x d_k):

  g_t   = sum_{i<=t} log a_i                         (within the chunk)
  A_ts  = b_t exp(g_t - g_s) k_t . k_s,  s < t        (strictly lower)
  T     = (I + A)^-1
  R     = diag(b) (V - diag(exp g) K S_0^T)
  Delta = T R                (row t is b_t (v_t - a_t S_{t-1} k_t))
  O     = scale (diag(exp g) Q S_0^T + (M o Q K^T) Delta),  M_ts = exp(g_t - g_s), s <= t
  S_n   = exp(g_n) S_0 + Delta^T diag(exp(g_n - g)) K

The chunk grid splits a sequence at every multiple of the chunk size, every multiple
of the cache block, and at both call ends, with positions counted from the start of
the sequence, so every crossed block boundary ends a chunk ("The prefix cache changed
the answer", section "The fix: one line").
"""
import numpy as np
import pytest

from oracle import oracle


def chunk_grid(p0, L, C, block):
    cuts = {p0, p0 + L}
    x = (p0 // C + 1) * C
    while x < p0 + L:
        cuts.add(x)
        x += C
    if block:
        x = (p0 // block + 1) * block
        while x < p0 + L:
            cuts.add(x)
            x += block
    cuts = sorted(cuts)
    return [(cuts[i], cuts[i + 1]) for i in range(len(cuts) - 1)]


def chunked(q, k, v, a, b, scale, S0, p0, block, C):
    L, Hqk, dk = k.shape
    Hv, dv = v.shape[1:]
    grp = Hv // Hqk
    o = np.zeros((L, Hv, dv))
    S = np.zeros((Hv, dv, dk)) if S0 is None else S0.copy()
    ckpts = []
    for (x0, x1) in chunk_grid(p0, L, C, block):
        r0, r1 = x0 - p0, x1 - p0
        n = r1 - r0
        for h in range(Hv):
            K = k[r0:r1, h // grp]
            Q = q[r0:r1, h // grp]
            V = v[r0:r1, h]
            bb = b[r0:r1, h]
            g = np.cumsum(np.log(a[r0:r1, h]))
            D = np.exp(g[:, None] - g[None, :])
            A = np.tril(bb[:, None] * D * (K @ K.T), -1)
            T = np.linalg.solve(np.eye(n) + A, np.eye(n))
            R = bb[:, None] * (V - np.exp(g)[:, None] * (K @ S[h].T))
            Delta = T @ R
            P = np.tril(D * (Q @ K.T))
            o[r0:r1, h] = scale * (np.exp(g)[:, None] * (Q @ S[h].T) + P @ Delta)
            S[h] = np.exp(g[-1]) * S[h] + (Delta * np.exp(g[-1] - g)[:, None]).T @ K
        if block and x1 % block == 0:
            ckpts.append(S.copy())
    return o, S, np.array(ckpts).reshape(-1, Hv, dv, dk)


def _inputs(L, Hqk, Hv, d, seed):
    r = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(r.standard_normal((L, Hqk, d)))
    k = unit(r.standard_normal((L, Hqk, d)))
    v = r.standard_normal((L, Hv, d))
    a = np.exp(-np.log1p(np.exp(r.standard_normal((L, Hv)))) * 0.1)
    b = 1 / (1 + np.exp(-r.standard_normal((L, Hv))))
    return q, k, v, a, b


def test_grid_rule():
    assert chunk_grid(0, 64, 64, 16) == [(0, 16), (16, 32), (32, 48), (48, 64)]
    assert chunk_grid(0, 200, 64, 896) == [(0, 64), (64, 128), (128, 192), (192, 200)]
    g = chunk_grid(700, 200, 64, 784)
    assert g == [(700, 704), (704, 768), (768, 784), (784, 832), (832, 896), (896, 900)]
    # every crossed block boundary ends a chunk
    for (x0, x1) in chunk_grid(100, 5000, 64, 784):
        assert (x0 // 784) == ((x1 - 1) // 784)


@pytest.mark.parametrize("p0,L,C,block,d,Hqk,Hv", [
    (0, 64, 64, 16, 16, 2, 2),        # tiny workload grid: four 16-token chunks
    (0, 200, 64, 0, 8, 1, 2),         # ragged tail, value heads sharing a key head
    (700, 260, 64, 784, 8, 2, 2),     # 784-token blocks, off the 64-grid
    (32, 150, 32, 48, 6, 1, 1),       # start on a boundary, small chunks
    (0, 97, 64, 0, 5, 1, 3),
])
def test_chunked_form_matches_token_loop(p0, L, C, block, d, Hqk, Hv):
    q, k, v, a, b = _inputs(L, Hqk, Hv, d, 100 + L)
    S0 = None if p0 == 0 else 0.3 * np.random.default_rng(1).standard_normal((Hv, d, d))
    o_ref, S_ref, ck_ref = oracle.recurrence(q, k, v, a, b, 0.9, S0, p0=p0, block=block)
    o, S, ck = chunked(q, k, v, a, b, 0.9, S0, p0, block, C)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12)
    assert ck.shape == ck_ref.shape
    np.testing.assert_allclose(ck, ck_ref, rtol=0, atol=1e-12)


def test_delta_rows_are_the_token_corrections():
    """Row t of Delta is b_t (v_t - a_t S_{t-1} k_t): compare with the token loop."""
    L, d = 20, 6
    q, k, v, a, b = _inputs(L, 1, 1, d, 7)
    S0 = np.random.default_rng(8).standard_normal((1, d, d))
    g = np.cumsum(np.log(a[:, 0]))
    K, V, bb = k[:, 0], v[:, 0], b[:, 0]
    A = np.tril(bb[:, None] * np.exp(g[:, None] - g[None, :]) * (K @ K.T), -1)
    R = bb[:, None] * (V - np.exp(g)[:, None] * (K @ S0[0].T))
    Delta = np.linalg.solve(np.eye(L) + A, R)
    S = S0.copy()
    for t in range(L):
        want = b[t, 0] * (v[t, 0] - a[t, 0] * S[0] @ k[t, 0])
        np.testing.assert_allclose(Delta[t], want, atol=1e-12)
        _, S, _ = oracle.recurrence(None, k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], 1.0, S,
                                    want_o=False)
