"""Pins of the fp64 CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against a closed form, an invariant of the mathematics,
a brute-force evaluation of the product form, or a number the pages print.  A
plausible mistake in the oracle (a dropped term, a wrong sign or index, a transposed
operand, an off-by-one checkpoint) fails at least one of them; test_mutants.py checks
that claim by compiling mutated copies of the oracle.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(L, Hqk, Hv, d, seed, a_range=(0.6, 1.0)):
    r = rng(seed)
    q = _unit(r.standard_normal((L, Hqk, d)))
    k = _unit(r.standard_normal((L, Hqk, d)))
    v = r.standard_normal((L, Hv, d))
    a = r.uniform(*a_range, size=(L, Hv))
    b = r.uniform(0.0, 1.0, size=(L, Hv))
    return q, k, v, a, b


# ---------------------------------------------------------------- recurrence pins

def test_identity_gate_leaves_state_unchanged():
    """a = 1, b = 0: the update is the identity and o_t = scale * S_0 q_t."""
    L, H, d = 9, 3, 8
    q, k, v, _, _ = _inputs(L, H, H, d, 1)
    S0 = rng(2).standard_normal((H, d, d))
    o, S, _ = oracle.recurrence(q, k, v, np.ones((L, H)), np.zeros((L, H)), 0.7, S0)
    assert np.array_equal(S, S0)
    want = 0.7 * np.einsum("hij,thj->thi", S0, q)
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-14)


def test_pure_decay_closed_form():
    """b = 0: S_t = (prod_{i<=t} a_i) S_0, so o_t = scale * prod a * S_0 q_t."""
    L, H, d = 12, 2, 5
    q, k, v, a, _ = _inputs(L, H, H, d, 3)
    S0 = rng(4).standard_normal((H, d, d))
    o, S, _ = oracle.recurrence(q, k, v, a, np.zeros((L, H)), 1.0, S0)
    decay = np.cumprod(a, axis=0)  # [L, H]
    np.testing.assert_allclose(S, decay[-1][:, None, None] * S0, rtol=1e-13)
    want = decay[:, :, None] * np.einsum("hij,thj->thi", S0, q)
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-14)


def test_full_write_recalls_value():
    """a = 1, b = 1, unit keys: right after writing (k_t, v_t) the memory returns v_t for
    k_t, so a query equal to the key reads back the value (o_t uses the updated state)."""
    L, H, d = 10, 2, 6
    _, k, v, _, _ = _inputs(L, H, H, d, 5)
    S0 = rng(6).standard_normal((H, d, d))
    o, S, _ = oracle.recurrence(k, k, v, np.ones((L, H)), np.ones((L, H)), 1.0, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.einsum("hij,hj->hi", S, k[-1]), v[-1], atol=1e-12)


def test_orthonormal_keys_closed_form():
    """a = 1, b = 1, orthonormal keys k_1..k_T: S_T = S_0 (I - sum k k^T) + sum v k^T."""
    d, H = 8, 2
    L = 5
    r = rng(7)
    k = np.empty((L, H, d))
    for h in range(H):
        Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
        k[:, h, :] = Qm[:, :L].T
    v = r.standard_normal((L, H, d))
    S0 = r.standard_normal((H, d, d))
    _, S, _ = oracle.recurrence(None, k, v, np.ones((L, H)), np.ones((L, H)), 1.0, S0, want_o=False)
    for h in range(H):
        P = k[:, h, :].T @ k[:, h, :]
        want = S0[h] @ (np.eye(d) - P) + v[:, h, :].T @ k[:, h, :]
        np.testing.assert_allclose(S[h], want, atol=1e-12)


def test_interpolation_and_orthogonal_invariance():
    """For a unit key, the new memory read at k_t is a(1-b) S_{t-1} k_t + b v_t, and any
    direction u orthogonal to k_t only decays: S_t u = a S_{t-1} u."""
    L, H, d = 6, 2, 7
    q, k, v, a, b = _inputs(L, H, H, d, 8)
    S = rng(9).standard_normal((H, d, d))
    r = rng(10)
    for t in range(L):
        _, S_new, _ = oracle.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1],
                                        b[t:t + 1], 1.0, S)
        for h in range(H):
            kt = k[t, h]
            want = a[t, h] * (1 - b[t, h]) * (S[h] @ kt) + b[t, h] * v[t, h]
            np.testing.assert_allclose(S_new[h] @ kt, want, atol=1e-12)
            u = r.standard_normal(d)
            u -= (u @ kt) * kt
            np.testing.assert_allclose(S_new[h] @ u, a[t, h] * (S[h] @ u), atol=1e-12)
        S = S_new


def test_matches_literal_product_form():
    """The oracle's three-step update equals the literal product form
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = scale S_t q_t,
    evaluated by brute force with dense matrices (non-unit keys, dk != dv)."""
    L, H, dk, dv = 7, 2, 5, 3
    r = rng(11)
    q = r.standard_normal((L, H, dk))
    k = r.standard_normal((L, H, dk)) * 0.6
    v = r.standard_normal((L, H, dv))
    a = r.uniform(0.3, 1.0, (L, H))
    b = r.uniform(0.0, 1.0, (L, H))
    S0 = r.standard_normal((H, dv, dk))
    o, S, _ = oracle.recurrence(q, k, v, a, b, 1.3, S0)
    for h in range(H):
        St = S0[h].copy()
        for t in range(L):
            kt = k[t, h][:, None]
            St = a[t, h] * St @ (np.eye(dk) - b[t, h] * kt @ kt.T) + b[t, h] * v[t, h][:, None] @ kt.T
            np.testing.assert_allclose(o[t, h], 1.3 * St @ q[t, h], atol=1e-12)
        np.testing.assert_allclose(S[h], St, atol=1e-12)


def test_scalar_case_brute_force():
    """d_k = d_v = 1 reduces to s_t = a_t s_{t-1} (1 - b_t k_t^2) + b_t v_t k_t."""
    L = 20
    r = rng(12)
    q, k, v = (r.standard_normal((L, 1, 1)) for _ in range(3))
    a = r.uniform(0.5, 1, (L, 1))
    b = r.uniform(0, 1, (L, 1))
    o, S, _ = oracle.recurrence(q, k, v, a, b, 1.0, np.array([[[0.3]]]))
    s = 0.3
    for t in range(L):
        s = a[t, 0] * s * (1 - b[t, 0] * k[t, 0, 0] ** 2) + b[t, 0] * v[t, 0, 0] * k[t, 0, 0]
        assert o[t, 0, 0] == pytest.approx(s * q[t, 0, 0], abs=1e-13)
    assert S[0, 0, 0] == pytest.approx(s, abs=1e-13)


def test_affine_in_initial_state():
    """For fixed inputs the map S_0 -> S_T is affine: f(x S_a + (1-x) S_b) = x f(S_a) + (1-x) f(S_b)."""
    L, H, d = 15, 2, 6
    q, k, v, a, b = _inputs(L, H, H, d, 13)
    Sa, Sb = rng(14).standard_normal((2, H, d, d))
    x = 0.3
    oa, fa, _ = oracle.recurrence(q, k, v, a, b, 1.0, Sa)
    ob, fb, _ = oracle.recurrence(q, k, v, a, b, 1.0, Sb)
    om, fm, _ = oracle.recurrence(q, k, v, a, b, 1.0, x * Sa + (1 - x) * Sb)
    np.testing.assert_allclose(fm, x * fa + (1 - x) * fb, atol=1e-12)
    np.testing.assert_allclose(om, x * oa + (1 - x) * ob, atol=1e-12)


def test_zero_state_source_equals_explicit_zeros():
    L, H, d = 5, 2, 4
    q, k, v, a, b = _inputs(L, H, H, d, 15)
    o1, S1, _ = oracle.recurrence(q, k, v, a, b, 1.0, None)
    o2, S2, _ = oracle.recurrence(q, k, v, a, b, 1.0, np.zeros((H, d, d)))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_value_heads_share_query_key_heads():
    """With Hv = 3 Hqk, value head h reads query/key head h // 3: same as repeating q, k."""
    L, Hqk, Hv, d = 8, 2, 6, 4
    q, k, v, a, b = _inputs(L, Hqk, Hv, d, 16)
    o1, S1, _ = oracle.recurrence(q, k, v, a, b, 1.0, None)
    qr, kr = np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1)
    o2, S2, _ = oracle.recurrence(qr, kr, v, a, b, 1.0, None)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# ---------------------------------------------------------------- checkpoints / resume

def test_checkpoints_are_prefix_states():
    """The checkpoint at block boundary p*block is the state after exactly p*block tokens."""
    L, H, d, block = 64, 2, 4, 16
    q, k, v, a, b = _inputs(L, H, H, d, 17)
    _, _, ck = oracle.recurrence(q, k, v, a, b, 1.0, None, p0=0, block=block)
    assert ck.shape[0] == 4
    for p in range(1, 5):
        n = p * block
        _, Sp, _ = oracle.recurrence(q[:n], k[:n], v[:n], a[:n], b[:n], 1.0, None)
        assert np.array_equal(ck[p - 1], Sp)


def test_checkpoint_count_and_offset_start():
    """Boundaries are absolute: a call starting at 20 with 50 tokens on 16-blocks crosses
    32, 48 and 64, i.e. after 12, 28 and 44 of its tokens."""
    L, H, d = 50, 1, 3
    q, k, v, a, b = _inputs(L, H, H, d, 18)
    S0 = rng(19).standard_normal((H, d, d))
    _, _, ck = oracle.recurrence(q, k, v, a, b, 1.0, S0, p0=20, block=16)
    assert ck.shape[0] == 3
    for i, n in enumerate((12, 28, 44)):
        _, Sn, _ = oracle.recurrence(q[:n], k[:n], v[:n], a[:n], b[:n], 1.0, S0)
        assert np.array_equal(ck[i], Sn)


def test_resume_from_checkpoint_equals_cold_run():
    L, H, d, block = 64, 2, 16, 16
    q, k, v, a, b = _inputs(L, H, H, d, 20)
    o, S, ck = oracle.recurrence(q, k, v, a, b, 1.0, None, p0=0, block=block)
    s = 32
    o2, S2, ck2 = oracle.recurrence(q[s:], k[s:], v[s:], a[s:], b[s:], 1.0, ck[1], p0=s, block=block)
    assert np.array_equal(o2, o[s:]) and np.array_equal(S2, S)
    assert np.array_equal(ck2, ck[2:])


def test_flush_equals_sequential_application_and_ignores_rejected_rows():
    """Folding n accepted rows at once equals n single-token updates; rows past n are
    never read, so NaN there changes nothing."""
    n, rows, H, d = 5, 8, 2, 6
    q, k, v, a, b = _inputs(rows, H, H, d, 21)
    k[n:] = np.nan
    v[n:] = np.nan
    a[n:] = np.nan
    S = rng(22).standard_normal((H, d, d))
    _, Sf, _ = oracle.recurrence(None, k[:n], v[:n], a[:n], b[:n], 1.0, S, want_o=False)
    St = S
    for t in range(n):
        _, St, _ = oracle.recurrence(None, k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], 1.0,
                                     St, want_o=False)
    assert np.array_equal(Sf, St)
    assert np.isfinite(Sf).all()


def test_replay_outputs_fold_the_log_then_read_the_new_rows():
    """Replay outputs from (state, log of m rows, n new rows) equal folding the m logged
    rows into the state first and then running the n new rows with their queries; log
    rows past m + n are never read."""
    m, n, rows, Hqk, Hv, d = 6, 4, 13, 1, 2, 5
    q, k, v, a, b = _inputs(rows, Hqk, Hv, d, 24)
    k[m + n:] = np.nan
    v[m + n:] = np.nan
    a[m + n:] = np.nan
    b[m + n:] = np.nan
    S = rng(25).standard_normal((Hv, d, d))
    o = oracle.replay_outputs(S, k, v, a, b, m, q[m:m + n], 0.7)
    _, Sm, _ = oracle.recurrence(None, k[:m], v[:m], a[:m], b[:m], 1.0, S, want_o=False)
    o2, _, _ = oracle.recurrence(q[m:m + n], k[m:m + n], v[m:m + n], a[m:m + n], b[m:m + n], 0.7, Sm)
    assert o.shape == (n, Hv, d)
    assert np.array_equal(o, o2)
    assert np.isfinite(o).all()


def test_replay_outputs_overwrite_closed_form():
    """a = b = 1 with one-hot keys: each row replaces one column of the state with its
    value (S <- S + (v - S k) k^T), so after log row t the state is S0 with the columns
    of rows 0..t overwritten in order; the output of new row i is scale times that
    state applied to its query."""
    m, n, d, scale = 3, 3, 6, 0.5
    cols = [4, 1, 4, 0, 2, 1]   # column 4 and column 1 are written twice
    r = rng(26)
    S0 = r.standard_normal((1, d, d))
    k = np.zeros((m + n, 1, d))
    for t, c in enumerate(cols):
        k[t, 0, c] = 1.0
    v = r.standard_normal((m + n, 1, d))
    a = np.ones((m + n, 1))
    b = np.ones((m + n, 1))
    qn = r.standard_normal((n, 1, d))
    o = oracle.replay_outputs(S0, k, v, a, b, m, qn, scale)
    St = S0[0].copy()
    want = []
    for t, c in enumerate(cols):
        St[:, c] = v[t, 0]
        if t >= m:
            want.append(scale * St @ qn[t - m, 0])
    assert np.allclose(o[:, 0], np.array(want), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- packed-core steps

def test_l2norm_qk_heads_hand_values():
    """A 3-4-5 head becomes (0.6, 0.8); value channels pass unchanged; a zero head stays 0."""
    y = np.array([[3.0, 4.0, 0.0, -2.5, 7.0, -2.0]])     # Hqk = 1, d = 2: q, k heads, then v
    out = oracle.l2norm_qk_heads(y, 1, 2, eps=0.0)
    assert np.array_equal(out[0, :4], [0.6, 0.8, 0.0, -1.0])
    assert np.array_equal(out[0, 4:], [7.0, -2.0])
    y[0, 2:4] = 0.0
    out = oracle.l2norm_qk_heads(y, 1, 2, eps=1e-6)
    assert np.array_equal(out[0, 2:4], [0.0, 0.0])
    assert abs(out[0, 0] - 3.0 / np.sqrt(25.0 + 1e-6)) == 0.0


def test_l2norm_qk_heads_unit_norm_and_direction():
    r = rng(27)
    y = r.standard_normal((5, 2 * 3 * 8 + 16)) * 4.0
    out = oracle.l2norm_qk_heads(y, 3, 8)
    h = out[:, :48].reshape(5, 6, 8)
    assert np.allclose(np.linalg.norm(h, axis=2), 1.0, atol=1e-7)
    hy = y[:, :48].reshape(5, 6, 8)
    cos = (h * hy).sum(axis=2) / np.linalg.norm(hy, axis=2)
    assert np.allclose(cos, 1.0, atol=1e-12)
    assert np.array_equal(out[:, 48:], y[:, 48:])


def test_gates_hand_values():
    """At zero inputs softplus is log 2: a = exp(-log 2) = 1/2 and b = sigmoid(0) = 1/2;
    with A_log = log 2 the decay doubles in log space, a = 1/4; large negative inputs
    give no decay and large positive b inputs full write strength."""
    Hv = 2
    ba = np.zeros((1, 2 * Hv))
    a, b = oracle.gates(ba, np.array([0.0, np.log(2.0)]), np.zeros(Hv), Hv)
    assert np.allclose(a, [[0.5, 0.25]], rtol=1e-15, atol=0) and np.array_equal(b, [[0.5, 0.5]])
    ba = np.array([[40.0, -3.0, -60.0, 1.5]])
    a, b = oracle.gates(ba, np.array([0.0, 0.0]), np.array([0.0, -1.5]), Hv)
    assert a[0, 0] == 1.0 and np.isclose(a[0, 1], 0.5, rtol=1e-15)   # softplus(0) for head 1
    assert b[0, 0] == 1.0 and np.isclose(b[0, 1], 1.0 / (1.0 + np.exp(3.0)), rtol=1e-15)
    # a decay past fp32's normal range stops at 2^-126: exp(-16 * 10) ~ 1e-70
    a, _ = oracle.gates(np.array([[0.0, 10.0]]), np.array([np.log(16.0)]), np.zeros(1), 1)
    assert a[0, 0] == 2.0 ** -126


def test_gated_norm_hand_values_and_scale_invariance():
    """o = (3, 4): mean square 12.5, so the normalized row is (3, 4) / sqrt(12.5); a zero
    gate input gives silu(0) = 0; scaling o leaves the output unchanged (eps = 0)."""
    o = np.array([[3.0, 4.0]])
    z = np.array([[1.0, 0.0]])
    w = np.array([2.0, 5.0])
    out = oracle.gated_norm(o, z, w, eps=0.0)
    silu1 = 1.0 / (1.0 + np.exp(-1.0))
    assert np.isclose(out[0, 0], 3.0 / np.sqrt(12.5) * 2.0 * silu1, rtol=1e-15) and out[0, 1] == 0.0
    r = rng(28)
    o = r.standard_normal((4, 3, 16))
    z = r.standard_normal((4, 3, 16))
    w = r.standard_normal(16)
    assert np.allclose(oracle.gated_norm(7.0 * o, z, w, eps=0.0), oracle.gated_norm(o, z, w, eps=0.0), rtol=1e-13)


# ---------------------------------------------------------------- conv

def test_conv_identity_taps():
    r = rng(23)
    x = r.standard_normal((10, 5))
    w = np.tile([0.0, 0.0, 0.0, 1.0], (5, 1))
    y, tail, _ = oracle.conv(x, w, None, act=0)
    assert np.array_equal(y, x)
    assert np.array_equal(tail, x[-3:])


def test_conv_impulse_response_reads_taps_in_time_order():
    """An impulse at token t0 gives y[t0 + m] = w[W-1-m]: the last tap multiplies the
    current token, the first tap the token W-1 steps back."""
    C, L, t0 = 3, 9, 2
    x = np.zeros((L, C))
    x[t0] = 1.0
    w = rng(24).standard_normal((C, 4))
    y, _, _ = oracle.conv(x, w, None, act=0)
    for m in range(4):
        np.testing.assert_array_equal(y[t0 + m], w[:, 3 - m])
    assert not y[:t0].any() and not y[t0 + 4:].any()


def test_conv_silu_values():
    x = np.array([[0.0], [2.0], [-3.0]])
    w = np.array([[0.0, 0.0, 0.0, 1.0]])
    y, _, _ = oracle.conv(x, w, None, act=1)
    np.testing.assert_allclose(y[:, 0], [0.0, 2.0 / (1 + np.exp(-2.0)), -3.0 / (1 + np.exp(3.0))],
                               rtol=1e-15)


def test_conv_split_call_equals_single_call_and_ckpt_tails():
    r = rng(25)
    L, C = 40, 6
    x = r.standard_normal((L, C))
    w = r.standard_normal((C, 4))
    tail0 = r.standard_normal((3, C))
    y, tail, ck = oracle.conv(x, w, tail0, act=1, p0=5, block=16)
    y1, t1, ck1 = oracle.conv(x[:17], w, tail0, act=1, p0=5, block=16)
    y2, t2, ck2 = oracle.conv(x[17:], w, t1, act=1, p0=22, block=16)
    assert np.array_equal(np.concatenate([y1, y2]), y) and np.array_equal(t2, tail)
    # boundaries at absolute 16 and 32 -> call tokens 11 and 27
    assert ck.shape[0] == 2
    assert np.array_equal(ck[0], x[8:11]) and np.array_equal(ck[1], x[24:27])
    assert np.array_equal(np.concatenate([ck1, ck2]), ck)


def test_conv_tail_shorter_than_window():
    """With fewer tokens than the window, the new tail keeps the older tail rows."""
    r = rng(26)
    x = r.standard_normal((2, 4))
    w = r.standard_normal((4, 4))
    tail0 = r.standard_normal((3, 4))
    _, tail, _ = oracle.conv(x, w, tail0, act=0)
    assert np.array_equal(tail, np.concatenate([tail0[2:], x]))


# ---------------------------------------------------------------- page figures

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_prefix_accounting_matches_pages():
    g = _golden("prefix_accounting.json")
    for c in g["cached_prefix"]:
        assert oracle.cached_prefix_tokens(c["shared"], c["block"]) == c["cached"], c["source"]
    for c in g["floor_chunk"]:
        assert oracle.floor_chunk(c["budget"], c["block"]) == c["chunk"], c["source"]
    for c in g["checkpoint_positions"]:
        n = oracle.count_boundaries(c["start"], c["tokens"], c["block"])
        assert n == len(c["positions"]), c["source"]


def test_boundary_counts_of_the_workloads():
    assert oracle.count_boundaries(0, 64, 16) == 4
    assert oracle.count_boundaries(0, 8192, 896) == 9
    assert oracle.count_boundaries(0, 229376, 896) == 256
    assert oracle.count_boundaries(1792, 12000 - 1792, 896) == 11


# ---------------------------------------------------------------- bf16 rounding
# Every bf16-typed expected value (conv outputs, conv + norm, gated norm) is the oracle's
# fp64 result passed through oracle.bf16_round.  These pins fix that rounding to
# round-to-nearest with ties to even on 8 significant bits (bf16 keeps fp32's exponent
# range, subnormals included), independently of how the oracle implements it.

def _bf16_exact(x: float) -> float:
    """Nearest bf16 to x by exact rational arithmetic, ties to even; inf past the
    largest finite bf16 (round-to-nearest overflow rule)."""
    from fractions import Fraction
    import math
    if x == 0 or math.isinf(x) or math.isnan(x):
        return x
    s = -1.0 if x < 0 else 1.0
    fx = Fraction(abs(x))
    e = max(math.frexp(abs(x))[1] - 1, -126)       # exponent of the leading bit, clamped to normal range
    quantum = Fraction(2) ** (e - 7)               # spacing of bf16 values at this exponent
    m = fx / quantum
    n = math.floor(m)
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** 128 - Fraction(2) ** 119:  # >= (max bf16 + half ulp) rounds to inf
        return s * math.inf
    return s * float(val)


def test_bf16_round_hand_ties():
    cases = [
        (1.0 + 2.0 ** -8, 1.0),                     # halfway between 1 and 1 + 2^-7: even is 1
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),     # halfway, the odd neighbour loses
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),   # just past halfway rounds up
        (1.0 + 2.0 ** -8 - 2.0 ** -20, 1.0),               # just below halfway rounds down
        (-(1.0 + 2.0 ** -8), -1.0),
        (-(1.0 + 3 * 2.0 ** -8), -(1.0 + 2.0 ** -6)),
        (2.0 ** -134, 0.0),                         # half the smallest bf16 subnormal: ties to 0
        (3 * 2.0 ** -134, 2.0 ** -132),             # 1.5 subnormal quanta: ties to the even 2
        (2.0 ** -133, 2.0 ** -133),                 # the smallest subnormal itself
        (255 * 2.0 ** -133 + 2.0 ** -134, 2.0 ** -125),  # largest subnormal + half: carries into normal
        (3.3895313892515355e38, 3.3895313892515355e38),  # the largest finite bf16
        (3.4028234663852886e38, np.inf),            # the largest fp32 rounds past it
        (0.0, 0.0), (np.inf, np.inf), (-np.inf, -np.inf),
    ]
    got = oracle.bf16_round(np.array([c[0] for c in cases]))
    for (x, want), y in zip(cases, got):
        assert y == want, (x, want, y)
    assert np.signbit(oracle.bf16_round(np.array([-0.0]))[0])
    assert np.isnan(oracle.bf16_round(np.array([np.nan]))[0])
    # a NaN whose payload sits only in the low 16 bits stays a NaN (no carry into inf)
    low_nan = np.array([0x7F800001], dtype=np.uint32).view(np.float32).astype(np.float64)
    assert np.isnan(oracle.bf16_round(low_nan)[0])


def test_bf16_round_matches_exact_rational_rounding():
    """On fp32-representable inputs (no double rounding), across normal, subnormal and
    near-overflow magnitudes, including constructed ties."""
    r = rng(77)
    bits = r.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    # force a quarter of them onto exact ties (low 16 bits = 0x8000)
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000
    f = bits.view(np.float32)
    x = f[np.isfinite(f)].astype(np.float64)
    got = oracle.bf16_round(x)
    want = np.array([_bf16_exact(float(v)) for v in x])
    assert np.array_equal(got, want)


def test_bf16_round_matches_torch_cpu_conversion():
    import torch
    r = rng(78)
    bits = r.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    bits[:5000] = (bits[:5000] & 0xFFFF0000) | 0x8000
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = oracle.bf16_round(f.astype(np.float64))
    assert np.array_equal(got, want)
