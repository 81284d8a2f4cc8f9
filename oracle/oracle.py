"""Python face of the fp64 CPU oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg are the only callers.  The GPU library never imports this
module and this module imports nothing from the GPU package.

All arrays are numpy float64.  Inputs that the GPU side sees as bf16 are passed here
as their exact float64 values (a bf16 value widens to float64 without rounding), so
both sides see the same numbers.

What each call computes is stated in ``gdn_oracle.c``: the gated delta rule token by
token (Yang, Kautz & Hatamizadeh, "Gated Delta Networks", ICLR 2025), the block
checkpoints of "Prefix caching on Gated DeltaNet hybrids" ("Why hits were wrong"),
the causal conv window, and the prefix accounting of "The cache block that is not a
cache setting" ("What that costs, exactly").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build() -> str:
    """Compile the oracle with gcc (plain IEEE fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", _LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    _lib = _open(_LIB_PATH)
    return _lib


def _open(path):
    lib = ctypes.CDLL(path)
    lib.gdn_oracle_recurrence.restype = ctypes.c_int
    lib.gdn_oracle_recurrence.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, ctypes.c_int64, ctypes.c_int64,
        _dp, _dp, _dp, ctypes.c_int32]
    lib.gdn_oracle_conv.restype = ctypes.c_int
    lib.gdn_oracle_conv.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _dp, _dp, _dp, ctypes.c_int32,
        ctypes.c_int64, ctypes.c_int64, _dp, _dp, _dp, ctypes.c_int32]
    lib.gdn_oracle_count_boundaries.restype = ctypes.c_int64
    lib.gdn_oracle_count_boundaries.argtypes = [ctypes.c_int64] * 3
    lib.gdn_oracle_cached_prefix_tokens.restype = ctypes.c_int64
    lib.gdn_oracle_cached_prefix_tokens.argtypes = [ctypes.c_int64] * 2
    lib.gdn_oracle_floor_chunk.restype = ctypes.c_int64
    lib.gdn_oracle_floor_chunk.argtypes = [ctypes.c_int64] * 2
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    return lib


def _swap_library(path):
    """Point this module at another build of the oracle (used by the mutation test to
    check that the pins reject deliberately broken copies).  Returns the previous one."""
    global _lib
    prev = _lib
    _lib = _open(path) if isinstance(path, str) else path
    return prev


def _ptr(x):
    if x is None:
        return None
    assert x.dtype == np.float64 and x.flags["C_CONTIGUOUS"]
    return x.ctypes.data_as(_dp)


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def count_boundaries(p0: int, length: int, block: int) -> int:
    """Number of block boundaries p*block (p >= 1) in (p0, p0 + length]."""
    return int(_load().gdn_oracle_count_boundaries(p0, length, block))


def recurrence(q, k, v, a, b, scale=1.0, S0=None, p0=0, block=0, want_o=True, threads=0):
    """Gated delta rule over one sequence.

    q, k: [L, Hqk, dk]; v: [L, Hv, dv]; a, b: [L, Hv]; S0: [Hv, dv, dk] or None (zero).
    Returns (o [L, Hv, dv] or None, S_final [Hv, dv, dk], ckpts [n, Hv, dv, dk]).
    ckpts[i] is the state after the i-th block boundary in (p0, p0 + L].
    """
    k = _f64(k)
    v = _f64(v)
    a = _f64(a)
    b = _f64(b)
    q = _f64(q) if q is not None else None
    L, Hqk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    assert v.shape[0] == L and a.shape == (L, Hv) and b.shape == (L, Hv)
    if q is not None:
        assert q.shape == k.shape
    S0 = _f64(S0)
    if S0 is not None:
        assert S0.shape == (Hv, dv, dk)
    o = np.zeros((L, Hv, dv)) if (want_o and q is not None) else None
    S_out = np.zeros((Hv, dv, dk))
    n_ck = count_boundaries(p0, L, block)
    ck = np.zeros((n_ck, Hv, dv, dk)) if n_ck > 0 else None
    rc = _load().gdn_oracle_recurrence(L, Hqk, Hv, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                       _ptr(b), float(scale), _ptr(S0), int(p0), int(block),
                                       _ptr(o), _ptr(S_out), _ptr(ck), int(threads))
    if rc != 0:
        raise ValueError("oracle recurrence: bad shapes")
    if ck is None:
        ck = np.zeros((0, Hv, dv, dk))
    return o, S_out, ck


def replay_outputs(S0, k, v, a, b, m, q_new, scale=1.0):
    """ReplaySSM verification outputs ("Caching less to serve more requests", section
    "What we changed": one state per request plus a log of the per-token inputs since
    it, and a layer's output computed from the two).

    S0: [Hv, dv, dk] (the request's state); k: [L, Hqk, dk], v: [L, Hv, dv], a, b:
    [L, Hv] the log rows 0 .. L-1 with L = m + n; q_new: [n, Hqk, dk] the queries of log
    rows m .. L-1.  Returns o [n, Hv, dv]: o[i] = scale * S_{m+i} q_new[i], with S_t the
    state after log row t of the gated delta rule run from S0.  Written as the token
    recurrence over all L rows with zero queries on the first m (whose outputs are
    dropped).
    """
    q_new = _f64(q_new)
    n = q_new.shape[0]
    L = m + n
    k = _f64(k)[:L]
    assert k.shape[0] == L
    q = np.zeros_like(k)
    q[m:] = q_new
    o, _, _ = recurrence(q, k, _f64(v)[:L], _f64(a)[:L], _f64(b)[:L], scale, S0)
    return o[m:]


def conv(x, w, tail=None, act=1, p0=0, block=0, threads=0):
    """Causal depthwise conv of width W = w.shape[1].

    x: [L, C]; w: [C, W]; tail: [W-1, C] or None (zeros). act: 0 none, 1 SiLU.
    Returns (y [L, C], tail_out [W-1, C], ckpt_tails [n, W-1, C]).
    """
    x = _f64(x)
    w = _f64(w)
    tail = _f64(tail)
    L, C = x.shape
    W = w.shape[1]
    assert w.shape == (C, W)
    if tail is not None:
        assert tail.shape == (W - 1, C)
    y = np.zeros((L, C))
    tail_out = np.zeros((W - 1, C))
    n_ck = count_boundaries(p0, L, block)
    ck = np.zeros((n_ck, W - 1, C)) if n_ck > 0 else None
    rc = _load().gdn_oracle_conv(L, C, W, _ptr(x), _ptr(w), _ptr(tail), int(act), int(p0),
                                 int(block), _ptr(y), _ptr(tail_out), _ptr(ck), int(threads))
    if rc != 0:
        raise ValueError("oracle conv: bad shapes")
    if ck is None:
        ck = np.zeros((0, W - 1, C))
    return y, tail_out, ck


# ---------------------------------------------------------------- packed-core steps
# "Hybrid linear attention (gated DeltaNet)", "Packed-core traces": the packed core
# takes qkvz plus the "ba" projection, owns the conv, dt_bias, an fp32 A_log and a norm
# scale replicated over heads, and returns gated-normalized value rows.  The page names
# the steps without formulas; the readings below are the standard gated DeltaNet ones.

def l2norm_qk_heads(y, n_qk_heads: int, head_dim: int, eps: float = 1e-6):
    """The post-conv step: each q and k head of a conv output row (channels
    [0, 2 * n_qk_heads * head_dim), head_dim values per head) scaled to unit L2 norm,
    y / sqrt(sum y^2 + eps); the value channels pass unchanged.  y: [L, C]."""
    y = _f64(y).copy()
    L = y.shape[0]
    qk = 2 * n_qk_heads * head_dim
    heads = y[:, :qk].reshape(L, 2 * n_qk_heads, head_dim)
    ss = (heads * heads).sum(axis=2, keepdims=True)
    y[:, :qk] = (heads / np.sqrt(ss + eps)).reshape(L, qk)
    return y


def gates(ba, A_log, dt_bias, n_v_heads: int):
    """The gates from the "ba" projection: b = sigmoid(ba[:, :Hv]) and
    a = exp(-exp(A_log) * softplus(ba[:, Hv:2Hv] + dt_bias)), a kept at or above 2^-126
    (the smallest normal fp32 value, so that the fp32 decay the prefill takes has a
    finite logarithm).  Returns (a, b), [L, Hv]."""
    ba = _f64(ba)
    Hv = n_v_heads
    x = ba[:, Hv:2 * Hv] + _f64(dt_bias)[None, :]
    softplus = np.logaddexp(0.0, x)
    a = np.maximum(np.exp(-np.exp(_f64(A_log))[None, :] * softplus), 2.0 ** -126)
    b = 1.0 / (1.0 + np.exp(-ba[:, :Hv]))
    return a, b


def gated_norm(o, z, weight, eps: float = 1e-6):
    """Gated RMSNorm of output rows: o * (mean(o^2) + eps)^(-1/2) * weight * silu(z) over
    the last axis (one row per token and value head).  o, z: [..., d]; weight: [d]."""
    o = _f64(o)
    z = _f64(z)
    r = 1.0 / np.sqrt((o * o).mean(axis=-1, keepdims=True) + eps)
    return o * r * _f64(weight) * (z / (1.0 + np.exp(-z)))


def cached_prefix_tokens(shared: int, block: int) -> int:
    return int(_load().gdn_oracle_cached_prefix_tokens(shared, block))


def floor_chunk(budget: int, block: int) -> int:
    return int(_load().gdn_oracle_floor_chunk(budget, block))


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Used to compare bf16-typed GPU results with oracle values rounded the same way.
    Goes through float32 first, then rounds the float32 bit pattern to 8 significant
    bits with ties to even (the float64 -> float32 step is the nearest float32; the
    double rounding this implies is documented where the comparison is made).  Values
    past the largest bf16 round to infinity; infinities and zeros keep their sign; a
    NaN stays a NaN (the rounding increment is not applied to it).
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) & 0xFFFF0000
    r = np.where(np.isnan(f), u | 0x00400000, r) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32).astype(np.float64)
