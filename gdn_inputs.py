"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method itself: only random draws and the
input recipe (value distributions, shapes, seeds).  Both the GPU path and the CPU
oracle consume what it returns, and it imports neither of them.

Recipe (same for every workload):
  * q, k ~ N(0, 1), then scaled to unit L2 norm per token and head (in fp32),
    then cast to the io dtype (bf16 with round-to-nearest-even, or kept fp32);
  * v ~ N(0, 1), cast to the io dtype;
  * b = sigmoid(N(0, 1));  a = exp(-softplus(N(0, 1)) * 0.1)   (fp32, per value head);
  * conv weights ~ 0.5 * N(0, 1);  conv inputs ~ N(0, 1);
  * states entering decode / flush ~ 0.1 * N(0, 1) (fp32).
Large tensors are drawn in token blocks, each block from its own generator seeded
from (seed, block index), so any block can be re-drawn alone and memory stays bounded.

Workload shapes (a "27B-shaped" layer is 48 value heads of 128 x 128 fp32 state; a
"4B-shaped" layer is 32 heads), following "Prefix caching on Gated DeltaNet hybrids"
("Why hits were wrong": 48 heads x 128 x 128 fp32, blocks of 896 tokens) and
"Caching less to serve more requests" ("What we changed": 2 MiB of fp32 state per
layer, a 32-slot input buffer, 16-row flush blocks).
"""
from __future__ import annotations

import dataclasses

import torch

TOKEN_BLOCK = 8192


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple
    n_qk_heads: int
    n_v_heads: int
    head_dim: int
    io_dtype: torch.dtype
    block: int
    seed: int

    @property
    def conv_channels(self) -> int:
        return (2 * self.n_qk_heads + self.n_v_heads) * self.head_dim

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))


# The parity / bench workloads.
TINY = Workload("tiny_fp32_T64_H2_d16_block16", (64,), 2, 2, 16, torch.float32, 16, 1000)
PREFILL_27B = Workload("prefill_27b_T8192_H48_d128_block896", (8192,), 48, 48, 128,
                       torch.bfloat16, 896, 1001)
VARLEN_27B = Workload("varlen_27b_4seq_block896", (2688, 5000, 6272, 12000), 48, 48, 128,
                      torch.bfloat16, 896, 1002)
LONG_27B = Workload("long_27b_T229376_H48_d128_block896", (229376,), 48, 48, 128,
                    torch.bfloat16, 896, 1004)

FLUSH_4B = dict(name="flush_4b_16req_H32_d128_32slots", n_req=16, n_heads=32, head_dim=128,
                buf_rows=32, seed=1003)
DECODE_27B = dict(name="decode_27b_256req_H48_d128", n_req=256, n_heads=48, head_dim=128,
                  seed=1005)


def _gen(seed: int, block_index: int = 0) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) * 1_000_003 + int(block_index))
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def qkvab(T: int, n_qk: int, n_v: int, d: int, io_dtype=torch.bfloat16, seed: int = 0,
          token_offset: int = 0, heads=None):
    """Draw q, k [T, n_qk, d], v [T, n_v, d] (io dtype) and a, b [T, n_v] (fp32).

    Tokens are drawn in blocks of TOKEN_BLOCK absolute token indices (token_offset is
    the absolute index of the first token), so a slice of a long sequence can be drawn
    without the rest.  `heads` optionally selects value heads (their query/key heads
    follow) after drawing, for oracle checks on a subset of heads.
    """
    qs, ks, vs, as_, bs = [], [], [], [], []
    t = token_offset
    end = token_offset + T
    while t < end:
        blk = t // TOKEN_BLOCK
        b0 = blk * TOKEN_BLOCK
        lo, hi = t - b0, min(end, b0 + TOKEN_BLOCK) - b0
        g = _gen(seed, blk)
        n = TOKEN_BLOCK
        q = torch.randn(n, n_qk, d, generator=g)[lo:hi]
        k = torch.randn(n, n_qk, d, generator=g)[lo:hi]
        v = torch.randn(n, n_v, d, generator=g)[lo:hi]
        b = torch.sigmoid(torch.randn(n, n_v, generator=g))[lo:hi]
        a = torch.exp(-torch.nn.functional.softplus(torch.randn(n, n_v, generator=g)) * 0.1)[lo:hi]
        qs.append(_unit_rows(q).to(io_dtype))
        ks.append(_unit_rows(k).to(io_dtype))
        vs.append(v.to(io_dtype))
        as_.append(a.contiguous())
        bs.append(b.contiguous())
        t = b0 + hi
    q, k, v = torch.cat(qs), torch.cat(ks), torch.cat(vs)
    a, b = torch.cat(as_), torch.cat(bs)
    if heads is not None:
        group = n_v // n_qk
        heads = list(heads)
        qk_heads = sorted({h // group for h in heads})
        q, k = q[:, qk_heads].contiguous(), k[:, qk_heads].contiguous()
        v, a, b = v[:, heads].contiguous(), a[:, heads].contiguous(), b[:, heads].contiguous()
    return q, k, v, a, b


def qkvab_device(T: int, n_qk: int, n_v: int, d: int, io_dtype=torch.bfloat16, seed: int = 0,
                 device="cuda"):
    """Same recipe as qkvab, drawn on the device with the device's seeded generator (for
    the long workload, whose host draw and upload would dominate a test).  The values
    differ from the host draw of the same seed; a test copies back the heads it checks.
    Drawn in token blocks into preallocated outputs, so temporaries stay bounded."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 77)
    q = torch.empty(T, n_qk, d, dtype=io_dtype, device=device)
    k = torch.empty(T, n_qk, d, dtype=io_dtype, device=device)
    v = torch.empty(T, n_v, d, dtype=io_dtype, device=device)
    a = torch.empty(T, n_v, dtype=torch.float32, device=device)
    b = torch.empty(T, n_v, dtype=torch.float32, device=device)
    for t0 in range(0, T, TOKEN_BLOCK):
        n = min(TOKEN_BLOCK, T - t0)
        q[t0:t0 + n] = _unit_rows(torch.randn(n, n_qk, d, generator=g, device=device)).to(io_dtype)
        k[t0:t0 + n] = _unit_rows(torch.randn(n, n_qk, d, generator=g, device=device)).to(io_dtype)
        v[t0:t0 + n] = torch.randn(n, n_v, d, generator=g, device=device).to(io_dtype)
        b[t0:t0 + n] = torch.sigmoid(torch.randn(n, n_v, generator=g, device=device))
        a[t0:t0 + n] = torch.exp(-torch.nn.functional.softplus(torch.randn(n, n_v, generator=g, device=device))
                                 * 0.1)
    return q, k, v, a, b


def conv_inputs(T: int, channels: int, width: int = 4, io_dtype=torch.bfloat16, seed: int = 0):
    """Draw conv inputs x [T, C] and weights w [C, width] in the io dtype."""
    g = _gen(seed, 10_000)
    w = (0.5 * torch.randn(channels, width, generator=g)).to(io_dtype)
    xs = []
    for blk in range((T + TOKEN_BLOCK - 1) // TOKEN_BLOCK):
        n = min(TOKEN_BLOCK, T - blk * TOKEN_BLOCK)
        xs.append(torch.randn(n, channels, generator=_gen(seed, 20_000 + blk)).to(io_dtype))
    x = torch.cat(xs) if xs else torch.zeros(0, channels, dtype=io_dtype)
    return x, w


def core_inputs(T: int, n_v_heads: int, head_dim: int, io_dtype=torch.bfloat16, seed: int = 0):
    """Inputs of the packed core's gate and output-norm steps: the "ba" projection rows
    [T, 2 Hv] (io dtype, N(0, 2)), A_log [Hv] (fp32, log of U[1, 16]), dt_bias [Hv] (io
    dtype, N(0, 1)), an output o [T, Hv, d] (fp32, N(0, 1)), the gate rows z [T, Hv, d]
    (io dtype, N(0, 1)) and the norm scale [d] (io dtype, 1 + 0.1 N(0, 1))."""
    g = _gen(seed, 40_000)
    ba = (2.0 * torch.randn(T, 2 * n_v_heads, generator=g)).to(io_dtype)
    A_log = torch.log(1.0 + 15.0 * torch.rand(n_v_heads, generator=g)).to(torch.float32)
    dt_bias = torch.randn(n_v_heads, generator=g).to(io_dtype)
    o = torch.randn(T, n_v_heads, head_dim, generator=g).to(torch.float32)
    z = torch.randn(T, n_v_heads, head_dim, generator=g).to(io_dtype)
    weight = (1.0 + 0.1 * torch.randn(head_dim, generator=g)).to(io_dtype)
    return ba, A_log, dt_bias, o, z, weight


def conv_tail(n: int, channels: int, width: int = 4, io_dtype=torch.bfloat16, seed: int = 0):
    """Draw n conv tails [n, width - 1, C]."""
    g = _gen(seed, 30_000)
    return torch.randn(n, width - 1, channels, generator=g).to(io_dtype)


def states(n: int, n_v: int, d: int, seed: int = 0, std: float = 0.1):
    """Draw n fp32 states [n, n_v, d, d] ~ std * N(0, 1)."""
    g = _gen(seed, 40_000)
    return std * torch.randn(n, n_v, d, d, generator=g)


def accepted_counts(n_req: int, seed: int, max_rows: int = 16):
    """Accepted rows per request: uniform in 0..max_rows-1 plus the bonus token."""
    g = _gen(seed, 50_000)
    return torch.randint(0, max_rows, (n_req,), generator=g, dtype=torch.int32) + 1


def permutation(n: int, seed: int):
    g = _gen(seed, 60_000)
    return torch.randperm(n, generator=g)


# ---------------------------------------------------------------- harder input domains
# Inputs at the edges of the contract (a in (0, 1], b in [0, 1]), for parity cases the
# workloads' distributions never reach: gates at the smallest normal decay (the value
# the packed core's gate step clamps to) and at exactly 1, write strengths of exactly 0
# and 1, keys far from unit norm and keys nearly parallel to each other.  The update
# stays bounded while b_t |k_t|^2 <= 2; the draws keep to that range.
A_CLAMP = 2.0 ** -126  # the smallest normal fp32 value


def edge_gates(T: int, n_v: int, seed: int = 0):
    """a, b [T, n_v] fp32: a is 2^-126 (a full reset) with probability 0.2, exactly 1
    with probability 0.2, else exp(-softplus(N(0,1)) * 0.1); b is exactly 0 or 1 with
    probability 0.25 each, else sigmoid(N(0,1))."""
    g = _gen(seed, 70_000)
    u = torch.rand(T, n_v, generator=g)
    a = torch.exp(-torch.nn.functional.softplus(torch.randn(T, n_v, generator=g)) * 0.1)
    a = torch.where(u < 0.2, torch.full_like(a, A_CLAMP), torch.where(u < 0.4, torch.ones_like(a), a))
    w = torch.rand(T, n_v, generator=g)
    b = torch.sigmoid(torch.randn(T, n_v, generator=g))
    b = torch.where(w < 0.25, torch.zeros_like(b), torch.where(w < 0.5, torch.ones_like(b), b))
    return a.float().contiguous(), b.float().contiguous()


def scaled_keys(T: int, n_qk: int, d: int, io_dtype=torch.bfloat16, seed: int = 0, lo: float = 0.25,
                hi: float = 4.0):
    """k [T, n_qk, d]: unit rows times a norm log-uniform in [lo, hi] (cast to io dtype),
    and the squared norm of each row as cast, [T, n_qk] fp32 (for bounding b)."""
    g = _gen(seed, 71_000)
    k = _unit_rows(torch.randn(T, n_qk, d, generator=g))
    r = torch.exp(torch.log(torch.tensor(lo)) + torch.rand(T, n_qk, 1, generator=g) *
                  (torch.log(torch.tensor(hi)) - torch.log(torch.tensor(lo))))
    k = (k * r).to(io_dtype)
    return k, (k.float() ** 2).sum(-1)


def collinear_keys(T: int, n_qk: int, d: int, io_dtype=torch.bfloat16, seed: int = 0, spread: float = 0.05,
                   run: int = 48):
    """k [T, n_qk, d] unit rows that stay nearly parallel over runs of `run` tokens: each
    run shares a base direction, and every row adds a random offset of norm about
    `spread` before normalising (cosines between rows of a run near 1 - spread^2)."""
    g = _gen(seed, 72_000)
    n_runs = (T + run - 1) // run
    base = _unit_rows(torch.randn(n_runs, n_qk, d, generator=g)).repeat_interleave(run, 0)[:T]
    k = _unit_rows(base + spread * torch.randn(T, n_qk, d, generator=g) / d ** 0.5)
    return k.to(io_dtype)


def conv_inputs_device(T: int, channels: int, width: int = 4, io_dtype=torch.bfloat16, seed: int = 0,
                       device="cuda"):
    """Same recipe as conv_inputs (x ~ N(0, 1), w ~ 0.5 N(0, 1)), drawn on the device in
    token blocks (for the long workload, whose host draw would dominate)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 99)
    w = (0.5 * torch.randn(channels, width, generator=g, device=device)).to(io_dtype)
    x = torch.empty(T, channels, dtype=io_dtype, device=device)
    for t0 in range(0, T, TOKEN_BLOCK):
        n = min(TOKEN_BLOCK, T - t0)
        x[t0:t0 + n] = torch.randn(n, channels, generator=g, device=device).to(io_dtype)
    return x, w
