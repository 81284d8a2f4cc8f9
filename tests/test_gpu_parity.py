"""GPU parity: libgdn (through the C ABI) against the fp64 oracle on the same seeded inputs.

Sizes span several 64-row chunks and a ragged tail; tolerances are the relative L2
bounds 1e-3 (bf16 inputs) and 1e-5 (fp32 inputs).  Bit-exactness is required only
GPU against GPU: resume-from-checkpoint against the cold run, and a sequence in a
varlen batch against the same sequence alone.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import TOL, bits, f64, make_pool, nan_fill_, rel_l2, same_bits, say
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_recurrent_chunk_amd as lib
    return lib


def _dev(*ts):
    return [t.cuda() for t in ts]


PREFILL_CASES = [
    # T, Hqk, Hv, D, dtype, block
    (64, 2, 2, 16, torch.float32, 16),       # the tiny workload: four 16-token chunks
    (300, 2, 4, 128, torch.bfloat16, 128),   # value heads sharing key heads, ragged tail
    (200, 1, 1, 64, torch.bfloat16, 80),     # block off the 64-grid
    (130, 2, 2, 32, torch.bfloat16, 0),      # no checkpoints
    (100, 1, 2, 32, torch.float32, 48),
    (257, 1, 1, 128, torch.bfloat16, 64),
    (90, 2, 2, 16, torch.bfloat16, 32),
    (200, 2, 4, 128, torch.float32, 96),    # fp32 rows at the full head dim
]


@pytest.mark.parametrize("T,Hqk,Hv,D,dtype,block", PREFILL_CASES)
def test_prefill_cold_matches_oracle(g, T, Hqk, Hv, D, dtype, block):
    say(f"prefill cold T={T} Hqk={Hqk} Hv={Hv} D={D} {dtype} block={block}")
    layer = g.Layer(Hqk, Hv, D, dtype, scale=0.5)
    q, k, v, a, b = gi.qkvab(T, Hqk, Hv, D, dtype, seed=11 + T)
    n_ck = oracle.count_boundaries(0, T, block)
    pool = make_pool(g, layer, n_ck + 3, block)
    page_ids = [int(p) for p in gi.permutation(n_ck + 3, 5)[:n_ck]]
    qd, kd, vd, ad, bd = _dev(q, k, v, a, b)
    o = torch.full((T, Hv, D), float("nan"), device="cuda")
    S = torch.empty(Hv, D, D, device="cuda")
    g.chunk_prefill(layer, qd, kd, vd, ad, bd, [0, T], [0], [("zero", None, S)], o, ckpt=pool,
                    page_ids=page_ids)
    torch.cuda.synchronize()
    o_ref, S_ref, ck_ref = oracle.recurrence(f64(q), f64(k), f64(v), f64(a), f64(b), 0.5, None, 0, block)
    tol = TOL[dtype]
    assert rel_l2(f64(o), o_ref) <= tol
    assert rel_l2(f64(S), S_ref) <= tol
    for i in range(n_ck):
        assert rel_l2(f64(pool.state_view(page_ids[i], layer)), ck_ref[i]) <= tol, i
    # pages not named by the call keep their contents
    for p in range(n_ck + 3):
        if p not in page_ids:
            assert (pool.pool[p].view(torch.int32) == 0x7FC0DEAD).all()


@pytest.mark.parametrize("T,Hqk,Hv,D,dtype,block", [c for c in PREFILL_CASES if c[5] > 0])
def test_resume_from_checkpoint_is_bit_identical_to_cold(g, T, Hqk, Hv, D, dtype, block):
    say(f"resume T={T} D={D} {dtype} block={block}")
    layer = g.Layer(Hqk, Hv, D, dtype)
    q, k, v, a, b = gi.qkvab(T, Hqk, Hv, D, dtype, seed=21 + T)
    n_ck = oracle.count_boundaries(0, T, block)
    pool = make_pool(g, layer, 2 * n_ck + 1, block)
    qd, kd, vd, ad, bd = _dev(q, k, v, a, b)
    o = torch.empty(T, Hv, D, device="cuda")
    S = torch.empty(Hv, D, D, device="cuda")
    g.chunk_prefill(layer, qd, kd, vd, ad, bd, [0, T], [0], [("zero", None, S)], o, ckpt=pool,
                    page_ids=list(range(n_ck)))
    for p in range(1, n_ck + 1):
        s0 = p * block
        if s0 >= T:
            break
        L = T - s0
        o2 = torch.empty(L, Hv, D, device="cuda")
        S2 = torch.empty(Hv, D, D, device="cuda")
        n2 = oracle.count_boundaries(s0, L, block)
        g.chunk_prefill(layer, qd[s0:], kd[s0:], vd[s0:], ad[s0:], bd[s0:], [0, L], [s0],
                        [("checkpoint", pool.page_ptr(p - 1), S2)], o2, ckpt=pool,
                        page_ids=list(range(n_ck, n_ck + n2)))
        torch.cuda.synchronize()
        assert same_bits(o2, o[s0:]), f"outputs after resume at {s0}"
        assert same_bits(S2, S), f"final state after resume at {s0}"
        for i in range(n2):
            assert torch.equal(pool.pool[n_ck + i, :layer.state_bytes], pool.pool[p + i, :layer.state_bytes])


def test_varlen_batch_is_bit_identical_to_solo_runs(g):
    D, H, dtype, block = 128, 2, torch.bfloat16, 128
    layer = g.Layer(H, H, D, dtype)
    lens = [150, 64, 1, 300, 0, 77]
    starts = [0, 128, 256, 0, 0, 384]
    say(f"varlen lens={lens} starts={starts}")
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    T = cu[-1]
    q, k, v, a, b = gi.qkvab(T, H, H, D, dtype, seed=31)
    qd, kd, vd, ad, bd = _dev(q, k, v, a, b)
    S0 = (0.1 * torch.randn(len(lens), H, D, D, generator=torch.Generator().manual_seed(3))).cuda()
    n_b = [oracle.count_boundaries(s, L, block) for s, L in zip(starts, lens)]
    pool = make_pool(g, layer, 2 * sum(n_b) + 1, block)
    o = torch.empty(T, H, D, device="cuda")
    Sf = torch.empty(len(lens), H, D, D, device="cuda")
    refs = [("zero" if s == 0 else "slot", None if s == 0 else S0[i], Sf[i]) for i, s in enumerate(starts)]
    g.chunk_prefill(layer, qd, kd, vd, ad, bd, cu, starts, refs, o, ckpt=pool, page_ids=list(range(sum(n_b))))
    base = sum(n_b)
    for i, (s, L) in enumerate(zip(starts, lens)):
        r0 = cu[i]
        o1 = torch.empty(max(L, 1), H, D, device="cuda")
        S1 = torch.empty(H, D, D, device="cuda")
        ref = ("zero" if s == 0 else "slot", None if s == 0 else S0[i], S1)
        g.chunk_prefill(layer, qd[r0:r0 + L] if L else qd, kd[r0:r0 + L] if L else kd, vd[r0:r0 + L] if L else vd,
                        ad[r0:r0 + L] if L else ad, bd[r0:r0 + L] if L else bd, [0, L], [s], [ref], o1, ckpt=pool,
                        page_ids=list(range(base, base + n_b[i])))
        torch.cuda.synchronize()
        if L:
            assert same_bits(o1[:L], o[r0:r0 + L]), i
        assert same_bits(S1, Sf[i]), i
        off = sum(n_b[:i])
        for j in range(n_b[i]):
            assert torch.equal(pool.pool[base + j, :layer.state_bytes], pool.pool[off + j, :layer.state_bytes])
        # and the oracle agrees
        if L:
            o_ref, S_ref, _ = oracle.recurrence(f64(q[r0:r0 + L]), f64(k[r0:r0 + L]), f64(v[r0:r0 + L]),
                                                f64(a[r0:r0 + L]), f64(b[r0:r0 + L]), 1.0,
                                                None if s == 0 else f64(S0[i]), s, block)
            assert rel_l2(f64(o1[:L]), o_ref) <= TOL[dtype]
            assert rel_l2(f64(S1), S_ref) <= TOL[dtype]
        elif s != 0:
            assert same_bits(S1, S0[i])
        else:
            assert not S1.any()


def test_identity_gate_is_bitwise_identity(g):
    """a = 1, b = 0: the state comes back bit for bit, o = scale * S_0 q."""
    D, H, T = 128, 2, 150
    layer = g.Layer(H, H, D, torch.bfloat16, scale=1.0)
    q, k, v, _, _ = gi.qkvab(T, H, H, D, torch.bfloat16, seed=41)
    a = torch.ones(T, H)
    b = torch.zeros(T, H)
    S0 = (0.1 * torch.randn(H, D, D, generator=torch.Generator().manual_seed(4))).cuda()
    o = torch.empty(T, H, D, device="cuda")
    S = torch.empty(H, D, D, device="cuda")
    qd, kd, vd, ad, bd = _dev(q, k, v, a, b)
    say("identity gate")
    g.chunk_prefill(layer, qd, kd, vd, ad, bd, [0, T], [64], [("slot", S0, S)], o)
    torch.cuda.synchronize()
    assert same_bits(S, S0)
    o_ref = np.einsum("hij,thj->thi", f64(S0), f64(q))
    assert rel_l2(f64(o), o_ref) <= 1e-3


# ------------------------------------------------------------------------- decode

@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (16, torch.float32), (64, torch.bfloat16),
                                     (128, torch.float32)])
def test_decode_matches_oracle_and_skips_padding(g, D, dtype):
    Hqk, Hv, n_slots = 2, 4, 5
    layer = g.Layer(Hqk, Hv, D, dtype, scale=0.7)
    slots = [3, -1, 0, 4]
    n = len(slots)
    say(f"decode D={D} {dtype} slots={slots}")
    q, k, v, a, b = gi.qkvab(n, Hqk, Hv, D, dtype, seed=51)
    pool = gi.states(n_slots, Hv, D, seed=52).cuda()
    nan_fill_(pool[1])
    nan_fill_(pool[2])
    before = pool.clone()
    o = nan_fill_(torch.empty(n, Hv, D, device="cuda"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    qd, kd, vd, ad, bd = _dev(q, k, v, a, b)
    g.decode_step(layer, qd, kd, vd, ad, bd, pool, torch.tensor(slots, dtype=torch.int32, device="cuda"), o,
                  status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    tol = TOL[dtype]
    for r, s in enumerate(slots):
        if s < 0:
            assert same_bits(o[r], nan_fill_(torch.empty_like(o[r])))
            continue
        o_ref, S_ref, _ = oracle.recurrence(f64(q[r:r + 1]), f64(k[r:r + 1]), f64(v[r:r + 1]), f64(a[r:r + 1]),
                                            f64(b[r:r + 1]), 0.7, f64(before[s]))
        assert rel_l2(f64(o[r]), o_ref[0]) <= tol
        assert rel_l2(f64(pool[s]), S_ref) <= tol
    assert same_bits(pool[1], before[1]) and same_bits(pool[2], before[2])


def test_decode_rejects_bad_slot_on_device(g):
    D, H = 32, 2
    layer = g.Layer(H, H, D, torch.bfloat16)
    q, k, v, a, b = [t.cuda() for t in gi.qkvab(2, H, H, D, torch.bfloat16, seed=61)]
    pool = gi.states(2, H, D, seed=62).cuda()
    before = pool.clone()
    o = torch.zeros(2, H, D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("decode bad slot")
    g.decode_step(layer, q, k, v, a, b, pool, torch.tensor([7, -1], dtype=torch.int32, device="cuda"), o,
                  status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 << 8
    assert same_bits(pool, before)


# ------------------------------------------------------------------------- flush

@pytest.mark.parametrize("D,dtype,rows", [(128, torch.bfloat16, 32), (16, torch.float32, 32),
                                          (64, torch.bfloat16, 64), (32, torch.bfloat16, 16),
                                          (128, torch.bfloat16, 64), (32, torch.bfloat16, 64),
                                          (64, torch.float32, 64), (128, torch.float32, 32),
                                          (128, torch.float32, 64)])
def test_flush_matches_sequential_oracle(g, D, dtype, rows):
    Hqk, Hv, n_slots = 2, 4, 6
    layer = g.Layer(Hqk, Hv, D, dtype)
    slots = [4, 0, 2, 5, -1, 1]
    # counts on both sides of the 32- and 64-row tiles
    acc = [min(rows, x) for x in ([16, 1, 17, 0, 5, rows] if rows <= 32 else [16, 1, 32, 0, 33, rows])]
    say(f"flush D={D} {dtype} rows={rows} acc={acc}")
    pool = gi.states(n_slots, Hv, D, seed=71).cuda()
    kk, vv, aa, bb = [], [], [], []
    for s in range(n_slots):
        _, k, v, a, b = gi.qkvab(rows, Hqk, Hv, D, dtype, seed=72 + s)
        kk.append(k), vv.append(v), aa.append(a), bb.append(b)
    buf_k, buf_v = torch.stack(kk).cuda(), torch.stack(vv).cuda()
    buf_a, buf_b = torch.stack(aa).cuda(), torch.stack(bb).cuda()
    # rejected rows hold NaN: they must never be read
    for r, s in enumerate(slots):
        if s >= 0:
            n = acc[r]
            nan_fill_(buf_k[s, n:]), nan_fill_(buf_v[s, n:]), nan_fill_(buf_a[s, n:]), nan_fill_(buf_b[s, n:])
    before = pool.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.replay_flush(layer, pool, torch.tensor(slots, dtype=torch.int32, device="cuda"), buf_k, buf_v, buf_a, buf_b,
                   torch.tensor(acc, dtype=torch.int32, device="cuda"), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    touched = set()
    for r, s in enumerate(slots):
        if s < 0:
            continue
        touched.add(s)
        n = acc[r]
        if n == 0:
            assert same_bits(pool[s], before[s])
            continue
        _, S_ref, _ = oracle.recurrence(None, f64(buf_k[s, :n]), f64(buf_v[s, :n]), f64(buf_a[s, :n]),
                                        f64(buf_b[s, :n]), 1.0, f64(before[s]), want_o=False)
        assert rel_l2(f64(pool[s]), S_ref) <= TOL[dtype], (r, s, n)
    for s in range(n_slots):
        if s not in touched:
            assert same_bits(pool[s], before[s])


def test_flush_rejects_bad_count_on_device(g):
    D, H = 32, 2
    layer = g.Layer(H, H, D, torch.bfloat16)
    pool = gi.states(2, H, D, seed=81).cuda()
    before = pool.clone()
    buf = torch.zeros(2, 32, H, D, dtype=torch.bfloat16, device="cuda")
    ab = torch.full((2, 32, H), 0.5, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("flush bad count")
    g.replay_flush(layer, pool, torch.tensor([0, 1], dtype=torch.int32, device="cuda"), buf, buf, ab, ab,
                   torch.tensor([33, -2], dtype=torch.int32, device="cuda"), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 << 8
    assert same_bits(pool, before)


# ------------------------------------------------------------------------- packed-core steps

@pytest.mark.parametrize("Hqk,Hv,D,dtype", [(2, 4, 128, torch.bfloat16), (1, 2, 16, torch.float32),
                                            (3, 3, 32, torch.bfloat16), (2, 2, 64, torch.float32),
                                            (1, 2, 128, torch.float32)])
def test_conv_with_qk_l2norm_matches_oracle(g, Hqk, Hv, D, dtype):
    """The conv with the post-conv step fused: q and k heads of every output row at unit
    norm, value channels and tails as without it."""
    block = 16
    layer = g.Layer(Hqk, Hv, D, dtype, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    lens, starts = [37, 70, 5], [0, 32, 7]
    say(f"conv+l2norm Hqk={Hqk} Hv={Hv} D={D} {dtype}")
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    x, w = gi.conv_inputs(cu[-1], C, 4, dtype, seed=111)
    tails0 = gi.conv_tail(len(lens), C, 4, dtype, seed=112)
    n_b = [oracle.count_boundaries(s_, L, block) for s_, L in zip(starts, lens)]
    pool = make_pool(g, layer, sum(n_b) + 1, block)
    td = tails0.cuda()
    out_t = nan_fill_(torch.empty(len(lens), 3, C, dtype=dtype, device="cuda"))
    refs = [("zero", None, out_t[0]), ("slot", td[1], out_t[1]), ("slot", td[2], out_t[2])]
    y = nan_fill_(torch.empty(cu[-1], C, dtype=dtype, device="cuda"))
    g.conv_update(layer, x.cuda(), w.cuda(), refs, cu, starts, y, ckpt=pool, page_ids=list(range(sum(n_b))))
    torch.cuda.synchronize()
    for i, (s_, L) in enumerate(zip(starts, lens)):
        r0 = cu[i]
        y_ref, t_ref, _ = oracle.conv(f64(x[r0:r0 + L]), f64(w), None if i == 0 else f64(tails0[i]), 1, s_, block)
        y_ref = oracle.l2norm_qk_heads(y_ref, Hqk, D)
        if dtype == torch.bfloat16:
            assert rel_l2(f64(y[r0:r0 + L]), oracle.bf16_round(y_ref)) <= 1e-3, i
        else:
            assert rel_l2(f64(y[r0:r0 + L]), y_ref) <= 1e-5, i
        assert np.array_equal(f64(out_t[i]), t_ref), i
    qk = 2 * Hqk * D
    heads = f64(y[:, :qk]).reshape(cu[-1], 2 * Hqk, D)
    assert np.allclose(np.linalg.norm(heads, axis=2), 1.0, atol=1e-2 if dtype == torch.bfloat16 else 1e-5)


@pytest.mark.parametrize("Hv,dtype", [(48, torch.bfloat16), (32, torch.float32), (5, torch.bfloat16)])
def test_gates_match_oracle(g, Hv, dtype):
    T = 301
    layer = g.Layer(Hv, Hv, 16, dtype)
    ba, A_log, dt_bias, _, _, _ = gi.core_inputs(T, Hv, 16, dtype, seed=121)
    say(f"gates Hv={Hv} {dtype}")
    # ba rows inside a wider packed row (stride 2 Hv + 6)
    wide = torch.zeros(T, 2 * Hv + 6, dtype=dtype)
    wide[:, :2 * Hv] = ba
    a = torch.full((T, Hv), float("nan"), device="cuda")
    b = torch.full((T, Hv), float("nan"), device="cuda")
    g.gates(layer, wide.cuda(), A_log.cuda(), dt_bias.cuda(), a, b)
    torch.cuda.synchronize()
    a_ref, b_ref = oracle.gates(f64(ba), f64(A_log), f64(dt_bias), Hv)
    # the decay is compared as the log-decay the prefill takes: fp32 evaluation of
    # exp(-E) carries a relative error of about E * 1e-7
    ga, g_ref = np.log(f64(a)), np.log(a_ref)
    assert np.max(np.abs(ga - g_ref) / np.maximum(np.abs(g_ref), 1.0)) <= 1e-5
    assert np.max(np.abs(f64(b) - b_ref) / b_ref) <= 1e-5
    assert (f64(a) >= 2.0 ** -126).all() and (f64(a) <= 1).all()


@pytest.mark.parametrize("Hv,D,dtype", [(48, 128, torch.bfloat16), (4, 16, torch.float32), (3, 64, torch.bfloat16),
                                        (2, 32, torch.float32)])
def test_gated_norm_matches_oracle(g, Hv, D, dtype):
    T = 77
    layer = g.Layer(Hv, Hv, D, dtype)
    _, _, _, o, z, wgt = gi.core_inputs(T, Hv, D, dtype, seed=131)
    say(f"gated norm Hv={Hv} D={D} {dtype}")
    out = nan_fill_(torch.empty(T, Hv, D, dtype=dtype, device="cuda"))
    g.gated_norm(layer, o.cuda(), z.cuda(), wgt.cuda(), out, eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.gated_norm(f64(o), f64(z), f64(wgt), 1e-6)
    if dtype == torch.bfloat16:
        assert rel_l2(f64(out), oracle.bf16_round(ref)) <= 1e-3
    else:
        assert rel_l2(f64(out), ref) <= 1e-5


# ------------------------------------------------------------------------- mixed batches

@pytest.mark.parametrize("Hqk,Hv,D,dtype", [(2, 4, 128, torch.bfloat16), (1, 2, 32, torch.float32),
                                            (1, 2, 128, torch.float32)])
def test_mixed_batch_decode_rows_and_prefill(g, Hqk, Hv, D, dtype):
    """One packed batch: 5 decode tokens (rows 0..4, in permuted order, one padding slot)
    and two prefill sequences behind them.  The decode tokens go to decode_mixed, the
    prefill rows to chunk_prefill; each result against the oracle, and decode_mixed
    bit-identical to decode_step on the same tokens gathered densely."""
    layer = g.Layer(Hqk, Hv, D, dtype, scale=0.5)
    n_dec, lens = 5, [130, 70]
    T = n_dec + sum(lens)
    say(f"mixed batch Hqk={Hqk} Hv={Hv} D={D} {dtype}")
    q, k, v, a, b = gi.qkvab(T, Hqk, Hv, D, dtype, seed=141)
    n_slots = 7
    pool0 = gi.states(n_slots, Hv, D, seed=142)
    slots = [2, 0, -1, 5, 1]
    rows = [3, 0, 4, 1, 2]
    qd, kd, vd, ad, bd = _dev(q, k, v, a, b)
    pool = pool0.cuda()
    o = torch.full((T, Hv, D), 777.0, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device="cuda")
    g.decode_mixed(layer, qd, kd, vd, ad, bd, pool, i32(slots), i32(rows), o, status=status)
    # the prefill rows: sequence A from zero, sequence B from the state in slot 6
    SA = torch.empty(Hv, D, D, device="cuda")
    SB = torch.empty(Hv, D, D, device="cuda")
    cu = [0, lens[0], lens[0] + lens[1]]
    pre = slice(n_dec, T)
    g.chunk_prefill(layer, qd[pre], kd[pre], vd[pre], ad[pre], bd[pre], cu, [0, 40],
                    [("zero", None, SA), ("slot", pool[6].clone(), SB)], o[pre], ckpt=g.no_checkpoints())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    out, pl = f64(o), f64(pool)
    for r, (s_, row) in enumerate(zip(slots, rows)):
        if s_ < 0:
            assert np.all(out[row] == 777.0)
            continue
        o_ref, S_ref, _ = oracle.recurrence(f64(q[row:row + 1]), f64(k[row:row + 1]), f64(v[row:row + 1]),
                                            f64(a[row:row + 1]), f64(b[row:row + 1]), 0.5, f64(pool0[s_]))
        assert rel_l2(out[row:row + 1], o_ref) <= TOL[dtype], r
        assert rel_l2(pl[s_], S_ref) <= TOL[dtype], r
    for s_ in (3, 4, 6):
        assert np.array_equal(pl[s_], f64(pool0[s_]))
    for i, (src, Sg) in enumerate(((None, SA), (f64(pool0[6]), SB))):
        r0 = n_dec + cu[i]
        sl_ = slice(r0, r0 + lens[i])
        o_ref, S_ref, _ = oracle.recurrence(f64(q[sl_]), f64(k[sl_]), f64(v[sl_]), f64(a[sl_]), f64(b[sl_]), 0.5, src)
        assert rel_l2(out[sl_], o_ref) <= TOL[dtype], i
        assert rel_l2(f64(Sg), S_ref) <= TOL[dtype], i
    # the same tokens, gathered densely, through decode_step: identical bits
    pool2 = pool0.cuda()
    idx = torch.tensor(rows, device="cuda")
    o2 = torch.full((n_dec, Hv, D), 777.0, device="cuda")
    g.decode_step(layer, qd[idx].contiguous(), kd[idx].contiguous(), vd[idx].contiguous(), ad[idx].contiguous(),
                  bd[idx].contiguous(), pool2, i32(slots), o2)
    torch.cuda.synchronize()
    assert same_bits(pool2, pool)
    assert same_bits(o2, o[idx])


def test_mixed_batch_rejects_rows_outside_the_arrays(g):
    D, H = 32, 2
    layer = g.Layer(H, H, D, torch.bfloat16)
    q, k, v, a, b = _dev(*gi.qkvab(4, H, H, D, torch.bfloat16, seed=151))
    pool = gi.states(2, H, D, seed=152).cuda()
    before = pool.clone()
    o = torch.zeros(4, H, D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("mixed batch bad rows")
    g.decode_mixed(layer, q, k, v, a, b, pool, torch.tensor([0, 1], dtype=torch.int32, device="cuda"),
                   torch.tensor([4, -1], dtype=torch.int32, device="cuda"), o, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 << 8
    assert same_bits(pool, before)
    assert torch.count_nonzero(o) == 0


# ------------------------------------------------------------------------- replay outputs

REPLAY_CASES = [
    # D, dtype, buf_rows, per request (slot, logged, new); slot -1 is padding
    (128, torch.bfloat16, 32, [(4, 16, 16), (0, 0, 17), (2, 15, 1), (5, 3, 0), (-1, 2, 5), (1, 15, 17), (3, 7, 9)]),
    (16, torch.float32, 32, [(1, 5, 11), (0, 0, 1), (3, 31, 1), (2, 12, 17)]),
    (64, torch.bfloat16, 64, [(0, 40, 17), (2, 0, 3), (1, 63, 1), (3, 47, 17)]),
    (32, torch.float32, 64, [(3, 30, 17), (0, 1, 16), (2, 0, 0)]),
    (128, torch.float32, 32, [(1, 20, 12), (0, 0, 17), (3, 31, 1), (2, 9, 0), (4, 15, 16)]),
    # 64-row logs at d = 128: blocks of 14, 32, 57 and 64 rows (one to four 16-row blocks)
    (128, torch.bfloat16, 64, [(0, 40, 17), (2, 5, 9), (1, 47, 17), (3, 16, 16)]),
]


@pytest.mark.parametrize("D,dtype,rows,reqs", REPLAY_CASES)
def test_replay_forward_matches_oracle(g, D, dtype, rows, reqs):
    """Outputs of the new rows from the slot's state and its log; the state, the log, the
    rows past each request's count and the padding requests' outputs are untouched."""
    Hqk, Hv, n_slots, max_new = 2, 4, 6, 17
    layer = g.Layer(Hqk, Hv, D, dtype, scale=0.5)
    say(f"replay D={D} {dtype} rows={rows} reqs={reqs}")
    n_req = len(reqs)
    pool = gi.states(n_slots, Hv, D, seed=91).cuda()
    kk, vv, aa, bb = [], [], [], []
    for s in range(n_slots):
        _, k, v, a, b = gi.qkvab(rows, Hqk, Hv, D, dtype, seed=92 + s)
        kk.append(k), vv.append(v), aa.append(a), bb.append(b)
    buf_k, buf_v = torch.stack(kk).cuda(), torch.stack(vv).cuda()
    buf_a, buf_b = torch.stack(aa).cuda(), torch.stack(bb).cuda()
    qn, _, _, _, _ = gi.qkvab(n_req * max_new, Hqk, Hv, D, dtype, seed=99)
    q_new = qn.view(n_req, max_new, Hqk, D).cuda()
    # log rows past m + n and queries past n hold NaN: they must never be read
    for r, (s, m, n) in enumerate(reqs):
        if s >= 0:
            nan_fill_(buf_k[s, m + n:]), nan_fill_(buf_v[s, m + n:])
            nan_fill_(buf_a[s, m + n:]), nan_fill_(buf_b[s, m + n:])
        nan_fill_(q_new[r, n:])
    o = torch.full((n_req, max_new, Hv, D), 1234.5, device="cuda")
    o_before = o.clone()
    before = pool.clone()
    logs = [t.clone() for t in (buf_k, buf_v, buf_a, buf_b)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device="cuda")
    g.replay_forward(layer, pool, i32([x[0] for x in reqs]), buf_k, buf_v, buf_a, buf_b, i32([x[1] for x in reqs]),
                     i32([x[2] for x in reqs]), q_new, o, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert same_bits(pool, before)
    for t0, t1 in zip(logs, (buf_k, buf_v, buf_a, buf_b)):
        assert same_bits(t0, t1)
    for r, (s, m, n) in enumerate(reqs):
        assert same_bits(o[r, n:], o_before[r, n:]), r
        if s < 0 or n == 0:
            assert same_bits(o[r], o_before[r]), r
            continue
        o_ref = oracle.replay_outputs(f64(before[s]), f64(buf_k[s]), f64(buf_v[s]), f64(buf_a[s]), f64(buf_b[s]), m,
                                      f64(q_new[r, :n]), 0.5)
        assert rel_l2(f64(o[r, :n]), o_ref) <= TOL[dtype], (r, s, m, n)


def test_replay_forward_rejects_bad_counts_on_device(g):
    D, H, rows, max_new = 32, 2, 32, 8
    layer = g.Layer(H, H, D, torch.bfloat16)
    pool = gi.states(2, H, D, seed=101).cuda()
    buf = torch.zeros(2, rows, H, D, dtype=torch.bfloat16, device="cuda")
    ab = torch.full((2, rows, H), 0.5, device="cuda")
    q_new = torch.zeros(4, max_new, H, D, dtype=torch.bfloat16, device="cuda")
    o = torch.full((4, max_new, H, D), 7.0, device="cuda")
    o_before = o.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device="cuda")
    say("replay bad counts")
    # logged + new past the log, new past max_new, a negative count, a slot out of range
    g.replay_forward(layer, pool, i32([0, 1, 0, 5]), buf, buf, ab, ab, i32([30, 0, -1, 0]), i32([3, 9, 2, 1]),
                     q_new, o, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 << 8
    assert same_bits(o, o_before)


# ------------------------------------------------------------------------- conv

@pytest.mark.parametrize("dtype,act", [(torch.bfloat16, 1), (torch.float32, 1), (torch.bfloat16, 0)])
def test_conv_matches_oracle_with_tails_and_checkpoints(g, dtype, act):
    Hqk, Hv, D, block = 2, 4, 16, 16
    layer = g.Layer(Hqk, Hv, D, dtype, conv_act=act)
    C = layer.conv_channels
    lens = [37, 64, 5, 2, 0, 130]
    starts = [0, 100, 32, 7, 9, 16]
    kinds = ["zero", "slot", "checkpoint", "slot", "slot", "checkpoint"]
    say(f"conv {dtype} act={act} lens={lens}")
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    x, w = gi.conv_inputs(cu[-1], C, 4, dtype, seed=91)
    tails0 = gi.conv_tail(len(lens), C, 4, dtype, seed=92)
    n_b = [oracle.count_boundaries(s, L, block) for s, L in zip(starts, lens)]
    pool = make_pool(g, layer, sum(n_b) + len(lens), block)
    # checkpoint sources: the tail region of a page
    src_pages = list(range(sum(n_b), sum(n_b) + len(lens)))
    for i, kd in enumerate(kinds):
        if kd == "checkpoint":
            pool.tail_view(src_pages[i], layer).copy_(tails0[i].cuda())
    xd, wd = x.cuda(), w.cuda()
    td = tails0.cuda()
    out_t = nan_fill_(torch.empty(len(lens), 3, C, dtype=dtype, device="cuda"))
    refs = []
    for i, kd in enumerate(kinds):
        src = None if kd == "zero" else (td[i] if kd == "slot" else pool.page_ptr(src_pages[i]))
        refs.append((kd, src, out_t[i]))
    y = nan_fill_(torch.empty(cu[-1], C, dtype=dtype, device="cuda"))
    g.conv_update(layer, xd, wd, refs, cu, starts, y, ckpt=pool, page_ids=list(range(sum(n_b))))
    torch.cuda.synchronize()
    off = 0
    for i, (s, L) in enumerate(zip(starts, lens)):
        r0 = cu[i]
        tail_in = None if kinds[i] == "zero" else f64(tails0[i])
        y_ref, t_ref, ck_ref = oracle.conv(f64(x[r0:r0 + L]), f64(w), tail_in, act, s, block)
        if L:
            if dtype == torch.bfloat16:
                assert rel_l2(f64(y[r0:r0 + L]), oracle.bf16_round(y_ref)) <= 1e-3
            else:
                assert rel_l2(f64(y[r0:r0 + L]), y_ref) <= 1e-5
        assert np.array_equal(f64(out_t[i]), t_ref), i
        for j in range(n_b[i]):
            assert np.array_equal(f64(pool.tail_view(off + j, layer)), ck_ref[j]), (i, j)
        off += n_b[i]


# ------------------------------------------------------------------------- staged tables

def test_staged_tables_match_inline_solo_runs(g):
    """Batches past the kernel-argument capacity (12 sequences; one sequence with 300
    block boundaries) copy their tables from a caller-owned pinned staging buffer.  Every
    sequence's outputs, final state and checkpoints equal its solo run (whose small
    table travels inline) bit for bit, and the conv over 20 sequences matches too."""
    D, H, dtype, block = 64, 2, torch.bfloat16, 16
    layer = g.Layer(H, H, D, dtype)
    lens = [40, 0, 17, 64, 1, 33, 80, 5, 48, 16, 31, 70]
    starts = [0, 0, 32, 0, 15, 0, 48, 0, 16, 0, 0, 64]
    assert len(lens) > g.INLINE_SEQS
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    T = cu[-1]
    say(f"staged tables: {len(lens)} sequences")
    q, k, v, a, b = gi.qkvab(T, H, H, D, dtype, seed=301)
    qd, kd, vd, ad, bd = _dev(q, k, v, a, b)
    S0 = gi.states(len(lens), H, D, seed=302).cuda()
    n_b = [oracle.count_boundaries(s, L, block) for s, L in zip(starts, lens)]
    pool = make_pool(g, layer, 2 * sum(n_b), block)
    need = g.prefill_staging_bytes(layer, cu, starts, block)
    assert need > 0
    staging = g.pinned_staging(need)
    o = torch.empty(T, H, D, device="cuda")
    Sf = torch.empty(len(lens), H, D, D, device="cuda")
    refs = [("zero" if s == 0 else "slot", None if s == 0 else S0[i], Sf[i]) for i, s in enumerate(starts)]
    g.chunk_prefill(layer, qd, kd, vd, ad, bd, cu, starts, refs, o, ckpt=pool, page_ids=list(range(sum(n_b))),
                    staging=staging)
    torch.cuda.synchronize()
    base = sum(n_b)
    for i, (s, L) in enumerate(zip(starts, lens)):
        r0 = cu[i]
        o1 = torch.empty(max(L, 1), H, D, device="cuda")
        S1 = torch.empty(H, D, D, device="cuda")
        ref = ("zero" if s == 0 else "slot", None if s == 0 else S0[i], S1)
        sl = slice(r0, r0 + L) if L else slice(0, 0)
        g.chunk_prefill(layer, qd[sl] if L else qd, kd[sl] if L else kd, vd[sl] if L else vd,
                        ad[sl] if L else ad, bd[sl] if L else bd, [0, L], [s], [ref], o1, ckpt=pool,
                        page_ids=list(range(base, base + n_b[i])))
        torch.cuda.synchronize()
        if L:
            assert same_bits(o1[:L], o[r0:r0 + L]), i
        assert same_bits(S1, Sf[i]), i
        off = sum(n_b[:i])
        for j in range(n_b[i]):
            assert torch.equal(pool.pool[base + j, :layer.state_bytes], pool.pool[off + j, :layer.state_bytes])

    # one sequence crossing 300 boundaries: more pages than the arguments carry
    L = 300 * block + 7
    q2, k2, v2, a2, b2 = _dev(*gi.qkvab(L, H, H, D, dtype, seed=303))
    pool2 = make_pool(g, layer, 300, block)
    assert g.prefill_staging_bytes(layer, [0, L], [0], block) > 0
    o2 = torch.empty(L, H, D, device="cuda")
    S2 = torch.empty(H, D, D, device="cuda")
    st2 = g.pinned_staging(g.prefill_staging_bytes(layer, [0, L], [0], block))
    ids = [int(p) for p in gi.permutation(300, 304)]
    g.chunk_prefill(layer, q2, k2, v2, a2, b2, [0, L], [0], [("zero", None, S2)], o2, ckpt=pool2, page_ids=ids,
                    staging=st2)
    torch.cuda.synchronize()
    o_ref, S_ref, ck_ref = oracle.recurrence(f64(q2), f64(k2), f64(v2), f64(a2), f64(b2), 1.0, None, 0, block)
    assert rel_l2(f64(o2), o_ref) <= TOL[dtype] and rel_l2(f64(S2), S_ref) <= TOL[dtype]
    errs = [rel_l2(f64(pool2.state_view(ids[i], layer)), ck_ref[i]) for i in range(300)]
    assert max(errs) <= TOL[dtype], int(np.argmax(errs))

    # the conv over 20 sequences, staged, against the oracle
    lc = g.Layer(1, 1, 16, dtype)
    C = lc.conv_channels
    clens = [(7 * i) % 23 for i in range(20)]
    ccu = np.concatenate([[0], np.cumsum(clens)]).tolist()
    x, w = gi.conv_inputs(ccu[-1], C, 4, dtype, seed=305)
    tails0 = gi.conv_tail(20, C, 4, dtype, seed=306)
    tout = torch.empty(20, 3, C, dtype=dtype, device="cuda")
    cst = [5 + i for i in range(20)]
    y = torch.empty(max(ccu[-1], 1), C, dtype=dtype, device="cuda")
    need = g.conv_staging_bytes(lc, ccu, cst, 0)
    assert need > 0
    g.conv_update(lc, x.cuda(), w.cuda(), [("slot", tails0[i].cuda(), tout[i]) for i in range(20)], ccu, cst, y,
                  ckpt=g.no_checkpoints(), staging=g.pinned_staging(need))
    torch.cuda.synchronize()
    for i in range(20):
        sl = slice(ccu[i], ccu[i + 1])
        y_ref, t_ref, _ = oracle.conv(f64(x[sl]), f64(w), f64(tails0[i]), 1, cst[i], 0)
        if clens[i]:
            assert rel_l2(f64(y[sl]), oracle.bf16_round(y_ref)) <= 1e-3, i
        assert np.array_equal(f64(tout[i]), t_ref), i
