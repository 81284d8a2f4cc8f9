"""GPU parity on the paths and input domains the workload distributions never reach.

  * strided operands: the conv's packed [q | k | v] output rows read in place by the
    prefill and by decode_mixed (qk_stride = v_stride = conv channels), and packed rows
    at head dims 16..64 in both input dtypes (the register scan and the small-head
    pre-pass);
  * the conv's decode regime: many one-row sequences with tails in and out;
  * gates at the contract's edges (a = 2^-126, the smallest normal decay; a = 1; b
    exactly 0 or 1), keys far from unit norm (0.25 .. 4, with b |k|^2 <= 2, the range in
    which the update stays bounded) and runs of nearly parallel keys, through the
    prefill, the replay flush and the replay outputs at d = 128.

Every expected value comes from the fp64 oracle on the same seeded inputs; the chained
cases run the oracle's own chain (conv, head norm, bf16 rounding of the conv output,
recurrence), never a GPU intermediate.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import TOL, assert_close_per, f64, make_pool, nan_fill_, same_bits, say
from oracle import oracle

pytestmark = pytest.mark.gpu

D = 128
BF = torch.bfloat16


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_recurrent_chunk_amd as lib
    return lib


def _i32(xs):
    return torch.tensor(xs, dtype=torch.int32, device="cuda")


def _domain_inputs(domain, T, Hqk, Hv, seed):
    """q, k, v (bf16) and a, b (fp32) for one input domain."""
    q, k, v, a, b = gi.qkvab(T, Hqk, Hv, D, BF, seed=seed)
    if domain in ("edge_gates", "all"):
        a, b = gi.edge_gates(T, Hv, seed=seed)
    if domain in ("scaled_keys", "all"):
        k, n2 = gi.scaled_keys(T, Hqk, D, BF, seed=seed)
        group = Hv // Hqk
        n2v = n2.repeat_interleave(group, dim=1)
        # keep b |k|^2 <= 1.9: the update stays bounded
        b = torch.minimum(b, 1.9 / n2v).float().contiguous()
    if domain in ("collinear", "all"):
        k = gi.collinear_keys(T, Hqk, D, BF, seed=seed)
        if domain == "collinear":
            b = torch.where(b > 0.5, torch.ones_like(b), b)  # strong writes on parallel keys
    return q, k, v, a, b


DOMAINS = ["edge_gates", "scaled_keys", "collinear", "all"]


@pytest.mark.parametrize("domain", DOMAINS)
def test_prefill_edge_domains(g, domain):
    T, Hqk, Hv, block = 333, 1, 2, 128
    say(f"prefill domain={domain}")
    layer = g.Layer(Hqk, Hv, D, BF, scale=0.5)
    q, k, v, a, b = _domain_inputs(domain, T, Hqk, Hv, seed=201)
    S0 = gi.states(1, Hv, D, seed=202)[0]
    n_ck = oracle.count_boundaries(64, T, block)
    pool = make_pool(g, layer, 2 * n_ck + 1, block)
    qd, kd, vd, ad, bd = (t.cuda() for t in (q, k, v, a, b))
    o = torch.empty(T, Hv, D, device="cuda")
    S = torch.empty(Hv, D, D, device="cuda")
    g.chunk_prefill(layer, qd, kd, vd, ad, bd, [0, T], [64], [("slot", S0.cuda(), S)], o, ckpt=pool,
                    page_ids=list(range(n_ck)))
    torch.cuda.synchronize()
    o_ref, S_ref, ck_ref = oracle.recurrence(f64(q), f64(k), f64(v), f64(a), f64(b), 0.5, f64(S0), 64, block)
    tol = TOL[BF]
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    assert_close_per(f64(o), o_ref, tol, 1, f"{domain}: o per head")
    assert_close_per(f64(S), S_ref, tol, 0, f"{domain}: state per head")
    for i in range(n_ck):
        assert_close_per(f64(pool.state_view(i, layer)), ck_ref[i], tol, 0, f"{domain}: checkpoint {i}")
    # resume from the first checkpoint: bit-identical to the cold run
    s0 = block
    r0 = s0 - 64
    o2 = torch.empty(T - r0, Hv, D, device="cuda")
    S2 = torch.empty(Hv, D, D, device="cuda")
    g.chunk_prefill(layer, qd[r0:], kd[r0:], vd[r0:], ad[r0:], bd[r0:], [0, T - r0], [s0],
                    [("checkpoint", pool.page_ptr(0), S2)], o2, ckpt=pool,
                    page_ids=list(range(n_ck, n_ck + oracle.count_boundaries(s0, T - r0, block))))
    torch.cuda.synchronize()
    assert same_bits(o2, o[r0:]) and same_bits(S2, S)


def _log(domain, n_slots, rows, Hqk, Hv, seed):
    kk, vv, aa, bb = [], [], [], []
    for s in range(n_slots):
        _, k, v, a, b = _domain_inputs(domain, rows, Hqk, Hv, seed=seed + s)
        kk.append(k), vv.append(v), aa.append(a), bb.append(b)
    return torch.stack(kk), torch.stack(vv), torch.stack(aa), torch.stack(bb)


@pytest.mark.parametrize("domain,rows", [(d, 32) for d in DOMAINS] + [("all", 64)])
def test_flush_edge_domains(g, domain, rows):
    """64-slot logs take two 32-row blocks (both factorized at once at head dim >= 64)."""
    Hqk, Hv = 2, 4
    layer = g.Layer(Hqk, Hv, D, BF)
    slots, acc = [3, 0, 2, 1], ([32, 17, 16, 5] if rows == 32 else [64, 33, 40, 5])
    say(f"flush domain={domain} rows={rows}")
    pool0 = gi.states(4, Hv, D, seed=211)
    bk, bv, ba, bb = _log(domain, 4, rows, Hqk, Hv, seed=212)
    pool = pool0.cuda()
    g.replay_flush(layer, pool, _i32(slots), bk.cuda(), bv.cuda(), ba.cuda(), bb.cuda(), _i32(acc))
    torch.cuda.synchronize()
    out = pool.cpu()
    for s, n in zip(slots, acc):
        _, S_ref, _ = oracle.recurrence(None, f64(bk[s, :n]), f64(bv[s, :n]), f64(ba[s, :n]), f64(bb[s, :n]), 1.0,
                                        f64(pool0[s]), want_o=False)
        assert torch.isfinite(out[s]).all()
        assert_close_per(f64(out[s]), S_ref, TOL[BF], 0, f"{domain}: slot {s} ({n} rows)")


@pytest.mark.parametrize("domain", DOMAINS)
def test_replay_edge_domains(g, domain):
    Hqk, Hv, rows, max_new = 2, 4, 32, 17
    layer = g.Layer(Hqk, Hv, D, BF, scale=0.5)
    reqs = [(3, 15, 17), (0, 0, 16), (2, 31, 1), (1, 8, 9)]
    say(f"replay domain={domain}")
    pool0 = gi.states(4, Hv, D, seed=221)
    bk, bv, ba, bb = _log(domain, 4, rows, Hqk, Hv, seed=222)
    qn = gi.qkvab(len(reqs) * max_new, Hqk, Hv, D, BF, seed=229)[0].view(len(reqs), max_new, Hqk, D)
    o = torch.zeros(len(reqs), max_new, Hv, D, device="cuda")
    g.replay_forward(layer, pool0.cuda(), _i32([r[0] for r in reqs]), bk.cuda(), bv.cuda(), ba.cuda(), bb.cuda(),
                     _i32([r[1] for r in reqs]), _i32([r[2] for r in reqs]), qn.cuda(), o)
    torch.cuda.synchronize()
    out = o.cpu()
    for i, (s, m, n) in enumerate(reqs):
        o_ref = oracle.replay_outputs(f64(pool0[s]), f64(bk[s]), f64(bv[s]), f64(ba[s]), f64(bb[s]), m,
                                      f64(qn[i, :n]), 0.5)
        assert torch.isfinite(out[i, :n]).all()
        assert_close_per(f64(out[i, :n]), o_ref, TOL[BF], 1, f"{domain}: request {i}")


# ------------------------------------------------------------------------- strided chains

def _oracle_conv_rows(x, w, tail, p0, block, Hqk):
    """The oracle's conv + SiLU + per-head q/k norm, rounded to bf16 as the conv stores it."""
    y, t, ck = oracle.conv(f64(x), f64(w), tail, 1, p0, block)
    return oracle.bf16_round(oracle.l2norm_qk_heads(y, Hqk, D)), t, ck


def test_conv_then_prefill_reads_packed_rows_in_place(g):
    """The packed core's chain: the conv (SiLU, q/k heads normalised) writes [q | k | v]
    rows; the prefill reads q, k and v straight out of those rows with
    qk_stride = v_stride = the conv's channel count."""
    Hqk, Hv, block = 2, 4, 128
    layer = g.Layer(Hqk, Hv, D, BF, scale=0.25, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    lens, starts = [200, 131], [0, 192]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    T = cu[-1]
    say(f"conv -> prefill strided lens={lens} starts={starts}")
    x, w = gi.conv_inputs(T, C, 4, BF, seed=231)
    tails0 = gi.conv_tail(2, C, 4, BF, seed=232)
    _, _, _, a, b = gi.qkvab(T, Hqk, Hv, D, BF, seed=233)
    S1 = gi.states(1, Hv, D, seed=234)[0]
    xd, wd = x.cuda(), w.cuda()
    y = nan_fill_(torch.empty(T, C, dtype=BF, device="cuda"))
    tail_out = torch.empty(2, 3, C, dtype=BF, device="cuda")
    n_b = [oracle.count_boundaries(s, L, block) for s, L in zip(starts, lens)]
    pool = make_pool(g, layer, sum(n_b), block)
    ids = list(range(sum(n_b)))
    g.conv_update(layer, xd, wd, [("zero", None, tail_out[0]), ("slot", tails0[1].cuda(), tail_out[1])], cu, starts,
                  y, ckpt=pool, page_ids=ids)
    qk = Hqk * D
    q_v, k_v, v_v = y[:, :qk], y[:, qk:2 * qk], y[:, 2 * qk:]
    o = torch.empty(T, Hv, D, device="cuda")
    Sf = torch.empty(2, Hv, D, D, device="cuda")
    g.chunk_prefill(layer, q_v, k_v, v_v, a.cuda(), b.cuda(), cu, starts,
                    [("zero", None, Sf[0]), ("slot", S1.cuda(), Sf[1])], o, ckpt=pool, page_ids=ids,
                    qk_stride=C, v_stride=C)
    torch.cuda.synchronize()
    for i, (s0, L) in enumerate(zip(starts, lens)):
        sl = slice(cu[i], cu[i + 1])
        yr, _, _ = _oracle_conv_rows(x[sl], w, None if i == 0 else f64(tails0[1]), s0, block, Hqk)
        qr = yr[:, :qk].reshape(L, Hqk, D)
        kr = yr[:, qk:2 * qk].reshape(L, Hqk, D)
        vr = yr[:, 2 * qk:].reshape(L, Hv, D)
        o_ref, S_ref, ck_ref = oracle.recurrence(qr, kr, vr, f64(a[sl]), f64(b[sl]), 0.25,
                                                 None if i == 0 else f64(S1), s0, block)
        assert_close_per(f64(o[sl]), o_ref, TOL[BF], 1, f"sequence {i} o")
        assert_close_per(f64(Sf[i]), S_ref, TOL[BF], 0, f"sequence {i} state")
        for j in range(n_b[i]):
            pid = sum(n_b[:i]) + j
            assert_close_per(f64(pool.state_view(pid, layer)), ck_ref[j], TOL[BF], 0, f"sequence {i} ckpt {j}")


def test_mixed_batch_decode_reads_conv_rows_through_strides(g):
    """A mixed batch in one packed conv output: 6 decode tokens (one-row conv sequences
    with their tails) and a prefill sequence; decode_mixed reads the decode rows and the
    prefill reads its rows, both in place through the conv's row stride."""
    Hqk, Hv, block = 2, 4, 64
    layer = g.Layer(Hqk, Hv, D, BF, scale=0.5, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    n_dec, Lp = 6, 150
    T = n_dec + Lp
    say("mixed batch strided")
    x, w = gi.conv_inputs(T, C, 4, BF, seed=241)
    tails0 = gi.conv_tail(n_dec, C, 4, BF, seed=242)
    _, _, _, a, b = gi.qkvab(T, Hqk, Hv, D, BF, seed=243)
    pool0 = gi.states(8, Hv, D, seed=244)
    dec_pos = [5, 63, 100, 127, 1000, 7]   # absolute positions of the decode tokens
    slots = [6, 1, -1, 3, 0, 7]
    cu = list(range(n_dec + 1)) + [T]
    starts = dec_pos + [0]
    td = tails0.cuda()
    tails_io = td.clone()
    P = torch.empty(Hv, D, D, device="cuda")
    ptail = torch.empty(3, C, dtype=BF, device="cuda")
    refs = [("slot", tails_io[i], tails_io[i]) for i in range(n_dec)] + [("zero", None, ptail)]
    y = nan_fill_(torch.empty(T, C, dtype=BF, device="cuda"))
    g.conv_update(layer, x.cuda(), w.cuda(), refs, cu, starts, y, ckpt=g.no_checkpoints())
    qk = Hqk * D
    q_v, k_v, v_v = y[:, :qk], y[:, qk:2 * qk], y[:, 2 * qk:]
    ad, bd = a.cuda(), b.cuda()
    o = torch.full((T, Hv, D), 555.0, device="cuda")
    pool = pool0.cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.decode_mixed(layer, q_v, k_v, v_v, ad, bd, pool, _i32(slots), _i32(list(range(n_dec))), o, status=status,
                   qk_stride=C, v_stride=C)
    pre = slice(n_dec, T)
    g.chunk_prefill(layer, q_v[pre], k_v[pre], v_v[pre], ad[pre], bd[pre], [0, Lp], [0], [("zero", None, P)],
                    o[pre], qk_stride=C, v_stride=C)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(n_dec):
        yr, t_ref, _ = _oracle_conv_rows(x[i:i + 1], w, f64(tails0[i]), dec_pos[i], 0, Hqk)
        assert np.array_equal(f64(tails_io[i]), t_ref), i
        if slots[i] < 0:
            assert (o[i] == 555.0).all()
            continue
        o_ref, S_ref, _ = oracle.recurrence(yr[:, :qk].reshape(1, Hqk, D), yr[:, qk:2 * qk].reshape(1, Hqk, D),
                                            yr[:, 2 * qk:].reshape(1, Hv, D), f64(a[i:i + 1]), f64(b[i:i + 1]), 0.5,
                                            f64(pool0[slots[i]]))
        assert_close_per(f64(o[i]), o_ref[0], TOL[BF], 0, f"decode token {i} o")
        assert_close_per(f64(pool[slots[i]]), S_ref, TOL[BF], 0, f"decode token {i} state")
    assert same_bits(pool[2], pool0[2].cuda()) and same_bits(pool[4], pool0[4].cuda()) and \
        same_bits(pool[5], pool0[5].cuda())
    yr, _, _ = _oracle_conv_rows(x[pre], w, None, 0, 0, Hqk)
    o_ref, S_ref, _ = oracle.recurrence(yr[:, :qk].reshape(Lp, Hqk, D), yr[:, qk:2 * qk].reshape(Lp, Hqk, D),
                                        yr[:, 2 * qk:].reshape(Lp, Hv, D), f64(a[pre]), f64(b[pre]), 0.5)
    assert_close_per(f64(o[pre]), o_ref, TOL[BF], 1, "prefill rows o")
    assert_close_per(f64(P), S_ref, TOL[BF], 0, "prefill state")


@pytest.mark.parametrize("dtype", [BF, torch.float32])
def test_conv_one_row_sequences(g, dtype):
    """The conv's decode regime: 256 one-row sequences, tails updated in place, a third
    of them landing on a block boundary (their checkpoint page gets the tail) and a few
    resuming from a checkpoint page's tail."""
    Hqk, Hv, Dd, block = 2, 4, 32, 64
    layer = g.Layer(Hqk, Hv, Dd, dtype)
    C = layer.conv_channels
    n = 256
    say(f"conv one-row sequences {dtype}")
    x, w = gi.conv_inputs(n, C, 4, dtype, seed=251)
    tails0 = gi.conv_tail(n, C, 4, dtype, seed=252)
    perm = gi.permutation(n, 253)
    # position of each token: p * block - 1 for a third (the row ends a block), a checkpoint
    # resume p * block for some, anything else for the rest
    starts, kinds = [], []
    for i in range(n):
        r = int(perm[i]) % 3
        if r == 0:
            starts.append(block * (1 + i % 5) - 1)
            kinds.append("slot")
        elif r == 1 and i % 4 == 0:
            starts.append(block * (1 + i % 3))
            kinds.append("checkpoint")
        else:
            starts.append(1 + i)
            kinds.append("slot")
    n_b = [oracle.count_boundaries(s, 1, block) for s in starts]
    n_src = kinds.count("checkpoint")
    pool = make_pool(g, layer, sum(n_b) + n_src, block)
    tails_io = tails0.cuda()
    refs, src_page = [], sum(n_b)
    for i in range(n):
        if kinds[i] == "checkpoint":
            pool.tail_view(src_page, layer).copy_(tails0[i].cuda())
            refs.append(("checkpoint", pool.page_ptr(src_page), tails_io[i]))
            src_page += 1
        else:
            refs.append(("slot", tails_io[i], tails_io[i]))
    y = nan_fill_(torch.empty(n, C, dtype=dtype, device="cuda"))
    cu = list(range(n + 1))
    g.conv_update(layer, x.cuda(), w.cuda(), refs, cu, starts, y, ckpt=pool, page_ids=list(range(sum(n_b))))
    torch.cuda.synchronize()
    yc, tc = f64(y), f64(tails_io)
    page = 0
    y_ref_all = np.zeros((n, C))
    for i in range(n):
        y_ref, t_ref, ck_ref = oracle.conv(f64(x[i:i + 1]), f64(w), f64(tails0[i]), 1, starts[i], block)
        y_ref_all[i] = y_ref[0]
        assert np.array_equal(tc[i], t_ref), i
        for j in range(n_b[i]):
            assert np.array_equal(f64(pool.tail_view(page, layer)), ck_ref[j]), (i, j)
            page += 1
    if dtype == BF:
        assert_close_per(yc, oracle.bf16_round(y_ref_all), 1e-3, 0, "one-row conv outputs per sequence")
    else:
        assert_close_per(yc, y_ref_all, 1e-5, 0, "one-row conv outputs per sequence")


@pytest.mark.parametrize("dtype,norm", [(BF, True), (torch.float32, False)])
def test_conv_decode_matches_oracle_and_one_row_conv(g, dtype, norm):
    """gdn_conv_decode: one new row per request, tails in a slot pool updated in place,
    rows of a packed batch in permuted order, a padding slot; against the oracle, and
    bit-identical to gdn_conv_update over the same tokens as one-row sequences."""
    Hqk, Hv, Dd = 2, 4, 64
    act = g.ACT_SILU | (g.CONV_QK_L2NORM if norm else 0)
    layer = g.Layer(Hqk, Hv, Dd, dtype, conv_act=act)
    C = layer.conv_channels
    n_req, n_rows, n_slots = 40, 45, 43
    say(f"conv decode {dtype} norm={norm}")
    x, w = gi.conv_inputs(n_rows, C, 4, dtype, seed=261)
    pool0 = gi.conv_tail(n_slots, C, 4, dtype, seed=262)
    slots = [int(s) for s in gi.permutation(n_slots, 263)[:n_req]]
    slots[7] = -1
    rows = [int(r) for r in gi.permutation(n_rows, 264)[:n_req]]
    xd, wd = x.cuda(), w.cuda()
    pool = pool0.cuda()
    y = nan_fill_(torch.empty(n_rows, C, dtype=dtype, device="cuda"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.conv_decode(layer, xd, wd, pool, _i32(slots), y, rows=_i32(rows), status=status)
    # the same tokens as one-row sequences of conv_update (tails as slot sources)
    pool_b = pool0.cuda()
    live = [i for i in range(n_req) if slots[i] >= 0]
    xs = xd[torch.tensor([rows[i] for i in live], device="cuda")].contiguous()
    y2 = torch.empty(len(live), C, dtype=dtype, device="cuda")
    refs = [("slot", pool_b[slots[i]], pool_b[slots[i]]) for i in live]
    g.conv_update(layer, xs, wd, refs, list(range(len(live) + 1)), [9] * len(live), y2, ckpt=g.no_checkpoints())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert same_bits(pool, pool_b)
    for j, i in enumerate(live):
        assert same_bits(y[rows[i]], y2[j]), i
    untouched = set(range(n_rows)) - {rows[i] for i in live}
    for r in untouched:
        assert same_bits(y[r], nan_fill_(torch.empty_like(y[r])))
    for s in set(range(n_slots)) - {slots[i] for i in live}:
        assert same_bits(pool[s], pool0[s].cuda())
    yc = f64(y)
    for i in live:
        y_ref, t_ref, _ = oracle.conv(f64(x[rows[i]:rows[i] + 1]), f64(w), f64(pool0[slots[i]]), 1, 9, 0)
        if norm:
            y_ref = oracle.l2norm_qk_heads(y_ref, Hqk, Dd)
        want = oracle.bf16_round(y_ref) if dtype == BF else y_ref
        from gpu_util import rel_l2
        assert rel_l2(yc[rows[i]:rows[i] + 1], want) <= TOL[dtype], i
        assert np.array_equal(f64(pool[slots[i]]), t_ref), i
    # a slot out of range and a row out of range leave everything untouched
    before, yb = pool.clone(), y.clone()
    g.conv_decode(layer, xd, wd, pool, _i32([n_slots, 0]), y, rows=_i32([0, n_rows]), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 << 8
    assert same_bits(pool, before) and same_bits(y, yb)


@pytest.mark.parametrize("d,dtype", [(16, BF), (32, BF), (64, BF), (16, torch.float32), (64, torch.float32)])
def test_prefill_reads_strided_rows_at_small_heads(g, d, dtype):
    """q, k and v as column ranges of one packed row buffer whose rows are wider than the
    heads (NaN in the unused columns), at head dims below 128 and both input dtypes, over
    ragged varlen chunks with checkpoints: every kernel of the prefill stays inside its
    heads' columns and follows the row stride."""
    Hqk, Hv, block = 2, 4, 64
    lens, starts = [150, 77], [0, 40]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    T = cu[-1]
    say(f"strided prefill d={d} {dtype}")
    q, k, v, a, b = gi.qkvab(T, Hqk, Hv, d, dtype, seed=241 + d)
    qk, vw = Hqk * d, Hv * d
    C = 2 * qk + vw + 8
    rows = torch.full((T, C), float("nan"), dtype=dtype)
    rows[:, :qk] = q.reshape(T, qk)
    rows[:, qk:2 * qk] = k.reshape(T, qk)
    rows[:, 2 * qk:2 * qk + vw] = v.reshape(T, vw)
    rd = rows.cuda()
    layer = g.Layer(Hqk, Hv, d, dtype, scale=0.5)
    S1 = gi.states(1, Hv, d, seed=242)[0]
    n_b = [oracle.count_boundaries(s, L, block) for s, L in zip(starts, lens)]
    pool = make_pool(g, layer, sum(n_b), block)
    ids = list(range(sum(n_b)))
    o = nan_fill_(torch.empty(T, Hv, d, device="cuda"))
    Sf = torch.empty(2, Hv, d, d, device="cuda")
    g.chunk_prefill(layer, rd[:, :qk], rd[:, qk:2 * qk], rd[:, 2 * qk:], a.cuda(), b.cuda(), cu, starts,
                    [("zero", None, Sf[0]), ("slot", S1.cuda(), Sf[1])], o, ckpt=pool, page_ids=ids,
                    qk_stride=C, v_stride=C)
    torch.cuda.synchronize()
    for i, (s0, L) in enumerate(zip(starts, lens)):
        sl = slice(cu[i], cu[i + 1])
        o_ref, S_ref, ck_ref = oracle.recurrence(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(a[sl]), f64(b[sl]), 0.5,
                                                 None if i == 0 else f64(S1), s0, block)
        assert_close_per(f64(o[sl]), o_ref, TOL[dtype], 1, f"d={d} sequence {i} o")
        assert_close_per(f64(Sf[i]), S_ref, TOL[dtype], 0, f"d={d} sequence {i} state")
        for j in range(n_b[i]):
            pid = sum(n_b[:i]) + j
            assert_close_per(f64(pool.state_view(pid, layer)), ck_ref[j], TOL[dtype], 0, f"d={d} sequence {i} ckpt {j}")
