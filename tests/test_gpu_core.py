"""GPU parity of the packed core (gdn_core_prefill) and the conv reading packed rows.

"Hybrid linear attention (gated DeltaNet)", "Packed-core traces": the core takes the packed
qkvz rows plus the "ba" projection and returns gated-normalized value rows.  Row layout
(a reading; the page gives none): [q | k | v | z], the name's order, each head's d values
contiguous; ba = [b | a].

The expected values come from the oracle's chain on the same seeded inputs: conv + SiLU,
per-head q/k norm, bf16 rounding of the conv output (the core stores it in the io dtype),
gates, recurrence, gated norm.  No GPU intermediate enters the oracle.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import TOL, assert_close_per, f64, make_pool, nan_fill_, rel_l2, same_bits, say
from oracle import oracle

pytestmark = pytest.mark.gpu

D = 128
BF = torch.bfloat16


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_recurrent_chunk_amd as lib
    return lib


def _packed_rows(T, Hqk, Hv, pad, seed):
    """qkvz rows [T, C + Hv d + pad] (q | k | v channels as the conv's inputs, z as the
    gate rows, `pad` extra columns) and ba rows [T, 2 Hv + 3]; plus the layer weights."""
    C = 2 * Hqk * D + Hv * D
    x, w = gi.conv_inputs(T, C, 4, BF, seed=seed)
    ba, A_log, dt_bias, _, z, wn = gi.core_inputs(T, Hv, D, BF, seed=seed + 1)
    qkvz = torch.zeros(T, C + Hv * D + pad, dtype=BF)
    qkvz[:, :C] = x
    qkvz[:, C:C + Hv * D] = z.reshape(T, Hv * D)
    ba_rows = torch.zeros(T, 2 * Hv + 3, dtype=BF)
    ba_rows[:, :2 * Hv] = ba
    return qkvz, ba_rows, w, A_log, dt_bias, wn


def _oracle_core(qkvz, ba_rows, w, A_log, dt_bias, wn, Hqk, Hv, scale, eps, tail, S0, p0, block):
    """The oracle's chain for one sequence: (out [L, Hv, D] before its bf16 rounding,
    final state, checkpoint states, new tail, checkpoint tails)."""
    C = 2 * Hqk * D + Hv * D
    L = qkvz.shape[0]
    y, tail_out, ck_tails = oracle.conv(f64(qkvz[:, :C]), f64(w), tail, 1, p0, block)
    y = oracle.bf16_round(oracle.l2norm_qk_heads(y, Hqk, D))
    qk = Hqk * D
    a, b = oracle.gates(f64(ba_rows[:, :2 * Hv]), f64(A_log), f64(dt_bias), Hv)
    o, S, ck = oracle.recurrence(y[:, :qk].reshape(L, Hqk, D), y[:, qk:2 * qk].reshape(L, Hqk, D),
                                 y[:, 2 * qk:].reshape(L, Hv, D), a, b, scale, S0, p0, block)
    z = f64(qkvz[:, C:C + Hv * D]).reshape(L, Hv, D)
    out = oracle.gated_norm(o, z, f64(wn), eps)
    return out, S, ck, tail_out, ck_tails


# The output is stored in bf16: against the oracle's value rounded the same way, an
# element differs by one bf16 step (2^-8 relative) when the prefill's error (<= 1e-3)
# carries its exact value across a rounding boundary.  That happens for a fraction of
# elements of order 1e-3 / 2^-8 of the error, so the rel-L2 of the rounded outputs stays
# below 1e-3 + 2^-9.
OUT_TOL = 1e-3 + 2.0 ** -9


def test_core_prefill_matches_oracle_chain(g):
    """Three sequences: a cold start, a resume from a slot (state and tail), a resume from
    a checkpoint page (state and tail read from the page); packed rows with padding
    columns; checkpoints at every crossed 128-token boundary."""
    Hqk, Hv, block, scale, eps = 2, 4, 128, D ** -0.5, 1e-6
    layer = g.Layer(Hqk, Hv, D, BF, scale=scale, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    lens, starts = [200, 131, 190], [0, 192, 128]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    T = cu[-1]
    say(f"core prefill lens={lens} starts={starts}")
    qkvz, ba_rows, w, A_log, dt_bias, wn = _packed_rows(T, Hqk, Hv, 24, seed=301)
    S1 = gi.states(1, Hv, D, seed=302)[0]
    t1 = gi.conv_tail(1, C, 4, BF, seed=303)[0]
    S2 = gi.states(1, Hv, D, seed=304)[0]
    t2 = gi.conv_tail(1, C, 4, BF, seed=305)[0]
    n_b = [oracle.count_boundaries(s, L, block) for s, L in zip(starts, lens)]
    pool = make_pool(g, layer, sum(n_b) + 1, block)
    src_page = sum(n_b)  # the page sequence 2 resumes from
    pool.state_view(src_page, layer).copy_(S2.cuda())
    pool.tail_view(src_page, layer).copy_(t2.cuda())
    ids = list(range(sum(n_b)))
    S_out = nan_fill_(torch.empty(3, Hv, D, D, device="cuda"))
    tails_out = nan_fill_(torch.empty(3, 3, C, dtype=BF, device="cuda"))
    page = pool.page_ptr(src_page)
    states = [("zero", None, S_out[0]), ("slot", S1.cuda(), S_out[1]), ("checkpoint", page, S_out[2])]
    tails = [("zero", None, tails_out[0]), ("slot", t1.cuda(), tails_out[1]), ("checkpoint", page, tails_out[2])]
    out = nan_fill_(torch.empty(T, Hv, D, dtype=BF, device="cuda"))
    g.core_prefill(layer, qkvz.cuda(), ba_rows.cuda(), w.cuda(), A_log.cuda(), dt_bias.cuda(), wn.cuda(), cu,
                   starts, tails, states, out, ckpt=pool, page_ids=ids, eps=eps)
    torch.cuda.synchronize()
    srcs = [(None, None), (f64(t1), f64(S1)), (f64(t2), f64(S2))]
    for i, (s0, L) in enumerate(zip(starts, lens)):
        sl = slice(cu[i], cu[i + 1])
        out_ref, S_ref, ck_ref, tail_ref, ckt_ref = _oracle_core(qkvz[sl], ba_rows[sl], w, A_log, dt_bias, wn, Hqk,
                                                                 Hv, scale, eps, srcs[i][0], srcs[i][1], s0, block)
        got = f64(out[sl])
        assert rel_l2(got, oracle.bf16_round(out_ref)) <= OUT_TOL, f"sequence {i} out"
        for h in range(Hv):
            assert rel_l2(got[:, h], oracle.bf16_round(out_ref[:, h])) <= OUT_TOL, f"sequence {i} out head {h}"
        assert_close_per(f64(S_out[i]), S_ref, TOL[BF], 0, f"sequence {i} state")
        assert np.array_equal(f64(tails_out[i]), tail_ref), f"sequence {i} tail"
        for j in range(n_b[i]):
            pid = sum(n_b[:i]) + j
            assert_close_per(f64(pool.state_view(pid, layer)), ck_ref[j], TOL[BF], 0, f"sequence {i} ckpt {j}")
            assert np.array_equal(f64(pool.tail_view(pid, layer)), ckt_ref[j]), f"sequence {i} ckpt tail {j}"


def test_core_prefill_is_its_stages(g):
    """Ten sequences (past the kernel-argument table, so the staged tables of both the
    conv and the prefill run): the core's outputs, states, tails and pages are
    bit-identical to its four stages called one by one on the same rows."""
    Hqk, Hv, block, scale, eps = 1, 2, 64, 0.3, 1e-5
    layer = g.Layer(Hqk, Hv, D, BF, scale=scale, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    lens = [70, 1, 64, 130, 5, 200, 63, 65, 3, 128]
    starts = [0] * len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    T = cu[-1]
    say(f"core prefill == stages, {len(lens)} sequences")
    assert g.core_prefill_staging_bytes(layer, cu, starts, block) > 0
    qkvz, ba_rows, w, A_log, dt_bias, wn = [t.cuda() for t in _packed_rows(T, Hqk, Hv, 8, seed=311)]
    n_b = [oracle.count_boundaries(s, L, block) for s, L in zip(starts, lens)]
    outs = []
    for mode in ("core", "stages"):
        pool = make_pool(g, layer, sum(n_b), block)
        ids = list(range(sum(n_b)))
        S_out = torch.zeros(len(lens), Hv, D, D, device="cuda")
        t_out = torch.zeros(len(lens), 3, C, dtype=BF, device="cuda")
        states = [("zero", None, S_out[i]) for i in range(len(lens))]
        tails = [("zero", None, t_out[i]) for i in range(len(lens))]
        out = torch.zeros(T, Hv, D, dtype=BF, device="cuda")
        if mode == "core":
            g.core_prefill(layer, qkvz, ba_rows, w, A_log, dt_bias, wn, cu, starts, tails, states, out, ckpt=pool,
                           page_ids=ids, eps=eps)
        else:
            y = torch.empty(T, C, dtype=BF, device="cuda")
            g.conv_update(layer, qkvz[:, :C], w, tails, cu, starts, y, ckpt=pool, page_ids=ids)
            a = torch.empty(T, Hv, device="cuda")
            b = torch.empty(T, Hv, device="cuda")
            g.gates(layer, ba_rows, A_log, dt_bias, a, b)
            o = torch.empty(T, Hv, D, device="cuda")
            qk = Hqk * D
            g.chunk_prefill(layer, y[:, :qk], y[:, qk:2 * qk], y[:, 2 * qk:], a, b, cu, starts, states, o, ckpt=pool,
                            page_ids=ids, qk_stride=C, v_stride=C)
            g.gated_norm(layer, o, qkvz[:, C:C + Hv * D], wn, out, eps=eps)
        torch.cuda.synchronize()
        outs.append((out, S_out, t_out, pool.pool.clone()))
    for x, y_, what in zip(outs[0], outs[1], ("out", "states", "tails", "pages")):
        assert same_bits(x, y_), what
    # and the outputs against the oracle's chain, every sequence
    for i, L in enumerate(lens):
        sl = slice(cu[i], cu[i + 1])
        out_ref, S_ref, _, _, _ = _oracle_core(qkvz[sl].cpu(), ba_rows[sl].cpu(), w.cpu(), A_log.cpu(),
                                               dt_bias.cpu(), wn.cpu(), Hqk, Hv, scale, eps, None, None, 0, block)
        assert rel_l2(f64(outs[0][0][sl]), oracle.bf16_round(out_ref)) <= OUT_TOL, f"sequence {i} out"
        assert_close_per(f64(outs[0][1][i]), S_ref, TOL[BF], 0, f"sequence {i} state")


def test_core_prefill_refuses_bad_operands_and_enqueues_nothing(g):
    """Fail closed: a too-narrow packed row, a missing staging buffer past the inline
    tables, and an off-boundary checkpoint resume each return an error, and no output,
    state, tail or page changes."""
    Hqk, Hv, block = 1, 2, 64
    layer = g.Layer(Hqk, Hv, D, BF, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    T = 100
    qkvz, ba_rows, w, A_log, dt_bias, wn = [t.cuda() for t in _packed_rows(T, Hqk, Hv, 0, seed=321)]
    pool = make_pool(g, layer, 4, block)
    before = pool.pool.clone()
    S = torch.full((Hv, D, D), 7.0, device="cuda")
    tl = torch.full((3, C), 7.0, dtype=BF, device="cuda")
    out = torch.full((T, Hv, D), 7.0, dtype=BF, device="cuda")
    say("core prefill refusals")
    with pytest.raises(ValueError):
        g.core_prefill(layer, qkvz[:, :C + Hv * D - 8], ba_rows, w, A_log, dt_bias, wn, [0, T], [0],
                       [("zero", None, tl)], [("zero", None, S)], out, ckpt=pool, page_ids=[0])
    with pytest.raises(g.GdnError) as e:
        g.core_prefill(layer, qkvz, ba_rows, w, A_log, dt_bias, wn, [0, T], [32],
                       [("checkpoint", pool.page_ptr(0), tl)], [("checkpoint", pool.page_ptr(0), S)], out,
                       ckpt=pool, page_ids=[0, 1])
    assert g.STATUS_NAMES[e.value.status] == "GDN_ERR_OFF_BOUNDARY"
    lens = [10] * 10
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    refs = [("zero", None, tl)] * 10
    with pytest.raises(g.GdnError) as e:
        g.core_prefill(layer, qkvz, ba_rows, w, A_log, dt_bias, wn, cu, [0] * 10, refs,
                       [("zero", None, S)] * 10, out, ckpt=pool, page_ids=[], staging=torch.empty(0, dtype=torch.uint8))
    assert g.STATUS_NAMES[e.value.status] == "GDN_ERR_STAGING"
    torch.cuda.synchronize()
    assert (S == 7.0).all() and (tl == 7.0).all() and (out == 7.0).all()
    assert same_bits(pool.pool, before)


def test_conv_decode_reads_packed_rows(g):
    """The conv's decode regime on the q|k|v channels of packed qkvz rows (row stride
    wider than the channels): bit-identical to the same rows made dense, and equal to the
    oracle's one-row conv with the slot's tail."""
    Hqk, Hv = 2, 4
    layer = g.Layer(Hqk, Hv, D, BF, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    n = 9
    qkvz, _, w, _, _, _ = _packed_rows(n, Hqk, Hv, 16, seed=331)
    tails0 = gi.conv_tail(n, C, 4, BF, seed=332)
    slots = torch.tensor([3, 0, 8, 1, -1, 5, 2, 7, 4], dtype=torch.int32, device="cuda")
    say("conv decode packed rows")
    res = []
    for x in (qkvz.cuda()[:, :C], qkvz[:, :C].contiguous().cuda()):
        tp = tails0.cuda()
        y = nan_fill_(torch.empty(n, C, dtype=BF, device="cuda"))
        g.conv_decode(layer, x, w.cuda(), tp, slots, y)
        torch.cuda.synchronize()
        res.append((y, tp))
    keep = slots >= 0
    assert same_bits(res[0][0][keep], res[1][0][keep])
    assert same_bits(res[0][1], res[1][1])
    for r, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        y_ref, t_ref, _ = oracle.conv(f64(qkvz[r:r + 1, :C]), f64(w), f64(tails0[s]), 1, 0, 0)
        y_ref = oracle.l2norm_qk_heads(y_ref, Hqk, D)
        assert rel_l2(f64(res[0][0][r]), oracle.bf16_round(y_ref[0])) <= TOL[BF], r
        assert np.array_equal(f64(res[0][1][s]), t_ref), r
