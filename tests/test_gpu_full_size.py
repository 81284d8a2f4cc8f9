"""GPU parity at the workloads' full sizes, in the launch configuration the bench times
(pre-pass and scan as separate calls for the prefill).

The fp64 oracle covers every value head, checkpoint, conv channel and decode request of
the 27B-shaped workloads (heads, channels and requests are independent, so the oracle
computes each exactly as it sits inside the full problem); the 229,376-token prefill is
checked on 16 heads spread over the layer, at every one of its 256 checkpoints.  Every
comparison asserts the relative L2 error per head (or per channel block, per request,
per checkpoint) beside the tensor-wide one, so one wrong head cannot hide under the
norm of the others.  Bit-exactness checks (resume against cold runs) cover every head.
"""
import gc

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import TOL, assert_close_per, f64, make_pool, rel_l2, same_bits, say
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_recurrent_chunk_amd as lib
    return lib


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _prefill_staged(g, layer, q, k, v, a, b, cu, starts, states, o, pool, page_ids, block):
    """The bench's launch configuration: the pre-pass, then the scan."""
    ws = torch.empty(g.prefill_workspace_bytes(layer, cu, starts, block), dtype=torch.uint8, device="cuda")
    g.prefill_factorize(layer, q, k, a, b, cu, starts, block, ws)
    g.prefill_scan(layer, q, k, v, cu, starts, states, o, ws, ckpt=pool, page_ids=page_ids)
    return ws


def test_prefill_27b_full_size_all_heads(g):
    w = gi.PREFILL_27B
    T, H, D, block = w.total_tokens, w.n_v_heads, w.head_dim, w.block
    say(f"full-size prefill {w.name}")
    layer = g.Layer(H, H, D, w.io_dtype)
    q, k, v, a, b = gi.qkvab(T, H, H, D, w.io_dtype, seed=w.seed)
    n_ck = oracle.count_boundaries(0, T, block)
    assert n_ck == 9
    pool = make_pool(g, layer, n_ck + 2, block)
    page_ids = [int(p) for p in gi.permutation(n_ck + 2, w.seed)[:n_ck]]
    qd, kd, vd, ad, bd = (t.cuda() for t in (q, k, v, a, b))
    o = torch.empty(T, H, D, device="cuda")
    S = torch.empty(H, D, D, device="cuda")
    _prefill_staged(g, layer, qd, kd, vd, ad, bd, [0, T], [0], [("zero", None, S)], o, pool, page_ids, block)
    torch.cuda.synchronize()
    say("full-size prefill: oracle on all 48 heads")
    o_ref, S_ref, ck_ref = oracle.recurrence(f64(q), f64(k), f64(v), f64(a), f64(b), 1.0, None, 0, block)
    tol = TOL[w.io_dtype]
    assert_close_per(f64(o), o_ref, tol, 1, "o per head")
    assert_close_per(f64(S), S_ref, tol, 0, "final state per head")
    for i in range(n_ck):
        assert_close_per(f64(pool.state_view(page_ids[i], layer)), ck_ref[i], tol, 0, f"checkpoint {i} per head")
    assert torch.isfinite(o).all() and torch.isfinite(S).all()


def test_conv_27b_full_size_all_channels(g):
    w = gi.PREFILL_27B
    T, block = w.total_tokens, w.block
    layer = g.Layer(w.n_qk_heads, w.n_v_heads, w.head_dim, w.io_dtype)
    C = layer.conv_channels
    say(f"full-size conv {T} x {C}")
    x, wt = gi.conv_inputs(T, C, 4, w.io_dtype, seed=w.seed)
    n_ck = oracle.count_boundaries(0, T, block)
    pool = make_pool(g, layer, n_ck, block)
    xd, wd = x.cuda(), wt.cuda()
    y = torch.empty_like(xd)
    tail_d = torch.empty(3, C, dtype=w.io_dtype, device="cuda")
    g.conv_update(layer, xd, wd, [("zero", None, tail_d)], [0, T], [0], y, ckpt=pool, page_ids=list(range(n_ck)))
    torch.cuda.synchronize()
    tol = TOL[w.io_dtype]
    yc, tc = y.cpu(), tail_d.cpu()
    tails = [pool.tail_view(i, layer).cpu() for i in range(n_ck)]
    # every channel, in blocks of 1,024 (one q, k or v head group each at d = 128): the
    # error per block and per channel inside it
    for c0 in range(0, C, 1024):
        sel = slice(c0, min(C, c0 + 1024))
        y_ref, t_ref, ck_ref = oracle.conv(f64(x[:, sel]), f64(wt[sel]), None, 1, 0, block)
        assert_close_per(f64(yc[:, sel]), oracle.bf16_round(y_ref), tol, 1, f"conv channels {c0}..")
        # raw rows are copied, so tails are exact
        assert np.array_equal(f64(tc[:, sel]), t_ref), c0
        for i in range(n_ck):
            assert np.array_equal(f64(tails[i][:, sel]), ck_ref[i]), (c0, i)


def test_varlen_27b_stepped_resume_is_bit_identical_to_cold(g):
    """Four sequences of 2,688 / 5,000 / 6,272 / 12,000 tokens at the 27B layer, processed
    in steps of at most floor_chunk(2048, 896) = 1,792 tokens per sequence per call, with
    checkpoints written by one call and read by the next.  Sequences 1 and 3 share a
    seeded common prefix of 3,000 tokens, of which the cache rule keeps 1,792 (two
    blocks), and each resumes at block 2 from the page the other one's cold run wrote
    (a writer of a different length, the case the prefix-cache page traces).  Every
    output row, final state and checkpoint page must equal the sequence's cold solo run
    bit for bit."""
    w = gi.VARLEN_27B
    H, D, block, dtype = w.n_v_heads, w.head_dim, w.block, w.io_dtype
    lens = list(w.seqlens)
    step = g.floor_chunk(2048, block)
    assert step == 1792
    layer = g.Layer(H, H, D, dtype)
    say(f"varlen stepped resume lens={lens} step={step}")
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    q, k, v, a, b = gi.qkvab(cu[-1], H, H, D, dtype, seed=w.seed)
    # the common prefix of sequences 1 and 3, and the tokens of it a cache hit keeps
    shared = 3000
    assert g.cached_prefix_tokens(shared, block) == step
    for t_ in (q, k, v, a, b):
        t_[cu[3]:cu[3] + shared] = t_[cu[1]:cu[1] + shared]
    qd, kd, vd, ad, bd = (t_.cuda() for t_ in (q, k, v, a, b))
    n_b = [oracle.count_boundaries(0, L, block) for L in lens]
    pool = make_pool(g, layer, 2 * sum(n_b) + 64, block)
    next_page = 0

    def take(n):
        nonlocal next_page
        ids = list(range(next_page, next_page + n))
        next_page += n
        return ids

    def rows(t_, i, lo, hi):
        return t_[cu[i] + lo:cu[i] + hi]

    # cold solo runs: outputs, final states, and the page of every boundary
    cold_o, cold_S, cold_pages = [], [], []
    for i, L in enumerate(lens):
        o1 = torch.empty(L, H, D, device="cuda")
        S1 = torch.empty(H, D, D, device="cuda")
        ids = take(n_b[i])
        _prefill_staged(g, layer, rows(qd, i, 0, L), rows(kd, i, 0, L), rows(vd, i, 0, L), rows(ad, i, 0, L),
                        rows(bd, i, 0, L), [0, L], [0], [("zero", None, S1)], o1, pool, ids, block)
        cold_o.append(o1)
        cold_S.append(S1)
        cold_pages.append(ids)
    # 1 and 3 resume from the block-2 page the other's cold run wrote
    pos = [0, step, 0, step]
    src = [None, pool.page_ptr(cold_pages[3][1]), None, pool.page_ptr(cold_pages[1][1])]
    outs = [[] for _ in lens]
    Sfin = torch.empty(len(lens), H, D, D, device="cuda")
    written = [dict() for _ in lens]  # boundary index -> page
    while any(pos[i] < lens[i] for i in range(len(lens))):
        live = [i for i in range(len(lens)) if pos[i] < lens[i]]
        spans = [(i, pos[i], min(step, lens[i] - pos[i])) for i in live]
        qs = torch.cat([rows(qd, i, p0, p0 + n) for i, p0, n in spans])
        ks = torch.cat([rows(kd, i, p0, p0 + n) for i, p0, n in spans])
        vs = torch.cat([rows(vd, i, p0, p0 + n) for i, p0, n in spans])
        as_ = torch.cat([rows(ad, i, p0, p0 + n) for i, p0, n in spans])
        bs = torch.cat([rows(bd, i, p0, p0 + n) for i, p0, n in spans])
        cu_s = np.concatenate([[0], np.cumsum([n for _, _, n in spans])]).tolist()
        starts = [p0 for _, p0, _ in spans]
        refs = [("zero", None, Sfin[i]) if src[i] is None else ("checkpoint", src[i], Sfin[i])
                for i, _, _ in spans]
        ids, firsts = [], []
        for i, p0, n in spans:
            nb = oracle.count_boundaries(p0, n, block)
            new = take(nb)
            for j, pid in enumerate(new):
                written[i][(p0 // block) + j + 1] = pid
            ids += new
        o = torch.empty(cu_s[-1], H, D, device="cuda")
        _prefill_staged(g, layer, qs, ks, vs, as_, bs, cu_s, starts, refs, o, pool, ids, block)
        for j, (i, p0, n) in enumerate(spans):
            outs[i].append(o[cu_s[j]:cu_s[j + 1]])
            pos[i] = p0 + n
            src[i] = pool.page_ptr(written[i][pos[i] // block]) if pos[i] % block == 0 else None
            assert src[i] is not None or pos[i] == lens[i]
    torch.cuda.synchronize()
    first = [0, step, 0, step]
    for i, L in enumerate(lens):
        o_all = torch.cat(outs[i])
        assert same_bits(o_all, cold_o[i][first[i]:]), f"outputs of sequence {i}"
        assert same_bits(Sfin[i], cold_S[i]), f"final state of sequence {i}"
        for bidx, pid in written[i].items():
            cold_pid = cold_pages[i][bidx - 1]
            assert torch.equal(pool.pool[pid, :layer.state_bytes], pool.pool[cold_pid, :layer.state_bytes]), (i, bidx)
    # and every cold run agrees with the oracle on every head, at every checkpoint
    for i, L in enumerate(lens):
        say(f"varlen: oracle on sequence {i}, all heads")
        sl = slice(cu[i], cu[i + 1])
        o_ref, S_ref, ck_ref = oracle.recurrence(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(a[sl]), f64(b[sl]), 1.0,
                                                 None, 0, block)
        assert_close_per(f64(cold_o[i]), o_ref, TOL[dtype], 1, f"sequence {i} o per head")
        assert_close_per(f64(cold_S[i]), S_ref, TOL[dtype], 0, f"sequence {i} state per head")
        for j, pid in enumerate(cold_pages[i]):
            assert_close_per(f64(pool.state_view(pid, layer)), ck_ref[j], TOL[dtype], 0, f"sequence {i} ckpt {j}")
        del o_ref


@pytest.mark.parametrize("counts,rows", [("uniform", None), (16, None), (17, None), (32, 64), (33, 64)])
def test_flush_4b_full_size_all_heads(g, counts, rows):
    """The flush at the 4B shape: 32-slot log (the pages' size) and a 64-slot log whose
    33 accepted rows take two 32-row blocks."""
    w = gi.FLUSH_4B
    n_req, H, D = w["n_req"], w["n_heads"], w["head_dim"]
    rows = rows or w["buf_rows"]
    layer = g.Layer(16, H, D, torch.bfloat16)
    acc = gi.accepted_counts(n_req, w["seed"]) if counts == "uniform" else torch.full((n_req,), counts, dtype=torch.int32)
    say(f"full-size flush counts={acc.tolist()}")
    n_slots = n_req + 2
    pool = gi.states(n_slots, H, D, seed=w["seed"])
    _, bk, bv, ba, bb = gi.qkvab(n_slots * rows, 16, H, D, torch.bfloat16, seed=w["seed"])
    bk, bv = bk.view(n_slots, rows, 16, D), bv.view(n_slots, rows, H, D)
    ba, bb = ba.view(n_slots, rows, H), bb.view(n_slots, rows, H)
    slots = torch.tensor(list(range(1, n_req + 1)), dtype=torch.int32)  # slot 0 and the last stay untouched
    pd = pool.cuda()
    g.replay_flush(layer, pd, slots.cuda(), bk.cuda(), bv.cuda(), ba.cuda(), bb.cuda(), acc.cuda())
    torch.cuda.synchronize()
    out = pd.cpu()
    assert torch.equal(out[0], pool[0]) and torch.equal(out[-1], pool[-1])
    for r in range(n_req):
        n = int(acc[r])
        sl = r + 1
        _, S_ref, _ = oracle.recurrence(None, f64(bk[sl, :n]), f64(bv[sl, :n]), f64(ba[sl, :n]), f64(bb[sl, :n]),
                                        1.0, f64(pool[sl]), want_o=False, threads=8)
        assert rel_l2(f64(out[r + 1]), S_ref) <= TOL[torch.bfloat16], r


def test_replay_4b_full_size_all_heads(g):
    """Replay outputs at the flush workload's shape: 16 requests x 32 heads, a 32-slot log
    holding the accepted rows (1..16 per request) and 16 new rows behind them."""
    w = gi.FLUSH_4B
    n_req, H, D, rows = w["n_req"], w["n_heads"], w["head_dim"], w["buf_rows"]
    n_new = 16
    layer = g.Layer(16, H, D, torch.bfloat16)
    logged = gi.accepted_counts(n_req, w["seed"])
    say(f"full-size replay logged={logged.tolist()} new={n_new}")
    pool = gi.states(n_req, H, D, seed=w["seed"])
    _, bk, bv, ba, bb = gi.qkvab(n_req * rows, 16, H, D, torch.bfloat16, seed=w["seed"])
    bk, bv = bk.view(n_req, rows, 16, D), bv.view(n_req, rows, H, D)
    ba, bb = ba.view(n_req, rows, H), bb.view(n_req, rows, H)
    qn, _, _, _, _ = gi.qkvab(n_req * n_new, 16, H, D, torch.bfloat16, seed=w["seed"] + 1)
    qn = qn.view(n_req, n_new, 16, D)
    pd = pool.cuda()
    o = torch.empty(n_req, n_new, H, D, device="cuda")
    slots = torch.arange(n_req, dtype=torch.int32)
    g.replay_forward(layer, pd, slots.cuda(), bk.cuda(), bv.cuda(), ba.cuda(), bb.cuda(), logged.cuda(),
                     torch.full((n_req,), n_new, dtype=torch.int32).cuda(), qn.cuda(), o)
    torch.cuda.synchronize()
    assert torch.equal(pd.cpu(), pool)
    out = o.cpu()
    for r in range(n_req):
        m = int(logged[r])
        o_ref = oracle.replay_outputs(f64(pool[r]), f64(bk[r]), f64(bv[r]), f64(ba[r]), f64(bb[r]), m, f64(qn[r]))
        assert rel_l2(f64(out[r]), o_ref) <= TOL[torch.bfloat16], r


def test_long_27b_prefill_then_decode(g):
    """229,376 tokens at the 27B layer (256 checkpoints), then 256 concurrent decode
    requests.  The oracle checks 16 heads of the prefill over every token and boundary,
    and every decode request on every head."""
    w = gi.LONG_27B
    T, H, D, block = w.total_tokens, w.n_v_heads, w.head_dim, w.block
    layer = g.Layer(H, H, D, w.io_dtype)
    say(f"long prefill {w.name}")
    qd, kd, vd, ad, bd = gi.qkvab_device(T, H, H, D, w.io_dtype, seed=w.seed)
    n_ck = oracle.count_boundaries(0, T, block)
    assert n_ck == 256
    pool = make_pool(g, layer, n_ck, block)
    o = torch.empty(T, H, D, device="cuda")
    S = torch.empty(H, D, D, device="cuda")
    ws = _prefill_staged(g, layer, qd, kd, vd, ad, bd, [0, T], [0], [("zero", None, S)], o, pool,
                         list(range(n_ck)), block)
    torch.cuda.synchronize()
    del ws
    tol = TOL[w.io_dtype]
    # 16 heads spread over the layer, in two groups of 8 (bounded host memory), at every
    # token and every one of the 256 checkpoints
    heads_all = [0, 3, 7, 10, 14, 17, 21, 24, 27, 30, 33, 36, 39, 42, 45, 47]
    for grp in (heads_all[:8], heads_all[8:]):
        say(f"long prefill: oracle on heads {grp}")
        hsel = torch.tensor(grp, device="cuda")
        qh, kh, vh = (t_.index_select(1, hsel).cpu() for t_ in (qd, kd, vd))
        ah, bh = ad.index_select(1, hsel).cpu(), bd.index_select(1, hsel).cpu()
        o_ref, S_ref, ck_ref = oracle.recurrence(f64(qh), f64(kh), f64(vh), f64(ah), f64(bh), 1.0, None, 0, block,
                                                 threads=len(grp))
        del qh, kh, vh
        assert_close_per(f64(o.index_select(1, hsel)), o_ref, tol, 1, f"long o, heads {grp}")
        del o_ref
        assert_close_per(f64(S.index_select(0, hsel)), S_ref, tol, 0, f"long final state, heads {grp}")
        for i in range(n_ck):
            assert_close_per(f64(pool.state_view(i, layer).index_select(0, hsel)), ck_ref[i], tol, 0,
                             f"long checkpoint {i}, heads {grp}")
        del ck_ref
    del qd, kd, vd, ad, bd, o
    torch.cuda.empty_cache()

    d = gi.DECODE_27B
    n_req = d["n_req"]
    say(f"decode {n_req} requests")
    states = gi.states(n_req, H, D, seed=d["seed"])
    states[0] = S.cpu()  # request 0 continues the long sequence
    dq, dk, dv, da, db = gi.qkvab(n_req, H, H, D, w.io_dtype, seed=d["seed"])
    sp = states.cuda()
    dout = torch.empty(n_req, H, D, device="cuda")
    g.decode_step(layer, dq.cuda(), dk.cuda(), dv.cuda(), da.cuda(), db.cuda(), sp,
                  torch.arange(n_req, dtype=torch.int32, device="cuda"), dout)
    torch.cuda.synchronize()
    out, spc = dout.cpu(), sp.cpu()
    # every request, each on every head
    for r in range(n_req):
        o_ref, S_ref, _ = oracle.recurrence(f64(dq[r:r + 1]), f64(dk[r:r + 1]), f64(dv[r:r + 1]), f64(da[r:r + 1]),
                                            f64(db[r:r + 1]), 1.0, f64(states[r]))
        assert_close_per(f64(out[r]), o_ref[0], tol, 0, f"decode request {r} o per head")
        assert_close_per(f64(spc[r]), S_ref, tol, 0, f"decode request {r} state per head")
