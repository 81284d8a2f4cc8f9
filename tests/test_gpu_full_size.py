"""GPU parity at the workloads' full sizes, in the launch configuration the bench times
(pre-pass and scan as separate calls for the prefill).

The fp64 oracle runs on a sample of each workload: a few value heads, conv channels or
requests, which it computes exactly as they are computed inside the full problem
(heads, channels and requests are independent).  Bit-exactness checks (resume against
cold runs) cover every head.
"""
import gc

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import TOL, f64, make_pool, rel_l2, same_bits, say
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


def test_prefill_27b_full_size_sampled_heads(g):
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
    heads = [0, 17, 47]
    qs, ks, vs, as_, bs = (t[:, heads] for t in (q, k, v, a, b))
    o_ref, S_ref, ck_ref = oracle.recurrence(f64(qs), f64(ks), f64(vs), f64(as_), f64(bs), 1.0, None, 0, block,
                                             threads=len(heads))
    tol = TOL[w.io_dtype]
    assert rel_l2(f64(o[:, heads]), o_ref) <= tol
    assert rel_l2(f64(S[heads]), S_ref) <= tol
    for i in range(n_ck):
        assert rel_l2(f64(pool.state_view(page_ids[i], layer)[heads]), ck_ref[i]) <= tol, i
    assert torch.isfinite(o).all() and torch.isfinite(S).all()


def test_conv_27b_full_size_sampled_channels(g):
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
    # channels at the q | k | v seams, the ends, and a seeded spread
    kq = w.n_qk_heads * w.head_dim
    sel = sorted(set([0, 1, kq - 1, kq, 2 * kq - 1, 2 * kq, C - 1] +
                     [int(c) for c in gi.permutation(C, w.seed)[:249]]))
    y_ref, t_ref, ck_ref = oracle.conv(f64(x[:, sel]), f64(wt[sel]), None, 1, 0, block)
    tol = TOL[w.io_dtype]
    assert rel_l2(f64(y[:, sel]), oracle.bf16_round(y_ref)) <= tol
    # raw rows are copied, so tails are exact
    assert np.array_equal(f64(tail_d[:, sel]), t_ref)
    for i in range(n_ck):
        assert np.array_equal(f64(pool.tail_view(i, layer)[:, sel]), ck_ref[i]), i


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
    # and the longest sequence agrees with the oracle on two heads
    heads = [3, 40]
    i = 3
    sl = slice(cu[i], cu[i + 1])
    o_ref, S_ref, _ = oracle.recurrence(f64(q[sl][:, heads]), f64(k[sl][:, heads]), f64(v[sl][:, heads]),
                                        f64(a[sl][:, heads]), f64(b[sl][:, heads]), 1.0, None, 0, block,
                                        threads=2)
    assert rel_l2(f64(cold_o[i][:, heads]), o_ref) <= TOL[dtype]
    assert rel_l2(f64(cold_S[i][heads]), S_ref) <= TOL[dtype]


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
    requests.  The oracle checks one head of the prefill over every token and boundary,
    and three decode requests on all heads."""
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
    h = 5
    say("long prefill: oracle on one head")
    qh, kh, vh = (t_[:, h:h + 1].cpu() for t_ in (qd, kd, vd))
    ah, bh = ad[:, h:h + 1].cpu(), bd[:, h:h + 1].cpu()
    o_ref, S_ref, ck_ref = oracle.recurrence(f64(qh), f64(kh), f64(vh), f64(ah), f64(bh), 1.0, None, 0, block)
    tol = TOL[w.io_dtype]
    assert rel_l2(f64(o[:, h:h + 1]), o_ref) <= tol
    assert rel_l2(f64(S[h:h + 1]), S_ref) <= tol
    errs = [rel_l2(f64(pool.state_view(i, layer)[h:h + 1]), ck_ref[i]) for i in range(n_ck)]
    assert max(errs) <= tol, int(np.argmax(errs))
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
    for r in (0, 100, n_req - 1):
        o_ref, S_ref, _ = oracle.recurrence(f64(dq[r:r + 1]), f64(dk[r:r + 1]), f64(dv[r:r + 1]), f64(da[r:r + 1]),
                                            f64(db[r:r + 1]), 1.0, f64(states[r]), threads=8)
        assert rel_l2(f64(dout[r]), o_ref[0]) <= tol, r
        assert rel_l2(f64(sp[r]), S_ref) <= tol, r
