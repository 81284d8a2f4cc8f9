"""gdn_chunk_prefill_noalloc against gdn_chunk_prefill: the entry point that allocates
nothing (its chunk factors live in the library's fixed per-device scratch array) gives
the workspace entry point's outputs, final states and checkpoints bit for bit, on two
calls in a row (the second smaller, so stale scratch contents from the first must not
matter), and refuses a batch beyond its capacity without touching anything."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import make_pool, same_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_recurrent_chunk_amd as lib
    return lib


def _run(g, layer, fn, q, k, v, a, b, cu, starts, S0, pool, page_ids):
    H, D = layer.n_v_heads, layer.head_dim
    T = cu[-1]
    o = torch.full((T, H, D), float("nan"), device="cuda")
    Sf = torch.empty(len(starts), H, D, D, device="cuda")
    refs = [("zero", None, Sf[i]) if s == 0 else ("slot", S0[i], Sf[i]) for i, s in enumerate(starts)]
    fn(layer, q, k, v, a, b, cu, starts, refs, o, ckpt=pool, page_ids=page_ids)
    return o, Sf


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 32)])
def test_noalloc_prefill_matches_workspace_prefill(g, dtype, D):
    H, block = 8, 128
    layer = g.Layer(H // 2, H, D, dtype, scale=0.5)
    # call 1: three sequences, 1,500 tokens; call 2: one sequence of 200 tokens
    for call, (lens, starts) in enumerate((([700, 513, 287], [0, 256, 0]), ([200], [128]))):
        say(f"noalloc call {call}: lens={lens} starts={starts} {dtype} D={D}")
        cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
        q, k, v, a, b = (t.cuda() for t in gi.qkvab(cu[-1], H // 2, H, D, dtype, seed=401 + call))
        S0 = gi.states(len(lens), H, D, seed=402 + call).cuda()
        n_b = sum(g.count_boundaries(s, L, block) for s, L in zip(starts, lens))
        ws_need = g.prefill_workspace_bytes(layer, cu, starts, block)
        assert 0 < ws_need <= g.NOALLOC_SCRATCH_BYTES
        pool_a = make_pool(g, layer, n_b, block)
        pool_b = make_pool(g, layer, n_b, block)
        ids = list(range(n_b))
        o1, S1 = _run(g, layer, g.chunk_prefill, q, k, v, a, b, cu, starts, S0, pool_a, ids)
        o2, S2 = _run(g, layer, g.chunk_prefill_noalloc, q, k, v, a, b, cu, starts, S0, pool_b, ids)
        torch.cuda.synchronize()
        assert same_bits(o1, o2), call
        assert same_bits(S1, S2), call
        assert torch.equal(pool_a.pool, pool_b.pool), call


def test_noalloc_prefill_refuses_batches_past_its_capacity(g):
    H, D, block = 48, 128, 896
    layer = g.Layer(H, H, D, torch.bfloat16)
    T = 8192  # 128 chunks x 48 heads of factor records: past the 64 MiB scratch
    assert g.prefill_workspace_bytes(layer, [0, T], [0], block) > g.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(T, H, D, dtype=torch.bfloat16, device="cuda")
    ab = torch.full((T, H), 0.5, device="cuda")
    o = torch.full((T, H, D), 3.0, device="cuda")
    S = torch.full((H, D, D), 7.0, device="cuda")
    with pytest.raises(g.GdnError) as e:
        g.chunk_prefill_noalloc(layer, q, q, q, ab, ab, [0, T], [0], [("zero", None, S)], o)
    assert g.STATUS_NAMES[e.value.status] == "GDN_ERR_CAPACITY"
    # nine sequences: a table past the kernel arguments
    with pytest.raises(g.GdnError) as e:
        g.chunk_prefill_noalloc(layer, q[:90], q[:90], q[:90], ab[:90], ab[:90], list(range(0, 100, 10)), [0] * 9,
                                [("zero", None, S)] * 9, o[:90])
    assert g.STATUS_NAMES[e.value.status] == "GDN_ERR_CAPACITY"
    torch.cuda.synchronize()
    assert (o == 3.0).all() and (S == 7.0).all()
