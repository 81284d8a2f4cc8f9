"""The C ABI without a GPU: the library loads, exports every symbol include/gdn.h
declares, its host helpers agree with the pages' numbers, and every validation error
is returned before anything is enqueued (no compute call is made here: each call
below fails validation first, so no HIP work is issued)."""
import ctypes
import json
import os
import re

import pytest
import torch

import gated_deltanet_recurrent_chunk_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
lib = g.lib_handle()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_every_declared_symbol_is_exported():
    header = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", header))
    assert declared, "no declarations found"
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(g.EXPORTED)
    assert lib.gdn_abi_version() == 3


def test_helpers_match_page_figures():
    pa = _golden("prefix_accounting.json")
    for c in pa["cached_prefix"]:
        assert g.cached_prefix_tokens(c["shared"], c["block"]) == c["cached"], c["source"]
    for c in pa["floor_chunk"]:
        assert g.floor_chunk(c["budget"], c["block"]) == c["chunk"], c["source"]
    for c in pa["checkpoint_positions"]:
        assert g.count_boundaries(c["start"], c["tokens"], c["block"]) == len(c["positions"])
    pf = _golden("page_figures.json")
    c = pf["checkpoint_bytes_27b"]
    L = c["layer"]
    layer = g.Layer(L["n_qk_heads"], L["n_v_heads"], L["head_dim"], torch.bfloat16)
    assert layer.checkpoint_bytes == c["value"] == layer.state_bytes + layer.conv_tail_bytes
    assert round(layer.checkpoint_bytes / 2 ** 20, 2) == pf["checkpoint_mib_27b"]["value"]
    assert round(100 * layer.state_bytes / layer.checkpoint_bytes) == pf["recurrent_share_percent_27b"]["value"]
    assert round(pf["per_sequence_mb_27b"]["gdn_layers"] * layer.checkpoint_bytes / 1e6, 1) == \
        pf["per_sequence_mb_27b"]["value"]
    for key in ("block_size_784", "block_size_896"):
        b = pf[key]
        assert g.block_size_for_state(b["state_bytes"], b["attn_bytes_per_token"], b["alignment"]) == b["value"]
    slots = pf["compact_slots_gib"]
    assert round(slots["slots"] * slots["layers_per_slot"] * layer.checkpoint_bytes / 2 ** 30, 1) == slots["value"]
    l4 = g.Layer(16, 32, 128, torch.bfloat16)
    assert l4.state_bytes == pf["state_mib_4b"]["value"] * 2 ** 20
    sc = pf["spec_copies_mib_4b"]
    assert (sc["drafts"] + 1) * sc["layers"] * sc["page_mib"] == sc["value"]
    rp = pf["replay_mib_per_request_4b"]
    slot_bytes = 2 * 16 * 128 * 2 + 32 * 128 * 2 + 2 * 32 * 4
    per_req = rp["layers"] * (rp["page_mib"] * 2 ** 20 + rp["buffer_slots"] * slot_bytes)
    assert round(per_req / 2 ** 20) == rp["value"]


def test_workloads_fit_checkpoint_pages():
    """Pages of block x 4096 B (one attention page per token) hold a checkpoint."""
    layer = g.Layer(48, 48, 128, torch.bfloat16)
    assert 896 * 4096 >= layer.checkpoint_bytes
    assert layer.state_bytes == 3 * 2 ** 20


# ------------------------------------------------------------------ fail closed

def _err(fn, *args, **kw):
    with pytest.raises(g.GdnError) as e:
        fn(*args, **kw)
    return g.STATUS_NAMES[e.value.status]


def _aligned_pool(n_pages, page_bytes, block):
    """A host page pool whose base is 256-byte aligned, as the C ABI requires."""
    raw = torch.zeros(n_pages * page_bytes + 256, dtype=torch.uint8)
    off = (-raw.data_ptr()) % 256
    return g.CheckpointPool(raw[off:off + n_pages * page_bytes].view(n_pages, page_bytes), block)


def _ops(layer, T=100):
    """Host tensors shaped for `layer` (validation fails before any device use)."""
    H, Hv, D = layer.n_qk_heads, layer.n_v_heads, layer.head_dim
    q = torch.zeros(T, H, D, dtype=layer.io_dtype)
    v = torch.zeros(T, Hv, D, dtype=layer.io_dtype)
    a = torch.ones(T, Hv)
    o = torch.zeros(T, Hv, D)
    S = torch.zeros(Hv, D, D)
    return q, v, a, o, S


def _prefill(layer, cu, sp, refs, T=100, **kw):
    q, v, a, o, S = _ops(layer, T)
    refs = [(k_, s_, S if d_ is None else d_) for (k_, s_, d_) in refs]
    return g.chunk_prefill(layer, q, q, v, a, a, cu, sp, refs, o, stream=0, **kw)


def test_prefill_validation_errors():
    ok_layer = g.Layer(2, 2, 32)
    ck = _aligned_pool(4, ok_layer.checkpoint_bytes, 16)
    zero = [("zero", None, None)]
    # head counts that do not divide
    assert _err(_prefill, g.Layer(2, 3, 32), [0, 100], [0], zero) == "GDN_ERR_BAD_SHAPE"
    # unsupported head dim
    assert _err(_prefill, g.Layer(2, 2, 48), [0, 100], [0], zero) == "GDN_ERR_BAD_SHAPE"
    # a zero source at a non-zero position
    assert _err(_prefill, ok_layer, [0, 100], [5], zero) == "GDN_ERR_OFF_BOUNDARY"
    # a checkpoint resume off the block grid
    assert _err(_prefill, ok_layer, [0, 50], [40], [("checkpoint", ck.page_ptr(0), None)], ckpt=ck,
                page_ids=[0, 1, 2]) == "GDN_ERR_OFF_BOUNDARY"
    # decreasing cu_seqlens
    assert _err(_prefill, ok_layer, [0, 60, 50], [0, 0], zero * 2) == "GDN_ERR_BAD_VARLEN"
    # page too small for a checkpoint
    small = _aligned_pool(4, 256, 16)
    assert _err(_prefill, ok_layer, [0, 40], [0], zero, ckpt=small, page_ids=[0, 1]) == "GDN_ERR_PAGE_TOO_SMALL"
    # a page named twice, or out of range
    assert _err(_prefill, ok_layer, [0, 40], [0], zero, ckpt=ck, page_ids=[1, 1]) == "GDN_ERR_BAD_PAGE"
    assert _err(_prefill, ok_layer, [0, 40], [0], zero, ckpt=ck, page_ids=[0, 4]) == "GDN_ERR_BAD_PAGE"
    # workspace too small
    ws = torch.zeros(256, dtype=torch.uint8)
    assert _err(_prefill, ok_layer, [0, 100], [0], zero, workspace=ws) == "GDN_ERR_WORKSPACE"
    # fp32 rows at head_dim 128 pass the shape checks like bf16 rows: both stop only at the
    # (too small) workspace, which is checked after every shape
    for dt in (torch.float32, torch.bfloat16):
        assert _err(_prefill, g.Layer(2, 2, 128, dt), [0, 100], [0], zero, workspace=ws) == "GDN_ERR_WORKSPACE"


def test_binding_rejects_undersized_operands():
    layer = g.Layer(2, 2, 32)
    q, v, a, o, S = _ops(layer, T=10)
    with pytest.raises(ValueError):
        g.chunk_prefill(layer, q, q, v, a, a, [0, 100], [0], [("zero", None, S)], o, stream=0)


def test_flush_and_decode_validation_errors():
    layer = g.Layer(2, 2, 32)
    pool = torch.zeros(2, 2, 32, 32)
    buf = torch.zeros(2, 65, 2, 32, dtype=torch.bfloat16)
    ab = torch.zeros(2, 65, 2)
    ids = torch.zeros(2, dtype=torch.int32)
    assert _err(g.replay_flush, layer, pool, ids, buf, buf, ab, ab, ids, stream=0) == "GDN_ERR_CAPACITY"
    # a state pool off the 16-byte grid
    pool32 = torch.zeros(2 * 2 * 128 * 128 + 1)[1:].view(2, 2, 128, 128)
    assert _err(g.replay_flush, g.Layer(2, 2, 128, torch.float32), pool32, ids,
                torch.zeros(2, 32, 2, 128), torch.zeros(2, 32, 2, 128), torch.zeros(2, 32, 2),
                torch.zeros(2, 32, 2), ids, stream=0) == "GDN_ERR_BAD_SHAPE"
    q = torch.zeros(2, 2, 32, dtype=torch.bfloat16)
    assert _err(g.decode_step, g.Layer(2, 2, 32, conv_width=3), q, q, q, torch.zeros(2, 2), torch.zeros(2, 2),
                pool, ids, torch.zeros(2, 2, 32), stream=0) == "GDN_ERR_BAD_SHAPE"


def test_replay_gates_norm_and_mixed_validation_errors():
    layer = g.Layer(2, 2, 32)
    pool = torch.zeros(2, 2, 32, 32)
    ids = torch.zeros(2, dtype=torch.int32)
    buf = torch.zeros(2, 65, 2, 32, dtype=torch.bfloat16)
    ab = torch.zeros(2, 65, 2)
    qn = torch.zeros(2, 4, 2, 32, dtype=torch.bfloat16)
    o = torch.zeros(2, 4, 2, 32)
    # a log longer than 64 rows
    assert _err(g.replay_forward, layer, pool, ids, buf, buf, ab, ab, ids, ids, qn, o, stream=0) == "GDN_ERR_CAPACITY"
    # fp32 inputs with d = 128: logs of more than 32 rows do not fit the verify kernel's LDS
    l32 = g.Layer(2, 2, 128, torch.float32)
    assert _err(g.replay_forward, l32, torch.zeros(2, 2, 128, 128), ids, torch.zeros(2, 33, 2, 128),
                torch.zeros(2, 33, 2, 128), torch.zeros(2, 33, 2), torch.zeros(2, 33, 2), ids, ids,
                torch.zeros(2, 4, 2, 128), torch.zeros(2, 4, 2, 128), stream=0) == "GDN_ERR_CAPACITY"
    # an unknown flag in the activation field
    bad = g.Layer(2, 2, 32, conv_act=0x200)
    ba = torch.zeros(5, 4, dtype=torch.bfloat16)
    A_log = torch.zeros(2)
    dt = torch.zeros(2, dtype=torch.bfloat16)
    gates_out = torch.zeros(5, 2)
    assert _err(g.gates, bad, ba, A_log, dt, gates_out, gates_out, stream=0) == "GDN_ERR_BAD_DTYPE"
    # gate rows not a multiple of 8 elements apart, and a negative epsilon
    zr = torch.zeros(5, 2 * 32 + 4, dtype=torch.bfloat16)
    w = torch.zeros(32, dtype=torch.bfloat16)
    out = torch.zeros(5, 2, 32, dtype=torch.bfloat16)
    assert _err(g.gated_norm, layer, torch.zeros(5, 2, 32), zr, w, out, stream=0) == "GDN_ERR_BAD_SHAPE"
    zz = torch.zeros(5, 2, 32, dtype=torch.bfloat16)
    assert _err(g.gated_norm, layer, torch.zeros(5, 2, 32), zz, w, out, eps=-1.0, stream=0) == "GDN_ERR_BAD_SHAPE"
    # token rows closer than one row of heads
    q = torch.zeros(4, 2, 32, dtype=torch.bfloat16)
    assert _err(g.decode_mixed, layer, q, q, q, torch.zeros(4, 2), torch.zeros(4, 2), pool, ids, ids,
                torch.zeros(4, 2, 32), stream=0, qk_stride=16) == "GDN_ERR_BAD_SHAPE"


def test_conv_validation_errors():
    layer = g.Layer(1, 1, 16, torch.bfloat16)
    C = layer.conv_channels
    x = torch.zeros(20, C, dtype=torch.bfloat16)
    w = torch.zeros(C, 4, dtype=torch.bfloat16)
    t = torch.zeros(3, C, dtype=torch.bfloat16)
    ck = _aligned_pool(4, layer.checkpoint_bytes, 8)
    assert _err(g.conv_update, layer, x, w, [("checkpoint", ck.page_ptr(0), t)], [0, 20], [4], x, ckpt=ck,
                page_ids=[0, 1, 2], stream=0) == "GDN_ERR_OFF_BOUNDARY"
    assert _err(g.conv_update, layer, x, w, [("slot", None, t)], [0, 20], [4], x,
                stream=0) == "GDN_ERR_NULL_ARG"


def _aligned_bytes(n):
    raw = torch.zeros(n + 256, dtype=torch.uint8)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + n]


def test_conv_rejects_a_row_stride_below_the_channels_or_off_16_bytes():
    layer = g.Layer(1, 1, 16, torch.bfloat16)
    C = layer.conv_channels
    w = torch.zeros(C, 4, dtype=torch.bfloat16)
    t = torch.zeros(3, C, dtype=torch.bfloat16)
    y = torch.zeros(20, C, dtype=torch.bfloat16)
    wide = torch.zeros(20, C + 4, dtype=torch.bfloat16)  # 8-byte row padding: loads would straddle
    assert _err(g.conv_update, layer, wide[:, :C], w, [("zero", None, t)], [0, 20], [0], y,
                stream=0) == "GDN_ERR_BAD_SHAPE"
    pool = torch.zeros(2, 3, C, dtype=torch.bfloat16)
    slots = torch.zeros(2, dtype=torch.int32)
    assert _err(g.conv_decode, layer, wide[:, :C], w, pool, slots, y, stream=0) == "GDN_ERR_BAD_SHAPE"


def test_core_prefill_validation_errors():
    """The packed core checks all four stages before anything is enqueued."""
    Hqk, Hv, D = 1, 2, 16
    layer = g.Layer(Hqk, Hv, D, torch.bfloat16, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    C = layer.conv_channels
    T = 40
    qkvz = torch.zeros(T, C + Hv * D, dtype=torch.bfloat16)
    ba = torch.zeros(T, 2 * Hv, dtype=torch.bfloat16)
    w = torch.zeros(C, 4, dtype=torch.bfloat16)
    A_log = torch.zeros(Hv)
    dtb = torch.zeros(Hv, dtype=torch.bfloat16)
    wn = torch.ones(D, dtype=torch.bfloat16)
    S = torch.zeros(Hv, D, D)
    tl = torch.zeros(3, C, dtype=torch.bfloat16)
    out = torch.zeros(T, Hv, D, dtype=torch.bfloat16)
    ck = _aligned_pool(4, layer.checkpoint_bytes, 16)
    ws = _aligned_bytes(g.core_prefill_workspace_bytes(layer, [0, T], [0], 16))
    args = (layer, qkvz, ba, w, A_log, dtb, wn)
    zero = ([("zero", None, tl)], [("zero", None, S)])
    # a checkpoint resume off the block grid (the conv stage's tail source is checked first)
    src = ck.page_ptr(3)
    assert _err(g.core_prefill, *args, [0, T], [8], [("checkpoint", src, tl)], [("checkpoint", src, S)], out,
                ckpt=ck, page_ids=[0, 1, 2], workspace=ws, stream=0) == "GDN_ERR_OFF_BOUNDARY"
    # a zero state source at a non-zero position (the prefill stage's check)
    assert _err(g.core_prefill, *args, [0, T], [16], [("slot", tl, tl)], [("zero", None, S)], out,
                ckpt=ck, page_ids=[0, 1, 2], workspace=ws, stream=0) == "GDN_ERR_OFF_BOUNDARY"
    # workspace too small
    assert _err(g.core_prefill, *args, [0, T], [0], *zero, out, ckpt=ck, page_ids=[0, 1],
                workspace=ws[:-256], stream=0) == "GDN_ERR_WORKSPACE"
    # a negative norm epsilon (the gated-norm stage's check)
    assert _err(g.core_prefill, *args, [0, T], [0], *zero, out, ckpt=ck, page_ids=[0, 1], eps=-1.0,
                workspace=ws, stream=0) == "GDN_ERR_BAD_SHAPE"
    # ten sequences need staging: an empty buffer is refused
    cu = list(range(0, 41, 4))
    assert _err(g.core_prefill, *args, cu, [0] * 10, [("zero", None, tl)] * 10, [("zero", None, S)] * 10, out,
                ckpt=ck, page_ids=[], workspace=_aligned_bytes(g.core_prefill_workspace_bytes(layer, cu, [0] * 10, 16)),
                staging=torch.empty(0, dtype=torch.uint8), stream=0) == "GDN_ERR_STAGING"
    # packed rows too narrow for q | k | v | z (the binding refuses them)
    with pytest.raises(ValueError):
        g.core_prefill(layer, qkvz[:, :C], ba, w, A_log, dtb, wn, [0, T], [0], *zero, out, ckpt=ck, page_ids=[0, 1],
                       workspace=ws, stream=0)
    assert not out.any() and not S.any() and not tl.any() and not ck.pool.any()


def test_core_prefill_workspace_holds_every_stage_output():
    layer = g.Layer(2, 4, 128, torch.bfloat16)
    cu, sp, block = [0, 300, 301], [0, 896], 896
    need = g.core_prefill_workspace_bytes(layer, cu, sp, block)
    T, C, Hv, D = 301, layer.conv_channels, 4, 128
    stage_outputs = T * C * 2 + 2 * T * Hv * 4 + T * Hv * D * 4
    assert need >= g.prefill_workspace_bytes(layer, cu, sp, block) + stage_outputs
    assert need <= g.prefill_workspace_bytes(layer, cu, sp, block) + stage_outputs + 5 * 256
    assert g.core_prefill_staging_bytes(layer, cu, sp, block) == 0


# ------------------------------------------------------------------ no library state

def _nm(*args):
    import subprocess
    return subprocess.run(["nm", *args, g.LIB_PATH], capture_output=True, text=True, check=True).stdout


def test_library_keeps_no_state_and_never_waits():
    """libgdn holds no memory and no state between calls, so calls on different streams
    cannot wait for each other: it imports no HIP call that allocates, frees, creates or
    waits on events, or synchronizes, and its only writable data are the compiler's and
    the HIP runtime's registration records (no variable of its own)."""
    imports = {line.split()[-1].split("@")[0] for line in _nm("-D", "--undefined-only").splitlines() if line.strip()}
    hip = {s for s in imports if s.lower().startswith("hip") or s.startswith("__hip")}
    forbidden = {s for s in hip if any(w in s for w in ("Synchronize", "Malloc", "Free", "Event", "Wait",
                                                         "HostRegister", "StreamCreate", "Query"))}
    assert not forbidden, sorted(forbidden)
    allowed = {"hipLaunchKernel", "hipGetLastError", "hipMemcpyAsync", "hipGetDevice", "hipGetSymbolAddress",
               "__hipPushCallConfiguration", "__hipPopCallConfiguration", "__hipRegisterFatBinary",
               "__hipRegisterFunction", "__hipUnregisterFatBinary", "__hipRegisterVar"}
    assert hip <= allowed, sorted(hip - allowed)
    runtime = re.compile(r"^(DW\.ref\.|_DYNAMIC$|_GLOBAL_OFFSET_TABLE_$|__do_(init|fini)\.|__dso_handle$|__(init|fini)$|"
                         r"__hip_(cuid|fatbin_wrapper|gpubin_handle)|__TMC_END__$|completed\.|__bss_start$|_edata$|_end$)")
    own = []
    for line in _nm().splitlines():
        parts = line.split()
        if len(parts) < 3 or parts[1] not in "bBdDsSgGvV" or runtime.match(parts[2]):
            continue
        # the host-side handle HIP emits for each __global__ function (its address names the
        # kernel at launch; nothing writes it)
        if parts[1] == "V" and parts[2].startswith("_ZN3gdn") and "_kernel" in parts[2]:
            continue
        own.append(parts[2])
    # the no-alloc entry point's scratch array and its per-device address table are the one
    # documented exception
    own = [s for s in own if "scratch" not in s]
    assert not own, own
