"""Benchmark of the libgdn hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-long]

Step = one pass of the prefill hot path over one 27B-shaped layer, as two library
calls: the causal conv update over the packed q|k|v channels (18,432 bf16 channels,
8,192 tokens) and the chunked prefill (pre-pass and scan in one call) of the gated delta
rule (48 heads, 128 x 128 fp32 state per head, bf16 q/k/v, fp32 o, 64-token chunks)
writing a checkpoint page at each of the nine 896-token block boundaries.  `value` is
prefill tokens per second per layer over the K timed steps (inputs resident in HBM,
synthetic, seeded).

Reported beside it, on the stream the kernels run on, as the median and the 10th / 90th
percentiles over batches of back-to-back launches timed with HIP events:
  * the stepped varlen prefill: 4 sequences of 2,688 / 5,000 / 6,272 / 12,000 tokens in
    calls of at most 1,792 tokens per sequence (the 2,048-token budget floored to the
    896-token block), two of them resuming at 1,792 from the checkpoint the other wrote;
  * the long prefill: 229,376 tokens (256 checkpoints);
  * per-kernel launch times of the 8,192-token step (conv, pre-pass, scan), and the
    roofline of the dominant kernel (the scan) with its measured matrix-core busy share;
  * the replay flush at the 4B-shaped layer (16 requests, 32 value heads x 128 x 128 fp32
    state, a 32-slot log): accepted rows uniform in 1..16, and a sweep over n = 1..33
    rows (33 in a 64-slot log), rotating over enough state pools that every launch
    streams from HBM; the replay outputs at the same layer;
  * the decode step for 256 requests at the 27B shape, the conv's decode regime for the
    same requests, and a mixed step (those decode tokens and the 8,192-token prefill in
    one packed batch);
  * the packed-core steps at the 27B layer (conv with the q/k norm, gates, gated norm);
  * the device, its clocks and the ROCm version;
  * the fp64 CPU oracle on the allotted host cores and on one core.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Published MI355X peaks.
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6

# Prefill workload: one 27B-shaped GDN layer.
T, H, D, BLOCK, CHUNK = 8192, 48, 128, 896, 64
PAGE_BYTES = BLOCK * 4096  # one attention page of 4,096 B per token
LONG_T = 229376
VARLEN = (2688, 5000, 6272, 12000)


def scan_algorithmic_flops(tokens, heads, d=D, c=CHUNK):
    """Products of the chunk scan, each counted once (not per bf16 pass), per token and
    value head: K S^T, Q S^T and the state update K^T Dt (2 d^2 each), and the two
    64 x 64 triangular products T'' R' and PT'' R' (C d each, half of a full 2 C d)."""
    return tokens * heads * (6 * d * d + 2 * c * d)


def scan_pass_flops(tokens, heads, d=D, c=CHUNK):
    """The same products weighted by the bf16 matrix-core passes they need with bf16
    inputs: an fp32 operand is two bf16 terms, so a bf16 x fp32 product (K S^T, Q S^T,
    the update) is 2 passes and an fp32 x fp32 product (T'' R', PT'' R') keeps 3 of the 4
    term pairs.  Time at the bf16 peak for this many flops is the kernel's MFMA roof."""
    return tokens * heads * (2 * 6 * d * d + 3 * 2 * c * d)


def scan_issued_flops(tokens, heads, d=D, c=CHUNK):
    """Matrix-core flops the scan kernel actually issues (16x16x32 bf16 MFMAs): per 16-row
    slab and chunk, 32 for K S^T, 32 for Q S^T, 2 x 18 for T'' R' (both key halves form
    it), 18 for PT'' R', 32 for the update."""
    chunks = tokens // c
    return chunks * heads * (d // 16) * (32 + 32 + 36 + 18 + 32) * 16 * 16 * 32 * 2


def kernel_sources_sha():
    """Hash of the sources the scan kernel is built from (a committed profile of the scan
    applies only while it matches)."""
    csrc = os.path.join(ROOT, "gated_deltanet_recurrent_chunk_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read()
                   for f in ("prefill_kernels.hip", "chunk_common.h", "device_common.h", "call_table.h", "plan.h"))
    return hashlib.sha256(src).hexdigest()


def profiled_scan_counters():
    """Counters of the scan launch from the committed profile (calibrated HBM traffic and
    matrix-core busy share), or None once the kernel sources differ from the ones the
    counters were taken on."""
    path = os.path.join(ROOT, "profiles", "prefill_27b_T8192_H48_counters.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    sha = re.search(r"source_sha256: ([0-9a-f]{64})", text)
    if not sha or sha.group(1) != kernel_sources_sha():
        return None
    out = {}
    for key in ("traffic_bytes_per_launch", "mfma_busy_fraction", "valu_busy_fraction", "lds_busy_fraction"):
        m = re.search(key + r": ([0-9.]+)", text)
        if m:
            out[key] = float(m.group(1))
    return out


def flush_bytes(n_acc, heads=32, qk_heads=16, d=D):
    """HBM bytes one flush must move: each touched state read and written once, plus
    the accepted log rows (bf16 k, v; fp32 a, b)."""
    state = heads * d * d * 4
    row = qk_heads * d * 2 + heads * d * 2 + 2 * heads * 4
    return sum(2 * state + n * row for n in n_acc if n > 0)


def replay_bytes(n_logged, n_new, heads=32, qk_heads=16, d=D):
    """HBM bytes one replay launch must move: each request's state read once, its logged
    and new log rows (bf16 k, v; fp32 a, b) and the new rows' queries read once, the new
    rows' fp32 outputs written once."""
    state = heads * d * d * 4
    row = qk_heads * d * 2 + heads * d * 2 + 2 * heads * 4
    return sum(state + (m + n_new) * row + n_new * (qk_heads * d * 2 + heads * d * 4) for m in n_logged)


def note(msg):
    """Progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dpm_levels(name):
    """Clock levels (MHz) of the first GPU's DPM table in sysfs, or None."""
    import glob
    for path in sorted(glob.glob(f"/sys/class/drm/card*/device/{name}")):
        try:
            lines = open(path).read().split("\n")
        except OSError:
            continue
        levels = []
        for line in lines:
            m = re.match(r"\s*(\d+):\s*(\d+)\s*[Mm]hz", line)
            if m:
                levels.append(int(m.group(2)))
        if levels:
            return {"levels_mhz": levels}
    return None


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    info["sclk"] = dpm_levels("pp_dpm_sclk")
    info["mclk"] = dpm_levels("pp_dpm_mclk")
    return info


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-long", action="store_true", help="skip the 229,376-token prefill")
    ap.add_argument("--step-only", action="store_true",
                    help="only the prefill step and its per-kernel times (a short run for profilers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "gpus_requested": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_recurrent_chunk_amd as g
    import gdn_inputs as gi

    torch.cuda.set_device(0)
    dev = "cuda"

    if args.copy_calibration:
        src = torch.ones(2 ** 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "launches": 5}), flush=True)
        return

    def spin_cycles_per_us():
        """Rate of torch's device spin kernel (cycles of its clock per microsecond)."""
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        e1.synchronize()
        return 2_000_000 / (e0.elapsed_time(e1) * 1e3)

    spin_rate = spin_cycles_per_us()

    def batches_us(fn, batches=30, per_batch=10, warm=3):
        """Per-launch device time in us: `batches` batches of `per_batch` back-to-back
        launches, each batch between two events on the current stream; fn(i) gets the
        launch index.  A spin kernel ahead of each batch keeps the device busy while the
        host queues the batch (for 1.5 times the host's fastest warm-up call), so the batch
        runs back to back as inside a larger step, never waiting for the host."""
        host_us = 0.0
        for i in range(warm):
            t_host = time.perf_counter()
            fn(i)
            dt = (time.perf_counter() - t_host) * 1e6
            host_us = dt if i == 0 else min(host_us, dt)
        torch.cuda.synchronize()
        lead = int(spin_rate * (1.5 * host_us * per_batch + 100.0))
        out = []
        i = 0
        for _ in range(batches):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(lead)
            e0.record()
            for _ in range(per_batch):
                fn(i)
                i += 1
            e1.record()
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / per_batch)
        return out

    def pct(xs):
        xs = sorted(xs)

        def q(f):
            return xs[min(len(xs) - 1, max(0, int(round(f * (len(xs) - 1)))))]

        return {"median": round(statistics.median(xs), 2), "p10": round(q(0.1), 2), "p90": round(q(0.9), 2),
                "n": len(xs)}

    # ------------------------------------------------------------ prefill step inputs
    layer = g.Layer(H, H, D, torch.bfloat16, scale=1.0)
    C = layer.conv_channels
    q, k, v, a, b = (t.to(dev) for t in gi.qkvab(T, H, H, D, torch.bfloat16, seed=1001))
    x, w = (t.to(dev) for t in gi.conv_inputs(T, C, 4, torch.bfloat16, seed=1001))
    y = torch.empty_like(x)
    tail = torch.empty(3, C, dtype=torch.bfloat16, device=dev)
    o = torch.empty(T, H, D, dtype=torch.float32, device=dev)
    S = torch.empty(H, D, D, dtype=torch.float32, device=dev)
    n_ck = g.count_boundaries(0, T, BLOCK)
    pool = g.CheckpointPool(torch.zeros(n_ck + 1, PAGE_BYTES, dtype=torch.uint8, device=dev), BLOCK)
    page_ids = list(range(n_ck))
    cu, sp = [0, T], [0]
    ws = torch.empty(g.prefill_workspace_bytes(layer, cu, sp, BLOCK), dtype=torch.uint8, device=dev)
    cws = torch.empty(max(256, g.conv_workspace_bytes(layer, cu, sp, BLOCK)), dtype=torch.uint8, device=dev)

    def step():
        g.conv_update(layer, x, w, [("zero", None, tail)], cu, sp, y, ckpt=pool, page_ids=page_ids, workspace=cws)
        g.chunk_prefill(layer, q, k, v, a, b, cu, sp, [("zero", None, S)], o, ckpt=pool, page_ids=page_ids,
                        workspace=ws)

    note(f"prefill step: {args.warmup} warmup + {args.steps} timed")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = T * args.steps / elapsed
    dev_info = device_info(torch)

    # per-kernel launch times of the step (each stage on its own)
    note("per-kernel times")
    conv_us = batches_us(lambda i: g.conv_update(layer, x, w, [("zero", None, tail)], cu, sp, y, ckpt=pool,
                                                 page_ids=page_ids, workspace=cws))
    fact_us = batches_us(lambda i: g.prefill_factorize(layer, q, k, a, b, cu, sp, BLOCK, ws))
    scan_us = batches_us(lambda i: g.prefill_scan(layer, q, k, v, cu, sp, [("zero", None, S)], o, ws, ckpt=pool,
                                                  page_ids=page_ids))
    scan_med = statistics.median(scan_us)
    alg = scan_algorithmic_flops(T, H)
    passes = scan_pass_flops(T, H)
    achieved_tflops = alg / (scan_med * 1e-6) / 1e12
    eff_peak = PEAK_BF16_TFLOPS * alg / passes
    prof = profiled_scan_counters()
    if args.step_only:
        print(json.dumps({"value": round(value, 1), "unit": "tokens/s/layer", "ms_per_step": round(ms_per_step, 4),
                          "kernel_us": {"conv": pct(conv_us), "factorize": pct(fact_us), "scan": pct(scan_us)}}),
              flush=True)
        return

    # packed-core steps at the same layer
    note("packed-core steps")
    nlayer = g.Layer(H, H, D, torch.bfloat16, scale=1.0, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    conv_norm_us = batches_us(lambda i: g.conv_update(nlayer, x, w, [("zero", None, tail)], cu, sp, y, ckpt=pool,
                                                      page_ids=page_ids, workspace=cws), batches=10)
    ba, A_log, dt_bias, _, zc, wn = gi.core_inputs(T, H, D, torch.bfloat16, seed=1006)
    ba, A_log, dt_bias, zc, wn = (t_.to(dev) for t_ in (ba, A_log, dt_bias, zc, wn))
    ga, gb = torch.empty(T, H, device=dev), torch.empty(T, H, device=dev)
    gates_us = batches_us(lambda i: g.gates(layer, ba, A_log, dt_bias, ga, gb), batches=10)
    onorm = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    norm_us = batches_us(lambda i: g.gated_norm(layer, o, zc, wn, onorm), batches=10)
    norm_bytes = T * H * D * (4 + 2 + 2)
    gate_bytes = T * 2 * H * 2 + 2 * T * H * 4

    # ------------------------------------------------------------ replay flush (4B layer)
    note("flush")
    fl_layer = g.Layer(16, 32, D, torch.bfloat16)
    n_req = 16
    state_mib = n_req * 32 * D * D * 4 / 2 ** 20
    n_pools = int(np.ceil(2 * 256 / state_mib)) + 1  # > 2 x 256 MB last-level cache in rotation
    fpools = [gi.states(n_req, 32, D, seed=1003 + i).to(dev) for i in range(n_pools)]
    slots = torch.arange(n_req, dtype=torch.int32, device=dev)
    acc_u = gi.accepted_counts(n_req, 1003)

    def log(rows, seed):
        _, bk_, bv_, ba_, bb_ = gi.qkvab(n_req * rows, 16, 32, D, torch.bfloat16, seed=seed)
        return (bk_.view(n_req, rows, 16, D).to(dev), bv_.view(n_req, rows, 32, D).to(dev),
                ba_.view(n_req, rows, 32).to(dev), bb_.view(n_req, rows, 32).to(dev))

    log32, log64 = log(32, 1003), log(64, 1007)

    def flush_us(acc, lg, batches=20):
        acc_d = acc.to(torch.int32).to(dev)
        return batches_us(lambda i: g.replay_flush(fl_layer, fpools[i % n_pools], slots, *lg, acc_d), batches=batches,
                          per_batch=20)

    flush_u = flush_us(acc_u, log32, batches=30)
    fb_u = flush_bytes(acc_u.tolist())
    sweep = {}
    for n in list(range(1, 33)) + [33]:
        sweep[str(n)] = round(statistics.median(flush_us(torch.full((n_req,), n), log32 if n <= 32 else log64,
                                                         batches=5)), 2)
    # the 64-slot log (the two-block form) at every length class: short, one block, two
    sweep64 = {str(n): round(statistics.median(flush_us(torch.full((n_req,), n), log64, batches=5)), 2)
               for n in (8, 16, 32, 48, 64)}
    sweep64["u1_16"] = round(statistics.median(flush_us(acc_u, log64, batches=5)), 2)

    # ------------------------------------------------------------ replay outputs (4B layer)
    note("replay outputs")
    n_new = 16
    rq_new = gi.qkvab(n_req * n_new, 16, 32, D, torch.bfloat16, seed=1004)[0].view(n_req, n_new, 16, D).to(dev)
    r_out = torch.empty(n_req, n_new, 32, D, dtype=torch.float32, device=dev)
    logged_d = acc_u.to(torch.int32).to(dev)
    new_d = torch.full((n_req,), n_new, dtype=torch.int32, device=dev)
    replay = batches_us(lambda i: g.replay_forward(fl_layer, fpools[i % n_pools], slots, *log32, logged_d, new_d,
                                                   rq_new, r_out))
    rb = replay_bytes(acc_u.tolist(), n_new)
    # a 64-slot log: 25..40 logged rows, 16 new (blocks of 41..56 rows)
    logged64 = (acc_u + 24).to(torch.int32).to(dev)
    replay64 = batches_us(lambda i: g.replay_forward(fl_layer, fpools[i % n_pools], slots, *log64, logged64, new_d,
                                                     rq_new, r_out), batches=10)
    rb64 = replay_bytes((acc_u + 24).tolist(), n_new)

    # ------------------------------------------------------------ decode (27B layer, 256 requests)
    note("decode")
    n_dec = 256
    dpool = gi.states(n_dec, H, D, seed=1005).to(dev)
    dq, dk, dv, da, db = (t.to(dev) for t in gi.qkvab(n_dec, H, H, D, torch.bfloat16, seed=1005))
    dout = torch.empty(n_dec, H, D, dtype=torch.float32, device=dev)
    dslots = torch.arange(n_dec, dtype=torch.int32, device=dev)
    decode = batches_us(lambda i: g.decode_step(layer, dq, dk, dv, da, db, dpool, dslots, dout), batches=20)
    dec_bytes = n_dec * (2 * H * D * D * 4 + 3 * H * D * 2 + 2 * H * 4 + H * D * 4)
    # the conv's decode regime for the same requests: one row each, tails in a slot pool
    dx = gi.conv_inputs(n_dec, C, 4, torch.bfloat16, seed=1008)[0].to(dev)
    dy = torch.empty_like(dx)
    dtails = torch.zeros(n_dec, 3, C, dtype=torch.bfloat16, device=dev)
    conv_dec = batches_us(lambda i: g.conv_decode(layer, dx, w, dtails, dslots, dy), batches=20)
    conv_dec_bytes = n_dec * C * 2 * 8  # three tail rows and the new row read, written back with y

    # ------------------------------------------------------------ mixed batch (27B layer)
    note("mixed step")
    # one packed batch: 256 decode tokens (rows 0..255) and the 8,192-token prefill behind
    # them; the conv runs over the prefill sequence and, in its decode regime, over the
    # decode tokens (their tails in a slot pool), the prefill over its rows, the decode
    # tokens through decode_mixed
    mT = n_dec + T
    mx = torch.cat([dx, x])
    my = torch.empty_like(mx)
    mq, mk, mv = (torch.cat([d_, p_]) for d_, p_ in ((dq, q), (dk, k), (dv, v)))
    ma, mb = torch.cat([da, a]), torch.cat([db, b])
    mo = torch.empty(mT, H, D, dtype=torch.float32, device=dev)
    mrows = torch.arange(n_dec, dtype=torch.int32, device=dev)
    pre = slice(n_dec, mT)

    def mixed_step(i=0):
        g.conv_update(layer, mx[pre], w, [("zero", None, tail)], cu, sp, my[pre], ckpt=pool, page_ids=page_ids,
                      workspace=cws)
        g.conv_decode(layer, mx, w, dtails, dslots, my, rows=mrows)
        g.chunk_prefill(layer, mq[pre], mk[pre], mv[pre], ma[pre], mb[pre], cu, sp, [("zero", None, S)], mo[pre],
                        ckpt=pool, page_ids=page_ids, workspace=ws)
        g.decode_mixed(layer, mq, mk, mv, ma, mb, dpool, dslots, mrows, mo)

    mixed = [u / 1e3 for u in batches_us(mixed_step, batches=10, per_batch=2)]

    # ------------------------------------------------------------ stepped varlen prefill
    note("stepped varlen prefill")
    # two of the four sequences share a 3,000-token prefix, of which the cache rule keeps
    # 1,792 tokens (two blocks); each resumes there from the page the other wrote
    step_tokens = g.floor_chunk(2048, BLOCK)
    shared = 3000
    assert g.cached_prefix_tokens(shared, BLOCK) == step_tokens
    vcu = np.concatenate([[0], np.cumsum(VARLEN)]).tolist()
    vq, vk, vv, va, vb = gi.qkvab_device(vcu[-1], H, H, D, torch.bfloat16, seed=1002)
    vx, _ = gi.conv_inputs_device(vcu[-1], C, 4, torch.bfloat16, seed=1002)
    for t_ in (vq, vk, vv, va, vb, vx):
        t_[vcu[3]:vcu[3] + shared] = t_[vcu[1]:vcu[1] + shared]
    n_b = [g.count_boundaries(0, L, BLOCK) for L in VARLEN]
    vpool = g.CheckpointPool(torch.zeros(2 * sum(n_b) + 8, PAGE_BYTES, dtype=torch.uint8, device=dev), BLOCK)
    # the prefix checkpoints the resumed sequences start from: sequences 3 and 1, cold, up
    # to the shared block boundary (pages 0 and 1)
    Sx = torch.empty(H, D, D, device=dev)
    tx = torch.empty(3, C, dtype=torch.bfloat16, device=dev)
    yx = torch.empty(step_tokens, C, dtype=torch.bfloat16, device=dev)
    ox = torch.empty(step_tokens, H, D, device=dev)
    prefix_page = {3: 0, 1: 1}
    for i, pg in prefix_page.items():
        sl = slice(vcu[i], vcu[i] + step_tokens)
        ids = [-1, pg]
        g.conv_update(layer, vx[sl], w, [("zero", None, tx)], [0, step_tokens], [0], yx, ckpt=vpool, page_ids=ids)
        g.chunk_prefill(layer, vq[sl], vk[sl], vv[sl], va[sl], vb[sl], [0, step_tokens], [0], [("zero", None, Sx)],
                        ox, ckpt=vpool, page_ids=ids)
    torch.cuda.synchronize()
    # the calls: packed rows of every active sequence, at most 1,792 each; a sequence's
    # state and tail continue in place from one call to the next
    pos = [0, step_tokens, 0, step_tokens]
    src_page = {1: prefix_page[3], 3: prefix_page[1]}  # each resumes from the other's page
    Sv = torch.empty(len(VARLEN), H, D, D, device=dev)
    tv = torch.empty(len(VARLEN), 3, C, dtype=torch.bfloat16, device=dev)
    src = {i: ("checkpoint", vpool.page_ptr(src_page[i])) if i in src_page else ("zero", None)
           for i in range(len(VARLEN))}
    next_page = 2
    calls = []
    while any(pos[i] < VARLEN[i] for i in range(len(VARLEN))):
        spans = [(i, pos[i], min(step_tokens, VARLEN[i] - pos[i])) for i in range(len(VARLEN)) if pos[i] < VARLEN[i]]
        idx = torch.cat([torch.arange(vcu[i] + p0, vcu[i] + p0 + n) for i, p0, n in spans]).to(dev)
        ccu = np.concatenate([[0], np.cumsum([n for _, _, n in spans])]).tolist()
        starts = [p0 for _, p0, _ in spans]
        ids = []
        for i, p0, n in spans:
            nb = g.count_boundaries(p0, n, BLOCK)
            ids += list(range(next_page, next_page + nb))
            next_page += nb
        st_refs, tl_refs = [], []
        for i, _, _ in spans:
            kind, ptr = src[i]
            st_refs.append((kind, ptr, Sv[i]) if kind != "slot" else ("slot", Sv[i], Sv[i]))
            tl_refs.append((kind, ptr, tv[i]) if kind != "slot" else ("slot", tv[i], tv[i]))
        calls.append(dict(q=vq[idx].contiguous(), k=vk[idx].contiguous(), v=vv[idx].contiguous(),
                          a=va[idx].contiguous(), b=vb[idx].contiguous(), x=vx[idx].contiguous(), cu=ccu,
                          starts=starts, states=st_refs, tails=tl_refs, ids=ids,
                          y=torch.empty(ccu[-1], C, dtype=torch.bfloat16, device=dev),
                          o=torch.empty(ccu[-1], H, D, device=dev),
                          ws=torch.empty(g.prefill_workspace_bytes(layer, ccu, starts, BLOCK), dtype=torch.uint8,
                                         device=dev),
                          cws=torch.empty(max(256, g.conv_workspace_bytes(layer, ccu, starts, BLOCK)),
                                          dtype=torch.uint8, device=dev)))
        for i, p0, n in spans:
            pos[i] = p0 + n
            src[i] = ("slot", None)
    assert next_page <= vpool.n_pages
    n_calls = len(calls)
    varlen_tokens = sum(VARLEN[i] - (step_tokens if i in src_page else 0) for i in range(len(VARLEN)))

    def varlen_run(i=0):
        for c_ in calls:
            g.conv_update(layer, c_["x"], w, c_["tails"], c_["cu"], c_["starts"], c_["y"], ckpt=vpool,
                          page_ids=c_["ids"], workspace=c_["cws"])
            g.chunk_prefill(layer, c_["q"], c_["k"], c_["v"], c_["a"], c_["b"], c_["cu"], c_["starts"],
                            c_["states"], c_["o"], ckpt=vpool, page_ids=c_["ids"], workspace=c_["ws"])

    varlen_ms = [u / 1e3 for u in batches_us(varlen_run, batches=10, per_batch=1, warm=1)]
    del vq, vk, vv, va, vb, vx, calls, vpool
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ long prefill (229,376 tokens)
    note("long prefill")
    long_res = None
    if not args.no_long:
        lq, lk, lv, la, lb = gi.qkvab_device(LONG_T, H, H, D, torch.bfloat16, seed=1004)
        lx, lw = gi.conv_inputs_device(LONG_T, C, 4, torch.bfloat16, seed=1004)
        ly = torch.empty_like(lx)
        lo = torch.empty(LONG_T, H, D, device=dev)
        n_lck = g.count_boundaries(0, LONG_T, BLOCK)
        lpool = g.CheckpointPool(torch.zeros(n_lck, PAGE_BYTES, dtype=torch.uint8, device=dev), BLOCK)
        lids = list(range(n_lck))
        lws = torch.empty(g.prefill_workspace_bytes(layer, [0, LONG_T], [0], BLOCK), dtype=torch.uint8, device=dev)
        lcws = torch.empty(max(256, g.conv_workspace_bytes(layer, [0, LONG_T], [0], BLOCK)), dtype=torch.uint8,
                           device=dev)
        lS = torch.empty(H, D, D, device=dev)
        ltail = torch.empty(3, C, dtype=torch.bfloat16, device=dev)

        def long_step(i=0):
            g.conv_update(layer, lx, lw, [("zero", None, ltail)], [0, LONG_T], [0], ly, ckpt=lpool, page_ids=lids,
                          workspace=lcws)
            g.chunk_prefill(layer, lq, lk, lv, la, lb, [0, LONG_T], [0], [("zero", None, lS)], lo, ckpt=lpool,
                            page_ids=lids, workspace=lws)

        long_ms = [u / 1e3 for u in batches_us(long_step, batches=3, per_batch=1, warm=1)]
        long_scan = batches_us(lambda i: g.prefill_scan(layer, lq, lk, lv, [0, LONG_T], [0], [("zero", None, lS)],
                                                        lo, lws, ckpt=lpool, page_ids=lids),
                               batches=3, per_batch=1, warm=0)
        long_res = {"ms_per_step": pct(long_ms),
                    "tokens_per_s": round(LONG_T / (statistics.median(long_ms) * 1e-3), 1),
                    "scan_ms": round(statistics.median(long_scan) / 1e3, 3), "checkpoints": n_lck,
                    "workload": "long_27b_T229376_H48_d128_block896 (conv + chunked prefill, 256 checkpoints)"}
        del lq, lk, lv, la, lb, lx, ly, lo, lpool, lws
        torch.cuda.empty_cache()

    conv_bytes = 2 * T * C * 2
    conv_med = statistics.median(conv_us)
    flush_med = statistics.median(flush_u)
    replay_med = statistics.median(replay)
    decode_med = statistics.median(decode)
    result = {
        "metric": "GDN prefill tokens/s/layer (48h x 128^2, fp32 state) + flush us/layer",
        "value": round(value, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, fp32 state/outputs (bf16-split fp32 products)",
        "data": "synthetic, seeded",
        "config": {"workload": "prefill_27b_T8192_H48_d128_block896 (conv 18432 ch + chunked prefill, "
                               "9 checkpoints)", "tokens": T, "heads": H, "head_dim": D, "block": BLOCK,
                   "chunk": CHUNK},
        "device": dev_info,
        "kernel_us": {"conv": pct(conv_us), "factorize": pct(fact_us), "scan": pct(scan_us)},
        "varlen_stepped": {"tokens": varlen_tokens, "calls": n_calls, "ms": pct(varlen_ms),
                           "tokens_per_s": round(varlen_tokens / (statistics.median(varlen_ms) * 1e-3), 1),
                           "workload": "varlen_27b_4seq_block896: 2688/5000/6272/12000 tokens in calls of <= 1792 "
                                       "per sequence, two resuming at 1792 from cross-written checkpoints "
                                       "(conv + chunked prefill per call)"},
        "long_prefill": long_res,
        "flush_us_per_layer": {"accepted_u1_16": pct(flush_u), "all_16": sweep["16"], "all_17": sweep["17"],
                               "sweep_all_n": sweep,
                               "sweep_64slot_log": sweep64,
                               "workload": "flush_4b_16req_H32_d128_32slots (64 slots for n = 33 and sweep_64slot_log)",
                               "hbm_gbs_u1_16": round(fb_u / (flush_med * 1e-6) / 1e9, 1),
                               "roof_us_u1_16": round(fb_u / (PEAK_HBM_GBS * 1e9) * 1e6, 2),
                               "frac_u1_16": round(fb_u / (flush_med * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)},
        "replay_forward_us": {"value": pct(replay),
                              "workload": "replay_4b_16req_H32_d128_32slots_logged_u1_16_new16",
                              "hbm_gbs": round(rb / (replay_med * 1e-6) / 1e9, 1),
                              "roof_us": round(rb / (PEAK_HBM_GBS * 1e9) * 1e6, 2),
                              "log64": {"value": pct(replay64),
                                        "workload": "replay_4b_16req_H32_d128_64slots_logged_25_40_new16",
                                        "roof_us": round(rb64 / (PEAK_HBM_GBS * 1e9) * 1e6, 2)}},
        "decode_us": {"value": pct(decode), "workload": "decode_27b_256req_H48_d128",
                      "hbm_gbs": round(dec_bytes / (decode_med * 1e-6) / 1e9, 1),
                      "roof_us": round(dec_bytes / (PEAK_HBM_GBS * 1e9) * 1e6, 2),
                      "frac": round(dec_bytes / (decode_med * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)},
        "conv_decode_us": {"value": pct(conv_dec), "workload": "conv decode regime, 256 requests x 18432 channels",
                           "hbm_gbs": round(conv_dec_bytes / (statistics.median(conv_dec) * 1e-6) / 1e9, 1)},
        "mixed_step": {"ms": pct(mixed), "prefill_tokens": T, "decode_tokens": n_dec,
                       "tokens_per_s": round((T + n_dec) / (statistics.median(mixed) * 1e-3), 1),
                       "workload": "27b layer: 256 decode tokens + the 8192-token prefill in one packed batch"},
        "conv": {"us": round(conv_med, 2), "hbm_gbs": round(conv_bytes / (conv_med * 1e-6) / 1e9, 1),
                 "frac": round(conv_bytes / (conv_med * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)},
        "core_steps_us": {"conv_with_qk_l2norm": pct(conv_norm_us), "gates": pct(gates_us),
                          "gated_norm": pct(norm_us),
                          "gated_norm_hbm_gbs": round(norm_bytes / (statistics.median(norm_us) * 1e-6) / 1e9, 1),
                          "gates_hbm_gbs": round(gate_bytes / (statistics.median(gates_us) * 1e-6) / 1e9, 1),
                          "workload": "27b layer, 8192 tokens x 48 heads x 128"},
        "roofline": {
            "kernel": "scan_staged_kernel<bf16,128>",
            "bound": "mfma",
            "achieved": round(achieved_tflops, 2),
            # the bf16 dense peak scaled by algorithmic / pass-weighted flops: the peak of
            # this product mix on the bf16 matrix cores
            "peak": round(eff_peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved_tflops / eff_peak, 4),
            "traffic": int(prof["traffic_bytes_per_launch"]) if prof and "traffic_bytes_per_launch" in prof else None,
            "mfma_busy": prof.get("mfma_busy_fraction") if prof else None,
            "launch_us": round(scan_med, 2),
            "algorithmic_flops_per_launch": alg,
            "pass_weighted_flops_per_launch": passes,
            "issued_mfma_flops_per_launch": scan_issued_flops(T, H),
            "bf16_dense_peak": PEAK_BF16_TFLOPS,
        },
    }

    # ------------------------------------------------------------ CPU oracle, bounded sample
    if not args.no_cpu:
        note("cpu oracle")
        from oracle import oracle
        qs, ks, vs, as_, bs = (t.float().double().cpu().numpy() for t in (q, k, v, a, b))
        threads = oracle.max_threads()
        runs = []
        # the whole prefill workload (all tokens, all heads) on the allotted cores, run
        # repeatedly until about 10 s of CPU time have passed
        while sum(runs) < 10.0 and len(runs) < 50:
            t1 = time.perf_counter()
            oracle.recurrence(qs, ks, vs, as_, bs, 1.0, None, 0, BLOCK, threads=threads)
            runs.append(time.perf_counter() - t1)
        cpu_s = statistics.median(runs)
        # one core: 4 of the 48 heads, scaled to the layer
        hsel = [0, 12, 24, 36]
        t1 = time.perf_counter()
        oracle.recurrence(qs[:, hsel], ks[:, hsel], vs[:, hsel], as_[:, hsel], bs[:, hsel], 1.0, None, 0, BLOCK,
                          threads=1)
        one_s = (time.perf_counter() - t1) * H / len(hsel)
        result["cpu_baseline"] = {"value": round(T / cpu_s, 1), "unit": "tokens/s/layer",
                                  "cores": threads, "kind": "oracle",
                                  "one_core_value": round(T / one_s, 1),
                                  "cpu_model": cpu_model(), "nproc": os.cpu_count(),
                                  "sample": f"the full prefill workload ({T} tokens x {H} heads, checkpoints "
                                            f"every {BLOCK}), fp64 token loop on {threads} threads, median of "
                                            f"{len(runs)} runs ({round(cpu_s, 3)} s each); one core: 4 heads, "
                                            f"scaled by 12"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
