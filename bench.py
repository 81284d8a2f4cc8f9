"""Benchmark of the libgdn hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Step = one pass of the prefill hot path over one 27B-shaped layer, as two library
calls: the causal conv update over the packed q|k|v channels (18,432 bf16 channels,
8,192 tokens) and the chunked prefill (pre-pass and scan in one call) of the gated delta rule (48 heads, 128 x 128 fp32 state per head,
bf16 q/k/v, fp32 o, 64-token chunks) writing a checkpoint page at each of the nine
896-token block boundaries.  `value` is prefill tokens per second per layer over the
K timed steps (inputs resident in HBM, synthetic, seeded).

Reported beside it, each timed with HIP events on the stream the kernels run on:
  * the replay flush at the 4B-shaped layer (16 requests, 32 value heads x 128 x 128
    fp32 state, a 32-slot log, accepted rows uniform in 1..16, plus all-16 and all-17;
    and long drafts in a 64-slot log, all-32 and all-33),
    rotating over enough state pools that every launch streams from HBM;
  * the replay outputs at the same layer: 16 new rows behind each request's accepted
    rows in the log, outputs of the new rows from the state and the log;
  * the decode step for 256 requests at the 27B shape, and a mixed step: those 256 decode
    tokens and the 8,192-token prefill in one packed batch (conv over all sequences,
    prefill over its rows, the decode rows through decode_mixed);
  * the conv update alone, and the packed-core steps at the same layer: the conv with
    the per-head q/k L2 norm fused, the gates from the "ba" projection, the gated RMSNorm
    of the output rows;
  * the roofline of the dominant kernel (the chunk scan);
  * the fp64 CPU oracle timed on a bounded sample of the same workload.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Published MI355X peaks.
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_MFMA_TFLOPS = 157.3

# Prefill workload: one 27B-shaped GDN layer.
T, H, D, BLOCK, CHUNK = 8192, 48, 128, 896, 64
PAGE_BYTES = BLOCK * 4096  # one attention page of 4,096 B per token


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


def measured_scan_traffic():
    """HBM bytes per scan launch from the committed counter profile (FETCH_SIZE and
    WRITE_SIZE, calibrated against a plain copy), or None once the kernel sources differ
    from the ones the counters were taken on."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "prefill_27b_T8192_H48_hbm_traffic.md")
    csrc = os.path.join(ROOT, "gated_deltanet_recurrent_chunk_amd", "csrc")
    try:
        text = open(path).read()
        src = b"".join(open(os.path.join(csrc, f), "rb").read()
                       for f in ("prefill_kernels.hip", "chunk_common.h", "device_common.h"))
    except OSError:
        return None
    sha = re.search(r"source_sha256[^:]*: ([0-9a-f]{64})", text)
    nbytes = re.search(r"scan_traffic_bytes_per_launch: (\d+)", text)
    if not sha or not nbytes or sha.group(1) != hashlib.sha256(src).hexdigest():
        return None
    return int(nbytes.group(1))


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
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

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

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
    cws = torch.empty(g.conv_workspace_bytes(layer, cu, sp, BLOCK), dtype=torch.uint8, device=dev)

    def step():
        g.conv_update(layer, x, w, [("zero", None, tail)], cu, sp, y, ckpt=pool, page_ids=page_ids, workspace=cws)
        g.chunk_prefill(layer, q, k, v, a, b, cu, sp, [("zero", None, S)], o, ckpt=pool, page_ids=page_ids,
                        workspace=ws)

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

    # Per-kernel launch durations: each stage launched `reps` times back to back between
    # two events on the stream the kernels run on (torch's current stream), so the host
    # planning of one call overlaps the previous launch and only GPU time counts.
    def time_stage(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev = events(2)
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    kreps = max(10, args.steps)
    conv_ms = time_stage(lambda: g.conv_update(layer, x, w, [("zero", None, tail)], cu, sp, y, ckpt=pool,
                                               page_ids=page_ids, workspace=cws), kreps)
    fact_ms = time_stage(lambda: g.prefill_factorize(layer, q, k, a, b, cu, sp, BLOCK, ws), kreps)
    scan_ms = time_stage(lambda: g.prefill_scan(layer, q, k, v, cu, sp, [("zero", None, S)], o, ws, ckpt=pool,
                                                page_ids=page_ids), kreps)
    # packed-core steps at the same layer: the conv with the per-head q/k L2 norm fused,
    # the gates from the "ba" projection, the gated RMSNorm of the output rows
    nlayer = g.Layer(H, H, D, torch.bfloat16, scale=1.0, conv_act=g.ACT_SILU | g.CONV_QK_L2NORM)
    conv_norm_ms = time_stage(lambda: g.conv_update(nlayer, x, w, [("zero", None, tail)], cu, sp, y, ckpt=pool,
                                                    page_ids=page_ids, workspace=cws), kreps)
    ba, A_log, dt_bias, _, zc, wn = gi.core_inputs(T, H, D, torch.bfloat16, seed=1006)
    ba, A_log, dt_bias, zc, wn = (t_.to(dev) for t_ in (ba, A_log, dt_bias, zc, wn))
    ga, gb = torch.empty(T, H, device=dev), torch.empty(T, H, device=dev)
    gates_ms = time_stage(lambda: g.gates(layer, ba, A_log, dt_bias, ga, gb), kreps)
    onorm = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    norm_ms = time_stage(lambda: g.gated_norm(layer, o, zc, wn, onorm), kreps)
    norm_bytes = T * H * D * (4 + 2 + 2)
    gate_bytes = T * 2 * H * 2 + 2 * T * H * 4

    alg = scan_algorithmic_flops(T, H)
    passes = scan_pass_flops(T, H)
    achieved_tflops = alg / (scan_ms * 1e-3) / 1e12
    eff_peak = PEAK_BF16_TFLOPS * alg / passes
    traffic = measured_scan_traffic()

    # ------------------------------------------------------------ replay flush (4B layer)
    fl_layer = g.Layer(16, 32, D, torch.bfloat16)
    n_req, rows = 16, 32
    state_mib = n_req * 32 * D * D * 4 / 2 ** 20
    n_pools = int(np.ceil(2 * 256 / state_mib)) + 1  # > 2 x 256 MB last-level cache in rotation
    fpools = [gi.states(n_req, 32, D, seed=1003 + i).to(dev) for i in range(n_pools)]
    _, bk, bv, ba, bb = gi.qkvab(n_req * rows, 16, 32, D, torch.bfloat16, seed=1003)
    bk = bk.view(n_req, rows, 16, D).to(dev)
    bv = bv.view(n_req, rows, 32, D).to(dev)
    ba = ba.view(n_req, rows, 32).to(dev)
    bb = bb.view(n_req, rows, 32).to(dev)
    slots = torch.arange(n_req, dtype=torch.int32, device=dev)
    acc_u = gi.accepted_counts(n_req, 1003)

    def time_flush(acc, reps):
        """Average duration of one flush launch: `reps` launches back to back between two
        events (rotating state pools), so launch gaps do not count."""
        acc_d = acc.to(torch.int32).to(dev)
        for i in range(3):
            g.replay_flush(fl_layer, fpools[i % n_pools], slots, bk, bv, ba, bb, acc_d)
        torch.cuda.synchronize()
        ev = events(2)
        ev[0].record()
        for r in range(reps):
            g.replay_flush(fl_layer, fpools[r % n_pools], slots, bk, bv, ba, bb, acc_d)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / reps

    reps = max(100, 5 * args.steps)
    flush_u = time_flush(acc_u, reps)
    flush_16 = time_flush(torch.full((n_req,), 16), reps)
    flush_17 = time_flush(torch.full((n_req,), 17), reps)
    fb_u = flush_bytes(acc_u.tolist())
    # long drafts: a 64-slot log, 32 accepted rows per request (and 33: no cliff past a block)
    rows64 = 64
    _, lk, lv, la, lb = gi.qkvab(n_req * rows64, 16, 32, D, torch.bfloat16, seed=1007)
    lk, lv = lk.view(n_req, rows64, 16, D).to(dev), lv.view(n_req, rows64, 32, D).to(dev)
    la, lb = la.view(n_req, rows64, 32).to(dev), lb.view(n_req, rows64, 32).to(dev)

    def time_flush64(acc, reps):
        acc_d = acc.to(torch.int32).to(dev)
        for i in range(3):
            g.replay_flush(fl_layer, fpools[i % n_pools], slots, lk, lv, la, lb, acc_d)
        torch.cuda.synchronize()
        ev = events(2)
        ev[0].record()
        for r in range(reps):
            g.replay_flush(fl_layer, fpools[r % n_pools], slots, lk, lv, la, lb, acc_d)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / reps

    flush_32 = time_flush64(torch.full((n_req,), 32), reps)
    flush_33 = time_flush64(torch.full((n_req,), 33), reps)

    # ------------------------------------------------------------ replay outputs (4B layer)
    # the verify step of the pages' drafts: 16 new rows behind each request's accepted
    # rows (uniform in 1..16) in the same 32-slot log, outputs of the 16 new rows
    n_new = 16
    rq_new = gi.qkvab(n_req * n_new, 16, 32, D, torch.bfloat16, seed=1004)[0].view(n_req, n_new, 16, D).to(dev)
    r_out = torch.empty(n_req, n_new, 32, D, dtype=torch.float32, device=dev)
    logged_d = acc_u.to(torch.int32).to(dev)
    new_d = torch.full((n_req,), n_new, dtype=torch.int32, device=dev)
    for i in range(3):
        g.replay_forward(fl_layer, fpools[i % n_pools], slots, bk, bv, ba, bb, logged_d, new_d, rq_new, r_out)
    torch.cuda.synchronize()
    ev = events(2)
    ev[0].record()
    for r in range(reps):
        g.replay_forward(fl_layer, fpools[r % n_pools], slots, bk, bv, ba, bb, logged_d, new_d, rq_new, r_out)
    ev[1].record()
    torch.cuda.synchronize()
    replay_us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    rb = replay_bytes(acc_u.tolist(), n_new)

    # ------------------------------------------------------------ decode (27B layer, 256 requests)
    # (the mixed-batch step, below, needs the prefill inputs and the decode pool)
    n_dec = 256
    dpool = gi.states(n_dec, H, D, seed=1005).to(dev)
    dq, dk, dv, da, db = (t.to(dev) for t in gi.qkvab(n_dec, H, H, D, torch.bfloat16, seed=1005))
    dout = torch.empty(n_dec, H, D, dtype=torch.float32, device=dev)
    dslots = torch.arange(n_dec, dtype=torch.int32, device=dev)
    for _ in range(3):
        g.decode_step(layer, dq, dk, dv, da, db, dpool, dslots, dout)
    torch.cuda.synchronize()
    ev = events(2)
    ev[0].record()
    for _ in range(reps):
        g.decode_step(layer, dq, dk, dv, da, db, dpool, dslots, dout)
    ev[1].record()
    torch.cuda.synchronize()
    decode_us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    dec_bytes = n_dec * (2 * H * D * D * 4 + 3 * H * D * 2 + 2 * H * 4 + H * D * 4)

    # ------------------------------------------------------------ mixed batch (27B layer)
    # one packed batch: 256 decode tokens (rows 0..255) and the 8,192-token prefill behind
    # them; the conv runs over the prefill sequence and, in its decode regime, over the
    # decode tokens (their tails in a slot pool), the prefill over its rows, the decode
    # tokens through decode_mixed
    mT = n_dec + T
    mx = torch.cat([gi.conv_inputs(n_dec, C, 4, torch.bfloat16, seed=1008)[0].to(dev), x])
    my = torch.empty_like(mx)
    mq, mk, mv = (torch.cat([d_, p_]) for d_, p_ in ((dq, q), (dk, k), (dv, v)))
    ma, mb = torch.cat([da, a]), torch.cat([db, b])
    mo = torch.empty(mT, H, D, dtype=torch.float32, device=dev)
    mtails = torch.zeros(n_dec, 3, C, dtype=torch.bfloat16, device=dev)
    mrows = torch.arange(n_dec, dtype=torch.int32, device=dev)
    pre = slice(n_dec, mT)

    def mixed_step():
        g.conv_update(layer, mx[pre], w, [("zero", None, tail)], cu, sp, my[pre], ckpt=pool, page_ids=page_ids,
                      workspace=cws)
        g.conv_decode(layer, mx, w, mtails, dslots, my, rows=mrows)
        g.chunk_prefill(layer, mq[pre], mk[pre], mv[pre], ma[pre], mb[pre], cu, sp, [("zero", None, S)], mo[pre],
                        ckpt=pool, page_ids=page_ids, workspace=ws)
        g.decode_mixed(layer, mq, mk, mv, ma, mb, dpool, dslots, mrows, mo)

    def time_steps(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / args.steps

    mixed_ms = time_steps(mixed_step)

    conv_bytes = 2 * T * C * 2
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
        "kernel_ms": {"conv": round(conv_ms, 4), "factorize": round(fact_ms, 4), "scan": round(scan_ms, 4)},
        "flush_us_per_layer": {"accepted_u1_16": round(flush_u, 2), "all_16": round(flush_16, 2),
                               "all_17": round(flush_17, 2),
                               "log64_all_32": round(flush_32, 2), "log64_all_33": round(flush_33, 2),
                               "hbm_gbs_log64_all_32": round(flush_bytes([32] * n_req) / (flush_32 * 1e-6) / 1e9, 1),
                               "workload": "flush_4b_16req_H32_d128_32slots",
                               "hbm_gbs_u1_16": round(fb_u / (flush_u * 1e-6) / 1e9, 1),
                               "roof_us_u1_16": round(fb_u / (PEAK_HBM_GBS * 1e9) * 1e6, 2)},
        "replay_forward_us": {"value": round(replay_us, 2),
                              "workload": "replay_4b_16req_H32_d128_32slots_logged_u1_16_new16",
                              "hbm_gbs": round(rb / (replay_us * 1e-6) / 1e9, 1),
                              "roof_us": round(rb / (PEAK_HBM_GBS * 1e9) * 1e6, 2)},
        "mixed_step": {"ms": round(mixed_ms, 4), "prefill_tokens": T, "decode_tokens": n_dec,
                       "tokens_per_s": round((T + n_dec) / (mixed_ms * 1e-3), 1),
                       "workload": "27b layer: 256 decode tokens + the 8192-token prefill in one packed batch"},
        "decode_us": {"value": round(decode_us, 2), "workload": "decode_27b_256req_H48_d128",
                      "hbm_gbs": round(dec_bytes / (decode_us * 1e-6) / 1e9, 1),
                      "roof_us": round(dec_bytes / (PEAK_HBM_GBS * 1e9) * 1e6, 2)},
        "conv": {"us": round(conv_ms * 1e3, 2), "hbm_gbs": round(conv_bytes / (conv_ms * 1e-3) / 1e9, 1)},
        "core_steps_us": {"conv_with_qk_l2norm": round(conv_norm_ms * 1e3, 2), "gates": round(gates_ms * 1e3, 2),
                          "gated_norm": round(norm_ms * 1e3, 2),
                          "gated_norm_hbm_gbs": round(norm_bytes / (norm_ms * 1e-3) / 1e9, 1),
                          "gates_hbm_gbs": round(gate_bytes / (gates_ms * 1e-3) / 1e9, 1),
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
            "traffic": traffic,
            "launch_us": round(scan_ms * 1e3, 2),
            "algorithmic_flops_per_launch": alg,
            "pass_weighted_flops_per_launch": passes,
            "issued_mfma_flops_per_launch": scan_issued_flops(T, H),
            "bf16_dense_peak": PEAK_BF16_TFLOPS,
            "fp32_mfma_equivalent": {"peak": PEAK_FP32_MFMA_TFLOPS,
                                     "frac": round(achieved_tflops / PEAK_FP32_MFMA_TFLOPS, 4)},
        },
    }

    # ------------------------------------------------------------ CPU oracle, bounded sample
    if not args.no_cpu:
        from oracle import oracle
        # the whole prefill workload (all tokens, all heads), run repeatedly until about
        # 10 s of CPU time have passed; the median run gives the rate
        qs, ks, vs, as_, bs = (t.float().double().cpu().numpy() for t in (q, k, v, a, b))
        threads = min(os.cpu_count() or 1, 16)
        runs = []
        while sum(runs) < 10.0 and len(runs) < 50:
            t1 = time.perf_counter()
            oracle.recurrence(qs, ks, vs, as_, bs, 1.0, None, 0, BLOCK, threads=threads)
            runs.append(time.perf_counter() - t1)
        cpu_s = statistics.median(runs)
        result["cpu_baseline"] = {"value": round(T / cpu_s, 1), "unit": "tokens/s/layer",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"the full prefill workload ({T} tokens x {H} heads, checkpoints "
                                            f"every {BLOCK}), fp64 token loop, median of {len(runs)} runs "
                                            f"({round(cpu_s, 3)} s each)"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
