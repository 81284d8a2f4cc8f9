"""Helpers for the GPU parity tests: conversions, error metrics, checkpoint pools.

Every expected value in the GPU tests comes from the fp64 oracle (oracle/) run on the
same seeded inputs (gdn_inputs.py); nothing expected is produced by the GPU path.
"""
import sys

import numpy as np
import torch

TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-5}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def f64(t):
    """Exact widening of a bf16 / fp32 tensor to a float64 numpy array."""
    return t.detach().to("cpu").float().double().numpy()


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def bits(t):
    """Raw bit pattern of a tensor (for bit-exactness comparisons, NaN payloads included)."""
    t = t.detach().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu()
    return t.cpu()


def same_bits(a, b):
    return torch.equal(bits(a), bits(b))


NAN_BITS = 0x7FC0DEAD


def nan_fill_(t):
    """Fill a tensor with a recognisable NaN pattern (unused pages, pad slots, rejected rows)."""
    if t.dtype == torch.uint8:
        t.view(torch.int32).fill_(NAN_BITS)
    elif t.dtype == torch.float32:
        t.view(torch.int32).fill_(NAN_BITS)
    elif t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(0x7FC1)
    else:
        raise TypeError(t.dtype)
    return t


def make_pool(g, layer, n_pages, block, page_bytes=None, device="cuda"):
    pb = page_bytes or layer.checkpoint_bytes
    pool = torch.empty(n_pages, pb, dtype=torch.uint8, device=device)
    nan_fill_(pool)
    return g.CheckpointPool(pool, block)


# fp32 holds no relative precision below its smallest normal value: a state decayed by
# a = 2^-126 (the gate step's clamp) sits at or under it, where the right fp32 answer
# is a subnormal or zero.  Per-slice checks therefore allow, beside the relative
# tolerance, an absolute error of one smallest normal per element.
FP32_TINY = 2.0 ** -126


def rel_l2_per(x, ref, axis):
    """Relative L2 error of every slice along `axis` (e.g. per value head): a wrong head
    or row cannot hide under a tensor-wide norm.  Returns (errors, floors): the slice's
    absolute floor sqrt(n) * 2^-126 divided by its reference norm."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, 0)
    ref = np.moveaxis(np.asarray(ref, dtype=np.float64), axis, 0)
    n = x.shape[0]
    d = (x - ref).reshape(n, -1)
    r = ref.reshape(n, -1)
    den = np.linalg.norm(r, axis=1)
    den = np.where(den > 0, den, 1.0)
    floor = np.sqrt(r.shape[1]) * FP32_TINY / den
    return np.linalg.norm(d, axis=1) / den, floor


def assert_close_per(x, ref, tol, axis, what):
    """Tensor-wide relative L2 within tol, and every slice along `axis` within tol plus
    the fp32 floor (see FP32_TINY); names the worst slice."""
    whole = rel_l2(x, ref)
    per, floor = rel_l2_per(x, ref, axis)
    excess = per - (tol + floor)
    worst = int(np.argmax(excess))
    assert whole <= tol, f"{what}: relative L2 {whole:.3e} > {tol}"
    assert excess[worst] <= 0, f"{what}: slice {worst} relative L2 {per[worst]:.3e} > {tol} (+ floor {floor[worst]:.1e})"
    return whole, float(per[worst])
