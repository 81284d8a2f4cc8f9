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
