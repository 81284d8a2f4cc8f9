"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/gdn_oracle.c with one plausible mistake (a flipped
sign, a dropped term, a wrong operand or index, an off-by-one boundary), compiled on
the CPU into a temporary library.  Every pin test of the oracle is then run against
it; at least one must fail.  The real oracle passes all of them (test_oracle_pins.py).
"""
import inspect
import numpy as np
import os
import subprocess

import pytest

from oracle import oracle
import test_chunked_form
import test_oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "gdn_oracle.c")

MUTANTS = {
    "write_sign": ("row[j] += w * k[j];", "row[j] -= w * k[j];"),
    "no_decay": ("row[j] = a * row[j];", "row[j] = row[j];"),
    "read_before_decay": ("double w = b * (v[i] - u);", "double w = b * (v[i] - u / a);"),
    "strength_on_read_only": ("double w = b * (v[i] - u);", "double w = v[i] - b * u;"),
    "output_reads_key": ("r += row[j] * q[j];", "r += row[j] * k[j];"),
    "output_unscaled": ("o[i] = scale * r;", "o[i] = r;"),
    "head_mapping": ("const int hk = h / group;", "const int hk = h % Hqk;"),
    "ckpt_off_by_one": ("pos_after % block == 0", "(pos_after - 1) % block == 0"),
    "conv_tap_order": ("s += w[(size_t)c * W + j] * xe[t + j];",
                       "s += w[(size_t)c * W + (W - 1 - j)] * xe[t + j];"),
    "conv_ckpt_tail_shift": ("xe[t + 1 + i]", "xe[t + i]"),
    "conv_silu_sign": ("s = s / (1.0 + exp(-s));", "s = s / (1.0 + exp(s));"),
    "cached_keeps_last_block": ("return full >= 1 ? (full - 1) * block : 0;",
                                "return full * block;"),
}


def _pins():
    fns = []
    for mod in (test_oracle_pins, test_chunked_form):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if name.startswith("test_") and not hasattr(fn, "pytestmark") \
                    and not inspect.signature(fn).parameters:
                fns.append(fn)
    # parametrised chunked-form cases
    for args in [(0, 64, 64, 16, 16, 2, 2), (700, 260, 64, 784, 8, 2, 2), (0, 97, 64, 0, 5, 1, 3)]:
        fns.append(lambda args=args: test_chunked_form.test_chunked_form_matches_token_loop(*args))
    return fns


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    path_c = tmp_path / f"{name}.c"
    path_c.write_text(src.replace(old, new))
    path_so = str(tmp_path / f"{name}.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(path_c), "-o",
                    path_so, "-lm"], check=True)
    oracle._load()
    prev = oracle._swap_library(path_so)
    failed = []
    try:
        for fn in _pins():
            try:
                fn()
            except Exception:  # an assertion or a shape mismatch both count as caught
                failed.append(getattr(fn, "__name__", "chunked"))
    finally:
        oracle._swap_library(prev)
    assert failed, f"no pin caught mutant {name}"


# bf16 rounding is Python (oracle.bf16_round); its mutants replace the function.
def _bf16_truncate(x):
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def _bf16_ties_away(x):
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x8000) & 0xFFFF0000).astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_ties_up_in_magnitude_only_for_odd(x):  # ties to odd
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + (1 - lsb)) & 0xFFFF0000).astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("mutant", [_bf16_truncate, _bf16_ties_away, _bf16_ties_up_in_magnitude_only_for_odd])
def test_pins_reject_bf16_rounding_mutant(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "bf16_round", mutant)
    failed = []
    for fn in _pins():
        if "bf16" not in getattr(fn, "__name__", ""):
            continue
        try:
            fn()
        except AssertionError:
            failed.append(fn.__name__)
    assert failed, f"no pin caught {mutant.__name__}"
