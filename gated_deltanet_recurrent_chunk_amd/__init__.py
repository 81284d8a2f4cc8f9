"""Python binding of libgdn, the Gated DeltaNet recurrent-state update for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libgdn.so`` behind the C ABI declared in ``include/gdn.h``.  PyTorch supplies device
memory and the current stream.  Importing this module loads the library and fails
loudly when it has not been built (``python gated_deltanet_recurrent_chunk_amd/build.py``).

Layouts (token-major, packed over a varlen batch), as in ``include/gdn.h``:
  q, k  [tokens, n_qk_heads, d]  (or rows of a wider packed tensor, see ``qk_stride``)
  v     [tokens, n_v_heads, d]
  a, b  [tokens, n_v_heads] fp32   (decay gate in (0, 1], write strength in [0, 1])
  o     [tokens, n_v_heads, d] fp32
  state [n_v_heads, d, d] fp32     (row = value channel, column = key channel)
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libgdn.so not found at {LIB_PATH}; build it with "
        "`python gated_deltanet_recurrent_chunk_amd/build.py` (there is no CPU fallback)")
_lib = ctypes.CDLL(LIB_PATH)

GDN_F32, GDN_BF16 = 0, 1
ACT_NONE, ACT_SILU = 0, 1
CONV_QK_L2NORM = 0x100  # OR into Layer.conv_act: unit L2 norm per q / k head after the conv
SRC_ZERO, SRC_SLOT, SRC_CHECKPOINT = 0, 1, 2
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL_ARG", 2: "GDN_ERR_BAD_SHAPE", 3: "GDN_ERR_BAD_DTYPE",
                4: "GDN_ERR_BAD_VARLEN", 5: "GDN_ERR_OFF_BOUNDARY", 6: "GDN_ERR_PAGE_TOO_SMALL",
                7: "GDN_ERR_BAD_PAGE", 8: "GDN_ERR_CAPACITY", 9: "GDN_ERR_WORKSPACE", 10: "GDN_ERR_HIP",
                11: "GDN_ERR_BAD_SOURCE", 12: "GDN_ERR_STAGING"}
INLINE_SEQS, INLINE_PAGES = 8, 256  # tables up to this size travel in the kernel arguments


class _Layer(ctypes.Structure):
    _fields_ = [("n_qk_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("conv_act", ctypes.c_int32), ("scale", ctypes.c_float)]


class _Varlen(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("cu_seqlens", ctypes.POINTER(ctypes.c_int64)),
                ("start_pos", ctypes.POINTER(ctypes.c_int64))]


class _StateRef(ctypes.Structure):
    _fields_ = [("src_kind", ctypes.c_int32), ("src", ctypes.c_void_p), ("dst", ctypes.c_void_p)]


class _Staging(ctypes.Structure):
    _fields_ = [("host", ctypes.c_void_p), ("bytes", ctypes.c_size_t)]


class _Ckpt(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("page_bytes", ctypes.c_int64), ("n_pages", ctypes.c_int64),
                ("block", ctypes.c_int32), ("page_ids", ctypes.POINTER(ctypes.c_int32))]


_P = ctypes.POINTER
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


def _decl(name, restype, argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = argtypes
    return f


_decl("gdn_abi_version", _i32, [])
_decl("gdn_status_string", ctypes.c_char_p, [_i32])
for _n in ("gdn_state_bytes", "gdn_conv_tail_bytes", "gdn_checkpoint_bytes", "gdn_conv_channels"):
    _decl(_n, _i64, [_P(_Layer)])
_decl("gdn_cached_prefix_tokens", _i64, [_i64, _i64])
_decl("gdn_floor_chunk", _i64, [_i64, _i64])
_decl("gdn_count_boundaries", _i64, [_i64, _i64, _i64])
_decl("gdn_block_size_for_state", _i64, [_i64, _i64, _i64])
_decl("gdn_prefill_workspace_bytes", _i64, [_P(_Layer), _P(_Varlen), _i32])
_decl("gdn_prefill_staging_bytes", _i64, [_P(_Layer), _P(_Varlen), _i32])
_decl("gdn_conv_workspace_bytes", _i64, [_P(_Layer), _P(_Varlen), _i32])
_decl("gdn_conv_staging_bytes", _i64, [_P(_Layer), _P(_Varlen), _i32])
_decl("gdn_conv_update", _i32, [_P(_Layer), _vp, _P(_Varlen), _vp, _i64, _vp, _P(_StateRef), _P(_Ckpt), _vp, _vp,
                                _sz, _P(_Staging)])
_decl("gdn_conv_decode", _i32, [_P(_Layer), _vp, _i32, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp])
_decl("gdn_chunk_prefill", _i32, [_P(_Layer), _vp, _P(_Varlen), _vp, _vp, _vp, _i64, _i64, _vp, _vp,
                                  _P(_StateRef), _P(_Ckpt), _vp, _vp, _sz, _P(_Staging)])
_decl("gdn_chunk_prefill_noalloc", _i32, [_P(_Layer), _vp, _P(_Varlen), _vp, _vp, _vp, _i64, _i64, _vp, _vp,
                                          _P(_StateRef), _P(_Ckpt), _vp])
_decl("gdn_prefill_factorize", _i32, [_P(_Layer), _vp, _P(_Varlen), _vp, _vp, _i64, _vp, _vp, _i32, _vp, _sz,
                                      _P(_Staging)])
_decl("gdn_prefill_scan", _i32, [_P(_Layer), _vp, _P(_Varlen), _vp, _vp, _vp, _i64, _i64, _P(_StateRef),
                                 _P(_Ckpt), _vp, _vp, _sz, _P(_Staging)])
_decl("gdn_decode_step", _i32, [_P(_Layer), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp])
_decl("gdn_replay_flush", _i32, [_P(_Layer), _vp, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp])
_decl("gdn_decode_mixed", _i32, [_P(_Layer), _vp, _i32, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _vp,
                                 _vp, _vp, _vp])
_decl("gdn_gates", _i32, [_P(_Layer), _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp])
_decl("gdn_gated_norm", _i32, [_P(_Layer), _vp, _i64, _vp, _vp, _i64, _vp, ctypes.c_float, _vp])
_decl("gdn_core_prefill_workspace_bytes", _i64, [_P(_Layer), _P(_Varlen), _i32])
_decl("gdn_core_prefill_staging_bytes", _i64, [_P(_Layer), _P(_Varlen), _i32])
_decl("gdn_core_prefill", _i32, [_P(_Layer), _vp, _P(_Varlen), _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                 ctypes.c_float, _P(_StateRef), _P(_StateRef), _P(_Ckpt), _vp, _vp, _sz,
                                 _P(_Staging)])
_decl("gdn_replay_forward", _i32, [_P(_Layer), _vp, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                   _i32, _vp, _vp])

EXPORTED = ("gdn_abi_version", "gdn_status_string", "gdn_state_bytes", "gdn_conv_tail_bytes",
            "gdn_checkpoint_bytes", "gdn_conv_channels", "gdn_cached_prefix_tokens", "gdn_floor_chunk",
            "gdn_count_boundaries", "gdn_block_size_for_state", "gdn_prefill_workspace_bytes",
            "gdn_prefill_staging_bytes", "gdn_conv_workspace_bytes", "gdn_conv_staging_bytes", "gdn_conv_update",
            "gdn_conv_decode", "gdn_chunk_prefill", "gdn_chunk_prefill_noalloc", "gdn_prefill_factorize",
            "gdn_prefill_scan", "gdn_decode_step", "gdn_replay_flush", "gdn_replay_forward",
            "gdn_gates", "gdn_gated_norm", "gdn_decode_mixed", "gdn_core_prefill_workspace_bytes",
            "gdn_core_prefill_staging_bytes", "gdn_core_prefill")


class GdnError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = _lib.gdn_status_string(status).decode()
        super().__init__(f"{call}: {STATUS_NAMES.get(status, status)} ({msg})")


def _check(status: int, call: str):
    if status != 0:
        raise GdnError(status, call)


# ------------------------------------------------------------------ descriptors

@dataclasses.dataclass(frozen=True)
class Layer:
    n_qk_heads: int
    n_v_heads: int
    head_dim: int
    io_dtype: torch.dtype = torch.bfloat16
    scale: float = 1.0
    conv_act: int = ACT_SILU
    conv_width: int = 4

    def c(self) -> _Layer:
        io = {torch.bfloat16: GDN_BF16, torch.float32: GDN_F32}.get(self.io_dtype, -1)
        return _Layer(self.n_qk_heads, self.n_v_heads, self.head_dim, self.conv_width, io, self.conv_act,
                      float(self.scale))

    @property
    def state_bytes(self) -> int:
        return int(_lib.gdn_state_bytes(ctypes.byref(self.c())))

    @property
    def conv_tail_bytes(self) -> int:
        return int(_lib.gdn_conv_tail_bytes(ctypes.byref(self.c())))

    @property
    def checkpoint_bytes(self) -> int:
        return int(_lib.gdn_checkpoint_bytes(ctypes.byref(self.c())))

    @property
    def conv_channels(self) -> int:
        return int(_lib.gdn_conv_channels(ctypes.byref(self.c())))


class _Varlens:
    """Keeps the host arrays alive for the duration of a call."""

    def __init__(self, cu_seqlens: Sequence[int], start_pos: Sequence[int]):
        n = len(start_pos)
        self.cu = (ctypes.c_int64 * (n + 1))(*[int(x) for x in cu_seqlens])
        self.sp = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in start_pos])
        self.c = _Varlen(n, self.cu, self.sp)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


@dataclasses.dataclass
class CheckpointPool:
    """Caller-owned checkpoint pages: ``pool`` is a uint8 device tensor [n_pages, page_bytes];
    a page holds the fp32 state, then the conv tail."""
    pool: torch.Tensor
    block: int

    @property
    def page_bytes(self) -> int:
        return int(self.pool.shape[1])

    @property
    def n_pages(self) -> int:
        return int(self.pool.shape[0])

    def page_ptr(self, page: int) -> int:
        return self.pool.data_ptr() + int(page) * self.page_bytes

    def state_view(self, page: int, layer: Layer) -> torch.Tensor:
        nb = layer.state_bytes
        return self.pool[page, :nb].view(torch.float32).view(layer.n_v_heads, layer.head_dim, layer.head_dim)

    def tail_view(self, page: int, layer: Layer) -> torch.Tensor:
        off, nb = layer.state_bytes, layer.conv_tail_bytes
        return self.pool[page, off:off + nb].view(layer.io_dtype).view(layer.conv_width - 1, layer.conv_channels)


def no_checkpoints() -> CheckpointPool:
    return CheckpointPool(torch.empty(0, 256, dtype=torch.uint8), 0)


def _ckpt_c(ckpt: Optional[CheckpointPool], page_ids: Optional[Sequence[int]]):
    if ckpt is None or ckpt.block == 0:
        return _Ckpt(None, 0, 0, 0, None), None
    ids = list(page_ids) if page_ids is not None else []
    arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
    return _Ckpt(ckpt.pool.data_ptr(), ckpt.page_bytes, ckpt.n_pages, int(ckpt.block), arr), arr


_KINDS = {"zero": SRC_ZERO, "slot": SRC_SLOT, "checkpoint": SRC_CHECKPOINT}


def _refs(refs):
    """refs: list of (kind, src, dst) with kind in {'zero','slot','checkpoint'}; src/dst are
    tensors or raw device addresses (a checkpoint src is a page base address)."""
    arr = (_StateRef * max(len(refs), 1))()
    for i, (kind, src, dst) in enumerate(refs):
        arr[i] = _StateRef(_KINDS[kind], _ptr(src), _ptr(dst))
    return arr


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _rows_ok(t, rows, row_elems, dtype, name):
    """t must hold at least `rows` token rows of `row_elems` elements of `dtype`."""
    if rows == 0 and t is None:
        return
    _need(t is not None, f"{name} is required")
    _need(t.dtype == dtype, f"{name}: dtype {t.dtype}, expected {dtype}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(t.numel() >= rows * row_elems, f"{name}: {t.numel()} elements < {rows} x {row_elems}")


def _strided_rows(t, rows, row_elems, dtype, name) -> int:
    """t: a 2-D [>= rows, >= row_elems] view with unit column stride (dense rows, or the
    leading columns of wider packed rows); returns its row stride in elements."""
    if rows == 0 and t is None:
        return row_elems
    _need(t is not None, f"{name} is required")
    _need(t.dtype == dtype, f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.dim() != 2 and t.is_contiguous():
        t = t.reshape(t.shape[0], -1)
    _need(t.dim() == 2 and t.stride(1) == 1 and t.shape[1] >= row_elems and t.shape[0] >= rows,
          f"{name}: [{rows}, >= {row_elems}] rows with unit column stride expected")
    stride = int(t.stride(0)) if t.shape[0] > 1 else max(int(t.stride(0)), row_elems)
    span = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    _need(span >= ((rows - 1) * stride + row_elems if rows else 0), f"{name}: storage too small for {rows} rows")
    return stride


def _state_ok(x, layer, name):
    if isinstance(x, int) or x is None:
        return
    _need(x.dtype == torch.float32 and x.is_contiguous(), f"{name}: contiguous fp32 state expected")
    _need(x.numel() >= layer.n_v_heads * layer.head_dim ** 2, f"{name}: too small for a state")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _sync(stream):
    if stream is None:
        torch.cuda.current_stream().synchronize()
    elif hasattr(stream, "synchronize"):
        stream.synchronize()
    else:
        torch.cuda.ExternalStream(int(stream)).synchronize()


# ------------------------------------------------------------------ helpers

def cached_prefix_tokens(shared: int, block: int) -> int:
    return int(_lib.gdn_cached_prefix_tokens(shared, block))


def floor_chunk(budget: int, block: int) -> int:
    return int(_lib.gdn_floor_chunk(budget, block))


def count_boundaries(start_pos: int, n_tokens: int, block: int) -> int:
    return int(_lib.gdn_count_boundaries(start_pos, n_tokens, block))


def block_size_for_state(state_bytes: int, attn_bytes_per_token: int, alignment: int) -> int:
    return int(_lib.gdn_block_size_for_state(state_bytes, attn_bytes_per_token, alignment))


def prefill_workspace_bytes(layer: Layer, cu_seqlens, start_pos, block: int) -> int:
    v = _Varlens(cu_seqlens, start_pos)
    return int(_lib.gdn_prefill_workspace_bytes(ctypes.byref(layer.c()), ctypes.byref(v.c), int(block)))


def conv_workspace_bytes(layer: Layer, cu_seqlens, start_pos, block: int) -> int:
    v = _Varlens(cu_seqlens, start_pos)
    return int(_lib.gdn_conv_workspace_bytes(ctypes.byref(layer.c()), ctypes.byref(v.c), int(block)))


def prefill_staging_bytes(layer: Layer, cu_seqlens, start_pos, block: int) -> int:
    v = _Varlens(cu_seqlens, start_pos)
    return int(_lib.gdn_prefill_staging_bytes(ctypes.byref(layer.c()), ctypes.byref(v.c), int(block)))


def conv_staging_bytes(layer: Layer, cu_seqlens, start_pos, block: int) -> int:
    v = _Varlens(cu_seqlens, start_pos)
    return int(_lib.gdn_conv_staging_bytes(ctypes.byref(layer.c()), ctypes.byref(v.c), int(block)))


def pinned_staging(nbytes: int) -> torch.Tensor:
    """A pinned host buffer for gdn_staging (keep it untouched until the stream has passed
    the call that used it)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, pin_memory=True)


def _staging(need: int, staging):
    """(struct pointer or None, wait): a call whose tables exceed the kernel arguments
    needs a staging buffer.  Without one from the caller, a pinned buffer is made here and
    the binding waits for the stream after the call, so that the buffer outlives the
    copy that reads it (the synchronous convenience path)."""
    if need <= 0:
        return None, None, False
    own = staging is None
    if own:
        staging = pinned_staging(need)
    _need(staging.device.type == "cpu" and staging.dtype == torch.uint8 and staging.is_contiguous(),
          "staging must be a contiguous uint8 host tensor (pin_memory=True)")
    st = _Staging(staging.data_ptr(), staging.numel())
    return st, staging, own


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    if nbytes < 0:
        return None
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ the hot path

def conv_update(layer: Layer, x, w, tails, cu_seqlens, start_pos, y, ckpt=None, page_ids=None,
                workspace=None, stream=None, staging=None):
    """Causal conv update (gdn_conv_update). tails: per sequence (kind, src, dst).  x may be
    the leading C columns of wider packed rows (its row stride is passed through)."""
    v = _Varlens(cu_seqlens, start_pos)
    rows = int(cu_seqlens[-1]) if len(cu_seqlens) else 0
    C = layer.conv_channels
    xs = _strided_rows(x, rows, C, layer.io_dtype, "x")
    _rows_ok(y, rows, C, layer.io_dtype, "y")
    _rows_ok(w, C, layer.conv_width, layer.io_dtype, "w")
    _need(len(tails) == len(start_pos), "one tail reference per sequence")
    for kind, src, dst in tails:
        for t_ in (src, dst):
            if t_ is not None and not isinstance(t_, int):
                _need(t_.dtype == layer.io_dtype and t_.numel() >= (layer.conv_width - 1) * C, "tail too small")
    block = ckpt.block if ckpt is not None else 0
    ws = _workspace(conv_workspace_bytes(layer, cu_seqlens, start_pos, block), x.device, workspace)
    ck, keep = _ckpt_c(ckpt, page_ids)
    refs = _refs(tails)
    sg, sg_keep, wait = _staging(conv_staging_bytes(layer, cu_seqlens, start_pos, block), staging)
    st = _lib.gdn_conv_update(ctypes.byref(layer.c()), _stream(stream), ctypes.byref(v.c), _ptr(x), xs, _ptr(w),
                              refs, ctypes.byref(ck), _ptr(y), _ptr(ws), ws.numel() if ws is not None else 0,
                              ctypes.byref(sg) if sg is not None else None)
    _check(st, "gdn_conv_update")
    if wait:
        _sync(stream)
    return ws


def conv_decode(layer: Layer, x, w, tail_pool, slot_ids, y, rows=None, status=None, stream=None):
    """The conv's decode regime (gdn_conv_decode): request r's new row is row rows[r] (or
    r) of x [n_rows, >= C] (dense or packed rows); its previous rows are slot slot_ids[r] of tail_pool [n_slots,
    conv_width - 1, C], updated in place; y row rows[r] gets the conv output."""
    n_req = int(slot_ids.numel())
    C = layer.conv_channels
    n_rows = int(x.shape[0])
    _need(slot_ids.dtype == torch.int32 and (rows is None or (rows.dtype == torch.int32 and rows.numel() >= n_req)),
          "int32 slot_ids / rows")
    xs = _strided_rows(x, n_rows, C, layer.io_dtype, "x")
    _rows_ok(y, n_rows, C, layer.io_dtype, "y")
    _rows_ok(w, C, layer.conv_width, layer.io_dtype, "w")
    _need(rows is not None or n_rows >= n_req, "x: one row per request")
    _need(tail_pool.dtype == layer.io_dtype and tail_pool.is_contiguous()
          and tuple(tail_pool.shape[1:]) == (layer.conv_width - 1, C), "tail_pool: [slots, conv_width - 1, C]")
    st = _lib.gdn_conv_decode(ctypes.byref(layer.c()), _stream(stream), n_req, n_rows, _ptr(x), xs, _ptr(w),
                              _ptr(tail_pool), int(tail_pool.shape[0]), _ptr(slot_ids), _ptr(rows), _ptr(y),
                              _ptr(status))
    _check(st, "gdn_conv_decode")


def _check_prefill_operands(layer, cu_seqlens, start_pos, q, k, v, a, b, o, states, qs, vs):
    rows = int(cu_seqlens[-1]) if len(cu_seqlens) else 0
    D, Hv, Hqk = layer.head_dim, layer.n_v_heads, layer.n_qk_heads
    # a strided packed operand must still cover its last row's heads
    for t_, st_, heads, name in ((q, qs, Hqk, "q"), (k, qs, Hqk, "k"), (v, vs, Hv, "v")):
        if t_ is None:
            continue
        _need(t_.dtype == layer.io_dtype, f"{name}: dtype {t_.dtype}, expected {layer.io_dtype}")
        need = (rows - 1) * st_ + heads * D if rows else 0
        span = t_.untyped_storage().nbytes() // t_.element_size() - t_.storage_offset()
        _need(span >= need, f"{name}: storage too small for {rows} rows")
    if a is not None:
        _rows_ok(a, rows, Hv, torch.float32, "a")
    if b is not None:
        _rows_ok(b, rows, Hv, torch.float32, "b")
    if o is not None:
        _rows_ok(o, rows, Hv * D, torch.float32, "o")
    _need(len(states) == len(start_pos), "one state reference per sequence")
    for kind, src, dst in states:
        if kind != "checkpoint":
            _state_ok(src, layer, "state src")
        _state_ok(dst, layer, "state dst")


def chunk_prefill(layer: Layer, q, k, v, a, b, cu_seqlens, start_pos, states, o, ckpt=None, page_ids=None,
                  workspace=None, stream=None, qk_stride=None, v_stride=None, staging=None):
    """Chunked varlen prefill with block checkpoints (gdn_chunk_prefill).
    states: per sequence (kind, src, dst)."""
    vl = _Varlens(cu_seqlens, start_pos)
    qs = qk_stride if qk_stride is not None else layer.n_qk_heads * layer.head_dim
    vs = v_stride if v_stride is not None else layer.n_v_heads * layer.head_dim
    _check_prefill_operands(layer, cu_seqlens, start_pos, q, k, v, a, b, o, states, qs, vs)
    block = ckpt.block if ckpt is not None else 0
    ws = _workspace(prefill_workspace_bytes(layer, cu_seqlens, start_pos, block), q.device, workspace)
    ck, keep = _ckpt_c(ckpt, page_ids)
    refs = _refs(states)
    sg, sg_keep, wait = _staging(prefill_staging_bytes(layer, cu_seqlens, start_pos, block), staging)
    st = _lib.gdn_chunk_prefill(ctypes.byref(layer.c()), _stream(stream), ctypes.byref(vl.c), _ptr(q), _ptr(k),
                                _ptr(v), qs, vs, _ptr(a), _ptr(b), refs, ctypes.byref(ck), _ptr(o), _ptr(ws),
                                ws.numel() if ws is not None else 0, ctypes.byref(sg) if sg is not None else None)
    _check(st, "gdn_chunk_prefill")
    if wait:
        _sync(stream)
    return ws


NOALLOC_SCRATCH_BYTES = 64 << 20


def chunk_prefill_noalloc(layer: Layer, q, k, v, a, b, cu_seqlens, start_pos, states, o, ckpt=None,
                          page_ids=None, stream=None, qk_stride=None, v_stride=None):
    """gdn_chunk_prefill_noalloc: chunk_prefill without a workspace (the library's fixed
    per-device scratch holds the chunk factors); nothing is allocated for the call."""
    vl = _Varlens(cu_seqlens, start_pos)
    qs = qk_stride if qk_stride is not None else layer.n_qk_heads * layer.head_dim
    vs = v_stride if v_stride is not None else layer.n_v_heads * layer.head_dim
    _check_prefill_operands(layer, cu_seqlens, start_pos, q, k, v, a, b, o, states, qs, vs)
    ck, keep = _ckpt_c(ckpt, page_ids)
    refs = _refs(states)
    st = _lib.gdn_chunk_prefill_noalloc(ctypes.byref(layer.c()), _stream(stream), ctypes.byref(vl.c), _ptr(q),
                                        _ptr(k), _ptr(v), qs, vs, _ptr(a), _ptr(b), refs, ctypes.byref(ck), _ptr(o))
    _check(st, "gdn_chunk_prefill_noalloc")


def prefill_factorize(layer: Layer, q, k, a, b, cu_seqlens, start_pos, block, workspace, stream=None,
                      qk_stride=None, staging=None):
    vl = _Varlens(cu_seqlens, start_pos)
    qs = qk_stride if qk_stride is not None else layer.n_qk_heads * layer.head_dim
    _check_prefill_operands(layer, cu_seqlens, start_pos, q, k, None, a, b, None,
                            [("zero", None, None)] * len(start_pos), qs, 0)
    sg, sg_keep, wait = _staging(prefill_staging_bytes(layer, cu_seqlens, start_pos, block), staging)
    st = _lib.gdn_prefill_factorize(ctypes.byref(layer.c()), _stream(stream), ctypes.byref(vl.c), _ptr(q),
                                    _ptr(k), qs, _ptr(a), _ptr(b), int(block), _ptr(workspace),
                                    workspace.numel(), ctypes.byref(sg) if sg is not None else None)
    _check(st, "gdn_prefill_factorize")
    if wait:
        _sync(stream)


def prefill_scan(layer: Layer, q, k, v, cu_seqlens, start_pos, states, o, workspace, ckpt=None, page_ids=None,
                 stream=None, qk_stride=None, v_stride=None, staging=None):
    vl = _Varlens(cu_seqlens, start_pos)
    ck, keep = _ckpt_c(ckpt, page_ids)
    refs = _refs(states)
    qs = qk_stride if qk_stride is not None else layer.n_qk_heads * layer.head_dim
    vs = v_stride if v_stride is not None else layer.n_v_heads * layer.head_dim
    _check_prefill_operands(layer, cu_seqlens, start_pos, q, k, v, None, None, o, states, qs, vs)
    block = ckpt.block if ckpt is not None else 0
    sg, sg_keep, wait = _staging(prefill_staging_bytes(layer, cu_seqlens, start_pos, block), staging)
    st = _lib.gdn_prefill_scan(ctypes.byref(layer.c()), _stream(stream), ctypes.byref(vl.c), _ptr(q), _ptr(k),
                               _ptr(v), qs, vs, refs, ctypes.byref(ck), _ptr(o), _ptr(workspace),
                               workspace.numel(), ctypes.byref(sg) if sg is not None else None)
    _check(st, "gdn_prefill_scan")
    if wait:
        _sync(stream)


def decode_step(layer: Layer, q, k, v, a, b, state_pool, slot_ids, o, status=None, stream=None):
    """One decode token per request (gdn_decode_step); slot -1 = padding."""
    n_req = int(slot_ids.numel())
    D, Hv, Hqk = layer.head_dim, layer.n_v_heads, layer.n_qk_heads
    _need(slot_ids.dtype == torch.int32, "slot_ids must be int32")
    _rows_ok(q, n_req, Hqk * D, layer.io_dtype, "q")
    _rows_ok(k, n_req, Hqk * D, layer.io_dtype, "k")
    _rows_ok(v, n_req, Hv * D, layer.io_dtype, "v")
    _rows_ok(a, n_req, Hv, torch.float32, "a")
    _rows_ok(b, n_req, Hv, torch.float32, "b")
    _rows_ok(o, n_req, Hv * D, torch.float32, "o")
    _need(state_pool.dtype == torch.float32 and state_pool.is_contiguous()
          and tuple(state_pool.shape[1:]) == (Hv, D, D), "state_pool must be fp32 [slots, Hv, d, d]")
    st = _lib.gdn_decode_step(ctypes.byref(layer.c()), _stream(stream), n_req, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                              _ptr(b), _ptr(state_pool), int(state_pool.shape[0]), _ptr(slot_ids), _ptr(o),
                              _ptr(status))
    _check(st, "gdn_decode_step")


def replay_flush(layer: Layer, state_pool, slot_ids, buf_k, buf_v, buf_a, buf_b, n_accepted, status=None,
                 stream=None):
    """ReplaySSM flush (gdn_replay_flush): fold the first n_accepted[r] logged rows of each
    request's slot into its state.  buf_*: [n_slots, buf_rows, heads, ...]."""
    n_req = int(slot_ids.numel())
    D, Hv, Hqk = layer.head_dim, layer.n_v_heads, layer.n_qk_heads
    n_slots = int(state_pool.shape[0])
    _need(slot_ids.dtype == torch.int32 and n_accepted.dtype == torch.int32, "int32 slot_ids / n_accepted")
    _need(n_accepted.numel() >= n_req, "n_accepted too short")
    _need(state_pool.dtype == torch.float32 and state_pool.is_contiguous()
          and tuple(state_pool.shape[1:]) == (Hv, D, D), "state_pool must be fp32 [slots, Hv, d, d]")
    rows = int(buf_k.shape[1])
    _rows_ok(buf_k, n_slots * rows, Hqk * D, layer.io_dtype, "buf_k")
    _rows_ok(buf_v, n_slots * rows, Hv * D, layer.io_dtype, "buf_v")
    _rows_ok(buf_a, n_slots * rows, Hv, torch.float32, "buf_a")
    _rows_ok(buf_b, n_slots * rows, Hv, torch.float32, "buf_b")
    st = _lib.gdn_replay_flush(ctypes.byref(layer.c()), _stream(stream), n_req, _ptr(state_pool),
                               int(state_pool.shape[0]), _ptr(slot_ids), _ptr(buf_k), _ptr(buf_v), _ptr(buf_a),
                               _ptr(buf_b), int(buf_k.shape[1]), _ptr(n_accepted), _ptr(status))
    _check(st, "gdn_replay_flush")


def decode_mixed(layer: Layer, q, k, v, a, b, state_pool, slot_ids, rows, o, status=None, stream=None,
                 qk_stride=None, v_stride=None):
    """Decode tokens of a mixed batch (gdn_decode_mixed): request r's token is row rows[r] of
    the packed token arrays q, k [n_rows, (row of qk_stride)], v, a, b [n_rows, Hv], o
    [n_rows, Hv, d] that the batch's prefill sequences share."""
    n_req = int(slot_ids.numel())
    D, Hv, Hqk = layer.head_dim, layer.n_v_heads, layer.n_qk_heads
    qs = qk_stride if qk_stride is not None else Hqk * D
    vs = v_stride if v_stride is not None else Hv * D
    n_rows = int(o.shape[0])
    _need(slot_ids.dtype == torch.int32 and rows.dtype == torch.int32 and rows.numel() >= n_req,
          "int32 slot_ids / rows")
    _need(state_pool.dtype == torch.float32 and state_pool.is_contiguous()
          and tuple(state_pool.shape[1:]) == (Hv, D, D), "state_pool must be fp32 [slots, Hv, d, d]")
    for t_, st_, heads, name in ((q, qs, Hqk, "q"), (k, qs, Hqk, "k"), (v, vs, Hv, "v")):
        _need(t_.dtype == layer.io_dtype, f"{name}: io dtype")
        span = t_.untyped_storage().nbytes() // t_.element_size() - t_.storage_offset()
        _need(n_rows == 0 or span >= (n_rows - 1) * st_ + heads * D, f"{name}: storage too small for {n_rows} rows")
    _rows_ok(a, n_rows, Hv, torch.float32, "a")
    _rows_ok(b, n_rows, Hv, torch.float32, "b")
    _rows_ok(o, n_rows, Hv * D, torch.float32, "o")
    st = _lib.gdn_decode_mixed(ctypes.byref(layer.c()), _stream(stream), n_req, n_rows, _ptr(q), _ptr(k), _ptr(v),
                               qs, vs, _ptr(a), _ptr(b), _ptr(state_pool), int(state_pool.shape[0]), _ptr(slot_ids),
                               _ptr(rows), _ptr(o), _ptr(status))
    _check(st, "gdn_decode_mixed")


def gates(layer: Layer, ba, A_log, dt_bias, a, b, stream=None):
    """Packed-core gates (gdn_gates): b = sigmoid(ba[:, :Hv]), a = exp(-exp(A_log) *
    softplus(ba[:, Hv:2Hv] + dt_bias)).  ba: [tokens, >= 2 Hv] io dtype (rows may be wider);
    A_log fp32 [Hv]; dt_bias io dtype [Hv]; a, b fp32 [tokens, Hv]."""
    Hv = layer.n_v_heads
    n = int(ba.shape[0])
    _need(ba.dim() == 2 and ba.shape[1] >= 2 * Hv and ba.stride(1) == 1, "ba: [tokens, >= 2 Hv], unit column stride")
    _need(ba.dtype == layer.io_dtype, "ba: io dtype")
    _need(A_log.dtype == torch.float32 and A_log.numel() == Hv, "A_log: fp32 [Hv]")
    _need(dt_bias.dtype == layer.io_dtype and dt_bias.numel() == Hv, "dt_bias: io dtype [Hv]")
    _rows_ok(a, n, Hv, torch.float32, "a")
    _rows_ok(b, n, Hv, torch.float32, "b")
    st = _lib.gdn_gates(ctypes.byref(layer.c()), _stream(stream), n, _ptr(ba), int(ba.stride(0)), _ptr(A_log),
                        _ptr(dt_bias), _ptr(a), _ptr(b))
    _check(st, "gdn_gates")


def gated_norm(layer: Layer, o, z, weight, out, eps=1e-6, stream=None):
    """Gated RMSNorm of the output rows (gdn_gated_norm): out = o * rsqrt(mean(o^2) + eps)
    * weight * silu(z) per (token, value head) row.  o fp32 [tokens, Hv, d]; z io dtype
    [tokens, >= Hv*d] rows (or [tokens, Hv, d]); weight io dtype [d]; out io dtype."""
    Hv, D = layer.n_v_heads, layer.head_dim
    n = int(o.shape[0])
    _rows_ok(o, n, Hv * D, torch.float32, "o")
    z2 = z.reshape(z.shape[0], -1) if z.dim() == 3 and z.is_contiguous() else z
    _need(z2.dim() == 2 and z2.shape[0] >= n and z2.shape[1] >= Hv * D and z2.stride(1) == 1, "z rows")
    _need(z2.dtype == layer.io_dtype, "z: io dtype")
    _need(weight.dtype == layer.io_dtype and weight.numel() == D and weight.is_contiguous(), "weight: io dtype [d]")
    _rows_ok(out, n, Hv * D, layer.io_dtype, "out")
    st = _lib.gdn_gated_norm(ctypes.byref(layer.c()), _stream(stream), n, _ptr(o), _ptr(z2), int(z2.stride(0)),
                             _ptr(weight), float(eps), _ptr(out))
    _check(st, "gdn_gated_norm")


def core_prefill_workspace_bytes(layer: Layer, cu_seqlens, start_pos, block: int) -> int:
    v = _Varlens(cu_seqlens, start_pos)
    return int(_lib.gdn_core_prefill_workspace_bytes(ctypes.byref(layer.c()), ctypes.byref(v.c), int(block)))


def core_prefill_staging_bytes(layer: Layer, cu_seqlens, start_pos, block: int) -> int:
    v = _Varlens(cu_seqlens, start_pos)
    return int(_lib.gdn_core_prefill_staging_bytes(ctypes.byref(layer.c()), ctypes.byref(v.c), int(block)))


def core_prefill(layer: Layer, qkvz, ba, conv_w, A_log, dt_bias, norm_weight, cu_seqlens, start_pos, tails, states,
                 out, ckpt=None, page_ids=None, eps=1e-6, workspace=None, stream=None, staging=None):
    """The packed core over a varlen batch (gdn_core_prefill): conv (+ q/k norm) over the
    q|k|v channels of the packed qkvz rows, gates from ba, the chunked prefill, and the
    gated norm with z from the packed rows.  qkvz [tokens, >= 2 Hqk d + 2 Hv d] and ba
    [tokens, >= 2 Hv] rows (io dtype, unit column stride); tails / states per sequence
    (kind, src, dst); out [tokens, Hv, d] io dtype."""
    vl = _Varlens(cu_seqlens, start_pos)
    rows = int(cu_seqlens[-1]) if len(cu_seqlens) else 0
    D, Hv = layer.head_dim, layer.n_v_heads
    C = layer.conv_channels
    qs = _strided_rows(qkvz, rows, C + Hv * D, layer.io_dtype, "qkvz")
    bs = _strided_rows(ba, rows, 2 * Hv, layer.io_dtype, "ba")
    _rows_ok(conv_w, C, layer.conv_width, layer.io_dtype, "conv_w")
    _need(A_log.dtype == torch.float32 and A_log.numel() == Hv, "A_log: fp32 [Hv]")
    _need(dt_bias.dtype == layer.io_dtype and dt_bias.numel() == Hv, "dt_bias: io dtype [Hv]")
    _need(norm_weight.dtype == layer.io_dtype and norm_weight.numel() == D, "norm_weight: io dtype [d]")
    _rows_ok(out, rows, Hv * D, layer.io_dtype, "out")
    _need(len(tails) == len(start_pos) and len(states) == len(start_pos), "one tail and one state per sequence")
    for kind, src, dst in states:
        if kind != "checkpoint":
            _state_ok(src, layer, "state src")
        _state_ok(dst, layer, "state dst")
    block = ckpt.block if ckpt is not None else 0
    ws = _workspace(core_prefill_workspace_bytes(layer, cu_seqlens, start_pos, block), qkvz.device, workspace)
    ck, keep = _ckpt_c(ckpt, page_ids)
    trefs, srefs = _refs(tails), _refs(states)
    sg, sg_keep, wait = _staging(core_prefill_staging_bytes(layer, cu_seqlens, start_pos, block), staging)
    st = _lib.gdn_core_prefill(ctypes.byref(layer.c()), _stream(stream), ctypes.byref(vl.c), _ptr(qkvz), qs,
                               _ptr(ba), bs, _ptr(conv_w), _ptr(A_log), _ptr(dt_bias), _ptr(norm_weight),
                               float(eps), trefs, srefs, ctypes.byref(ck), _ptr(out), _ptr(ws),
                               ws.numel() if ws is not None else 0, ctypes.byref(sg) if sg is not None else None)
    _check(st, "gdn_core_prefill")
    if wait:
        _sync(stream)
    return ws


def replay_forward(layer: Layer, state_pool, slot_ids, buf_k, buf_v, buf_a, buf_b, n_logged, n_new, q_new, o,
                   status=None, stream=None):
    """ReplaySSM verification outputs (gdn_replay_forward): o[r, i] = scale * S q_new[r, i]
    after log rows 0 .. n_logged[r] + i of request r's slot, from the slot's state, for
    i < n_new[r].  Neither the state nor the log is written.  buf_*: [n_slots, buf_rows,
    heads, ...]; q_new: [n_req, max_new, n_qk_heads, d]; o: [n_req, max_new, n_v_heads, d]
    fp32."""
    n_req = int(slot_ids.numel())
    D, Hv, Hqk = layer.head_dim, layer.n_v_heads, layer.n_qk_heads
    n_slots = int(state_pool.shape[0])
    _need(slot_ids.dtype == torch.int32 and n_logged.dtype == torch.int32 and n_new.dtype == torch.int32,
          "int32 slot_ids / n_logged / n_new")
    _need(n_logged.numel() >= n_req and n_new.numel() >= n_req, "n_logged / n_new too short")
    _need(state_pool.dtype == torch.float32 and state_pool.is_contiguous()
          and tuple(state_pool.shape[1:]) == (Hv, D, D), "state_pool must be fp32 [slots, Hv, d, d]")
    rows = int(buf_k.shape[1])
    _rows_ok(buf_k, n_slots * rows, Hqk * D, layer.io_dtype, "buf_k")
    _rows_ok(buf_v, n_slots * rows, Hv * D, layer.io_dtype, "buf_v")
    _rows_ok(buf_a, n_slots * rows, Hv, torch.float32, "buf_a")
    _rows_ok(buf_b, n_slots * rows, Hv, torch.float32, "buf_b")
    max_new = int(q_new.shape[1]) if q_new.dim() >= 2 else 0
    _need(q_new.shape[0] >= n_req, "q_new: one row block per request")
    _rows_ok(q_new, q_new.shape[0] * max_new, Hqk * D, layer.io_dtype, "q_new")
    _need(tuple(o.shape[:2]) == (q_new.shape[0], max_new), "o: [n_req, max_new, n_v_heads, d]")
    _rows_ok(o, o.shape[0] * max_new, Hv * D, torch.float32, "o")
    st = _lib.gdn_replay_forward(ctypes.byref(layer.c()), _stream(stream), n_req, _ptr(state_pool), n_slots,
                                 _ptr(slot_ids), _ptr(buf_k), _ptr(buf_v), _ptr(buf_a), _ptr(buf_b), rows,
                                 _ptr(n_logged), _ptr(n_new), _ptr(q_new), max_new, _ptr(o), _ptr(status))
    _check(st, "gdn_replay_forward")


def lib_handle():
    return _lib
