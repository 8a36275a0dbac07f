"""Frame-aligned block-sparse video attention (forward) for AMD MI355X (gfx950).

A thin ctypes binding over ``libbsvf.so``: every step of the computation runs
in the library (host C++ for the integer block lists, HIP kernels for norms
and attention).  PyTorch is used only for device memory and the current
stream.  The library must be built first (``python -m
block_sparse_video_frame_amd.build``); without it every call raises.

    blocks = build_blocks(num_frames=13, tokens_per_frame=3600, win_before=1,
                          win_after=1, global_frames=(0,), block_q=256)
    dev = blocks.to_device(torch.device("cuda"), batch=1, heads=8)
    qn, kg, hm = norms(q, k)
    o, lse = attention(q, k, v, dev, mode=SOFTMAX_BOUND, norms=(qn, kg, hm))
"""
from __future__ import annotations

import ctypes
from typing import Optional
import math
import os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "SOFTMAX_ONLINE", "SOFTMAX_BOUND", "SOFTMAX_BOUND_FORCED", "SOFTMAX_BOUND_TILE", "SOFTMAX_BOUND_EXACT",
    "SOFTMAX_BOUND_CHECKED", "PATH_ONLINE", "PATH_BOUND",
    "MAX_BLOCK_Q", "ELIGIBLE_NATS", "PRESCALE_NATS", "CHECK_NATS", "CHECK_LOG2_L", "CHECK_SHIFT_NATS", "AttnError", "lib", "library_path", "abi_version",
    "Blocks", "DeviceBlocks", "build_blocks", "build_blocks_granular", "build_schedule", "norms", "qk_prep",
    "attention",
]

SOFTMAX_ONLINE, SOFTMAX_BOUND, SOFTMAX_BOUND_FORCED, SOFTMAX_BOUND_TILE, SOFTMAX_BOUND_EXACT = 0, 1, 2, 3, 4
SOFTMAX_BOUND_CHECKED = 5
PATH_ONLINE, PATH_BOUND = 0, 1
MAX_BLOCK_Q = 256
ELIGIBLE_NATS = 60.0
PRESCALE_NATS = 40.0
CHECK_NATS = 256.0
CHECK_LOG2_L = -100.0
CHECK_SHIFT_NATS = 40.0
ABI_VERSION = 5

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    """The in-tree build, or the file named by ``BSVF_LIBRARY``."""
    return os.environ.get("BSVF_LIBRARY") or os.path.join(_HERE, "libbsvf.so")


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _Pattern(ctypes.Structure):
    _fields_ = [
        ("num_frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
        ("win_before", ctypes.c_int32), ("win_after", ctypes.c_int32),
        ("num_global", ctypes.c_int32), ("global_frames", ctypes.POINTER(ctypes.c_int32)),
    ]


class _Blocks(ctypes.Structure):
    _fields_ = [
        ("q_tiles", ctypes.c_void_p), ("kv_ptr", ctypes.c_void_p), ("kv_iv", ctypes.c_void_p),
        ("n_qt", ctypes.c_int32), ("nnz", ctypes.c_int32), ("block_q", ctypes.c_int32),
        ("work_order", ctypes.c_void_p), ("n_work", ctypes.c_int32),
        ("num_xcd", ctypes.c_int32), ("work_ctr", ctypes.c_void_p),
    ]


_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_VP = ctypes.c_void_p


def lib():
    """Loads ``libbsvf.so`` (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_video_frame_amd.build`")
    L = ctypes.CDLL(path)
    L.attn_abi_version.restype = ctypes.c_int
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_status_str.argtypes = [ctypes.c_int]
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_build_blocks.restype = ctypes.c_int
    L.attn_build_blocks.argtypes = [ctypes.POINTER(_Pattern), ctypes.c_int32, _I32P, _I32P, _I32P,
                                    _I64P, _I32P, _I32P]
    L.attn_build_blocks_granular.restype = ctypes.c_int
    L.attn_build_blocks_granular.argtypes = [ctypes.POINTER(_Pattern), ctypes.c_int32, ctypes.c_int32, _I32P,
                                             _I32P, _I32P, _I32P, _I64P, _I32P, _I32P]
    L.attn_build_schedule.restype = ctypes.c_int
    L.attn_build_schedule.argtypes = [_I32P, _I32P, _I32P, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _I32P, _I32P]
    L.attn_norms.restype = ctypes.c_int
    L.attn_norms.argtypes = [_VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                             _I64P, _I64P, _VP, _VP, _VP, _VP]
    L.attn_fwd_masked.restype = ctypes.c_int
    L.attn_fwd_masked.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, _I64P, ctypes.c_float,
                                  ctypes.POINTER(_Blocks), _VP, ctypes.POINTER(_Pattern), _VP, _VP, _VP,
                                  ctypes.c_int32, _VP, _VP]
    L.attn_fwd.restype = ctypes.c_int
    L.attn_fwd.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int32, ctypes.c_int32,
                           ctypes.c_int32, ctypes.c_int32, _I64P, ctypes.c_float,
                           ctypes.POINTER(_Blocks), _VP, _VP, _VP, ctypes.c_int32, _VP, _VP]
    L.attn_fwd_noalloc.restype = ctypes.c_int
    L.attn_fwd_noalloc.argtypes = L.attn_fwd.argtypes
    L.attn_qk_prep.restype = ctypes.c_int
    L.attn_qk_prep.argtypes = [_VP, _VP, _VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_int32, _I64P, _VP, _VP, ctypes.c_float, _VP, _VP, _VP, _VP, _VP, _VP]
    if L.attn_abi_version() != ABI_VERSION:
        raise RuntimeError("libbsvf.so ABI version mismatch; rebuild it")
    _LIB = L
    return L


def abi_version() -> int:
    return lib().attn_abi_version()


def _check(status: int):
    if status != 0:
        L = lib()
        raise AttnError(status, L.attn_last_error().decode() or L.attn_status_str(status).decode())


def _i32(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


@dataclass
class Blocks:
    """Host block list (canonical form) of one pattern and tile size."""
    q_tiles: np.ndarray   # [n_qt, 2] int32 (first token, rows)
    kv_ptr: np.ndarray    # [n_qt + 1] int32
    kv_iv: np.ndarray     # [nnz, 2] int32 (first key, length)
    useful_pairs: int     # unmasked (query, key) pairs of one head
    block_q: int
    seq_len: int
    kv_flag: Optional[np.ndarray] = None  # [nnz] int32, frame-unaware layout only
    pattern: object = None                # the pattern of a frame-unaware layout

    @property
    def n_qt(self) -> int:
        return int(self.q_tiles.shape[0])

    @property
    def nnz(self) -> int:
        return int(self.kv_iv.shape[0])

    def to_device(self, device, batch: int, heads: int, schedule: bool = True, group: int = 0,
                  num_xcd: int = 8, persistent: bool = True) -> "DeviceBlocks":
        """Device copy of the list.  With ``schedule`` the launch order comes from
        :func:`build_schedule`; with ``persistent`` as well, attention runs
        one workgroup per CU taking items from the order's per-die queues,
        each item on its own softmax path (see ``attn_blocks_t.work_ctr``);
        otherwise one workgroup per item."""
        import torch
        order = build_schedule(self, batch, heads, group, num_xcd) if schedule else None

        def up(x):
            return torch.from_numpy(np.ascontiguousarray(x)).to(device)

        persistent = persistent and order is not None
        # slot counters of the persistent launch: zero once, left zero by every call
        ctr = torch.zeros(num_xcd + 1, dtype=torch.int32, device=device) if persistent else None
        return DeviceBlocks(self, up(self.q_tiles), up(self.kv_ptr), up(self.kv_iv),
                            up(order) if order is not None else None, batch, heads,
                            up(self.kv_flag) if self.kv_flag is not None else None,
                            num_xcd, ctr)


@dataclass
class DeviceBlocks:
    host: Blocks
    q_tiles: object
    kv_ptr: object
    kv_iv: object
    work_order: object
    batch: int
    heads: int
    kv_flag: object = None
    num_xcd: int = 8
    # The persistent launch's slot counters (attn_blocks_t.work_ctr) or None.
    # Calls that use the same counters must not overlap; order_on() keeps
    # them ordered across streams.
    work_ctr: object = None
    _last_stream: object = None

    def order_on(self, stream) -> None:
        """Called before each launch that uses ``work_ctr`` on ``stream``: when
        the previous such launch went to another stream, ``stream`` first waits
        for everything queued on that stream so far (``wait_stream`` records an
        event there), so two calls never hand out items from the same counters
        at once.  On a single stream this does nothing.  Not itself
        thread-safe: threads sharing one DeviceBlocks must serialise calls."""
        if self.work_ctr is None:
            return
        last = self._last_stream
        if last is not None and last != stream:
            stream.wait_stream(last)
        self._last_stream = stream

    def c_struct(self) -> _Blocks:
        return _Blocks(self.q_tiles.data_ptr(), self.kv_ptr.data_ptr(), self.kv_iv.data_ptr(),
                       self.host.n_qt, self.host.nnz, self.host.block_q,
                       self.work_order.data_ptr() if self.work_order is not None else None,
                       int(self.work_order.numel()) if self.work_order is not None else 0,
                       self.num_xcd, self.work_ctr.data_ptr() if self.work_ctr is not None else None)


def build_blocks(num_frames: int, tokens_per_frame: int, win_before: int, win_after: int,
                 global_frames=(), block_q: int = MAX_BLOCK_Q) -> Blocks:
    """Block list of a frame-window pattern (``attn_build_blocks``)."""
    L = lib()
    g = np.ascontiguousarray(np.asarray(global_frames, dtype=np.int32).reshape(-1))
    p = _Pattern(num_frames, tokens_per_frame, win_before, win_after, len(g),
                 _i32(g) if len(g) else None)
    n_qt = ctypes.c_int32(0)
    nnz = ctypes.c_int32(0)
    useful = ctypes.c_int64(0)
    _check(L.attn_build_blocks(ctypes.byref(p), block_q, None, None, None, ctypes.byref(useful),
                               ctypes.byref(n_qt), ctypes.byref(nnz)))
    qt = np.zeros((n_qt.value, 2), np.int32)
    kp = np.zeros(n_qt.value + 1, np.int32)
    kv = np.zeros((nnz.value, 2), np.int32)
    _check(L.attn_build_blocks(ctypes.byref(p), block_q, _i32(qt), _i32(kp), _i32(kv),
                               ctypes.byref(useful), ctypes.byref(n_qt), ctypes.byref(nnz)))
    return Blocks(qt, kp, kv, int(useful.value), block_q, num_frames * tokens_per_frame)


def build_blocks_granular(pattern, granule: int = 128, block_q: int = MAX_BLOCK_Q) -> Blocks:
    """Block list of the frame-unaware layout (``attn_build_blocks_granular``):
    fixed tiles and key blocks that ignore frame edges, with ``kv_flag`` marking
    the partly masked runs."""
    L = lib()
    g = np.ascontiguousarray(np.asarray(tuple(pattern.global_frames), dtype=np.int32).reshape(-1))
    p = _Pattern(pattern.num_frames, pattern.tokens_per_frame, pattern.win_before, pattern.win_after,
                 len(g), _i32(g) if len(g) else None)
    n_qt = ctypes.c_int32(0)
    nnz = ctypes.c_int32(0)
    useful = ctypes.c_int64(0)
    _check(L.attn_build_blocks_granular(ctypes.byref(p), granule, block_q, None, None, None, None,
                                        ctypes.byref(useful), ctypes.byref(n_qt), ctypes.byref(nnz)))
    qt = np.zeros((n_qt.value, 2), np.int32)
    kp = np.zeros(n_qt.value + 1, np.int32)
    kv = np.zeros((nnz.value, 2), np.int32)
    fl = np.zeros(nnz.value, np.int32)
    _check(L.attn_build_blocks_granular(ctypes.byref(p), granule, block_q, _i32(qt), _i32(kp), _i32(kv), _i32(fl),
                                        ctypes.byref(useful), ctypes.byref(n_qt), ctypes.byref(nnz)))
    return Blocks(qt, kp, kv, int(useful.value), block_q, pattern.num_frames * pattern.tokens_per_frame,
                  kv_flag=fl, pattern=pattern)


def build_blocks_for(pattern, block_q: int = MAX_BLOCK_Q) -> Blocks:
    """``build_blocks`` from any object with the pattern's five attributes."""
    return build_blocks(pattern.num_frames, pattern.tokens_per_frame, pattern.win_before,
                        pattern.win_after, tuple(pattern.global_frames), block_q)


def build_schedule(blocks: Blocks, batch: int, heads: int, group: int = 0, num_xcd: int = 8) -> np.ndarray:
    """Launch order of the attention workgroups (``attn_build_schedule``)."""
    L = lib()
    n = ctypes.c_int32(0)
    _check(L.attn_build_schedule(_i32(blocks.q_tiles), _i32(blocks.kv_ptr), _i32(blocks.kv_iv),
                                 blocks.n_qt, batch, heads, group, num_xcd, None, ctypes.byref(n)))
    out = np.zeros(n.value, np.int32)
    _check(L.attn_build_schedule(_i32(blocks.q_tiles), _i32(blocks.kv_ptr), _i32(blocks.kv_iv),
                                 blocks.n_qt, batch, heads, group, num_xcd, _i32(out), ctypes.byref(n)))
    return out


def _strides(t):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, N, D] tensor with unit stride in D")
    return [int(t.stride(0)), int(t.stride(1)), int(t.stride(2))]


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_qkv(*ts):
    import torch
    for t in ts:
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError("q, k, v must be bfloat16 CUDA (HIP) tensors")


def _same_shape(shape, **ts):
    """The library sees pointers and strides only: a tensor smaller than the
    stated sizes would be read or written past its end, so shapes are checked
    here, before anything else."""
    for name, t in ts.items():
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _check_aux(device, specs):
    """Auxiliary tensors: (name, tensor or None, shape, dtype), each contiguous
    on ``device``."""
    for name, t, shape, dtype in specs:
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != device:
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {list(shape)} on {device}")


def _norm_specs(B, H, N, nm, prefix=""):
    import torch
    if nm is None:
        return []
    if len(nm) != 3:
        raise ValueError("norms must be the (q_norm, k_gmax, head_max) triple")
    return [(prefix + "q_norm", nm[0], (B, H, N), torch.float32),
            (prefix + "k_gmax", nm[1], (B, H, N // 16), torch.float32),
            (prefix + "head_max", nm[2], (B, H, 2), torch.float32)]


def _norms(q, k, out=None):
    """``(q_norm [B,H,N], k_gmax [B,H,N/16], head_max [B,H,2])`` fp32 (``attn_norms``)."""
    import torch
    if q.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor with unit stride in D")
    B, H, N, D = q.shape
    _same_shape(q.shape, k=k)
    _check_qkv(q, k)
    _check_aux(q.device, _norm_specs(B, H, N, out, "out."))
    if out is None:
        out = (torch.empty(B, H, N, dtype=torch.float32, device=q.device),
               torch.empty(B, H, N // 16, dtype=torch.float32, device=q.device),
               torch.empty(B, H, 2, dtype=torch.float32, device=q.device))
    qs = (ctypes.c_int64 * 3)(*_strides(q))
    ks = (ctypes.c_int64 * 3)(*_strides(k))
    _check(lib().attn_norms(q.data_ptr(), k.data_ptr(), B, H, N, D, qs, ks, out[0].data_ptr(),
                            out[1].data_ptr(), out[2].data_ptr(), _stream(q)))
    return out


norms = _norms


def qk_prep(q_in, k_in, q_gamma, k_gamma, rope_cos, rope_sin, eps: float = 1e-6, q_out=None, k_out=None,
            norms: bool = True, norms_out=None):
    """The Q/K producer (``attn_qk_prep``): per-head RMS norm with weights
    ``q_gamma``/``k_gamma`` (fp32 ``[D]``), rotary embedding of adjacent pairs by
    the fp32 ``[N, D/2]`` tables, bf16 out.  Returns ``(q_out, k_out, norms)``
    where ``norms`` is the ``(q_norm, k_gmax, head_max)`` triple of the rows
    written (as :func:`norms` would give), or None when ``norms`` is False.
    Outputs default to new contiguous ``[B, H, N, D]`` tensors; passing
    ``q_out=q_in`` (same strides) works in place."""
    import torch
    if q_in.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor with unit stride in D")
    B, H, N, D = q_in.shape
    _same_shape(q_in.shape, k_in=k_in, q_out=q_out, k_out=k_out)
    _check_qkv(q_in, k_in)
    if norms:
        _check_aux(q_in.device, _norm_specs(B, H, N, norms_out, "norms_out."))
    for name, t, shape in (("q_gamma", q_gamma, (D,)), ("k_gamma", k_gamma, (D,)),
                           ("rope_cos", rope_cos, (N, D // 2)), ("rope_sin", rope_sin, (N, D // 2))):
        if t.dtype != torch.float32 or t.device != q_in.device or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on the inputs' device")
    if q_out is None:
        q_out = torch.empty(B, H, N, D, dtype=torch.bfloat16, device=q_in.device)
    if k_out is None:
        k_out = torch.empty(B, H, N, D, dtype=torch.bfloat16, device=q_in.device)
    _check_qkv(q_out, k_out)
    nm = None
    if norms:
        nm = norms_out if norms_out is not None else (
            torch.empty(B, H, N, dtype=torch.float32, device=q_in.device),
            torch.empty(B, H, N // 16, dtype=torch.float32, device=q_in.device),
            torch.empty(B, H, 2, dtype=torch.float32, device=q_in.device))
    st = (ctypes.c_int64 * 12)(*(_strides(q_in) + _strides(k_in) + _strides(q_out) + _strides(k_out)))
    qn, kg, hm = (x.data_ptr() for x in nm) if nm is not None else (None, None, None)
    _check(lib().attn_qk_prep(q_in.data_ptr(), k_in.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), B, H, N, D,
                              st, q_gamma.data_ptr(), k_gamma.data_ptr(), ctypes.c_float(eps),
                              rope_cos.data_ptr(), rope_sin.data_ptr(), qn, kg, hm, _stream(q_in)))
    return q_out, k_out, nm


def attention(q, k, v, blocks: DeviceBlocks, scale: float | None = None, mode: int = SOFTMAX_BOUND,
              norms=None, out=None, lse=None, shift_out=None, head_path=None, noalloc: bool = False):
    """Block-sparse attention forward (``attn_fwd``; ``attn_fwd_masked`` for
    blocks of :func:`build_blocks_granular`); returns ``(out, lse)``.

    ``norms``: the ``(q_norm, k_gmax, head_max)`` triple from :func:`norms`
    (computed here when the mode needs it and none is given).
    ``noalloc``: call ``attn_fwd_noalloc`` instead, whose persistent launch
    keeps its counters in the library (the block list needs a launch order;
    its own counters are not used).  Pass ``out``, ``lse`` and ``norms`` to
    allocate nothing here either.
    """
    import torch
    if q.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor with unit stride in D")
    B, H, N, D = q.shape
    _same_shape(q.shape, k=k, v=v, out=out)
    if blocks.host.seq_len != N:
        raise ValueError(f"the block list is for {blocks.host.seq_len} tokens, the tensors have {N}")
    if blocks.work_order is not None and (blocks.batch, blocks.heads) != (B, H):
        raise ValueError(f"the block list's launch order is for batch {blocks.batch} x {blocks.heads} heads, "
                         f"the tensors have {B} x {H}")
    _check_qkv(q, k, v)
    if blocks.q_tiles.device != q.device:
        raise ValueError("the block list lives on another device")
    _check_aux(q.device, _norm_specs(B, H, N, norms) + [
        ("lse", lse, (B, H, N), torch.float32), ("shift_out", shift_out, (B, H, N), torch.float32),
        ("head_path", head_path, (B, H), torch.int32)])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nm = norms
    if mode != SOFTMAX_ONLINE and nm is None:
        nm = _norms(q, k)
    if out is None:
        out = torch.empty(B, H, N, D, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    st = (ctypes.c_int64 * 12)(*(_strides(q) + _strides(k) + _strides(v) + _strides(out)))
    cb = blocks.c_struct()
    if noalloc:
        if blocks.kv_flag is not None or blocks.work_order is None:
            raise ValueError("noalloc needs a frame-aligned block list with a launch order")
        cb.work_ctr = None
    else:
        blocks.order_on(torch.cuda.current_stream(q.device))
    qn, kg, hm = (x.data_ptr() for x in nm) if nm is not None else (None, None, None)
    so = shift_out.data_ptr() if shift_out is not None else None
    hp = head_path.data_ptr() if head_path is not None else None
    if noalloc:
        _check(lib().attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                      so, B, H, N, D, st, ctypes.c_float(scale), ctypes.byref(cb), qn, kg, hm,
                                      mode, hp, _stream(q)))
    elif blocks.kv_flag is None:
        _check(lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), so,
                              B, H, N, D, st, ctypes.c_float(scale), ctypes.byref(cb), qn, kg, hm, mode,
                              hp, _stream(q)))
    else:
        pat = blocks.host.pattern
        g = np.ascontiguousarray(np.asarray(tuple(pat.global_frames), dtype=np.int32).reshape(-1))
        p = _Pattern(pat.num_frames, pat.tokens_per_frame, pat.win_before, pat.win_after, len(g),
                     _i32(g) if len(g) else None)
        _check(lib().attn_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                     so, B, H, N, D, st, ctypes.c_float(scale), ctypes.byref(cb),
                                     blocks.kv_flag.data_ptr(), ctypes.byref(p), qn, kg, hm, mode, hp,
                                     _stream(q)))
    return out, lse
