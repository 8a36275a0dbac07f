"""attn_fwd_noalloc (the attention entry point that allocates nothing: its
persistent launch's counters live in a fixed device array of the library)
against attn_fwd with a caller-given workspace, through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input, fewer
heads, another head size and fewer queues, so the second starts from the
array the first left behind.  Each must give attn_fwd's bits exactly (same
kernels, same per-item arithmetic; only where the counters live differs) and
meet the parity bar against the fp64 oracle on every row.
"""
import ctypes

import numpy as np
import pytest

from oracle import attention as OA
from synth import Pattern, random_qkv

pytestmark = pytest.mark.gpu

import block_sparse_video_frame_amd as bs
from gpu_util import bf16_to_f64, errors, to_device, within


def _noalloc(q, k, v, blocks, scale, mode, nm, o, lse, hp):
    """attn_fwd_noalloc called directly through ctypes (no binding logic)."""
    import torch
    B, H, N, D = q.shape
    st = (ctypes.c_int64 * 12)(*([int(x) for x in q.stride()[:3]] * 4))
    cb = blocks.c_struct()
    cb.work_ctr = None
    qn, kg, hm = (x.data_ptr() for x in nm) if nm is not None else (None, None, None)
    return bs.lib().attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), None,
                                     B, H, N, D, st, ctypes.c_float(scale), ctypes.byref(cb), qn, kg, hm, mode,
                                     hp.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_attn_fwd_on_two_calls():
    import torch
    dev = torch.device("cuda")
    cases = [
        # (pattern, batch, heads, D, mode, num_xcd, seed): the second is smaller in every way
        (Pattern(6, 272, 1, 1, (0,)), 2, 4, 128, bs.SOFTMAX_BOUND, 8, 11),
        (Pattern(3, 144, 1, 0), 1, 2, 64, bs.SOFTMAX_ONLINE, 4, 12),
    ]
    for pattern, B, H, D, mode, nx, seed in cases:
        N = pattern.seq_len
        scale = float(np.float32(1.0 / np.sqrt(D)))
        qh, kh, vh = random_qkv(B, H, N, D, seed=seed)
        q, k, v = to_device(qh), to_device(kh), to_device(vh)
        blocks = bs.build_blocks_for(pattern, 256).to_device(dev, B, H, num_xcd=nx)
        nm = bs.norms(q, k) if mode != bs.SOFTMAX_ONLINE else None
        o_ref, lse_ref = bs.attention(q, k, v, blocks, scale, mode, norms=nm)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        hp = torch.full((B, H), -1, dtype=torch.int32, device=dev)
        assert _noalloc(q, k, v, blocks, scale, mode, nm, o, lse, hp) == 0, bs.lib().attn_last_error()
        torch.cuda.synchronize()
        print(f"noalloc case B{B} H{H} N{N} D{D} mode {mode} num_xcd {nx}", flush=True)
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        O, L = OA.attention(qh, kh, vh, pattern, scale)
        e = errors(bf16_to_f64(o), lse.cpu().numpy().astype(np.float64), O, L)
        assert within(e), e
        # the caller's workspace is left zero by its call, and was not touched by the other
        assert not blocks.work_ctr.any()
        if mode != bs.SOFTMAX_ONLINE:
            assert (hp.cpu().numpy() == bs.PATH_BOUND).all()
