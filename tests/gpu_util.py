"""Helpers of the GPU parity tests: moving seeded bf16 inputs to the device, running the HIP path through the C ABI, choosing
sampled rows, and the tolerance check against the fp64 oracle.
"""
from __future__ import annotations

import json
import os

import numpy as np

# Float tolerances of the parity bar: O max |err| <= 1e-2, mean |err| <= 1e-3,
# LSE |err| / max(|LSE|, 1) <= 1e-3.
TOL_MAX_ABS = 1e-2
TOL_MEAN_ABS = 1e-3
TOL_LSE_REL = 1e-3


def to_device(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_to_f64(t) -> np.ndarray:
    import torch
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def run_gpu(q, k, v, pattern, scale, mode, block_q=256, schedule=True, layout="bhnd", repeat=1, granule=None,
            persistent=True):
    """Runs norms + attention on the GPU; returns a dict of host arrays.  With
    ``granule`` the block list is the frame-unaware one (masked kernel); with
    ``schedule`` the launch follows build_schedule's order, taken item by item
    by one workgroup per CU (``persistent``) or one workgroup per item."""
    import torch
    import block_sparse_video_frame_amd as bs
    B, H, N, D = q.shape
    if layout == "bhnd":
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
        out = None
    else:  # [B, N, H, D] storage, passed as strided [B, H, N, D] views
        qd, kd, vd = (to_device(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3) for x in (q, k, v))
        out = torch.empty(B, N, H, D, dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    host = bs.build_blocks_for(pattern, block_q) if granule is None else bs.build_blocks_granular(pattern, granule, block_q)
    blk = host.to_device(torch.device("cuda"), B, H, schedule=schedule, persistent=persistent)
    nm = bs.norms(qd, kd) if mode != bs.SOFTMAX_ONLINE else None
    hp = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    shift = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    o = lse = None
    for _ in range(repeat):
        o, lse = bs.attention(qd, kd, vd, blk, scale, mode, norms=nm, out=out, shift_out=shift, head_path=hp)
    torch.cuda.synchronize()
    res = {"o": bf16_to_f64(o), "lse": lse.cpu().numpy().astype(np.float64),
           "head_path": hp.cpu().numpy(), "shift": shift.cpu().numpy().astype(np.float64),
           "o_bytes": o.contiguous().view(torch.int16).cpu().numpy().tobytes(),
           "lse_bytes": lse.cpu().numpy().tobytes()}
    if nm is not None:
        res["norms"] = tuple(x.cpu().numpy().astype(np.float64) for x in nm)
    return res


def sample_rows(blocks_q_tiles, n_random, seq_len, seed=0):
    """Every tile's first and last row plus a seeded random sample."""
    rows = set()
    for s, r in blocks_q_tiles:
        rows.add(int(s)); rows.add(int(s + r - 1))
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, seq_len, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def errors(o, lse, o_ref, lse_ref):
    d = np.abs(o - o_ref)
    le = np.abs(lse - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    fro = np.linalg.norm((o - o_ref).ravel()) / max(np.linalg.norm(o_ref.ravel()), 1e-300)
    return {"max_abs": float(np.nanmax(d)) if np.isfinite(d).all() else float("inf"),
            "mean_abs": float(d.mean()) if np.isfinite(d).all() else float("inf"),
            "lse_rel": float(le.max()) if np.isfinite(le).all() else float("inf"),
            "rel_fro": float(fro)}


def within(e) -> bool:
    return e["max_abs"] <= TOL_MAX_ABS and e["mean_abs"] <= TOL_MEAN_ABS and e["lse_rel"] <= TOL_LSE_REL


def record(test: str, case: str, mode: int, e: dict) -> None:
    """Appends one parity measurement (errors against the oracle) as a JSON
    line to the file named by BSVF_PARITY_LOG, when that is set."""
    path = os.environ.get("BSVF_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": test, "case": case, "mode": int(mode), **e}) + "\n")
