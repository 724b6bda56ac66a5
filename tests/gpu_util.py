"""Helpers for the GPU parity tests (device upload, tolerance checks)."""
import sys

import numpy as np
import torch

OUT_TOL = 2e-2      # max|out - oracle| <= OUT_TOL * RMS(oracle out)
W_TOL = 1e-5        # |topk_w - oracle| (binary32 vs binary64 weights)
GATE_TOL = 1e-5     # |s - oracle|


def announce(msg: str):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(a, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def rel_err(out_gpu: np.ndarray, ref: np.ndarray) -> float:
    """max|gpu - ref| / RMS(ref)."""
    err = np.abs(out_gpu.astype(np.float64) - ref).max()
    rms = np.sqrt((ref ** 2).mean())
    return float(err / rms)


def assert_out(out_gpu, ref, tol=OUT_TOL):
    r = rel_err(out_gpu, ref)
    assert r <= tol, f"max|err|/rms = {r:.3e} > {tol}"
    return r
