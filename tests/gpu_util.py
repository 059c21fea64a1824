"""Helpers for the GPU parity tests (oracle vs HIP path through the C ABI)."""

import sys

import numpy as np

# fp16 outputs against the unrounded float64 oracle
REL_FRO_TOL = 1e-3
MAX_ABS_TOL = 5e-2


def announce(msg):
    """Name the case before a GPU step, so a crash can be traced to it."""
    sys.stdout.write(f"[case] {msg}\n")
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def fp16_errors(y_gpu, y64):
    y = np.asarray(y_gpu, dtype=np.float64)
    ref = np.asarray(y64, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    if ref.size == 0:
        return 0.0, 0.0, 0.0
    diff = y - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    return float(rel), float(np.max(np.abs(diff))), float(np.max(np.abs(ref)))


def assert_fp16_close(y_gpu, y64, what):
    y = np.asarray(y_gpu)
    assert np.all(np.isfinite(y.astype(np.float64))), f"{what}: non-finite output"
    rel, mx, ymax = fp16_errors(y_gpu, y64)
    msg = f"{what}: rel_fro={rel:.3e} max_abs={mx:.3e} max|y|={ymax:.3g}"
    print(msg)
    assert rel <= REL_FRO_TOL and mx <= MAX_ABS_TOL, msg
    return rel, mx
