"""Helpers shared by the tests: library build/load, uploads, parity metric."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lb.h")

# Parity bar for fp16 outputs with fp32 accumulation (relative L2 and
# max-abs relative to the reference rms), against the float64 oracle.
REL_L2 = 1e-3
MAX_ABS_OVER_RMS = 1e-2


def ensure_built():
    import binary_rank_gemv_littlebitlinear_amd as lbm
    if not os.path.exists(lbm.LIB_PATH):
        from binary_rank_gemv_littlebitlinear_amd import build
        build.build()
    return lbm


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def parity_stats(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = y - ref
    nref = np.linalg.norm(ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    mx = float(np.max(np.abs(d))) if d.size else 0.0
    return rel, mx, rms


def assert_parity(y, ref, what=""):
    rel, mx, rms = parity_stats(y, ref)
    assert np.isfinite(np.asarray(y, np.float64)).all(), f"{what}: non-finite output"
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_OVER_RMS * rms, f"{what}: max abs {mx:.3e} > 1e-2 * rms {rms:.3e}"
    return rel, mx, rms


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test needs a visible MI355X"
    return torch


def to_dev(x_np):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(x_np)).to("cuda")


def gpu_forward(layer, x_np, b):
    """Run lb_forward on a host fp16 array, return the fp16 result on host."""
    torch = torch_dev()
    x = to_dev(x_np.astype(np.float16))
    y = torch.empty((x_np.shape[0], b), dtype=torch.float16, device="cuda")
    layer.forward(x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()
