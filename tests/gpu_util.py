"""Helpers of the GPU parity tests: move seeded inputs to the device and
compare against the oracle with the tolerances of the acceptance bar."""
import os
import sys

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-4}

# lines printed in the run's summary by tests/conftest.py (near-tie counts,
# elements that needed a storage-rounding allowance)
REPORT = []


def report(line):
    REPORT.append(line)
    log(line)


def device():
    import torch
    import block_diffusion_draft_ctx_amd as dfl
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    dfl.lib()  # raises if the HIP library is missing: no fallback path exists
    return torch.device("cuda:0")


def up(a, kind):
    import torch
    dev = device()
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(dev)
    if kind == "i32":
        return torch.from_numpy(a.astype(np.int32)).to(dev)
    raise ValueError(kind)


def down(t):
    """Device tensor -> numpy float64 (or int64 for integer tensors)."""
    import torch
    if t.dtype in (torch.int32, torch.int64):
        return t.cpu().numpy().astype(np.int64)
    return t.float().cpu().numpy().astype(np.float64)


def bits(t):
    """Raw storage bits of a bf16 / fp32 device tensor as unsigned ints."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.abs(gpu - ref).max() / rms)


def rel_err_chained(gpu, ref, dtype, what=None):
    """rel_err after allowing one unit in the last place of the stored value
    (bf16: 2^-7 |ref|): for results that pass two storage roundings in a chain
    (the K projection is stored, then the K epilogue's output), where the
    kernel's and the oracle's values may each land on the other side of a
    rounding boundary once.  With ``what`` the number of elements that are
    over the plain bar without the allowance is reported."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -23
    if what is not None:
        plain = np.abs(gpu - ref) / rms
        over = int((plain > TOL[dtype]).sum())
        report(f"{what}: plain max-abs/RMS {plain.max():.3g}; {over} of {plain.size} elements "
               f"over {TOL[dtype]} without the one-unit allowance")
    return float(np.maximum(np.abs(gpu - ref) - ulp * np.abs(ref), 0.0).max() / rms)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()
