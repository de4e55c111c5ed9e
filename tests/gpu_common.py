"""Shared helpers of the GPU tests: seeded inputs on the device, the oracle
run on the same inputs, and the error metric."""
import numpy as np
import pytest
import torch

from synth import make_inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_device(storage, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(storage)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(storage).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def device_inputs(B, H, N, d, dtype, seed):
    raw = make_inputs(B, H, N, d, dtype, seed)
    dev = {k: to_device(v[0], dtype) for k, v in raw.items()}
    exact = {k: v[1] for k, v in raw.items()}
    return dev, exact


def rel_err(gpu, ref, floor=0.0):
    """max|gpu - ref| / max|ref| (the denominator at least `floor`)."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), floor, 1e-30))


def log(msg):
    print(msg, flush=True)
