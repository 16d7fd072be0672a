"""Helpers shared by the GPU tests: upload seeded inputs, download results,
and the per-tensor tolerance check.

Tolerance (per output tensor, both must hold):
  bf16: max|gpu - ref| <= 1e-2 * max|ref| and ||gpu - ref||_F <= 5e-3 ||ref||_F
  fp32: max|gpu - ref| <= 1e-2 * max|ref| and ||gpu - ref||_F <= 1e-5 ||ref||_F
"""
import sys

import numpy as np
import torch

from rank_bottleneck_online_amd import synth

TOL_FROB = {"bf16": 5e-3, "f32": 1e-5}
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    """fp64 numpy array of dtype-representable values -> device tensor."""
    from rank_bottleneck_online_amd import binding
    return binding.upload(a, dtype)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite values"
    diff = gpu - ref
    maxabs = float(np.max(np.abs(diff))) / max(float(np.max(np.abs(ref))), 1e-300)
    frob = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    return maxabs, frob


def check(name, gpu, ref, dtype, report=None):
    maxabs, frob = errors(gpu, ref)
    say(f"    {name:10s} max-abs/max|ref| {maxabs:.3e}  rel-frob {frob:.3e}")
    if report is not None:
        report[name] = (maxabs, frob)
    assert maxabs <= 1e-2, f"{name}: max-abs error {maxabs:.3e} > 1e-2 max|ref|"
    assert frob <= TOL_FROB[dtype], f"{name}: relative Frobenius error {frob:.3e} > {TOL_FROB[dtype]}"
