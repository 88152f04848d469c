"""Helpers shared by the GPU tests: moving seeded inputs to the device, running the
HIP library through its C ABI, and the per-(b,h,frame) error metric."""
import sys

import numpy as np
import torch

import workloads as W
from frame_wise_delta_vda_amd import vda as binding

# Parity bar: max over (b,h,frame) of ||O_gpu - O_ref||_F / ||O_ref||_F.  FP8 inputs are
# converted exactly to bfloat16 and take the bfloat16 path, so they share its bar.
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 1e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_device(w, arrays, device="cuda"):
    out = {}
    for key, arr in arrays.items():
        if w.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
        elif w.dtype == "fp8":
            t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8))  # e4m3 codes
        else:
            t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
        out[key] = t.to(device)
    return out


def out_to_float64(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(w, dev, plan=None, out=None):
    """Run the whole forward pass; returns (out tensor, plan)."""
    own = plan is None
    if own:
        plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    if out is None:
        out = torch.empty(w.shapes()["out"], device=dev["q"].device,
                          dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16)
    plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out)
    torch.cuda.synchronize()
    return out, plan


def frame_errors(gpu, ref):
    """Relative Frobenius error per leading index tuple (b,h,f) of [.., n, dv] arrays."""
    diff = np.sqrt(np.sum((gpu - ref) ** 2, axis=(-2, -1)))
    nrm = np.sqrt(np.sum(ref ** 2, axis=(-2, -1)))
    return diff / np.maximum(nrm, 1e-300)
