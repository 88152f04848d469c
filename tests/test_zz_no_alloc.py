"""vda_forward_noalloc (include/vda.h): the forward pass with no plan and no device allocation.
Each call is checked against vda_forward on a plan of the same shape running the serial scan (the
same kernels on the same inputs: bit for bit) and against the oracle (max per-(b,h,frame) relative Frobenius error
<= 1e-4 for float32, 1e-2 for bfloat16 and FP8), on calls in a row whose inputs shrink, so the
fixed scratch holds a larger problem's data when a smaller one starts."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from vda_gpu_util import TOL, frame_errors, out_to_float64, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

# in call order, each smaller than the one before: three heads of the 768p shape (53.4 MB of
# the 64 MiB scratch), a ragged bfloat16 problem with no text, the tiny float32 workload
CALLS = [
    W.WORKLOADS[3].replace(name="noalloc_768p_3_heads", H=3, seed=301),
    W.WORKLOADS[2].replace(name="noalloc_bf16_small", H=2, F=5, n=300, T=0, d=64, dv=128, seed=302),
    W.WORKLOADS[1].replace(name="noalloc_tiny_fp32", seed=303),
]


def _workspace_bytes(w):
    frames = w.B * w.H * w.F
    x = frames * w.d * w.dv * (4 if w.dtype == "f32" else 2)
    return (w.B * w.H * (w.F + 1) * (w.d * w.d + w.d * w.dv)) * 4 + 2 * x


def _noalloc(w, dev, out):
    binding.vda_forward_noalloc(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype, dev["q"], dev["k"],
                                dev["v"], dev["text_k"], dev["text_v"], out)


def _free_bytes():
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def test_noalloc_matches_plan_and_oracle_on_calls_in_a_row():
    for w in CALLS:
        assert _workspace_bytes(w) <= binding.VDA_NOALLOC_SCRATCH_BYTES
        say(f"[gpu] noalloc {w.name}: B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T} "
            f"workspace {_workspace_bytes(w) / 1e6:.1f} MB")
        arrays = W.full_storage(w)
        dev = to_device(w, arrays)
        if w.T == 0:
            dev["text_k"] = dev["text_v"] = None
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        got = torch.full(w.shapes()["out"], float("nan"), dtype=dt, device="cuda")
        torch.cuda.synchronize()
        _noalloc(w, dev, got)
        torch.cuda.synchronize()
        # the entry point runs the serial scan: compare with a plan that runs it too
        plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
        if w.dtype != "f32":
            plan.set_scan_chunk(0)
        ref_plan, _ = run_gpu(w, dev, plan=plan)
        plan.close()
        assert torch.equal(got.view(torch.uint8), ref_plan.view(torch.uint8)), w.name
        g = out_to_float64(got)
        worst = 0.0
        for b in range(w.B):
            for h in range(w.H):
                x = {k: W.storage_to_float64(w, arrays[k][b, h]) for k in W.TENSORS}
                ref = oracle.vda_forward_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam)
                worst = max(worst, float(frame_errors(g[b, h], ref).max()))
        say(f"  max rel err {worst:.3e}")
        assert worst <= TOL[w.dtype], (w.name, worst)


def test_noalloc_allocates_nothing_and_rejects_larger_problems():
    w = CALLS[1]
    dev = to_device(w, W.full_storage(w, threads=1))
    out1 = torch.empty(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out1)
    _noalloc(w, dev, out1)  # the device is set up by now (earlier tests or this call)
    torch.cuda.synchronize()
    free0 = _free_bytes()
    _noalloc(w, dev, out2)
    torch.cuda.synchronize()
    assert _free_bytes() == free0
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    # four 768p heads need 71.2 MB: rejected before anything is enqueued
    big = W.WORKLOADS[3].replace(H=4)
    assert _workspace_bytes(big) > binding.VDA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(binding.VdaError) as e:
        binding.vda_forward_noalloc(big.B, big.H, big.F, big.n, big.d, big.dv, big.T, big.lam, "bf16",
                                    dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out2)
    assert e.value.status == binding.VDA_ERROR_TOO_LARGE
