"""C-ABI behaviour on the GPU: argument checks at vda_forward, plan reuse, streams,
empty problems.  Every failing call must leave the output untouched."""
import numpy as np
import pytest
import torch

import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from vda_gpu_util import TOL, frame_errors, out_to_float64, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


def _small(**kw):
    return W.WORKLOADS[2].replace(**{**dict(H=2, F=3, n=100, T=8), **kw})


def test_forward_argument_errors_leave_output_untouched():
    w = _small()
    say("[gpu] abi argument errors")
    dev = to_device(w, W.full_storage(w, threads=1))
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    out = torch.zeros(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
    q, k, v, tk, tv = (dev[x] for x in W.TENSORS)
    lib = binding.load_library()
    h = plan.handle
    s = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    # NULL input
    assert lib.vda_forward(h, P(q), None, P(v), P(tk), P(tv), P(out), s) == binding.VDA_ERROR_INVALID_VALUE
    # misaligned input (2 bytes off)
    assert lib.vda_forward(h, P(q) + 2, P(k), P(v), P(tk), P(tv), P(out), s) == binding.VDA_ERROR_MISALIGNED
    # output aliasing an input
    assert lib.vda_forward(h, P(q), P(k), P(v), P(tk), P(tv), P(q), s) == binding.VDA_ERROR_INVALID_VALUE
    # stage mask outside the defined stages
    assert lib.vda_forward_stages(h, 8, P(q), P(k), P(v), P(tk), P(tv), P(out), s) == \
        binding.VDA_ERROR_INVALID_VALUE
    # NULL text pointers with T > 0
    assert lib.vda_forward(h, P(q), P(k), P(v), None, P(tv), P(out), s) == binding.VDA_ERROR_INVALID_VALUE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0
    plan.close()


def test_plan_reuse_two_plans_two_streams():
    w1, w2 = _small(seed=201), _small(seed=202, n=63, T=0)
    say("[gpu] plan reuse / streams")
    d1 = to_device(w1, W.full_storage(w1, threads=1))
    d2 = to_device(w2, W.full_storage(w2, threads=1))
    ref1, p1 = run_gpu(w1, d1)
    ref2, p2 = run_gpu(w2, d2)
    # reuse p1 on the same data: identical
    again, _ = run_gpu(w1, d1, plan=p1)
    assert torch.equal(again.view(torch.int16), ref1.view(torch.int16))
    # two plans concurrently on two streams
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1, o2 = torch.empty_like(ref1), torch.empty_like(ref2)
    torch.cuda.synchronize()
    for _ in range(3):
        p1.forward(d1["q"], d1["k"], d1["v"], d1["text_k"], d1["text_v"], o1, stream=s1)
        p2.forward(d2["q"], d2["k"], d2["v"], d2["text_k"], d2["text_v"], o2, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), ref1.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), ref2.view(torch.int16))
    p1.close()
    p2.close()


def test_workspace_size():
    w = _small()
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    BH = w.B * w.H
    state_bytes = 4 if w.dtype == "f32" else 2  # bf16 plans keep the states in bf16
    expect = 4 * BH * (w.F + 1) * (w.d * w.d + w.d * w.dv) + state_bytes * 2 * BH * w.F * w.d * w.dv
    assert plan.workspace_bytes == expect
    plan.close()


@pytest.mark.parametrize("shape", [dict(F=0), dict(n=0), dict(B=0), dict(H=0)])
def test_empty_problems_are_noops(shape):
    w = _small(**shape)
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    dev = to_device(w, W.full_storage(w, threads=1)) if w.B * w.H * w.F * w.n else None
    if dev is None:
        binding.vda_forward(plan.handle, None, None, None, None, None, None)
    else:
        out = torch.zeros(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
        plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out)
    torch.cuda.synchronize()
    plan.close()


def test_nan_inputs_propagate_to_their_frame_only():
    w = _small(H=1)
    say("[gpu] nan propagation")
    arrs = W.full_storage(w, threads=1)
    arrs["q"] = arrs["q"].copy()
    arrs["q"][0, 0, 1, 5, 3] = 0x7FC0  # bf16 NaN in one query of frame 1
    dev = to_device(w, arrs)
    out, plan = run_gpu(w, dev)
    o = out_to_float64(out)
    assert np.isnan(o[0, 0, 1, 5]).all()
    o[0, 0, 1, 5] = 0
    assert np.isfinite(o).all()
    plan.close()


def test_timing_of_whole_passes():
    """Timing records only whole passes, at most `capacity` of them, and each stage of a
    pass takes positive time; enabling with a bad capacity is an argument error."""
    w = W.WORKLOADS[2].replace(H=2, F=3, n=300, T=10)
    say("[gpu] timing")
    dev = to_device(w, W.full_storage(w, threads=1))
    out, plan = run_gpu(w, dev)
    with pytest.raises(binding.VdaError):
        plan.enable_timing(-1)
    plan.enable_timing(2)
    for _ in range(3):
        run_gpu(w, dev, plan=plan, out=out)
    plan.stages(binding.VDA_STAGE_SCAN)
    calls, st, sc, rd = plan.timings()
    assert calls == 2 and st > 0 and sc > 0 and rd > 0
    assert plan.timings()[0] == 0
    plan.enable_timing(0)
    run_gpu(w, dev, plan=plan, out=out)
    assert plan.timings()[0] == 0
    plan.close()


def test_fp8_plan_sizes_and_nan_codes():
    """FP8 plans: inputs are one byte per element, the output and the workspace are the
    bfloat16 plan's, and a NaN code (S.1111.111) in one key reaches the output."""
    w = W.WORKLOADS[6].replace(H=1, F=3, n=100, T=8, d=64, dv=64)
    say("[gpu] fp8 sizes and NaN codes")
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    assert plan.workspace_bytes == 4 * (w.F + 1) * (w.d * w.d + w.d * w.dv) + 2 * 2 * w.F * w.d * w.dv
    arrs = W.full_storage(w, threads=1)
    arrs["k"] = arrs["k"].copy()
    arrs["k"][0, 0, 1, 7, 2] = 0x7F  # frame 2 of 3 (index 1)
    dev = to_device(w, arrs)
    # a bfloat16-sized output argument is what the plan writes; q of the wrong byte size is
    # not detectable, but a misaligned one is
    out = torch.zeros(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    qv = dev["q"].view(-1)
    assert lib.vda_forward(plan.handle, P(qv) + 8, P(dev["k"]), P(dev["v"]), P(dev["text_k"]),
                           P(dev["text_v"]), P(out), s) == binding.VDA_ERROR_MISALIGNED
    plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out)
    torch.cuda.synchronize()
    o = out_to_float64(out)[0, 0]
    # frame 1's statistics are NaN; the forward chain carries that to frames 1..2 and the
    # backward chain to frames 0..1, so every frame reads out NaN
    assert np.isnan(o).all()
    plan.close()
