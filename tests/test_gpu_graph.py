"""vda_forward captured in a HIP graph: every replay equals an eager call on the same
inputs, with eager work and synchronisations between replays, also after the inputs
change in place.  A forward pass makes no runtime call but kernel launches (kernel
attributes are set when the plan is created), so the whole pass can be captured."""
import pytest
import torch

import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from vda_gpu_util import run_gpu, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx,over", [
    (3, dict(H=2, F=5, n=333, T=20)),                 # bf16 d = dv = 128
    (2, dict(H=2, F=4, n=200, T=9)),                  # bf16 d = dv = 64
    (1, dict(H=2, F=3, n=100, T=16)),                 # fp32 d = dv = 32
    (6, dict(H=2, F=5, n=333, T=20)),                 # FP8 inputs, d = dv = 128
    (3, dict(H=1, F=50, n=64, T=8)),                  # one head, 50 frames: the chunked scan
])
def test_forward_replays_in_a_graph(idx, over):
    w = W.WORKLOADS[idx].replace(name=f"graph_{idx}", **over)
    say(f"[gpu] graph replay {w.name}")
    dev = to_device(w, W.full_storage(w, threads=1))
    eager, plan = run_gpu(w, dev)
    ints = torch.int32 if w.dtype == "f32" else torch.int16

    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up away from the default stream
        plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(ints), eager.view(ints)), f"replay {i}"

    # new input values in the captured buffers: the replay follows them
    if w.dtype == "fp8":  # e4m3 codes: negate v, reverse the features of q
        dev["v"].bitwise_xor_(0x80)
        dev["q"].copy_(dev["q"].flip(-1))
    else:
        dev["v"].mul_(-0.5)
        dev["q"].mul_(2.0)
    ref2, _ = run_gpu(w, dev, plan=plan)
    ref2 = ref2.clone()
    for i in range(2):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(ints), ref2.view(ints)), f"replay after update {i}"
    assert not torch.equal(ref2.view(ints), eager.view(ints))
    del g
    plan.close()


def test_gated_forward_and_backward_replay_in_graphs():
    """vda_forward_gated and vda_backward (after its first call, which allocates the backward
    workspace) launch kernels only, so each can be captured and replayed."""
    import numpy as np
    w = W.WORKLOADS[3].replace(name="graph_gated_bwd", H=2, F=4, n=200, T=20)
    say("[gpu] graph replay gated + backward")
    dev = to_device(w, W.full_storage(w, threads=1))
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    g = W.gate_weights(w)
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    wg, wo = bits(g["w_gate"]), bits(g["w_out"])
    bg = torch.from_numpy(np.ascontiguousarray(g["b_gate"])).cuda()
    args = (dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"])
    y_eager = plan.forward_gated(*args, wg, bg, wo)
    d_out = torch.randn(w.shapes()["out"], generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    plan.forward(*args, torch.empty_like(y_eager))
    grads_eager = [t.clone() for t in plan.backward(*args, d_out)]  # first call allocates
    torch.cuda.synchronize()

    y = torch.empty_like(y_eager)
    grads = tuple(torch.empty_like(t) for t in grads_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.forward_gated(*args, wg, bg, wo, out=y)
        plan.backward(*args, d_out, grads=grads)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        # the gated pass writes the same statistics and states the backward pass reads
        plan.forward_gated(*args, wg, bg, wo, out=y)
        plan.backward(*args, d_out, grads=grads)
    for i in range(3):
        y.zero_()
        for t in grads:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), f"replay {i}"
        for a, b in zip(grads, grads_eager):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {i}"
    del graph
    plan.close()


def test_noalloc_forward_replays_in_a_graph():
    """vda_forward_noalloc, the entry point for callers that cannot allocate, launches kernels
    only once its device is set up (on its first call): captured in a graph, every replay
    equals vda_forward on a plan running the same serial scan, also after the inputs change
    in place."""
    w = W.WORKLOADS[3].replace(name="graph_noalloc", H=2, F=5, n=333, T=20, seed=41)
    say("[gpu] graph replay noalloc")
    dev = to_device(w, W.full_storage(w, threads=1))
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    plan.set_scan_chunk(0)
    eager, _ = run_gpu(w, dev, plan=plan)
    out = torch.empty_like(eager)

    def call():
        binding.vda_forward_noalloc(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype, dev["q"], dev["k"],
                                    dev["v"], dev["text_k"], dev["text_v"], out)

    call()  # sets the device up outside the capture
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
    dev["v"].mul_(-0.5)
    dev["q"].mul_(2.0)
    ref2, _ = run_gpu(w, dev, plan=plan)
    ref2 = ref2.clone()
    for i in range(2):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref2.view(torch.int16)), f"replay after update {i}"
    del g
    plan.close()
