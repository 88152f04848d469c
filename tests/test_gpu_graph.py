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
