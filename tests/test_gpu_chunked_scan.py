"""The chunked scan (vda_plan_set_scan_chunk): the forward pass with its state chains split into
chunks of frames -- a local pass per chunk from a zero state together with the chunk's transition,
a serial pass over the chunk ends, and a rerun of every chunk from its true start -- against the
oracle, at the same bar as the serial scan (max per-(b,h,frame) relative Frobenius error <= 1e-2
for bfloat16 and FP8 inputs), and its states against the oracle's."""
import numpy as np
import pytest
import torch

import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from test_gpu_parity import _check_every_head, _check_heads, check_intermediates, fetch_intermediates
from vda_gpu_util import frame_errors, out_to_float64, say, to_device

pytestmark = pytest.mark.gpu


def _run(w, dev, chunk, out=None):
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    plan.set_scan_chunk(chunk)
    if out is None:
        out = torch.empty(w.shapes()["out"], device="cuda", dtype=torch.bfloat16)
    plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out)
    torch.cuda.synchronize()
    return out, plan


SMALL = [
    # name, chunk frames, workload overrides: K = ceil(F / chunk) chunks; K = 2 has no carry
    # pass, a chunk of one frame is the shortest segment, a last chunk shorter than the others
    ("bf16_128_F7_c2", 2, dict(dtype="bf16", d=128, dv=128, n=200, T=37, F=7, B=2, H=2)),
    ("bf16_128_F7_c3", 3, dict(dtype="bf16", d=128, dv=128, n=130, T=5, F=7, B=1, H=2)),
    ("bf16_128_F6_c1", 1, dict(dtype="bf16", d=128, dv=128, n=64, T=8, F=6, B=1, H=1)),
    ("bf16_128_F9_c8", 8, dict(dtype="bf16", d=128, dv=128, n=97, T=20, F=9, B=1, H=2)),
    ("bf16_64x128_F10_c3", 3, dict(dtype="bf16", d=64, dv=128, n=100, T=5, F=10, B=1, H=3)),
    ("bf16_128x64_F8_c2", 2, dict(dtype="bf16", d=128, dv=64, n=77, T=64, F=8, B=1, H=2)),
    ("bf16_32x32_F12_c5", 5, dict(dtype="bf16", d=32, dv=32, n=300, T=1, F=12, B=1, H=2)),
    ("bf16_128x32_F5_c2", 2, dict(dtype="bf16", d=128, dv=32, n=64, T=3, F=5, B=1, H=1)),
    ("bf16_no_text_F6_c2", 2, dict(dtype="bf16", d=128, dv=128, n=64, T=0, F=6, B=1, H=1)),
    ("bf16_n1_F16_c4", 4, dict(dtype="bf16", d=64, dv=64, n=1, T=1, F=16, B=1, H=2)),
    ("bf16_lowrank_F12_c3", 3, dict(dtype="bf16", d=128, dv=128, n=300, T=16, F=12, B=1, H=1,
                                    kind="lowrank", lam=0.05)),
    ("fp8_128_F7_c2", 2, dict(dtype="fp8", d=128, dv=128, n=200, T=37, F=7, B=1, H=2)),
    ("fp8_64x64_F9_c4", 4, dict(dtype="fp8", d=64, dv=64, n=130, T=5, F=9, B=1, H=2)),
]


@pytest.mark.parametrize("name,chunk,over", SMALL, ids=[s[0] for s in SMALL])
def test_chunked_scan_small_shapes(name, chunk, over):
    w = W.WORKLOADS[2].replace(name=name, seed=700 + [s[0] for s in SMALL].index(name), **over)
    say(f"[gpu] chunked scan {name}: chunk {chunk}, K = {-(-w.F // chunk)}")
    dev = to_device(w, W.full_storage(w, threads=1))
    if w.T == 0:
        dev["text_k"] = dev["text_v"] = None
    out, plan = _run(w, dev, chunk)
    # the states themselves against the oracle's (and the inverses and K^T V)
    ainv, bm, xf, xb = fetch_intermediates(w, plan)
    plan.close()
    check_intermediates(w, ainv, bm, xf, xb)
    _check_heads(w, out, [(b, h) for b in range(w.B) for h in range(w.H)])
    # against the serial scan on the same inputs: the same values up to rounding
    serial = torch.empty_like(out)
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    plan.set_scan_chunk(0)
    plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], serial)
    torch.cuda.synchronize()
    plan.close()
    e = frame_errors(out_to_float64(out), out_to_float64(serial))
    say(f"  chunked against serial: max rel diff {e.max():.3e}")
    assert e.max() <= 2.0 ** -7


def test_chunked_scan_is_repeatable_and_can_be_switched_off():
    w = W.WORKLOADS[2].replace(name="chunk_switch", d=128, dv=128, n=150, T=10, F=9, H=2, seed=750)
    dev = to_device(w, W.full_storage(w, threads=1))
    out1, plan = _run(w, dev, 3)
    out2 = torch.full_like(out1, float("nan"))
    plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out2)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    ws = plan.workspace_bytes
    plan.set_scan_chunk(0)  # back to the serial scan: bit for bit a fresh serial plan's output
    assert plan.workspace_bytes < ws
    out3 = torch.empty_like(out1)
    plan.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], out3)
    ref = torch.empty_like(out1)
    plan2 = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    plan2.forward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], ref)
    torch.cuda.synchronize()
    assert torch.equal(out3.view(torch.int16), ref.view(torch.int16))
    plan.set_scan_chunk(100)  # one chunk: the serial scan, no chunk workspace
    assert plan.workspace_bytes == plan2.workspace_bytes
    plan.close()
    plan2.close()


def test_chunked_scan_argument_errors():
    w32 = W.WORKLOADS[1]
    plan = binding.Plan(w32.B, w32.H, w32.F, w32.n, w32.d, w32.dv, w32.T, w32.lam, "f32")
    with pytest.raises(binding.VdaError) as e:
        plan.set_scan_chunk(2)
    assert e.value.status == binding.VDA_ERROR_NOT_SUPPORTED
    plan.set_scan_chunk(0)
    plan.set_scan_chunk(binding.VDA_SCAN_CHUNK_AUTO)  # float32 plans: the serial scan
    assert plan.scan_chunk == 0
    with pytest.raises(binding.VdaError) as e:
        plan.set_scan_chunk(-2)
    assert e.value.status == binding.VDA_ERROR_INVALID_VALUE
    plan.close()


# full size: the long clip (361-step chains) and the ill-conditioned workload, every head
@pytest.mark.parametrize("idx,chunk", [(4, 45), (5, 9)])
def test_chunked_scan_full_size_every_head(idx, chunk):
    w = W.WORKLOADS[idx]
    say(f"[gpu] chunked scan full size {w.name}, chunk {chunk}: generating inputs")
    arrays = W.full_storage(w)
    dev = to_device(w, arrays)
    out, plan = _run(w, dev, chunk)
    del dev
    plan.close()
    say(f"[gpu] chunked scan full size {w.name}: oracle on every head")
    _check_every_head(w, out, arrays)


def test_automatic_choice_of_the_scan():
    """Plans start in the automatic mode: the serial scan where its chains fill the GPU, the
    chunked scan for few heads with many frames (one GPU's share of a head-sharded 768p or
    long-clip problem)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    expect = {3: 0, 4: 0, 5: 0, 7: None, 8: None}
    for idx, want in expect.items():
        w = W.WORKLOADS[idx]
        plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
        got = plan.scan_chunk
        plan.close()
        serial_wgs = 2 * w.B * w.H * (w.dv // 32)
        say(f"  {w.name}: {serial_wgs} serial workgroups on {cus} compute units -> chunk {got}")
        if want == 0:
            assert got == 0
        else:
            assert serial_wgs * 4 <= cus and 1 <= got < w.F
            k = -(-w.F // got)
            assert 2 <= k <= 8
