"""GPU parity of the gated fusion epilogue (vda_forward_gated) against the float64 oracle:
Y = sigmoid(O W_g^T + b_g) * (O W_o^T) per head on the forward pass's output O, with seeded
synthetic bfloat16 weights.  Bar: max per-(b,h,frame) relative Frobenius error <= 1e-2."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from vda_gpu_util import TOL, frame_errors, out_to_float64, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


def _gate_to_device(g):
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return {"w_gate": bits(g["w_gate"]), "w_out": bits(g["w_out"]),
            "b_gate": torch.from_numpy(np.ascontiguousarray(g["b_gate"], dtype=np.float32)).cuda()}


def _run_gated(w, dev, gdev, plan=None):
    own = plan is None
    if own:
        plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    out = torch.empty(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
    plan.forward_gated(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"],
                       gdev["w_gate"], gdev["b_gate"], gdev["w_out"], out)
    torch.cuda.synchronize()
    return out, plan


def _check(w, out, g, heads):
    got = out_to_float64(out)
    g64 = W.gate_weights_float64(w, g)
    worst = 0.0
    for b, h in heads:
        x = W.head_float64(w, b, h)
        ref = oracle.vda_forward_gated_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam,
                                            g64["w_gate"][h], g64["b_gate"][h], g64["w_out"][h])
        worst = max(worst, float(frame_errors(got[b, h], ref).max()))
    say(f"  gated {w.name} B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T}: "
        f"max rel err {worst:.3e} over {len(heads)} heads")
    assert np.all(np.isfinite(got))
    assert worst <= TOL[w.dtype], worst


SMALL = [
    ("g_bf16_128x128_ragged", dict(dtype="bf16", d=128, dv=128, n=200, T=37, F=5, B=2, H=2)),
    ("g_bf16_64x128", dict(dtype="bf16", d=64, dv=128, n=130, T=5, F=4, B=1, H=3)),
    ("g_bf16_128x64", dict(dtype="bf16", d=128, dv=64, n=97, T=64, F=3, B=1, H=2)),
    ("g_bf16_32x32", dict(dtype="bf16", d=32, dv=32, n=300, T=1, F=6, B=1, H=2)),
    ("g_bf16_128x32", dict(dtype="bf16", d=128, dv=32, n=64, T=3, F=2, B=1, H=1)),
    ("g_bf16_32x128", dict(dtype="bf16", d=32, dv=128, n=65, T=0, F=2, B=1, H=1)),
    ("g_bf16_split_frames", dict(dtype="bf16", d=128, dv=128, n=4000, T=10, F=2, B=1, H=1)),
    ("g_bf16_n1", dict(dtype="bf16", d=64, dv=64, n=1, T=1, F=7, B=1, H=2)),
    ("g_fp8_128x128_ragged", dict(dtype="fp8", d=128, dv=128, n=200, T=37, F=5, B=2, H=2)),
    ("g_fp8_64x64", dict(dtype="fp8", d=64, dv=64, n=130, T=5, F=4, B=1, H=3)),
    ("g_fp8_32x64", dict(dtype="fp8", d=32, dv=64, n=77, T=9, F=3, B=1, H=2)),
]


@pytest.mark.parametrize("name,over", SMALL, ids=[s[0] for s in SMALL])
def test_gated_small_shapes_parity(name, over):
    w = W.WORKLOADS[2].replace(name=name, seed=300 + [s[0] for s in SMALL].index(name), **over)
    say(f"[gpu] gated parity {name}")
    g = W.gate_weights(w)
    dev = to_device(w, W.full_storage(w, threads=1))
    if w.T == 0:
        dev["text_k"] = dev["text_v"] = None
    out, plan = _run_gated(w, dev, _gate_to_device(g))
    _check(w, out, g, [(b, h) for b in range(w.B) for h in range(w.H)])
    plan.close()


def _check_every_head(w, out, g, arrays, threads=8):
    """Every (b,h) slice of a full-size gated output against the oracle, from the stored inputs
    (no regeneration); slices run on a thread pool with one BLAS thread each."""
    import threadpoolctl
    from concurrent.futures import ThreadPoolExecutor

    g64 = W.gate_weights_float64(w, g)

    def one(bh):
        b, h = bh
        x = {k: W.storage_to_float64(w, arrays[k][b, h]) for k in W.TENSORS}
        ref = oracle.vda_forward_gated_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam,
                                            g64["w_gate"][h], g64["b_gate"][h], g64["w_out"][h])
        got = out[b, h].float().cpu().numpy().astype(np.float64)
        return bh, float(frame_errors(got, ref).max()), bool(np.all(np.isfinite(got)))

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, heads))
    worst_bh, worst, _ = max(res, key=lambda r: r[1])
    say(f"  gated {w.name} B={w.B} H={w.H} F={w.F} n={w.n}: max rel err {worst:.3e} at (b,h)={worst_bh} "
        f"over all {len(heads)} heads")
    assert all(r[2] for r in res)
    assert worst <= TOL[w.dtype], (worst, worst_bh)


@pytest.mark.parametrize("idx", [3, 6])
def test_gated_full_size_every_head_parity(idx):
    """The gated pass at 768p (bfloat16 and FP8 inputs) in the launch configuration the
    benchmark times; the oracle recomputes every (b,h) slice and every frame of it."""
    w = W.WORKLOADS[idx]
    say(f"[gpu] gated full-size {w.name}: generating inputs")
    g = W.gate_weights(w)
    arrays = W.full_storage(w)
    dev = to_device(w, arrays)
    say(f"[gpu] gated full-size {w.name}: running")
    out, plan = _run_gated(w, dev, _gate_to_device(g))
    del dev
    plan.close()
    say(f"[gpu] gated full-size {w.name}: oracle on every head")
    _check_every_head(w, out, g, arrays)


def test_open_gate_with_identity_projection_is_the_plain_output():
    """b_g = +60 opens every gate fully and W_o = I, so Y is the plain pass's O up to the
    rounding of the folded matrices and the order of the MFMA sums."""
    w = W.WORKLOADS[3].replace(name="gate_identity", H=2, F=4, n=333, T=20)
    say("[gpu] gated identity limit")
    dev = to_device(w, W.full_storage(w, threads=1))
    eye = np.broadcast_to(np.eye(w.dv, dtype=np.float32), (w.H, w.dv, w.dv))
    g = {"w_gate": W.float32_to_bf16_bits(np.zeros((w.H, w.dv, w.dv), np.float32)),
         "w_out": W.float32_to_bf16_bits(eye), "b_gate": np.full((w.H, w.dv), 60.0, np.float32)}
    y, plan = _run_gated(w, dev, _gate_to_device(g))
    o, _ = run_gpu(w, dev, plan=plan)
    e = frame_errors(out_to_float64(y), out_to_float64(o))
    say(f"  max rel diff {e.max():.3e}")
    assert e.max() <= 2.0 ** -8
    plan.close()


def test_gated_argument_errors():
    w = W.WORKLOADS[2].replace(H=2, F=3, n=100, T=8)
    say("[gpu] gated argument errors")
    dev = to_device(w, W.full_storage(w, threads=1))
    gdev = _gate_to_device(W.gate_weights(w))
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    out = torch.zeros(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    q, k, v, tk, tv = (P(dev[x]) for x in W.TENSORS)
    wg, bg, wo = P(gdev["w_gate"]), P(gdev["b_gate"]), P(gdev["w_out"])
    f = lib.vda_forward_gated
    assert f(plan.handle, q, k, v, tk, tv, None, bg, wo, P(out), s) == binding.VDA_ERROR_INVALID_VALUE
    assert f(plan.handle, q, k, v, tk, tv, wg, None, wo, P(out), s) == binding.VDA_ERROR_INVALID_VALUE
    assert f(plan.handle, q, k, v, tk, tv, wg, bg, None, P(out), s) == binding.VDA_ERROR_INVALID_VALUE
    assert f(plan.handle, q, k, v, tk, tv, wg + 2, bg, wo, P(out), s) == binding.VDA_ERROR_MISALIGNED
    big = torch.zeros(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
    assert f(plan.handle, q, k, v, tk, tv, P(big), bg, wo, P(big), s) == binding.VDA_ERROR_INVALID_VALUE
    torch.cuda.synchronize()
    assert not out.any()
    plan.close()
    w32 = W.WORKLOADS[1]
    p32 = binding.Plan(w32.B, w32.H, w32.F, w32.n, w32.d, w32.dv, w32.T, w32.lam, w32.dtype)
    assert f(p32.handle, q, k, v, tk, tv, wg, bg, wo, P(out), s) == binding.VDA_ERROR_NOT_SUPPORTED
    p32.close()
