"""GPU parity of the backward pass (vda_backward) against the float64 oracle's gradients.

Metric: relative Frobenius error per (b, h, frame) for dq, dk, dv and per (b, h) for the
text gradients, max over all.  Bar: 1e-2, the forward's bfloat16 bar.  The adjoint chains
and the recomputed forward states are float32 and dB, dA + dA^T reach the products as bf16
hi + lo pairs, so what is left is the bfloat16 rounding of the inputs and outputs (with a
single bf16 rounding of dB or of the states, ill-conditioned frames came out at 5e-2)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from vda_gpu_util import frame_errors, out_to_float64, run_gpu, say, to_device

pytestmark = pytest.mark.gpu
TOL_BWD = 1e-2


def _d_out(w):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((w.seed, 0xD0))))
    return W.float32_to_bf16_bits(rng.standard_normal(w.shapes()["out"], dtype=np.float32))


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _rel(got, ref, axes):
    return np.sqrt(np.sum((got - ref) ** 2, axis=axes)) / np.maximum(np.sqrt(np.sum(ref ** 2, axis=axes)), 1e-300)


def _run_backward(w, dev, dO):
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    run_gpu(w, dev, plan=plan)  # the forward pass leaves the statistics and states
    grads = plan.backward(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dO)
    torch.cuda.synchronize()
    return grads, plan


def _check(w, grads, dO_bits, heads):
    dO64 = W.bf16_bits_to_float32(dO_bits).astype(np.float64)
    got = [out_to_float64(g) if g is not None else None for g in grads]
    worst = [0.0] * 5
    for b, h in heads:
        x = W.head_float64(w, b, h)
        ref = oracle.vda_backward_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam, dO64[b, h])
        for i in range(3):
            worst[i] = max(worst[i], float(frame_errors(got[i][b, h], ref[i]).max()))
        if w.T > 0:
            for i in (3, 4):
                worst[i] = max(worst[i], float(_rel(got[i][b, h], ref[i], (-2, -1))))
    say(f"  backward {w.name} B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T}: max rel err "
        f"dq {worst[0]:.2e} dk {worst[1]:.2e} dv {worst[2]:.2e} dtk {worst[3]:.2e} dtv {worst[4]:.2e}")
    for g in got:
        if g is not None:
            assert np.all(np.isfinite(g))
    assert max(worst) <= TOL_BWD, worst


SMALL = [
    ("b_128x128_ragged", dict(d=128, dv=128, n=200, T=37, F=5, B=2, H=2)),
    ("b_64x128", dict(d=64, dv=128, n=130, T=5, F=4, B=1, H=3)),
    ("b_128x64", dict(d=128, dv=64, n=97, T=64, F=3, B=1, H=2)),
    ("b_32x32", dict(d=32, dv=32, n=300, T=1, F=6, B=1, H=2)),
    ("b_128x32", dict(d=128, dv=32, n=64, T=3, F=2, B=1, H=1)),
    ("b_32x128", dict(d=32, dv=128, n=65, T=9, F=2, B=1, H=1)),
    ("b_no_text", dict(d=128, dv=128, n=100, T=0, F=3, B=1, H=1)),
    ("b_split_frames", dict(d=128, dv=128, n=4000, T=10, F=2, B=1, H=1)),
    ("b_F1", dict(d=64, dv=64, n=333, T=20, F=1, B=1, H=2)),
    ("b_lowrank_lam_small", dict(d=128, dv=128, n=300, T=16, F=6, B=1, H=1, kind="lowrank", lam=0.05)),
    # at d = dv = 128 dQ is formed in the Q^T dO pass, 64 tokens a chunk: a frame shorter than
    # one chunk, a one-token frame, one frame
    ("b_128x128_short", dict(d=128, dv=128, n=37, T=4, F=3, B=1, H=2)),
    ("b_128x128_n1", dict(d=128, dv=128, n=1, T=2, F=4, B=1, H=1)),
    ("b_128x128_F1", dict(d=128, dv=128, n=129, T=7, F=1, B=2, H=1)),
]


@pytest.mark.parametrize("name,over", SMALL, ids=[s[0] for s in SMALL])
def test_backward_small_shapes_parity(name, over):
    w = W.WORKLOADS[2].replace(name=name, seed=500 + [s[0] for s in SMALL].index(name), **over)
    say(f"[gpu] backward parity {name}")
    dev = to_device(w, W.full_storage(w, threads=1))
    if w.T == 0:
        dev["text_k"] = dev["text_v"] = None
    dO = _d_out(w)
    grads, plan = _run_backward(w, dev, _bf16(dO))
    _check(w, grads, dO, [(b, h) for b in range(w.B) for h in range(w.H)])
    plan.close()


def test_backward_full_size_every_head_parity():
    """The backward pass at 768p; the oracle's gradients of every (b,h) slice, from the stored
    inputs, each slice converted on its own (a whole gradient in float64 would be 18 GB)."""
    import threadpoolctl
    from concurrent.futures import ThreadPoolExecutor

    w = W.WORKLOADS[3]
    say(f"[gpu] backward full-size {w.name}: generating inputs")
    arrays = W.full_storage(w)
    dev = to_device(w, arrays)
    dO = _d_out(w)
    say(f"[gpu] backward full-size {w.name}: running")
    grads, plan = _run_backward(w, dev, _bf16(dO))
    del dev
    plan.close()
    say(f"[gpu] backward full-size {w.name}: oracle on every head")

    def one(bh):
        b, h = bh
        x = {k: W.storage_to_float64(w, arrays[k][b, h]) for k in W.TENSORS}
        dO64 = W.bf16_bits_to_float32(dO[b, h]).astype(np.float64)
        ref = oracle.vda_backward_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam, dO64)
        got = [g[b, h].float().cpu().numpy().astype(np.float64) for g in grads]
        errs = [float(frame_errors(got[i], ref[i]).max()) for i in range(3)]
        errs += [float(_rel(got[i], ref[i], (-2, -1))) for i in (3, 4)]
        return bh, errs, all(bool(np.all(np.isfinite(a))) for a in got)

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, heads))
    worst = [max(r[1][i] for r in res) for i in range(5)]
    say(f"  backward {w.name}: max rel err over all {len(heads)} heads: dq {worst[0]:.2e} dk {worst[1]:.2e} "
        f"dv {worst[2]:.2e} dtk {worst[3]:.2e} dtv {worst[4]:.2e}")
    assert all(r[2] for r in res)
    assert max(worst) <= TOL_BWD, worst


def test_backward_empty_frames_give_zero_text_gradients():
    w = W.WORKLOADS[2].replace(H=2, F=0, n=100, T=8)
    say("[gpu] backward F = 0")
    dev = to_device(w, W.full_storage(w, threads=1))
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    dtk = torch.full_like(dev["text_k"], 7.0)
    dtv = torch.full_like(dev["text_v"], 7.0)
    empty = torch.empty((w.B, w.H, 0, w.n, w.d), dtype=torch.bfloat16, device="cuda")
    plan.backward(empty, empty, empty, dev["text_k"], dev["text_v"], empty,
                  grads=(empty, empty, empty, dtk, dtv))
    torch.cuda.synchronize()
    assert not dtk.any() and not dtv.any()
    plan.close()


def test_backward_argument_errors():
    w = W.WORKLOADS[2].replace(H=2, F=3, n=100, T=8)
    say("[gpu] backward argument errors")
    dev = to_device(w, W.full_storage(w, threads=1))
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    run_gpu(w, dev, plan=plan)
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    dO = torch.zeros(w.shapes()["out"], dtype=torch.bfloat16, device="cuda")
    g = [torch.zeros_like(dev[x]) for x in W.TENSORS]
    ins = [P(dev[x]) for x in W.TENSORS]
    f = lib.vda_backward
    assert f(plan.handle, *ins, None, *[P(t) for t in g], s) == binding.VDA_ERROR_INVALID_VALUE
    assert f(plan.handle, *ins, P(dO), P(g[0]) + 2, *[P(t) for t in g[1:]], s) == binding.VDA_ERROR_MISALIGNED
    # an output over an input, and two outputs over each other
    assert f(plan.handle, *ins, P(dO), ins[1], *[P(t) for t in g[1:]], s) == binding.VDA_ERROR_INVALID_VALUE
    assert f(plan.handle, *ins, P(dO), P(g[0]), P(g[0]), *[P(t) for t in g[2:]], s) == \
        binding.VDA_ERROR_INVALID_VALUE
    torch.cuda.synchronize()
    assert not any(t.any() for t in g)
    ws_fwd = plan.workspace_bytes
    assert f(plan.handle, *ins, P(dO), *[P(t) for t in g], s) == binding.VDA_SUCCESS
    torch.cuda.synchronize()
    assert plan.workspace_bytes > ws_fwd  # the backward workspace is counted once allocated
    plan.close()
    # no forward pass on this plan yet: nothing to differentiate
    fresh = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    assert f(fresh.handle, *ins, P(dO), *[P(t) for t in g], s) == binding.VDA_ERROR_INVALID_VALUE
    fresh.close()
    for dtype, idx in (("fp8", 6), ("f32", 1)):
        wx = W.WORKLOADS[idx].replace(H=1, F=2, n=64, T=4)
        px = binding.Plan(wx.B, wx.H, wx.F, wx.n, wx.d, wx.dv, wx.T, wx.lam, wx.dtype)
        assert f(px.handle, *ins, P(dO), *[P(t) for t in g], s) == binding.VDA_ERROR_NOT_SUPPORTED
        px.close()
