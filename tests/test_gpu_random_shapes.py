"""Seeded random shapes against the oracle: every width pair, ragged and tiny token counts, one
to many frames, with and without text, float32, bfloat16 and FP8 inputs, Gaussian and low-rank
keys over a range of lambda, and the serial, automatic and chunked scans.  Every frame of every
head is compared (max per-(b,h,frame) relative Frobenius error <= 1e-4 for float32, 1e-2 for
bfloat16 and FP8).  The draws stay inside the verified conditioning range (the condition
number of lam I + K_f^T K_f below about 1e4 for bfloat16 and FP8; float32 cases use Gaussian
keys and lam >= 0.5, whose condition numbers are small)."""
import numpy as np
import pytest

import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from test_gpu_parity import _check_heads
from vda_gpu_util import run_gpu, say, to_device

pytestmark = pytest.mark.gpu


def _cases(count=96, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        dtype = ["f32", "bf16", "bf16", "fp8"][int(rng.integers(4))]
        d, dv = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
        n = int(rng.choice([1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 333, 517, 1000]))
        F = int(rng.choice([1, 2, 3, 5, 8, 13, 50, 64]))
        T = int(rng.choice([0, 1, 7, 64, 100]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        if dtype == "f32":
            kind, lam = "gaussian", float(rng.choice([0.5, 1.0, 2.0]))
            chunk = 0
        else:
            kind = "lowrank" if rng.random() < 0.3 else "gaussian"
            lam = float(rng.choice([0.05, 0.1, 0.5, 1.0, 2.0]))
            chunk = int(rng.choice([0, binding.VDA_SCAN_CHUNK_AUTO, 1, 3, 7]))
        w = W.WORKLOADS[2].replace(name=f"rand{i:02d}", B=B, H=H, F=F, n=n, d=d, dv=dv, T=T, lam=lam,
                                   dtype=dtype, kind=kind, seed=4000 + i)
        cases.append((w, chunk))
    return cases


CASES = _cases()


@pytest.mark.parametrize("w,chunk", CASES, ids=[c[0].name for c in CASES])
def test_random_shape_parity(w, chunk):
    say(f"[gpu] {w.name}: {w.dtype} B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T} "
        f"lam={w.lam} {w.kind} scan chunk {chunk}")
    dev = to_device(w, W.full_storage(w, threads=1))
    if w.T == 0:
        dev["text_k"] = dev["text_v"] = None
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    plan.set_scan_chunk(chunk)
    out, _ = run_gpu(w, dev, plan=plan)
    plan.close()
    _check_heads(w, out, [(b, h) for b in range(w.B) for h in range(w.H)])


def _epilogue_cases(count, seed, dtypes):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        dtype = dtypes[int(rng.integers(len(dtypes)))]
        d, dv = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
        w = W.WORKLOADS[2].replace(
            name=f"rand_{seed}_{i:02d}", B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)),
            F=int(rng.choice([1, 2, 3, 5, 8])), n=int(rng.choice([1, 31, 64, 65, 129, 200, 333])), d=d, dv=dv,
            T=int(rng.choice([0, 1, 7, 64])), lam=float(rng.choice([0.1, 0.5, 1.0, 2.0])), dtype=dtype,
            kind="lowrank" if rng.random() < 0.3 else "gaussian", seed=5000 + seed + i)
        cases.append(w)
    return cases


GATED = _epilogue_cases(24, 11, ["bf16", "bf16", "fp8"])


@pytest.mark.parametrize("w", GATED, ids=[w.name for w in GATED])
def test_random_shape_gated_parity(w):
    from test_gpu_gated import _check, _gate_to_device, _run_gated
    say(f"[gpu] gated {w.name}: {w.dtype} B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T} "
        f"lam={w.lam} {w.kind}")
    g = W.gate_weights(w)
    dev = to_device(w, W.full_storage(w, threads=1))
    if w.T == 0:
        dev["text_k"] = dev["text_v"] = None
    out, plan = _run_gated(w, dev, _gate_to_device(g))
    plan.close()
    _check(w, out, g, [(b, h) for b in range(w.B) for h in range(w.H)])


BACKWARD = _epilogue_cases(24, 12, ["bf16"])


@pytest.mark.parametrize("w", BACKWARD, ids=[w.name for w in BACKWARD])
def test_random_shape_backward_parity(w):
    from test_gpu_backward import _bf16, _check, _d_out, _run_backward
    say(f"[gpu] backward {w.name}: B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T} "
        f"lam={w.lam} {w.kind}")
    dev = to_device(w, W.full_storage(w, threads=1))
    if w.T == 0:
        dev["text_k"] = dev["text_v"] = None
    dO = _d_out(w)
    grads, plan = _run_backward(w, dev, _bf16(dO))
    plan.close()
    _check(w, grads, dO, [(b, h) for b in range(w.B) for h in range(w.H)])
