"""GPU parity: the HIP library (through its C ABI) against the float64 oracle, on the
same seeded, identically rounded inputs.  Bar: max per-(b,h,frame) relative Frobenius
error <= 1e-4 for float32 workloads and <= 1e-2 for bfloat16 and FP8 (e4m3) workloads."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from frame_wise_delta_vda_amd import vda as binding
from vda_gpu_util import TOL, frame_errors, out_to_float64, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


def _oracle_heads(w, heads):
    """Oracle output for the listed (b,h) slices: dict (b,h) -> [F,n,dv] float64."""
    res = {}
    for b, h in heads:
        x = W.head_float64(w, b, h)
        res[(b, h)] = oracle.vda_forward_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam)
    return res


def _check_heads(w, out, heads):
    got = out_to_float64(out)
    ref = _oracle_heads(w, heads)
    worst = 0.0
    for (b, h), r in ref.items():
        e = frame_errors(got[b, h], r)
        worst = max(worst, float(e.max()))
    say(f"  {w.name} B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T}: "
        f"max rel err {worst:.3e} over {len(heads)} heads")
    assert np.all(np.isfinite(got))
    assert worst <= TOL[w.dtype], worst
    return worst


@pytest.mark.parametrize("idx", [1, 2])
def test_named_workload_full_parity(idx):
    w = W.WORKLOADS[idx]
    say(f"[gpu] full parity {w.name}")
    dev = to_device(w, W.full_storage(w))
    out, plan = run_gpu(w, dev)
    _check_heads(w, out, [(b, h) for b in range(w.B) for h in range(w.H)])
    plan.close()


@pytest.mark.parametrize("idx", [3, 4, 5, 6])
def test_named_workload_sampled_parity(idx):
    """Full-size problem in the launch configuration the benchmark times; the oracle
    recomputes three whole (b,h) slices, every other slice is checked for finiteness."""
    w = W.WORKLOADS[idx]
    say(f"[gpu] full-size {w.name}: generating inputs")
    dev = to_device(w, W.full_storage(w))
    say(f"[gpu] full-size {w.name}: running")
    out, plan = run_gpu(w, dev)
    del dev
    heads = [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 2)]
    _check_heads(w, out, sorted(set(heads)))
    plan.close()


SMALL = [
    # name, overrides: span several 64-token chunks and 32-token units with ragged tails
    ("bf16_128x128_ragged", dict(dtype="bf16", d=128, dv=128, n=200, T=37, F=5, B=2, H=2)),
    ("bf16_64x128", dict(dtype="bf16", d=64, dv=128, n=130, T=5, F=4, B=1, H=3)),
    ("bf16_128x64", dict(dtype="bf16", d=128, dv=64, n=97, T=64, F=3, B=1, H=2)),
    ("bf16_32x32", dict(dtype="bf16", d=32, dv=32, n=300, T=1, F=6, B=1, H=2)),
    ("bf16_32x128", dict(dtype="bf16", d=32, dv=128, n=65, T=0, F=2, B=1, H=1)),
    ("bf16_128x32", dict(dtype="bf16", d=128, dv=32, n=64, T=3, F=2, B=1, H=1)),
    ("bf16_128x128_no_text", dict(dtype="bf16", d=128, dv=128, n=64, T=0, F=3, B=1, H=1)),
    # few frames: the readout splits each frame into 4 parts of 16, 16, 16 and 15 tiles
    ("bf16_split_frames", dict(dtype="bf16", d=128, dv=128, n=4000, T=10, F=2, B=1, H=1)),
    ("bf16_n1", dict(dtype="bf16", d=64, dv=64, n=1, T=1, F=7, B=1, H=2)),
    ("bf16_F1", dict(dtype="bf16", d=128, dv=128, n=333, T=20, F=1, B=1, H=1)),
    ("f32_128x128", dict(dtype="f32", d=128, dv=128, n=150, T=9, F=3, B=1, H=2)),
    ("f32_64x32", dict(dtype="f32", d=64, dv=32, n=77, T=0, F=4, B=2, H=1)),
    ("f32_32x64", dict(dtype="f32", d=32, dv=64, n=33, T=40, F=3, B=1, H=1)),
    ("bf16_lowrank_lam_small", dict(dtype="bf16", d=128, dv=128, n=300, T=16, F=6, B=1, H=1,
                                    kind="lowrank", lam=0.05)),
    # FP8 e4m3 inputs: the d = dv = 128 staging (16-byte loads of 16 codes) and the others
    # (8-byte loads of 8 codes), ragged chunks and tiles, split frames
    ("fp8_128x128_ragged", dict(dtype="fp8", d=128, dv=128, n=200, T=37, F=5, B=2, H=2)),
    ("fp8_64x128", dict(dtype="fp8", d=64, dv=128, n=130, T=5, F=4, B=1, H=3)),
    ("fp8_128x64", dict(dtype="fp8", d=128, dv=64, n=97, T=64, F=3, B=1, H=2)),
    ("fp8_32x32", dict(dtype="fp8", d=32, dv=32, n=300, T=1, F=6, B=1, H=2)),
    ("fp8_128x128_no_text", dict(dtype="fp8", d=128, dv=128, n=64, T=0, F=3, B=1, H=1)),
    ("fp8_split_frames", dict(dtype="fp8", d=128, dv=128, n=4000, T=10, F=2, B=1, H=1)),
    ("fp8_n1", dict(dtype="fp8", d=64, dv=64, n=1, T=1, F=7, B=1, H=2)),
    ("fp8_lowrank_lam_small", dict(dtype="fp8", d=128, dv=128, n=300, T=16, F=6, B=1, H=1,
                                   kind="lowrank", lam=0.05)),
]


@pytest.mark.parametrize("name,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_parity(name, over):
    w = W.WORKLOADS[2].replace(name=name, seed=100 + [s[0] for s in SMALL].index(name), **over)
    say(f"[gpu] small parity {name}")
    dev = to_device(w, W.full_storage(w, threads=1))
    if w.T == 0:
        dev["text_k"] = dev["text_v"] = None  # NULL text pointers are allowed when T == 0
    out, plan = run_gpu(w, dev)
    _check_heads(w, out, [(b, h) for b in range(w.B) for h in range(w.H)])
    plan.close()


def test_readout_last_round_in_parts():
    """600 frames of 16 tiles on 512 resident readout workgroups (two per CU on 256 CUs):
    frames 512..599 are read out in quarter frames.  Head 5 holds frames 500..599."""
    w = W.WORKLOADS[3].replace(name="readout_tail_parts", H=6, F=100, n=1000, T=10, seed=77)
    say("[gpu] readout tail parts")
    dev = to_device(w, W.full_storage(w))
    out, plan = run_gpu(w, dev)
    _check_heads(w, out, [(0, 5), (0, 2)])
    plan.close()


def test_intermediates_match_oracle():
    """Workspace after a forward pass: Ainv_f (lam I + K_f^T K_f) = I, Bm_f = K_f^T V_f, and
    the forward/backward states against the oracle's."""
    for w in (W.WORKLOADS[1], W.WORKLOADS[2].replace(H=2, F=5, n=200, T=30),
              W.WORKLOADS[3].replace(H=1, F=4, n=300, T=20),
              W.WORKLOADS[2].replace(H=1, F=3, n=100, T=8, d=32, dv=128),
              W.WORKLOADS[6].replace(H=1, F=4, n=300, T=20),
              W.WORKLOADS[6].replace(H=1, F=3, n=100, T=8, d=64, dv=32)):
        say(f"[gpu] intermediates {w.name}")
        dev = to_device(w, W.full_storage(w, threads=1))
        out, plan = run_gpu(w, dev)
        ainv_p, bm_p, xf_p, xb_p = plan.debug_workspace()
        BH, F1, d, dv = w.B * w.H, w.F + 1, w.d, w.dv

        def fetch(ptr, shape, dtype=torch.float32):
            t = torch.empty(shape, dtype=dtype, device="cuda")
            nbytes = t.numel() * t.element_size()
            torch.cuda.synchronize()
            import ctypes
            hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
            hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
            assert hip.hipMemcpy(t.data_ptr(), ptr, nbytes, 3) == 0  # device to device
            if dtype == torch.int16:
                return t.cpu().numpy().view(np.uint16)
            return t.cpu().numpy().astype(np.float64)

        if w.dtype == "f32":
            ainv = fetch(ainv_p, (BH, F1, d, d))
        else:
            # per frame two bfloat16 planes, hi then lo, each the packed upper triangle of
            # 16 x 16 row-major blocks: block (R, C), R <= C, at R*NB - R*(R-1)/2 + C - R
            nb = d // 16
            nub = nb * (nb + 1) // 2
            u16 = fetch(ainv_p, (BH, F1, 2 * d * d), torch.int16)[:, :, :2 * nub * 256]
            planes = W.bf16_bits_to_float32(u16.reshape(BH, F1, 2, nub, 16, 16)).astype(np.float64)
            blocks = planes[:, :, 0] + planes[:, :, 1]
            ainv = np.zeros((BH, F1, d, d))
            for R in range(nb):
                for Cb in range(R, nb):
                    blk = blocks[:, :, R * nb - R * (R - 1) // 2 + Cb - R]
                    ainv[:, :, 16 * R:16 * R + 16, 16 * Cb:16 * Cb + 16] = blk
                    ainv[:, :, 16 * Cb:16 * Cb + 16, 16 * R:16 * R + 16] = np.swapaxes(blk, -1, -2)
        def unblock(a):  # [..., d*dv] blocked -> [..., d, dv] row-major (layout in include/vda.h)
            lead = a.shape[:-1]
            a = a.reshape(lead + (dv // 16, d // 16, 4, 16, 4))
            nl = len(lead)
            perm = tuple(range(nl)) + (nl + 1, nl + 2, nl + 4, nl, nl + 3)
            return np.transpose(a, perm).reshape(lead + (d, dv))

        bm = unblock(fetch(bm_p, (BH, F1, d * dv)))
        if w.dtype == "f32":
            xf = unblock(fetch(xf_p, (BH, w.F, d * dv)))
            xb = unblock(fetch(xb_p, (BH, w.F, d * dv)))
        else:
            def unfrag_state(u16):  # [c/16][r/32][(r%32)/8][c%16][r%8] -> [r][c] (include/vda.h)
                a = u16.reshape(BH, w.F, dv // 16, d // 32, 4, 16, 8)
                a = np.transpose(a, (0, 1, 3, 4, 6, 2, 5)).reshape(BH, w.F, d, dv)
                if w.dtype == "fp8" and d >= 64:  # row r is stored at position paired(r)
                    r = np.arange(d)
                    a = a[:, :, (r & ~0x38) | ((r & 0x08) << 2) | ((r & 0x30) >> 1), :]
                return W.bf16_bits_to_float32(a).astype(np.float64)
            xf = unfrag_state(fetch(xf_p, (BH, w.F, d * dv), torch.int16))
            xb = unfrag_state(fetch(xb_p, (BH, w.F, d * dv), torch.int16))
        tol = 1e-5 if w.dtype == "f32" else 1e-4
        # bf16 plans store the states rounded once to bf16: each element within 2^-8 relative
        xtol = tol if w.dtype == "f32" else tol + 2.0 ** -8
        for b in range(w.B):
            for h in range(w.H):
                x = W.head_float64(w, b, h)
                i = b * w.H + h
                frames = [(x["text_k"], x["text_v"])] + [(x["k"][f], x["v"][f]) for f in range(w.F)]
                for fi, (K, V) in enumerate(frames):
                    G, Bm = oracle.frame_statistics(K, V)
                    A = w.lam * np.eye(d) + G
                    assert np.abs(ainv[i, fi] @ A - np.eye(d)).max() < tol * 10
                    assert np.abs(bm[i, fi] - Bm).max() <= tol * (1 + np.abs(Bm).max())
                xt, Xf, Xb = oracle.head_states(x["k"], x["v"], x["text_k"], x["text_v"], w.lam)
                for f in range(w.F):
                    assert np.linalg.norm(xf[i, f] - Xf[f]) <= xtol * np.linalg.norm(Xf[f])
                    assert np.linalg.norm(xb[i, f] - Xb[f]) <= xtol * np.linalg.norm(Xb[f])
        plan.close()


def test_bitwise_repeatable_and_no_unwritten_outputs():
    w = W.WORKLOADS[2].replace(H=3, F=4, n=777, T=50)
    say("[gpu] repeatability")
    dev = to_device(w, W.full_storage(w, threads=1))
    out1 = torch.full(w.shapes()["out"], float("nan"), dtype=torch.bfloat16, device="cuda")
    out1, plan = run_gpu(w, dev, out=out1)
    assert not torch.isnan(out1).any()
    out2 = torch.full_like(out1, float("nan"))
    run_gpu(w, dev, plan=plan, out=out2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    plan.close()


def test_stages_compose_to_forward():
    w = W.WORKLOADS[2].replace(H=2, F=3, n=300, T=10)
    say("[gpu] stages")
    dev = to_device(w, W.full_storage(w, threads=1))
    full, plan = run_gpu(w, dev)
    staged = torch.empty_like(full)
    plan.stages(binding.VDA_STAGE_STATS, k=dev["k"], v=dev["v"], text_k=dev["text_k"],
                text_v=dev["text_v"])
    plan.stages(binding.VDA_STAGE_SCAN)
    plan.stages(binding.VDA_STAGE_READOUT, q=dev["q"], out=staged)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), staged.view(torch.int16))
    plan.close()



@pytest.mark.parametrize("d,dv", [(128, 128), (64, 128), (128, 32), (32, 64)])
def test_fp8_plan_matches_bf16_plan_on_the_same_values(d, dv):
    """Every e4m3 value is exact in bfloat16.  Where the FP8 plan converts right after
    loading, it must give the bfloat16 plan's output bit for bit; at d = dv = 128 its
    statistics run on the FP8 MFMA (exact products, fp32 sums in another order), so there
    the outputs agree to the rounding of the bfloat16 output."""
    w8 = W.WORKLOADS[6].replace(H=2, F=3, n=333, T=21, d=d, dv=dv)
    w16 = w8.replace(dtype="bf16")
    say(f"[gpu] fp8 vs bf16 d={d} dv={dv}")
    codes = W.full_storage(w8, threads=1)
    as_bf16 = {k: W.float32_to_bf16_bits(W.e4m3_codes_to_float32(c)) for k, c in codes.items()}
    out8, p8 = run_gpu(w8, to_device(w8, codes))
    out16, p16 = run_gpu(w16, to_device(w16, as_bf16))
    assert out8.dtype == torch.bfloat16
    if (d, dv) == (128, 128):
        e = frame_errors(out_to_float64(out8), out_to_float64(out16))
        say(f"  max rel diff {e.max():.3e}")
        assert e.max() <= 2.0 ** -9
    else:
        assert torch.equal(out8.view(torch.int16), out16.view(torch.int16))
    p8.close()
    p16.close()
