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


def _check_every_head(w, out, arrays, threads=8):
    """Every (b,h) slice of a full-size output against the oracle, from the stored inputs (no
    regeneration); slices run on a thread pool with one BLAS thread each."""
    import threadpoolctl
    from concurrent.futures import ThreadPoolExecutor

    def one(bh):
        b, h = bh
        x = {k: W.storage_to_float64(w, arrays[k][b, h]) for k in W.TENSORS}
        ref = oracle.vda_forward_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam)
        got = out[b, h].float().cpu().numpy().astype(np.float64)
        finite = bool(np.all(np.isfinite(got)))
        return bh, float(frame_errors(got, ref).max()), finite

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, heads))
    worst_bh, worst, _ = max(res, key=lambda r: r[1])
    say(f"  {w.name} B={w.B} H={w.H} F={w.F} n={w.n} d={w.d} dv={w.dv} T={w.T} lam={w.lam}: "
        f"max rel err {worst:.3e} at (b,h)={worst_bh} over all {len(heads)} heads")
    assert all(r[2] for r in res)
    assert worst <= TOL[w.dtype], (worst, worst_bh)
    return worst


@pytest.mark.parametrize("idx", [3, 4, 5, 6])
def test_named_workload_every_head_parity(idx):
    """Full-size problem in the launch configuration the benchmark times; the oracle
    recomputes every (b,h) slice and every frame of it."""
    w = W.WORKLOADS[idx]
    say(f"[gpu] full-size {w.name}: generating inputs")
    arrays = W.full_storage(w)
    dev = to_device(w, arrays)
    say(f"[gpu] full-size {w.name}: running")
    out, plan = run_gpu(w, dev)
    del dev
    plan.close()
    say(f"[gpu] full-size {w.name}: oracle on every head")
    _check_every_head(w, out, arrays)


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


def test_longest_frame_sampled_parity():
    """One frame of the most tokens the header allows, n = 2^24 - 256, at d = dv = 128: the
    statistics kernel's frame-wide K and V descriptors then span 2^32 - 65536 bytes.  The
    oracle computes the frame's state from all of its tokens; the output is compared on
    sampled rows (both ends, the rows where K and V byte offsets cross 2^31, and 2048 seeded
    random rows) by the relative Frobenius error over those rows."""
    n = 16776960
    w = W.WORKLOADS[3].replace(name="longest_frame", B=1, H=1, F=1, n=n, T=0, seed=901)
    say(f"[gpu] longest frame n={n}: generating inputs")
    arrays = W.full_storage(w)
    dev = to_device(w, arrays)
    dev["text_k"] = dev["text_v"] = None
    say("[gpu] longest frame: running")
    out, plan = run_gpu(w, dev)
    plan.close()
    del dev
    rng = np.random.default_rng(901)
    half = (1 << 31) // (2 * w.d)  # first token whose K row starts at byte 2^31
    rows = np.unique(np.concatenate([np.arange(256), np.arange(half - 64, half + 64), np.arange(n - 300, n),
                                     rng.integers(0, n, 2048)]))
    got = out[0, 0, 0][torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    del out
    torch.cuda.empty_cache()
    say("[gpu] longest frame: oracle")
    k64 = W.storage_to_float64(w, arrays["k"][0, 0])
    v64 = W.storage_to_float64(w, arrays["v"][0, 0])
    empty_k, empty_v = np.zeros((0, w.d)), np.zeros((0, w.dv))
    _, x_fwd, x_bwd = oracle.head_states(k64, v64, empty_k, empty_v, w.lam)
    del k64, v64
    q_rows = W.storage_to_float64(w, arrays["q"][0, 0, 0][rows])[None]
    ref = oracle.readout(q_rows, x_fwd, x_bwd)[0]
    err = float(np.sqrt(np.sum((got - ref) ** 2)) / np.sqrt(np.sum(ref ** 2)))
    say(f"  longest frame: rel err {err:.3e} over {len(rows)} sampled rows")
    assert np.all(np.isfinite(got))
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("chunk", [0, binding.VDA_SCAN_CHUNK_AUTO])
def test_long_chain_every_frame_parity(chunk):
    """4000 frames of 37 tokens (a ragged part of one 64-token chunk) per head: chains of
    4001 steps, run serially and with the automatic choice (chunked for so few heads), every
    frame against the oracle.  The state must neither drift nor lose accuracy with the
    length of the chain."""
    w = W.WORKLOADS[3].replace(name="long_chain", B=1, H=2, F=4000, n=37, T=16, seed=902)
    say(f"[gpu] long chain F={w.F}, scan chunk {chunk}")
    dev = to_device(w, W.full_storage(w))
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    plan.set_scan_chunk(chunk)
    say(f"  scan chunk frames chosen: {plan.scan_chunk}")
    if chunk != 0:
        assert plan.scan_chunk > 0
    out, _ = run_gpu(w, dev, plan=plan)
    plan.close()
    _check_heads(w, out, [(0, 0), (0, 1)])


def fetch_intermediates(w, plan):
    """The plan's workspace after a synchronised forward pass, as float64 row-major arrays:
    ainv [BH,F+1,d,d], bm [BH,F+1,d,dv], xf, xb [BH,F,d,dv] (layouts in include/vda.h)."""
    import ctypes
    ainv_p, bm_p, xf_p, xb_p = plan.debug_workspace()
    BH, F1, d, dv = w.B * w.H, w.F + 1, w.d, w.dv

    def fetch(ptr, shape, dtype=torch.float32):
        t = torch.empty(shape, dtype=dtype, device="cuda")
        nbytes = t.numel() * t.element_size()
        torch.cuda.synchronize()
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

    def unblock(a):  # [..., d*dv] blocked -> [..., d, dv] row-major
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
        def unfrag_state(u16):  # [c/16][r/32][(r%32)/8][c%16][r%8] -> [r][c]
            a = u16.reshape(BH, w.F, dv // 16, d // 32, 4, 16, 8)
            a = np.transpose(a, (0, 1, 3, 4, 6, 2, 5)).reshape(BH, w.F, d, dv)
            if w.dtype == "fp8" and d >= 64:  # row r is stored at position paired(r)
                r = np.arange(d)
                a = a[:, :, (r & ~0x38) | ((r & 0x08) << 2) | ((r & 0x30) >> 1), :]
            return W.bf16_bits_to_float32(a).astype(np.float64)
        xf = unfrag_state(fetch(xf_p, (BH, w.F, d * dv), torch.int16))
        xb = unfrag_state(fetch(xb_p, (BH, w.F, d * dv), torch.int16))
    return ainv, bm, xf, xb


def check_intermediates(w, ainv, bm, xf, xb):
    """Ainv_f against the oracle's inverse of lam I + K_f^T K_f, Bm_f = K_f^T V_f, and the
    forward/backward states against the oracle's.  Bounds:
      inverse: relative Frobenius error <= e_store + 4 sqrt(d) u kappa(A), the usual error growth
               of a stable float32 inversion (u = 2^-24) at the frame's condition number, plus the
               storage rounding e_store (float32: none; bf16 hi + lo planes: 2^-16);
      Bm:      float32 accumulation of exact products, 1e-5 (float32) or 1e-4 of its largest entry;
      states:  1e-5 (float32) or 1e-4 + 2^-8 (bf16 plans store each state rounded once to bf16).
    Returns (max inverse error / its bound, max kappa, max state error)."""
    d = w.d
    u = 2.0 ** -24
    e_store = 0.0 if w.dtype == "f32" else 2.0 ** -16
    tol = 1e-5 if w.dtype == "f32" else 1e-4
    xtol = tol if w.dtype == "f32" else tol + 2.0 ** -8
    worst_ratio, worst_kappa, worst_x = 0.0, 0.0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            x = W.head_float64(w, b, h)
            i = b * w.H + h
            frames = [(x["text_k"], x["text_v"])] + [(x["k"][f], x["v"][f]) for f in range(w.F)]
            for fi, (K, V) in enumerate(frames):
                G, Bm = oracle.frame_statistics(K, V)
                A = w.lam * np.eye(d) + G
                ref = np.linalg.inv(A)
                kappa = np.linalg.cond(A)
                err = np.linalg.norm(ainv[i, fi] - ref) / np.linalg.norm(ref)
                bound = e_store + 4.0 * np.sqrt(d) * u * kappa
                worst_ratio = max(worst_ratio, err / bound)
                worst_kappa = max(worst_kappa, kappa)
                assert err <= bound, (b, h, fi, err, bound, kappa)
                assert np.abs(bm[i, fi] - Bm).max() <= tol * (1 + np.abs(Bm).max())
            xt, Xf, Xb = oracle.head_states(x["k"], x["v"], x["text_k"], x["text_v"], w.lam)
            for f in range(w.F):
                ef = np.linalg.norm(xf[i, f] - Xf[f]) / np.linalg.norm(Xf[f])
                eb = np.linalg.norm(xb[i, f] - Xb[f]) / np.linalg.norm(Xb[f])
                worst_x = max(worst_x, ef, eb)
                assert ef <= xtol and eb <= xtol, (b, h, f, ef, eb)
    return worst_ratio, worst_kappa, worst_x


INTERMEDIATE_CASES = [
    ("tiny_fp32", W.WORKLOADS[1]),
    ("small_bf16", W.WORKLOADS[2].replace(H=2, F=5, n=200, T=30)),
    ("768p_frames", W.WORKLOADS[3].replace(H=1, F=4, n=300, T=20)),
    ("bf16_32x128", W.WORKLOADS[2].replace(H=1, F=3, n=100, T=8, d=32, dv=128)),
    ("fp8_128", W.WORKLOADS[6].replace(H=1, F=4, n=300, T=20)),
    ("fp8_64x32", W.WORKLOADS[6].replace(H=1, F=3, n=100, T=8, d=64, dv=32)),
    # the ill-conditioned workload's frames at full size: rank-16 keys with 0.05 noise,
    # n = 2016, lam = 0.1 (condition numbers near 2e3), where the explicit inverse is least
    # accurate
    ("ill_conditioned_frames", W.WORKLOADS[5].replace(B=1, H=2, F=4)),
]


@pytest.mark.parametrize("name,w", INTERMEDIATE_CASES, ids=[c[0] for c in INTERMEDIATE_CASES])
def test_intermediates_match_oracle(name, w):
    """Workspace after a forward pass: Ainv_f, Bm_f and the forward/backward states against
    the oracle's."""
    say(f"[gpu] intermediates {name}")
    dev = to_device(w, W.full_storage(w, threads=1))
    out, plan = run_gpu(w, dev)
    ainv, bm, xf, xb = fetch_intermediates(w, plan)
    plan.close()
    ratio, kappa, xerr = check_intermediates(w, ainv, bm, xf, xb)
    say(f"  inverse error at {ratio:.3f} of its bound (max condition number {kappa:.3g}); "
        f"max state error {xerr:.3e}")


# Conditioning range of the explicit inverse and the split-bf16 chain: rank-16 keys at the
# ill-conditioned workload's frame shape (n = 2016, d = dv = 128), lam from the workload's 0.1
# down, and less full-rank noise in the keys (the workload's is 0.05) to go further.  The
# condition number of lam I + K^T K is about 1.7e3 at (0.05, 0.1), 3.8e3 at (0.05, 0.03), 5.8e3
# at (0.05, 0.01), 7.6e3 at (0.05, 0.001) -- the noise floor of K^T K bounds it near 8e3 -- then
# 3.9e4 at (0.02, 0.001), 1.0e5 at (0.01, 0.001) and 5.5e5 at (0.005, 1e-4).
_BEYOND = ("outside the verified conditioning range: the float32 inverse and the split-bf16 chain "
           "keep the 1e-2 bar up to condition numbers near 1e4 (5.2e-3 at 8.2e3); measured on one "
           "MI355X at this case: ")
CONDITIONING = [
    (0.05, 0.1), (0.05, 0.03), (0.05, 0.01), (0.05, 0.001),
    pytest.param(0.02, 0.001, marks=pytest.mark.skip(reason=_BEYOND + "condition number 4.3e4, error 2.0e-2")),
    pytest.param(0.01, 0.001, marks=pytest.mark.skip(reason=_BEYOND + "condition number 1.1e5, error 1.0e-1")),
    pytest.param(0.005, 1e-4, marks=pytest.mark.skip(reason=_BEYOND + "condition number 5.7e5, error 8.4e-1")),
]


@pytest.mark.parametrize("noise,lam", CONDITIONING,
                         ids=["noise0.05_lam0.1", "noise0.05_lam0.03", "noise0.05_lam0.01", "noise0.05_lam0.001",
                              "noise0.02_lam0.001", "noise0.01_lam0.001", "noise0.005_lam0.0001"])
def test_conditioning_range(noise, lam):
    w = W.WORKLOADS[5].replace(name=f"lowrank_noise{noise}_lam{lam}", B=1, H=2, F=6, T=64, seed=500,
                               lam=lam, noise=noise)
    say(f"[gpu] conditioning noise={noise} lam={lam}")
    arrays = W.full_storage(w, threads=1)
    out, plan = run_gpu(w, to_device(w, arrays))
    plan.close()
    kappa = 0.0
    for h in range(w.H):
        x = W.head_float64(w, 0, h)
        for f in range(w.F):
            kappa = max(kappa, np.linalg.cond(lam * np.eye(w.d) + x["k"][f].T @ x["k"][f]))
    say(f"  noise={noise} lam={lam}: max condition number {kappa:.3g}")
    _check_heads(w, out, [(0, h) for h in range(w.H)])


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
