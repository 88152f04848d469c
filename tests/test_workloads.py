"""The seeded input generator (CPU only): determinism, rounding, recipe."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0], np.float32)])
    ours = W.float32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_float32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_slices_are_deterministic_and_independent_of_threads():
    w = W.WORKLOADS[2].replace(H=3, F=2, n=50, T=5)
    a = W.full_storage(w, threads=1)
    b = W.full_storage(w, threads=3)
    for key in W.TENSORS:
        assert np.array_equal(a[key], b[key])
    one = W.head_storage(w, 0, 2)
    for key in W.TENSORS:
        assert np.array_equal(a[key][0, 2], one[key])
    assert not np.array_equal(a["q"][0, 0], a["q"][0, 1])


def test_keys_are_unit_rows_and_dtypes():
    for idx in (1, 5):
        w = W.WORKLOADS[idx].replace(B=1, H=1, F=2, n=40)
        s = W.head_storage(w, 0, 0)
        assert s["q"].dtype == (np.float32 if w.dtype == "f32" else np.uint16)
        k = W.storage_to_float64(w, s["k"])
        tol = 1e-6 if w.dtype == "f32" else 1e-2
        assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=tol)
        assert np.allclose(np.linalg.norm(W.storage_to_float64(w, s["text_k"]), axis=-1), 1.0, atol=tol)


def test_lowrank_keys_are_nearly_rank_r():
    w = W.WORKLOADS[5].replace(B=1, H=1, F=1, n=400)
    k = W.head_float32(w, 0, 0)["k"][0].astype(np.float64)
    s = np.linalg.svd(k, compute_uv=False)
    assert s[15] > 5 * s[16]          # rank-16 signal well above the 0.05 noise


def test_shapes_and_algorithmic_bytes():
    w = W.WORKLOADS[3]
    assert w.shapes()["q"] == (1, 24, 90, 4032, 128)
    assert w.video_tokens == 362880
    assert w.algorithmic_bytes() == (24 * (90 * 4032 * 512 + 256 * 256)) * 2
