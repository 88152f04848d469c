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


# ---- OCP FP8 E4M3 storage (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
# infinities; S.1111.111 is NaN; largest finite magnitude 448)

def test_e4m3_known_codes():
    codes = np.array([0x00, 0x80, 0x38, 0x7E, 0xFE, 0x01, 0x07, 0x08, 0xC0, 0x3C, 0x77], np.uint8)
    want = [0.0, -0.0, 1.0, 448.0, -448.0, 2.0**-9, 7 * 2.0**-9, 2.0**-6, -2.0, 1.5, 240.0]
    got = W.e4m3_codes_to_float32(codes)
    assert got.tolist() == want
    assert np.signbit(got[1])
    assert np.isnan(W.e4m3_codes_to_float32(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_codes_increase_with_value():
    pos = W.e4m3_codes_to_float32(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()
    neg = W.e4m3_codes_to_float32(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_e4m3_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(W.float32_to_e4m3_codes(W.e4m3_codes_to_float32(codes)), codes)


def test_e4m3_rounding_ties_to_even_and_saturates():
    x = np.array([1.0625, 1.1875, 2.0**-10, 3 * 2.0**-10, 15.5, 0.0, -0.0,
                  448.0, 463.9, 464.0, 500.0, -1000.0], np.float32)
    got = W.e4m3_codes_to_float32(W.float32_to_e4m3_codes(x))
    assert got.tolist() == [1.0, 1.25, 0.0, 2.0**-8, 16.0, 0.0, 0.0, 448.0, 448.0, 448.0, 448.0, -448.0]
    assert np.signbit(got[6])


def test_e4m3_rounding_matches_torch_float8_e4m3fn():
    # torch's conversion rounds to nearest even as well (it turns overflow into NaN, so the
    # comparison stays below 448 + half a step)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-14, 9, 100000))).astype(np.float32)
    x = x[np.abs(x) < 460]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(W.float32_to_e4m3_codes(x), ref)


def test_fp8_workload_storage_and_bytes():
    w = W.by_name("768p_fp8")
    assert (w.elem_bytes, w.out_bytes) == (1, 2)
    assert w.algorithmic_bytes() == 24 * (90 * 4032 * 384 + 256 * 256) + 24 * 90 * 4032 * 128 * 2
    s = W.head_storage(w.replace(F=2, n=40, T=8), 0, 0)
    assert s["q"].dtype == np.uint8
    k = W.storage_to_float64(w, s["k"])
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=0.1)  # 3-bit mantissa
    assert np.array_equal(W.float32_to_e4m3_codes(k.astype(np.float32)), s["k"])
