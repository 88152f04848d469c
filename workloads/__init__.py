"""Seeded synthetic inputs for the Video Delta Attention (VDA) forward pass.

This module is shared by the oracle side (tests, the CPU baseline) and the GPU
side (tests, bench).  It holds only the input recipe -- shapes, random draws,
key normalisation and rounding to the storage type -- and none of the VDA
arithmetic itself.

Workloads.  The pages measure a 768p, 14.4 s clip (VDN-MiniMax-H3 pages, the
"performance numbers" table of the agentlenshq project page and the results
section of the model card).  No dataset, prompt or weight is used: every input
is Gaussian noise of the shape of that workload, drawn from a seed.

Recipe, per (batch b, head h), from ``Generator(PCG64(SeedSequence((seed, b, h))))``
with ``seed`` the workload's seed; all draws are float32 in this order:

* gaussian workloads:  q ~ N(0,1) [F,n,d];  k ~ N(0,1) [F,n,d];  v ~ N(0,1) [F,n,dv];
  text_k ~ N(0,1) [T,d];  text_v ~ N(0,1) [T,dv].
* low-rank ("ill-conditioned") workloads:  m ~ N(0,1) [dv,d] once per (b,h); then per
  frame f = 0..F-1 in order: u_f ~ N(0,1) [n,r], w_f ~ N(0,1) [r,d], e_f ~ N(0,1) [n,d],
  z_f ~ N(0,1) [n,dv], with k_f = rownorm(u_f w_f / sqrt(r) + s e_f) (s = 0.05 unless a
  workload states another noise level) and
  v_f = k_f m^T + 0.1 z_f (float32, before any rounding); then q ~ N(0,1) [F,n,d],
  text_k ~ N(0,1) [T,d], text_v ~ N(0,1) [T,dv].

Every row of k and text_k is scaled to unit L2 norm in float32.  For bfloat16
workloads every tensor is then rounded to bfloat16 with round-to-nearest-even; for
fp8 workloads the inputs are rounded to OCP FP8 e4m3 (round-to-nearest-even, magnitudes
above 448 saturate to 448) and the output is bfloat16.  The oracle receives the rounded
values upcast exactly.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

TENSORS = ("q", "k", "v", "text_k", "text_v")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic VDA input set."""
    name: str
    B: int
    H: int
    F: int
    n: int
    d: int
    dv: int
    T: int
    lam: float
    dtype: str            # "f32", "bf16" or "fp8": storage type of q,k,v,text_k,text_v
    seed: int
    kind: str = "gaussian"  # "gaussian" or "lowrank"
    rank: int = 16
    noise: float = 0.05     # low-rank workloads: relative size of the full-rank noise in k
    grid: Optional[tuple] = None  # spatial token grid (rows, cols), informational

    @property
    def video_tokens(self) -> int:
        return self.B * self.F * self.n

    @property
    def elem_bytes(self) -> int:
        """Bytes per input element."""
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def out_bytes(self) -> int:
        """Bytes per output element: float32 for float32 workloads, else bfloat16."""
        return 4 if self.dtype == "f32" else 2

    def shapes(self) -> Dict[str, tuple]:
        B, H, F, n, d, dv, T = self.B, self.H, self.F, self.n, self.d, self.dv, self.T
        return {"q": (B, H, F, n, d), "k": (B, H, F, n, d), "v": (B, H, F, n, dv),
                "text_k": (B, H, T, d), "text_v": (B, H, T, dv), "out": (B, H, F, n, dv)}

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: q, k, v, text read once and out written once."""
        B, H, F, n, d, dv, T = self.B, self.H, self.F, self.n, self.d, self.dv, self.T
        inputs = B * H * (F * n * (2 * d + dv) + T * (d + dv))
        return inputs * self.elem_bytes + B * H * F * n * dv * self.out_bytes

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five named workloads.  Index = seed.
WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_fp32", B=1, H=2, F=6, n=64, d=32, dv=32, T=16, lam=1.0,
                dtype="f32", seed=1, grid=(8, 8)),
    2: Workload("small_bf16", B=1, H=8, F=24, n=1024, d=64, dv=64, T=64, lam=1.0,
                dtype="bf16", seed=2, grid=(32, 32)),
    3: Workload("768p_bf16", B=1, H=24, F=90, n=4032, d=128, dv=128, T=256, lam=1.0,
                dtype="bf16", seed=3, grid=(84, 48)),
    4: Workload("long_clip_bf16", B=1, H=24, F=360, n=1024, d=128, dv=128, T=256, lam=1.0,
                dtype="bf16", seed=4, grid=(32, 32)),
    5: Workload("ill_conditioned_bf16", B=4, H=16, F=45, n=2016, d=128, dv=128, T=128,
                lam=0.1, dtype="bf16", seed=5, kind="lowrank", rank=16, grid=(56, 36)),
    # the 768p shape with FP8 (e4m3) inputs and a bfloat16 output
    6: Workload("768p_fp8", B=1, H=24, F=90, n=4032, d=128, dv=128, T=256, lam=1.0,
                dtype="fp8", seed=6, grid=(84, 48)),
    # one GPU's share of the 768p and long-clip shapes when 8 GPUs split the 24 heads: 3 heads
    # each, every frame (the shape a head-sharded layout gives each GPU)
    7: Workload("768p_shard8_bf16", B=1, H=3, F=90, n=4032, d=128, dv=128, T=256, lam=1.0,
                dtype="bf16", seed=7, grid=(84, 48)),
    8: Workload("long_clip_shard8_bf16", B=1, H=3, F=360, n=1024, d=128, dv=128, T=256, lam=1.0,
                dtype="bf16", seed=8, grid=(32, 32)),
}


def by_name(name: str) -> Workload:
    for w in WORKLOADS.values():
        if w.name == name:
            return w
    raise KeyError(name)


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (pure data conversion)
# ----------------------------------------------------------------------------

def float32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the uint16 bits.
    Inputs here are finite, so no NaN special case is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# FP8 e4m3 storage helpers (OCP 8-bit format: 1 sign bit, 4 exponent bits with bias 7,
# 3 mantissa bits; subnormals below 2^-6; no infinities; S.1111.111 is NaN; the largest
# finite magnitude is 448)
# ----------------------------------------------------------------------------

def float32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round to e4m3, to nearest with ties to even; magnitudes above 448 saturate to 448.
    Inputs here are finite.  Returns the uint8 codes."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    neg = np.signbit(x)
    # binade of a (normal range 2^-6 .. 2^8; below 2^-6 the subnormal quantum 2^-9 applies)
    e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6, 8)
    quantum = np.exp2(e - 3)
    r = np.minimum(np.round(a / quantum) * quantum, 448.0)  # np.round: ties to even
    e2 = np.clip(np.floor(np.log2(np.where(r > 0, r, 1.0))), -6, 8)
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, e2 + 7, 0)
    man_field = np.where(normal, r / np.exp2(e2) * 8 - 8, r / 2.0 ** -9)
    code = (neg.astype(np.uint32) << 7) | (exp_field.astype(np.uint32) << 3) | man_field.astype(np.uint32)
    return code.astype(np.uint8)


def e4m3_codes_to_float32(c: np.ndarray) -> np.ndarray:
    """Exact value of e4m3 codes as float32 (NaN for the NaN codes)."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return (s * v).astype(np.float32)


def _rownorm(x: np.ndarray) -> np.ndarray:
    nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    return (x / nrm).astype(np.float32)


def _rng(w: Workload, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((w.seed, b, h))))


def head_float32(w: Workload, b: int, h: int) -> Dict[str, np.ndarray]:
    """Draw the float32 tensors of one (b,h) slice, before rounding to storage."""
    g = _rng(w, b, h)
    F, n, d, dv, T = w.F, w.n, w.d, w.dv, w.T
    if w.kind == "gaussian":
        q = g.standard_normal((F, n, d), dtype=np.float32)
        k = _rownorm(g.standard_normal((F, n, d), dtype=np.float32))
        v = g.standard_normal((F, n, dv), dtype=np.float32)
    elif w.kind == "lowrank":
        m = g.standard_normal((dv, d), dtype=np.float32)
        k = np.empty((F, n, d), np.float32)
        v = np.empty((F, n, dv), np.float32)
        scale = np.float32(1.0 / np.sqrt(w.rank))
        for f in range(F):
            u = g.standard_normal((n, w.rank), dtype=np.float32)
            wf = g.standard_normal((w.rank, d), dtype=np.float32)
            e = g.standard_normal((n, d), dtype=np.float32)
            z = g.standard_normal((n, dv), dtype=np.float32)
            kf = _rownorm((u @ wf) * scale + np.float32(w.noise) * e)
            k[f] = kf
            v[f] = kf @ m.T + np.float32(0.1) * z
        q = g.standard_normal((F, n, d), dtype=np.float32)
    else:
        raise ValueError(w.kind)
    tk = _rownorm(g.standard_normal((T, d), dtype=np.float32)) if T > 0 else np.zeros((0, d), np.float32)
    tv = g.standard_normal((T, dv), dtype=np.float32)
    return {"q": q, "k": k, "v": v, "text_k": tk, "text_v": tv}


def to_storage(w: Workload, x: np.ndarray) -> np.ndarray:
    """float32 -> storage array (float32, uint16 bfloat16 bits or uint8 e4m3 codes)."""
    if w.dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if w.dtype == "fp8":
        return float32_to_e4m3_codes(x)
    return float32_to_bf16_bits(x)


def storage_to_float64(w: Workload, s: np.ndarray) -> np.ndarray:
    """Storage array -> the exact values as float64 (what the oracle receives)."""
    if w.dtype == "f32":
        return np.asarray(s, dtype=np.float32).astype(np.float64)
    if w.dtype == "fp8":
        return e4m3_codes_to_float32(s).astype(np.float64)
    return bf16_bits_to_float32(s).astype(np.float64)


def head_storage(w: Workload, b: int, h: int) -> Dict[str, np.ndarray]:
    """One (b,h) slice in storage form."""
    return {key: to_storage(w, val) for key, val in head_float32(w, b, h).items()}


def head_float64(w: Workload, b: int, h: int) -> Dict[str, np.ndarray]:
    """One (b,h) slice as the exact float64 values of its stored inputs."""
    return {key: storage_to_float64(w, val) for key, val in head_storage(w, b, h).items()}


def storage_dtype(w: Workload):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[w.dtype]


def full_storage(w: Workload, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All (b,h) slices, in storage form, shaped [B,H,...].  Slices are generated on a
    thread pool; each slice uses its own generator, so the result does not depend on
    the number of threads."""
    shapes = w.shapes()
    out = {key: np.empty(shapes[key], storage_dtype(w)) for key in TENSORS}
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))

    def fill(bh):
        b, h = bh
        for key, val in head_storage(w, b, h).items():
            out[key][b, h] = val

    jobs = [(b, h) for b in range(w.B) for h in range(w.H)]
    if threads <= 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, jobs))
    return out


# ----------------------------------------------------------------------------
# Synthetic weights of the gated fusion epilogue (per head, shared by the batch)
# ----------------------------------------------------------------------------

def gate_weights(w: Workload) -> Dict[str, np.ndarray]:
    """Seeded gate and output-projection weights, [output feature][input feature] like a
    torch Linear weight: w_gate, w_out [H, dv, dv] ~ N(0, 1/dv), b_gate [H, dv] ~ N(0, 1).
    The matrices are stored as bfloat16 bits for bfloat16 and FP8 workloads (float32 for
    float32 workloads); the bias is float32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((w.seed, 0x6A7E))))
    scale = np.float32(1.0 / np.sqrt(w.dv))
    wg = rng.standard_normal((w.H, w.dv, w.dv), dtype=np.float32) * scale
    wo = rng.standard_normal((w.H, w.dv, w.dv), dtype=np.float32) * scale
    bg = rng.standard_normal((w.H, w.dv), dtype=np.float32)
    if w.dtype != "f32":
        wg, wo = float32_to_bf16_bits(wg), float32_to_bf16_bits(wo)
    return {"w_gate": wg, "b_gate": bg, "w_out": wo}


def gate_weights_float64(w: Workload, g: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """The stored gate weights as exact float64 values."""
    dec = (lambda a: np.asarray(a, np.float32)) if w.dtype == "f32" else bf16_bits_to_float32
    return {"w_gate": dec(g["w_gate"]).astype(np.float64), "w_out": dec(g["w_out"]).astype(np.float64),
            "b_gate": np.asarray(g["b_gate"], np.float32).astype(np.float64)}
