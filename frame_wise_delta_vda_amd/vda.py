"""Python binding of the VDA C ABI (include/vda.h): argument marshalling only.

Each ``vda_*`` function mirrors the C call of the same name.  Tensors are passed as
device pointers (torch tensors or plain ints); every step of the computation runs
in the HIP library.  There is no fallback: if libvda.so is missing, importing the
binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("VDA_LIBRARY", os.path.join(HERE, "libvda.so"))
HEADER = os.path.join(os.path.dirname(HERE), "include", "vda.h")

VDA_DTYPE_F32, VDA_DTYPE_BF16, VDA_DTYPE_FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": VDA_DTYPE_F32, "bf16": VDA_DTYPE_BF16, "fp8": VDA_DTYPE_FP8_E4M3}
STATUS = {0: "VDA_SUCCESS", 1: "VDA_ERROR_INVALID_VALUE", 2: "VDA_ERROR_NOT_SUPPORTED",
          3: "VDA_ERROR_MISALIGNED", 4: "VDA_ERROR_OUT_OF_MEMORY", 5: "VDA_ERROR_DEVICE",
          6: "VDA_ERROR_TOO_LARGE"}
VDA_SUCCESS, VDA_ERROR_INVALID_VALUE, VDA_ERROR_NOT_SUPPORTED = 0, 1, 2
VDA_ERROR_MISALIGNED, VDA_ERROR_OUT_OF_MEMORY, VDA_ERROR_DEVICE = 3, 4, 5
VDA_ERROR_TOO_LARGE = 6
VDA_NOALLOC_SCRATCH_BYTES = 64 << 20
VDA_SCAN_CHUNK_AUTO = -1
VDA_STAGE_STATS, VDA_STAGE_SCAN, VDA_STAGE_READOUT, VDA_STAGE_ALL = 1, 2, 4, 7


class VdaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}" if what else STATUS.get(status, str(status)))


_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libvda.so (built by frame_wise_delta_vda_amd.build) and declare its C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    try:  # share the HIP runtime torch loads (same soname), whatever the import order
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise RuntimeError(f"libvda.so not found at {p}; run `python -m frame_wise_delta_vda_amd.build`")
    lib = ctypes.CDLL(p)
    c_i64, c_vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.vda_plan_create.argtypes = [c_i64] * 7 + [ctypes.c_float, c_int, ctypes.POINTER(c_vp)]
    lib.vda_plan_create.restype = c_int
    lib.vda_forward.argtypes = [c_vp] * 8
    lib.vda_forward.restype = c_int
    lib.vda_forward_gated.argtypes = [c_vp] * 11
    lib.vda_forward_gated.restype = c_int
    lib.vda_backward.argtypes = [c_vp] * 13
    lib.vda_backward.restype = c_int
    lib.vda_forward_stages.argtypes = [c_vp, ctypes.c_uint] + [c_vp] * 7
    lib.vda_forward_stages.restype = c_int
    lib.vda_plan_destroy.argtypes = [c_vp]
    lib.vda_plan_destroy.restype = c_int
    lib.vda_plan_workspace_bytes.argtypes = [c_vp]
    lib.vda_plan_workspace_bytes.restype = ctypes.c_size_t
    lib.vda_status_string.argtypes = [c_int]
    lib.vda_status_string.restype = ctypes.c_char_p
    fp = ctypes.POINTER(ctypes.c_void_p)
    lib.vda_debug_workspace.argtypes = [c_vp, fp, fp, fp, fp]
    lib.vda_debug_workspace.restype = c_int
    lib.vda_plan_enable_timing.argtypes = [c_vp, c_int]
    lib.vda_plan_enable_timing.restype = c_int
    flp = ctypes.POINTER(ctypes.c_float)
    lib.vda_plan_timings.argtypes = [c_vp, ctypes.POINTER(c_int), flp, flp, flp]
    lib.vda_plan_timings.restype = c_int
    lib.vda_forward_noalloc.argtypes = [c_i64] * 7 + [ctypes.c_float, c_int] + [c_vp] * 7
    lib.vda_forward_noalloc.restype = c_int
    lib.vda_plan_set_scan_chunk.argtypes = [c_vp, c_i64]
    lib.vda_plan_set_scan_chunk.restype = c_int
    lib.vda_plan_get_scan_chunk.argtypes = [c_vp, ctypes.POINTER(c_i64)]
    lib.vda_plan_get_scan_chunk.restype = c_int
    lib.vda_plan_set_timed_stages.argtypes = [c_vp, ctypes.c_uint]
    lib.vda_plan_set_timed_stages.restype = c_int
    if path is None:
        _lib = lib
    return lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/vda.h declares."""
    with open(header) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(vda_[a-z_]+)\s*\(", text)))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != VDA_SUCCESS:
        raise VdaError(status, what)


def vda_status_string(status: int) -> str:
    return load_library().vda_status_string(status).decode()


def vda_plan_create(B, H, F, n, d, dv, T, lam, dtype) -> int:
    """Returns the plan handle (an int).  dtype: a VDA_DTYPE_* value or "f32", "bf16", "fp8"."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    h = ctypes.c_void_p()
    _check(load_library().vda_plan_create(B, H, F, n, d, dv, T, ctypes.c_float(lam), dtype,
                                          ctypes.byref(h)), "vda_plan_create")
    return h.value


def vda_forward(plan, q, k, v, text_k, text_v, out, stream=None):
    _check(load_library().vda_forward(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(text_k), _ptr(text_v),
                                      _ptr(out), _stream(stream)), "vda_forward")


def vda_forward_noalloc(B, H, F, n, d, dv, T, lam, dtype, q, k, v, text_k, text_v, out, stream=None):
    """The forward pass with no plan and no device allocation (include/vda.h)."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    _check(load_library().vda_forward_noalloc(B, H, F, n, d, dv, T, ctypes.c_float(lam), dtype, _ptr(q), _ptr(k),
                                              _ptr(v), _ptr(text_k), _ptr(text_v), _ptr(out), _stream(stream)),
           "vda_forward_noalloc")


def vda_forward_gated(plan, q, k, v, text_k, text_v, w_gate, b_gate, w_out, out, stream=None):
    _check(load_library().vda_forward_gated(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(text_k), _ptr(text_v),
                                            _ptr(w_gate), _ptr(b_gate), _ptr(w_out), _ptr(out),
                                            _stream(stream)), "vda_forward_gated")


def vda_backward(plan, q, k, v, text_k, text_v, d_out, d_q, d_k, d_v, d_text_k, d_text_v, stream=None):
    _check(load_library().vda_backward(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(text_k), _ptr(text_v),
                                       _ptr(d_out), _ptr(d_q), _ptr(d_k), _ptr(d_v), _ptr(d_text_k),
                                       _ptr(d_text_v), _stream(stream)), "vda_backward")


def vda_forward_stages(plan, stages, q, k, v, text_k, text_v, out, stream=None):
    _check(load_library().vda_forward_stages(plan, stages, _ptr(q), _ptr(k), _ptr(v), _ptr(text_k),
                                             _ptr(text_v), _ptr(out), _stream(stream)),
           "vda_forward_stages")


def vda_plan_set_scan_chunk(plan, chunk_frames: int):
    """0: serial scans; > 0: the chunked scan with chunks of that many frames;
    VDA_SCAN_CHUNK_AUTO: the plan's own choice (include/vda.h)."""
    _check(load_library().vda_plan_set_scan_chunk(plan, chunk_frames), "vda_plan_set_scan_chunk")


def vda_plan_get_scan_chunk(plan) -> int:
    c = ctypes.c_int64()
    _check(load_library().vda_plan_get_scan_chunk(plan, ctypes.byref(c)), "vda_plan_get_scan_chunk")
    return c.value


def vda_plan_destroy(plan):
    _check(load_library().vda_plan_destroy(plan), "vda_plan_destroy")


def vda_plan_workspace_bytes(plan) -> int:
    return int(load_library().vda_plan_workspace_bytes(plan))


def vda_debug_workspace(plan):
    """Device addresses (ainv, bm, x_fwd, x_bwd) in the plan's workspace (layouts: include/vda.h)."""
    ptrs = [ctypes.c_void_p() for _ in range(4)]
    _check(load_library().vda_debug_workspace(plan, *[ctypes.byref(p) for p in ptrs]),
           "vda_debug_workspace")
    return tuple(p.value for p in ptrs)


def vda_plan_enable_timing(plan, capacity: int):
    _check(load_library().vda_plan_enable_timing(plan, capacity), "vda_plan_enable_timing")


def vda_plan_set_timed_stages(plan, stages: int):
    _check(load_library().vda_plan_set_timed_stages(plan, stages), "vda_plan_set_timed_stages")


def vda_plan_timings(plan):
    """(calls, stats_ms, scan_ms, readout_ms) of the timed whole passes since the last read."""
    calls = ctypes.c_int()
    ms = [ctypes.c_float() for _ in range(3)]
    _check(load_library().vda_plan_timings(plan, ctypes.byref(calls), *[ctypes.byref(m) for m in ms]),
           "vda_plan_timings")
    return (calls.value,) + tuple(m.value for m in ms)


class Plan:
    """Owns one vda plan; `forward` takes torch tensors in the documented layouts."""

    def __init__(self, B, H, F, n, d, dv, T, lam, dtype="bf16"):
        self.shape = dict(B=B, H=H, F=F, n=n, d=d, dv=dv, T=T)
        self.lam = lam
        self.dtype = dtype
        self.handle = vda_plan_create(B, H, F, n, d, dv, T, lam, dtype)

    def close(self):
        if self.handle:
            vda_plan_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def workspace_bytes(self) -> int:
        return vda_plan_workspace_bytes(self.handle)

    def out_like(self, q):
        """Output tensor for inputs like q: float32 for float32 plans, else bfloat16."""
        import torch
        s = self.shape
        dt = torch.float32 if self.dtype in ("f32", VDA_DTYPE_F32) else torch.bfloat16
        return torch.empty((s["B"], s["H"], s["F"], s["n"], s["dv"]), dtype=dt, device=q.device)

    def forward(self, q, k, v, text_k, text_v, out=None, stream=None):
        if out is None:
            out = self.out_like(q)
        vda_forward(self.handle, q, k, v, text_k, text_v, out, stream)
        return out

    def forward_gated(self, q, k, v, text_k, text_v, w_gate, b_gate, w_out, out=None, stream=None):
        """The forward pass followed by the gated epilogue (include/vda.h, vda_forward_gated)."""
        if out is None:
            out = self.out_like(q)
        vda_forward_gated(self.handle, q, k, v, text_k, text_v, w_gate, b_gate, w_out, out, stream)
        return out

    def backward(self, q, k, v, text_k, text_v, d_out, grads=None, stream=None):
        """Gradients (dq, dk, dv, d_text_k, d_text_v) of sum(d_out * O) after a forward call on
        the same inputs (include/vda.h, vda_backward).  grads: optional output tensors."""
        import torch
        if grads is None:
            grads = tuple(torch.empty_like(t) if t is not None else None for t in (q, k, v, text_k, text_v))
        vda_backward(self.handle, q, k, v, text_k, text_v, d_out, *grads, stream=stream)
        return grads

    def stages(self, stages, q=None, k=None, v=None, text_k=None, text_v=None, out=None, stream=None):
        vda_forward_stages(self.handle, stages, q, k, v, text_k, text_v, out, stream)
        return out

    def debug_workspace(self):
        return vda_debug_workspace(self.handle)

    def set_scan_chunk(self, chunk_frames: int):
        vda_plan_set_scan_chunk(self.handle, chunk_frames)

    @property
    def scan_chunk(self) -> int:
        """Frames per chunk of the chunked scan, 0 for the serial scan."""
        return vda_plan_get_scan_chunk(self.handle)

    def enable_timing(self, capacity: int):
        vda_plan_enable_timing(self.handle, capacity)

    def set_timed_stages(self, stages: int):
        vda_plan_set_timed_stages(self.handle, stages)

    def timings(self):
        return vda_plan_timings(self.handle)
