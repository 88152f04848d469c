// C ABI of the VDA forward library: plans, argument checks, stage dispatch.
// The operation and the layouts are documented in include/vda.h.
#include "vda.h"
#include "vda_internal.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>

struct vda_plan_s {
  vda::Problem p;
  int device;
  void* workspace;
  size_t workspace_bytes;
  // Per-stage timing of whole passes: kTimingEvents events per call in a ring of
  // timing_capacity calls; timed_calls counts the calls recorded since the last read.
  int timing_capacity;
  int timed_calls;
  unsigned timed_stages;  // stages whose kernels record their events (vda_plan_set_timed_stages)
  hipEvent_t* timing_events;
  // backward-pass workspace, allocated by the first vda_backward call
  void* bwd_workspace;
  size_t bwd_workspace_bytes;
  // set once a forward pass (whole, or its statistics stage) has been enqueued: the backward
  // pass reads the statistics it leaves in the workspace
  bool has_statistics;
  // the chunked scan's workspace (vda_plan_set_scan_chunk)
  void* chunk_workspace;
  size_t chunk_workspace_bytes;
};

namespace {
// Event slots of one timed call: begin and end of each stage.
enum { kEvStatsBegin, kEvStatsEnd, kEvScanBegin, kEvScanEnd, kEvReadBegin, kEvReadEnd,
       kTimingEvents };

void free_timing(vda_plan_s* plan) {
  for (int i = 0; i < plan->timing_capacity * kTimingEvents; ++i)
    if (plan->timing_events[i] != nullptr) (void)hipEventDestroy(plan->timing_events[i]);
  delete[] plan->timing_events;
  plan->timing_events = nullptr;
  plan->timing_capacity = 0;
  plan->timed_calls = 0;
}
}  // namespace

namespace {

bool supported_width(int64_t x) { return x == 32 || x == 64 || x == 128; }

// a*b into *out; false on overflow of the positive int64 range.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_mul_overflow(a, b, out) && *out >= 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

}  // namespace

namespace vda {

vda_status make_problem(int64_t B, int64_t H, int64_t F, int64_t n, int64_t d, int64_t dv, int64_t T,
                        float lambda, vda_dtype dtype, Problem* out, size_t* workspace_bytes) {
  if (B < 0 || H < 0 || F < 0 || n < 0 || T < 0) return VDA_ERROR_INVALID_VALUE;
  if (!(std::isfinite(lambda) && lambda > 0.0f)) return VDA_ERROR_INVALID_VALUE;
  if (dtype != VDA_DTYPE_F32 && dtype != VDA_DTYPE_BF16 && dtype != VDA_DTYPE_FP8_E4M3)
    return VDA_ERROR_NOT_SUPPORTED;
  if (!supported_width(d) || !supported_width(dv)) return VDA_ERROR_NOT_SUPPORTED;
  // a frame (or the text) is addressed with 32-bit byte offsets
  if (n > kMaxFrameTokens || T > kMaxFrameTokens) return VDA_ERROR_NOT_SUPPORTED;

  // Every element count the kernels index must fit in int64; grids are 1-D.  F + 1 (the frames
  // with the text) must itself fit.
  int64_t bh, frames, tok, elems, ws_frames, ws_elems, tmp, f1;
  if (__builtin_add_overflow(F, int64_t(1), &f1)) return VDA_ERROR_INVALID_VALUE;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, f1, &ws_frames) || !mul_ok(bh, F, &frames) ||
      !mul_ok(frames, n, &tok) || !mul_ok(tok, 128, &elems) || !mul_ok(bh, T, &tmp) ||
      !mul_ok(tmp, 128, &tmp))
    return VDA_ERROR_INVALID_VALUE;
  if (ws_frames > (int64_t(1) << 30)) return VDA_ERROR_INVALID_VALUE;
  // ainv + bm over F+1 frames, xf + xb over F frames; each block <= 128*128 floats
  if (!mul_ok(ws_frames, d * d + d * dv, &ws_elems) || !mul_ok(frames, 2 * d * dv, &tmp) ||
      __builtin_add_overflow(ws_elems, tmp, &ws_elems) || !mul_ok(ws_elems, 4, &tmp))
    return VDA_ERROR_INVALID_VALUE;
  (void)elems;

  Problem p{};
  p.B = B; p.H = H; p.F = F; p.n = n; p.d = d; p.dv = dv; p.T = T;
  p.lam = lambda;
  p.bf16 = (dtype != VDA_DTYPE_F32);  // FP8 inputs run the bfloat16 path after conversion
  p.fp8 = (dtype == VDA_DTYPE_FP8_E4M3);
  p.states_f32 = false;
  p.bm_only = false;
  p.num_cus = 0;
  p.ainv = p.bm = p.xf = p.xb = nullptr;
  const size_t ainv_n = size_t(ws_frames) * d * d;
  const size_t bm_n = size_t(ws_frames) * d * dv;
  // states: float32 for float32 plans; bfloat16 (half the bytes) for the others
  const size_t x_n = size_t(frames) * d * dv / (p.bf16 ? 2 : 1);
  *workspace_bytes = (ainv_n + bm_n + 2 * x_n) * sizeof(float);
  *out = p;
  return VDA_SUCCESS;
}

void carve_workspace(Problem& p, void* base) {
  const size_t ws_frames = size_t(p.B) * size_t(p.H) * size_t(p.F + 1);
  const size_t frames = size_t(p.B) * size_t(p.H) * size_t(p.F);
  const size_t ainv_n = ws_frames * size_t(p.d) * size_t(p.d);
  const size_t bm_n = ws_frames * size_t(p.d) * size_t(p.dv);
  const size_t x_n = frames * size_t(p.d) * size_t(p.dv) / (p.bf16 ? 2 : 1);
  float* f = static_cast<float*>(base);
  p.ainv = f;
  p.bm = p.ainv + ainv_n;
  p.xf = p.bm + bm_n;
  p.xb = p.xf + x_n;
}

}  // namespace vda

extern "C" {

const char* vda_status_string(vda_status s) {
  switch (s) {
    case VDA_SUCCESS: return "VDA_SUCCESS";
    case VDA_ERROR_INVALID_VALUE: return "VDA_ERROR_INVALID_VALUE";
    case VDA_ERROR_NOT_SUPPORTED: return "VDA_ERROR_NOT_SUPPORTED";
    case VDA_ERROR_MISALIGNED: return "VDA_ERROR_MISALIGNED";
    case VDA_ERROR_OUT_OF_MEMORY: return "VDA_ERROR_OUT_OF_MEMORY";
    case VDA_ERROR_DEVICE: return "VDA_ERROR_DEVICE";
    case VDA_ERROR_TOO_LARGE: return "VDA_ERROR_TOO_LARGE";
  }
  return "VDA_ERROR_UNKNOWN";
}

vda_status vda_plan_create(int64_t B, int64_t H, int64_t F, int64_t n, int64_t d, int64_t dv,
                           int64_t T, float lambda, vda_dtype dtype, vda_plan_t* plan_out) {
  if (plan_out == nullptr) return VDA_ERROR_INVALID_VALUE;
  *plan_out = nullptr;
  vda::Problem shape;
  size_t total = 0;
  const vda_status st = vda::make_problem(B, H, F, n, d, dv, T, lambda, dtype, &shape, &total);
  if (st != VDA_SUCCESS) return st;

  vda_plan_s* plan = new (std::nothrow) vda_plan_s();
  if (plan == nullptr) return VDA_ERROR_OUT_OF_MEMORY;
  if (hipGetDevice(&plan->device) != hipSuccess) {
    (void)hipGetLastError();
    delete plan;
    return VDA_ERROR_DEVICE;
  }
  vda::Problem& p = plan->p;
  p = shape;
  if (hipDeviceGetAttribute(&p.num_cus, hipDeviceAttributeMultiprocessorCount, plan->device) !=
          hipSuccess ||
      p.num_cus <= 0) {
    (void)hipGetLastError();
    delete plan;
    return VDA_ERROR_DEVICE;
  }
  plan->workspace = nullptr;
  plan->workspace_bytes = 0;
  if (total > 0) {
    void* ws = nullptr;
    if (hipMalloc(&ws, total) != hipSuccess || ws == nullptr) {
      (void)hipGetLastError();
      delete plan;
      return VDA_ERROR_OUT_OF_MEMORY;
    }
    plan->workspace = ws;
    plan->workspace_bytes = total;
    vda::carve_workspace(p, ws);
  }
  plan->timing_capacity = 0;
  plan->timed_calls = 0;
  plan->timed_stages = VDA_STAGE_ALL;
  plan->timing_events = nullptr;
  plan->bwd_workspace = nullptr;
  plan->bwd_workspace_bytes = 0;
  plan->has_statistics = false;
  plan->chunk_workspace = nullptr;
  plan->chunk_workspace_bytes = 0;
  // kernel attributes once, here, so that a forward pass makes no runtime call but launches
  if (vda::prepare_stats(p) != hipSuccess || vda::prepare_scan(p) != hipSuccess ||
      vda::prepare_readout(p) != hipSuccess ||
      (p.bf16 && !p.fp8 && (vda::prepare_bwd_frames(p) != hipSuccess || vda::prepare_grad(p) != hipSuccess))) {
    (void)hipGetLastError();
    if (plan->workspace != nullptr) (void)hipFree(plan->workspace);
    delete plan;
    return VDA_ERROR_DEVICE;
  }
  // the scan the plan runs by default: chunked only where the serial chains leave most of the
  // GPU idle
  const vda_status cs = vda_plan_set_scan_chunk(plan, VDA_SCAN_CHUNK_AUTO);
  if (cs != VDA_SUCCESS) {
    if (plan->workspace != nullptr) (void)hipFree(plan->workspace);
    delete plan;
    return cs;
  }
  *plan_out = plan;
  return VDA_SUCCESS;
}

vda_status vda_plan_destroy(vda_plan_t plan) {
  if (plan == nullptr) return VDA_SUCCESS;
  vda_status st = VDA_SUCCESS;
  auto check = [&](hipError_t e) {
    if (e != hipSuccess) {
      (void)hipGetLastError();
      st = VDA_ERROR_DEVICE;
    }
  };
  free_timing(plan);
  if (plan->workspace != nullptr) check(hipFree(plan->workspace));
  if (plan->bwd_workspace != nullptr) check(hipFree(plan->bwd_workspace));
  if (plan->chunk_workspace != nullptr) check(hipFree(plan->chunk_workspace));
  delete plan;
  return st;
}

size_t vda_plan_workspace_bytes(vda_plan_t plan) {
  return plan == nullptr ? 0
                         : plan->workspace_bytes + plan->bwd_workspace_bytes + plan->chunk_workspace_bytes;
}

vda_status vda_plan_set_scan_chunk(vda_plan_t plan, int64_t chunk_frames) {
  if (plan == nullptr || chunk_frames < VDA_SCAN_CHUNK_AUTO) return VDA_ERROR_INVALID_VALUE;
  vda::Problem& p = plan->p;
  if (chunk_frames > 0 && !p.bf16) return VDA_ERROR_NOT_SUPPORTED;
  if (chunk_frames == VDA_SCAN_CHUNK_AUTO) chunk_frames = vda::auto_scan_chunk(p);
  const size_t bytes = vda::chunk_workspace_bytes(p, chunk_frames);
  if (plan->chunk_workspace != nullptr) {
    const hipError_t e = hipFree(plan->chunk_workspace);
    plan->chunk_workspace = nullptr;
    plan->chunk_workspace_bytes = 0;
    p.chunk_ws = nullptr;
    p.scan_chunk = 0;
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return VDA_ERROR_DEVICE;
    }
  }
  p.scan_chunk = 0;
  if (bytes == 0) return VDA_SUCCESS;  // one chunk: the serial scan
  void* ws = nullptr;
  if (hipMalloc(&ws, bytes) != hipSuccess || ws == nullptr) {
    (void)hipGetLastError();
    return VDA_ERROR_OUT_OF_MEMORY;
  }
  plan->chunk_workspace = ws;
  plan->chunk_workspace_bytes = bytes;
  p.chunk_ws = static_cast<float*>(ws);
  p.scan_chunk = chunk_frames;
  return VDA_SUCCESS;
}

vda_status vda_plan_get_scan_chunk(vda_plan_t plan, int64_t* chunk_frames) {
  if (plan == nullptr || chunk_frames == nullptr) return VDA_ERROR_INVALID_VALUE;
  *chunk_frames = plan->p.scan_chunk;
  return VDA_SUCCESS;
}

vda_status vda_debug_workspace(vda_plan_t plan, const void** ainv, const void** bm,
                               const void** x_fwd, const void** x_bwd) {
  if (plan == nullptr) return VDA_ERROR_INVALID_VALUE;
  if (ainv) *ainv = plan->p.ainv;
  if (bm) *bm = plan->p.bm;
  if (x_fwd) *x_fwd = plan->p.xf;
  if (x_bwd) *x_bwd = plan->p.xb;
  return VDA_SUCCESS;
}

}  // extern "C"

namespace {

}  // namespace

namespace vda {

vda_status enqueue_problem(const Problem& p, int device, unsigned stages, const void* q, const void* k,
                           const void* v, const void* text_k, const void* text_v, const GateWeights* gate,
                           void* out, void* stream, hipEvent_t* tev) {
  if (stages == 0 || (stages & ~unsigned(VDA_STAGE_ALL)) != 0) return VDA_ERROR_INVALID_VALUE;
  // No output element: nothing to compute and no pointer is read.
  if (p.B == 0 || p.H == 0 || p.F == 0 || p.n == 0) return VDA_SUCCESS;
  const size_t es = p.fp8 ? 1 : p.bf16 ? 2 : 4;  // input element bytes
  const size_t eo = p.bf16 ? 2 : 4;              // output element bytes
  const size_t bh = size_t(p.B) * size_t(p.H);
  const size_t qk_bytes = bh * size_t(p.F) * size_t(p.n) * size_t(p.d) * es;
  const size_t v_bytes = bh * size_t(p.F) * size_t(p.n) * size_t(p.dv) * es;
  const size_t o_bytes = bh * size_t(p.F) * size_t(p.n) * size_t(p.dv) * eo;
  const size_t tk_bytes = bh * size_t(p.T) * size_t(p.d) * es;
  const size_t tv_bytes = bh * size_t(p.T) * size_t(p.dv) * es;
  const bool do_stats = stages & VDA_STAGE_STATS;
  const bool do_scan = stages & VDA_STAGE_SCAN;
  const bool do_read = stages & VDA_STAGE_READOUT;

  // Pointer checks: a tensor the selected stages read or write must be non-NULL
  // and 16-byte aligned when it has any element.
  struct Arg {
    const void* ptr;
    size_t bytes;
    bool used;
  } args[9] = {{q, qk_bytes, do_read},         {k, qk_bytes, do_stats},
               {v, v_bytes, do_stats},         {text_k, tk_bytes, do_stats},
               {text_v, tv_bytes, do_stats},
               {gate ? gate->w_gate : nullptr, size_t(p.H) * size_t(p.dv) * size_t(p.dv) * 2, gate != nullptr},
               {gate ? gate->b_gate : nullptr, size_t(p.H) * size_t(p.dv) * 4, gate != nullptr},
               {gate ? gate->w_out : nullptr, size_t(p.H) * size_t(p.dv) * size_t(p.dv) * 2, gate != nullptr},
               {out, o_bytes, do_read}};
  for (const Arg& a : args) {
    if (!a.used || a.bytes == 0) continue;
    if (a.ptr == nullptr) return VDA_ERROR_INVALID_VALUE;
    if (!aligned16(a.ptr)) return VDA_ERROR_MISALIGNED;
  }
  if (do_read && o_bytes > 0) {
    Range o{reinterpret_cast<uintptr_t>(out), reinterpret_cast<uintptr_t>(out) + o_bytes};
    for (int i = 0; i < 8; ++i) {
      if (args[i].ptr == nullptr || args[i].bytes == 0) continue;
      Range r{reinterpret_cast<uintptr_t>(args[i].ptr),
              reinterpret_cast<uintptr_t>(args[i].ptr) + args[i].bytes};
      if (overlaps(o, r)) return VDA_ERROR_INVALID_VALUE;
    }
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return VDA_ERROR_DEVICE;
  }
  if (dev != device) return VDA_ERROR_INVALID_VALUE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // each stage is one kernel launch (the chunked scan: the first and last of its launches),
  // which records the stage's two events itself; a stage that is not timed has none
  auto timed = [&](int begin, int end) {
    vda::Problem ps = p;
    if (tev != nullptr && tev[begin] != nullptr) {
      ps.ev_start = tev[begin];
      ps.ev_stop = tev[end];
    }
    return ps;
  };
  if (do_stats) e = vda::launch_stats(timed(kEvStatsBegin, kEvStatsEnd), k, v, text_k, text_v, s);
  if (e == hipSuccess && do_scan) e = vda::launch_scan(timed(kEvScanBegin, kEvScanEnd), s);
  if (e == hipSuccess && do_read) {
    const vda::Problem pr = timed(kEvReadBegin, kEvReadEnd);
    e = gate ? vda::launch_readout_gated(pr, q, *gate, out, s) : vda::launch_readout(pr, q, out, s);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return VDA_ERROR_DEVICE;
  }
  return VDA_SUCCESS;
}

}  // namespace vda

namespace {

// Checks and enqueues the selected stages of a plan; gate != nullptr runs the gated readout.
vda_status enqueue(vda_plan_t plan, unsigned stages, const void* q, const void* k, const void* v,
                   const void* text_k, const void* text_v, const vda::GateWeights* gate, void* out,
                   void* stream) {
  if (plan == nullptr) return VDA_ERROR_INVALID_VALUE;
  // timing events of this call (whole passes only, the timed stages' slots), or none
  hipEvent_t* tev = nullptr;
  hipEvent_t slots[kTimingEvents] = {};
  if (stages == VDA_STAGE_ALL && plan->timing_capacity > 0 && plan->timed_calls < plan->timing_capacity) {
    hipEvent_t* ev = plan->timing_events + size_t(plan->timed_calls) * kTimingEvents;
    const unsigned bits[3] = {VDA_STAGE_STATS, VDA_STAGE_SCAN, VDA_STAGE_READOUT};
    for (int i = 0; i < 3; ++i)
      if (plan->timed_stages & bits[i]) {
        slots[2 * i] = ev[2 * i];
        slots[2 * i + 1] = ev[2 * i + 1];
      }
    tev = slots;
  }
  const vda_status st = vda::enqueue_problem(plan->p, plan->device, stages, q, k, v, text_k, text_v, gate,
                                             out, stream, tev);
  if (st != VDA_SUCCESS) return st;
  const vda::Problem& p = plan->p;
  if (p.B == 0 || p.H == 0 || p.F == 0 || p.n == 0) return VDA_SUCCESS;  // nothing was enqueued
  if (tev != nullptr) ++plan->timed_calls;
  if (stages & VDA_STAGE_STATS) plan->has_statistics = true;
  return VDA_SUCCESS;
}


// Layout of the backward workspace (byte offsets, each 256-aligned).
struct BwdLayout {
  size_t dw, xf, xb, sf, sb, wt, db2, z, db2_text, z_text, total;
};
BwdLayout bwd_layout(const vda::Problem& p) {
  const size_t BH = size_t(p.B) * size_t(p.H), F = size_t(p.F), d = size_t(p.d), dv = size_t(p.dv);
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  };
  L.dw = take(BH * (F + 1) * d * dv * 4);
  L.xf = take(BH * F * d * dv * 4);
  L.xb = take(BH * F * d * dv * 4);
  L.sf = take(BH * F * d * dv * 4);
  L.sb = take(BH * F * d * dv * 4);
  // W^T for the dQ readout; at d = dv = 128 dQ is formed with dW and needs none
  L.wt = take(p.d == 128 && p.dv == 128 ? 0 : BH * F * dv * d * 2);
  L.db2 = take(BH * F * 2 * d * dv * 2);
  L.z = take(BH * F * (2 * d + 2 * dv) * d * 2);
  L.db2_text = take(BH * 2 * d * dv * 2);
  L.z_text = take(BH * (2 * d + 2 * dv) * d * 2);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

vda_status vda_backward(vda_plan_t plan, const void* q, const void* k, const void* v,
                        const void* text_k, const void* text_v, const void* d_out, void* d_q,
                        void* d_k, void* d_v, void* d_text_k, void* d_text_v, void* stream) {
  if (plan == nullptr) return VDA_ERROR_INVALID_VALUE;
  const vda::Problem& p = plan->p;
  if (!p.bf16 || p.fp8) return VDA_ERROR_NOT_SUPPORTED;
  const size_t BH = size_t(p.B) * size_t(p.H);
  const size_t tok = BH * size_t(p.F) * size_t(p.n), ttok = BH * size_t(p.T);
  // the statistics of a forward pass must be in the workspace (problems with no output
  // element need none)
  if (tok > 0 && !plan->has_statistics) return VDA_ERROR_INVALID_VALUE;
  const size_t qk = tok * size_t(p.d) * 2, vo = tok * size_t(p.dv) * 2;
  const size_t tkb = ttok * size_t(p.d) * 2, tvb = ttok * size_t(p.dv) * 2;
  struct Arg {
    const void* ptr;
    size_t bytes;
  } in[6] = {{q, qk}, {k, qk}, {v, vo}, {text_k, tkb}, {text_v, tvb}, {d_out, vo}},
    outs[5] = {{d_q, qk}, {d_k, qk}, {d_v, vo}, {d_text_k, tkb}, {d_text_v, tvb}};
  for (const Arg& a : in) {
    if (a.bytes == 0) continue;
    if (a.ptr == nullptr) return VDA_ERROR_INVALID_VALUE;
    if (!aligned16(a.ptr)) return VDA_ERROR_MISALIGNED;
  }
  for (const Arg& a : outs) {
    if (a.bytes == 0) continue;
    if (a.ptr == nullptr) return VDA_ERROR_INVALID_VALUE;
    if (!aligned16(a.ptr)) return VDA_ERROR_MISALIGNED;
  }
  // no output may overlap an input or another output
  for (int i = 0; i < 5; ++i) {
    if (outs[i].bytes == 0) continue;
    const Range o{reinterpret_cast<uintptr_t>(outs[i].ptr), reinterpret_cast<uintptr_t>(outs[i].ptr) + outs[i].bytes};
    for (const Arg& a : in)
      if (a.bytes > 0 && overlaps(o, Range{reinterpret_cast<uintptr_t>(a.ptr), reinterpret_cast<uintptr_t>(a.ptr) + a.bytes}))
        return VDA_ERROR_INVALID_VALUE;
    for (int j = 0; j < i; ++j)
      if (outs[j].bytes > 0 &&
          overlaps(o, Range{reinterpret_cast<uintptr_t>(outs[j].ptr), reinterpret_cast<uintptr_t>(outs[j].ptr) + outs[j].bytes}))
        return VDA_ERROR_INVALID_VALUE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return VDA_ERROR_DEVICE;
  }
  if (dev != plan->device) return VDA_ERROR_INVALID_VALUE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (BH == 0) return VDA_SUCCESS;
  if (p.F == 0 || p.n == 0) {
    // no output element: every gradient is zero (the text's included)
    hipError_t e = hipSuccess;
    if (tkb > 0) e = vda::launch_zero(d_text_k, tkb, s);
    if (e == hipSuccess && tvb > 0) e = vda::launch_zero(d_text_v, tvb, s);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return VDA_ERROR_DEVICE;
    }
    return VDA_SUCCESS;
  }
  const BwdLayout L = bwd_layout(p);
  if (plan->bwd_workspace == nullptr) {
    void* ws = nullptr;
    if (hipMalloc(&ws, L.total) != hipSuccess || ws == nullptr) {
      (void)hipGetLastError();
      return VDA_ERROR_OUT_OF_MEMORY;
    }
    plan->bwd_workspace = ws;
    plan->bwd_workspace_bytes = L.total;
  }
  unsigned char* w = static_cast<unsigned char*>(plan->bwd_workspace);
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(w + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(w + off); };

  hipError_t e = hipSuccess;
  hipEvent_t* tev = nullptr;
  if (plan->timing_capacity > 0 && plan->timed_calls < plan->timing_capacity)
    tev = plan->timing_events + size_t(plan->timed_calls) * kTimingEvents;
  const unsigned slot_stage[kTimingEvents] = {VDA_STAGE_STATS, VDA_STAGE_STATS, VDA_STAGE_SCAN, VDA_STAGE_SCAN,
                                              VDA_STAGE_READOUT, VDA_STAGE_READOUT};
  auto mark = [&](int slot) {
    if (tev != nullptr && e == hipSuccess && (plan->timed_stages & slot_stage[slot]))
      e = hipEventRecord(tev[slot], s);
  };
  // The forward states again, in float32 (the forward pass keeps them in bf16): the scan on
  // the forward's statistics with float32 state stores.
  vda::Problem px = p;
  px.scan_chunk = 0;  // the backward pass's chains run serially
  px.states_f32 = true;
  px.xf = f32(L.xf);
  px.xb = f32(L.xb);
  // dW_f = Q_f^T dO_f: the statistics stage on (Q, dO), Bm only, with no text (frame 0 is zero)
  vda::Problem pw = p;
  pw.T = 0;
  pw.bm_only = true;
  pw.ainv = nullptr;
  pw.bm = f32(L.dw);
  // At d = dv = 128 one pass over (Q, dO) forms dW and dQ = dO W^T (W from the float32
  // states), so the recomputed states come first; elsewhere dQ is a readout of W^T from the
  // per-frame kernel.
  const bool fused_dq = p.d == 128 && p.dv == 128;
  mark(kEvStatsBegin);
  if (fused_dq) {
    if (e == hipSuccess) e = vda::launch_scan(px, s);
    if (e == hipSuccess) e = vda::launch_stats_dq(pw, q, d_out, f32(L.xf), f32(L.xb), d_q, s);
  } else if (e == hipSuccess) {
    e = vda::launch_stats(pw, q, d_out, nullptr, nullptr, s);
  }
  mark(kEvStatsEnd);
  // the adjoint chains (twice the adjoints): the scan on (A^{-1} of the forward, dW), float32
  // states; then the per-frame terms
  mark(kEvScanBegin);
  if (!fused_dq && e == hipSuccess) e = vda::launch_scan(px, s);
  vda::Problem ps = p;
  ps.scan_chunk = 0;
  ps.states_f32 = true;
  ps.bm = f32(L.dw);
  ps.xf = f32(L.sf);
  ps.xb = f32(L.sb);
  if (e == hipSuccess) e = vda::launch_scan(ps, s);
  vda::BwdProblem b{p, f32(L.xf), f32(L.xb), f32(L.sf), f32(L.sb), fused_dq ? nullptr : u16(L.wt), u16(L.db2),
                    u16(L.z), u16(L.db2_text), u16(L.z_text)};
  if (e == hipSuccess) e = vda::launch_bwd_frames(b, s);
  mark(kEvScanEnd);
  // the gradient products: dQ = dO W^T (unless formed above), dV = [K K] [dB hi ; lo],
  // dK = [K K V V] [M hi ; M lo ; dB^T hi ; dB^T lo]
  mark(kEvReadBegin);
  if (!fused_dq) {
    vda::Problem pq = p;
    pq.d = p.dv;
    pq.dv = p.d;
    pq.xf = pq.xb = f32(L.wt);
    if (e == hipSuccess) e = vda::launch_readout(pq, d_out, d_q, s);
  }
  if (e == hipSuccess) e = vda::launch_grad_kv(p, k, v, u16(L.z), u16(L.db2), d_k, d_v, s);
  if (p.T > 0) {
    vda::Problem pt = p;
    pt.F = 1;
    pt.n = p.T;
    if (e == hipSuccess)
      e = vda::launch_grad_kv(pt, text_k, text_v, u16(L.z_text), u16(L.db2_text), d_text_k, d_text_v, s);
  }
  mark(kEvReadEnd);
  if (tev != nullptr && e == hipSuccess) ++plan->timed_calls;
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return VDA_ERROR_DEVICE;
  }
  return VDA_SUCCESS;
}

}  // extern "C"

namespace {
}  // namespace

extern "C" {

vda_status vda_forward_stages(vda_plan_t plan, unsigned stages, const void* q, const void* k,
                              const void* v, const void* text_k, const void* text_v, void* out,
                              void* stream) {
  return enqueue(plan, stages, q, k, v, text_k, text_v, nullptr, out, stream);
}

vda_status vda_forward_gated(vda_plan_t plan, const void* q, const void* k, const void* v,
                             const void* text_k, const void* text_v, const void* w_gate,
                             const void* b_gate, const void* w_out, void* out, void* stream) {
  if (plan == nullptr) return VDA_ERROR_INVALID_VALUE;
  if (!plan->p.bf16) return VDA_ERROR_NOT_SUPPORTED;
  const vda::GateWeights gw{w_gate, b_gate, w_out};
  return enqueue(plan, VDA_STAGE_ALL, q, k, v, text_k, text_v, &gw, out, stream);
}

vda_status vda_plan_enable_timing(vda_plan_t plan, int capacity) {
  if (plan == nullptr || capacity < 0 || capacity > 100000) return VDA_ERROR_INVALID_VALUE;
  free_timing(plan);
  if (capacity == 0) return VDA_SUCCESS;
  const int nev = capacity * kTimingEvents;
  plan->timing_events = new (std::nothrow) hipEvent_t[nev]();
  if (plan->timing_events == nullptr) return VDA_ERROR_OUT_OF_MEMORY;
  plan->timing_capacity = capacity;
  for (int i = 0; i < nev; ++i) {
    if (hipEventCreate(&plan->timing_events[i]) != hipSuccess) {
      (void)hipGetLastError();
      free_timing(plan);
      return VDA_ERROR_DEVICE;
    }
  }
  return VDA_SUCCESS;
}

vda_status vda_plan_set_timed_stages(vda_plan_t plan, unsigned stages) {
  if (plan == nullptr || (stages & ~unsigned(VDA_STAGE_ALL)) != 0) return VDA_ERROR_INVALID_VALUE;
  if (plan->timed_calls != 0) return VDA_ERROR_INVALID_VALUE;  // read the recorded calls first
  plan->timed_stages = stages;
  return VDA_SUCCESS;
}

vda_status vda_plan_timings(vda_plan_t plan, int* calls, float* stats_ms, float* scan_ms,
                            float* readout_ms) {
  if (plan == nullptr || calls == nullptr) return VDA_ERROR_INVALID_VALUE;
  const int n = plan->timed_calls;
  double acc[3] = {0.0, 0.0, 0.0};
  for (int c = 0; c < n; ++c) {
    hipEvent_t* ev = plan->timing_events + size_t(c) * kTimingEvents;
    const int spans[3][3] = {{kEvStatsBegin, kEvStatsEnd, 0},
                             {kEvScanBegin, kEvScanEnd, 1},
                             {kEvReadBegin, kEvReadEnd, 2}};
    const unsigned bits[3] = {VDA_STAGE_STATS, VDA_STAGE_SCAN, VDA_STAGE_READOUT};
    for (const auto& sp : spans) {
      if (!(plan->timed_stages & bits[sp[2]])) continue;  // not timed: reported as 0
      float ms = 0.0f;
      if (hipEventSynchronize(ev[sp[1]]) != hipSuccess ||
          hipEventElapsedTime(&ms, ev[sp[0]], ev[sp[1]]) != hipSuccess) {
        (void)hipGetLastError();
        return VDA_ERROR_DEVICE;
      }
      acc[sp[2]] += ms;
    }
  }
  *calls = n;
  const double div = n > 0 ? double(n) : 1.0;
  if (stats_ms) *stats_ms = float(acc[0] / div);
  if (scan_ms) *scan_ms = float(acc[1] / div);
  if (readout_ms) *readout_ms = float(acc[2] / div);
  plan->timed_calls = 0;
  return VDA_SUCCESS;
}

vda_status vda_forward(vda_plan_t plan, const void* q, const void* k, const void* v,
                       const void* text_k, const void* text_v, void* out, void* stream) {
  return vda_forward_stages(plan, VDA_STAGE_ALL, q, k, v, text_k, text_v, out, stream);
}

}  // extern "C"
