// Internal interface between the C ABI layer (vda_api.cpp) and the HIP kernels.
#pragma once

// The kernel sources (HIP language mode) get the launch helper below; the C ABI layer is plain
// host C++ and needs only the runtime API.
#if defined(__HIP__)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#else
#include <hip/hip_runtime_api.h>
#endif
#include <cstddef>
#include <cstdint>

#include "vda.h"

namespace vda {

// Largest token count of one frame or of the text: a frame's K and V are read through
// buffer descriptors with 32-bit byte offsets (up to 256 B per token, plus a chunk).
constexpr int64_t kMaxFrameTokens = (int64_t(1) << 24) - 256;

// Problem shape and float32 workspace of one plan.
struct Problem {
  int64_t B, H, F, n, d, dv, T;
  float lam;
  bool bf16;        // bfloat16 path: bfloat16 out and states (set for FP8 inputs as well)
  bool fp8;         // q, k, v and text are OCP FP8 e4m3 codes (bfloat16 path otherwise)
  bool states_f32;  // bf16 path: the scan stores float32 blocked states (backward pass)
  bool bm_only;     // bf16 path: the statistics stage writes Bm = K^T V only (ainv unused)
  int num_cus;      // compute units of the plan's device (sizes persistent grids)
  // workspace (float32), frame index 0 = text, 1..F = frames
  float* ainv;      // [BH][F+1][d][d]
  float* bm;        // [BH][F+1][d][dv]
  float* xf;        // [BH][F][d][dv]; bf16 plans: bf16 elements in state_index order
  float* xb;        // [BH][F][d][dv]; likewise
  // bfloat16 path: chain steps per chunk of the chunked scan (0: the serial scan), and its
  // workspace of chunk summaries (float32, [2BH][K] of d*d + 2*d*dv, K = ceil(F / scan_chunk))
  int64_t scan_chunk = 0;
  float* chunk_ws = nullptr;
  // when set, the kernel a forward stage launches (the first and last of them, for a stage of
  // several launches) records these around itself, inside its dispatch (per-stage timing
  // without separate event packets between the kernels)
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;
};

// Chunk length the plan chooses by itself: the chunked scan only where the serial chains
// leave most compute units idle (their workgroups fill at most a quarter of them) and are long
// (at least 48 frames: below that its two extra launches cost about what the shorter chains
// save), with about as many chunks as fill the compute units in the local pass, at most 8 (the
// carry pass is serial over the chunks).  0: the serial scan.
inline int64_t auto_scan_chunk(const Problem& p) {
  if (!p.bf16 || p.F < 48 || p.num_cus <= 0) return 0;
  const int64_t nchains = 2 * p.B * p.H;
  const int64_t serial_wgs = nchains * (p.dv / 32);
  if (serial_wgs * 4 > p.num_cus) return 0;
  int64_t k = (p.num_cus + nchains * (p.dv / 32 + p.d / 32) / 2) / (nchains * (p.dv / 32 + p.d / 32)) + 1;
  const int64_t kmax = p.F / 4 < 8 ? p.F / 4 : 8;
  k = k < 2 ? 2 : k > kmax ? kmax : k;
  return (p.F + k - 1) / k;
}

// Bytes of the chunked scan's workspace for chunks of `chunk` chain steps (0 when the scan is
// serial: chunk == 0 or a single chunk).
inline size_t chunk_workspace_bytes(const Problem& p, int64_t chunk) {
  if (chunk <= 0 || p.F <= chunk) return 0;
  const size_t K = size_t((p.F + chunk - 1) / chunk);
  return size_t(2 * p.B * p.H) * K * size_t(p.d * p.d + 2 * p.d * p.dv) * sizeof(float);
}

#if defined(__HIP__)
// Launch a kernel of a forward stage, with the stage's timing events if the problem carries them.
template <typename K, typename... Args>
inline void launch_kernel(const Problem& p, K kern, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                          Args... args) {
  if (p.ev_start != nullptr || p.ev_stop != nullptr)
    hipExtLaunchKernelGGL(kern, grid, block, lds, s, p.ev_start, p.ev_stop, 0u, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, s, args...);
}
#endif

// Validates a problem shape (the checks of vda_plan_create) and fills *out with it, no
// workspace attached; *workspace_bytes is what the forward pass needs (vda_api.cpp).
vda_status make_problem(int64_t B, int64_t H, int64_t F, int64_t n, int64_t d, int64_t dv, int64_t T,
                        float lambda, vda_dtype dtype, Problem* out, size_t* workspace_bytes);
// Points p's workspace buffers (ainv, bm, xf, xb) into the block at base, of the size
// make_problem reported.
void carve_workspace(Problem& p, void* base);
struct GateWeights;
// Argument checks (pointers, alignment, overlap, current device == device) and the launches of
// the selected stages of p on `stream`; tev, when not NULL, holds the stages' timing events.
// A problem with no output element enqueues nothing and returns VDA_SUCCESS.
vda_status enqueue_problem(const Problem& p, int device, unsigned stages, const void* q, const void* k,
                           const void* v, const void* text_k, const void* text_v, const GateWeights* gate,
                           void* out, void* stream, hipEvent_t* tev);

// Each launcher enqueues one stage on `stream` and returns the launch status.
hipError_t launch_stats(const Problem& p, const void* k, const void* v, const void* tk,
                        const void* tv, hipStream_t stream);
hipError_t launch_scan(const Problem& p, hipStream_t stream);
// Backward pass, d = dv = 128: dW_f = Q_f^T dO_f into p.bm (frame 0 zero; p.T must be 0) and,
// from the same pass over dO, dQ_f = dO_f W_f^T with W_f the mean of the float32 blocked
// states xf32 / xb32.
hipError_t launch_stats_dq(const Problem& p, const void* q, const void* d_out, const float* xf32,
                           const float* xb32, void* d_q, hipStream_t stream);
hipError_t launch_readout(const Problem& p, const void* q, void* out, hipStream_t stream);
// Weights of the gated fusion epilogue (bfloat16 [H][dv][dv] matrices, float32 [H][dv] bias).
struct GateWeights {
  const void* w_gate;
  const void* b_gate;
  const void* w_out;
};
// Backward pass: the forward problem (its workspace holds the saved statistics), the
// forward states recomputed in float32 (xf32, xb32, blocked), the adjoint chains of the
// scan run on (A^{-1}, Q^T dO) (sf: forward chain, sb: backward chain, float32 blocked,
// both twice the adjoints), and the per-frame outputs in the readouts' state order (bf16):
// wt = W^T [BH][F][dv*d], db2 = [dB hi ; lo] [BH][F][2d*dv],
// z = [M hi ; M lo ; dB^T hi ; dB^T lo] [BH][F][(2d+2dv)*d], and the text's db2_text,
// z_text [BH][...].
struct BwdProblem {
  Problem p;
  const float* xf32;
  const float* xb32;
  const float* sf;
  const float* sb;
  uint16_t* wt;
  uint16_t* db2;
  uint16_t* z;
  uint16_t* db2_text;
  uint16_t* z_text;
};
hipError_t launch_bwd_frames(const BwdProblem& b, hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t prepare_bwd_frames(const Problem& p);
// The backward pass's gradient products, bf16 in and out, per frame:
//   split_dv:  out (n x dv) = [K K] DB2,           DB2 a 2d x dv state (dB hi ; lo)
//   split_dk:  out (n x d)  = [K K V V] Z,         Z a (2d + 2dv) x d state
hipError_t launch_grad_dv(const Problem& p, const void* k, const void* state, void* out, hipStream_t stream);
hipError_t prepare_grad(const Problem& p);
// dK and dV of the backward pass together (one pass over K and V at d = dv = 128)
hipError_t launch_grad_kv(const Problem& p, const void* k, const void* v, const void* zk, const void* zv,
                          void* dk, void* dv, hipStream_t stream);
hipError_t launch_grad_dk(const Problem& p, const void* k, const void* v, const void* state, void* out,
                          hipStream_t stream);
// The readout followed by the gated epilogue (bfloat16 and FP8 plans).
hipError_t launch_readout_gated(const Problem& p, const void* q, const GateWeights& gw, void* out,
                                hipStream_t stream);
// Per-function attributes (dynamic LDS above 64 KB) of the kernels a plan launches, set
// once at plan creation on the plan's device, so that launches make no other runtime
// call (they can then be captured in a graph).
hipError_t prepare_stats(const Problem& p);
hipError_t prepare_scan(const Problem& p);
hipError_t prepare_readout(const Problem& p);

}  // namespace vda
