// Stage 2 of the VDA forward pass: the bidirectional state scans.
//
// Each head keeps a d x dv state X (= S^T) that is carried across frames with
// constant cost (comfyui-wiki page, "how Video DeltaNet speeds up H3": a
// bidirectional linear-attention branch with a recurrent state).  Both scans start
// from the text state, written once at initialisation (aiezz page, section 03,
// bullet "dual text injection"), which is the update applied to a zero state:
//   X_text = Ainv_0 Bm_0
//   forward  f = 1..F:  X_f = Ainv_f (lam X_{f-1} + Bm_f)
//   backward f = F..1:  X_f = Ainv_f (lam X_{f+1} + Bm_f)
// Ainv_f and Bm_f come from the statistics stage, so each step is one d x d by
// d x dv product -- the serial chain does no triangular solves.
//
// Columns of X are independent (the left factor Ainv_f is shared), so a chain is
// split over DV/16 workgroups of 16 columns each; all workgroups of one chain are
// placed on one XCD so that Ainv_f is fetched from HBM once and hit in L2 after.
// Within a workgroup each wave owns 16-row blocks of X; a step is a 16x16x4 fp32
// MFMA product whose right operand R = lam X + Bm is exchanged through LDS.
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

template <int D, int DV>
struct ScanCfg {
  static constexpr int RB = D / 16;               // 16-row blocks of X
  static constexpr int NW = RB < 4 ? RB : 4;      // waves holding rows
  static constexpr int RBW = RB / NW;             // row blocks per wave
  static constexpr int NCB = DV / 16;             // 16-column workgroups per chain
  static constexpr int RS_FLOATS = D * 16;        // one R buffer: D rows x 16 columns
  static constexpr int LDS_BYTES = 2 * RS_FLOATS * 4;
};

template <int D, int DV>
__global__ void __launch_bounds__(kThreads)
scan_kernel(const float* __restrict__ ainv, const float* __restrict__ bm,
            float* __restrict__ xf, float* __restrict__ xb, int64_t nchains, int64_t F,
            float lam, int64_t grid) {
  using C = ScanCfg<D, DV>;
  __shared__ __align__(16) float rs[2 * C::RS_FLOATS];

  const int64_t L = xcd_remap(blockIdx.x, grid);
  const int64_t chain = L / C::NCB;
  const int cb = int(L % C::NCB);
  if (chain >= nchains) return;
  const int64_t bh = chain >> 1;
  const bool backward = chain & 1;
  const int64_t F1 = F + 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const bool active = wave < C::NW;
  const int c0 = cb * 16;

  const float* ainv_h = ainv + bh * F1 * int64_t(D) * D;
  const float* bm_h = bm + bh * F1 * int64_t(D) * DV;
  float* xo_h = (backward ? xb : xf) + bh * F * int64_t(D) * DV;

  // frame index (0 = text) used at chain step s
  auto frame_at = [&](int64_t s) -> int64_t { return (s == 0 || !backward) ? s : F + 1 - s; };

  // A operand: rows 16*rb + n of Ainv_f, columns 16j + 4g .. +3 (one float4 per j)
  float4 a_cur[C::RBW][C::RB], a_nxt[C::RBW][C::RB];
  // Bm values for this lane's rows 16*rb + 4g + r, column c0 + n
  float b_cur[C::RBW][4], b_nxt[C::RBW][4];

  auto load_a = [&](int64_t fr, float4 (&dst)[C::RBW][C::RB]) {
    const float* src = ainv_h + fr * int64_t(D) * D;
#pragma unroll
    for (int i = 0; i < C::RBW; ++i) {
      const int row = (wave * C::RBW + i) * 16 + n;
#pragma unroll
      for (int j = 0; j < C::RB; ++j)
        dst[i][j] = *reinterpret_cast<const float4*>(src + row * D + 16 * j + 4 * g);
    }
  };
  auto load_b = [&](int64_t fr, float (&dst)[C::RBW][4]) {
    const float* src = bm_h + fr * int64_t(D) * DV + c0 + n;
#pragma unroll
    for (int i = 0; i < C::RBW; ++i) {
      const int row0 = (wave * C::RBW + i) * 16 + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[i][r] = src[int64_t(row0 + r) * DV];
    }
  };
  // R buffer layout: [row block j][g][column n][r], so lane (n, g) reads one float4
  auto rs_at = [&](int buf, int j) -> float* {
    return rs + buf * C::RS_FLOATS + ((j * 4 + g) * 16 + n) * 4;
  };

  if (active) {
    load_a(0, a_cur);
    load_b(0, b_cur);
    // R_0 = lam * 0 + Bm_0
#pragma unroll
    for (int i = 0; i < C::RBW; ++i)
      *reinterpret_cast<float4*>(rs_at(0, wave * C::RBW + i)) =
          make_float4(b_cur[i][0], b_cur[i][1], b_cur[i][2], b_cur[i][3]);
    if (F >= 1) load_b(frame_at(1), b_cur);
  }
  __syncthreads();

  for (int64_t s = 0; s <= F; ++s) {
    const int buf = int(s & 1);
    if (active) {
      if (s + 1 <= F) load_a(frame_at(s + 1), a_nxt);
      if (s + 2 <= F) load_b(frame_at(s + 2), b_nxt);
      f32x4 acc[C::RBW];
#pragma unroll
      for (int i = 0; i < C::RBW; ++i) acc[i] = f32x4{};
#pragma unroll
      for (int j = 0; j < C::RB; ++j) {
        const float4 rr = *reinterpret_cast<const float4*>(rs_at(buf, j));
#pragma unroll
        for (int i = 0; i < C::RBW; ++i) {
          acc[i] = mfma16_f32(a_cur[i][j].x, rr.x, acc[i]);
          acc[i] = mfma16_f32(a_cur[i][j].y, rr.y, acc[i]);
          acc[i] = mfma16_f32(a_cur[i][j].z, rr.z, acc[i]);
          acc[i] = mfma16_f32(a_cur[i][j].w, rr.w, acc[i]);
        }
      }
      if (s >= 1) {
        const int64_t f = frame_at(s);  // 1..F
        float* dst = xo_h + (f - 1) * int64_t(D) * DV + c0 + n;
#pragma unroll
        for (int i = 0; i < C::RBW; ++i) {
          const int row0 = (wave * C::RBW + i) * 16 + 4 * g;
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[int64_t(row0 + r) * DV] = acc[i][r];
        }
      }
      if (s + 1 <= F) {
#pragma unroll
        for (int i = 0; i < C::RBW; ++i)
          *reinterpret_cast<float4*>(rs_at(buf ^ 1, wave * C::RBW + i)) =
              make_float4(__builtin_fmaf(lam, acc[i][0], b_cur[i][0]),
                          __builtin_fmaf(lam, acc[i][1], b_cur[i][1]),
                          __builtin_fmaf(lam, acc[i][2], b_cur[i][2]),
                          __builtin_fmaf(lam, acc[i][3], b_cur[i][3]));
#pragma unroll
        for (int i = 0; i < C::RBW; ++i)
#pragma unroll
          for (int j = 0; j < C::RB; ++j) a_cur[i][j] = a_nxt[i][j];
#pragma unroll
        for (int i = 0; i < C::RBW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) b_cur[i][r] = b_nxt[i][r];
      }
    }
    __syncthreads();
  }
}

template <int D, int DV>
hipError_t launch_scan_t(const Problem& p, hipStream_t s) {
  using C = ScanCfg<D, DV>;
  const int64_t nchains = 2 * p.B * p.H;
  const int64_t grid = ((nchains + kXcds - 1) / kXcds) * kXcds * C::NCB;
  hipLaunchKernelGGL((scan_kernel<D, DV>), dim3(unsigned(grid)), dim3(kThreads), 0, s, p.ainv,
                     p.bm, p.xf, p.xb, nchains, p.F, p.lam, grid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const Problem& p, hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_scan_t<DD, VV>(p, s);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda
