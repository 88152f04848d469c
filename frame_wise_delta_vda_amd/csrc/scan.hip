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
// Within a workgroup each wave owns 16-row blocks of X; the right operand
// R = lam X + Bm of a step is exchanged through LDS.
//
// float32 plans: 16x16x4 fp32 MFMA.
// bfloat16 plans: split-bf16 products on 16x16x32 bf16 MFMA.  Ainv_f arrives as two
// bf16 planes (hi + lo) and R is split the same way each step; Ainv R is taken as
// hi*hi + hi*lo + lo*hi, which leaves a relative error of order 2^-16 per product
// (far below the bf16 rounding of the inputs and output).  Operand fragments of the
// next two steps are kept in flight in a register ring.
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
    const float* src = bm_h + fr * int64_t(D) * DV;
#pragma unroll
    for (int i = 0; i < C::RBW; ++i) {
      const float4 b4 = *reinterpret_cast<const float4*>(
          src + blk_index((wave * C::RBW + i) * 16 + 4 * g, c0 + n, D));
      dst[i][0] = b4.x; dst[i][1] = b4.y; dst[i][2] = b4.z; dst[i][3] = b4.w;
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
        float* dst = xo_h + (f - 1) * int64_t(D) * DV;
#pragma unroll
        for (int i = 0; i < C::RBW; ++i)
          *reinterpret_cast<float4*>(dst + blk_index((wave * C::RBW + i) * 16 + 4 * g, c0 + n, D)) =
              make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
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
struct ScanBf16Cfg {
  static constexpr int RB = D / 16;               // 16-row blocks of X
  static constexpr int NW = RB < 4 ? RB : 4;      // waves holding rows
  static constexpr int RBW = RB / NW;             // row blocks per wave
  static constexpr int KS = D / 32;               // k-steps of the 16x16x32 MFMA
  static constexpr int NCB = DV / 16;             // 16-column workgroups per chain
  static constexpr int NPF = 2;                   // steps of operand prefetch
  static constexpr int NSLOT = NPF + 1;           // register ring slots
  static constexpr int RS_ELEMS = 2 * KS * 4 * 16 * 8;  // one R buffer: [hi/lo][ks][kg][n][8]
};

template <int D, int DV>
__global__ void __launch_bounds__(kThreads, 2)
scan_bf16_kernel(const uint16_t* __restrict__ ainv_planes, const float* __restrict__ bm,
                 float* __restrict__ xf, float* __restrict__ xb, int64_t nchains, int64_t F,
                 float lam, int64_t grid) {
  using C = ScanBf16Cfg<D, DV>;
  __shared__ __align__(16) uint16_t rs[2][C::RS_ELEMS];

  const int64_t L = xcd_remap(blockIdx.x, grid);
  const int64_t chain = L / C::NCB;
  const int cb = int(L % C::NCB);
  if (chain >= nchains) return;
  const int64_t bh = chain >> 1;
  const bool backward = chain & 1;
  const int64_t F1 = F + 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int n = lane & 15, g = lane >> 4;
  const bool active = wave < C::NW;
  const int c0 = cb * 16;

  const uint16_t* ainv_h = ainv_planes + bh * F1 * int64_t(2 * D * D);
  const float* bm_h = bm + bh * F1 * int64_t(D) * DV;
  float* xo_h = (backward ? xb : xf) + bh * F * int64_t(D) * DV;

  // frame index (0 = text) of chain step s; steps past the end re-read the last frame
  auto frame_at = [&](int64_t s) -> int64_t {
    if (s > F) s = F;
    return (s == 0 || !backward) ? s : F + 1 - s;
  };
  // slot t of the ring holds Ainv of step t and the Bm that step t adds for step t+1
  uint4 A[C::NSLOT][C::RBW][C::KS][2];
  float Bv[C::NSLOT][C::RBW][4];
  auto load_slot = [&](int64_t t, uint4 (&a)[C::RBW][C::KS][2], float (&bv)[C::RBW][4]) {
    const uint16_t* hi = ainv_h + frame_at(t) * int64_t(2 * D * D);
    const uint16_t* lo = hi + D * D;
    const float* bsrc = bm_h + frame_at(t + 1) * int64_t(D) * DV;
#pragma unroll
    for (int i = 0; i < C::RBW; ++i) {
      const int row = (wave * C::RBW + i) * 16 + n;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        a[i][ks][0] = *reinterpret_cast<const uint4*>(hi + row * D + ks * 32 + g * 8);
        a[i][ks][1] = *reinterpret_cast<const uint4*>(lo + row * D + ks * 32 + g * 8);
      }
      const float4 b4 = *reinterpret_cast<const float4*>(
          bsrc + blk_index((wave * C::RBW + i) * 16 + 4 * g, c0 + n, D));
      bv[i][0] = b4.x; bv[i][1] = b4.y; bv[i][2] = b4.z; bv[i][3] = b4.w;
    }
  };
  // R fragment (8 consecutive k of column n) and the 4-row output slot of a lane
  auto rs_frag = [&](int buf, int hl, int ks) -> const uint4* {
    return reinterpret_cast<const uint4*>(&rs[buf][((hl * C::KS + ks) * 4 + g) * 128 + n * 8]);
  };
  auto rs_out = [&](int buf, int hl, int rbx) -> uint2* {
    return reinterpret_cast<uint2*>(
        &rs[buf][((hl * C::KS + rbx / 2) * 4 + 2 * (rbx % 2) + g / 2) * 128 + n * 8 + 4 * (g % 2)]);
  };
  auto write_r = [&](int buf, int i, float r0, float r1, float r2, float r3) {
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    split_bf16(r0, h0, l0);
    split_bf16(r1, h1, l1);
    split_bf16(r2, h2, l2);
    split_bf16(r3, h3, l3);
    const int rbx = wave * C::RBW + i;
    *rs_out(buf, 0, rbx) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
    *rs_out(buf, 1, rbx) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
  };

  if (active) {
    // R_0 = lam * 0 + Bm_0
#pragma unroll
    for (int i = 0; i < C::RBW; ++i) {
      const float4 b4 = *reinterpret_cast<const float4*>(
          bm_h + blk_index((wave * C::RBW + i) * 16 + 4 * g, c0 + n, D));
      write_r(0, i, b4.x, b4.y, b4.z, b4.w);
    }
#pragma unroll
    for (int t = 0; t < C::NPF; ++t) load_slot(t, A[t], Bv[t]);
  }
  __syncthreads();

  auto step = [&](int64_t s, uint4 (&a)[C::RBW][C::KS][2], float (&bv)[C::RBW][4],
                  uint4 (&a_fill)[C::RBW][C::KS][2], float (&bv_fill)[C::RBW][4]) {
    const int buf = int(s & 1);
    if (active) {
      load_slot(s + C::NPF, a_fill, bv_fill);
      f32x4 hh[C::RBW], hl[C::RBW], lh[C::RBW];
#pragma unroll
      for (int i = 0; i < C::RBW; ++i) hh[i] = hl[i] = lh[i] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const uint4 rh = *rs_frag(buf, 0, ks);
        const uint4 rl = *rs_frag(buf, 1, ks);
#pragma unroll
        for (int i = 0; i < C::RBW; ++i) {
          hh[i] = mfma16_bf16(a[i][ks][0], rh, hh[i]);
          hl[i] = mfma16_bf16(a[i][ks][0], rl, hl[i]);
          lh[i] = mfma16_bf16(a[i][ks][1], rh, lh[i]);
        }
      }
      f32x4 x[C::RBW];
#pragma unroll
      for (int i = 0; i < C::RBW; ++i) x[i] = hh[i] + (hl[i] + lh[i]);
      if (s >= 1) {
        float* dst = xo_h + (frame_at(s) - 1) * int64_t(D) * DV;
#pragma unroll
        for (int i = 0; i < C::RBW; ++i)
          *reinterpret_cast<float4*>(dst + blk_index((wave * C::RBW + i) * 16 + 4 * g, c0 + n, D)) =
              make_float4(x[i][0], x[i][1], x[i][2], x[i][3]);
      }
      if (s < F) {
#pragma unroll
        for (int i = 0; i < C::RBW; ++i)
          write_r(buf ^ 1, i, __builtin_fmaf(lam, x[i][0], bv[i][0]),
                  __builtin_fmaf(lam, x[i][1], bv[i][1]), __builtin_fmaf(lam, x[i][2], bv[i][2]),
                  __builtin_fmaf(lam, x[i][3], bv[i][3]));
      }
    }
    __syncthreads();
  };

  static_assert(C::NSLOT == 3, "ring unrolled for three slots");
  for (int64_t s0 = 0; s0 <= F; s0 += 3) {
    step(s0, A[0], Bv[0], A[2], Bv[2]);
    if (s0 + 1 > F) break;
    step(s0 + 1, A[1], Bv[1], A[0], Bv[0]);
    if (s0 + 2 > F) break;
    step(s0 + 2, A[2], Bv[2], A[1], Bv[1]);
  }
}

template <int D, int DV>
hipError_t launch_scan_t(const Problem& p, hipStream_t s) {
  const int64_t nchains = 2 * p.B * p.H;
  if (p.bf16) {
    using C = ScanBf16Cfg<D, DV>;
    const int64_t grid = ((nchains + kXcds - 1) / kXcds) * kXcds * C::NCB;
    hipLaunchKernelGGL((scan_bf16_kernel<D, DV>), dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(p.ainv), p.bm, p.xf, p.xb, nchains, p.F,
                       p.lam, grid);
  } else {
    using C = ScanCfg<D, DV>;
    const int64_t grid = ((nchains + kXcds - 1) / kXcds) * kXcds * C::NCB;
    hipLaunchKernelGGL((scan_kernel<D, DV>), dim3(unsigned(grid)), dim3(kThreads), 0, s, p.ainv,
                       p.bm, p.xf, p.xb, nchains, p.F, p.lam, grid);
  }
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
