// Stage 3 of the VDA forward pass: the readout.
//
// Every frame reads the bidirectional state out with its queries (linear-attention
// readout; model card introduction, bullet "hybrid architecture": a frame-wise
// linear-attention branch), using the mean of the two directional states after
// that frame's own update:
//   W_f = (X_fwd_f + X_bwd_f) / 2,   O_f = Q_f W_f   (n x dv)
//
// bfloat16 path: a workgroup owns one frame (or a contiguous token range of it).
// It forms W_f in fp32, rounds it to bf16 and stores W_f^T in LDS; each wave then
// streams 32-token units of Q straight from HBM into MFMA operands (16-byte loads)
// and computes O^T = W^T Q^T on 32x32x16 bf16 MFMA, so each lane ends up with four
// consecutive output columns of one token, written as one 8-byte store.
// float32 path: the same scheme with W kept in fp32 and 32x32x2 fp32 MFMA.
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

template <int D, int DV>
struct ReadBf16 {
  static constexpr int WROW = D + 8;  // bf16 per LDS row of W^T (conflict-free fragment reads)
  static constexpr int LDS_BYTES = DV * WROW * 2;
  static constexpr int NDB = DV / 32;  // 32-wide output column blocks
  static constexpr int KS = D / 16;    // MFMA k-steps
};

// W^T (bf16) into LDS from the two fp32 states of frame index f (0-based).
template <int D, int DV>
__device__ __forceinline__ void build_wt_bf16(const float* xf, const float* xb, uint16_t* wt) {
  using C = ReadBf16<D, DV>;
  // thread handles rows (2kp, 2kp+1) of W for column j -> one dword of W^T row j
  for (int idx = threadIdx.x; idx < (D / 2) * DV; idx += kThreads) {
    const int j = idx % DV, kp = idx / DV;
    const int r0 = 2 * kp;
    const float w0 = 0.5f * (xf[r0 * DV + j] + xb[r0 * DV + j]);
    const float w1 = 0.5f * (xf[(r0 + 1) * DV + j] + xb[(r0 + 1) * DV + j]);
    *reinterpret_cast<uint32_t*>(wt + j * C::WROW + r0) = pack_bf16x2(w0, w1);
  }
}

template <int D, int DV>
__global__ void __launch_bounds__(kThreads, 2)
readout_bf16_kernel(const uint16_t* __restrict__ q, const float* __restrict__ xf,
                    const float* __restrict__ xb, uint16_t* __restrict__ out, int64_t F,
                    int64_t n, int64_t splits, int64_t tokens_per_split) {
  using C = ReadBf16<D, DV>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* wt = reinterpret_cast<uint16_t*>(smem);

  const int64_t split = blockIdx.x % splits;
  const int64_t frame = blockIdx.x / splits;  // bh * F + f
  const int64_t t_begin = split * tokens_per_split;
  const int64_t t_end = t_begin + tokens_per_split < n ? t_begin + tokens_per_split : n;

  build_wt_bf16<D, DV>(xf + frame * int64_t(D) * DV, xb + frame * int64_t(D) * DV, wt);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const uint16_t* qf = q + frame * n * D;
  uint16_t* of = out + frame * n * DV;

  const int64_t units = (t_end - t_begin + 31) / 32;
  uint4 qa[C::KS], qn[C::KS];
  auto load_q = [&](int64_t u, uint4 (&dst)[C::KS]) {
    const int64_t t = t_begin + u * 32 + col;
    const bool ok = t < t_end;
    const uint16_t* src = qf + t * D + half * 8;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      dst[s] = make_uint4(0, 0, 0, 0);
      if (ok) dst[s] = *reinterpret_cast<const uint4*>(src + s * 16);
    }
  };

  int64_t u = wave;
  if (u < units) load_q(u, qa);
  for (; u < units; u += 4) {
    if (u + 4 < units) load_q(u + 4, qn);
    const int64_t t = t_begin + u * 32 + col;
    uint16_t* dst = of + t * DV + half * 4;
    // one 32-column output block at a time keeps 16 accumulators live
#pragma unroll
    for (int b = 0; b < C::NDB; ++b) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4*>(wt + (b * 32 + col) * C::WROW + s * 16 +
                                                        half * 8);
        acc = mfma32_bf16(w, qa[s], acc);
      }
      if (t < t_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[4 * i + 0], acc[4 * i + 1]);
          pk.y = pack_bf16x2(acc[4 * i + 2], acc[4 * i + 3]);
          *reinterpret_cast<uint2*>(dst + b * 32 + 8 * i) = pk;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qa[s] = qn[s];
  }
}

template <int D, int DV>
struct ReadF32 {
  static constexpr int WROW = DV + 4;
  static constexpr int LDS_BYTES = D * WROW * 4;
  static constexpr int NDB = DV / 32;
};

template <int D, int DV>
__global__ void __launch_bounds__(kThreads)
readout_f32_kernel(const float* __restrict__ q, const float* __restrict__ xf,
                   const float* __restrict__ xb, float* __restrict__ out, int64_t F, int64_t n,
                   int64_t splits, int64_t tokens_per_split) {
  using C = ReadF32<D, DV>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* w = reinterpret_cast<float*>(smem);

  const int64_t split = blockIdx.x % splits;
  const int64_t frame = blockIdx.x / splits;
  const int64_t t_begin = split * tokens_per_split;
  const int64_t t_end = t_begin + tokens_per_split < n ? t_begin + tokens_per_split : n;
  const float* xff = xf + frame * int64_t(D) * DV;
  const float* xbf = xb + frame * int64_t(D) * DV;
  for (int idx = threadIdx.x; idx < D * DV; idx += kThreads) {
    const int kr = idx / DV, j = idx % DV;
    w[kr * C::WROW + j] = 0.5f * (xff[idx] + xbf[idx]);
  }
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const float* qf = q + frame * n * D;
  float* of = out + frame * n * DV;
  const int64_t units = (t_end - t_begin + 31) / 32;
  for (int64_t u = wave; u < units; u += 4) {
    const int64_t t = t_begin + u * 32 + col;
    const bool ok = t < t_end;
    f32x16 acc[C::NDB];
#pragma unroll
    for (int b = 0; b < C::NDB; ++b) acc[b] = f32x16{};
    for (int ks = 0; ks < D / 2; ++ks) {
      const int kr = 2 * ks + half;
      const float qv = ok ? qf[t * D + kr] : 0.0f;
#pragma unroll
      for (int b = 0; b < C::NDB; ++b)
        acc[b] = mfma32_f32(w[kr * C::WROW + b * 32 + col], qv, acc[b]);
    }
    if (ok) {
      float* dst = of + t * DV + half * 4;
#pragma unroll
      for (int b = 0; b < C::NDB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(dst + b * 32 + 8 * i) =
              make_float4(acc[b][4 * i], acc[b][4 * i + 1], acc[b][4 * i + 2], acc[b][4 * i + 3]);
    }
  }
}

template <int D, int DV>
hipError_t launch_readout_t(const Problem& p, const void* q, void* out, hipStream_t s) {
  const int64_t frames = p.B * p.H * p.F;
  // one workgroup per frame; split frames only when there are too few of them to
  // fill the chip
  int64_t splits = 1;
  while (frames * splits < 1024 && p.n > 256 * splits) splits *= 2;
  const int64_t tps = ((p.n + splits - 1) / splits + 31) / 32 * 32;
  splits = (p.n + tps - 1) / tps;
  const int64_t grid = frames * splits;
  if (p.bf16) {
    constexpr int lds = ReadBf16<D, DV>::LDS_BYTES;
    auto kern = readout_bf16_kernel<D, DV>;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), lds, s,
                       static_cast<const uint16_t*>(q), p.xf, p.xb, static_cast<uint16_t*>(out),
                       p.F, p.n, splits, tps);
  } else {
    constexpr int lds = ReadF32<D, DV>::LDS_BYTES;
    auto kern = readout_f32_kernel<D, DV>;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), lds, s,
                       static_cast<const float*>(q), p.xf, p.xb, static_cast<float*>(out), p.F,
                       p.n, splits, tps);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_readout(const Problem& p, const void* q, void* out, hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_readout_t<DD, VV>(p, q, out, s);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda
