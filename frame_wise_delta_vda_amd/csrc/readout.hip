// Stage 3 of the VDA forward pass: the readout.
//
// Every frame reads the bidirectional state out with its queries (linear-attention
// readout; model card introduction, bullet "hybrid architecture": a frame-wise
// linear-attention branch), using the mean of the two directional states after
// that frame's own update:
//   W_f = (X_fwd_f + X_bwd_f) / 2,   O_f = Q_f W_f   (n x dv)
//
// float32 path: one workgroup per frame (or token range), W kept in fp32 in LDS,
// 32x32x2 fp32 MFMA, operands loaded straight from HBM.
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

// bfloat16 path.  Each workgroup owns a contiguous range of 64-token tiles (a tile
// never straddles two frames) and keeps the W^T fragments of the current frame in
// registers.  Q tiles are loaded with 16-byte loads where one workgroup instruction
// covers whole rows (4 KB contiguous), staged through padded LDS, and read back as
// MFMA operands; each wave computes O^T = W^T Q^T for one 32-wide output-column block
// (32x32x16 bf16 MFMA); the bf16 O tile goes back through LDS so the stores are whole
// rows as well.  The next two tiles are always in flight in registers.
template <int D, int DV>
struct ReadBf16 {
  static constexpr int TT = 64;                 // tokens per tile
  static constexpr int QROW = D * 2 + 16;       // bytes per LDS row of Q (padded)
  static constexpr int OROW = DV * 2 + 16;      // bytes per LDS row of O
  static constexpr int WROW = D + 8;            // bf16 per LDS row of W^T
  static constexpr int QCH = D / 8, OCH = DV / 8;        // 16-byte chunks per row
  static constexpr int QLD = TT * QCH / kThreads;        // 16-byte loads per thread per tile
  static constexpr int OST = TT * OCH / kThreads;        // 16-byte stores per thread per tile
  static constexpr int NB = DV / 32;            // 32-wide output column blocks
  static constexpr int NT = TT / 32;            // 32-token sub-tiles
  static constexpr int WPB = 4 / NB < 1 ? 1 : 4 / NB;     // waves per column block
  static constexpr int SPW = NT / WPB < 1 ? 1 : NT / WPB;  // sub-tiles per wave
  static constexpr int KS = D / 16;             // MFMA k-steps
  static constexpr int QS_BYTES = TT * QROW, OS_BYTES = TT * OROW, WT_BYTES = DV * WROW * 2;
  static constexpr int LDS_BYTES = QS_BYTES + OS_BYTES + WT_BYTES;
  static_assert(QLD >= 1 && OST >= 1, "tile too small for the workgroup");
};

template <int D, int DV>
__global__ void __launch_bounds__(kThreads, 2)
readout_bf16_kernel(const uint16_t* __restrict__ q, const float* __restrict__ xf,
                    const float* __restrict__ xb, uint16_t* __restrict__ out, int64_t n,
                    int64_t total_tiles, int64_t tiles_per_frame, int64_t per_wg) {
  using C = ReadBf16<D, DV>;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* qs = smem;
  unsigned char* os = smem + C::QS_BYTES;
  uint16_t* wt = reinterpret_cast<uint16_t*>(smem + C::QS_BYTES + C::OS_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int64_t t_first = blockIdx.x * per_wg;
  const int64_t t_last = (t_first + per_wg < total_tiles) ? t_first + per_wg : total_tiles;
  if (t_first >= t_last) return;

  const int b = wave % C::NB;                    // output column block of this wave
  const int sub0 = (wave / C::NB) * C::SPW;      // first 32-token sub-tile of this wave
  const bool mfma_wave = (wave / C::NB) < C::WPB && sub0 < C::NT;
  constexpr int RPI = kThreads / C::QCH;         // rows per load instruction
  const int lrow = tid / C::QCH, lch = tid % C::QCH;
  constexpr int SRPI = kThreads / C::OCH;
  const int srow = tid / C::OCH, sch = tid % C::OCH;

  uint4 pfa[C::QLD], pfb[C::QLD];
  // Q tiles load through a buffer descriptor bounded by the frame's last row: rows past
  // it read as zero (their outputs are not stored), so the loads carry no branch and the
  // tile two ahead stays in flight.
  auto load_tile = [&](int64_t tile, uint4 (&dst)[C::QLD]) {
    const int64_t frame = tile / tiles_per_frame;
    const int64_t tok0 = (tile % tiles_per_frame) * C::TT;
    const int64_t rows = n - tok0 < C::TT ? n - tok0 : C::TT;
    const auto qrsrc = make_rsrc(q + (frame * n + tok0) * D, uint32_t(rows * D * 2));
#pragma unroll
    for (int i = 0; i < C::QLD; ++i) {
      const int r = i * RPI + lrow;
      dst[i] = buffer_load16(qrsrc, uint32_t(r * D * 2 + lch * 16));
    }
  };

  int64_t cur_frame = -1;
  uint4 wf[C::KS];  // W^T fragments of this wave's column block

  auto step = [&](int64_t tile, uint4 (&pf)[C::QLD]) {
    const int64_t frame = tile / tiles_per_frame;
    const int64_t tok0 = (tile % tiles_per_frame) * C::TT;
    if (frame != cur_frame) {
      // W = (X_fwd + X_bwd) / 2 of the new frame, rounded to bf16, into LDS as W^T
      __syncthreads();
      const float* xff = xf + frame * int64_t(D) * DV;
      const float* xbf = xb + frame * int64_t(D) * DV;
      // the states are stored blocked: each float4 holds rows row..row+3 of one column
      for (int i4 = tid; i4 < D * DV / 4; i4 += kThreads) {
        const int blk = i4 >> 6, g = (i4 >> 4) & 3, col = (blk / (D / 16)) * 16 + (i4 & 15);
        const int row = (blk % (D / 16)) * 16 + 4 * g;
        const float4 a = reinterpret_cast<const float4*>(xff)[i4];
        const float4 c = reinterpret_cast<const float4*>(xbf)[i4];
        *reinterpret_cast<uint2*>(wt + col * C::WROW + row) =
            make_uint2(pack_bf16x2(0.5f * (a.x + c.x), 0.5f * (a.y + c.y)),
                       pack_bf16x2(0.5f * (a.z + c.z), 0.5f * (a.w + c.w)));
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < C::KS; ++s)
        wf[s] = *reinterpret_cast<const uint4*>(wt + (b * 32 + col) * C::WROW + s * 16 + half * 8);
      cur_frame = frame;
    }
    // this tile: registers -> LDS; refill the registers with the tile two ahead
#pragma unroll
    for (int i = 0; i < C::QLD; ++i)
      *reinterpret_cast<uint4*>(qs + (i * RPI + lrow) * C::QROW + lch * 16) = pf[i];
    load_tile(tile + 2 < t_last ? tile + 2 : t_last - 1, pf);  // unconditional: no phi, no copy
    __syncthreads();
    if (mfma_wave) {
#pragma unroll
      for (int si = 0; si < C::SPW; ++si) {
        const int sub = sub0 + si;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          const uint4 qv = *reinterpret_cast<const uint4*>(qs + (sub * 32 + col) * C::QROW +
                                                           s * 32 + half * 16);
          acc = mfma32_bf16(wf[s], qv, acc);
        }
        // lane holds O[token sub*32+col][b*32 + 8i + 4*half + 0..3]
        unsigned char* orow = os + (sub * 32 + col) * C::OROW + (b * 32 + half * 4) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[4 * i + 0], acc[4 * i + 1]);
          pk.y = pack_bf16x2(acc[4 * i + 2], acc[4 * i + 3]);
          *reinterpret_cast<uint2*>(orow + 16 * i) = pk;
        }
      }
    }
    __syncthreads();
    // stores through a buffer descriptor bounded by the frame's last row: rows past it
    // are dropped by the hardware range check, without a branch
    const int64_t rows = n - tok0 < C::TT ? n - tok0 : C::TT;
    const auto orsrc = make_rsrc(out + (frame * n + tok0) * DV, uint32_t(rows * DV * 2));
#pragma unroll
    for (int i = 0; i < C::OST; ++i) {
      const int r = i * SRPI + srow;
      buffer_store16(orsrc, uint32_t(r * DV * 2 + sch * 16),
                     *reinterpret_cast<const uint4*>(os + r * C::OROW + sch * 16));
    }
  };

  load_tile(t_first, pfa);
  load_tile(t_first + 1 < t_last ? t_first + 1 : t_first, pfb);
  for (int64_t tile = t_first; tile < t_last; tile += 2) {
    step(tile, pfa);
    if (tile + 1 < t_last) step(tile + 1, pfb);
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
    const int blk = idx >> 8, g = (idx >> 6) & 3, j = (blk / (D / 16)) * 16 + ((idx >> 2) & 15);
    const int kr = (blk % (D / 16)) * 16 + 4 * g + (idx & 3);
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
  if (p.bf16) {
    using C = ReadBf16<D, DV>;
    const int64_t tpf = (p.n + C::TT - 1) / C::TT;
    const int64_t total = frames * tpf;
    int64_t grid = 2 * int64_t(p.num_cus);        // two persistent workgroups per CU
    if (grid > total) grid = total;
    const int64_t per = (total + grid - 1) / grid;
    grid = (total + per - 1) / per;
    auto kern = readout_bf16_kernel<D, DV>;
    if (C::LDS_BYTES > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), C::LDS_BYTES, s,
                       static_cast<const uint16_t*>(q), p.xf, p.xb, static_cast<uint16_t*>(out),
                       p.n, total, tpf, per);
  } else {
    // one workgroup per frame, split only when there are too few frames to fill the chip
    int64_t splits = 1;
    while (frames * splits < 1024 && p.n > 256 * splits) splits *= 2;
    const int64_t tps = ((p.n + splits - 1) / splits + 31) / 32 * 32;
    splits = (p.n + tps - 1) / tps;
    const int64_t grid = frames * splits;
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
