// Backward pass of the VDA forward: the per-frame adjoint terms.
//
// Training the branch (aiezz page, section 03, and laicaila page, "technical principles":
// bullet "three-stage training adaptation") needs the op's gradient.  With dO the
// gradient of the output, the statistics stage run on (Q, dO) gives dW_f = Q_f^T dO_f,
// and the scan run on (A^{-1}, dW) gives the two adjoint chains scaled by two:
//   S_fwd_f = A_f^{-1} (dW_f + lam S_fwd_{f-1})  = 2 V_f,
//   S_bwd_f = A_f^{-1} (dW_f + lam S_bwd_{f+1})  = 2 U_f,
// both from a zero start, stored in float32 (as are the forward states, recomputed by the
// scan for this pass).  Per frame this file forms, in the layouts the readout kernels take
// as their state (state_index), with dB and M as bf16 hi + lo pairs:
//   WT_f = W_f^T,            W_f = (X_fwd_f + X_bwd_f) / 2          (dQ_f = dO_f W_f^T)
//   DB2_f = [dB hi ; dB lo], dB_f = (S_fwd_f + S_bwd_f) / 2          (dV_f = [K K] DB2_f)
//   Z_f  = [M hi ; M lo ; dB^T hi ; dB^T lo],  M_f = dA_f + dA_f^T,
//          dA_f = -(S_bwd_f X_fwd_f^T + S_fwd_f X_bwd_f^T) / 2       (dK_f = [K K V V] Z_f)
// and for the text (frame 0 of a head), with Gamma = lam (S_bwd_1 + S_fwd_F) / 2:
//   U_0 = A_0^{-1} Gamma,  dB_0 = U_0,  dA_0 = -U_0 X_text^T,  X_text = A_0^{-1} Bm_0.
// The arithmetic is fp32 on the vector units: it is O(d^3) per frame, against the
// O(n d^2) token work of the readouts that consume these matrices.
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

// position of the 8-element run (rows 8 (e / 8) .. +7 of one column) that state-order
// chunk q holds, for a D-row state: returns (row0, col)
template <int D>
__device__ __forceinline__ void chunk_rc(int q, int& row0, int& col) {
  const int c15 = q & 15, t = q >> 4, g = t & 3, u = t >> 2;
  const int rb = u % (D / 32), cb = u / (D / 32);
  row0 = rb * 32 + g * 8;
  col = cb * 16 + c15;
}

// bf16 hi / lo of x: hi = rne(x), lo = rne(x - hi)
__device__ __forceinline__ float lo_part(float x) { return x - bf16_bits_to_f32(f32_to_bf16_bits(x)); }

// Threads of a per-frame workgroup: 8 waves, so the float32 state loads, conversions and
// stores that dominate a frame have twice the work in flight that 4 waves had at one
// workgroup per CU (the planes take 139 KB of LDS).
constexpr int kBwdThreads = 512;

template <int D, int DV>
struct BwdFrame {
  static constexpr int TR = D + 8;                // bf16 per LDS plane row (row c: value feature c)
  static constexpr int PROW = D + 4;              // floats per LDS row of P (D x D)
  static constexpr int LDS_BYTES = cmax(4 * DV * TR * 2, D * PROW * 4);
  static constexpr int ZR = 2 * D + 2 * DV;       // rows of Z: M hi, M lo, dB^T hi, dB^T lo
  static_assert(D % 32 == 0 && DV % 16 == 0, "P tiles of 32 x 32, k-steps of 16");
};

// One workgroup per video frame.  Inputs are float32 and blocked (blk_index): the forward
// states X_fwd, X_bwd recomputed for the backward pass, and the adjoint chains S_fwd, S_bwd.
// Outputs, in the readout's state order (bf16): WT = W^T; DB2 = [dB hi ; dB lo]; Z = [M hi ;
// M lo ; dB^T hi ; dB^T lo] -- the gradient products take each factor as hi + lo, since
// for ill-conditioned frames dB and M are large along directions that K maps to small
// values, and one bf16 rounding there shows in K dB.
template <int D, int DV>
__device__ __forceinline__ void frame_terms(const float* __restrict__ xf, const float* __restrict__ xb,
                                            const float* __restrict__ sf, const float* __restrict__ sb,
                                            uint16_t* __restrict__ wt, uint16_t* __restrict__ db2,
                                            uint16_t* __restrict__ z, int64_t fr, unsigned char* smem) {
  using C = BwdFrame<D, DV>;
  const int64_t base = fr * int64_t(D) * DV;
  const float* XF = xf + base;
  const float* XB = xb + base;
  const float* SF = sf + base;
  const float* SB = sb + base;
  const int tid = threadIdx.x;

  // 1. element-wise outputs straight from the inputs, each adjoint state read once.  In the
  //    blocked layout four consecutive rows of a column are one float4; a thread takes 4 rows x
  //    8 columns and writes, from the same registers, the outputs that run along a row (WT and
  //    the dB^T rows of Z: 8 consecutive value features of one input feature, 16 bytes) and its
  //    half of those that run down a column (DB2: 8 consecutive rows of a column, 8 bytes of
  //    the 16).  The forward states are read here only for WT (widths other than d = dv = 128).
  auto chunk_of = [](int row0, int col, int R) -> int {  // inverse of chunk_rc for an R-row state
    return (((col >> 4) * (R / 32) + (row0 >> 5)) * 4 + ((row0 & 31) >> 3)) * 16 + (col & 15);
  };
  uint16_t* dbf = db2 + fr * int64_t(2 * D) * DV;
  uint16_t* zf = z + fr * int64_t(C::ZR) * D;
  const bool want_wt = wt != nullptr;
  for (int u = tid; u < (D / 4) * (DV / 8); u += kBwdThreads) {
    const int i0 = 4 * (u % (D / 4)), c0 = 8 * (u / (D / 4));
    float4 xf4[8], xb4[8], sf4[8], sb4[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int e = blk_index(i0, c0 + m, D) / 4;
      sf4[m] = reinterpret_cast<const float4*>(SF)[e];
      sb4[m] = reinterpret_cast<const float4*>(SB)[e];
    }
    if (want_wt) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int e = blk_index(i0, c0 + m, D) / 4;
        xf4[m] = reinterpret_cast<const float4*>(XF)[e];
        xb4[m] = reinterpret_cast<const float4*>(XB)[e];
      }
    }
    auto comp = [](const float4& a, int r) { return r == 0 ? a.x : r == 1 ? a.y : r == 2 ? a.z : a.w; };
    float db[4][8];  // dB = (S_bwd + S_fwd) / 2 at rows i0 + r, columns c0 + m
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < 8; ++m) db[r][m] = 0.5f * (comp(sb4[m], r) + comp(sf4[m], r));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int m = 0; m < 8; m += 2) {
        h[m / 2] = pack_bf16x2(db[r][m], db[r][m + 1]);
        l[m / 2] = pack_bf16x2(lo_part(db[r][m]), lo_part(db[r][m + 1]));
      }
      // Z rows 2D + c0.. (dB^T hi) and 2D + DV + c0.. (lo) of column i0 + r
      reinterpret_cast<uint4*>(zf)[chunk_of(2 * D + c0, i0 + r, C::ZR)] = make_uint4(h[0], h[1], h[2], h[3]);
      reinterpret_cast<uint4*>(zf)[chunk_of(2 * D + DV + c0, i0 + r, C::ZR)] = make_uint4(l[0], l[1], l[2], l[3]);
      if (want_wt) {
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 8; m += 2)
          w[m / 2] = pack_bf16x2(0.5f * (comp(xf4[m], r) + comp(xb4[m], r)),
                                 0.5f * (comp(xf4[m + 1], r) + comp(xb4[m + 1], r)));
        // WT: rows c0.. (value features) of column i0 + r
        reinterpret_cast<uint4*>(wt + base)[chunk_of(c0, i0 + r, DV)] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    // DB2 rows (i0 & ~7) .. +7 of column c0 + m, hi then lo: this thread's 4 rows are the
    // first or the second 8 bytes of each chunk
    const int half = (i0 >> 2) & 1;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int c = c0 + m;
      const uint2 hv = make_uint2(pack_bf16x2(db[0][m], db[1][m]), pack_bf16x2(db[2][m], db[3][m]));
      const uint2 lv = make_uint2(pack_bf16x2(lo_part(db[0][m]), lo_part(db[1][m])),
                                  pack_bf16x2(lo_part(db[2][m]), lo_part(db[3][m])));
      reinterpret_cast<uint2*>(dbf)[2 * chunk_of(i0 & ~7, c, 2 * D) + half] = hv;
      reinterpret_cast<uint2*>(dbf)[2 * chunk_of(D + (i0 & ~7), c, 2 * D) + half] = lv;
    }
  }

  // 2. P = S_bwd X_fwd^T + S_fwd X_bwd^T (D x D) on the 32x32x16 bf16 MFMA with split
  //    operands (S = S_hi + S_lo, X likewise; S_hi X_hi + S_hi X_lo + S_lo X_hi leaves an
  //    error of order 2^-16 of the products, as in the scan), in two passes, each with the
  //    hi / lo planes of one S and one X in LDS laid out value-feature-major ([c][i]): the
  //    operands (8 consecutive value features of one row of S or X) are then two
  //    transposing reads, as in the statistics kernel.  Wave w owns the 32-row block w of
  //    P when D = 128 (the 32-column tiles of all rows otherwise, split over the waves).
  constexpr int TR = C::TR;
  constexpr int PL = DV * TR;  // bf16 per plane
  uint16_t* pl = reinterpret_cast<uint16_t*>(smem);  // [S hi, S lo, X hi, X lo]
  auto load_planes = [&](const float* M, uint16_t* hi, uint16_t* lo) {
    for (int g = tid; g < D * DV / 4; g += kBwdThreads) {
      const int c15 = g & 15, t = g >> 4, q4 = t & 3, u = t >> 2;
      const int i = (u % (D / 16)) * 16 + q4 * 4, c = (u / (D / 16)) * 16 + c15;
      const float4 x = reinterpret_cast<const float4*>(M)[g];  // rows i..i+3 of column c
      uint32_t h0, l0, h1, l1;
      split_bf16x2(x.x, x.y, h0, l0);
      split_bf16x2(x.z, x.w, h1, l1);
      *reinterpret_cast<uint2*>(hi + c * TR + i) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lo + c * TR + i) = make_uint2(l0, l1);
    }
  };
  const int lane = tid & 63, wave = tid >> 6;
  const int fr_off = (8 * (lane >> 5) + ((lane & 15) >> 2)) * TR + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto frag = [&](const uint16_t* plane, int k0, int f0) -> uint4 {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const uint16_t* q = plane + k0 * TR + fr_off + f0;
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(q));
    const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(q + 4 * TR));
    const uint2 xl = __builtin_bit_cast(uint2, x), yl = __builtin_bit_cast(uint2, y);
    return make_uint4(xl.x, xl.y, yl.x, yl.y);
  };
  constexpr int NT = D / 32;              // 32 x 32 tiles per side of P
  constexpr int NW = kBwdThreads / 64;
  constexpr int TPW = NT * NT / NW > 0 ? NT * NT / NW : 1;  // tiles per wave
  f32x16 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x16{};
  auto tile_of = [&](int t, int& ti, int& tj) {  // tile t of this wave
    const int idx = wave * TPW + t;
    ti = idx / NT;
    tj = idx % NT;
  };
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    load_planes(pass == 0 ? SB : SF, pl, pl + PL);
    load_planes(pass == 0 ? XF : XB, pl + 2 * PL, pl + 3 * PL);
    __syncthreads();
    if (wave * TPW < NT * NT) {
      for (int k0 = 0; k0 < DV; k0 += 16) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          int ti, tj;
          tile_of(t, ti, tj);
          const uint4 sh = frag(pl, k0, 32 * ti), sl = frag(pl + PL, k0, 32 * ti);
          const uint4 xh = frag(pl + 2 * PL, k0, 32 * tj), xl = frag(pl + 3 * PL, k0, 32 * tj);
          acc[t] = mfma32_bf16(sh, xh, acc[t]);
          acc[t] = mfma32_bf16(sh, xl, acc[t]);
          acc[t] = mfma32_bf16(sl, xh, acc[t]);
        }
      }
    }
    __syncthreads();
  }
  float* LP = reinterpret_cast<float*>(smem);
  if (wave * TPW < NT * NT) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      int ti, tj;
      tile_of(t, ti, tj);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        LP[(32 * ti + mfma32_row(e, lane)) * C::PROW + 32 * tj + (lane & 31)] = acc[t][e];
    }
  }
  __syncthreads();

  // 3. Z rows 0..2D-1: M = dA + dA^T = -(P + P^T) / 2, hi then lo
  for (int qc = tid; qc < C::ZR * D / 8; qc += kBwdThreads) {
    int r0, c;
    chunk_rc<C::ZR>(qc, r0, c);
    if (r0 >= 2 * D) continue;
    const bool lo = r0 >= D;
    const int i0 = lo ? r0 - D : r0;
    uint32_t w[4];
#pragma unroll
    for (int m = 0; m < 8; m += 2) {
      const int r = i0 + m;
      const float a = -0.5f * (LP[r * C::PROW + c] + LP[c * C::PROW + r]);
      const float b = -0.5f * (LP[(r + 1) * C::PROW + c] + LP[c * C::PROW + r + 1]);
      w[m / 2] = lo ? pack_bf16x2(lo_part(a), lo_part(b)) : pack_bf16x2(a, b);
    }
    reinterpret_cast<uint4*>(zf)[qc] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The text frame of each head: one workgroup per (b, h), fp32 through LDS.
//   Gamma = lam (S_bwd_1 + S_fwd_F) / 2,  X_text = A_0^{-1} Bm_0,  U_0 = A_0^{-1} Gamma,
//   DB2_text = [U_0 hi ; lo],  Z_text = [M hi ; M lo ; U_0^T hi ; lo] with M = -(P + P^T),
//   P = U_0 X_text^T.  A_0^{-1} arrives as the packed bf16 hi / lo planes of the statistics.
template <int D, int DV>
struct BwdText {
  static constexpr int AROW = D + 1;
  static constexpr int RROW = DV + 1;
  static constexpr int ASZ = D * cmax(AROW, RROW);  // A_0^{-1}, later U_0
  static constexpr int LDS_BYTES = (ASZ + D * RROW) * 4;
};

template <int D, int DV>
__device__ __forceinline__ void text_terms(const uint16_t* __restrict__ ainv, const float* __restrict__ bm,
                                           const float* __restrict__ sf, const float* __restrict__ sb,
                                           uint16_t* __restrict__ db2_text, uint16_t* __restrict__ z_text,
                                           int64_t F, float lam, int64_t bh, unsigned char* smem) {
  using C = BwdText<D, DV>;
  float* LA = reinterpret_cast<float*>(smem);   // A_0^{-1} [D][AROW]
  float* LR = LA + C::ASZ;                       // right-hand sides / results [D][RROW]
  float* LU = LA;                                // U_0 [D][RROW], over A once it is used
  const int tid = threadIdx.x;
  const int64_t F1 = F + 1;
  const uint16_t* hi = ainv + bh * F1 * int64_t(2 * D * D);
  const uint16_t* lo = hi + sym_blocks(D) * 256;
  for (int e = tid; e < D * D; e += kBwdThreads) {
    const int r = e / D, c = e % D;
    const int rr = (r >> 4) <= (c >> 4) ? r : c, cc = (r >> 4) <= (c >> 4) ? c : r;
    const int idx = sym_index(rr, cc, D);
    LA[r * C::AROW + c] = bf16_bits_to_f32(hi[idx]) + bf16_bits_to_f32(lo[idx]);
  }
  const float* bm0 = bm + bh * F1 * int64_t(D) * DV;
  for (int e = tid; e < D * DV; e += kBwdThreads) {
    const int r = e / DV, c = e % DV;
    LR[r * C::RROW + c] = bm0[blk_index(r, c, D)];
  }
  __syncthreads();
  constexpr int RI = D / 16, RJ = DV / 16;
  const int ti = tid >> 4, tj = tid & 15;
  const bool comp = tid < 256;  // the 8 x 8 blocks of the products: threads 0..255
  auto solve_product = [&](float (&y)[RI][RJ]) {
#pragma unroll
    for (int a = 0; a < RI; ++a)
#pragma unroll
      for (int b = 0; b < RJ; ++b) y[a][b] = 0.0f;
    for (int k = 0; k < D; ++k) {
#pragma unroll
      for (int a = 0; a < RI; ++a) {
        const float av = LA[(ti * RI + a) * C::AROW + k];
#pragma unroll
        for (int b = 0; b < RJ; ++b) y[a][b] = __builtin_fmaf(av, LR[k * C::RROW + tj * RJ + b], y[a][b]);
      }
    }
  };
  float xt[RI][RJ], u0[RI][RJ];
  if (comp) solve_product(xt);             // X_text
  __syncthreads();
  // Gamma = lam (S_bwd_1 + S_fwd_F) / 2 (frame f of a chain at index f - 1)
  const float* s1 = sb + (bh * F + 0) * int64_t(D) * DV;
  const float* sF = sf + (bh * F + (F - 1)) * int64_t(D) * DV;
  for (int e = tid; e < D * DV; e += kBwdThreads) {
    const int r = e / DV, c = e % DV;
    const int idx = blk_index(r, c, D);
    LR[r * C::RROW + c] = 0.5f * lam * (s1[idx] + sF[idx]);
  }
  __syncthreads();
  if (comp) solve_product(u0);             // U_0
  __syncthreads();
  if (comp) {
#pragma unroll
    for (int a = 0; a < RI; ++a)
#pragma unroll
      for (int b = 0; b < RJ; ++b) {
        LU[(ti * RI + a) * C::RROW + tj * RJ + b] = u0[a][b];
        LR[(ti * RI + a) * C::RROW + tj * RJ + b] = xt[a][b];
      }
  }
  __syncthreads();
  auto put = [&](uint16_t* dst, int r, int c, int R, float x) {  // hi at row r, lo at row r + R
    dst[state_index(r, c, 2 * R)] = uint16_t(f32_to_bf16_bits(x));
    dst[state_index(r + R, c, 2 * R)] = uint16_t(f32_to_bf16_bits(lo_part(x)));
  };
  uint16_t* dbt = db2_text + bh * int64_t(2 * D) * DV;
  for (int e = tid; e < D * DV; e += kBwdThreads) {
    const int r = e / DV, c = e % DV;
    put(dbt, r, c, D, LU[r * C::RROW + c]);
  }
  constexpr int ZR = 2 * D + 2 * DV;
  uint16_t* zt = z_text + bh * int64_t(ZR) * D;
  for (int e = tid; e < DV * D; e += kBwdThreads) {  // rows 2D + c (hi), 2D + DV + c (lo): U_0^T
    const int c = e / D, i = e % D;
    const float x = LU[i * C::RROW + c];
    zt[state_index(2 * D + c, i, ZR)] = uint16_t(f32_to_bf16_bits(x));
    zt[state_index(2 * D + DV + c, i, ZR)] = uint16_t(f32_to_bf16_bits(lo_part(x)));
  }
  for (int e = tid; e < D * D; e += kBwdThreads) {  // rows i (hi), D + i (lo): M = -(P + P^T)
    const int i = e / D, j = e % D;
    float pij = 0.0f, pji = 0.0f;
    for (int c = 0; c < DV; ++c) {
      pij = __builtin_fmaf(LU[i * C::RROW + c], LR[j * C::RROW + c], pij);
      pji = __builtin_fmaf(LU[j * C::RROW + c], LR[i * C::RROW + c], pji);
    }
    const float x = -(pij + pji);
    zt[state_index(i, j, ZR)] = uint16_t(f32_to_bf16_bits(x));
    zt[state_index(D + i, j, ZR)] = uint16_t(f32_to_bf16_bits(lo_part(x)));
  }
}

// One launch for both: the text workgroups (one per head) come first in the grid, so they
// run beside the frame workgroups instead of after them.
template <int D, int DV>
__global__ void __launch_bounds__(kBwdThreads)
bwd_frames_kernel(const float* __restrict__ xf, const float* __restrict__ xb,
                  const float* __restrict__ sf, const float* __restrict__ sb,
                  uint16_t* __restrict__ wt, uint16_t* __restrict__ db2, uint16_t* __restrict__ z,
                  const uint16_t* __restrict__ ainv, const float* __restrict__ bm,
                  uint16_t* __restrict__ db2_text, uint16_t* __restrict__ z_text, int64_t F, float lam,
                  int64_t text_blocks) {
  extern __shared__ __align__(16) unsigned char smem[];
  if (int64_t(blockIdx.x) < text_blocks)
    text_terms<D, DV>(ainv, bm, sf, sb, db2_text, z_text, F, lam, blockIdx.x, smem);
  else
    frame_terms<D, DV>(xf, xb, sf, sb, wt, db2, z, blockIdx.x - text_blocks, smem);
}

template <int D, int DV>
hipError_t launch_bwd_frames_t(const BwdProblem& b, hipStream_t s, bool prepare) {
  constexpr int lds = cmax(BwdFrame<D, DV>::LDS_BYTES, BwdText<D, DV>::LDS_BYTES);
  auto kern = bwd_frames_kernel<D, DV>;
  if (prepare)
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               lds);
  const int64_t BH = b.p.B * b.p.H;
  if (BH == 0 || b.p.F == 0) return hipSuccess;
  const int64_t text_blocks = b.p.T > 0 ? BH : 0;
  hipLaunchKernelGGL(kern, dim3(unsigned(text_blocks + BH * b.p.F)), dim3(kBwdThreads), lds, s, b.xf32, b.xb32,
                     b.sf, b.sb, b.wt, b.db2, b.z, reinterpret_cast<const uint16_t*>(b.p.ainv), b.p.bm,
                     b.db2_text, b.z_text, b.p.F, b.p.lam, text_blocks);
  return hipGetLastError();
}

__global__ void zero_kernel(uint4* __restrict__ p, int64_t n16, uint8_t* __restrict__ tail, int64_t ntail) {
  for (int64_t i = blockIdx.x * int64_t(kThreads) + threadIdx.x; i < n16; i += int64_t(gridDim.x) * kThreads)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

// Zero a device buffer with a kernel (so the call may sit in a captured graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = int64_t(bytes / 16), ntail = int64_t(bytes % 16);
  int64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, static_cast<uint4*>(p), n16,
                     static_cast<uint8_t*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

hipError_t launch_bwd_frames(const BwdProblem& b, hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (b.p.d == DD && b.p.dv == VV) return launch_bwd_frames_t<DD, VV>(b, s, false);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

hipError_t prepare_bwd_frames(const Problem& p) {
  BwdProblem b{};
  b.p = p;
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_bwd_frames_t<DD, VV>(b, nullptr, true);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda
