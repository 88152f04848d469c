// Device helpers for the gfx950 (CDNA4) VDA kernels: vector types, MFMA wrappers,
// bfloat16 packing, the XCD-aware block remap and the in-LDS SPD inversion.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace vda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // 4 waves per workgroup (the bf16 scan alone uses d / 16 waves)
constexpr int kXcds = 8;       // MI355X: 8 XCDs, workgroups dealt round-robin

template <typename T>
__host__ __device__ constexpr T cmax(T a, T b) { return a > b ? a : b; }

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lane layout: lane l holds row
// (A) / column (B) l%32 and 8 consecutive k values starting at 8*(l/32).
// Result lane layout: column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ f32x16 mfma32_bf16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 32x32x64 FP8 (OCP e4m3) MFMA, fp32 accumulate (scale operands 0: no block scaling).
// Lane l holds row (A) / column (B) l%32 and 32 k values, one per byte; byte p of lane l
// of A multiplies byte p of the lane of B with the same l/32, so A and B formed by the same
// procedure contract over the same 64 k values in whatever order they are held.  Result
// layout as for mfma32_bf16.  Products of e4m3 values are exact in fp32.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 32x32x2 fp32 MFMA.  Lane l holds A[l%32][l/32] and B[l/32][l%32]; result
// layout as for mfma32_bf16.
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 16x16x4 fp32 MFMA.  Lane l holds A[l%16][l/16] and B[l/16][l%16]; result lane
// layout: column l%16, rows 4*(l/16) + r for r = 0..3.
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// float -> bfloat16, round to nearest even, NaN stays NaN: gfx950's packed conversion
// (v_cvt_pk_bf16_f32), one instruction for two values and no branch.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// bits of (bf16(lo), bf16(hi)), lo in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) { return pack_bf16x2(x, 0.0f) & 0xffffu; }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// Split two floats into bfloat16 hi + lo pairs, x - hi - lo = O(2^-17 |x|):
// hi = rne(x), lo = rne(x - hi); each result packs (value a, value b).
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - bf16_bits_to_f32(hi & 0xffffu), b - bf16_bits_to_f32(hi >> 16));
}

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l holds row (A) / column (B) l%16 and
// 8 consecutive k values starting at 8*(l/16); result: column l%16, rows 4*(l/16)+r.
__device__ __forceinline__ f32x4 mfma16_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a),
                                                 __builtin_bit_cast(bf16x8v, b), c, 0, 0, 0);
}

// Dword made of the low (sel=0) or high (sel=1) 16-bit halves of a (low) and b (high).
__device__ __forceinline__ uint32_t interleave16(uint32_t a, uint32_t b, int hi) {
  return __builtin_amdgcn_perm(b, a, hi ? 0x07060302u : 0x05040100u);
}

// Transpose an 8x8 block of 16-bit elements held as 8 rows of 4 dwords:
// out[j] dword p = (in[2p] element j, in[2p+1] element j).
__device__ __forceinline__ void transpose8x8_b16(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1, hi = j & 1;
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4 a = in[2 * p], b = in[2 * p + 1];
      const uint32_t aw = w == 0 ? a.x : w == 1 ? a.y : w == 2 ? a.z : a.w;
      const uint32_t bw = w == 0 ? b.x : w == 1 ? b.y : w == 2 ? b.z : b.w;
      d[p] = interleave16(aw, bw, hi);
    }
    out[j] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// OCP FP8 e4m3 -> bfloat16.  Every e4m3 value is exact in bfloat16 (3 mantissa bits,
// exponents 2^-9 .. 2^8), and gfx950 converts two codes per instruction
// (v_cvt_scalef32_pk_bf16_fp8, scale 1: the codes' own values; the NaN codes give NaN).
// Codes 0 and 1 of `w` (HI = false) or 2 and 3 (HI = true) -> bits of (bf16, bf16), low
// first.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// 8 codes (byte i of the pair = element i) -> 8 bfloat16, element order kept
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 x) {
  return make_uint4(e4m3x2_to_bf16x2<false>(x.x), e4m3x2_to_bf16x2<true>(x.x),
                    e4m3x2_to_bf16x2<false>(x.y), e4m3x2_to_bf16x2<true>(x.y));
}

// Blocked layout of a d x dv float32 matrix in the workspace (Bm and the states X):
// 16-column blocks, then 16-row blocks, then the lane pattern of a 16x16 MFMA tile,
// [row/4 within the tile][column][row%4], so each lane of a tile owns 4 contiguous floats.
__host__ __device__ constexpr int blk_index(int row, int col, int d) {
  return ((((col >> 4) * (d >> 4) + (row >> 4)) * 4 + ((row & 15) >> 2)) * 16 + (col & 15)) * 4 +
         (row & 3);
}

// Mean of two vectors of 8 bfloat16, (a + b) / 2 in fp32, rounded once to bfloat16.
__device__ __forceinline__ uint4 mean_bf16x8(uint4 a, uint4 b) {
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = 0.5f * (__uint_as_float(aw[i] << 16) + __uint_as_float(bw[i] << 16));
    const float hi = 0.5f * (__uint_as_float(aw[i] & 0xffff0000u) + __uint_as_float(bw[i] & 0xffff0000u));
    r[i] = pack_bf16x2(lo, hi);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// Fragment-ordered layout of a d x d bfloat16 plane (the hi and lo planes of Ainv for
// the scan): the 16-row x 32-column operand block (row block r/16, column block c/32)
// of a 16x16x32 MFMA is 1 KB contiguous, in lane order, lane 16*((c%32)/8) + r%16
// holding the 8 consecutive columns it feeds to the MFMA.  One 16-byte load per lane
// then reads a whole operand with a single contiguous wave access.
__host__ __device__ constexpr int frag_index(int row, int col, int d) {
  return ((((row >> 4) * (d >> 5) + (col >> 5)) * 4 + ((col & 31) >> 3)) * 16 + (row & 15)) * 8 +
         (col & 7);
}

// Packed upper triangle of a symmetric d x d bfloat16 plane (A^{-1} is symmetric): the
// 16 x 16 blocks (R, C) with R <= C, block (R, C) at index R*NB - R*(R-1)/2 + (C - R)
// for NB = d/16, each block row-major (element (r, c) of the block at 16 r + c).
// Block (R, C) with R > C is the transpose of block (C, R).
__host__ __device__ constexpr int sym_blocks(int d) { return (d / 16) * (d / 16 + 1) / 2; }
__host__ __device__ constexpr int sym_block(int R, int C, int d) {
  return R * (d / 16) - R * (R - 1) / 2 + (C - R);
}
// element (row, col) of the plane, for row / 16 <= col / 16
__host__ __device__ constexpr int sym_index(int row, int col, int d) {
  return sym_block(row >> 4, col >> 4, d) * 256 + (row & 15) * 16 + (col & 15);
}

// Layout of a d x dv bfloat16 state for the readout: the transpose in fragment order,
// so the operand block of W^T (16 value columns x 32 key rows) that a 16x16x32 MFMA of
// the readout takes is 1 KB contiguous, lane 16*((r%32)/8) + c%16 holding rows
// r..r+7 of column c.  Four consecutive rows (r%4 == 0) are 8 contiguous bytes.
__host__ __device__ constexpr int state_index(int row, int col, int d) {
  return frag_index(col, row, d);
}
// Row order of the states of plans with FP8 inputs (d >= 64): the readout feeds each
// lane two k-steps from one 16-byte load of 16 consecutive FP8 query features, so state
// row r = [r/64][g][h][r%8] (g = (r/16)%4, h = (r/8)%2) must sit where the plain order
// keeps row [r/64][h][g][r%8]: bit 3 of the row moves above bits 4-5.  Rows 4i..4i+3
// stay contiguous.
__host__ __device__ constexpr int paired_row(int r) {
  return (r & ~0x38) | ((r & 0x08) << 2) | ((r & 0x30) >> 1);
}
__host__ __device__ constexpr int state_index_paired(int row, int col, int d) {
  return frag_index(col, paired_row(row), d);
}

// Raw buffer access: the descriptor (base, byte size) lives in SGPRs and must be
// wave-uniform; the hardware range-checks every access against the size, so
// out-of-range loads return zero and out-of-range stores are dropped, with no
// branches around the memory instructions.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
// Cache policy of a buffer access: kCacheNt marks data that is touched once (streamed).
// kCacheStreamOut (SC1 | NT) is for streamed output: in the readout it stores ~1% faster
// than NT alone and ~7% faster than the default policy.  kCacheSc1 (SC1 alone) is for the
// statistics kernel's outputs, which a workgroup writes in one burst at its end, as whole
// 512-byte pieces per store instruction, while the other workgroups stream their reads:
// 6% faster statistics at 768p than the default policy (NT or SC1 | NT were slower, and
// SC1 on stores that fill only half of each 32-byte row was slower too).
constexpr int kCacheDefault = 0, kCacheNt = 2, kCacheSc1 = 16, kCacheStreamOut = 16 | 2;
template <int CPOL = kCacheDefault>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, CPOL));
}
template <int CPOL = kCacheDefault>
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, CPOL));
}
template <int CPOL = kCacheDefault>
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)byte_off, 0, CPOL);
}
template <int CPOL = kCacheDefault>
__device__ __forceinline__ void buffer_store8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint2 v) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, (int)byte_off, 0, CPOL);
}

// Workgroup index remap so that consecutive logical indices land on one XCD.
// Hardware deals workgroup id w to XCD w % 8; logical index i = xcd * per + slot.
// `count` must be the padded grid size (a multiple of 8).
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t count) {
  const int64_t per = count / kXcds;
  return (w % kXcds) * per + (w / kXcds);
}

// In-place inversion of the SPD matrix A = G + lam*I by Gauss-Jordan elimination
// without pivoting (pivots of an SPD matrix are positive Schur complements).
// G is read from LDS (row stride gs floats); each of the 256 threads owns a
// TS x TS tile, TS = D/16, of the result, returned in `a`.
// rowv/colv: LDS scratch of 2*D floats each (pivot row / column, double buffered).
template <int D>
__device__ __forceinline__ void spd_inverse_gj(const float* gsm, int gs, float lam,
                                               float* rowv, float* colv,
                                               float (&a)[D / 16][D / 16]) {
  constexpr int TS = D / 16;
  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) {
      const int gi = tr * TS + i, gj = tc * TS + j;
      a[i][j] = gsm[gi * gs + gj] + (gi == gj ? lam : 0.0f);
    }
  // pivot row / column 0 into slot 0
  if (tr == 0) {
#pragma unroll
    for (int j = 0; j < TS; ++j) rowv[tc * TS + j] = a[0][j];
  }
  if (tc == 0) {
#pragma unroll
    for (int i = 0; i < TS; ++i) colv[tr * TS + i] = a[i][0];
  }
  for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
    for (int kk = 0; kk < TS; ++kk) {
      const int k = kb * TS + kk;
      const int slot = kk & 1;  // TS is even, so k & 1 == kk & 1
      const float* rv = rowv + slot * D;
      const float* cv = colv + slot * D;
      __syncthreads();
      const float p = rv[k];
      const float ip = 1.0f / p;
      float c[TS], r[TS];
#pragma unroll
      for (int i = 0; i < TS; ++i) c[i] = cv[tr * TS + i];
#pragma unroll
      for (int j = 0; j < TS; ++j) r[j] = rv[tc * TS + j] * ip;
      const bool own_row = (tr == kb), own_col = (tc == kb);
      float rk[TS], ck[TS];
#pragma unroll
      for (int j = 0; j < TS; ++j) rk[j] = r[j];
#pragma unroll
      for (int i = 0; i < TS; ++i) ck[i] = -c[i] * ip;
      if (own_row) c[kk] = 0.0f;
      if (own_col) r[kk] = 0.0f;
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TS; ++j) a[i][j] = __builtin_fmaf(-c[i], r[j], a[i][j]);
      if (own_row) {
#pragma unroll
        for (int j = 0; j < TS; ++j) a[kk][j] = rk[j];
      }
      if (own_col) {
#pragma unroll
        for (int i = 0; i < TS; ++i) a[i][kk] = ck[i];
      }
      if (own_row && own_col) a[kk][kk] = ip;
      // publish pivot row / column k+1 into the other slot
      if (k + 1 < D) {
        const int kk1 = (kk + 1) % TS;
        const int kb1 = (kk + 1 == TS) ? kb + 1 : kb;
        float* rv1 = rowv + (slot ^ 1) * D;
        float* cv1 = colv + (slot ^ 1) * D;
        if (tr == kb1) {
#pragma unroll
          for (int j = 0; j < TS; ++j) rv1[tc * TS + j] = a[kk1][j];
        }
        if (tc == kb1) {
#pragma unroll
          for (int i = 0; i < TS; ++i) cv1[tr * TS + i] = a[i][kk1];
        }
      }
    }
  }
}

}  // namespace vda
