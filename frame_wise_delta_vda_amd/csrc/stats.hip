// Stage 1 of the VDA forward pass: per-frame normal-equation statistics.
//
// For every (batch, head) and every frame f (index 0 = the text tokens, written
// once into the state at initialisation; 1..F = video frames) this computes
//   G_f = K_f^T K_f  (d x d),   Bm_f = K_f^T V_f  (d x dv, blocked layout),
//   Ainv_f = (lam I + G_f)^{-1},
// the statistics through which all spatial tokens of a frame jointly set the new
// state (VDN-MiniMax-H3 pages: aiezz section 03 and laicaila "technical
// principles", bullets "Video Delta Attention" and "dual text injection").
//
// One workgroup per (b, h, frame).  K and V stream once through LDS in chunks of
// 64 tokens; G and Bm accumulate in MFMA registers (fp32).  The reduction runs
// over tokens, so both MFMA operands need 8 consecutive tokens of one feature per
// lane:
//  - d = dv = 128: chunks are staged in LDS token-major exactly as loaded, two chunks
//    in flight per thread, and each operand is formed by two transposing LDS reads
//    (ds_read_b64_tr_b16); with FP8 inputs the codes stay FP8 in LDS, operands come from
//    transposing 8-bit reads (ds_read_b64_tr_b8) and G and Bm run on the FP8 MFMA;
//  - other widths: each lane loads an 8-token x 8-feature block with 16-byte loads (8-byte
//    loads of FP8 codes, converted exactly to bfloat16), transposes it in registers
//    (v_perm_b32) and stores it token-contiguous into LDS, from where operands are read
//    with 16-byte LDS loads.
// After the last chunk the workgroup inverts lam I + G: at d = 128 by a blocked
// symmetric sweep on the MFMA accumulators, at smaller d by Gauss-Jordan in LDS.  Bm
// and Ainv go to the workspace.
#include <type_traits>

#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

// -(lam I + G)^{-1} in place, for d = 128, with G held in the MFMA accumulators of the
// four waves of a workgroup: wave w holds rows 32w..32w+31 as four 32x32 tiles t[c]
// (columns 32c..32c+31, lane l: column l%32, register e: row mfma32_row(e, l)).
//
// Blocked symmetric sweep.  Sweeping an SPD matrix on every index in turn gives minus
// its inverse; sweeping a block K of 16 indices at once is, with the old panel
// P = M[K,:] (= M[:,K]^T), its rows swept on the pivot columns W (which holds
// S = -M[K,K]^{-1} on those columns):
//   M <- M - P^T W,  then  M[K,:] = W,  M[:,K] = W^T,  M[K,K] = S.
// Rounding makes M drift from symmetric, and the update takes panel rows for panel
// columns, so P is taken as the mean of the panel rows and the transposed panel columns
// (without it the inverse of an ill-conditioned frame loses two orders of magnitude of
// accuracy).  W is swept inside each wave (every wave its own 32 columns plus a copy of
// the pivot columns); forming W as -S P instead loses about one more.  The rank-16
// update runs on fp32 MFMA straight on the accumulator tiles -- 8 panels, two barriers
// each.  lds needs 3 * 2 * 16 * kPbs floats.
constexpr int kPbs = 132;  // floats per LDS row of a panel (128 + pad)

__device__ __forceinline__ void sweep_neg_inverse_128(f32x16 (&t)[4], float* lds, int wave,
                                                      int lane) {
  float* pb = lds;                  // [2][16][kPbs] old panel rows M[K,:]
  float* cb = lds + 2 * 16 * kPbs;  // [2][16][kPbs] old panel columns, transposed: M[:,K]^T
  float* wb = lds + 4 * 16 * kPbs;  // [2][16][kPbs] W (S in the pivot columns)
  const int l32 = lane & 31, h = lane >> 5;
  const int c16 = lane & 15;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int wo = p >> 1, hp = p & 1, b = p & 1;
    float* P = pb + b * 16 * kPbs;
    float* Pc = cb + b * 16 * kPbs;
    float* Wb = wb + b * 16 * kPbs;
    // 1. the owner wave publishes the 16 panel rows, every wave its rows of the 16 panel
    // columns.  The old panel used below is their mean: rounding makes the swept matrix
    // drift from symmetric, and the update takes panel rows for panel columns.
    if (wave == wo) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 8 * hp; e < 8 * hp + 8; ++e)
          P[(mfma32_row(e, lane) - 16 * hp) * kPbs + 32 * c + l32] = t[c][e];
    }
    if ((l32 >> 4) == hp) {
#pragma unroll
      for (int e = 0; e < 16; ++e) Pc[(l32 - 16 * hp) * kPbs + 32 * wave + mfma32_row(e, lane)] = t[wo][e];
    }
    __syncthreads();
    // 2. sweep the 16 panel rows on the 16 pivot columns.  Lane l < 32 takes column
    // 32 wave + l, lanes 32..63 a copy of pivot column 16p + l%16; a lane holds its
    // column's 16 rows, so the pivot row is a register and the pivot column comes from
    // lane 32 + kk by readlane.  Afterwards the panel holds W off the pivot columns and
    // S = -M[K,K]^{-1} on them.
    const int col = lane < 32 ? 32 * wave + lane : 16 * p + c16;
    // The pivot column's own update (m -> m / pivot) is kept as a per-lane scale sc and
    // applied once after the 16 steps: a lane stores its column divided by sc, and every
    // later step's update m -= ck * (m[kk] / pivot) holds for the stored values as well.
    float m[16], sc = 1.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = 0.5f * (P[r * kPbs + col] + Pc[r * kPbs + col]);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float ck[16];  // the pivot column, not yet pivoted, so stored unscaled
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ck[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m[r]), 32 + kk));
      const float ip = __builtin_amdgcn_rcpf(ck[kk]);
      const bool isk = col == 16 * p + kk;
      const float rki = isk ? 0.0f : m[kk] * ip;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r != kk) m[r] = __builtin_fmaf(-ck[r], rki, m[r]);
      m[kk] = isk ? -1.0f : m[kk] * ip;
      sc = isk ? sc * ip : sc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] *= sc;
    // 3. this wave's 32 columns of the swept panel
    if (lane < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Wb[r * kPbs + col] = m[r];
    }
    __syncthreads();
    // 4. M -= P^T W on the accumulator tiles (k = 2s + l/32 per 32x32x2 MFMA)
    {
      float a[8], bw[8][4];  // all operands first, so the LDS reads overlap
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int k = 2 * s + h;
        a[s] = -0.5f * (P[k * kPbs + 32 * wave + l32] + Pc[k * kPbs + 32 * wave + l32]);
#pragma unroll
        for (int c = 0; c < 4; ++c) bw[s][c] = Wb[k * kPbs + 32 * c + l32];
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMA chain
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) t[c] = mfma32_f32(a[s], bw[s][c], t[c]);
    }
    // 5. panel rows become W (S in the pivot block), panel columns W^T
    if (wave == wo) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 8 * hp; e < 8 * hp + 8; ++e)
          t[c][e] = Wb[(mfma32_row(e, lane) - 16 * hp) * kPbs + 32 * c + l32];
    }
    {
      const bool kcol = (l32 >> 4) == hp;
      const float* src = Wb + (kcol ? l32 - 16 * hp : 0) * kPbs + 32 * wave + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v4 = *reinterpret_cast<const float4*>(src + 8 * q);
        if (kcol) {
          t[wo][4 * q + 0] = v4.x;
          t[wo][4 * q + 1] = v4.y;
          t[wo][4 * q + 2] = v4.z;
          t[wo][4 * q + 3] = v4.w;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- bfloat16 inputs
// sym_tiles, the d = 128 split of the 32x32 output tiles over the four waves.  Wave w
// holds the K operand fragments of all four 32-feature blocks, rotated so that a[i] is
// block (w + i) % 4 (a[0], its own block, is also the column operand of its G tiles), and
// accumulates
//   acc[0] = G(w, w),  acc[1] = G(w, w + 1),  acc[2] = G(w, w + 2) (waves 0 and 1 only),
//   acc[3 + i] = Bm((w + i) % 4, w),
// block indices mod 4.  That is each of the ten G tiles on and above the block diagonal
// once (G is symmetric; the epilogue writes the mirror of each off-diagonal tile) and all
// sixteen Bm tiles: 7, 7, 6 and 6 MFMAs and 5 operand fragments per wave and k-step.
template <int D, int DV>
struct StatsBf16 {
  static constexpr int TC = 64;                  // tokens per chunk
  static constexpr int ROW = TC + 8;             // bf16 per LDS row (144 B: conflict-free reads)
  static constexpr int NK = D / 32, NV = DV / 32, NC = NK + NV;
  static constexpr int RPW = 4 / NK;             // waves sharing one 32-row block of G
  static constexpr int CPW = (NC + RPW - 1) / RPW;  // 32x32 output tiles per wave
  // d = 128: wave j accumulates column tile j of Bm over all four row blocks and its share
  // of the ten tiles on and above the diagonal of G (sym_tiles); other widths: wave row
  // blocks as above
  static constexpr bool COLW = D == 128;
  // d = dv = 128: every thread loads, and waves split evenly between K and V
  static constexpr bool DEEP = D == 128 && DV == 128;
  static constexpr int ACC = COLW ? 7 : CPW;
  static constexpr int NSEG = (D + DV) / 8;      // 8-feature segments per token (K then V)
  // d = dv = 128 stage token-major instead: a row per token (K then V, padded to 576 B so
  // the transposing LDS reads of four consecutive rows hit distinct banks)
  static constexpr int TROW = D + DV + 32;
  static constexpr int BUF = DEEP ? TC * TROW : (D + DV) * ROW;  // bf16 per staging buffer
  // d = dv = 128 with FP8 inputs: raw codes, 128-token chunks, rows of 288 bytes
  static constexpr int TC8 = 128;
  static constexpr int TROW8 = 288;
  static constexpr int BUF8 = TC8 * TROW8;       // bytes per FP8 staging buffer
  static constexpr int STAGE_BYTES = cmax(2 * BUF * 2, DEEP ? 2 * BUF8 : 0);
  static constexpr int GS = D + 4;               // floats per LDS row of G
  static constexpr int G_BYTES = D * GS * 4;
  static constexpr int MAIN_BYTES = cmax(STAGE_BYTES, G_BYTES);
  static constexpr int LDS_BYTES = MAIN_BYTES + 4 * D * 4;  // + pivot row/col buffers
};

// In: uint16_t (bfloat16 inputs) or uint8_t (FP8 e4m3 inputs, converted to bfloat16 as
// they are written to LDS, so everything after the staging is the same).
// MODE kStatsBm computes Bm = K^T V alone (no G, no inverse, nothing written to ainv): the
// backward pass's dW = Q^T dO.  MODE kStatsBmDq (d = dv = 128, bfloat16) also forms, from
// the same staged chunks of V = dO, the backward pass's dQ = dO W^T, with
// W = (X_fwd + X_bwd) / 2 taken from the float32 blocked states xf32 / xb32.
enum : int { kStatsGram = 0, kStatsBm = 1, kStatsBmDq = 2 };
template <int D, int DV, typename In, int MODE = kStatsGram>
__global__ void __launch_bounds__(kThreads, 2)
stats_bf16_kernel(const In* __restrict__ k, const In* __restrict__ v,
                  const In* __restrict__ tk, const In* __restrict__ tv,
                  float* __restrict__ ainv, float* __restrict__ bm,
                  int64_t F, int64_t n, int64_t T, float lam,
                  const float* __restrict__ xf32, const float* __restrict__ xb32, uint16_t* __restrict__ dq) {
  using C = StatsBf16<D, DV>;
  constexpr bool GRAM = MODE == kStatsGram;
  constexpr bool DQ = MODE == kStatsBmDq;
  static_assert(!DQ || (C::DEEP && sizeof(In) == 2), "dQ is formed at d = dv = 128, bfloat16");
  constexpr bool FP8 = sizeof(In) == 1;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem);

  const int64_t F1 = F + 1;
  const int64_t fi = blockIdx.x % F1;          // 0 = text, 1..F = frames
  const int64_t bh = blockIdx.x / F1;
  const In* kp;
  const In* vp;
  int64_t ntok;
  if (fi == 0) {
    kp = tk + bh * T * D;
    vp = tv + bh * T * DV;
    ntok = T;
  } else {
    kp = k + ((bh * F + (fi - 1)) * n) * D;
    vp = v + ((bh * F + (fi - 1)) * n) * DV;
    ntok = n;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // loader role: token group tg (8 tokens), 8-feature segment seg of K (seg < D/8) or V
  const int tg = tid & 7, seg = tid >> 3;
  const bool loader = C::DEEP || seg < C::NSEG;
  const bool seg_is_k = seg < D / 8;
  const In* src = seg_is_k ? kp + seg * 8 : vp + (seg - D / 8) * 8;
  const int64_t src_stride = seg_is_k ? D : DV;
  const int lds_row0 = seg * 8;  // transposed rows 8*seg .. 8*seg+7 (K rows, then V rows)

  // compute role: row block rb of G (and Bm), column tiles c = jj*RPW + cofs
  const int rb = wave % C::NK;
  const int cofs = wave / C::NK;

  f32x16 acc[C::ACC];
#pragma unroll
  for (int j = 0; j < C::ACC; ++j) acc[j] = f32x16{};

  const int64_t nchunks = (ntok + C::TC - 1) / C::TC;

  // 8 features of one token: 16 bytes (bfloat16) or 8 (FP8)
  using Raw = typename std::conditional<FP8, uint2, uint4>::type;
  auto load_chunk = [&](int64_t ch, Raw (&r)[8]) {
    const int64_t t0 = ch * C::TC + tg * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (FP8) r[i] = make_uint2(0, 0);
      else r[i] = make_uint4(0, 0, 0, 0);
      if (loader && t0 + i < ntok)
        r[i] = *reinterpret_cast<const Raw*>(src + (t0 + i) * src_stride);
    }
  };
  auto store_chunk = [&](int buf, const Raw (&r)[8]) {
    if (!loader) return;
    uint4 x[8], c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (FP8) x[i] = e4m3x8_to_bf16x8(r[i]);
      else x[i] = r[i];
    }
    transpose8x8_b16(x, c);
    uint16_t* dst = stage + buf * C::BUF + lds_row0 * C::ROW + tg * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(dst + j * C::ROW) = c[j];
  };

  // one 16-token k-step of the chunk in LDS buffer buf
  auto mult_kstep = [&](int buf, int ks) {
    const uint16_t* kt = stage + buf * C::BUF;
    const uint16_t* vt = kt + D * C::ROW;
    const int col = ks * 16 + (lane >> 5) * 8;
    if constexpr (C::COLW) {
      // the tiles of sym_tiles
      uint4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const uint4*>(kt + (32 * ((wave + i) & 3) + (lane & 31)) * C::ROW + col);
      if (C::NV >= 4 || wave < C::NV) {
        const uint4 bv = *reinterpret_cast<const uint4*>(vt + (wave * 32 + (lane & 31)) * C::ROW + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[3 + i] = mfma32_bf16(a[i], bv, acc[3 + i]);
      }
      if constexpr (GRAM) {
        acc[0] = mfma32_bf16(a[0], a[0], acc[0]);
        acc[1] = mfma32_bf16(a[0], a[1], acc[1]);
        if (wave < 2) acc[2] = mfma32_bf16(a[0], a[2], acc[2]);
      }
    } else {
      const uint4 a = *reinterpret_cast<const uint4*>(kt + (rb * 32 + (lane & 31)) * C::ROW + col);
#pragma unroll
      for (int jj = 0; jj < C::CPW; ++jj) {
        const int c = jj * C::RPW + cofs;
        if (c < C::NC && (GRAM || c >= C::NK)) {
          const uint16_t* bs = c < C::NK ? kt + (c * 32 + (lane & 31)) * C::ROW
                                         : vt + ((c - C::NK) * 32 + (lane & 31)) * C::ROW;
          const uint4 b = *reinterpret_cast<const uint4*>(bs + col);
          acc[jj] = mfma32_bf16(a, b, acc[jj]);
        }
      }
    }
  };
  auto mult_chunk = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < C::TC / 16; ++ks) mult_kstep(buf, ks);
  };

  if constexpr (C::DEEP && FP8) {
    // FP8 codes are staged as loaded, token-major, in 128-token chunks (rows of TROW8
    // bytes: K then V, 256 bytes + 32 of padding so the transposing reads of a 32-lane half
    // hit 64 distinct banks), and G and Bm run on the 32x32x64 FP8 MFMA: e4m3 products are
    // exact and accumulate in fp32, as on the bfloat16 MFMA, at twice its rate and with half
    // the LDS bytes.  Waves 0-1 load K, waves 2-3 V; instruction i of a wave covers 8 whole
    // 128-byte rows (lane: token 64 (wave % 2) + 8 i + lane / 8, bytes 16 (lane % 8)).  Loads
    // past the frame's last token return zeros.
    const int64_t nch8 = (ntok + C::TC8 - 1) / C::TC8;
    uint8_t* const stage8 = reinterpret_cast<uint8_t*>(smem);
    const int tok_l = 64 * (wave & 1) + (lane >> 3);
    const auto rs = make_rsrc(wave < 2 ? kp : vp, uint32_t(ntok * 128));
    const uint32_t voff = uint32_t(tok_l * 128 + (lane & 7) * 16);
    uint8_t* const st_lane = stage8 + tok_l * C::TROW8 + (wave >> 1) * 128 + (lane & 7) * 16;
    uint4 ra[8], rn[8];
    auto chunk_base = [&](int64_t ch) -> uint32_t {
      // chunk indices past the end stay at nch8: their bytes are past the frame
      return voff + uint32_t((ch < nch8 ? ch : nch8) * C::TC8 * 128);
    };
    auto load8 = [&](int64_t ch, uint4 (&r)[8]) {
      const uint32_t base = chunk_base(ch);
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = buffer_load16<kCacheNt>(rs, base + uint32_t(i * 1024));
    };
    auto store8 = [&](int buf, const uint4 (&r)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint4*>(st_lane + buf * C::BUF8 + 8 * i * C::TROW8) = r[i];
    };
    // FP8 MFMA operand: feature f0 + l % 32 of tokens 32 (l / 32) + 0..31, byte 8q + j holding
    // token 32 (l / 32) + 8q + j, by four transposing 8-bit LDS reads (ds_read_b64_tr_b8).  In
    // each 16-lane group that read hands lane i element i % 8 of the 8-byte reads of lanes
    // i / 8, i / 8 + 2, ..., i / 8 + 14; so lane L of group g points at token
    // 32 (g / 2) + 8q + L / 2 and bytes 16 (g % 2) + 8 (L % 2) of the 32-feature block, and
    // receives one feature of 8 consecutive tokens.
    const int fr8 = (32 * (lane >> 5) + ((lane & 15) >> 1)) * C::TROW8 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
    auto frag8 = [&](const uint8_t* rows, int f0) -> i32x8 {
      typedef int v2i __attribute__((ext_vector_type(2)));
      typedef __attribute__((address_space(3))) v2i* lds_v2i;
      const uint8_t* p = rows + fr8 + f0;
      i32x8 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(p + 8 * q * C::TROW8));
        r[2 * q] = x[0];
        r[2 * q + 1] = x[1];
      }
      return r;
    };
    // the tiles of sym_tiles over one 64-token k-step
    auto kstep8 = [&](int buf, int ks) {
      const uint8_t* rows = stage8 + buf * C::BUF8 + ks * 64 * C::TROW8;
      i32x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = frag8(rows, 32 * ((wave + i) & 3));
      const i32x8 bv = frag8(rows, 128 + wave * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[3 + i] = mfma32_fp8(a[i], bv, acc[3 + i]);
      if constexpr (GRAM) {
        acc[0] = mfma32_fp8(a[0], a[0], acc[0]);
        acc[1] = mfma32_fp8(a[0], a[1], acc[1]);
        if (wave < 2) acc[2] = mfma32_fp8(a[0], a[2], acc[2]);
      }
    };
    // multiply the chunk in buffer buf while loading chunk ch (4 loads before each k-step)
    auto mult_load8 = [&](int buf, int64_t ch, uint4 (&r)[8]) {
      const uint32_t base = chunk_base(ch);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 * ks + j] = buffer_load16<kCacheNt>(rs, base + uint32_t((4 * ks + j) * 1024));
        kstep8(buf, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    load8(0, ra);
    load8(1, rn);
    store8(0, ra);
    __syncthreads();
    for (int64_t ch = 0; ch < nch8; ch += 2) {
      mult_load8(0, ch + 2, ra);
      store8(1, rn);
      __syncthreads();
      mult_load8(1, ch + 3, rn);
      store8(0, ra);
      __syncthreads();
    }
  } else if constexpr (C::DEEP) {
    // Two chunks in flight per thread, staged in LDS token-major, exactly as loaded.
    // Waves 0-1 load K, waves 2-3 V; instruction i of a wave covers 4 whole token rows
    // (lane: token 32 (wave % 2) + 4 i + lane / 16, 8 features from 8 (lane % 16)).  The
    // buffer descriptor spans the frame, so loads past its last token return zeros and a
    // ragged or missing chunk multiplies in nothing.
    const int tok_l = 32 * (wave & 1) + (lane >> 4);
    const auto rs = make_rsrc(wave < 2 ? kp : vp, uint32_t(ntok * 256));
    const uint32_t voff = uint32_t(tok_l * 256 + (lane & 15) * 16);
    uint16_t* const st_lane = stage + tok_l * C::TROW + (wave >> 1) * D + (lane & 15) * 8;
    uint4 ra[8], rn[8];
    auto chunk_base = [&](int64_t ch) -> uint32_t {
      // chunk indices past the end stay at nchunks: their bytes are past the frame
      return voff + uint32_t((ch < nchunks ? ch : nchunks) * C::TC * 256);
    };
    auto load_deep = [&](int64_t ch, uint4 (&r)[8]) {
      const uint32_t base = chunk_base(ch);
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = buffer_load16<kCacheNt>(rs, base + uint32_t(i * 1024));
    };
    auto store_rows = [&](int buf, const uint4 (&r)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(st_lane + buf * C::BUF + 4 * i * C::TROW) = r[i];
    };
    // MFMA operand of 8 consecutive tokens of one feature from the token-major rows, by two
    // transposing LDS reads (ds_read_b64_tr_b16).  In each 16-lane group the read hands
    // lane 4a + b element b of the 4-element reads of lanes a, a+4, a+8, a+12; so lane l
    // points at token 8 (l / 32) + (l % 16) / 4 (+4 for the second read) and features
    // 16 ((l / 16) % 2) + 4 (l % 4), and receives feature l % 32 of 4 consecutive tokens.
    const int fr_off = (8 * (lane >> 5) + ((lane & 15) >> 2)) * C::TROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto frag = [&](const uint16_t* rows, int f0) -> uint4 {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s* lds_v4s;
      const uint16_t* p = rows + fr_off + f0;
      const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p));
      const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * C::TROW));
      const uint2 xl = __builtin_bit_cast(uint2, x), yl = __builtin_bit_cast(uint2, y);
      return make_uint4(xl.x, xl.y, yl.x, yl.y);
    };
    // the tiles of sym_tiles over one 16-token k-step
    auto kstep_tm = [&](int buf, int ks) {
      const uint16_t* rows = stage + buf * C::BUF + ks * 16 * C::TROW;
      uint4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = frag(rows, 32 * ((wave + i) & 3));
      const uint4 bv = frag(rows, D + wave * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[3 + i] = mfma32_bf16(a[i], bv, acc[3 + i]);
      if constexpr (GRAM) {
        acc[0] = mfma32_bf16(a[0], a[0], acc[0]);
        acc[1] = mfma32_bf16(a[0], a[1], acc[1]);
        if (wave < 2) acc[2] = mfma32_bf16(a[0], a[2], acc[2]);
      }
    };
    // dQ = dO W^T (DQ): wave w forms dQ^T rows 32w..32w+31 (key features) for the chunk's 64
    // tokens on the 32x32x16 MFMA.  Its W operand (rows 32w.., k = value features) stays in
    // registers for the frame; the dO^T operand is 8 value features of one token, a plain
    // 16-byte read of the token's staged row.
    uint4 wq[DQ ? DV / 16 : 1];
    f32x16 dqa[2] = {f32x16{}, f32x16{}};
    const bool dq_on = DQ && fi > 0;
    const auto rq = make_rsrc(dq + (dq_on ? (bh * F + fi - 1) * n * D : 0), dq_on ? uint32_t(ntok * D * 2) : 0u);
    auto dq_part = [&](int buf, int ks) {  // value-feature blocks 2ks, 2ks+1 of both token halves
      const uint16_t* rows = stage + buf * C::BUF + D + 8 * (lane >> 5);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kb = 2 * ks + u;
          const uint4 b = *reinterpret_cast<const uint4*>(rows + (32 * tb + (lane & 31)) * C::TROW + 16 * kb);
          dqa[tb] = mfma32_bf16(wq[kb], b, dqa[tb]);
        }
    };
    // dQ of a finished chunk goes out through this wave's own part of a staging buffer that
    // every wave has finished reading (its rows 32 (w % 2)..+31, columns of K or V by w / 2:
    // only this wave's stores of the next chunk write there, later in its program order, and
    // one wave's LDS accesses complete in order).  Token t of the chunk takes row t % 32,
    // bytes 64 (t / 32)..+63, so the read-back gives four lanes 64 contiguous bytes of a
    // token's output row: the global stores are whole 64-byte pieces.
    auto dq_flush = [&](int buf, int64_t chunk) {
      uint16_t* fp = stage + buf * C::BUF + 32 * (wave & 1) * C::TROW + (wave >> 1) * D;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(fp + (lane & 31) * C::TROW + 32 * tb + 8 * g + 4 * (lane >> 5)) =
              make_uint2(pack_bf16x2(dqa[tb][4 * g], dqa[tb][4 * g + 1]),
                         pack_bf16x2(dqa[tb][4 * g + 2], dqa[tb][4 * g + 3]));
        dqa[tb] = f32x16{};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * j + (lane >> 2), pc = lane & 3;
        const uint4 x = *reinterpret_cast<const uint4*>(fp + (t & 31) * C::TROW + 32 * (t >> 5) + 8 * pc);
        buffer_store16<kCacheStreamOut>(rq, uint32_t(((chunk * C::TC + t) * D + 32 * wave + 8 * pc) * 2), x);
      }
    };
    // Multiply the chunk in LDS buffer buf while loading chunk ch into r.  The memory
    // queue is usually full, so a load can stall its wave at issue; two loads go out
    // before each k-step, and a stalled issue waits beside the previous k-step's MFMAs
    // rather than ahead of all of them.
    auto mult_load = [&](int buf, int64_t ch, uint4 (&r)[8]) {
      const uint32_t base = chunk_base(ch);
#pragma unroll
      for (int ks = 0; ks < C::TC / 16; ++ks) {
        r[2 * ks] = buffer_load16<kCacheNt>(rs, base + uint32_t(2 * ks * 1024));
        r[2 * ks + 1] = buffer_load16<kCacheNt>(rs, base + uint32_t((2 * ks + 1) * 1024));
        kstep_tm(buf, ks);
        if constexpr (DQ) dq_part(buf, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    load_deep(0, ra);
    load_deep(1, rn);
    if (dq_on) {
      // W^T of the frame into the staging area (rows = value features j, the key features i
      // along a row, bfloat16, the staging row stride), then every wave's W fragments by the
      // transposing reads the main loop uses.  A float4 of the blocked states is rows
      // i0..i0+3 of one column j.
      const float4* xf4 = reinterpret_cast<const float4*>(xf32 + (bh * F + fi - 1) * int64_t(D) * DV);
      const float4* xb4 = reinterpret_cast<const float4*>(xb32 + (bh * F + fi - 1) * int64_t(D) * DV);
#pragma unroll 4
      for (int m = 0; m < D * DV / 4 / kThreads; ++m) {
        const int qi = m * kThreads + tid;
        const float4 a = xf4[qi], b = xb4[qi];
        const int blk = qi >> 6;
        const int i0 = (blk % (D / 16)) * 16 + ((qi >> 4) & 3) * 4, j = (blk / (D / 16)) * 16 + (qi & 15);
        *reinterpret_cast<uint2*>(stage + j * C::TROW + i0) =
            make_uint2(pack_bf16x2(0.5f * (a.x + b.x), 0.5f * (a.y + b.y)),
                       pack_bf16x2(0.5f * (a.z + b.z), 0.5f * (a.w + b.w)));
      }
      __syncthreads();
      if constexpr (DQ) {
#pragma unroll
        for (int kb = 0; kb < DV / 16; ++kb) wq[kb] = frag(stage + 16 * kb * C::TROW, 32 * wave);
      }
      __syncthreads();
    }
    store_rows(0, ra);
    __syncthreads();
    for (int64_t ch = 0; ch < nchunks; ch += 2) {
      mult_load(0, ch + 2, ra);
      store_rows(1, rn);
      __syncthreads();
      if constexpr (DQ) {
        if (dq_on) dq_flush(0, ch);
      }
      mult_load(1, ch + 3, rn);
      store_rows(0, ra);
      __syncthreads();
      if constexpr (DQ) {
        if (dq_on) dq_flush(1, ch + 1);
      }
    }
  } else {
    Raw r[8];
    if (nchunks > 0) {
      load_chunk(0, r);
      store_chunk(0, r);
    }
    __syncthreads();
    for (int64_t ch = 0; ch < nchunks; ++ch) {
      const int buf = int(ch & 1);
      if (ch + 1 < nchunks) load_chunk(ch + 1, r);
      mult_chunk(buf);
      if (ch + 1 < nchunks) store_chunk(buf ^ 1, r);
      __syncthreads();
    }
  }

  float* bmo = bm + (bh * F1 + fi) * int64_t(D) * DV;
  if constexpr (D == 128) {
    // ---- epilogue (d = 128): lam I + G inverted in the accumulators by the blocked sweep;
    // A^{-1} = -(swept matrix), then the Bm tiles (held in their accumulators through the
    // sweep) written out together: a workgroup's outputs leave in one burst, and each burst of
    // writes into the other workgroups' read stream costs read bandwidth.
    const int l32 = lane & 31;
    // accumulator registers 4m..4m+3 of a lane are rows 4j..4j+3 of one column, which the
    // blocked layout keeps as 4 consecutive floats: one 16-byte store each, and a store
    // instruction writes two whole 512-byte pieces
    auto store_bm = [&] {
      if (wave < C::NV) {
        const auto rs = make_rsrc(bmo, uint32_t(D * DV * 4));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x16& a = acc[3 + i];
            const int off = blk_index(32 * ((wave + i) & 3) + mfma32_row(4 * m, lane), wave * 32 + l32, D);
            buffer_store16<kCacheSc1>(rs, uint32_t(off * 4),
                                      make_uint4(__float_as_uint(a[4 * m]), __float_as_uint(a[4 * m + 1]),
                                                 __float_as_uint(a[4 * m + 2]), __float_as_uint(a[4 * m + 3])));
          }
      }
    };
    if constexpr (!GRAM) {
      store_bm();
      return;
    }
    // the frame's A^{-1} as two bf16 planes, hi then lo, each sym_blocks(D) 16 x 16 blocks
    uint16_t* hi_plane = reinterpret_cast<uint16_t*>(ainv + (bh * F1 + fi) * int64_t(D) * D);
    // G tiles (and the mirror of each off-diagonal one) -> LDS -> G row block in the
    // accumulator layout the sweep works on
    float* gsm = reinterpret_cast<float*>(smem);
    {
      const int r0 = 32 * wave, r1 = 32 * ((wave + 1) & 3), r2 = 32 * ((wave + 2) & 3);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = mfma32_row(e, lane);
        gsm[(r0 + r) * C::GS + r0 + l32] = acc[0][e];
        gsm[(r0 + r) * C::GS + r1 + l32] = acc[1][e];
        gsm[(r1 + l32) * C::GS + r0 + r] = acc[1][e];
        if (wave < 2) {
          gsm[(r0 + r) * C::GS + r2 + l32] = acc[2][e];
          gsm[(r2 + l32) * C::GS + r0 + r] = acc[2][e];
        }
      }
    }
    __syncthreads();
    f32x16 t[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wave * 32 + mfma32_row(e, lane), colg = c * 32 + l32;
        t[c][e] = gsm[row * C::GS + colg] + (row == colg ? lam : 0.0f);
      }
    __syncthreads();
    static_assert(6 * 16 * kPbs * 4 <= C::MAIN_BYTES, "sweep buffers exceed the staging area");
    sweep_neg_inverse_128(t, reinterpret_cast<float*>(smem), wave, lane);
    // A^{-1} is symmetric: lane l's column j of tile c is row j of A^{-1}, and its
    // registers 4q..4q+3 are columns 32 wave + 8q + 4h .. +3 of that row (h = lane / 32).
    // Only the 16 x 16 blocks on and above the diagonal are stored (sym_index).  Lanes l and
    // l + 32 trade a quarter-row so that each holds 8 consecutive columns (h = 0: columns
    // 0..7 of a 16-column block, h = 1: 8..15): a store instruction then writes each plane's
    // rows whole, two 512-byte blocks.
    {
      const auto rs = make_rsrc(hi_plane, uint32_t(2 * sym_blocks(D) * 256 * 2));
      const int h = lane >> 5;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
          uint32_t hw[2][2], lw[2][2];  // [j][word]: columns 16 qp + 8 j + 4 h .. +3
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int q = 2 * qp + j;
            split_bf16x2(-t[c][4 * q + 0], -t[c][4 * q + 1], hw[j][0], lw[j][0]);
            split_bf16x2(-t[c][4 * q + 2], -t[c][4 * q + 3], hw[j][1], lw[j][1]);
          }
          // h = 0 gives its columns 8..11 and takes the partner's 4..7; h = 1 gives 4..7 and
          // takes 8..11
          uint32_t rh[2], rl[2];
#pragma unroll
          for (int w2 = 0; w2 < 2; ++w2) {
            rh[w2] = uint32_t(__shfl_xor(int(h ? hw[0][w2] : hw[1][w2]), 32));
            rl[w2] = uint32_t(__shfl_xor(int(h ? lw[0][w2] : lw[1][w2]), 32));
          }
          const int row = 32 * c + l32, col = 32 * wave + 16 * qp + 8 * h;
          if ((row >> 4) > (col >> 4)) continue;
          const uint4 vh = h ? make_uint4(rh[0], rh[1], hw[1][0], hw[1][1]) : make_uint4(hw[0][0], hw[0][1], rh[0], rh[1]);
          const uint4 vl = h ? make_uint4(rl[0], rl[1], lw[1][0], lw[1][1]) : make_uint4(lw[0][0], lw[0][1], rl[0], rl[1]);
          const int off = sym_index(row, col, D);
          buffer_store16<kCacheSc1>(rs, uint32_t(off * 2), vh);
          buffer_store16<kCacheSc1>(rs, uint32_t((off + sym_blocks(D) * 256) * 2), vl);
        }
    }
    store_bm();
    return;
  }
  // ---- epilogue: Bm tiles to the workspace, G tiles to LDS, then invert lam I + G
  float* gsm = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int jj = 0; jj < C::CPW; ++jj) {
    const int c = jj * C::RPW + cofs;
    if (c >= C::NC) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = rb * 32 + mfma32_row(e, lane);
      if (c < C::NK) {
        if constexpr (GRAM) gsm[row * C::GS + c * 32 + (lane & 31)] = acc[jj][e];
      } else {
        bmo[blk_index(row, (c - C::NK) * 32 + (lane & 31), D)] = acc[jj][e];
      }
    }
  }
  if constexpr (!GRAM) return;
  __syncthreads();
  uint16_t* hi_plane = reinterpret_cast<uint16_t*>(ainv + (bh * F1 + fi) * int64_t(D) * D);
  uint16_t* lo_plane = hi_plane + sym_blocks(D) * 256;
  float* rowv = reinterpret_cast<float*>(smem + C::MAIN_BYTES);
  float* colv = rowv + 2 * D;
  float a[D / 16][D / 16];
  spd_inverse_gj<D>(gsm, C::GS, lam, rowv, colv, a);
  // A^{-1} as two bfloat16 planes, hi then lo (hi + lo = A^{-1} to ~2^-17 relative), for
  // the split-bf16 MFMA products of the scan.  Only the 16 x 16 blocks on and above the
  // diagonal are stored (sym_index, row-major blocks): a thread's TS consecutive columns of
  // a row stay contiguous, so each row goes out as one TS*2-byte store per plane.
  constexpr int TS = D / 16;
  const int tr = tid >> 4, tcol = tid & 15;
#pragma unroll
  for (int i = 0; i < TS; ++i) {
    if (((tr * TS + i) >> 4) > ((tcol * TS) >> 4)) continue;
    uint32_t hw[TS / 2], lw[TS / 2];
#pragma unroll
    for (int j = 0; j < TS; j += 2) {
      split_bf16x2(a[i][j], a[i][j + 1], hw[j / 2], lw[j / 2]);
    }
    const int off = sym_index(tr * TS + i, tcol * TS, D);
    if constexpr (TS == 8) {
      *reinterpret_cast<uint4*>(hi_plane + off) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(lo_plane + off) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    } else if constexpr (TS == 4) {
      *reinterpret_cast<uint2*>(hi_plane + off) = make_uint2(hw[0], hw[1]);
      *reinterpret_cast<uint2*>(lo_plane + off) = make_uint2(lw[0], lw[1]);
    } else {
      *reinterpret_cast<uint32_t*>(hi_plane + off) = hw[0];
      *reinterpret_cast<uint32_t*>(lo_plane + off) = lw[0];
    }
  }
}

// ---------------------------------------------------------------- float32 inputs
// fp32 operands are one value per lane for the 32x32x2 MFMA, so the chunk is kept
// row-major (as loaded) and no transpose is needed.
template <int D, int DV>
struct StatsF32 {
  static constexpr int TC = 32;
  static constexpr int NK = D / 32, NV = DV / 32, NC = NK + NV;
  static constexpr int RPW = 4 / NK;
  static constexpr int CPW = (NC + RPW - 1) / RPW;
  static constexpr int ROWF = D + DV + 4;        // floats per token row in LDS (K then V)
  static constexpr int STAGE_BYTES = TC * ROWF * 4;
  static constexpr int GS = D + 4;
  static constexpr int G_BYTES = D * GS * 4;
  static constexpr int MAIN_BYTES = cmax(STAGE_BYTES, G_BYTES);
  static constexpr int LDS_BYTES = MAIN_BYTES + 4 * D * 4;
};

template <int D, int DV>
__global__ void __launch_bounds__(kThreads)
stats_f32_kernel(const float* __restrict__ k, const float* __restrict__ v,
                 const float* __restrict__ tk, const float* __restrict__ tv,
                 float* __restrict__ ainv, float* __restrict__ bm,
                 int64_t F, int64_t n, int64_t T, float lam) {
  using C = StatsF32<D, DV>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* st = reinterpret_cast<float*>(smem);

  const int64_t F1 = F + 1;
  const int64_t fi = blockIdx.x % F1;
  const int64_t bh = blockIdx.x / F1;
  const float* kp;
  const float* vp;
  int64_t ntok;
  if (fi == 0) {
    kp = tk + bh * T * D;
    vp = tv + bh * T * DV;
    ntok = T;
  } else {
    kp = k + ((bh * F + (fi - 1)) * n) * D;
    vp = v + ((bh * F + (fi - 1)) * n) * DV;
    ntok = n;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = wave % C::NK, cofs = wave / C::NK;
  f32x16 acc[C::CPW];
#pragma unroll
  for (int j = 0; j < C::CPW; ++j) acc[j] = f32x16{};

  constexpr int Q = (D + DV) / 4;  // float4 pieces per token
  for (int64_t t0 = 0; t0 < ntok; t0 += C::TC) {
    for (int idx = tid; idx < C::TC * Q; idx += kThreads) {
      const int t = idx / Q, p = idx % Q;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t0 + t < ntok) {
        x = p < D / 4 ? *reinterpret_cast<const float4*>(kp + (t0 + t) * D + 4 * p)
                      : *reinterpret_cast<const float4*>(vp + (t0 + t) * DV + 4 * (p - D / 4));
      }
      *reinterpret_cast<float4*>(st + t * C::ROWF + 4 * p) = x;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < C::TC / 2; ++ks) {
      const int t = ks * 2 + (lane >> 5);
      const float a = st[t * C::ROWF + rb * 32 + (lane & 31)];
#pragma unroll
      for (int jj = 0; jj < C::CPW; ++jj) {
        const int c = jj * C::RPW + cofs;
        if (c < C::NC) {
          const float b = st[t * C::ROWF + c * 32 + (lane & 31)];
          acc[jj] = mfma32_f32(a, b, acc[jj]);
        }
      }
    }
    __syncthreads();
  }

  float* gsm = st;
  float* bmo = bm + (bh * F1 + fi) * int64_t(D) * DV;
#pragma unroll
  for (int jj = 0; jj < C::CPW; ++jj) {
    const int c = jj * C::RPW + cofs;
    if (c >= C::NC) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = rb * 32 + mfma32_row(e, lane);
      if (c < C::NK) {
        gsm[row * C::GS + c * 32 + (lane & 31)] = acc[jj][e];
      } else {
        bmo[blk_index(row, (c - C::NK) * 32 + (lane & 31), D)] = acc[jj][e];
      }
    }
  }
  __syncthreads();
  float* rowv = reinterpret_cast<float*>(smem + C::MAIN_BYTES);
  float* colv = rowv + 2 * D;
  float a[D / 16][D / 16];
  spd_inverse_gj<D>(gsm, C::GS, lam, rowv, colv, a);
  constexpr int TS = D / 16;
  float* ao = ainv + (bh * F1 + fi) * int64_t(D) * D;
  const int tr = tid >> 4, tcol = tid & 15;
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) ao[(tr * TS + i) * D + tcol * TS + j] = a[i][j];
}

template <int D, int DV>
hipError_t launch_stats_t(const Problem& p, const void* k, const void* v, const void* tk,
                          const void* tv, hipStream_t s, bool prepare) {
  const int64_t blocks = p.B * p.H * (p.F + 1);
  if (p.bf16) {
    constexpr int lds = StatsBf16<D, DV>::LDS_BYTES;
    auto launch = [&](auto kern, auto in) -> hipError_t {
      using In = decltype(in);
      if (prepare)
        return lds > 65536 ? hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds)
                           : hipSuccess;
      launch_kernel(p, kern, dim3(unsigned(blocks)), dim3(kThreads), lds, s,
                    static_cast<const In*>(k), static_cast<const In*>(v),
                    static_cast<const In*>(tk), static_cast<const In*>(tv), p.ainv, p.bm, p.F,
                    p.n, p.T, p.lam, static_cast<const float*>(nullptr), static_cast<const float*>(nullptr),
                    static_cast<uint16_t*>(nullptr));
      return hipGetLastError();
    };
    if (prepare && !p.fp8) {
      const hipError_t e = launch(stats_bf16_kernel<D, DV, uint16_t, kStatsBm>, uint16_t{});
      if (e != hipSuccess) return e;
      if constexpr (D == 128 && DV == 128) {
        const hipError_t e2 = launch(stats_bf16_kernel<D, DV, uint16_t, kStatsBmDq>, uint16_t{});
        if (e2 != hipSuccess) return e2;
      }
    }
    if (p.bm_only) {
      if (p.fp8) return hipErrorInvalidValue;
      return launch(stats_bf16_kernel<D, DV, uint16_t, kStatsBm>, uint16_t{});
    }
    return p.fp8 ? launch(stats_bf16_kernel<D, DV, uint8_t>, uint8_t{})
                 : launch(stats_bf16_kernel<D, DV, uint16_t>, uint16_t{});
  } else {
    if (p.bm_only) return hipErrorInvalidValue;
    constexpr int lds = StatsF32<D, DV>::LDS_BYTES;
    auto kern = stats_f32_kernel<D, DV>;
    if (prepare)
      return lds > 65536 ? hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds)
                         : hipSuccess;
    launch_kernel(p, kern, dim3(unsigned(blocks)), dim3(kThreads), lds, s,
                  static_cast<const float*>(k), static_cast<const float*>(v),
                  static_cast<const float*>(tk), static_cast<const float*>(tv), p.ainv, p.bm,
                  p.F, p.n, p.T, p.lam);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stats(const Problem& p, const void* k, const void* v, const void* tk,
                        const void* tv, hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_stats_t<DD, VV>(p, k, v, tk, tv, s, false);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_stats_dq(const Problem& p, const void* q, const void* d_out, const float* xf32,
                           const float* xb32, void* d_q, hipStream_t s) {
  if (!(p.d == 128 && p.dv == 128 && p.bf16 && !p.fp8 && p.T == 0)) return hipErrorInvalidValue;
  const int64_t blocks = p.B * p.H * (p.F + 1);
  constexpr int lds = StatsBf16<128, 128>::LDS_BYTES;
  hipLaunchKernelGGL((stats_bf16_kernel<128, 128, uint16_t, kStatsBmDq>), dim3(unsigned(blocks)), dim3(kThreads),
                     lds, s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(d_out), nullptr,
                     nullptr, nullptr, p.bm, p.F, p.n, int64_t(0), p.lam, xf32, xb32, static_cast<uint16_t*>(d_q));
  return hipGetLastError();
}

hipError_t prepare_stats(const Problem& p) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) \
    return launch_stats_t<DD, VV>(p, nullptr, nullptr, nullptr, nullptr, nullptr, true);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda
