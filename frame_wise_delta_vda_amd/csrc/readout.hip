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
#include <type_traits>

#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

// bfloat16 path.  One workgroup per frame (or per equal part of a frame when there
// are too few frames to fill the chip), so W is formed once per frame and the
// workgroups that run together stream neighbouring frames.  Wave w of a workgroup
// takes tokens 16w..16w+15 of every 64-token tile and, after one barrier at the start,
// works alone:
//  - at the start the four waves form the W^T operand fragments from the two bf16
//    states, which the scan stores in exactly that operand order (state_index), a
//    quarter each (one 16-byte load per state and fragment, mean in fp32, one
//    rounding) into LDS; after the barrier every wave takes all of them into registers.
//    Each state byte crosses into the compute unit once per workgroup, not once per
//    wave (a quarter of the traffic, 1-2% of the readout at d = dv = 128);
//  - the wave's Q rows are loaded straight into MFMA operands (lane: token l%16, eight
//    consecutive features), two tiles ahead;
//  - O^T = W^T Q^T goes through a wave-private LDS patch so the stores are whole rows
//    (1 KB contiguous per wave instruction).
// Q is loaded with the default cache policy and O stored with a streaming one (SC1 | NT),
// through buffer descriptors bounded by the frame's last row, so ragged frame ends need no
// branch.  Loading Q non-temporally instead was up to 30% slower with short frames (long
// clip 0.914 against 0.957 ms, small workload 0.010 against 0.014 ms) and no faster at 768p.  FP8 e4m3 Q
// (In = uint8_t) is converted to bfloat16 just before its MFMA; the output is bfloat16
// either way.  At d >= 64 a lane loads 16 consecutive FP8 features at once and feeds
// them to two k-steps (features 16 (g + 4 m) .. +15 to k-steps 2m and 2m + 1, g = lane /
// 16), which keeps the loads as wide as the bfloat16 ones; the scan stores the states
// of such plans with their rows in the same order (paired_row), so the W fragments are
// loaded exactly as for bfloat16.  8-byte loads of one k-step each were 25% slower.
template <int D, int DV>
struct ReadBf16 {
  static constexpr int TT = 64;                 // tokens per tile (16 per wave)
  static constexpr int KS = D / 32;             // k-steps of the 16x16x32 MFMA
  static constexpr int NBF = DV / 16;           // 16-feature output blocks
  static constexpr int OWROW = DV + 8;          // bf16 per LDS row of a wave's O patch
  static constexpr int OCH = DV / 8;            // 16-byte chunks per output row
  static constexpr int ORPI = 64 / OCH;         // output rows per wave store instruction
  static constexpr int OST = 16 / ORPI;         // store instructions per wave per tile
  static constexpr int OW_BYTES = 16 * OWROW * 2;  // per wave
  static constexpr int NFR = NBF * KS;           // W^T fragments of a frame
  static constexpr int WF_BYTES = NFR * 64 * 16;  // formed once per workgroup, shared through LDS
  static constexpr int LDS_BYTES = 4 * OW_BYTES + WF_BYTES;
  static_assert(OST >= 1, "value width too large for one wave store pass");
};

template <int D, int DV, typename In>
__global__ void __launch_bounds__(kThreads, 2)
readout_bf16_kernel(const In* __restrict__ q, const uint16_t* __restrict__ xf,
                    const uint16_t* __restrict__ xb, uint16_t* __restrict__ out, int64_t n,
                    int64_t tiles_per_frame, int64_t splits, int64_t tiles_per_split,
                    int64_t head_blocks, int64_t tail_splits, int64_t tail_tiles_per_split) {
  using C = ReadBf16<D, DV>;
  constexpr int EB = int(sizeof(In));  // bytes per Q element
  constexpr bool PAIR = EB == 1 && C::KS >= 2;  // one FP8 load feeds two k-steps
  constexpr int NQL = PAIR ? C::KS / 2 : C::KS;  // Q loads per lane and tile
  // a Q load: 8 bfloat16 features (16 bytes), 16 FP8 features (16 bytes) or, at d = 32,
  // 8 FP8 features (8 bytes)
  using QRaw = typename std::conditional<EB == 1 && !PAIR, uint2, uint4>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* ow = reinterpret_cast<uint16_t*>(smem + wave * C::OW_BYTES);
  const int c16 = lane & 15, g4 = lane >> 4;
  // blocks past head_blocks take the frames of the last, partial round of resident
  // workgroups in smaller parts, so the launch does not end on a few long workgroups
  int64_t frame, t_first, tps;
  if (blockIdx.x < head_blocks) {
    frame = blockIdx.x / splits;
    t_first = (blockIdx.x % splits) * tiles_per_split;
    tps = tiles_per_split;
  } else {
    const int64_t i = blockIdx.x - head_blocks;
    frame = head_blocks / splits + i / tail_splits;
    t_first = (i % tail_splits) * tail_tiles_per_split;
    tps = tail_tiles_per_split;
  }
  const int64_t t_last = (t_first + tps < tiles_per_frame) ? t_first + tps : tiles_per_frame;
  if (t_first >= t_last) return;

  // rows of this wave's 16 tokens that lie inside the frame (0 past its end)
  auto wave_rows = [&](int64_t tok0) -> uint32_t {
    const int64_t r = n - tok0;
    return uint32_t(r < 0 ? 0 : (r < 16 ? r : 16));
  };
  auto load_q = [&](int64_t tile, QRaw (&dst)[NQL]) {
    const int64_t tok0 = tile * C::TT + 16 * wave;
    const auto rs = make_rsrc(q + (frame * n + tok0) * D, wave_rows(tok0) * D * EB);
#pragma unroll
    for (int i = 0; i < NQL; ++i) {
      if constexpr (PAIR) dst[i] = buffer_load16(rs, uint32_t(c16 * D + 16 * (g4 + 4 * i)));
      else if constexpr (EB == 1) dst[i] = buffer_load8(rs, uint32_t(c16 * D + 32 * i + 8 * g4));
      else dst[i] = buffer_load16(rs, uint32_t((c16 * D + 32 * i + 8 * g4) * 2));
    }
  };

  QRaw pfa[NQL], pfb[NQL];
  load_q(t_first, pfa);
  load_q(t_first + 1 < t_last ? t_first + 1 : t_first, pfb);

  // W = (X_fwd + X_bwd) / 2 of the frame, rounded once to bf16; fragment (nb, ks) of
  // both states is the 1 KB at ((nb * KS + ks) * 64 + lane) * 8, and in LDS.  The early
  // return above is the same for the whole workgroup, so every wave reaches the barrier.
  uint4 wfr[C::NBF][C::KS];  // W^T fragments: rows = output features, k = input features
  {
    // each wave forms a quarter of the fragments into LDS (fragment order), then every wave
    // takes all of them
    uint4* wsm = reinterpret_cast<uint4*>(smem + 4 * C::OW_BYTES);
    const uint4* sf = reinterpret_cast<const uint4*>(xf + frame * int64_t(D) * DV) + lane;
    const uint4* sb = reinterpret_cast<const uint4*>(xb + frame * int64_t(D) * DV) + lane;
    for (int fr = wave; fr < C::NFR; fr += 4) wsm[fr * 64 + lane] = mean_bf16x8(sf[fr * 64], sb[fr * 64]);
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < C::NBF; ++nb)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) wfr[nb][ks] = wsm[(nb * C::KS + ks) * 64 + lane];
  }

  auto step = [&](int64_t tile, QRaw (&pf)[NQL]) {
    const int64_t tok0 = tile * C::TT + 16 * wave;
    uint4 qf[C::KS];
#pragma unroll
    for (int i = 0; i < NQL; ++i) {
      if constexpr (PAIR) {
        qf[2 * i] = e4m3x8_to_bf16x8(make_uint2(pf[i].x, pf[i].y));
        qf[2 * i + 1] = e4m3x8_to_bf16x8(make_uint2(pf[i].z, pf[i].w));
      } else if constexpr (EB == 1) {
        qf[i] = e4m3x8_to_bf16x8(pf[i]);
      } else {
        qf[i] = pf[i];
      }
    }
    load_q(tile + 2 < t_last ? tile + 2 : t_last - 1, pf);  // unconditional: no phi, no copy
    // O^T block nb: the lane holds token c16, output features 16 nb + 4 g4 + 0..3
#pragma unroll
    for (int nb = 0; nb < C::NBF; ++nb) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) acc = mfma16_bf16(wfr[nb][ks], qf[ks], acc);
      *reinterpret_cast<uint2*>(ow + c16 * C::OWROW + 16 * nb + 4 * g4) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
    // the patch is private to this wave, whose LDS accesses complete in order
    const auto rs = make_rsrc(out + (frame * n + tok0) * DV, wave_rows(tok0) * DV * 2);
    const int orow = lane / C::OCH, och = lane % C::OCH;
#pragma unroll
    for (int j = 0; j < C::OST; ++j) {
      const int r = orow + j * C::ORPI;
      buffer_store16<kCacheStreamOut>(rs, uint32_t(r * DV * 2 + och * 16),
                               *reinterpret_cast<const uint4*>(ow + r * C::OWROW + och * 8));
    }
  };

  for (int64_t tile = t_first; tile < t_last; tile += 2) {
    step(tile, pfa);
    if (tile + 1 < t_last) step(tile + 1, pfb);
  }
}

// Gated readout: the readout followed by the linear branch's gated fusion epilogue
// (aiezz page, section 03, and laicaila page, "technical principles": bullet "gated
// fusion" -- each branch gets a content-dependent sigmoid gate and its own output
// projection before the branches merge).  Per head h, with W_g, W_o (dv x dv, [output
// feature][input feature]) and b_g:
//   Y_f = sigmoid(O_f W_g^T + b_g) * (O_f W_o^T),   O_f = Q_f W_f
// Both products fold into the frame's state: O_f W_o^T = Q_f (W_f W_o^T), so per token the
// epilogue is two readout products instead of one and O never leaves the registers.
//  - Per frame the workgroup builds W_f^T = (X_fwd + X_bwd)^T / 2 in LDS (bf16, value
//    feature rows), then the four waves fold W'_o = W_f W_o^T and W'_g = W_f W_g^T on the
//    16x16x32 MFMA, each wave a quarter of the output blocks, with W_f as the A operand
//    (transposing LDS reads) and the weight rows as B (16-byte loads).  The fold's A rows are
//    taken in the order that leaves each lane's accumulators holding exactly the readout's
//    operand fragments of W'^T (4 input features from each of two row tiles), and the
//    fragments go to LDS in fragment order (1 KB per fragment, lane-contiguous).
//  - Every wave then copies all of W'_o into registers (the plain readout's W budget), and
//    W'_g stays in LDS, read once per tile, conflict-free.
//  - Waves split the tokens only, as in the plain readout: wave w takes tokens 16w..16w+15 of
//    every 64-token tile and all output features, so each Q row is loaded once, two tiles
//    ahead.
//  - Y goes through a wave-private LDS patch (in the space W_f^T held during the fold), so
//    a store instruction writes whole rows.
template <int D, int DV>
struct ReadGated {
  static constexpr int TT = 64;                 // tokens per tile (16 per wave)
  static constexpr int KS = D / 32;             // readout k-steps (input features)
  static constexpr int NBF = DV / 16;           // 16-feature output blocks
  static constexpr int KC = DV / 32;            // fold k-steps (value features)
  static constexpr int NFR = NBF * KS;          // fragments of one folded matrix (and of a state)
  static constexpr int WTROW = D + 8;           // bf16 per LDS row of W_f^T
  static constexpr int WT_BYTES = DV * WTROW * 2;
  static constexpr int FR_BYTES = NFR * 64 * 16;  // one folded matrix in fragment order
  static constexpr int OWROW = DV + 8;          // bf16 per LDS row of a wave's Y patch
  static constexpr int OCH = DV / 8;            // 16-byte chunks per output row
  static constexpr int ORPI = 64 / OCH;         // output rows per wave store instruction
  static constexpr int OST = 16 / ORPI;         // store instructions per wave per tile
  static constexpr int OW_BYTES = 16 * OWROW * 2;
  static constexpr int A_BYTES = cmax(WT_BYTES, 4 * OW_BYTES);  // W_f^T, later the Y patches
  static constexpr int LDS_BYTES = A_BYTES + FR_BYTES + DV * 4;  // + folded W_g + the bias
  static_assert(KC >= 1 && OST >= 1, "value width must be 32..128");
};

template <int D, int DV, typename In>
__global__ void __launch_bounds__(kThreads, 2)
readout_gated_kernel(const In* __restrict__ q, const uint16_t* __restrict__ xf,
                     const uint16_t* __restrict__ xb, const uint16_t* __restrict__ w_gate,
                     const float* __restrict__ b_gate, const uint16_t* __restrict__ w_out,
                     uint16_t* __restrict__ out, int64_t n, int64_t F, int64_t H,
                     int64_t tiles_per_frame, int64_t splits, int64_t tiles_per_split,
                     int64_t head_blocks, int64_t tail_splits, int64_t tail_tiles_per_split) {
  using C = ReadGated<D, DV>;
  constexpr int EB = int(sizeof(In));
  constexpr bool PAIR = EB == 1 && C::KS >= 2;
  constexpr int NQL = PAIR ? C::KS / 2 : C::KS;
  using QRaw = typename std::conditional<EB == 1 && !PAIR, uint2, uint4>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* wt = reinterpret_cast<uint16_t*>(smem);                      // W_f^T [DV][WTROW]
  uint4* frg = reinterpret_cast<uint4*>(smem + C::A_BYTES);               // [NFR][64] fragments
  float* bias_s = reinterpret_cast<float*>(smem + C::A_BYTES + C::FR_BYTES);  // [DV]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  int64_t frame, t_first, tps;
  if (blockIdx.x < head_blocks) {
    frame = blockIdx.x / splits;
    t_first = (blockIdx.x % splits) * tiles_per_split;
    tps = tiles_per_split;
  } else {
    const int64_t i = blockIdx.x - head_blocks;
    frame = head_blocks / splits + i / tail_splits;
    t_first = (i % tail_splits) * tail_tiles_per_split;
    tps = tail_tiles_per_split;
  }
  const int64_t t_last = (t_first + tps < tiles_per_frame) ? t_first + tps : tiles_per_frame;
  if (t_first >= t_last) return;
  const int64_t head = (frame / F) % H;

  // input feature held at slot m of k-step ks by lane group g, for the Q operand and the
  // states alike (FP8 plans at d >= 64 pair k-steps; see the plain readout)
  auto qmap = [&](int ks, int g, int m) -> int {
    return PAIR ? 16 * (g + 4 * (ks >> 1)) + 8 * (ks & 1) + m : 32 * ks + 8 * g + m;
  };

  // ---- W_f^T = (X_fwd + X_bwd)^T / 2 into LDS: fragment (nb, ks) of the stored states
  // holds rows 16 nb + lane % 16 of W^T and input features qmap(ks, lane / 16, 0..7); and the
  // head's gate bias
  {
    const uint4* sf = reinterpret_cast<const uint4*>(xf + frame * int64_t(D) * DV) + lane;
    const uint4* sb = reinterpret_cast<const uint4*>(xb + frame * int64_t(D) * DV) + lane;
    for (int fr = wave; fr < C::NFR; fr += 4) {
      const int nb = fr / C::KS, ks = fr % C::KS;
      const uint4 m = mean_bf16x8(sf[fr * 64], sb[fr * 64]);
      *reinterpret_cast<uint4*>(wt + (16 * nb + c16) * C::WTROW + qmap(ks, g4, 0)) = m;
    }
    for (int i = tid; i < DV; i += kThreads) bias_s[i] = b_gate[head * DV + i];
  }
  __syncthreads();

  // ---- fold of one weight matrix into the fragment region: fragment (jb, ks) of (W_f Wl^T)^T.
  // Row slot 16t + s of the fold's A operand is input feature qmap(t / 2, s / 4, 4 (t % 2) + s % 4),
  // so lane (j, g) of accumulator tile t holds the features of slots 4 (t % 2) .. +3 of k-step
  // t / 2 for lane group g: half a fragment.  The A operand comes from W_f^T by two transposing
  // reads (ds_read_b64_tr_b16): lane L of a 16-lane group points at value feature (row)
  // 32 kc + 8 g + L / 4 (+4) and input features qmap(t / 2, L % 4, 4 (t % 2)) .. +3, and receives
  // 8 consecutive value features of input feature i(lane % 16).
  auto fold_a = [&](int t, int kc) -> uint4 {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const uint16_t* p = wt + (32 * kc + 8 * g4 + (c16 >> 2)) * C::WTROW + qmap(t >> 1, c16 & 3, 4 * (t & 1));
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p));
    const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * C::WTROW));
    const uint2 xl = __builtin_bit_cast(uint2, x), yl = __builtin_bit_cast(uint2, y);
    return make_uint4(xl.x, xl.y, yl.x, yl.y);
  };
  auto fold = [&](const uint16_t* wl) {
    for (int jb = wave; jb < C::NBF; jb += 4) {  // this wave's output blocks
      const int j = 16 * jb + c16;               // output feature of this lane
      uint4 bw[C::KC];
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) bw[kc] = *reinterpret_cast<const uint4*>(wl + j * DV + 32 * kc + 8 * g4);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        uint32_t wd[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x4 acc = f32x4{};
#pragma unroll
          for (int kc = 0; kc < C::KC; ++kc) acc = mfma16_bf16(fold_a(2 * ks + h2, kc), bw[kc], acc);
          wd[2 * h2] = pack_bf16x2(acc[0], acc[1]);
          wd[2 * h2 + 1] = pack_bf16x2(acc[2], acc[3]);
        }
        frg[(jb * C::KS + ks) * 64 + lane] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
  };
  // W'_o first: every wave keeps all of it in registers
  fold(w_out + head * DV * DV);
  __syncthreads();
  uint4 wo[C::NBF][C::KS];
#pragma unroll
  for (int jb = 0; jb < C::NBF; ++jb)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) wo[jb][ks] = frg[(jb * C::KS + ks) * 64 + lane];
  __syncthreads();  // every wave has its copy before W'_g takes the region
  fold(w_gate + head * DV * DV);
  __syncthreads();  // W'_g complete; W_f^T no longer needed, its space holds the Y patches
  uint16_t* ow = reinterpret_cast<uint16_t*>(smem + wave * C::OW_BYTES);

  auto wave_rows = [&](int64_t tok0) -> uint32_t {
    const int64_t r = n - tok0;
    return uint32_t(r < 0 ? 0 : (r < 16 ? r : 16));
  };
  auto load_q = [&](int64_t tile, QRaw (&dst)[NQL]) {
    const int64_t tok0 = tile * C::TT + 16 * wave;
    const auto rs = make_rsrc(q + (frame * n + tok0) * D, wave_rows(tok0) * D * EB);
#pragma unroll
    for (int i = 0; i < NQL; ++i) {
      if constexpr (PAIR) dst[i] = buffer_load16(rs, uint32_t(c16 * D + 16 * (g4 + 4 * i)));
      else if constexpr (EB == 1) dst[i] = buffer_load8(rs, uint32_t(c16 * D + 32 * i + 8 * g4));
      else dst[i] = buffer_load16(rs, uint32_t((c16 * D + 32 * i + 8 * g4) * 2));
    }
  };
  QRaw pfa[NQL], pfb[NQL];
  load_q(t_first, pfa);
  load_q(t_first + 1 < t_last ? t_first + 1 : t_first, pfb);

  auto step = [&](int64_t tile, QRaw (&pf)[NQL]) {
    const int64_t tok0 = tile * C::TT + 16 * wave;
    uint4 qf[C::KS];
#pragma unroll
    for (int i = 0; i < NQL; ++i) {
      if constexpr (PAIR) {
        qf[2 * i] = e4m3x8_to_bf16x8(make_uint2(pf[i].x, pf[i].y));
        qf[2 * i + 1] = e4m3x8_to_bf16x8(make_uint2(pf[i].z, pf[i].w));
      } else if constexpr (EB == 1) {
        qf[i] = e4m3x8_to_bf16x8(pf[i]);
      } else {
        qf[i] = pf[i];
      }
    }
    load_q(tile + 2 < t_last ? tile + 2 : t_last - 1, pf);
    // Y^T block jb: the lane holds token c16, output features 16 jb + 4 g4 + 0..3; W'_g's
    // fragments of the next block are read while this one multiplies
    uint4 gcur[C::KS], gnxt[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) gcur[ks] = frg[ks * 64 + lane];
#pragma unroll
    for (int jb = 0; jb < C::NBF; ++jb) {
      if (jb + 1 < C::NBF) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) gnxt[ks] = frg[((jb + 1) * C::KS + ks) * 64 + lane];
      }
      f32x4 ga = f32x4{}, pa = f32x4{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        ga = mfma16_bf16(gcur[ks], qf[ks], ga);
        pa = mfma16_bf16(wo[jb][ks], qf[ks], pa);
      }
      const float4 b4 = *reinterpret_cast<const float4*>(bias_s + 16 * jb + 4 * g4);
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = pa[r] * __builtin_amdgcn_rcpf(1.0f + __expf(-(ga[r] + bb[r])));
      *reinterpret_cast<uint2*>(ow + c16 * C::OWROW + 16 * jb + 4 * g4) =
          make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
      if (jb + 1 < C::NBF) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) gcur[ks] = gnxt[ks];
      }
    }
    // the patch is private to this wave, whose LDS accesses complete in order
    const auto rs = make_rsrc(out + (frame * n + tok0) * DV, wave_rows(tok0) * DV * 2);
    const int orow = lane / C::OCH, och = lane % C::OCH;
#pragma unroll
    for (int j = 0; j < C::OST; ++j) {
      const int r = orow + j * C::ORPI;
      buffer_store16<kCacheStreamOut>(rs, uint32_t(r * DV * 2 + och * 16),
                                      *reinterpret_cast<const uint4*>(ow + r * C::OWROW + och * 8));
    }
  };

  for (int64_t tile = t_first; tile < t_last; tile += 2) {
    step(tile, pfa);
    if (tile + 1 < t_last) step(tile + 1, pfb);
  }
}

// Gradient products of the backward pass: out_f = [Q1 (R1 times) Q2 (R2 times)] S_f, with
// the state S_f (R1 D1 + R2 D2 rows x DV) in state order.  Each factor of a product
// arrives as bf16 hi + lo rows (R = 2), so each input's operand fragments feed two MFMAs
// (dV = [K K] [dB hi ; lo], dK = [K K V V] [M hi ; M lo ; dB^T hi ; dB^T lo]).  The state
// is up to four times as deep as a forward state, so the waves split the output features
// WF ways (and the tokens of a 16 (4 / WF)-token tile the rest), to keep each wave's
// fragments within 32 x 16 bytes per lane.
template <int D1, int R1, int D2, int R2, int DV, int WF>
struct ReadParts {
  static constexpr int KS1 = D1 / 32, KS2 = D2 / 32;
  static constexpr int KS = R1 * KS1 + R2 * KS2;  // k-steps over the state's rows
  static constexpr int DS = 32 * KS;              // state rows
  static constexpr int WT = 4 / WF;               // waves across the tokens of a tile
  static constexpr int TT = 16 * WT;
  static constexpr int FH = DV / WF;              // output features per wave
  static constexpr int NBW = FH / 16;
  static constexpr int NQ = KS1 + KS2;            // operand loads per lane and tile
  static constexpr int OWROW = FH + 8;
  static constexpr int OCH = FH / 8;
  static constexpr int ORPI = 64 / OCH < 16 ? 64 / OCH : 16;
  static constexpr int OST = 16 / ORPI;
  static constexpr int OW_BYTES = 16 * OWROW * 2;
  static constexpr int LDS_BYTES = 4 * OW_BYTES;
  static_assert(NBW >= 1 && NBW * KS <= 32, "fragments exceed the register budget");
};

template <int D1, int R1, int D2, int R2, int DV, int WF>
__global__ void __launch_bounds__(kThreads, 2)
readout_parts_kernel(const uint16_t* __restrict__ q1, const uint16_t* __restrict__ q2,
                     const uint16_t* __restrict__ st, uint16_t* __restrict__ out, int64_t n,
                     int64_t tiles_per_frame, int64_t splits, int64_t tiles_per_split,
                     int64_t head_blocks, int64_t tail_splits, int64_t tail_tiles_per_split) {
  using C = ReadParts<D1, R1, D2, R2, DV, WF>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int th = wave % C::WT, fh = wave / C::WT;
  uint16_t* ow = reinterpret_cast<uint16_t*>(smem + wave * C::OW_BYTES);
  const int c16 = lane & 15, g4 = lane >> 4;
  int64_t frame, t_first, tps;
  if (blockIdx.x < head_blocks) {
    frame = blockIdx.x / splits;
    t_first = (blockIdx.x % splits) * tiles_per_split;
    tps = tiles_per_split;
  } else {
    const int64_t i = blockIdx.x - head_blocks;
    frame = head_blocks / splits + i / tail_splits;
    t_first = (i % tail_splits) * tail_tiles_per_split;
    tps = tail_tiles_per_split;
  }
  const int64_t t_last = (t_first + tps < tiles_per_frame) ? t_first + tps : tiles_per_frame;
  if (t_first >= t_last) return;

  uint4 wfr[C::NBW][C::KS];
  {
    const uint4* sp = reinterpret_cast<const uint4*>(st + frame * int64_t(C::DS) * DV) + lane;
#pragma unroll
    for (int jb = 0; jb < C::NBW; ++jb)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) wfr[jb][ks] = sp[((fh * C::NBW + jb) * C::KS + ks) * 64];
  }
  auto wave_rows = [&](int64_t tok0) -> uint32_t {
    const int64_t r = n - tok0;
    return uint32_t(r < 0 ? 0 : (r < 16 ? r : 16));
  };
  auto load_q = [&](int64_t tile, uint4 (&dst)[C::NQ]) {
    const int64_t tok0 = tile * C::TT + 16 * th;
    const auto r1 = make_rsrc(q1 + (frame * n + tok0) * D1, wave_rows(tok0) * D1 * 2);
#pragma unroll
    for (int ks = 0; ks < C::KS1; ++ks) dst[ks] = buffer_load16(r1, uint32_t((c16 * D1 + 32 * ks + 8 * g4) * 2));
    if constexpr (C::KS2 > 0) {
      const auto r2 = make_rsrc(q2 + (frame * n + tok0) * D2, wave_rows(tok0) * D2 * 2);
#pragma unroll
      for (int ks = 0; ks < C::KS2; ++ks)
        dst[C::KS1 + ks] = buffer_load16(r2, uint32_t((c16 * D2 + 32 * ks + 8 * g4) * 2));
    }
  };
  uint4 pfa[C::NQ], pfb[C::NQ];
  load_q(t_first, pfa);
  load_q(t_first + 1 < t_last ? t_first + 1 : t_first, pfb);

  auto step = [&](int64_t tile, uint4 (&pf)[C::NQ]) {
    const int64_t tok0 = tile * C::TT + 16 * th;
    uint4 qf[C::NQ];
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) qf[i] = pf[i];
    load_q(tile + 2 < t_last ? tile + 2 : t_last - 1, pf);
#pragma unroll
    for (int jb = 0; jb < C::NBW; ++jb) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        // k-step ks of the state: copy r of input 1 (ks < R1 KS1) or of input 2
        const int qi = ks < R1 * C::KS1 ? ks % C::KS1 : C::KS1 + (ks - R1 * C::KS1) % (C::KS2 > 0 ? C::KS2 : 1);
        acc = mfma16_bf16(wfr[jb][ks], qf[qi], acc);
      }
      *reinterpret_cast<uint2*>(ow + c16 * C::OWROW + 16 * jb + 4 * g4) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
    const auto rs = make_rsrc(out + (frame * n + tok0) * DV, wave_rows(tok0) * DV * 2);
    const int orow = lane / C::OCH, och = lane % C::OCH;
    if (orow < C::ORPI) {
#pragma unroll
      for (int j = 0; j < C::OST; ++j) {
        const int r = orow + j * C::ORPI;
        buffer_store16<kCacheStreamOut>(rs, uint32_t(r * DV * 2 + fh * C::FH * 2 + och * 16),
                                        *reinterpret_cast<const uint4*>(ow + r * C::OWROW + och * 8));
      }
    }
  };
  for (int64_t tile = t_first; tile < t_last; tile += 2) {
    step(tile, pfa);
    if (tile + 1 < t_last) step(tile + 1, pfb);
  }
}

// dK product, staged: out_f = [K K V V] Z_f with Z_f the (2 D1 + 2 D2) x DV state (M hi ; M lo ;
// dB^T hi ; dB^T lo).  The state is four times as deep as a forward state, so each wave
// keeps the fragments of a quarter of the output features; the workgroup loads each
// 64-token tile of K and V once (whole 16-byte pieces, coalesced) into LDS, and every
// wave reads its operands from there (double-buffered, one barrier per tile).
template <int D1, int D2, int DV>
struct ReadStaged {
  static constexpr int KS1 = D1 / 32, KS2 = D2 / 32;
  static constexpr int KS = 2 * KS1 + 2 * KS2;
  static constexpr int DS = 32 * KS;
  static constexpr int TT = 64;                   // tokens per tile
  static constexpr int FH = DV / 4;               // output features per wave
  static constexpr int NBW = FH / 16;
  static constexpr int RW = D1 + D2 + 8;          // bf16 per LDS token row (K then V, padded)
  static constexpr int BUF = TT * RW;             // bf16 per tile buffer
  static constexpr int PIECES = TT * (D1 + D2) / 8;  // 16-byte pieces per tile
  static constexpr int PPT = PIECES / kThreads;   // per thread
  static constexpr int OWROW = FH + 8;
  static constexpr int OCH = FH / 8;
  static constexpr int ORPI = 64 / OCH < 16 ? 64 / OCH : 16;
  static constexpr int OST = 16 / ORPI;
  static constexpr int OW_BYTES = 16 * OWROW * 2;
  static constexpr int LDS_BYTES = 2 * BUF * 2 + 4 * OW_BYTES;
  static_assert(NBW >= 1 && PIECES % kThreads == 0, "shape outside the staged product");
};

template <int D1, int D2, int DV>
__global__ void __launch_bounds__(kThreads, 2)
readout_staged_kernel(const uint16_t* __restrict__ q1, const uint16_t* __restrict__ q2,
                      const uint16_t* __restrict__ st, uint16_t* __restrict__ out, int64_t n,
                      int64_t tiles_per_frame, int64_t splits, int64_t tiles_per_split,
                      int64_t head_blocks, int64_t tail_splits, int64_t tail_tiles_per_split) {
  using C = ReadStaged<D1, D2, DV>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* buf = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* ow = reinterpret_cast<uint16_t*>(smem + 2 * C::BUF * 2 + wave * C::OW_BYTES);
  const int c16 = lane & 15, g4 = lane >> 4;
  int64_t frame, t_first, tps;
  if (blockIdx.x < head_blocks) {
    frame = blockIdx.x / splits;
    t_first = (blockIdx.x % splits) * tiles_per_split;
    tps = tiles_per_split;
  } else {
    const int64_t i = blockIdx.x - head_blocks;
    frame = head_blocks / splits + i / tail_splits;
    t_first = (i % tail_splits) * tail_tiles_per_split;
    tps = tail_tiles_per_split;
  }
  const int64_t t_last = (t_first + tps < tiles_per_frame) ? t_first + tps : tiles_per_frame;
  if (t_first >= t_last) return;

  uint4 wfr[C::NBW][C::KS];
  {
    const uint4* sp = reinterpret_cast<const uint4*>(st + frame * int64_t(C::DS) * DV) + lane;
#pragma unroll
    for (int jb = 0; jb < C::NBW; ++jb)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) wfr[jb][ks] = sp[((wave * C::NBW + jb) * C::KS + ks) * 64];
  }
  // tile loads: piece p of a tile is token p / (PR) and 16 bytes (p % PR) of its K (first
  // D1 / 8 pieces) or V row; loads past the frame's last token return zeros
  constexpr int PR = (D1 + D2) / 8;  // pieces per token
  auto load_tile = [&](int64_t tile, uint4 (&r)[C::PPT]) {
    const int64_t tok0 = tile * C::TT;
    const int64_t left = n - tok0;
    const uint32_t rows = uint32_t(left < 0 ? 0 : (left < C::TT ? left : C::TT));
    const auto r1 = make_rsrc(q1 + (frame * n + tok0) * D1, rows * D1 * 2);
    const auto r2 = make_rsrc(q2 + (frame * n + tok0) * D2, rows * D2 * 2);
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int p = i * kThreads + tid, t = p / PR, c = p % PR;
      r[i] = c < D1 / 8 ? buffer_load16(r1, uint32_t((t * D1 + 8 * c) * 2))
                        : buffer_load16(r2, uint32_t((t * D2 + 8 * (c - D1 / 8)) * 2));
    }
  };
  auto store_tile = [&](int b, const uint4 (&r)[C::PPT]) {
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int p = i * kThreads + tid, t = p / PR, c = p % PR;
      *reinterpret_cast<uint4*>(buf + b * C::BUF + t * C::RW + 8 * c) = r[i];
    }
  };
  uint4 ra[C::PPT];
  load_tile(t_first, ra);
  store_tile(0, ra);
  if (t_first + 1 < t_last) load_tile(t_first + 1, ra);
  __syncthreads();

  for (int64_t tile = t_first; tile < t_last; ++tile) {
    const int b = int((tile - t_first) & 1);
    const uint16_t* tb = buf + b * C::BUF;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {  // 16-token groups of the tile
      uint4 qf[C::KS1 + C::KS2];
#pragma unroll
      for (int ks = 0; ks < C::KS1 + C::KS2; ++ks)
        qf[ks] = *reinterpret_cast<const uint4*>(tb + (16 * tg + c16) * C::RW + 32 * ks + 8 * g4);
#pragma unroll
      for (int jb = 0; jb < C::NBW; ++jb) {
        f32x4 acc = f32x4{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          // state k-steps: K (hi rows), K (lo rows), V (hi), V (lo)
          const int qi = ks < 2 * C::KS1 ? ks % C::KS1 : C::KS1 + (ks - 2 * C::KS1) % C::KS2;
          acc = mfma16_bf16(wfr[jb][ks], qf[qi], acc);
        }
        *reinterpret_cast<uint2*>(ow + c16 * C::OWROW + 16 * jb + 4 * g4) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      }
      const int64_t tok0 = tile * C::TT + 16 * tg;
      const int64_t left = n - tok0;
      const uint32_t rows = uint32_t(left < 0 ? 0 : (left < 16 ? left : 16));
      const auto rs = make_rsrc(out + (frame * n + tok0) * DV, rows * DV * 2);
      const int orow = lane / C::OCH, och = lane % C::OCH;
      if (orow < C::ORPI) {
#pragma unroll
        for (int j = 0; j < C::OST; ++j) {
          const int r = orow + j * C::ORPI;
          buffer_store16<kCacheStreamOut>(rs, uint32_t(r * DV * 2 + wave * C::FH * 2 + och * 16),
                                          *reinterpret_cast<const uint4*>(ow + r * C::OWROW + och * 8));
        }
      }
    }
    // the next tile (already in registers) into the other buffer, the one after into registers
    if (tile + 1 < t_last) {
      store_tile(b ^ 1, ra);
      if (tile + 2 < t_last) load_tile(tile + 2, ra);
    }
    __syncthreads();
  }
}

// dK and dV together at d = dv = 128: both products read K, so one workgroup of 8 waves
// stages each 64-token tile of K and V once; waves 0-3 compute quarters of dK = [K K V V] Z
// (as in the staged product above) and waves 4-7 quarters of dV = [K K] DB2 from the same
// staged K, each keeping its own state fragments.
struct ReadKV {
  static constexpr int D = 128;
  static constexpr int THREADS = 512;
  static constexpr int KSK = 16, KSV = 8;           // state k-steps of dK (K hi, K lo, V hi, V lo) and dV
  static constexpr int NBW = 2;                     // 16-feature output blocks per wave (32 features)
  static constexpr int TT = 64;
  static constexpr int RW = 2 * D + 8;              // bf16 per LDS token row (K then V, padded)
  static constexpr int BUF = TT * RW;
  static constexpr int PIECES = TT * 2 * D / 8;
  static constexpr int PPT = PIECES / THREADS;
  static constexpr int OWROW = 32 + 8;
  static constexpr int OW_BYTES = 16 * OWROW * 2;
  static constexpr int LDS_BYTES = 2 * BUF * 2 + 8 * OW_BYTES;
};

__global__ void __launch_bounds__(ReadKV::THREADS)
readout_kv_kernel(const uint16_t* __restrict__ kq, const uint16_t* __restrict__ vq,
                  const uint16_t* __restrict__ zk, const uint16_t* __restrict__ zv,
                  uint16_t* __restrict__ dk, uint16_t* __restrict__ dvo, int64_t n,
                  int64_t tiles_per_frame, int64_t splits, int64_t tiles_per_split,
                  int64_t head_blocks, int64_t tail_splits, int64_t tail_tiles_per_split) {
  using C = ReadKV;
  constexpr int D = C::D;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* buf = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_k = wave < 4;                       // dK waves 0-3, dV waves 4-7
  const int q4 = wave & 3;                          // quarter of the output features
  uint16_t* ow = reinterpret_cast<uint16_t*>(smem + 2 * C::BUF * 2 + wave * C::OW_BYTES);
  const int c16 = lane & 15, g4 = lane >> 4;
  int64_t frame, t_first, tps;
  if (blockIdx.x < head_blocks) {
    frame = blockIdx.x / splits;
    t_first = (blockIdx.x % splits) * tiles_per_split;
    tps = tiles_per_split;
  } else {
    const int64_t i = blockIdx.x - head_blocks;
    frame = head_blocks / splits + i / tail_splits;
    t_first = (i % tail_splits) * tail_tiles_per_split;
    tps = tail_tiles_per_split;
  }
  const int64_t t_last = (t_first + tps < tiles_per_frame) ? t_first + tps : tiles_per_frame;
  if (t_first >= t_last) return;

  // state fragments: dK waves 2 x 16, dV waves 2 x 8 (the first half of the array)
  uint4 wfr[C::NBW][C::KSK];
  {
    const int ks_n = is_k ? C::KSK : C::KSV;
    const int64_t rows = is_k ? 4 * D : 2 * D;
    const uint4* sp = reinterpret_cast<const uint4*>((is_k ? zk : zv) + frame * rows * D) + lane;
#pragma unroll
    for (int jb = 0; jb < C::NBW; ++jb)
#pragma unroll
      for (int ks = 0; ks < C::KSK; ++ks)
        if (ks < ks_n) wfr[jb][ks] = sp[((q4 * C::NBW + jb) * ks_n + ks) * 64];
  }
  constexpr int PR = 2 * D / 8;  // 16-byte pieces per token (K then V)
  uint4 ra[C::PPT];
  auto load_tile = [&](int64_t tile) {
    const int64_t tok0 = tile * C::TT;
    const int64_t left = n - tok0;
    const uint32_t rows = uint32_t(left < 0 ? 0 : (left < C::TT ? left : C::TT));
    const auto r1 = make_rsrc(kq + (frame * n + tok0) * D, rows * D * 2);
    const auto r2 = make_rsrc(vq + (frame * n + tok0) * D, rows * D * 2);
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int p = i * C::THREADS + tid, t = p / PR, c = p % PR;
      ra[i] = c < D / 8 ? buffer_load16(r1, uint32_t((t * D + 8 * c) * 2))
                        : buffer_load16(r2, uint32_t((t * D + 8 * (c - D / 8)) * 2));
    }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int p = i * C::THREADS + tid, t = p / PR, c = p % PR;
      *reinterpret_cast<uint4*>(buf + b * C::BUF + t * C::RW + 8 * c) = ra[i];
    }
  };
  load_tile(t_first);
  store_tile(0);
  if (t_first + 1 < t_last) load_tile(t_first + 1);
  __syncthreads();

  uint16_t* outp = is_k ? dk : dvo;
  for (int64_t tile = t_first; tile < t_last; ++tile) {
    const int b = int((tile - t_first) & 1);
    const uint16_t* tb = buf + b * C::BUF;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      uint4 qf[8];  // K features 0..127 (4 k-steps), then V (4)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        if (is_k || ks < 4) qf[ks] = *reinterpret_cast<const uint4*>(tb + (16 * tg + c16) * C::RW + 32 * ks + 8 * g4);
#pragma unroll
      for (int jb = 0; jb < C::NBW; ++jb) {
        f32x4 acc = f32x4{};
        if (is_k) {
#pragma unroll
          for (int ks = 0; ks < C::KSK; ++ks) acc = mfma16_bf16(wfr[jb][ks], qf[ks < 8 ? ks % 4 : 4 + ks % 4], acc);
        } else {
#pragma unroll
          for (int ks = 0; ks < C::KSV; ++ks) acc = mfma16_bf16(wfr[jb][ks], qf[ks % 4], acc);
        }
        *reinterpret_cast<uint2*>(ow + c16 * C::OWROW + 16 * jb + 4 * g4) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      }
      const int64_t tok0 = tile * C::TT + 16 * tg;
      const int64_t left = n - tok0;
      const uint32_t rows = uint32_t(left < 0 ? 0 : (left < 16 ? left : 16));
      const auto rs = make_rsrc(outp + (frame * n + tok0) * D, rows * D * 2);
      const int orow = lane >> 2, och = lane & 3;  // 16 rows x 4 chunks of 16 bytes
      buffer_store16<kCacheStreamOut>(rs, uint32_t(orow * D * 2 + q4 * 64 + och * 16),
                                      *reinterpret_cast<const uint4*>(ow + orow * C::OWROW + och * 8));
    }
    if (tile + 1 < t_last) {
      store_tile(b ^ 1);
      if (tile + 2 < t_last) load_tile(tile + 2);
    }
    __syncthreads();
  }
}

// smallest output-feature split whose fragments fit 32 x 16 bytes per lane
template <int KS, int DV>
constexpr int parts_wf() {
  return (DV / 16) * KS <= 32 ? 1 : (DV / 32) * KS <= 32 ? 2 : 4;
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
                   const float* __restrict__ xb, float* __restrict__ out, int64_t n,
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

// Grid of the bfloat16 readouts: one workgroup per frame; frames are split in equal
// parts only while there are fewer than four workgroups per compute unit and each part
// keeps 8+ tiles.  Whole frames leave a last, partial round of R frames on S resident
// workgroups (two per CU); those R frames go in k equal parts so that round is about as
// wide as the others.
struct ReadGrid {
  int64_t tpf, splits, tps, head_blocks, tail_splits, tail_tps, grid;
};
ReadGrid readout_grid(int64_t frames, int64_t tpf, int num_cus) {
  ReadGrid g;
  g.tpf = tpf;
  int64_t splits = 1;
  while (frames * splits < 4 * int64_t(num_cus) && tpf >= 16 * splits) splits *= 2;
  g.tps = (tpf + splits - 1) / splits;
  g.splits = (tpf + g.tps - 1) / g.tps;
  int64_t head_frames = frames;
  g.tail_splits = 1;
  g.tail_tps = tpf;
  const int64_t slots = 2 * int64_t(num_cus);
  const int64_t rem = frames % slots;
  if (g.splits == 1 && frames > slots && rem > 0) {
    int64_t k = slots / rem;
    if (k > 4) k = 4;
    if (tpf < 4 * k) k = tpf / 4;
    if (k >= 2) {
      g.tail_tps = (tpf + k - 1) / k;
      g.tail_splits = (tpf + g.tail_tps - 1) / g.tail_tps;
      head_frames = frames - rem;
    }
  }
  g.head_blocks = head_frames * g.splits;
  g.grid = g.head_blocks + (frames - head_frames) * g.tail_splits;
  return g;
}

template <int D, int DV>
hipError_t launch_readout_t(const Problem& p, const void* q, void* out, hipStream_t s, bool prepare) {
  const int64_t frames = p.B * p.H * p.F;
  if (p.bf16) {
    if (prepare) return hipSuccess;  // 17 KB of LDS: no attribute to set
    using C = ReadBf16<D, DV>;
    const ReadGrid gr = readout_grid(frames, (p.n + C::TT - 1) / C::TT, p.num_cus);
    auto launch = [&](auto kern, auto in) {
      using In = decltype(in);
      launch_kernel(p, kern, dim3(unsigned(gr.grid)), dim3(kThreads), C::LDS_BYTES, s,
                    static_cast<const In*>(q), reinterpret_cast<const uint16_t*>(p.xf),
                    reinterpret_cast<const uint16_t*>(p.xb), static_cast<uint16_t*>(out),
                    p.n, gr.tpf, gr.splits, gr.tps, gr.head_blocks, gr.tail_splits, gr.tail_tps);
    };
    if (p.fp8) launch(readout_bf16_kernel<D, DV, uint8_t>, uint8_t{});
    else launch(readout_bf16_kernel<D, DV, uint16_t>, uint16_t{});
  } else {
    // one workgroup per frame, split only when there are too few frames to fill the chip
    int64_t splits = 1;
    while (frames * splits < 1024 && p.n > 256 * splits) splits *= 2;
    const int64_t tps = ((p.n + splits - 1) / splits + 31) / 32 * 32;
    splits = (p.n + tps - 1) / tps;
    const int64_t grid = frames * splits;
    constexpr int lds = ReadF32<D, DV>::LDS_BYTES;
    auto kern = readout_f32_kernel<D, DV>;
    if (prepare)
      return lds > 65536 ? hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds)
                         : hipSuccess;
    launch_kernel(p, kern, dim3(unsigned(grid)), dim3(kThreads), lds, s,
                  static_cast<const float*>(q), p.xf, p.xb, static_cast<float*>(out), p.n,
                  splits, tps);
  }
  return hipGetLastError();
}


template <int D, int DV>
hipError_t launch_readout_gated_t(const Problem& p, const void* q, const GateWeights& gw, void* out,
                                  hipStream_t s, bool prepare) {
  if (!p.bf16) return hipErrorInvalidValue;
  using C = ReadGated<D, DV>;
  if (prepare) {
    if (C::LDS_BYTES <= 65536) return hipSuccess;
    for (const void* k : {reinterpret_cast<const void*>(readout_gated_kernel<D, DV, uint16_t>),
                          reinterpret_cast<const void*>(readout_gated_kernel<D, DV, uint8_t>)}) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const ReadGrid gr = readout_grid(p.B * p.H * p.F, (p.n + C::TT - 1) / C::TT, p.num_cus);
  auto launch = [&](auto kern, auto in) {
    using In = decltype(in);
    launch_kernel(p, kern, dim3(unsigned(gr.grid)), dim3(kThreads), C::LDS_BYTES, s,
                  static_cast<const In*>(q), reinterpret_cast<const uint16_t*>(p.xf),
                  reinterpret_cast<const uint16_t*>(p.xb),
                  static_cast<const uint16_t*>(gw.w_gate), static_cast<const float*>(gw.b_gate),
                  static_cast<const uint16_t*>(gw.w_out), static_cast<uint16_t*>(out), p.n, p.F,
                  p.H, gr.tpf, gr.splits, gr.tps, gr.head_blocks, gr.tail_splits, gr.tail_tps);
  };
  if (p.fp8) launch(readout_gated_kernel<D, DV, uint8_t>, uint8_t{});
  else launch(readout_gated_kernel<D, DV, uint16_t>, uint16_t{});
  return hipGetLastError();
}

template <int D1, int D2, int DV>
hipError_t launch_staged_t(const Problem& p, const void* q1, const void* q2, const void* state, void* out,
                           hipStream_t s, bool prepare) {
  using C = ReadStaged<D1, D2, DV>;
  auto kern = readout_staged_kernel<D1, D2, DV>;
  if (prepare)
    return C::LDS_BYTES > 65536 ? hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES)
                                : hipSuccess;
  const ReadGrid gr = readout_grid(p.B * p.H * p.F, (p.n + C::TT - 1) / C::TT, p.num_cus);
  hipLaunchKernelGGL(kern, dim3(unsigned(gr.grid)), dim3(kThreads), C::LDS_BYTES, s,
                     static_cast<const uint16_t*>(q1), static_cast<const uint16_t*>(q2),
                     static_cast<const uint16_t*>(state), static_cast<uint16_t*>(out), p.n, gr.tpf,
                     gr.splits, gr.tps, gr.head_blocks, gr.tail_splits, gr.tail_tps);
  return hipGetLastError();
}

hipError_t launch_kv_t(const Problem& p, const void* k, const void* v, const void* zk, const void* zv,
                       void* dk, void* dv, hipStream_t s, bool prepare) {
  using C = ReadKV;
  if (prepare)
    return hipFuncSetAttribute(reinterpret_cast<const void*>(readout_kv_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  const ReadGrid gr = readout_grid(p.B * p.H * p.F, (p.n + C::TT - 1) / C::TT, p.num_cus);
  hipLaunchKernelGGL(readout_kv_kernel, dim3(unsigned(gr.grid)), dim3(C::THREADS), C::LDS_BYTES, s,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(zk), static_cast<const uint16_t*>(zv), static_cast<uint16_t*>(dk),
                     static_cast<uint16_t*>(dv), p.n, gr.tpf, gr.splits, gr.tps, gr.head_blocks, gr.tail_splits,
                     gr.tail_tps);
  return hipGetLastError();
}

template <int D1, int R1, int D2, int R2, int DV>
hipError_t launch_parts_t(const Problem& p, const void* q1, const void* q2, const void* state, void* out,
                          hipStream_t s) {
  constexpr int KS = R1 * (D1 / 32) + R2 * (D2 / 32);
  constexpr int WF = parts_wf<KS, DV>();
  using C = ReadParts<D1, R1, D2, R2, DV, WF>;
  const ReadGrid gr = readout_grid(p.B * p.H * p.F, (p.n + C::TT - 1) / C::TT, p.num_cus);
  hipLaunchKernelGGL((readout_parts_kernel<D1, R1, D2, R2, DV, WF>), dim3(unsigned(gr.grid)), dim3(kThreads),
                     C::LDS_BYTES, s, static_cast<const uint16_t*>(q1), static_cast<const uint16_t*>(q2),
                     static_cast<const uint16_t*>(state), static_cast<uint16_t*>(out), p.n, gr.tpf,
                     gr.splits, gr.tps, gr.head_blocks, gr.tail_splits, gr.tail_tps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_readout(const Problem& p, const void* q, void* out, hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_readout_t<DD, VV>(p, q, out, s, false);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

hipError_t prepare_readout(const Problem& p) {
  // the plain readout, and for bfloat16 and FP8 plans the gated one (above 64 KB of LDS)
#define VDA_CASE(DD, VV)                                                                          \
  if (p.d == DD && p.dv == VV) {                                                                   \
    const hipError_t e = launch_readout_t<DD, VV>(p, nullptr, nullptr, nullptr, true);            \
    if (e != hipSuccess || !p.bf16) return e;                                                      \
    return launch_readout_gated_t<DD, VV>(p, nullptr, GateWeights{nullptr, nullptr, nullptr}, nullptr, nullptr, true); \
  }
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda

namespace vda {

hipError_t launch_readout_gated(const Problem& p, const void* q, const GateWeights& gw, void* out,
                                hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_readout_gated_t<DD, VV>(p, q, gw, out, s, false);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda

namespace vda {

hipError_t launch_grad_kv(const Problem& p, const void* k, const void* v, const void* zk, const void* zv,
                          void* dk, void* dv, hipStream_t s) {
  if (p.d == 128 && p.dv == 128) return launch_kv_t(p, k, v, zk, zv, dk, dv, s, false);
  const hipError_t e = launch_grad_dv(p, k, zv, dv, s);
  return e != hipSuccess ? e : launch_grad_dk(p, k, v, zk, dk, s);
}

hipError_t launch_grad_dv(const Problem& p, const void* k, const void* state, void* out, hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_parts_t<DD, 2, 0, 0, VV>(p, k, nullptr, state, out, s);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_grad_dk(const Problem& p, const void* k, const void* v, const void* state, void* out,
                          hipStream_t s) {
  // d = 128: the staged product (a quarter of the output features per wave); narrower
  // outputs keep every operand in the waves' own registers
  if (p.d == 128 && p.dv == 128) return launch_staged_t<128, 128, 128>(p, k, v, state, out, s, false);
  if (p.d == 128 && p.dv == 64) return launch_staged_t<128, 64, 128>(p, k, v, state, out, s, false);
  if (p.d == 128 && p.dv == 32) return launch_staged_t<128, 32, 128>(p, k, v, state, out, s, false);
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_parts_t<DD, 2, VV, 2, DD>(p, k, v, state, out, s);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda

namespace vda {

hipError_t prepare_grad(const Problem& p) {
  if (p.d == 128 && p.dv == 128) {
    const hipError_t e = launch_staged_t<128, 128, 128>(p, nullptr, nullptr, nullptr, nullptr, nullptr, true);
    return e != hipSuccess ? e : launch_kv_t(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true);
  }
  if (p.d == 128 && p.dv == 64) return launch_staged_t<128, 64, 128>(p, nullptr, nullptr, nullptr, nullptr, nullptr, true);
  if (p.d == 128 && p.dv == 32) return launch_staged_t<128, 32, 128>(p, nullptr, nullptr, nullptr, nullptr, nullptr, true);
  return hipSuccess;
}

}  // namespace vda
