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
// split over several workgroups, each owning a slice of the columns; all workgroups
// of one chain are placed on one XCD so that Ainv_f is fetched from HBM once and hit
// in L2 after.  Within a workgroup each wave owns 16-row blocks of X; the right
// operand R = lam X + Bm of a step is exchanged through LDS.
//
// float32 plans: 16x16x4 fp32 MFMA, 16 columns per workgroup.
// bfloat16 plans: split-bf16 products on 16x16x32 bf16 MFMA, 32 columns per workgroup
// and one wave per 16 rows.  Ainv_f arrives as two bf16 planes (hi + lo) and R is split
// the same way each step; Ainv R is taken as hi*hi + hi*lo + lo*hi, which leaves a
// relative error of order 2^-16 per product (far below the bf16 rounding of the inputs
// and output).  The operands of the next step are in flight while a step computes.
// The states leave the chain only for the readout: float32 and blocked for float32
// plans, bf16 in the readout's operand order for bfloat16 plans (rows in the paired
// order when the inputs are FP8 and d >= 64).
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

// bfloat16 plans.  One wave per 16-row block of X (D/16 waves), 32 columns of X per
// workgroup (DV/32 workgroups per chain).  Each wave loads only its own 16 rows of
// Ainv_f, as 1 KB fragment-ordered runs (frag_index), and the 32-column slice of Bm.
// How the bfloat16 scan stores its states: bf16 in the readout's operand order, the same
// with the FP8 plans' paired row order, or float32 blocked (for the backward pass).
constexpr int kStoreBf16 = 0, kStorePairedBf16 = 1, kStoreF32 = 2;

template <int D, int DV>
struct ScanBf16Cfg {
  static constexpr int NW = D / 16;               // waves; wave w owns rows 16w..16w+15
  static constexpr int THREADS = 64 * NW;
  static constexpr int KS = D / 32;               // k-steps of the 16x16x32 MFMA
  static constexpr int CW = 2;                    // 16-column blocks per workgroup
  static constexpr int NCB = DV / (16 * CW);      // workgroups per chain
  static constexpr int NSLOT = 2;                 // operand ring: this step and the next
  static constexpr int CBE = 2 * KS * 4 * 16 * 8;  // R of one 16-column block: [hi/lo][ks][kg][n][8]
  static constexpr int NUB = sym_blocks(D);       // stored 16 x 16 blocks of Ainv per plane
  static constexpr int ABUF = 2 * NUB * 256;      // bf16 of one frame's two packed planes
  static constexpr int APIECES = ABUF / 8;        // their 16-byte pieces
  static constexpr int APT = (APIECES + THREADS - 1) / THREADS;  // pieces per thread
  static constexpr int RSB = CW * CBE;            // bf16 of one R buffer
  static constexpr int LDS_BYTES = (2 * ABUF + 2 * RSB) * 2;
  static_assert(DV % (16 * CW) == 0, "value width must be a multiple of 32");
  static_assert(APIECES % 64 == 0 && THREADS % 64 == 0, "pieces must split into whole waves");
};

// What one launch of the bfloat16 scan kernel runs (chain steps: 0 = the text, 1..F = the
// frames in the chain's order):
//   kSegSerial: every chain from step 0 to F, storing every state;
//   kSegLocal:  the chunked scan's local pass.  A chunk is `len` consecutive chain steps,
//               chunk 0 being steps 0..len and chunk j >= 1 steps 1 + j len .. (j+1) len.  For
//               chunks 0..K-2 of every chain it runs the update from a zero state, giving the
//               chunk's end state C_j (chunk 0: the true end state, stored with every state on
//               the way), and, for chunks 1..K-2, the chunk's transition P_j = product of
//               lam Ainv_f over its steps, in step order (the same chain on lam I with no Bm);
//   kSegRerun:  the chunked scan's last pass: chunks 1..K-1 from their true start states,
//               storing every state.
// Chunk summaries (float32): P_j row-major d x d, C_j and the start states blocked d x dv.
constexpr int kSegSerial = 0, kSegLocal = 1, kSegRerun = 2;
struct ChunkArgs {
  int64_t len;      // chain steps per chunk (chunk 0 also holds step 0)
  int64_t nchunks;  // K >= 2 for the chunked passes
  float* pc;        // [nchains][K][d*d]  P_j
  float* cc;        // [nchains][K][d*dv] C_j
  float* starts;    // [nchains][K][d*dv] true state before chunk j's first step (j >= 1)
};

template <int D, int DV, int MODE>
__global__ void __launch_bounds__(4 * D)
scan_bf16_kernel(const uint16_t* __restrict__ ainv_planes, const float* __restrict__ bm,
                 float* __restrict__ xf, float* __restrict__ xb, int64_t nchains, int64_t F,
                 float lam, int64_t grid, int store_mode, ChunkArgs ch) {
  using C = ScanBf16Cfg<D, DV>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* abuf = reinterpret_cast<uint16_t*>(smem);  // [2][ABUF]: packed Ainv planes of two steps
  uint16_t* rsb = abuf + 2 * C::ABUF;                   // [2][RSB]: R of this step and the next

  const int64_t L = xcd_remap(blockIdx.x, grid);
  int64_t chain, s_begin = 0, s_end = F, j = 0;
  int cb;
  bool transition = false;  // this workgroup runs P_j (no Bm, columns of a d x d product)
  if constexpr (MODE == kSegSerial) {
    chain = L / C::NCB;
    cb = int(L % C::NCB);
  } else if constexpr (MODE == kSegLocal) {
    constexpr int G = C::NCB + D / 32;  // C_j's column blocks, then P_j's
    const int64_t grp = L / G;
    const int slot = int(L % G);
    chain = grp / (ch.nchunks - 1);
    j = grp % (ch.nchunks - 1);
    transition = slot >= C::NCB;
    cb = transition ? slot - C::NCB : slot;
    if (transition && j == 0) return;  // chunk 0 starts from the text state: no P_0
    s_begin = j == 0 ? 0 : 1 + j * ch.len;
    s_end = (j + 1) * ch.len < F ? (j + 1) * ch.len : F;
  } else {
    const int64_t grp = L / C::NCB;
    cb = int(L % C::NCB);
    chain = grp / (ch.nchunks - 1);
    j = 1 + grp % (ch.nchunks - 1);
    s_begin = 1 + j * ch.len;
    s_end = (j + 1) * ch.len < F ? (j + 1) * ch.len : F;
  }
  if (chain >= nchains) return;
  // every state of the segment is stored (the serial scan, the rerun, and chunk 0 of the local
  // pass, whose zero start is the true one); the local pass also keeps its end state
  const bool store_all = MODE != kSegLocal || (j == 0 && !transition);
  const int64_t bh = chain >> 1;
  const bool backward = chain & 1;
  const int64_t F1 = F + 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int c0 = cb * 16 * C::CW;
  const int row0 = wave * 16 + 4 * g;  // first of the 4 output rows of this lane
  // where those rows go in the stored state (FP8 plans: the paired row order)
  const int srow0 = store_mode == kStorePairedBf16 ? paired_row(row0) : row0;

  const uint16_t* ainv_h = ainv_planes + bh * F1 * int64_t(2 * D * D);
  const float* bm_h = bm + bh * F1 * int64_t(D) * DV;
  uint16_t* xo_h = reinterpret_cast<uint16_t*>(backward ? xb : xf) + bh * F * int64_t(D) * DV;

  // frame index (0 = text) of chain step s; steps past the end re-read the last frame
  auto frame_at = [&](int64_t s) -> int64_t {
    if (s > F) s = F;
    return (s == 0 || !backward) ? s : F + 1 - s;
  };

  // Ainv of a step: the frame's packed planes (one contiguous run) are copied into an LDS
  // buffer two steps ahead, and every wave forms its operand fragments from there one
  // step ahead.  Blocks on and above the diagonal are read directly (lane: row n, 8
  // consecutive columns); a block below it is the mirrored block read with the
  // transposing LDS read: in each 16-lane group lane 4a + b receives element b of the
  // 4-element reads of lanes a, a+4, a+8, a+12, so lane i points at row k + i/4 (+4 for
  // the second read) and columns 4(i%4)..+3 of the mirrored block, and receives column
  // i of 4 consecutive rows.
  // The planes travel HBM -> registers -> LDS: the loads of step s + 3 are issued at the start
  // of step s into one of two register sets, and committed to LDS at the end of step s + 1,
  // so each load has a whole step to land instead of being waited for in the step that
  // issued it.
  uint4 ast0[C::APT], ast1[C::APT];
  auto stage_a = [&](int64_t t, uint4 (&dst)[C::APT]) {
    const auto rsrc = make_rsrc(ainv_h + frame_at(t) * int64_t(2 * D * D), uint32_t(C::APIECES * 16));
#pragma unroll
    for (int i = 0; i < C::APT; ++i) dst[i] = buffer_load16(rsrc, uint32_t((i * C::THREADS + tid) * 16));
  };
  auto commit_a = [&](int b, const uint4 (&src)[C::APT]) {
#pragma unroll
    for (int i = 0; i < C::APT; ++i) {
      const int piece = i * C::THREADS + tid;  // whole waves fall on either side of the end
      if (piece < C::APIECES) *reinterpret_cast<uint4*>(abuf + b * C::ABUF + piece * 8) = src[i];
    }
  };
  auto tr_frag = [&](const uint16_t* blk, int kh) -> uint4 {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const uint16_t* p = blk + (8 * kh + (n >> 2)) * 16 + 4 * (n & 3);
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p));
    const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 64));
    const uint2 xl = __builtin_bit_cast(uint2, x), yl = __builtin_bit_cast(uint2, y);
    return make_uint4(xl.x, xl.y, yl.x, yl.y);
  };
  auto frags_a = [&](int b, uint4 (&a)[C::KS][2]) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int bc = 2 * ks + (g >> 1);  // column block of this lane's half of the k-step
      const int lo_b = wave < bc ? wave : bc, hi_b = wave < bc ? bc : wave;
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        const uint16_t* blk = abuf + b * C::ABUF + pl * C::NUB * 256 + sym_block(lo_b, hi_b, D) * 256;
        if (wave <= 2 * ks) {               // every lane on or above the diagonal
          a[ks][pl] = *reinterpret_cast<const uint4*>(blk + n * 16 + 8 * (g & 1));
        } else if (wave > 2 * ks + 1) {     // every lane below it
          a[ks][pl] = tr_frag(blk, g & 1);
        } else {                            // the diagonal block of one half, mirrored block of the other
          const uint4 d = *reinterpret_cast<const uint4*>(blk + n * 16 + 8 * (g & 1));
          const uint4 t = tr_frag(blk, g & 1);
          a[ks][pl] = bc >= wave ? d : t;
        }
      }
    }
  };

  // slot t of the ring holds the Ainv fragments of step t and the Bm that step t adds for t+1
  uint4 A[C::NSLOT][C::KS][2];
  float4 Bv[C::NSLOT][C::CW];
  auto load_bm = [&](int64_t t, float4 (&bv)[C::CW]) {
    if (MODE == kSegLocal && transition) {  // a transition adds no Bm
#pragma unroll
      for (int cw = 0; cw < C::CW; ++cw) bv[cw] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      return;
    }
    const float* bsrc = bm_h + frame_at(t + 1) * int64_t(D) * DV;
#pragma unroll
    for (int cw = 0; cw < C::CW; ++cw)
      bv[cw] = *reinterpret_cast<const float4*>(bsrc + blk_index(row0, c0 + 16 * cw + n, D));
  };
  // R fragment (8 consecutive k of column n) and the 4-row output slot of a lane
  auto rs_frag = [&](int buf, int cw, int hl, int ks) -> const uint4* {
    return reinterpret_cast<const uint4*>(&rsb[buf * C::RSB + cw * C::CBE + ((hl * C::KS + ks) * 4 + g) * 128 + n * 8]);
  };
  auto rs_out = [&](int buf, int cw, int hl) -> uint2* {
    return reinterpret_cast<uint2*>(&rsb[buf * C::RSB + cw * C::CBE +
                                         ((hl * C::KS + wave / 2) * 4 + 2 * (wave % 2) + g / 2) * 128 +
                                         n * 8 + 4 * (g % 2)]);
  };
  auto write_r = [&](int buf, int cw, float r0, float r1, float r2, float r3) {
    uint32_t h01, l01, h23, l23;
    split_bf16x2(r0, r1, h01, l01);
    split_bf16x2(r2, r3, h23, l23);
    *rs_out(buf, cw, 0) = make_uint2(h01, h23);
    *rs_out(buf, cw, 1) = make_uint2(l01, l23);
  };

  // R of the segment's first step: lam X_prev + Bm with X_prev = 0 (the text step, and the local
  // pass's zero starts), the chunk's true start state (rerun), or lam I for a transition
#pragma unroll
  for (int cw = 0; cw < C::CW; ++cw) {
    const int col = c0 + 16 * cw + n;
    float4 r4;
    if (MODE == kSegLocal && transition) {
      r4 = make_float4(row0 == col ? lam : 0.0f, row0 + 1 == col ? lam : 0.0f, row0 + 2 == col ? lam : 0.0f,
                       row0 + 3 == col ? lam : 0.0f);
    } else {
      r4 = *reinterpret_cast<const float4*>(bm_h + frame_at(s_begin) * int64_t(D) * DV + blk_index(row0, col, D));
      if constexpr (MODE == kSegRerun) {
        const float4 x4 = *reinterpret_cast<const float4*>(ch.starts + (chain * ch.nchunks + j) * int64_t(D) * DV +
                                                           blk_index(row0, col, D));
        r4 = make_float4(__builtin_fmaf(lam, x4.x, r4.x), __builtin_fmaf(lam, x4.y, r4.y),
                         __builtin_fmaf(lam, x4.z, r4.z), __builtin_fmaf(lam, x4.w, r4.w));
      }
    }
    write_r(0, cw, r4.x, r4.y, r4.z, r4.w);
  }
  stage_a(s_begin, ast0);
  commit_a(0, ast0);
  stage_a(s_begin + 1, ast0);
  commit_a(1, ast0);
  stage_a(s_begin + 2, ast0);  // committed at the end of the first step
  load_bm(s_begin, Bv[0]);
  __syncthreads();
  frags_a(0, A[0]);
  __syncthreads();  // every wave has its first fragments before the first step overwrites buffer 0

  // r: the step's index within the segment (its LDS buffers and register slots alternate)
  auto step = [&](int64_t s, int64_t r, uint4 (&a)[C::KS][2], float4 (&bv)[C::CW], uint4 (&a_fill)[C::KS][2],
                  float4 (&bv_fill)[C::CW], uint4 (&as_issue)[C::APT], const uint4 (&as_commit)[C::APT]) {
    const int buf = int(r & 1);
    stage_a(s + 3, as_issue);  // committed at the end of the next step
    load_bm(s + 1, bv_fill);
    // every R fragment of the step in one LDS round trip; then, so that their LDS traffic
    // overlaps the MFMA chains, the next step's fragments (its planes were committed before the
    // last barrier) and the planes of step s+2 (loaded during the last step) into the buffer
    // whose fragments were taken before the last barrier
    uint4 rf[C::CW][C::KS][2];
#pragma unroll
    for (int cw = 0; cw < C::CW; ++cw)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        rf[cw][ks][0] = *rs_frag(buf, cw, 0, ks);
        rf[cw][ks][1] = *rs_frag(buf, cw, 1, ks);
      }
    frags_a(buf ^ 1, a_fill);
    commit_a(buf, as_commit);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 x[C::CW];
#pragma unroll
    for (int cw = 0; cw < C::CW; ++cw) {
      f32x4 hh = f32x4{}, hl = f32x4{}, lh = f32x4{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        hh = mfma16_bf16(a[ks][0], rf[cw][ks][0], hh);
        hl = mfma16_bf16(a[ks][0], rf[cw][ks][1], hl);
        lh = mfma16_bf16(a[ks][1], rf[cw][ks][0], lh);
      }
      x[cw] = hh + (hl + lh);
    }
    if constexpr (MODE == kSegLocal) {
      if (s == s_end) {
        // the segment's end state, float32: the true start of chunk 1 (chunk 0), C_j, or P_j
        if (transition) {
          float* dst = ch.pc + (chain * ch.nchunks + j) * int64_t(D) * D;
#pragma unroll
          for (int cw = 0; cw < C::CW; ++cw)
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[(row0 + q) * D + c0 + 16 * cw + n] = x[cw][q];
        } else {
          float* dst = (j == 0 ? ch.starts + (chain * ch.nchunks + 1) * int64_t(D) * DV
                               : ch.cc + (chain * ch.nchunks + j) * int64_t(D) * DV);
#pragma unroll
          for (int cw = 0; cw < C::CW; ++cw)
            *reinterpret_cast<float4*>(dst + blk_index(row0, c0 + 16 * cw + n, D)) =
                make_float4(x[cw][0], x[cw][1], x[cw][2], x[cw][3]);
        }
      }
    }
    if (store_all && s >= 1) {
      // The states leave the chain only for the readout, which rounds their mean to bf16
      // for its MFMA: they are stored as bf16 in the readout's operand order (state_index),
      // a lane's 4 rows as 8 bytes, and kept out of the caches.
      if (store_mode == kStoreF32) {
        // float32 and blocked (the backward pass, where the states meet cancellation)
        float* dst = reinterpret_cast<float*>(backward ? xb : xf) + (bh * F + frame_at(s) - 1) * int64_t(D) * DV;
#pragma unroll
        for (int cw = 0; cw < C::CW; ++cw)
          *reinterpret_cast<float4*>(dst + blk_index(row0, c0 + 16 * cw + n, D)) =
              make_float4(x[cw][0], x[cw][1], x[cw][2], x[cw][3]);
      } else {
        uint16_t* dst = xo_h + (frame_at(s) - 1) * int64_t(D) * DV;
#pragma unroll
        for (int cw = 0; cw < C::CW; ++cw)
          __builtin_nontemporal_store(
              u32x2{pack_bf16x2(x[cw][0], x[cw][1]), pack_bf16x2(x[cw][2], x[cw][3])},
              reinterpret_cast<u32x2*>(dst + state_index(srow0, c0 + 16 * cw + n, D)));
      }
    }
    if (s < s_end) {
#pragma unroll
      for (int cw = 0; cw < C::CW; ++cw)
        write_r(buf ^ 1, cw, __builtin_fmaf(lam, x[cw][0], bv[cw].x), __builtin_fmaf(lam, x[cw][1], bv[cw].y),
                __builtin_fmaf(lam, x[cw][2], bv[cw].z), __builtin_fmaf(lam, x[cw][3], bv[cw].w));
    }
    __syncthreads();
  };

  static_assert(C::NSLOT == 2, "the plane registers alternate with the step's parity");
  const int64_t nsteps = s_end - s_begin + 1;
  for (int64_t r0 = 0; r0 < nsteps; r0 += 2) {
    step(s_begin + r0, r0, A[0], Bv[0], A[1], Bv[1], ast1, ast0);
    if (r0 + 1 >= nsteps) break;
    step(s_begin + r0 + 1, r0 + 1, A[1], Bv[1], A[0], Bv[0], ast0, ast1);
  }
}

// The chunked scan's carry pass: for every chain, the true start states of chunks 2..K-1 from
// that of chunk 1, X_{j+1} = P_j X_j + C_j for j = 1..K-2, in float32 on the 16x16x4 float32
// MFMA.  One workgroup per chain and 16-column slice of X (d/16 waves of 16 rows each); the
// right operand goes through LDS.
template <int D, int DV>
__global__ void __launch_bounds__(kThreads)
chunk_carry_kernel(ChunkArgs ch, int64_t nchains) {
  constexpr int RB = D / 16, NW = RB < 4 ? RB : 4, RBW = RB / NW, NCB = DV / 16;
  __shared__ __align__(16) float rs[D * 16];  // X_j, this workgroup's 16 columns: [row block][g][col][r]
  const int64_t chain = blockIdx.x / NCB;
  const int cb = int(blockIdx.x % NCB);
  if (chain >= nchains) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const bool active = wave < NW;
  const int c0 = cb * 16;
  const int64_t K = ch.nchunks;
  auto rs_at = [&](int jb) -> float* { return rs + ((jb * 4 + g) * 16 + n) * 4; };
  float* st = ch.starts + chain * K * int64_t(D) * DV;
  if (active) {
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const int row = (wave * RBW + i) * 16 + 4 * g;
      *reinterpret_cast<float4*>(rs_at(wave * RBW + i)) =
          *reinterpret_cast<const float4*>(st + 1 * int64_t(D) * DV + blk_index(row, c0 + n, D));
    }
  }
  __syncthreads();
  for (int64_t jj = 1; jj + 1 < K; ++jj) {
    f32x4 acc[RBW];
    if (active) {
      const float* P = ch.pc + (chain * K + jj) * int64_t(D) * D;
#pragma unroll
      for (int i = 0; i < RBW; ++i) acc[i] = f32x4{};
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        const float4 rr = *reinterpret_cast<const float4*>(rs_at(jb));
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
          const int row = (wave * RBW + i) * 16 + n;
          const float4 a = *reinterpret_cast<const float4*>(P + row * D + 16 * jb + 4 * g);
          acc[i] = mfma16_f32(a.x, rr.x, acc[i]);
          acc[i] = mfma16_f32(a.y, rr.y, acc[i]);
          acc[i] = mfma16_f32(a.z, rr.z, acc[i]);
          acc[i] = mfma16_f32(a.w, rr.w, acc[i]);
        }
      }
    }
    __syncthreads();  // every wave has read X_j
    if (active) {
      const float* Cj = ch.cc + (chain * K + jj) * int64_t(D) * DV;
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        const int row = (wave * RBW + i) * 16 + 4 * g;
        const int idx = blk_index(row, c0 + n, D);
        const float4 c4 = *reinterpret_cast<const float4*>(Cj + idx);
        const float4 x4 = make_float4(acc[i][0] + c4.x, acc[i][1] + c4.y, acc[i][2] + c4.z, acc[i][3] + c4.w);
        *reinterpret_cast<float4*>(st + (jj + 1) * int64_t(D) * DV + idx) = x4;
        *reinterpret_cast<float4*>(rs_at(wave * RBW + i)) = x4;
      }
    }
    __syncthreads();
  }
}

// The chunk summaries' place in the plan's chunk workspace: P_j, C_j and the start states,
// [2BH][K] of each.
template <int D, int DV>
ChunkArgs chunk_args(const Problem& p) {
  const int64_t nchains = 2 * p.B * p.H, K = (p.F + p.scan_chunk - 1) / p.scan_chunk;
  ChunkArgs ch;
  ch.len = p.scan_chunk;
  ch.nchunks = K;
  ch.pc = p.chunk_ws;
  ch.cc = ch.pc + nchains * K * int64_t(D) * D;
  ch.starts = ch.cc + nchains * K * int64_t(D) * DV;
  return ch;
}

template <int D, int DV>
hipError_t launch_scan_t(const Problem& p, hipStream_t s, bool prepare) {
  const int64_t nchains = 2 * p.B * p.H;
  if (p.bf16) {
    using C = ScanBf16Cfg<D, DV>;
    auto kern = scan_bf16_kernel<D, DV, kSegSerial>;
    auto kern_local = scan_bf16_kernel<D, DV, kSegLocal>;
    auto kern_rerun = scan_bf16_kernel<D, DV, kSegRerun>;
    if (prepare) {
      if (C::LDS_BYTES <= 65536) return hipSuccess;
      for (const void* k : {reinterpret_cast<const void*>(kern), reinterpret_cast<const void*>(kern_local),
                            reinterpret_cast<const void*>(kern_rerun)}) {
        const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
    const int store = p.states_f32 ? kStoreF32 : (p.fp8 && D >= 64) ? kStorePairedBf16 : kStoreBf16;
    const int64_t K = p.scan_chunk > 0 ? (p.F + p.scan_chunk - 1) / p.scan_chunk : 1;
    const auto planes = reinterpret_cast<const uint16_t*>(p.ainv);
    if (K < 2 || p.chunk_ws == nullptr) {
      const int64_t grid = ((nchains + kXcds - 1) / kXcds) * kXcds * C::NCB;
      launch_kernel(p, kern, dim3(unsigned(grid)), dim3(C::THREADS), C::LDS_BYTES, s, planes, p.bm, p.xf, p.xb,
                    nchains, p.F, p.lam, grid, store, ChunkArgs{});
      return hipGetLastError();
    }
    // chunked: local pass, carry pass (K > 2), rerun; the stage's timing events go on the
    // first and the last launch
    const ChunkArgs ch = chunk_args<D, DV>(p);
    Problem first = p, mid = p, last = p;
    first.ev_stop = nullptr;
    mid.ev_start = mid.ev_stop = nullptr;
    last.ev_start = nullptr;
    const int64_t groups = ((nchains * (K - 1) + kXcds - 1) / kXcds) * kXcds;
    const int64_t grid_local = groups * (C::NCB + D / 32);
    launch_kernel(first, kern_local, dim3(unsigned(grid_local)), dim3(C::THREADS), C::LDS_BYTES, s, planes, p.bm,
                  p.xf, p.xb, nchains, p.F, p.lam, grid_local, store, ch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (K > 2) {
      launch_kernel(mid, chunk_carry_kernel<D, DV>, dim3(unsigned(nchains * (DV / 16))), dim3(kThreads), 0, s, ch,
                    nchains);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int64_t grid_rerun = groups * C::NCB;
    launch_kernel(last, kern_rerun, dim3(unsigned(grid_rerun)), dim3(C::THREADS), C::LDS_BYTES, s, planes, p.bm,
                  p.xf, p.xb, nchains, p.F, p.lam, grid_rerun, store, ch);
  } else {
    using C = ScanCfg<D, DV>;
    if (prepare) return hipSuccess;  // static LDS only
    const int64_t grid = ((nchains + kXcds - 1) / kXcds) * kXcds * C::NCB;
    launch_kernel(p, scan_kernel<D, DV>, dim3(unsigned(grid)), dim3(kThreads), 0, s, p.ainv,
                  p.bm, p.xf, p.xb, nchains, p.F, p.lam, grid);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const Problem& p, hipStream_t s) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_scan_t<DD, VV>(p, s, false);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

hipError_t prepare_scan(const Problem& p) {
#define VDA_CASE(DD, VV) \
  if (p.d == DD && p.dv == VV) return launch_scan_t<DD, VV>(p, nullptr, true);
  VDA_CASE(32, 32) VDA_CASE(32, 64) VDA_CASE(32, 128)
  VDA_CASE(64, 32) VDA_CASE(64, 64) VDA_CASE(64, 128)
  VDA_CASE(128, 32) VDA_CASE(128, 64) VDA_CASE(128, 128)
#undef VDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace vda
