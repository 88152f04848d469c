/*
 * vda.h -- C ABI of the MI355X (gfx950) Video Delta Attention forward library.
 *
 * Video Delta Attention (VDA) is the linear-attention branch of VDN-MiniMax-H3.
 * What it computes, per (batch b, head h), is described on the VDN-MiniMax-H3
 * pages: the aiezz page, section 03 "technical principles", bullets "Video Delta
 * Attention" (each frame's spatial tokens jointly set the new state through the
 * normal equations; the frame-wise extension of the token-wise delta rule) and
 * "dual text injection" (the text is written once, at initialisation, into the
 * bidirectional state); the laicaila page, section "technical principles", the
 * same two bullets; and the comfyui-wiki page, section "how Video DeltaNet speeds
 * up H3" (a bidirectional linear-attention branch with a constant-cost recurrent
 * state).  The pages give no formula; this library computes the regularised
 * frame-level least-squares reading of them.  With the state X = S^T (d x dv):
 *
 *   X_text   = (lam I + Kt^T Kt)^{-1} (Kt^T Vt)                 text tokens, zero start
 *   X_fwd_0  = X_text,  X_fwd_f = (lam I + K_f^T K_f)^{-1} (lam X_fwd_{f-1} + K_f^T V_f),  f = 1..F
 *   X_bwd_F+1= X_text,  X_bwd_f = (lam I + K_f^T K_f)^{-1} (lam X_bwd_{f+1} + K_f^T V_f),  f = F..1
 *   O_f      = Q_f (X_fwd_f + X_bwd_f) / 2                      n x dv per frame
 *
 * There is no feature map, 1/sqrt(d) scaling, decay or gate inside the op, and
 * no output rows for the text tokens.
 *
 * Conventions for every call:
 *  - Every call returns a vda_status.  Nothing aborts, and no C++ exception
 *    crosses this boundary.
 *  - All tensors are device pointers into the memory of the GPU that was current
 *    when the plan was created, contiguous and row-major, in the plan's dtype
 *    (vda_dtype), 16-byte aligned.  The caller owns them; the library never frees or
 *    keeps them past the call.
 *  - Layouts (head-major, one contiguous n x d slab per (b,h,frame)):
 *      q, k   [B][H][F][n][d]      v, out [B][H][F][n][dv]
 *      text_k [B][H][T][d]         text_v [B][H][T][dv]
 *  - out must not overlap any input.
 */
#ifndef VDA_H
#define VDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct vda_plan_s* vda_plan_t;

/* Element types.  Accumulation and the solves are float32 in every case.
 *   F32:      q, k, v, text_k, text_v and out are float32.
 *   BF16:     all six are bfloat16, as raw 16-bit words.
 *   FP8_E4M3: q, k, v, text_k and text_v are OCP FP8 E4M3 codes, one byte each (sign,
 *             4 exponent bits with bias 7, 3 mantissa bits; largest magnitude 448; no
 *             infinities; S.1111.111 is NaN); out is bfloat16.  Every code's value is
 *             exact in bfloat16, and from there the pass is the BF16 one. */
typedef enum {
  VDA_DTYPE_F32 = 0,
  VDA_DTYPE_BF16 = 1,
  VDA_DTYPE_FP8_E4M3 = 2
} vda_dtype;

typedef enum {
  VDA_SUCCESS = 0,
  VDA_ERROR_INVALID_VALUE = 1,  /* bad size, lambda, NULL pointer, aliasing, wrong device */
  VDA_ERROR_NOT_SUPPORTED = 2,  /* d or dv outside {32, 64, 128}, unknown dtype, n or T too large */
  VDA_ERROR_MISALIGNED = 3,     /* a tensor pointer is not 16-byte aligned */
  VDA_ERROR_OUT_OF_MEMORY = 4,  /* workspace allocation failed */
  VDA_ERROR_DEVICE = 5,         /* a HIP runtime call or kernel launch failed */
  VDA_ERROR_TOO_LARGE = 6       /* vda_forward_noalloc: the problem needs more workspace than
                                   its fixed scratch (VDA_NOALLOC_SCRATCH_BYTES) holds */
} vda_status;

/* Pipeline stages of one forward pass, in the order they must run. */
typedef enum {
  VDA_STAGE_STATS = 1,    /* per frame (and the text): G = K^T K, Bm = K^T V, (lam I + G)^{-1} */
  VDA_STAGE_SCAN = 2,     /* forward and backward state scans over the frames */
  VDA_STAGE_READOUT = 4,  /* O_f = Q_f (X_fwd_f + X_bwd_f) / 2 */
  VDA_STAGE_ALL = 7
} vda_stage;

/* Create a plan for one problem shape.
 *   B, H, F, n, T >= 0: batch, heads, frames, spatial tokens per frame, text tokens.
 *     n and T are at most 16776960 (2^24 - 256); larger gives NOT_SUPPORTED.
 *     B*H*F*n == 0 gives a plan whose forward pass has no output element: it does
 *     nothing, reads no pointer and returns VDA_SUCCESS.  T == 0 means no text: the
 *     text state is zero and text_k / text_v may be NULL.
 *   d, dv in {32, 64, 128}: key/query width and value width.
 *   lambda: the regulariser, finite and > 0, shared by the text and every frame.
 *     Accuracy depends on the condition number kappa of lam I + K_f^T K_f (the inverse is
 *     formed explicitly in float32 and the chains run in split bfloat16).  Verified against a
 *     float64 reference at a max per-frame relative error <= 1e-2 for bfloat16 and FP8 inputs
 *     up to kappa ~ 8e3 (5.2e-3 at 8.2e3: rank-16 keys, lam = 1e-3).  Beyond that the error
 *     grows with kappa: 2.0e-2 at 4.3e4, 1.0e-1 at 1.1e5.  Unit-norm keys with lam = 1 give
 *     kappa near 1 + n/d.
 *   dtype: element types of the tensors (vda_dtype).
 * The plan allocates its workspace (hipMalloc, one block) on the current device and
 * keeps it until vda_plan_destroy.  Its scans start in the automatic mode of
 * vda_plan_set_scan_chunk (the chunked scan for few heads and many frames, which allocates
 * its chunk summaries here too).  On error *plan_out is set to NULL.
 * Errors: INVALID_VALUE, NOT_SUPPORTED, OUT_OF_MEMORY, DEVICE. */
vda_status vda_plan_create(int64_t B, int64_t H, int64_t F, int64_t n, int64_t d, int64_t dv,
                           int64_t T, float lambda, vda_dtype dtype, vda_plan_t* plan_out);

/* Choose how the forward pass runs its state scans (row f1 of the hot path: a chunked
 * scan over the frames, the composition of the affine step X -> lam A_f^{-1} X + A_f^{-1} B_f
 * being associative).  chunk_frames == 0 runs each chain serially over its F + 1 steps.
 * chunk_frames > 0 splits each chain into K = ceil(F / chunk_frames) chunks of that many
 * frames and runs three passes: every chunk from a zero state, together with its transition
 * P_j = product of lam A_f^{-1} over its frames, in parallel; the true start of every chunk,
 * serially over the K chunk ends (X_{j+1} = P_j X_j + C_j, in float32); and every chunk again
 * from its true start, writing the states.  The result is that of the serial scan up to
 * rounding (the same bar against the oracle).  It pays where the serial chains leave the GPU
 * idle -- few heads per GPU, as in a head-sharded share of the problem -- and costs about
 * three times the scan's work where they do not (measured on one MI355X: 768p with 3 heads,
 * scan 0.137 -> 0.094 ms; the long clip with 3 heads, 0.533 -> 0.250 ms; the long clip with
 * 24 heads, 0.745 -> 1.21 ms or more).
 * chunk_frames == VDA_SCAN_CHUNK_AUTO (the choice every plan starts with) takes the chunked
 * scan only when the serial chains' workgroups (2*B*H*dv/32 of them) fill at most a quarter of
 * the GPU's compute units and F >= 48, with K = the number of chunks whose local pass about
 * fills the compute units (2 <= K <= min(8, F/4)); otherwise the serial scan.
 * The plan allocates the chunk summaries here (hipMalloc; 2*B*H*K*(d*d + 2*d*dv) floats, none
 * when the scan is serial) and frees any earlier ones; the forward calls then allocate nothing.
 * Call it with no pass of the plan in flight.  The backward pass always runs its chains
 * serially.
 * Errors: INVALID_VALUE (NULL plan, chunk_frames < VDA_SCAN_CHUNK_AUTO), NOT_SUPPORTED
 * (chunk_frames > 0 on a float32 plan), OUT_OF_MEMORY, DEVICE. */
#define VDA_SCAN_CHUNK_AUTO (-1)
vda_status vda_plan_set_scan_chunk(vda_plan_t plan, int64_t chunk_frames);

/* The chunk length the plan's forward passes use: 0 for the serial scan, else frames per
 * chunk (the automatic choice resolved).  Errors: INVALID_VALUE (NULL argument). */
vda_status vda_plan_get_scan_chunk(vda_plan_t plan, int64_t* chunk_frames);

/* Enqueue the whole forward pass on `stream` (a hipStream_t; NULL is the null
 * stream) and return without waiting.  Arguments are checked on the host before
 * anything is enqueued; an error leaves out untouched.  Faults during execution
 * surface at the caller's next synchronisation, as for any HIP work.
 * The plan's workspace is reused by every call, so at most one forward pass per
 * plan may be in flight; separate plans are independent.
 * Results are bitwise reproducible for the same inputs and plan.
 * The call makes no runtime call on the stream but kernel launches (and timing events,
 * when enabled), so it may be captured into a HIP graph; the plan's workspace stays at
 * the same address for the plan's lifetime, and a replay reads the captured pointers.
 * Errors: INVALID_VALUE, MISALIGNED, DEVICE. */
vda_status vda_forward(vda_plan_t plan, const void* q, const void* k, const void* v,
                       const void* text_k, const void* text_v, void* out, void* stream);

/* Enqueue only the stages in `stages` (a bitwise OR of vda_stage), in pipeline
 * order.  A stage reads what the previous stage last wrote into the plan's
 * workspace, so running SCAN or READOUT alone is valid only after the earlier
 * stages have run on this plan.  Pointers a selected stage does not read may be
 * NULL (STATS reads k, v, text_k, text_v; SCAN none; READOUT q and writes out).
 * Used for per-stage timing and for checking intermediate results.
 * Errors: as vda_forward, and INVALID_VALUE for stages outside VDA_STAGE_ALL. */
vda_status vda_forward_stages(vda_plan_t plan, unsigned stages, const void* q, const void* k,
                              const void* v, const void* text_k, const void* text_v, void* out,
                              void* stream);

/* The forward pass followed by the linear branch's gated fusion epilogue, per head h
 * and output row O (1 x dv) of the pass:
 *   Y = sigmoid(O W_g^T + b_g) * (O W_o^T)          (elementwise product)
 * The pages give each attention branch a content-dependent sigmoid gate and an output
 * projection of its own before the branches merge (the aiezz page, section 03, and the
 * laicaila page, section "technical principles": bullet "gated fusion"); this is that
 * step for the linear branch, with the branch output as the gate's content and a
 * per-head dv x dv projection.  Merging with the other branch is not part of it.
 *   w_gate, w_out  [H][dv][dv] bfloat16, [output feature][input feature] (the layout of a
 *                  torch Linear weight), shared by every batch entry;
 *   b_gate         [H][dv] float32;
 *   out            [B][H][F][n][dv] bfloat16: Y in place of the plain output.
 * Other arguments, pointer rules, stream and capture behaviour as for vda_forward; the
 * weights may not overlap out.  Timing, when enabled, records these passes too.
 * Errors: as vda_forward, and NOT_SUPPORTED for float32 plans. */
vda_status vda_forward_gated(vda_plan_t plan, const void* q, const void* k, const void* v,
                             const void* text_k, const void* text_v, const void* w_gate,
                             const void* b_gate, const void* w_out, void* out, void* stream);

/* Backward pass: the gradients of L = sum(d_out * O) with respect to q, k, v, text_k
 * and text_v, where O is the output of vda_forward.  The pages train the branch (the
 * aiezz page, section 03, and the laicaila page, "technical principles": bullet "three-
 * stage training adaptation"), which needs them.  With A_f = lam I + K_f^T K_f and
 * dW_f = Q_f^T dO_f, the two chains' adjoints run in the opposite directions with the same
 * solves, U_f = A_f^{-1}(dW_f/2 + lam U_{f+1}) and V_f = A_f^{-1}(dW_f/2 + lam V_{f-1});
 * then dB_f = U_f + V_f, dA_f = -(U_f X_fwd_f^T + V_f X_bwd_f^T),
 * dK_f = V_f dB_f^T + K_f (dA_f + dA_f^T), dV_f = K_f dB_f, dQ_f = dO_f W_f^T, and the text
 * gets the same terms from U_0 = A_0^{-1} lam (U_1 + V_F).
 * The call reads the statistics (the inverses and K^T V of every frame) that the last
 * vda_forward (or vda_forward_gated) on this plan left in its workspace, and recomputes the
 * states from them in float32: run the forward pass first,
 * with the same k, v, text_k, text_v, and keep the plan's workspace untouched in between.
 * On a plan whose workspace holds no statistics yet (no forward pass enqueued) the call
 * returns INVALID_VALUE.
 *   d_out          [B][H][F][n][dv], the gradient of the output;
 *   d_q, d_k, d_v, d_text_k, d_text_v: written, same layouts as q, k, v, text_k, text_v.
 * All tensors are bfloat16.  Only bfloat16 plans are supported.  The first call on a plan
 * allocates its backward workspace (hipMalloc, kept until vda_plan_destroy); later calls
 * make no runtime call but kernel launches and may be captured.  Outputs may not overlap
 * inputs or each other.  With no output element (F or n = 0) every gradient is zero.
 * When timing is enabled (vda_plan_enable_timing) a backward call is recorded as one
 * timed pass with three spans.  At d = dv = 128: the state recompute with one pass over
 * (Q, dO) that forms Q^T dO and dQ; the adjoint chains with the per-frame terms; dK and dV.
 * At other widths: Q^T dO; the state recompute, the adjoint chains and the per-frame terms;
 * dQ, dK and dV.
 * Errors: INVALID_VALUE, MISALIGNED, OUT_OF_MEMORY, DEVICE; NOT_SUPPORTED for float32 and
 * FP8 plans. */
vda_status vda_backward(vda_plan_t plan, const void* q, const void* k, const void* v,
                        const void* text_k, const void* text_v, const void* d_out, void* d_q,
                        void* d_k, void* d_v, void* d_text_k, void* d_text_v, void* stream);

/* Bytes of the fixed device scratch of vda_forward_noalloc, per GPU. */
#define VDA_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* The whole forward pass, as vda_forward computes it, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes the problem shape directly (no plan; arguments as for vda_plan_create) and the
 * tensors as for vda_forward, and allocates nothing: the pass's workspace (the inverses,
 * K^T V and the state sequences) lives in a fixed array of VDA_NOALLOC_SCRATCH_BYTES of
 * device memory that the library holds on every GPU it runs on until the process ends.  The
 * workspace a problem needs is the one vda_plan_workspace_bytes reports for a plan of the same
 * shape; a problem that needs more returns VDA_ERROR_TOO_LARGE before anything is enqueued
 * (at d = dv = 128 in bfloat16 that is about 17.8 MB per head at 90 frames of any n, so three
 * 768p heads fit).  The first call on a device looks up the array's address on that device and
 * sets the kernels' attributes there (no allocation); later calls make no runtime call but
 * kernel launches.  Every call on a GPU uses that GPU's one array: calls that overlap in time on
 * one GPU (on different streams, or from different threads) race and give undefined results;
 * calls ordered on one stream are safe.  The scans run serially, so results are bitwise those of
 * vda_forward on a plan of the same shape running the serial scan (vda_plan_set_scan_chunk 0;
 * a plan in the automatic mode that chose the chunked scan agrees up to rounding).  The output
 * is complete when the stream reaches the end of the pass.
 * Errors: as vda_plan_create and vda_forward (but never OUT_OF_MEMORY), and TOO_LARGE. */
vda_status vda_forward_noalloc(int64_t B, int64_t H, int64_t F, int64_t n, int64_t d, int64_t dv,
                               int64_t T, float lambda, vda_dtype dtype, const void* q,
                               const void* k, const void* v, const void* text_k, const void* text_v,
                               void* out, void* stream);

/* Per-stage timing of whole forward passes, for benchmarks.  After
 * vda_plan_enable_timing(plan, capacity) with capacity > 0, each of the next `capacity`
 * vda_forward calls times each stage with a pair of HIP events on the stream it runs on,
 * recorded by the stage's kernel launch itself (hipExtLaunchKernelGGL), so that no event
 * packet sits between the kernels.  capacity == 0 turns timing off; enabling again discards what was recorded.  The
 * events are created on the current device, which must be the plan's.
 * Errors: INVALID_VALUE (capacity < 0 or > 100000), OUT_OF_MEMORY, DEVICE. */
vda_status vda_plan_enable_timing(vda_plan_t plan, int capacity);

/* Which stages' kernels record their events in timed calls (a bitwise OR of vda_stage; the
 * default is VDA_STAGE_ALL).  Each timed stage adds a pair of events to a pass; a benchmark that
 * needs one stage's live duration can time that stage alone.  Stages not timed are reported as
 * 0 ms by vda_plan_timings.  Errors: INVALID_VALUE (NULL plan, bits outside VDA_STAGE_ALL, or
 * timed calls recorded and not yet read). */
vda_status vda_plan_set_timed_stages(vda_plan_t plan, unsigned stages);

/* Waits for the timed calls recorded since timing was enabled or last read, and returns
 * their number in *calls and the mean duration in milliseconds of each stage launch
 * (statistics, scan, readout).  Any of the float pointers may be NULL.  Resets the count.
 * Errors: INVALID_VALUE (NULL plan or calls), DEVICE. */
vda_status vda_plan_timings(vda_plan_t plan, int* calls, float* stats_ms, float* scan_ms,
                            float* readout_ms);

/* Free the plan and its workspace.  The caller must make sure no forward pass on
 * the plan is still running (synchronise its stream first).  NULL is accepted. */
vda_status vda_plan_destroy(vda_plan_t plan);

/* Bytes of device workspace the plan holds (0 for NULL): the forward workspace, plus the
 * backward workspace once vda_backward has allocated it, plus the chunked scan's summaries
 * (vda_plan_set_scan_chunk). */
size_t vda_plan_workspace_bytes(vda_plan_t plan);

/* Static, human-readable name of a status code. */
const char* vda_status_string(vda_status s);

/* Device pointers into the plan's workspace, for checking intermediate results
 * after a synchronised forward pass.  Layouts, with BH = B*H and frame index 0 for
 * the text and 1..F for the frames:
 * The pointers are untyped: what each buffer holds depends on the plan's dtype, as follows.
 *   ainv  [BH][F+1][d][d]   (lam I + K^T K)^{-1}: float32 row-major for float32 plans.  For
 *                           bfloat16 and FP8 plans each frame's d*d*4 bytes start with two
 *                           bfloat16 planes, hi then lo, with hi + lo = the inverse; the
 *                           inverse is symmetric and a plane stores only its 16 x 16 blocks
 *                           (R, C) with R <= C, NB = d/16 of them per side: block (R, C) at
 *                           index R*NB - R*(R-1)/2 + (C - R), 256 elements each, row-major;
 *                           a plane is NB*(NB+1)/2 * 256 elements
 *   bm    [BH][F+1][d*dv]   K^T V, float32, blocked (below)
 *   x_fwd [BH][F][d*dv]     forward state after frame f (f = 1..F at index f-1)
 *   x_bwd [BH][F][d*dv]     backward state after frame f
 * Blocked layout of a d x dv matrix M: element (r, c) is at
 *   (((c/16 * d/16 + r/16) * 4 + (r%16)/4) * 16 + c%16) * 4 + r%4.
 * The states are float32 and blocked for float32 plans.  For the others they are
 * bfloat16 (d*dv bfloat16 per frame, in a slot of d*dv*4 bytes per frame), rounded
 * once from the float32 chain, with element (r, c) at
 *   (((c/16 * d/32 + r/32) * 4 + (r%32)/8) * 16 + c%16) * 8 + r%8
 * (the operand order of the readout's MFMA); the chain itself runs in float32.  For FP8
 * plans with d >= 64, r in that formula is the row with bit 3 moved above bits 4-5:
 *   (row & ~0x38) | ((row & 0x08) << 2) | ((row & 0x30) >> 1).
 * The memory stays owned by the plan.  Any output pointer may be NULL. */
vda_status vda_debug_workspace(vda_plan_t plan, const void** ainv, const void** bm,
                               const void** x_fwd, const void** x_bwd);

#ifdef __cplusplus
}
#endif

#endif /* VDA_H */
