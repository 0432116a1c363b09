/*
 * lvsa.h -- C ABI of the MI355X (gfx950) LVSA frame-block-sparse attention.
 *
 * LVSA ("LVSA: Training-Free Sparse Attention for Long Video Diffusion";
 * gist.science explainer, Technical Summary §2 "Core Mechanism") restricts
 * every latent query frame t of a video diffusion transformer to a key-frame
 * set A(t) = G_s ∪ W(t): rotating global anchor frames G_s plus an expanded
 * local window W(t), with |A(t)| held at a budget C.  The mask is rebuilt on
 * the host every denoising step (TechWalker article on LVSA, §二 and §三) and
 * the attention runs only over the frame blocks it lists.
 *
 * Conventions for every call:
 *   - Return value: LVSA_OK (0) or a negative LVSA_ERR_* code.  A readable
 *     message for the last failure on the calling thread is returned by
 *     lvsa_last_error().
 *   - Ownership: the caller owns every buffer, host and device, including
 *     the optional workspace of lvsa_attention_ws.  The library allocates no
 *     device memory, frees nothing, keeps no pointer after the call returns,
 *     and never synchronises a stream.
 *   - Thread safety: all calls are reentrant; error messages are per thread.
 */
#ifndef LVSA_H_
#define LVSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LVSA_ABI_VERSION 2

/* Status codes. */
#define LVSA_OK            0
#define LVSA_ERR_ARG      -1 /* argument out of domain or null pointer           */
#define LVSA_ERR_CAPACITY -2 /* caller buffer smaller than the required size     */
#define LVSA_ERR_SHAPE    -3 /* tensor shapes/strides/alignment not supported    */
#define LVSA_ERR_DTYPE    -4 /* element type not supported (bf16 only)           */
#define LVSA_ERR_HIP      -5 /* no gfx950 device, or a HIP launch error          */
#define LVSA_ERR_MASK     -6 /* CSR mask malformed                               */

/* Anchor rotation flags for lvsa_build_mask.
 *   LVSA_ROT_MOD_TPER (default): anchor offset o_s = step mod Tper, the shift
 *     the gist.science explainer prints (Technical Summary §2, "Rotating
 *     Global Anchors": G_s shifts by s mod Tper).
 *   LVSA_ROT_MOD_T: o_s = step mod T, anchors advancing one frame per step
 *     cyclically over the frame count (TechWalker article, §三).  Identical
 *     to the default whenever Tper divides T.
 *   LVSA_FIXED_GRID: o_s = 0 at every step, the non-rotating grid the pages
 *     describe as the cause of fixed-grid bias (ablation).
 *   LVSA_WINDOW_ONLY: no anchors; A(t) = the min(C, T) frames nearest to t
 *     (ties to the lower index), i.e. plain sliding-window attention, the
 *     prior-art pattern the pages contrast LVSA with (ablation; t_per and
 *     n_anchor are reported as 0). */
#define LVSA_ROT_MOD_TPER 0
#define LVSA_ROT_MOD_T    1
#define LVSA_FIXED_GRID   2
#define LVSA_WINDOW_ONLY  3

/* Element types. */
#define LVSA_DTYPE_BF16 1

/* What lvsa_build_mask derived for the step. */
typedef struct lvsa_mask_info {
  int32_t c_eff;    /* min(C, T): key frames per query frame                  */
  int32_t t_per;    /* anchor spacing Tper = ceil(T/(C-W)); 0 when T <= C     */
  int32_t n_anchor; /* anchor count n_g = ceil(T/Tper); 0 when T <= C         */
  int32_t offset;   /* anchor offset o_s used at this step; 0 when T <= C     */
  int32_t nnz;      /* T * c_eff entries written to col_idx                   */
} lvsa_mask_info;

/* A 4-D tensor [B, H, N, D] in device memory, D contiguous (stride 1).
 * Strides are in elements.  N is the token count T*P, token index t*P + p
 * (frame-major).  data must be 16-byte aligned and stride_b, stride_h,
 * stride_n multiples of 8 elements (16 bytes). */
typedef struct lvsa_tensor {
  void *data;
  int64_t B, H, N, D;
  int64_t stride_b, stride_h, stride_n;
  int32_t dtype; /* LVSA_DTYPE_BF16 */
} lvsa_tensor;

/* ABI version (LVSA_ABI_VERSION).  A library convention; no passage of the
 * pages defines it. */
int lvsa_version(void);

/* Message describing the last failure on this thread ("" if none).  The
 * string is owned by the library and valid until the next call on this
 * thread.  A library convention; no passage of the pages defines it. */
const char *lvsa_last_error(void);

/* Number of col_idx entries lvsa_build_mask writes for (T, C, W):
 * T * min(C, T), every query frame keeping exactly the budget of key frames
 * (TechWalker article, §二: the window is extended until the effective
 * count is back at the target C; fewer than C frames exist when T < C).
 * Same argument domain as lvsa_build_mask (step and flags do not change
 * the size).  Errors: LVSA_ERR_ARG. */
int lvsa_mask_nnz(int32_t T, int32_t C, int32_t W, int32_t *nnz_out);

/* Host mask builder: the key frames of every query frame at one denoising
 * step, as CSR.
 *
 * Source: gist.science explainer, Technical Summary §2 "Core Mechanism"
 * (A(t) = G ∪ W(t); rotating periodic anchors; window extended over anchors
 * so |A(t)| stays at the budget C); TechWalker article §二 (C = training
 * horizon in latent frames; Tper ≈ T/(C−W); extension on the CPU) and §三
 * (rotation; constant anchor count; each frame an anchor once per period).
 *
 * Definition (readings of the pages where they leave a step open):
 *   T <= C : every row is 0..T-1 (dense; at the training horizon the method
 *            is the dense model).
 *   T >  C, flags != LVSA_WINDOW_ONLY : Tper = ceil(T/(C-W)), n_g = ceil(T/Tper),
 *            G = { (o_s + k*Tper) mod T : 0 <= k < n_g }, o_s per flags;
 *            W(t) = the C - n_g non-anchor frames nearest to t, ties to the
 *            lower frame index (so the window slides inward at the ends and
 *            grows past anchors it overlaps);
 *            A(t) = G ∪ W(t), |A(t)| = C.
 *
 * Arguments (all host memory, caller-owned):
 *   T >= 1 frames, C >= 2 budget, 1 <= W <= C-1 window, step >= 0, flags one
 *   of LVSA_ROT_MOD_TPER / LVSA_ROT_MOD_T / LVSA_FIXED_GRID /
 *   LVSA_WINDOW_ONLY.
 *   row_ptr [T+1] out: row_ptr[t] = t * c_eff.
 *   col_idx [cap] out: rows concatenated, each ascending and unique.
 *   info    out, may be NULL.
 * Errors: LVSA_ERR_ARG (domain, null row_ptr/col_idx, host memory exhausted
 *   for the builder's O(T) scratch), LVSA_ERR_CAPACITY (cap < T * min(C,T));
 *   on error nothing is written. */
int lvsa_build_mask(int32_t T, int32_t C, int32_t W, int32_t step, int32_t flags,
                    int32_t *row_ptr, int32_t *col_idx, int32_t cap,
                    lvsa_mask_info *info);

/* Host mask builder for a run of denoising steps: the masks of steps
 * step0 .. step0+n_steps-1, as lvsa_build_mask builds them, in one buffer, so
 * that a whole sampling run's masks can be copied to the device once and the
 * step sequence launched (or captured in a HIP graph) with no per-step host
 * work.  (The pages put the mask on the CPU every step -- TechWalker article,
 * §二 and §三 -- and name per-step pattern scheduling as the overhead that
 * keeps short sequences from gaining -- same article, §五.)
 *
 * Every step's rows have c_eff entries, so all steps share one row_ptr:
 *   row_ptr [T+1]               out: row_ptr[t] = t * c_eff.
 *   col_idx [n_steps * nnz]     out: step step0+i's col_idx at offset i*nnz,
 *                                    nnz = T * min(C, T).
 *   info    [n_steps]           out, may be NULL: lvsa_mask_info of each step.
 * The step-i mask is (row_ptr, col_idx + i*nnz, nnz) for lvsa_attention.
 * Arguments otherwise as lvsa_build_mask; n_steps >= 1 and
 * step0 + n_steps - 1 <= INT32_MAX.  Errors: LVSA_ERR_ARG, LVSA_ERR_CAPACITY
 * (cap < n_steps * nnz); on an argument or capacity error nothing is written
 * (if host memory runs out part way, earlier steps may have been). */
int lvsa_build_mask_steps(int32_t T, int32_t C, int32_t W, int32_t step0, int32_t n_steps,
                          int32_t flags, int32_t *row_ptr, int32_t *col_idx, int64_t cap,
                          lvsa_mask_info *info);

/* Host check of a CSR frame mask (any source), a library convention (the
 * pages define no mask format): row_ptr[0] == 0,
 * non-decreasing, row_ptr[T] == nnz, every row non-empty, ascending, unique
 * and within [0, T).  Errors: LVSA_ERR_ARG (null/negative sizes),
 * LVSA_ERR_MASK (the first violation, described by lvsa_last_error()). */
int lvsa_validate_mask(int32_t T, const int32_t *row_ptr, const int32_t *col_idx,
                       int32_t nnz);

/* Frame-block-sparse attention on the GPU.
 *
 * Source: gist.science explainer, Technical Summary §2 ("Core Mechanism":
 * query frame t attends to the frames of A(t) only; "Complexity": per query
 * O(C·P·d), so the sparsity block is the frame).  For every (b, h) and query
 * token i of frame t = i / P:
 *   out[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:]·k[b,h,j,:]) v[b,h,j,:]
 * over the key tokens j of the frames in A(t) (non-causal, no bias).
 * Arithmetic: bf16 products on the matrix cores with fp32 accumulation, fp32
 * online softmax, probabilities rounded to bf16 for the P·V product, output
 * rounded to bf16 (nearest-even).
 *
 * Arguments:
 *   q, k, v, out : [B, H, N, D] bf16 device tensors, identical B/H/N/D,
 *                  D in {64, 128}, N = T * P.  out must not overlap q/k/v
 *                  (byte extents) and no two of its (b, h, token) rows may
 *                  share memory; q/k/v may (a stride of 0 broadcasts, e.g.
 *                  one K/V head shared by several query heads).
 *   row_ptr_dev  : [T+1] int32 device array, CSR row offsets into col_idx.
 *   col_idx_dev  : [nnz] int32 device array, key frames of each query frame,
 *                  ascending and unique per row (lvsa_build_mask's output
 *                  copied to the device).  An entry outside [0, T), or not
 *                  above the last entry kept before it in its row, is
 *                  skipped, and offsets are clamped to [0, nnz], so a
 *                  malformed mask gives wrong numbers, never an
 *                  out-of-bounds access; a row with no kept frame yields
 *                  zeros.
 *   T            : frames (N % T must be 0).
 *   nnz          : length of col_idx_dev.
 *   scale        : softmax scale; <= 0 selects 1/sqrt(D).
 *   stream       : hipStream_t to launch on (NULL = default stream).
 * Tensors, mask arrays and stream belong to the current HIP device.
 * The call is asynchronous on `stream`.  Argument errors are reported
 * synchronously and launch nothing.  Errors: LVSA_ERR_ARG, LVSA_ERR_SHAPE,
 * LVSA_ERR_DTYPE, LVSA_ERR_HIP (no gfx950 device current, launch failure). */
int lvsa_attention(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                   const int32_t *row_ptr_dev, const int32_t *col_idx_dev,
                   int32_t T, int32_t nnz, lvsa_tensor *out, float scale,
                   void *stream);

/* Bytes of device workspace lvsa_attention_ws needs for tensors of B, H, N
 * tokens and head size D split into T frames (a library convention; the
 * pages define no workspace): one float per (b, h, frame) rounded up to
 * 256, 256 bytes of work counters, and room for the partial results of the
 * work items that run as two halves (see lvsa_attention_ws: at most 32 per
 * XCD of 8-wave records when frames hold >= 384 tokens, 96 of 4-wave
 * records otherwise; about 109 MB at D = 128 once there are enough items,
 * none below 32 items).
 * Errors: LVSA_ERR_ARG, LVSA_ERR_SHAPE (D not 64/128, N % T != 0). */
int lvsa_attention_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t T, int64_t *bytes);

/* Work items (both attention entry points).  Frames of at least 384 tokens
 * (every video workload): items of 384 consecutive query tokens of one
 * (b, h), run by 8-wave workgroups of 48 rows per wave, one per CU; an item
 * that crosses a frame boundary walks the union of the two frames' rows,
 * each wave (or, for a wave whose rows straddle the boundary, each row)
 * taking only its own frame's key frames.  Shorter frames: items of 128
 * rows of one frame, 4-wave workgroups.  Items are cut into 8 contiguous
 * ranges, one per XCD.
 *
 * lvsa_attention with a caller-provided device workspace (a library
 * convention: the pages define the computation, not this split of it),
 * used to drop the online softmax's running maximum where that is safe.
 *
 * Source: the same computation as lvsa_attention (gist.science explainer,
 * Technical Summary §2).  The workspace changes only the softmax's reference
 * point, which cancels in the normalisation: a first kernel writes the
 * largest key norm of every (b, h, frame) to the workspace.  By
 * Cauchy-Schwarz, R_i = scale·log2(e)·|q_i|·(largest key norm over A(t))
 * bounds |score·log2(e)| of query i; a wave whose 64 lanes all have
 * 2·R_i <= 96 (every row's largest probability then >= 2^-96) takes R_i as
 * a fixed reference -- no running maximum, no rescaling, and the subtraction
 * folded into the Q·K^T product (its Q rows are pre-scaled by
 * scale·log2(e) and rounded to bf16, one extra rounding: relative RMS error
 * about 2.9e-3 against 2.3e-3 for lvsa_attention on unit-variance inputs).
 * Other waves keep the running-maximum arithmetic of lvsa_attention.
 * Results agree with lvsa_attention to that accuracy, not bit for bit; rows
 * whose waves all fall back are bit-identical unless their work item runs
 * as two merged halves (below), which rounds differently.
 *
 * The workspace also holds one work counter per XCD: workgroups take their
 * (b, h, frame, query tile) items from counters instead of a fixed split,
 * so that faster XCDs take over items of slower ones; and the last items of
 * each XCD's share run as two halves of their CSR row, whose partial
 * results a second kernel merges (shorter items at the end of the launch,
 * where the last workgroups finish at different times).  Which workgroup
 * computes an item does not change its result: outputs are bitwise
 * reproducible from call to call.
 *
 * Arguments as lvsa_attention, plus:
 *   workspace        : device memory of at least
 *                      lvsa_attention_workspace_bytes(B, H, N, D, T) bytes,
 *                      16-byte aligned, not overlapping q/k/v/out.  Owned by
 *                      the caller; overwritten by the call (stream-ordered),
 *                      so concurrent calls need separate workspaces.
 *   workspace_bytes  : its size.
 * After the call (stream-ordered), the workspace's first B·H·T floats hold
 * the largest key norm of every (b, h, frame) at index (b·H + h)·T + t,
 * computed in fp32 from the bf16 keys; the rest of it is scratch.
 * Errors: those of lvsa_attention; LVSA_ERR_ARG (NULL, misaligned or
 * overlapping workspace), LVSA_ERR_CAPACITY (too small). */
int lvsa_attention_ws(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                      const int32_t *row_ptr_dev, const int32_t *col_idx_dev,
                      int32_t T, int32_t nnz, lvsa_tensor *out, float scale,
                      void *workspace, int64_t workspace_bytes, void *stream);

/* lvsa_attention_ws without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not allocate, harnesses that forbid it).  It calls no allocating
 * routine: the workspace is the library's own static device array of
 * LVSA_STATIC_SCRATCH_BYTES bytes, one per GPU, held until the process ends.
 *
 * Same computation, arguments and errors as lvsa_attention_ws minus the
 * workspace arguments.  The key-norm table (one float per (b, h, frame)) and
 * the work counters must fit the array: B·H·T <= (LVSA_STATIC_SCRATCH_BYTES
 * - 512) / 4, else LVSA_ERR_CAPACITY and nothing is launched.  The items run
 * as two merged halves are limited to what the rest of the array holds, so
 * results can differ from lvsa_attention_ws in rounding (same accuracy).
 * The counters are cleared by the call's own first kernel.
 *
 * Every call on one GPU uses that GPU's single array: calls whose kernels
 * can overlap on one GPU (different streams, or several host threads without
 * ordering) race and give wrong results.  Calls ordered on one stream are
 * safe.  The array keeps the last call's contents. */
#define LVSA_STATIC_SCRATCH_BYTES (16 << 20)
int lvsa_attention_ws_static(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                             const int32_t *row_ptr_dev, const int32_t *col_idx_dev,
                             int32_t T, int32_t nnz, lvsa_tensor *out, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LVSA_H_ */
