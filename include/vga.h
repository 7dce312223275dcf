/*
 * vga.h -- C ABI of the alternating-attention library (libvga.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation set follows three pages:
 *  - "VGGT CVPR25 Best Paper" notes, section "Alternating-Attention": a
 *    trunk that alternates frame-wise self-attention (each frame's tokens
 *    attend to their own frame) with global self-attention (every token of
 *    every frame attends to all N*L tokens); the N*L x N*L matrix must never
 *    be materialised (FlashAttention remark in the same section).
 *  - "AVGGT: Rethinking Global Attention for Accelerating VGGT", technical
 *    summary, section 3 (Methodology): step one converts the early global
 *    layers to frame attention; step two, Subsampled Global Attention (SGA),
 *    keeps every query, keeps K/V only on a strided s_h x s_w patch grid
 *    (plus the special tokens), keeps each token's own diagonal term,
 *    replaces all dropped K/V columns by one global mean column, and puts
 *    the three parts under one shared softmax.
 *  - "VGGT-Omega" notes, section 2 (first architectural change, Register
 *    Attention) and architecture section 2.3: some global layers restrict
 *    the cross-frame exchange to the per-frame register and camera tokens
 *    (the special tokens here); image tokens stay inside their frame.
 *
 * Tensor layout (all calls): Q, K, V and O are contiguous device arrays of
 * shape [T, H, D] with T = N * L tokens, token-major and frame-major: token
 * t = f * L + u belongs to frame f; inside a frame the gh*gw patch tokens
 * come first in row-major grid order (u = r * gw + c), then the S special
 * tokens (u >= gh*gw).  D (head_dim) must be 64.  The element type is fp32
 * or bf16 for all four arrays of one call; accumulation is always fp32.
 *
 * Conventions for every call:
 *  - Ownership: the caller allocates and frees every device buffer (Q, K, V,
 *    O, workspace).  The library allocates no device memory and keeps no
 *    pointer after it returns.
 *  - Asynchrony: work is only enqueued on `stream` (a hipStream_t; NULL is
 *    the default stream).  No call synchronises the host, except when the
 *    environment variable VGA_DEBUG_SYNC=1 is set (then each call waits for
 *    its own work and reports asynchronous faults as VGA_ERR_HIP).
 *  - Errors: a status code, never an exception.  All argument checks run
 *    before anything is enqueued, so a failing call enqueues nothing;
 *    vga_last_error() gives a thread-local text for the last failure.
 *  - Requirements: Q/K/V/O (and the workspace) 16-byte aligned; O must not
 *    overlap Q, K, V or the workspace; each array at most 2^31 elements.
 *  - Thread safety: all calls are stateless and may run concurrently on
 *    different streams.
 *  - Graph capture: a call enqueues kernel launches only (no allocation, no
 *    memset, no host synchronisation without VGA_DEBUG_SYNC), so it may be
 *    captured into a HIP graph; a replay recomputes the same result.
 */
#ifndef VGA_H
#define VGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VGA_ABI_VERSION 6

typedef enum {
  VGA_OK = 0,
  VGA_ERR_NULL = 1,        /* a required pointer is NULL                    */
  VGA_ERR_SHAPE = 2,       /* inconsistent N, L, grid, S, H or size limit   */
  VGA_ERR_DTYPE = 3,       /* dtype is not VGA_F32 / VGA_BF16               */
  VGA_ERR_PARAM = 4,       /* bad SGA stride/phase/flag or schedule counts  */
  VGA_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned       */
  VGA_ERR_ALIAS = 6,       /* O overlaps an input or the workspace          */
  VGA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required       */
  VGA_ERR_UNSUPPORTED = 8, /* head_dim != 64, or more heads than supported */
  VGA_ERR_HIP = 9          /* the HIP runtime reported an error             */
} vga_status;

typedef enum { VGA_F32 = 0, VGA_BF16 = 1 } vga_dtype;

/* Shape of Q/K/V/O: N frames of L = grid_h*grid_w + num_special tokens. */
typedef struct {
  int32_t num_frames;       /* N >= 1                                        */
  int32_t tokens_per_frame; /* L; must equal grid_h*grid_w + num_special     */
  int32_t grid_h, grid_w;   /* patch grid, e.g. 37 x 37 for 518px / 14px    */
  int32_t num_special;      /* S >= 0, stored after the patches of a frame   */
  int32_t num_heads;        /* 1 <= H <= 64 (bf16) or 32 (fp32), else      *
                             * VGA_ERR_UNSUPPORTED                          */
  int32_t head_dim;         /* D; must be 64                                 */
  int32_t dtype;            /* vga_dtype of Q, K, V and O                    */
  float scale;              /* softmax scale; <= 0 selects 1/sqrt(head_dim)  */
} vga_frames;

/* Subsampled Global Attention parameters (AVGGT, section 3, step two).
 * Patch (r, c) of every frame is kept as a K/V column iff
 * r mod stride_h == phase_h and c mod stride_w == phase_w; the special
 * tokens are always kept.  A truncated window at the grid edge gets no extra
 * sample.  The kept-per-frame count is
 *   kpf = S + ceil((gh - phase_h) / stride_h) * ceil((gw - phase_w) / stride_w). */
typedef struct {
  int32_t stride_h, stride_w; /* 1..grid_h, 1..grid_w                        */
  int32_t phase_h, phase_w;   /* 0..stride-1; -1 selects (stride - 1) / 2    */
  int32_t diagonal;  /* 0/1: add the query's own (k_i, v_i) column iff its
                        token was dropped (never counted twice)             */
  int32_t mean_fill; /* 0: no mean column.  1 (count-weighted): one column
                        with key kmean and value vmean (means over all |D|
                        dropped tokens, per head) whose logit is
                        scale*<q,kmean> + ln|D|, i.e. it weighs as |D|
                        copies.  2 (unit weight): the same column with logit
                        scale*<q,kmean>.  Absent when |D| == 0.            */
} vga_sga;

typedef enum {
  VGA_MODE_FRAME = 0,
  VGA_MODE_GLOBAL = 1,
  VGA_MODE_SGA = 2,
  VGA_MODE_REGISTER = 3
} vga_mode;

typedef struct {
  int32_t mode;  /* vga_mode                                                 */
  vga_sga sga;   /* meaningful when mode == VGA_MODE_SGA (phases resolved)   */
} vga_layer;

/* Byte offsets of the SGA workspace sections (each 256-byte aligned) and
 * the selection sizes.  The workspace holds, after vga_sga_attn:
 *   keep_idx  int32 [num_kept]   kept token indices, ascending
 *   keep_mask uint8 [T]          1 iff the token is kept
 *   kmean     fp32  [H, 64]      mean key over the dropped tokens
 *   vmean     fp32  [H, 64]      mean value over the dropped tokens
 *   kc, vc    dtype [num_kept, H, 64]  the kept K and V rows, compacted
 *   partials  fp32  [partial_blocks, 2, H, 64]  per-block dropped sums   */
typedef struct {
  uint64_t keep_idx, keep_mask, kmean, vmean, kc, vc, partials;
  uint64_t total;           /* bytes the workspace must hold               */
  int64_t kept_per_frame;   /* kpf                                         */
  int64_t num_kept;         /* N * kpf                                     */
  int64_t num_dropped;      /* |D| = T - N * kpf                           */
  int64_t partial_blocks;   /* number of partial-sum blocks                */
} vga_sga_ws_layout;

/* Byte offsets of the register-attention workspace sections (each 256-byte
 * aligned): the special-token rows of Q, K, V and of the output, compacted
 * to [N*S, H, 64] in the element type, frame-major then special order. */
typedef struct {
  uint64_t qs, ks, vs, os;
  uint64_t total;           /* bytes the workspace must hold (0 when S == 0) */
  int64_t num_special_rows; /* N * S                                         */
} vga_register_ws_layout;

/* Frame attention ("VGGT CVPR25 Best Paper" notes, "Alternating-Attention";
 * AVGGT section 3, step one): for every frame f, head h and token i of f,
 *   O[i,h] = softmax_j(scale * <Q[i,h], K[j,h]>) V[j,h]
 * over the L tokens j of frame f (specials included).
 * Returns VGA_OK or an error status; nothing is enqueued on error. */
vga_status vga_frame_attn(const vga_frames* shape, const void* q, const void* k,
                          const void* v, void* o, void* stream);

/* Exact global attention (same section): as above with j over all T
 * tokens of all frames; the T x T matrix is never written to memory. */
vga_status vga_global_attn(const vga_frames* shape, const void* q, const void* k,
                           const void* v, void* o, void* stream);

/* Fills *out with the SGA workspace layout for (shape, sga) -- host only,
 * no device work.  Returns VGA_OK or the same validation errors as
 * vga_sga_attn. */
vga_status vga_sga_workspace_layout(const vga_frames* shape, const vga_sga* sga,
                                    vga_sga_ws_layout* out);

/* Subsampled Global Attention (AVGGT section 3, step two).  For every token
 * i and head h, one softmax over: the kept columns (keep_idx), the own column
 * (k_i, v_i) iff diagonal and token i was dropped, and the mean column iff
 * mean_fill and |D| > 0.  workspace: device buffer of at least
 * vga_sga_workspace_layout().total bytes, owned by the caller; its sections
 * are rewritten by every call. */
vga_status vga_sga_attn(const vga_frames* shape, const vga_sga* sga, const void* q,
                        const void* k, const void* v, void* o, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The key selection and compaction of SGA alone (AVGGT section 3, step two:
 * uniform grid sampling and the mean of the dropped columns): fills the
 * workspace sections keep_idx, keep_mask, kmean, vmean, kc and vc (and the
 * partials) exactly as vga_sga_attn does before its attention, from K and
 * V ([T, H, 64], 16-byte aligned); no output tensor.  Same workspace rules
 * and errors as vga_sga_attn (VGA_ERR_NULL for k or v, VGA_ERR_ALIAS when k
 * or v overlaps the workspace).  Reads K and V once: the HBM-bound step. */
vga_status vga_sga_select(const vga_frames* shape, const vga_sga* sga, const void* k,
                          const void* v, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Per-layer schedule of the training-free pipeline (AVGGT section 3):
 * slot g < num_early_to_frame becomes VGA_MODE_FRAME; the remaining slots
 * are VGA_MODE_SGA with *sga (phases resolved), or VGA_MODE_GLOBAL when sga
 * is NULL.  out: host array of num_global_layers entries.  Host only.
 * Errors: VGA_ERR_NULL (out NULL with num_global_layers > 0), VGA_ERR_PARAM
 * (counts out of range or bad SGA strides/phases/flags). */
vga_status vga_layer_schedule(int32_t num_global_layers, int32_t num_early_to_frame,
                              const vga_sga* sga, vga_layer* out);

/* Unit-weight mean-fill (vga_sga.mean_fill == 2) is accepted by every SGA
 * call above and below; it is the ablation of the count weighting, which
 * the AVGGT notes leave open. */

/* Register attention (VGGT-Omega notes, section 2, Register Attention):
 * a special-token query i (u >= gh*gw in its frame) attends over the
 * special tokens of every frame (N*S columns); a patch query attends over
 * the L tokens of its own frame, exactly as vga_frame_attn.  With S == 0 it
 * is frame attention.  workspace: device buffer of at least
 * vga_register_workspace_layout().total bytes (may be NULL when that is 0),
 * owned by the caller and rewritten by every call. */
vga_status vga_register_workspace_layout(const vga_frames* shape,
                                         vga_register_ws_layout* out);
vga_status vga_register_attn(const vga_frames* shape, const void* q, const void* k,
                             const void* v, void* o, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Schedule with register attention: as vga_layer_schedule, except that
 * among the slots g >= num_early_to_frame, those with
 * g mod register_every == register_every - 1 become VGA_MODE_REGISTER
 * (register_every = 4 replaces a quarter of the global layers, as in the
 * VGGT-Omega notes; 0 replaces none).  Errors as vga_layer_schedule, plus
 * VGA_ERR_PARAM for register_every < 0. */
vga_status vga_layer_schedule_register(int32_t num_global_layers,
                                       int32_t num_early_to_frame,
                                       int32_t register_every, const vga_sga* sga,
                                       vga_layer* out);

/* Schedule with per-slot SGA parameters (AVGGT section 3 names the stride
 * as the knob and leaves its per-layer choice open): slot
 * g < num_early_to_frame becomes VGA_MODE_FRAME; slot g >= num_early_to_frame
 * becomes VGA_MODE_SGA with per_slot_sga[g - num_early_to_frame] (phases
 * resolved), so that, e.g., later layers can sample more coarsely.
 * per_slot_sga: host array of num_global_layers - num_early_to_frame
 * entries (may be NULL when that is 0); out: host array of
 * num_global_layers entries.  Host only.  Errors: VGA_ERR_PARAM (counts out
 * of range, or any slot's strides/phases/flags), VGA_ERR_NULL; on error
 * nothing is written to out. */
vga_status vga_layer_schedule_sga(int32_t num_global_layers, int32_t num_early_to_frame,
                                  const vga_sga* per_slot_sga, vga_layer* out);

/* Row-range variants: the share of one device when the query rows are
 * split across devices (each device holds all of K and V and its own rows
 * of Q and O).  q_rows and o_rows hold rows [row_begin, row_end) of the
 * full [T, H, 64] Q and O (q_rows[r] is token row_begin + r); k and v are
 * the full [T, H, 64] tensors.  The result equals the same rows of the
 * full call.  0 <= row_begin <= row_end <= T; an empty range enqueues
 * nothing and reads no pointer (they may be NULL; the SGA variant still
 * validates its parameters).  vga_frame_attn_rows needs whole frames (row_begin and row_end
 * multiples of L), else VGA_ERR_SHAPE.  The SGA variant selects and
 * averages over all T tokens (its workspace is the full-call layout). */
vga_status vga_frame_attn_rows(const vga_frames* shape, int64_t row_begin, int64_t row_end,
                               const void* q_rows, const void* k, const void* v,
                               void* o_rows, void* stream);
vga_status vga_global_attn_rows(const vga_frames* shape, int64_t row_begin, int64_t row_end,
                                const void* q_rows, const void* k, const void* v,
                                void* o_rows, void* stream);
vga_status vga_sga_attn_rows(const vga_frames* shape, const vga_sga* sga, int64_t row_begin,
                             int64_t row_end, const void* q_rows, const void* k,
                             const void* v, void* o_rows, void* workspace,
                             size_t workspace_bytes, void* stream);

/* vga_sga_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and the same
 * result as vga_sga_attn, with the workspace in a static device array of
 * the library, VGA_SGA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which each
 * GPU that runs the call holds from its first call until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); its first call on a device takes the array's device address
 * (hipGetSymbolAddress, with that device current) and keeps it.  The
 * device is the one that runs `stream` (the current device for NULL).
 * Every section of the workspace is written by the call before it is read,
 * so nothing carries over between calls, but all calls on one GPU share
 * the array: calls that overlap in time on one GPU (other streams, other
 * threads) race and must not be issued.  Arguments as vga_sga_attn.
 * Errors: as vga_sga_attn; VGA_ERR_WORKSPACE (checked before any device
 * call) when the layout of vga_sga_workspace_layout needs more than the
 * scratch holds (at 16 heads of bf16: about 44 frames of 37x37+5 tokens at
 * stride 2x2, 109 at 3x3). */
#define VGA_SGA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
vga_status vga_sga_attn_noalloc(const vga_frames* shape, const vga_sga* sga, const void* q,
                                const void* k, const void* v, void* o, void* stream);

/* The projections around an attention layer ("VGGT CVPR25 Best Paper"
 * notes, section "Alternating-Attention": the frame and global blocks are
 * self-attention layers over the tokens).  The pages leave the projections
 * open; they are taken as plain nn.Linear-style layers,
 *   y[t][n] = sum_c x[t][c] * w[n][c] + b[n],
 * with C = 64 * num_heads input features per token, all arrays of the
 * shape's dtype (fp32 or bf16; accumulation in fp32).  No positional
 * encoding is applied (the pages do not specify VGGT's).
 *
 * vga_qkv_proj: x [T, C] token features; w_qkv [3C, C] row-major (row n is
 * output feature n); b_qkv [3C] or NULL for no bias.  Output features
 * [0, C), [C, 2C) and [2C, 3C) are written to q, k and v, each [T, H, 64]
 * (feature 64*h + e is head h, dim e) -- the layout the attention calls take.
 *
 * vga_out_proj: o [T, H, 64] (an attention output, read as [T, C]);
 * w_o [C, C]; b_o [C] or NULL; y [T, C].
 *
 * x, w, q, k, v, o and y must be 16-byte aligned and the bias aligned to
 * its element size; the outputs must not overlap an input or each other.
 * Errors: VGA_ERR_NULL, VGA_ERR_SHAPE, VGA_ERR_DTYPE, VGA_ERR_ALIGN,
 * VGA_ERR_ALIAS, VGA_ERR_UNSUPPORTED (shape checks), VGA_ERR_HIP. */
vga_status vga_qkv_proj(const vga_frames* shape, const void* x, const void* w_qkv,
                        const void* b_qkv, void* q, void* k, void* v, void* stream);
vga_status vga_out_proj(const vga_frames* shape, const void* o, const void* w_o,
                        const void* b_o, void* y, void* stream);

const char* vga_status_string(vga_status status);
const char* vga_last_error(void); /* thread-local detail of the last failure */
int32_t vga_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VGA_H */
