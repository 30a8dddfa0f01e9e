/*
 * libvggtattn -- one VGGT Aggregator attention block per call, on an AMD
 * Instinct MI355X (gfx950).
 *
 * What a call computes (sources are the web pages this library is built from):
 *   - Token recipe, "VGGT-Omega Aggregator explainer" (ksqn.cn), section 二:
 *     every frame is [1 camera token][16 register tokens][grid_h*grid_w patch
 *     tokens], so T = 17 + grid_h*grid_w; patches are in row-major grid order.
 *   - Per attention set: [q|k|v] = x Wqkv^T (no bias); q and k are
 *     LayerNorm-ed over the Dh features of each head (biased variance, eps =
 *     ln_eps) with a per-head affine (gamma, beta) -- the page's "use_qk_norm"
 *     (section 三); then patch tokens get a 2D rotary encoding (section 三, and
 *     the HTTM article, section 04, RoPE-effect paragraph): the first Dh/2 features
 *     turn with the grid row + pos_offset, the last Dh/2 with the grid column
 *     + pos_offset; feature i of a half pairs with feature i + Dh/4 and turns
 *     by pos * rope_base^(-i/(Dh/4)).  Camera and register tokens are not
 *     rotated, and nothing encodes the frame index.  Then, per head,
 *     softmax(q k^T / sqrt(Dh)) v, heads concatenated, times Wo^T.  No bias,
 *     no residual, no LayerScale: Y is the raw attention-branch output.
 *   - vggt_attn_frame: one set per frame (the frame block, section 三).
 *   - vggt_attn_global: all S*T tokens in one set (global mode, section 三;
 *     the dominant cost per the HTTM article section 02 and the AVGGT summary).
 *   - vggt_attn_global_register: only the 17 special tokens of every frame, as
 *     one set of 17*S tokens (register mode, section 三); patch rows of Y are
 *     a copy of X (patch tokens keep to their own frame in this block).
 *   - vggt_attn_global_subsampled: global mode with AVGGT's subsampled keys and
 *     values (see its declaration).
 *   - vggt_attn_global_rows: a window of query rows of the global mode (one
 *     GPU's share of a query-row split; see its declaration).
 *
 * Conventions for every entry point below:
 *   - Tensor pointers are DEVICE pointers on the current HIP device; dense,
 *     row-major, no strides.  X, Y: bf16 [S][T][d].  Wqkv: bf16 [3d][d], rows
 *     = [Q heads 0..H-1; K heads; V heads], Dh rows per head.  Wo: bf16 [d][d]
 *     (Y = O Wo^T).  q_gamma, q_beta, k_gamma, k_beta: fp32 [H][Dh] (replicate
 *     one row H times for an affine shared across heads).
 *   - X, Y, Wqkv, Wo must be 16-byte aligned, gamma/beta 4-byte aligned, the
 *     workspace 256-byte aligned.
 *   - v1 limits: Dh = d/H must be 64, d a multiple of 128, S >= 1, grid_h,
 *     grid_w >= 0, T = 17 + grid_h*grid_w, S*T < 2^31 tokens, and at most
 *     2^28 key / value rows per head in the workspace (the tokens, each set
 *     padded to 64 and the total to a multiple of 2,048 when that adds at
 *     most 1/64 of the rows, else of 256 -- frame sets: query / key rows
 *     padded to 16 per frame, value columns to 64 per frame; or the kept,
 *     merged or descriptor keys padded to 256): ESHAPE beyond, and
 *     vggt_attn_workspace_bytes reports 0.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it and the call returns without synchronising; kernel
 *     faults surface at the caller's next synchronisation.
 *   - Ownership: the caller owns every buffer, including the workspace of at
 *     least vggt_attn_workspace_bytes() bytes.  The library allocates and frees
 *     nothing and keeps no pointer after the call returns (beyond the work it
 *     enqueued).  It holds no mutable global state and is re-entrant; calls
 *     that share a workspace must be ordered on one stream.
 *   - Aliasing: Y must not overlap X, the weights, gamma/beta or the
 *     workspace, with one exception: vggt_attn_global_register accepts Y == X
 *     (in place), and then writes only the 17*S special rows.
 *   - Errors: every argument is checked before anything is enqueued; on a
 *     nonzero return nothing was launched and Y is untouched.  Value ranges
 *     are checked on the device, without a host synchronisation: the call's
 *     first stage writes VGGT_ATTN_RANGE_* bits into the workspace's status
 *     word when an input holds a non-finite value, when a QK-norm affine
 *     could overflow fp16 q / k, or when a bound is beyond what the call's
 *     power-of-two pre-scales bring into fp16 range (the cases in which Y
 *     may hold inf or NaN).  The kernels still run; read the word with
 *     vggt_attn_range_status() after the call, which reports ERANGE.
 */
#ifndef LIBVGGTATTN_H
#define LIBVGGTATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define VGGT_ATTN_OK          0
#define VGGT_ATTN_EINVAL     (-1) /* null pointer, unknown mode/stage, forbidden aliasing */
#define VGGT_ATTN_ESHAPE     (-2) /* shape outside the supported set (see above) */
#define VGGT_ATTN_EALIGN     (-3) /* pointer misaligned */
#define VGGT_ATTN_EWORKSPACE (-4) /* workspace smaller than vggt_attn_workspace_bytes() */
#define VGGT_ATTN_EHIP       (-5) /* the HIP runtime rejected a launch */
#define VGGT_ATTN_ERANGE     (-6) /* rope_base / ln_eps not finite and positive, pos_offset out of
                                     range, subsampling window < 1, row window outside the set,
                                     descriptor count outside the cache; from
                                     vggt_attn_range_status: a value range bit is set */
#define VGGT_ATTN_ESCRATCH   (-7) /* vggt_attn_block_noalloc: the call needs more workspace than
                                     VGGT_ATTN_STATIC_SCRATCH_BYTES */

/* Value range bits, found on the device by a call's first stage and kept in
   the 32-bit status word at byte VGGT_ATTN_STATUS_OFFSET of its workspace. */
#define VGGT_ATTN_STATUS_OFFSET 16
#define VGGT_ATTN_RANGE_X      1u  /* an X row (or appended descriptor) holds a non-finite
                                      value, or its squared norm overflows fp32 */
#define VGGT_ATTN_RANGE_WQKV   2u  /* Wqkv holds a non-finite value */
#define VGGT_ATTN_RANGE_WO     4u  /* Wo holds a non-finite value */
#define VGGT_ATTN_RANGE_AFFINE 8u  /* a q / k gamma or beta is non-finite, or 8|gamma| + |beta|
                                      >= 2^15 (a LayerNorm-ed q / k could leave fp16) */
#define VGGT_ATTN_RANGE_SCALE 16u  /* max||x|| max||w_v|| or max|Wo| needs a power-of-two
                                      scale beyond 2^+-60 to reach fp16 range, or the output
                                      bound d max||x|| max||w_v|| max|Wo| reaches 3e38 */

/* Block modes. */
#define VGGT_ATTN_MODE_FRAME    0
#define VGGT_ATTN_MODE_GLOBAL   1
#define VGGT_ATTN_MODE_REGISTER 2
#define VGGT_ATTN_MODE_SUBSAMPLED 3 /* global mode, AVGGT subsampled keys / values */
#define VGGT_ATTN_MODE_DESCRIPTOR 4 /* every token attends to a descriptor key / value cache */
#define VGGT_ATTN_MODE_MERGED     5 /* global mode, HTTM head-wise temporal token merging */

/* Stages of one call, in order (see vggt_attn_stage). */
#define VGGT_ATTN_STAGE_PREP 0 /* range bounds, RoPE table, fp16 copy of Wo */
#define VGGT_ATTN_STAGE_QKV  1 /* QKV projection + per-head QK LayerNorm + 2D RoPE */
#define VGGT_ATTN_STAGE_CORE 2 /* softmax(q k^T / sqrt(Dh)) v for every set and head */
#define VGGT_ATTN_STAGE_OUT  3 /* output projection (+ register-mode patch copy) */
#define VGGT_ATTN_STAGE_ALL  (-1) /* all four (vggt_attn_bf16ops) */

typedef struct vggt_attn_shape {
  int32_t S;          /* frames */
  int32_t T;          /* tokens per frame = 17 + grid_h*grid_w */
  int32_t d;          /* model width */
  int32_t H;          /* heads; Dh = d/H */
  int32_t grid_h;     /* patch grid rows (26 for a 416-pixel-high image at 16 px) */
  int32_t grid_w;     /* patch grid columns (39 for 624 px) */
  float rope_base;    /* RoPE frequency base, e.g. 100 */
  float ln_eps;       /* QK LayerNorm epsilon, e.g. 1e-5 */
  int32_t pos_offset; /* patch (r, c) sits at position (r + off, c + off); 0..65535 */
} vggt_attn_shape;

/* Bytes of device workspace a call in `mode` needs for `shape`; 0 if the
   mode or shape is not supported.  Pure host arithmetic, no HIP call.  For
   VGGT_ATTN_MODE_SUBSAMPLED the size covers every subsampling window. */
size_t vggt_attn_workspace_bytes(int mode, const vggt_attn_shape* shape);

/* Frame block: attention inside each frame (S sets of T tokens). */
int vggt_attn_frame(const vggt_attn_shape* shape, const void* X, const void* Wqkv,
                    const void* Wo, const float* q_gamma, const float* q_beta,
                    const float* k_gamma, const float* k_beta, void* Y,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Global mode: all S*T tokens form one set. */
int vggt_attn_global(const vggt_attn_shape* shape, const void* X, const void* Wqkv,
                     const void* Wo, const float* q_gamma, const float* q_beta,
                     const float* k_gamma, const float* k_beta, void* Y,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Register mode: tokens 0..16 of every frame form one set of 17*S tokens;
   patch rows of Y are copied from X (nothing is written there when Y == X). */
int vggt_attn_global_register(const vggt_attn_shape* shape, const void* X,
                              const void* Wqkv, const void* Wo, const float* q_gamma,
                              const float* q_beta, const float* k_gamma,
                              const float* k_beta, void* Y, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Global mode with AVGGT subsampled global attention ("AVGGT: Rethinking
   Global Attention for Accelerating VGGT", gist.science summary, technical
   summary section 2B).  Every token stays a query, but the keys / values are
   only (a) the 17 special tokens of every frame and (b) one patch per
   sub_h x sub_w window of the patch grid -- patch (r, c) with r % sub_h == 0
   and c % sub_w == 0 (the window's top-left cell; windows cut by the grid edge
   keep theirs) -- plus (c) each query's own key / value (the diagonal), and
   (d) one mean key / value pair, the mean over the discarded tokens of the
   normalised, rotated keys and of the values, which stands in for every
   discarded column of the query's row: it enters the softmax with
   multiplicity n_i = (discarded tokens) - [query i itself is discarded].
   sub_h = sub_w = 1 is exact global attention.  sub_h, sub_w >= 1 (else
   VGGT_ATTN_ERANGE).  Workspace: vggt_attn_workspace_bytes(VGGT_ATTN_MODE_SUBSAMPLED). */
int vggt_attn_global_subsampled(const vggt_attn_shape* shape, int32_t sub_h, int32_t sub_w,
                                const void* X, const void* Wqkv, const void* Wo,
                                const float* q_gamma, const float* q_beta,
                                const float* k_gamma, const float* k_beta, void* Y,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Global mode with HTTM head-wise temporal token merging ("HTTM: Head-wise
   Temporal Token Merging for Faster VGGT", 10100.com, sections 02, 04, 05):
   merging shortens the query, key and value sequences, every head merging on
   its own, inside spatio-temporal blocks.  The page names the parts, not the
   rule; this call's reading:
     - blocks: frames in consecutive runs of `frames` (the last run may be
       shorter) x the patch grid in windows of win_h x win_w cells (row-major,
       cut by the grid edge); the 17 special tokens of every frame never merge;
     - per head and block: destinations = the run's first frame's patches,
       sources = the other frames' patches (frame by frame, row-major); a
       source's similarity to a destination is the dot product of their
       normalised, rotated keys in that head (fp16 keys, fp32 sum in feature
       order); each source takes its most similar destination (ties: the
       first), and the r sources of highest similarity (ties: the first)
       merge into theirs;
     - a merged token's query, key and value are its members' means; in the
       softmax a merged key counts n times (weight n exp(logit), n = members);
       every token takes its merged token's output, per head; heads
       concatenated, times Wo^T.
   r = 0 is the global block (up to the fp32 summation order).  Requires
   frames, win_h, win_w >= 1, r >= 0 and min(frames, S) * min(win_h, grid_h) *
   grid_w <= 400 (else VGGT_ATTN_ERANGE).  Workspace:
   vggt_attn_workspace_bytes(VGGT_ATTN_MODE_MERGED) (covers every parameter
   choice). */
int vggt_attn_global_merged(const vggt_attn_shape* shape, int32_t frames, int32_t win_h,
                            int32_t win_w, int32_t r, const void* X, const void* Wqkv,
                            const void* Wo, const float* q_gamma, const float* q_beta,
                            const float* k_gamma, const float* k_beta, void* Y, void* workspace,
                            size_t workspace_bytes, void* stream);

/* One stage of vggt_attn_global_merged, as vggt_attn_stage (the CORE stage
   merges, attends and unmerges). */
int vggt_attn_merged_stage(int stage, const vggt_attn_shape* shape, int32_t frames, int32_t win_h,
                           int32_t win_w, int32_t r, const void* X, const void* Wqkv,
                           const void* Wo, const float* q_gamma, const float* q_beta,
                           const float* k_gamma, const float* k_beta, void* Y, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Rows [row_begin, row_begin + row_count) of the global block's output: the
   queries of those tokens (flat index s*T + t) attend to every token of the
   set, exactly as in vggt_attn_global.  This is one GPU's share when the
   global set is split across GPUs by query rows ("HTTM" article, section 02,
   and the AVGGT summary, technical summary 1: the global set is one long
   sequence whose keys every query needs); on one GPU it computes keys and
   values for all tokens and queries, attention and the output projection for
   the window only.  Y_rows is bf16 [row_count][d] (row i = token
   row_begin + i).  Requires 0 <= row_begin, 1 <= row_count,
   row_begin + row_count <= S*T (else VGGT_ATTN_ERANGE).  Workspace:
   vggt_attn_workspace_bytes(VGGT_ATTN_MODE_GLOBAL).  The rows equal those
   vggt_attn_global writes for them up to the fp32 summation order of the
   query blocks that either call runs as split key ranges (the partly filled
   last round of workgroups on the device); with the split off (tuning build,
   VGGT_ATTN_SPLIT=1) they are bitwise equal. */
int vggt_attn_global_rows(const vggt_attn_shape* shape, int64_t row_begin, int64_t row_count,
                          const void* X, const void* Wqkv, const void* Wo, const float* q_gamma,
                          const float* q_beta, const float* k_gamma, const float* k_beta,
                          void* Y_rows, void* workspace, size_t workspace_bytes, void* stream);

/* One stage of a call in `mode` (VGGT_ATTN_STAGE_*), same arguments and
   checks as the full call.  Running the four stages in order on one stream
   with one workspace is exactly the full call; a stage reads what the
   previous stages left in the workspace.  Meant for timing and profiling
   the kernels one by one. */
int vggt_attn_stage(int mode, int stage, const vggt_attn_shape* shape, const void* X,
                    const void* Wqkv, const void* Wo, const float* q_gamma,
                    const float* q_beta, const float* k_gamma, const float* k_beta,
                    void* Y, void* workspace, size_t workspace_bytes, void* stream);

/* The frame, global and register blocks with bf16 attention operands: the
   computation of vggt_attn_frame / vggt_attn_global /
   vggt_attn_global_register, but q, k and v are stored in bf16, the
   probabilities and O are rounded to bf16, and the output projection reads O
   and Wo (times the same exact power of two) in bf16 -- bf16 x bf16 MFMA with
   fp32 accumulation throughout, the precision the HTTM article (10100.com,
   section 05) runs its attention in.  The default calls keep these operands
   in fp16 (11-bit significands against bf16's 8): with bf16 operands the
   error of Y against the exact block is about 2.5x larger (relative L1 near
   4e-3 instead of 1.5e-3).  mode: VGGT_ATTN_MODE_FRAME, _GLOBAL or _REGISTER
   (else VGGT_ATTN_EINVAL); stage: one VGGT_ATTN_STAGE_* or
   VGGT_ATTN_STAGE_ALL for the whole call.  Workspace, checks and status as
   the mode's default call. */
int vggt_attn_bf16ops(int mode, int stage, const vggt_attn_shape* shape, const void* X,
                      const void* Wqkv, const void* Wo, const float* q_gamma,
                      const float* q_beta, const float* k_gamma, const float* k_beta,
                      void* Y, void* workspace, size_t workspace_bytes, void* stream);

/* One stage of vggt_attn_global_subsampled, as vggt_attn_stage. */
int vggt_attn_subsampled_stage(int stage, const vggt_attn_shape* shape, int32_t sub_h,
                               int32_t sub_w, const void* X, const void* Wqkv, const void* Wo,
                               const float* q_gamma, const float* q_beta, const float* k_gamma,
                               const float* k_beta, void* Y, void* workspace,
                               size_t workspace_bytes, void* stream);

/* One stage of vggt_attn_global_rows, as vggt_attn_stage. */
int vggt_attn_global_rows_stage(int stage, const vggt_attn_shape* shape, int64_t row_begin,
                                int64_t row_count, const void* X, const void* Wqkv,
                                const void* Wo, const float* q_gamma, const float* q_beta,
                                const float* k_gamma, const float* k_beta, void* Y_rows,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
   Descriptor attention ("FlashVGGT: Efficient and Scalable Visual Geometry
   Transformers with Compressed Descriptor Attention", chatpaper.ai, abstract):
   the global step is cross-attention from every image token to a compact set
   of descriptor tokens, and long sequences run chunk by chunk, reusing the
   cached descriptors of earlier chunks.  How descriptors are made is not
   described there: they are the caller's tokens (bf16 [m][d], the model's
   token width).  Their keys and values go through the layer's Wqkv (K and V
   rows) and the key LayerNorm (k_gamma, k_beta); they have no place on the
   patch grid and are not rotated.  The keys / values live in a caller-owned
   device cache that grows by appends; the caller keeps the fill count.
   One cache belongs to one layer: every append must pass the same Wqkv,
   k_gamma and k_beta.
   --------------------------------------------------------------------------- */

/* Bytes of a descriptor cache for `capacity` descriptors (1 <= capacity <
   2^31) at the shape's H; 0 if unsupported.  Host arithmetic only. */
size_t vggt_attn_desc_cache_bytes(const vggt_attn_shape* shape, int64_t capacity);

/* Makes `cache` (256-byte aligned, >= vggt_attn_desc_cache_bytes bytes) an
   empty cache: every stored key / value zero, no bounds yet.  Required once
   before the first append. */
int vggt_attn_desc_cache_init(const vggt_attn_shape* shape, int64_t capacity, void* cache,
                              size_t cache_bytes, void* stream);

/* Appends the m descriptor tokens D (bf16 [m][d], 16-byte aligned) at
   positions count .. count + m - 1 of the cache (count = descriptors already
   appended; 0 <= count, 1 <= m, count + m <= capacity, else
   VGGT_ATTN_ERANGE).  The stored values carry one power-of-two scale for the
   whole cache, chosen from the largest descriptor norm seen so far; when an
   append raises that bound, the values already stored are rescaled (exactly,
   by a power of two) before the new ones are written.  D must not overlap the
   cache. */
int vggt_attn_desc_append(const vggt_attn_shape* shape, int64_t capacity, int64_t count,
                          const void* D, int64_t m, const void* Wqkv, const float* k_gamma,
                          const float* k_beta, void* cache, size_t cache_bytes, void* stream);

/* Y = softmax(q k^T / sqrt(Dh)) v Wo^T per head, heads concatenated, for
   every token of X (bf16 [S][T][d]): q from X exactly as in the global block
   (LayerNorm with q_gamma / q_beta, 2D RoPE on patch tokens), keys / values
   the first `count` cached descriptors (1 <= count <= capacity).
   Workspace: vggt_attn_workspace_bytes(VGGT_ATTN_MODE_DESCRIPTOR).  Y must
   not overlap X, the weights, the cache or the workspace; the cache is only
   read. */
int vggt_attn_desc_attend(const vggt_attn_shape* shape, int64_t capacity, int64_t count,
                          const void* cache, size_t cache_bytes, const void* X, const void* Wqkv,
                          const void* Wo, const float* q_gamma, const float* q_beta, void* Y,
                          void* workspace, size_t workspace_bytes, void* stream);

/* One stage of vggt_attn_desc_attend, as vggt_attn_stage. */
int vggt_attn_desc_attend_stage(int stage, const vggt_attn_shape* shape, int64_t capacity,
                                int64_t count, const void* cache, size_t cache_bytes,
                                const void* X, const void* Wqkv, const void* Wo,
                                const float* q_gamma, const float* q_beta, void* Y,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
   Layer schedule.  "VGGT-Omega Aggregator explainer", section 三: the
   Aggregator is 24 layers deep and every layer runs a frame block and then an
   inter-frame block, each a residual branch scaled by LayerScale; the
   inter-frame block is in register mode at layers [2, 6, 9, 14, 20] (read as
   0-based layer indices, global mode at the others); section 四: the token
   states after the frame block and after the inter-frame block of layers 4,
   11, 17, 23 are kept, concatenated along channels (2d features).  AVGGT
   summary, technical summary 2B: early global layers may run as frame
   attention, the remaining ones as subsampled global attention.
   --------------------------------------------------------------------------- */

/* Residual update: for rows r with r % period < active,
   Z[r][c] = X[r][c] + gamma[c] * Y[r][c] (fp32 fused multiply-add of the bf16
   inputs, rounded once to bf16); other rows Z = X (register layers pass
   period = T, active = 17, so patch rows keep their state).  X, Y, Z: bf16
   [rows][d]; gamma: fp32 [d] (the LayerScale vector); all device pointers,
   16-byte aligned, d % 8 == 0.  Z may be X (in place) but must not overlap Y
   or gamma.  If C is not NULL, Z is also written to C + r * c_stride (bf16
   elements; c_stride >= d, a multiple of 8), e.g. one half of a [rows][2d]
   cache; C must not overlap the other buffers.  Errors: EINVAL (null X / Y /
   Z / gamma, overlap), ESHAPE (rows < 0, d, period < 1, active < 0,
   c_stride), EALIGN; nothing is launched on error. */
int vggt_attn_residual(const void* X, const void* Y, void* Z, int64_t rows, int32_t d,
                       const float* gamma, int32_t period, int32_t active, void* C,
                       int64_t c_stride, void* stream);

/* Weights of one block of the schedule (device pointers, layouts as for the
   block calls above). */
typedef struct vggt_attn_block_weights {
  const void* Wqkv;          /* bf16 [3d][d] */
  const void* Wo;            /* bf16 [d][d] */
  const float* q_gamma;      /* fp32 [H][Dh] */
  const float* q_beta;
  const float* k_gamma;
  const float* k_beta;
  const float* layer_scale;  /* fp32 [d], 16-byte aligned: LayerScale of the residual branch */
} vggt_attn_block_weights;

typedef struct vggt_attn_schedule {
  int32_t n_layers;          /* 1..64 (24 in the model) */
  int32_t early_frame;       /* inter-frame blocks of layers l < early_frame that are not
                                register layers run as frame blocks (AVGGT); 0: none */
  uint64_t register_layers;  /* bit l: layer l's inter-frame block is in register mode */
  uint64_t cached_layers;    /* bit l: layer l's two states are kept */
  int32_t sub_h, sub_w;      /* 1, 1: the remaining inter-frame blocks are global; else they
                                are subsampled global blocks with these windows */
  int32_t merge_frames;      /* 0: off; else the remaining inter-frame blocks (not register,
                                not early frame) are global blocks with HTTM merging,
                                vggt_attn_global_merged(merge_frames, merge_win_h,
                                merge_win_w, merge_r) (HTTM article, 10100.com, section
                                02: merging serves the global attention layers); not
                                together with subsampling */
  int32_t merge_win_h, merge_win_w, merge_r;
} vggt_attn_schedule;

/* Workspace of vggt_attn_schedule_run: the block output buffer plus the
   largest block workspace the schedule uses; 0 if the shape or the schedule
   is not supported. */
size_t vggt_attn_schedule_workspace_bytes(const vggt_attn_shape* shape,
                                          const vggt_attn_schedule* sched);

/* The attention part of the Aggregator's forward pass.  With x = X:
     for l in 0 .. n_layers-1:
       a = x + ls_f * frame_l(x)                    (all rows)
       x = a + ls_i * inter_l(a)                    (register mode: the 17 special
                                                      rows of every frame only)
       if bit l of cached_layers: cache[k] = [a | x], k counting cached layers
   where frame_l / inter_l are the block calls above with the weights
   blocks[2l] / blocks[2l+1] (a HOST array of 2 * n_layers entries holding
   device pointers), ls_f / ls_i their layer_scale vectors, and every block
   output and state is bf16.  state receives the final x (bf16 [S][T][d]; it
   may be X itself, else it must not overlap X).  caches: NULL (nothing kept)
   or bf16 [popcount(cached_layers)][S][T][2d], channels [0, d) the state after
   the frame block, [d, 2d) the state after the inter-frame block.  Masks with
   bits at or above n_layers, early_frame outside 0..n_layers, windows < 1,
   merging with subsampling or merge parameters out of range give
   VGGT_ATTN_ERANGE; every block and residual call is checked before the
   first launch, so on any error nothing is enqueued. */
int vggt_attn_schedule_run(const vggt_attn_shape* shape, const vggt_attn_schedule* sched,
                           const vggt_attn_block_weights* blocks, const void* X, void* state,
                           void* caches, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
   For callers that cannot allocate device memory -- code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc: the block
   call of `mode` (VGGT_ATTN_MODE_FRAME, _GLOBAL or _REGISTER; anything else
   is EINVAL) with the same arguments as vggt_attn_frame / _global /
   _global_register minus the workspace, which is instead a static device
   array of the library, VGGT_ATTN_STATIC_SCRATCH_BYTES bytes on every device
   the library runs on, held until the process ends.  The call allocates
   nothing (no hipMalloc, no allocating library routine) and computes exactly
   what the block call of that mode computes with a workspace of its own.
   Calls whose workspace need (vggt_attn_workspace_bytes) exceeds the array
   return VGGT_ATTN_ESCRATCH before anything is enqueued (e.g. 128 MiB holds
   register mode up to 587 frames, frame mode up to 20 and global mode up to
   9 frames of 26 x 39 patches at d = 1024).  All other checks and status codes are the
   block call's.  Every call on a device shares that device's array: calls
   that overlap in time on one device (different streams, or several host
   threads) race; order them on one stream.  Nothing needs clearing between
   calls.  The first call on a device looks the array's address up (one HIP
   symbol query, no allocation). */
#define VGGT_ATTN_STATIC_SCRATCH_BYTES (128u << 20)
int vggt_attn_block_noalloc(int mode, const vggt_attn_shape* shape, const void* X,
                            const void* Wqkv, const void* Wo, const float* q_gamma,
                            const float* q_beta, const float* k_gamma, const float* k_beta,
                            void* Y, void* stream);

/* Value range check of the last call that used `workspace` (any block call
   or stage sequence above, including descriptor attention, or a whole
   vggt_attn_schedule_run, whose blocks OR their bits together).  The call's
   first stage wrote the VGGT_ATTN_RANGE_* bits into the status word at byte
   VGGT_ATTN_STATUS_OFFSET of the workspace without any host
   synchronisation.  This function enqueues a 4-byte device-to-host copy of
   that word on `stream` (the call's stream), waits for the stream, stores the
   bits in *bits (when bits is not NULL) and returns VGGT_ATTN_OK if none is
   set, VGGT_ATTN_ERANGE if any is.  EINVAL for a null or misaligned
   workspace, EHIP if the copy fails.  It synchronises, so it does not belong
   inside a graph capture; a caller can instead copy the word itself. */
int vggt_attn_range_status(const void* workspace, uint32_t* bits, void* stream);

/* Static, human-readable text for a status code. */
const char* vggt_attn_status_str(int status);

/* Library version, major*10000 + minor*100 + patch. */
int vggt_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBVGGTATTN_H */
