/*
 * pv_tower.h -- C ABI of the MI355X (gfx950) Pixtral-class vision tower.
 *
 * The tower maps normalised pixels of one or more images to merged image
 * embeddings:
 *
 *   conv patch embedding -> RMS pre-norm -> L blocks of
 *   [RMSNorm -> q,k,v -> 2-D rotary -> block-diagonal attention -> out-proj
 *    + residual -> RMSNorm -> gated-SiLU MLP + residual]
 *   -> 2x2 patch merge + bias-free projection to the text width
 *      (or, without merge, one output row per patch).
 *
 * Sources: "Mistral 3" (KerasFormers model page) -- Mistral3VisionModel
 * (patch embedding, RMS pre-norm, 2-D rotary blocks over a packed
 * variable-resolution patch sequence), Mistral3Model argument table (vision
 * width 1024, MLP 4096, depth 24, heads 16, patch 14, rotary base 1e4,
 * spatial_merge_size 2, projector without bias, text width 5120), "Several
 * images in one conversation" (each image keeps its own patch count);
 * "Pixtral-12B-2409" (inference-research record), part (1) Vision and
 * VISION TOKENS (patch 16, no merge, 1024x1024 tiles); NeMo Automodel
 * "mistral3_vlm" API page, forward() (float pixel values plus image sizes).
 *
 * Conventions for every entry point:
 *  - Every function returns a pv_status.  No C++ exception crosses this ABI.
 *    On failure, pv_last_error() returns a thread-local message.
 *  - Argument, shape and capacity checks happen on the host before anything
 *    is enqueued, so they need no GPU.
 *  - "device" pointers are HIP device memory; "host" pointers are ordinary
 *    host memory.  All buffers are owned by the caller; the library keeps
 *    borrowed weight pointers (they must outlive the tower).
 *  - Work is enqueued on the caller's hipStream_t (passed as void*; NULL is
 *    the null stream) and the call returns without synchronising.  Device
 *    faults surface at the caller's next synchronisation.  One tower object
 *    must not be used by two streams (or threads) at once.
 *  - A forward call uploads its per-call plan (image metadata, attention work
 *    list, rotary table) from a ring of up to 8 pinned host staging buffers
 *    owned by the tower.  A call whose upload equals the bytes a slot already
 *    holds copies from that slot without rewriting it; otherwise it takes a
 *    slot whose last copy has completed (or adds one).  The host therefore
 *    never waits for the GPU, except when 8 distinct uploads are still in
 *    flight: then it waits for the oldest copy (not for kernels).
 */
#ifndef PV_TOWER_H
#define PV_TOWER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pv_status {
  PV_OK = 0,
  PV_ERR_ARG = -1,         /* null pointer, n_images < 1, bad config value   */
  PV_ERR_SHAPE = -2,       /* H or W <= 0, off the patch*merge grid, > max_side */
  PV_ERR_CAPACITY = -3,    /* output rows or workspace bytes too small        */
  PV_ERR_HIP = -4,         /* a HIP runtime or launch error (message kept)    */
  PV_ERR_UNSUPPORTED = -5  /* valid but not implemented (e.g. head_dim != 64) */
} pv_status;

typedef enum pv_dtype {
  PV_BF16 = 0, /* bf16 matrices and activations, fp32 accumulation and residual */
  PV_F32 = 1   /* fp32 everywhere */
} pv_dtype;

/* Tower hyper-parameters.  head_dim = hidden / heads must be 64. */
typedef struct pv_config {
  int32_t patch;      /* patch edge in pixels (14 for Mistral 3, 16 for Pixtral-12B) */
  int32_t hidden;     /* D, a multiple of 256 (1024) */
  int32_t heads;      /* attention heads (16) */
  int32_t mlp;        /* F, MLP width, a multiple of 256, at most 2^20 (4096) */
  int32_t layers;     /* number of blocks L >= 0 (24) */
  int32_t merge;      /* 2 = 2x2 patch merge + projection, 1 = no merge */
  int32_t out_dim;    /* projection width when merge == 2 (5120), a multiple of 128 */
  int32_t max_side;   /* largest accepted H or W in pixels (e.g. 1540 or 1024) */
  double rope_theta;  /* rotary base (1e4) */
  double rms_eps;     /* RMSNorm epsilon (1e-5) */
  int32_t dtype;      /* pv_dtype of the weights and activations */
  int32_t out_dtype;  /* pv_dtype of the output buffer for the bf16 tower: PV_BF16
                         (default) or PV_F32 (keeps the result unrounded); the
                         fp32 tower always writes fp32 */
  int32_t flags;      /* PV_FLAG_* bits, 0 by default */
} pv_config;

/* pv_config.flags: the bf16 attention normally runs a softmax whose per-query
 * offset is fixed from the first key tile and falls back to an online softmax
 * with a running max only if the sums overflow or underflow; this bit makes it
 * always take the online form (testing and diagnosis). */
#define PV_FLAG_ATTN_ONLINE_MAX 1
/* pv_config.flags, bf16 tower only: the four linear maps of every block
 * (q/k/v, out-projection, gate/up, down) run as fp8 e4m3 products with one
 * power-of-two (E8M0) scale per 32 k on both operands
 * (v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation): the weights are
 * quantised once by pv_tower_prepare (else per layer into the workspace of
 * every call), the activations by the norm
 * kernels and by quantisation passes over the attention output and
 * silu(gate) * up.  Scale X = floor(log2(block max)) - 7, values rounded to
 * nearest even.  The patch embedding, attention, the residual stream and the
 * merger keep their bf16/fp32 arithmetic.  An fp8 variant of the tower
 * (the NeMo Automodel page registers FP8-native Mistral 3 VLM checkpoints);
 * its accuracy is that of e4m3, not the bf16 tower's. */
#define PV_FLAG_FP8 2
/* pv_config.flags, bf16 tower with merge == 2 only: a deeper projector in
 * place of the single bias-free merge projection (the pages name only "a
 * 2x2 patch-merging projector" without bias; this variant is a reading of a
 * deeper adapter, off by default):
 *   y   = RMSNorm(h_L) * proj->norm         per patch, eps = cfg.rms_eps
 *   z   = 2x2 gather of y (as the plain merge: (dy,dx) order, channel fastest)
 *   m   = z merge_w^T                       merge_w [D][4D] (4D -> D)
 *   a   = GELU(m w1^T)                      w1 [out_dim][D], GELU(x) = x Phi(x)
 *   out = a w2^T                            w2 [out_dim][out_dim]
 * all without bias.  The weights come from pv_weights.merge_w and
 * pv_weights.proj. */
#define PV_FLAG_DEEP_PROJECTOR 4
/* pv_config.flags, both dtypes: the other split of the 2-D rotary
 * frequencies between the axes.  By default both the row pairs (0..15 of a
 * head) and the column pairs (16..31) turn at omega_m = theta^(-2m/32),
 * m = 0..15.  With this bit the two axes share one ladder theta^(-j/32),
 * j = 0..31: rows take the even steps (omega_m = theta^(-2m/32), as by
 * default) and columns the odd ones (omega_m = theta^(-(2m+1)/32)).  The
 * pages fix the rotary base ("Mistral 3", Mistral3Model table,
 * vision_rope_theta) and the row/column split of the pairs, not which
 * ladder steps each axis takes; only the host-built rotation table
 * changes. */
#define PV_FLAG_ROPE_INTERLEAVED 8

/* Per-block weights: borrowed device pointers, row-major, "out x in" like a
 * linear layer (y = x W^T).  Gains are always fp32; matrices use cfg.dtype. */
typedef struct pv_layer_weights {
  const float* attn_norm; /* [D]    */
  const void* wq;         /* [D][D] */
  const void* wk;         /* [D][D] */
  const void* wv;         /* [D][D] */
  const void* wo;         /* [D][D] */
  const float* ffn_norm;  /* [D]    */
  const void* w_gate;     /* [F][D] */
  const void* w_up;       /* [F][D] */
  const void* w_down;     /* [D][F] */
} pv_layer_weights;

/* Weights of the deeper projector (PV_FLAG_DEEP_PROJECTOR): borrowed device
 * pointers, matrices in cfg.dtype. */
typedef struct pv_projector_weights {
  const float* norm;  /* [D] fp32 gain of the RMSNorm before the merge */
  const void* w1;     /* [out_dim][D]       */
  const void* w2;     /* [out_dim][out_dim] */
} pv_projector_weights;

typedef struct pv_weights {
  const void* patch_w;             /* [D][3][p][p] device, cfg.dtype (conv kernel, no bias) */
  const float* ln_pre;             /* [D] device fp32 */
  const pv_layer_weights* layers;  /* HOST array of cfg.layers entries; copied at create */
  const void* merge_w;             /* [out_dim][4D] device, cfg.dtype; K order (dy,dx,channel)
                                      with channel fastest; NULL when merge == 1.  With
                                      PV_FLAG_DEEP_PROJECTOR: [D][4D] (4D -> D) */
  const pv_projector_weights* proj; /* HOST pointer, read at create; NULL unless
                                       PV_FLAG_DEEP_PROJECTOR */
} pv_weights;

typedef struct pv_tower pv_tower;

typedef struct pv_plan_info {
  int64_t n_patches;       /* sum over images of (H/p)(W/p) */
  int64_t out_rows;        /* merged tokens (merge 2) or n_patches (merge 1) */
  int64_t out_cols;        /* out_dim (merge 2) or hidden (merge 1) */
  int64_t workspace_bytes; /* device workspace that forward() needs */
  int32_t n_images;
  int32_t max_patches;     /* longest image, in patches */
  int32_t attn_q_tile;     /* queries per attention work item chosen for the
                            * call: bf16 256 (8 waves) or 384 (12 waves, when
                            * those items fill the chip's rounds of
                            * workgroups better at no more padding); f32 64 */
} pv_plan_info;

/* Creates a tower.  cfg and w are read (w->layers is copied); the device
 * pointers inside w are borrowed.  Builds the rotary cos/sin table on the host
 * in double precision.  Allocates no device memory.
 * Errors: PV_ERR_ARG (null, bad field, PV_FLAG_DEEP_PROJECTOR without
 * proj weights), PV_ERR_UNSUPPORTED (head_dim != 64, hidden or mlp not a
 * multiple of 256, mlp above 2^20, out_dim not a multiple of 128, the deeper
 * projector with the fp32 tower or without merge). */
pv_status pv_tower_create(const pv_config* cfg, const pv_weights* w, pv_tower** out);

/* Frees the tower's host resources.  Waits for the tower's own pending
 * host-to-device uploads first.  NULL is ignored. */
void pv_tower_destroy(pv_tower* t);

/* Derived weight copies, made once instead of in every forward call: the
 * bf16 tower's patch weights zero-padded to the GEMM's K, per block the fp16
 * copies of the gate, up and down weights for the MLP's fp16 products (round
 * to nearest even, saturated to +-65504) -- or, with PV_FLAG_FP8, the
 * block-scaled e4m3 copies of all seven block matrices -- and with merge 2
 * the fp4 (e2m1, 32-k scale blocks) copy of the merge weights that
 * multiplies the merger input's low part.
 * pv_tower_prepared_bytes: device bytes those copies need (0 for the fp32
 *   tower, which uses its weights as given).  Host-only.
 * pv_tower_prepare: writes the copies into mem (device, caller-owned,
 *   256-byte aligned, at least pv_tower_prepared_bytes) on stream and makes
 *   every later forward of this tower read them there (its workspace then
 *   shrinks by the regions they used to take).  Allocates nothing.  mem is
 *   borrowed: keep it allocated and unmodified while the tower is used, and
 *   prepare again after changing the weights.  Work on another stream must be
 *   ordered after this stream's copies by the caller.  mem == NULL detaches:
 *   forward calls derive the copies per call again.  A failed preparation
 *   leaves the tower detached.
 * Errors: PV_ERR_ARG (null tower or bytes, misaligned mem), PV_ERR_CAPACITY
 * (mem_bytes too small), PV_ERR_HIP. */
pv_status pv_tower_prepared_bytes(const pv_tower* t, int64_t* bytes);
pv_status pv_tower_prepare(pv_tower* t, void* mem, int64_t mem_bytes, void* stream);

/* Host-only, pure: validates image_hw (host, [n_images][2] = (H, W) pixels)
 * and fills *info.  Errors: PV_ERR_ARG, PV_ERR_SHAPE. */
pv_status pv_tower_plan(const pv_tower* t, const int32_t* image_hw, int32_t n_images,
                        pv_plan_info* info);

/* Runs the whole tower.
 *  pixels    device fp32, normalised; image i's 3 x H_i x W_i planes (channel,
 *            row, column; column fastest) follow image i-1's.
 *  image_hw  host int32 [n_images][2].
 *  out       device [out_rows][out_cols] in cfg.out_dtype (fp32 for the fp32
 *            tower); images in input order,
 *            merged tokens row-major within an image.
 *  out_rows_cap  rows the caller allocated for out.
 *  workspace device, at least pv_plan_info.workspace_bytes, 256-byte aligned.
 *  stream    hipStream_t.
 * Errors: PV_ERR_ARG, PV_ERR_SHAPE, PV_ERR_CAPACITY, PV_ERR_HIP. */
pv_status pv_tower_forward(pv_tower* t, const float* pixels, const int32_t* image_hw,
                           int32_t n_images, void* out, int64_t out_rows_cap,
                           void* workspace, size_t ws_bytes, void* stream);

/* Debug entry: runs the tower up to a stage and copies that tensor into dst
 * (device, dst_bytes large enough).  Stages:
 *   PV_STAGE_PATCH_EMBED  X = conv(pixels)               [N][D] fp32
 *   PV_STAGE_LN_PRE       h0 = RMSNorm(X) * ln_pre       [N][D] fp32
 *   PV_STAGE_QKV          layer l: [q|k|v], q,k rotated  [N][3D] cfg.dtype
 *                         (bf16 tower: q is stored times log2(e)/sqrt(64),
 *                         the units of its softmax)
 *   PV_STAGE_ATTN         layer l: attention output      [N][D] cfg.dtype
 *   PV_STAGE_ATTN_RESID   layer l: h after attention     [N][D] fp32
 *   PV_STAGE_MLP_HIDDEN   layer l: silu(gate)*up         [N][F] fp16 (bf16
 *                         tower; bf16 with PV_FLAG_FP8), fp32 (fp32 tower)
 *   PV_STAGE_BLOCK_OUT    layer l: h after the block     [N][D] fp32
 * Errors: as pv_tower_forward, PV_ERR_ARG for a bad stage or layer. */
enum {
  PV_STAGE_PATCH_EMBED = 0,
  PV_STAGE_LN_PRE = 1,
  PV_STAGE_QKV = 2,
  PV_STAGE_ATTN = 3,
  PV_STAGE_ATTN_RESID = 4,
  PV_STAGE_MLP_HIDDEN = 5,
  PV_STAGE_BLOCK_OUT = 6
};
pv_status pv_tower_forward_stage(pv_tower* t, const float* pixels, const int32_t* image_hw,
                                 int32_t n_images, int32_t stage, int32_t layer, void* dst,
                                 int64_t dst_bytes, void* workspace, size_t ws_bytes,
                                 void* stream);

/* Index maps of a batch ("Mistral 3", Mistral3VisionModel: packed sequence;
 * "Several images in one conversation": per-image counts):
 *   cu_seqlens [n+1]     prefix sums of patch counts
 *   patch_rc   [N][2]    (row, column) of every patch within its image
 *   merge_src  [T][4]    the four patches of each merged token, order
 *                        (0,0),(0,1),(1,0),(1,1); unused when merge == 1
 * on_device == 0: host pointers, computed by the host planner.
 * on_device == 1: device pointers, written by the same GPU kernel whose maps
 *   the hot kernels read; workspace as for forward; enqueued on stream.
 * merge_src may be NULL.  Errors: PV_ERR_ARG, PV_ERR_SHAPE, PV_ERR_CAPACITY,
 * PV_ERR_HIP. */
pv_status pv_tower_index_maps(pv_tower* t, const int32_t* image_hw, int32_t n_images,
                              int32_t* cu_seqlens, int32_t* patch_rc, int32_t* merge_src,
                              int32_t on_device, void* workspace, size_t ws_bytes,
                              void* stream);

/* Per-kernel-class timing of forward calls, measured with HIP events
 * recorded on the caller's stream around every launch of that class.
 * pv_tower_set_profiling(t, 1) starts recording (and clears earlier records),
 * 0 stops.  pv_tower_read_profile waits for the recorded events (host
 * synchronisation), then writes, per class, the summed kernel time in
 * milliseconds and the number of launches (host arrays of PV_K_COUNT
 * entries); reset != 0 clears the records.  Recording adds two event records
 * per launch; leave it off for throughput runs.
 * Errors: PV_ERR_ARG (null), PV_ERR_HIP. */
enum {
  PV_K_MAPS = 0,     /* per-row index maps                                    */
  PV_K_PATCH = 1,    /* patch embedding GEMM (+ weight padding when unprepared) */
  PV_K_NORM = 2,     /* RMSNorm passes before attention (ln_pre + first one fused) */
  PV_K_QKV = 3,      /* q,k,v GEMM with the rotary epilogue (+ the fp8 variant's
                        weight copies when unprepared)                        */
  PV_K_ATTN = 4,     /* block-diagonal attention                              */
  PV_K_OPROJ = 5,    /* out-projection GEMM (+ residual)                      */
  PV_K_GATEUP = 6,   /* MLP gate/up GEMM (silu * up) (+ the fp16 weight
                        copies when unprepared)                               */
  PV_K_DOWN = 7,     /* MLP down GEMM (+ residual) (+ the fp16 weight copy
                        when unprepared)                                      */
  PV_K_MERGE = 8,    /* 2x2 merge GEMM                                        */
  PV_K_NORM_MLP = 9, /* RMSNorm passes before the MLP (fp16 output)          */
  PV_K_OPERAND = 10, /* operand passes: im2col hi | lo split (or the uint8
                        resize into it), final residual hi | lo split or
                        output copy                                           */
  PV_K_COUNT = 11
};
pv_status pv_tower_set_profiling(pv_tower* t, int32_t enable);
pv_status pv_tower_read_profile(pv_tower* t, double* ms, int64_t* launches, int32_t reset);

/* Merge of the tower output into a text-embedding sequence ("Mistral 3"
 * (KerasFormers) model page: Mistral3Model argument table, image_token_id --
 * the placeholder token the processor expands to each image's own number of
 * merged tokens -- and "Several images in one conversation"; the
 * inference-research record's masked-scatter merge of projected image
 * features into the decoder's input embeddings).
 * Position p of the sequence (0 <= p < seq_len) with token_ids[p] ==
 * image_token_id is the k-th such position (k counted from 0 in sequence
 * order); row p of text_emb is replaced by row k of image_emb when
 * k < n_image_rows.  Other rows are left unchanged.
 *   token_ids   device int32 [seq_len]
 *   image_emb   device [n_image_rows][dim], elements of elem_bytes bytes
 *               (2 = bf16, 4 = fp32; the tower output as written)
 *   text_emb    device [seq_len][dim], same element size; updated in place
 *   status      device int32 [1], written: 0 if the number of placeholder
 *               positions equals n_image_rows, else 1 (the copy then covers
 *               min(count, n_image_rows) rows)
 *   workspace   device, >= pv_scatter_workspace_bytes(seq_len) bytes,
 *               256-byte aligned
 * Rows must be 16-byte multiples (dim * elem_bytes % 16 == 0) and all
 * pointers 16-byte aligned.  Enqueued on stream; no synchronisation.
 * Errors: PV_ERR_ARG (null pointer, seq_len < 0, n_image_rows < 0, dim < 1,
 * elem_bytes not 2 or 4, misalignment), PV_ERR_CAPACITY (workspace),
 * PV_ERR_HIP. */
size_t pv_scatter_workspace_bytes(int64_t seq_len);
pv_status pv_scatter_image_embeddings(const int32_t* token_ids, int64_t seq_len, int32_t image_token_id,
                                      const void* image_emb, int64_t n_image_rows, void* text_emb,
                                      int32_t dim, int32_t elem_bytes, int32_t* status, void* workspace,
                                      size_t ws_bytes, void* stream);

/* pv_scatter_image_embeddings for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same operation and arguments without the workspace.  Its
 * scratch (the list of placeholder positions and their count) is a fixed
 * 4 MB array in the library's device memory, one per GPU, held until the
 * process ends; nothing is allocated by the call.  seq_len is at most
 * 1,048,576 (2^20) positions.  The array of the current device is used (the
 * stream must belong to it); every call on one GPU shares it, so calls that
 * overlap on one GPU (different streams, or host threads) race -- serialise
 * them, e.g. on one stream.  Nothing in it needs clearing: each call writes
 * the count and the list before reading them.
 * Errors: as pv_scatter_image_embeddings, and PV_ERR_CAPACITY when seq_len
 * exceeds 2^20. */
pv_status pv_scatter_image_embeddings_noalloc(const int32_t* token_ids, int64_t seq_len, int32_t image_token_id,
                                              const void* image_emb, int64_t n_image_rows, void* text_emb,
                                              int32_t dim, int32_t elem_bytes, int32_t* status, void* stream);

/* ---- uint8 input: resize onto the patch grid + normalisation ----
 * Sources: "Mistral 3" (KerasFormers) model page, description (images are
 * resized so that the longest edge fits longest_edge and the sides stay on
 * the patch grid) and Mistral3ImageProcessor table (longest_edge 1540, patch
 * 14, per-channel mean and std).  Readings where the page is silent:
 *  - target size: if max(H, W) > longest_edge, each side becomes
 *    floor(side * longest_edge / max(H, W)) (at least 1; images are never
 *    enlarged); then each side is rounded up to a multiple of grid, capped at
 *    the largest multiple of grid within longest_edge.  For a tower, grid =
 *    patch * merge (the merge needs whole 2x2 patch windows) and
 *    longest_edge = max_side.
 *  - resampling: bilinear, pixel centres at half-integers (source coordinate
 *    (t + 0.5) * in / out - 0.5, clamped at the first pixel; the upper tap
 *    clamped at the last), no antialiasing, computed in fp32 on the uint8
 *    values (no re-quantisation).
 *  - normalisation: (x / 255 - mean_c) / std_c.
 * Image layout: uint8 H x W x 3 (row, column, channel; RGB, channel fastest);
 * image i follows image i-1 with no padding.  Every source side must be in
 * [1, 32768].  mean_std: host float [6] = mean R, G, B then std R, G, B, or
 * NULL for the processor table's values (0.48145466, 0.4578275,
 * 0.40821073; 0.26862954, 0.26130258, 0.27577711). */

/* Host-only, pure: target sizes (dst_hw, host [n_images][2]) of source sizes
 * (src_hw, host [n_images][2]) under the rule above.
 * Errors: PV_ERR_ARG (null, n_images < 1, grid < 1, longest_edge < grid),
 * PV_ERR_SHAPE (a source side outside [1, 32768]). */
pv_status pv_resize_target(const int32_t* src_hw, int32_t n_images, int32_t longest_edge,
                           int32_t grid, int32_t* dst_hw);

/* Host-only, pure: as pv_tower_plan for uint8 sources of sizes src_hw, with
 * the tower's own longest_edge (max_side) and grid (patch * merge); writes
 * the target sizes to dst_hw (host [n_images][2], may be NULL).  The
 * workspace size is the same as for pv_tower_plan of the target sizes.
 * Errors: PV_ERR_ARG, PV_ERR_SHAPE. */
pv_status pv_tower_plan_u8(const pv_tower* t, const int32_t* src_hw, int32_t n_images,
                           int32_t* dst_hw, pv_plan_info* info);

/* Runs the whole tower from uint8 images: the resize and the normalisation
 * happen inside the patch embedding's operand load (bf16 tower: no
 * intermediate image; fp32 tower: the normalised planes go through the
 * workspace).  Output, out_rows_cap, workspace, stream: as pv_tower_forward,
 * for the target sizes pv_tower_plan_u8 reports.
 *  images  device uint8, the layout above; src_hw host [n_images][2].
 * Errors: PV_ERR_ARG (null, misaligned output/workspace, bad mean_std),
 * PV_ERR_SHAPE, PV_ERR_CAPACITY, PV_ERR_HIP. */
pv_status pv_tower_forward_u8(pv_tower* t, const uint8_t* images, const int32_t* src_hw,
                              int32_t n_images, const float* mean_std, void* out,
                              int64_t out_rows_cap, void* workspace, size_t ws_bytes,
                              void* stream);

/* The preprocessing alone, to any target size: image i (src_hw[i], uint8,
 * layout above) is resampled to dst_hw[i] and normalised into out (device
 * fp32, 4-byte aligned): image i's 3 x tH x tW planes (channel, row, column)
 * after image i-1's -- the pixel layout pv_tower_forward takes.  src_hw and
 * dst_hw are host [n_images][2]; every side in [1, 32768].  No workspace;
 * one launch per image on stream.
 * Errors: PV_ERR_ARG (null, n_images < 1, misaligned out, bad mean_std),
 * PV_ERR_SHAPE, PV_ERR_HIP. */
pv_status pv_preprocess_u8(const uint8_t* images, const int32_t* src_hw, const int32_t* dst_hw,
                           int32_t n_images, const float* mean_std, float* out, void* stream);

/* ---- tiles ("Pixtral-12B-2409" inference-research record, VISION TOKENS:
 * large images are split into 1024x1024 tiles -- a 4096x4096 image is a 4x4
 * grid of 16 tiles, 65,536 patches -- and the processor caps the tile count
 * with max_num_tiles).  Readings: the image is scaled by the largest
 * s <= 1 whose tile grid ceil(s*H/tile) x ceil(s*W/tile) has at most
 * max_num_tiles tiles (exact fractions; s = 1 when the unscaled grid fits),
 * each side becoming max(1, floor(s*side)) rounded up to a multiple of grid;
 * the resized image is cut row-major into tile x tile tiles, the last row
 * and column keeping the remainder (multiples of grid).  Each tile is one
 * image of the tower (its own attention block, positions from 0).  Pixels
 * are resampled and normalised as for pv_tower_forward_u8. */

/* Host-only, pure: layout (host [n_images][4]) = resized H, resized W, tile
 * rows, tile columns of each source size (src_hw, host [n_images][2]).
 * Errors: PV_ERR_ARG (null, n_images < 1, grid < 1, tile not a positive
 * multiple of grid or > 32768, max_num_tiles outside [1, 65536]),
 * PV_ERR_SHAPE (a source side outside [1, 32768]). */
pv_status pv_tile_layout(const int32_t* src_hw, int32_t n_images, int32_t tile, int32_t grid,
                         int32_t max_num_tiles, int32_t* layout);

/* Host-only, pure: plan of the tiles of uint8 sources with tile = the
 * tower's max_side and grid = patch * merge; layout as pv_tile_layout (may
 * be NULL).  info counts every tile as an image.
 * Errors: PV_ERR_ARG, PV_ERR_SHAPE, PV_ERR_UNSUPPORTED (max_side not a
 * multiple of patch * merge). */
pv_status pv_tower_plan_tiles_u8(const pv_tower* t, const int32_t* src_hw, int32_t n_images,
                                 int32_t max_num_tiles, int32_t* layout, pv_plan_info* info);

/* Runs the tower over the tiles of uint8 images (layout as for
 * pv_tower_forward_u8); the resampling happens per tile inside the patch
 * embedding's operand load.  Output rows: tiles row-major within an image,
 * images in order; per tile its merged tokens (merge 2) or patches (merge 1),
 * row-major.  Errors: as pv_tower_forward_u8, PV_ERR_ARG for
 * max_num_tiles < 1, PV_ERR_UNSUPPORTED as pv_tower_plan_tiles_u8. */
pv_status pv_tower_forward_tiles_u8(pv_tower* t, const uint8_t* images, const int32_t* src_hw,
                                    int32_t n_images, int32_t max_num_tiles, const float* mean_std,
                                    void* out, int64_t out_rows_cap, void* workspace,
                                    size_t ws_bytes, void* stream);

/* Configurations of the two towers the pages describe, filled into *cfg
 * (dtype and out_dtype = dtype, flags 0):
 *   PV_PRESET_MISTRAL3    "Mistral 3", Mistral3Model argument table and
 *                         Mistral3ImageProcessor: patch 14, width 1024, MLP
 *                         4096, 24 layers, 16 heads, rotary base 1e4, 2x2
 *                         merge to 5120, longest edge 1540.
 *   PV_PRESET_PIXTRAL12B  "Pixtral-12B-2409", part (1) Vision: patch 16,
 *                         width 1024, MLP 4096, 24 layers, 16 heads, rotary
 *                         base 1e4, no merge, image size (tile) 1024.
 * rms_eps 1e-5 in both.  Errors: PV_ERR_ARG (null, unknown preset or
 * dtype). */
enum { PV_PRESET_MISTRAL3 = 0, PV_PRESET_PIXTRAL12B = 1 };
pv_status pv_config_preset(int32_t preset, int32_t dtype, pv_config* cfg);

/* ---- multimodal embeddings cache (the inference-research record: an engine
 * keeps a per-model cache of multimodal embeddings next to an encoder side
 * stream).  The cache maps an image's content key to its output rows, kept
 * in caller-owned device memory; a hit skips the tower.  The side stream
 * needs no entry point: every call runs on the stream it is given, so the
 * encoder can be enqueued on its own stream and the consumer can wait on an
 * event recorded after it. */

/* Content keys of uint8 images (layout as for pv_tower_forward_u8; images
 * 4-byte aligned): keys (device uint64 [n_images][2]) = two 64-bit lanes per
 * image over its bytes and size.  Definition (exact, so a caller can compute
 * the same key on the host): mix(z) is SplitMix64's output function
 * (z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 * z *= 0x94D049BB133111EB; z ^= z >> 31); w_i are the image's 3HW bytes as
 * little-endian 64-bit words, the last one zero-padded;
 * acc_s = sum_i mix(w_i + (i + 1) * G_s) mod 2^64;
 * key_s = mix(acc_s + mix(((H << 32) | W) ^ G_s)), G_0 = 0x9E3779B97F4A7C15,
 * G_1 = 0xD1B54A32D192ED03.  Not cryptographic.  workspace: device,
 * >= pv_image_keys_workspace_bytes(n_images), 256-byte aligned.
 * Errors: PV_ERR_ARG, PV_ERR_SHAPE, PV_ERR_CAPACITY, PV_ERR_HIP. */
size_t pv_image_keys_workspace_bytes(int32_t n_images);
pv_status pv_image_keys_u8(const uint8_t* images, const int32_t* src_hw, int32_t n_images,
                           uint64_t* keys, void* workspace, size_t ws_bytes, void* stream);

typedef struct pv_embcache pv_embcache;

/* Creates a cache over cache_mem (device, cache_bytes, 16-byte aligned,
 * owned by the caller) for tower t (borrowed; it must outlive the cache).
 * It holds cache_bytes / row_bytes output rows (row_bytes = out_cols times
 * the output element size).  mean_std (host [6] or NULL, copied) is the
 * normalisation every cached forward uses.  Errors: PV_ERR_ARG,
 * PV_ERR_CAPACITY (not one row). */
pv_status pv_embcache_create(pv_tower* t, const float* mean_std, void* cache_mem,
                             int64_t cache_bytes, pv_embcache** out);
void pv_embcache_destroy(pv_embcache* c);
/* Forgets every entry (the memory is kept). */
pv_status pv_embcache_clear(pv_embcache* c);
/* stats (host int64 [5]): entries, rows in use, capacity in rows, images
 * served from the cache, images computed. */
pv_status pv_embcache_stats(const pv_embcache* c, int64_t* stats);
/* Workspace (bytes) of a cached forward of these uint8 sources. */
pv_status pv_embcache_workspace_bytes(const pv_embcache* c, const int32_t* src_hw,
                                      int32_t n_images, int64_t* bytes);

/* pv_tower_forward_u8 through the cache.  keys: host uint64 [n_images][2]
 * chosen by the caller (one key per distinct image content and size), or
 * NULL: then the keys are computed on the device (pv_image_keys_u8) and read
 * back, which synchronises the stream.  Images whose key is cached are
 * copied from the cache; the others (each distinct key once) run through
 * one tower forward into a contiguous run of cache rows at the ring head,
 * evicting the entries that run overlaps (oldest insertions first), and are
 * copied out.  out/out_rows_cap: as pv_tower_forward_u8.  hit: host int32
 * [n_images] or NULL; 1 where the image was served from the cache (also a
 * repeat of an image computed earlier in the same call), 0 where the tower
 * ran for it.  Use one stream per cache.
 * Errors: PV_ERR_ARG, PV_ERR_SHAPE, PV_ERR_CAPACITY (workspace, output, or
 * the missed images need more rows than the cache holds), PV_ERR_HIP. */
pv_status pv_tower_forward_cached_u8(pv_embcache* c, const uint8_t* images, const int32_t* src_hw,
                                     int32_t n_images, const uint64_t* keys, void* out,
                                     int64_t out_rows_cap, void* workspace, size_t ws_bytes,
                                     void* stream, int32_t* hit);

/* The block-scaled fp8 quantisation the PV_FLAG_FP8 tower applies to its
 * weights, as a standalone pass (e.g. to inspect or store fp8 weights):
 *  src     device bf16 [rows][K], K a multiple of 128, 16-byte aligned
 *  codes   device uint8 [rows][K]: e4m3 bytes (OCP E4M3FN) of src / 2^X,
 *          rounded to nearest even, 16-byte aligned
 *  scales  device uint8: for row r and 32-column block b, the E8M0 byte
 *          X + 127 at scales[((b / 4) * rows + r) * 4 + b % 4], where
 *          X = floor(log2(max |block|)) - 7 clamped to [-120, 120]
 * Errors: PV_ERR_ARG, PV_ERR_HIP. */
pv_status pv_quantize_fp8(const void* src, int64_t rows, int32_t K, void* codes, void* scales,
                          void* stream);

/* Thread-local message of the last failure in this thread ("" if none). */
const char* pv_last_error(void);

/* Static name of a status code. */
const char* pv_status_str(pv_status s);

#ifdef __cplusplus
}
#endif

#endif /* PV_TOWER_H */
