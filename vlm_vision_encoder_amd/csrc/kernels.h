// Launch functions of the tower's kernels (host side).  All enqueue on the
// given stream and return the launch status; none synchronises.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace pv {

enum GemmKind {
  GEMM_PATCH = 0,   // im2col(pixels) x patch_w^T -> fp32 X
  GEMM_QKV = 1,     // y x [wq|wk|wv]^T -> bf16 q,k (rotated), v
  GEMM_OPROJ = 2,   // attn x wo^T added into the fp32 residual
  GEMM_GATEUP = 3,  // silu(y gate^T) * (y up^T) -> bf16
  GEMM_DOWN = 4,    // hm x w_down^T added into the fp32 residual
  GEMM_MERGE = 5,   // gather2x2(residual) x merge_w^T -> bf16 out
  GEMM_PLAIN = 6,   // dense A x B^T -> bf16 (tests and measurement)
  GEMM_MERGE_F32 = 7,  // as GEMM_MERGE with an fp32 output
  GEMM_GELU = 8,       // dense A x B^T -> bf16 GELU(.) (deeper projector)
  GEMM_PLAIN_F32 = 9   // dense A x B^T -> fp32
};

// bf16 MFMA GEMM family (gemm_bf16.hip).
hipError_t gemm_bf16(GemmKind kind, const GemmArgs& g, hipStream_t s);

// fp32 GEMM family, same kinds and operand conventions (f32_path.hip).
hipError_t gemm_f32(GemmKind kind, const GemmArgs& g, hipStream_t s);

// RMSNorm kernels (norm.hip).  Rows of width D (a multiple of 256).
//   rmsnorm:      y = x / sqrt(mean(x^2) + eps) * g           (x fp32 -> y bf16 or fp32)
//   rmsnorm_dual: h = norm(x) * g1 written back in place (fp32), y = norm(h) * g2
hipError_t rmsnorm(const float* x, const float* g, void* y, int rows, int D, float eps,
                   bool y_f32, hipStream_t s);
// rmsnorm_f16: y = norm(x) * g as fp16 [N][D] (round to nearest even,
// saturated to +-65504)
hipError_t rmsnorm_f16(const float* x, const float* g, void* y, int rows, int D, float eps, hipStream_t s);
// rmsnorm_fp8: y = norm(x) * g as fp8 e4m3 [N][D] with a power-of-two scale
// byte per 32 columns, step-major: ys[(col / 128) * srows + row][(col / 32) % 4]
hipError_t rmsnorm_fp8(const float* x, const float* g, void* y8, void* ys, int rows, int srows, int D, float eps,
                       hipStream_t s);
// merge_hi_lo4: the merger's input x [N][D] as bf16 hi rows yh [N][D] plus
// the fp4 low part gathered in merged-token order: y4 [T][4D/2] (row t =
// the low parts of source rows msrc[t][0..3]), scale bytes
// ys[(k / 256) * srows + t][(k / 32) % 8], k = j D + col
hipError_t merge_hi_lo4(const float* x, const int32_t* msrc, void* yh, void* y4, void* ys, int tokens, int srows,
                        int D, hipStream_t s);
hipError_t rmsnorm_dual(float* x, const float* g1, const float* g2, void* y, int rows, int D,
                        float eps, bool y_f32, hipStream_t s);

// Block-diagonal attention over the packed sequence (attn_bf16.hip, f32_path.hip).
struct AttnArgs {
  const void* qkv;   // [N][3D]: q (rotated) | k (rotated) | v
  void* out;         // [N][D]
  const ImageMeta* meta;
  const AttnItem* items;
  int32_t n_items;
  int32_t heads;
  int32_t hidden;
  int32_t online_max;  // 1: always use the running-max softmax (bf16 path)
  int32_t q_tile;      // queries per work item (bf16: kAttnQTileBf16 or kAttnQTileBf16Wide)
  int32_t head_major;  // bf16: 1 when every image has the same length (work order below)
};
hipError_t attention_bf16(const AttnArgs& a, hipStream_t s);
hipError_t attention_f32(const AttnArgs& a, hipStream_t s);
// bf16 attention shape: each wave owns 32 * PV_ATTN_QB queries, a work item
// PV_ATTN_WAVES waves.
#ifndef PV_ATTN_QB
#define PV_ATTN_QB 1
#endif
#ifndef PV_ATTN_WAVES
#define PV_ATTN_WAVES 8
#endif
constexpr int kAttnQTileBf16 = 32 * PV_ATTN_QB * PV_ATTN_WAVES;
constexpr int kNumCUs = 256;  // MI355X: 8 XCDs x 32 CUs
// the wide work item: 12 waves, one workgroup per CU
constexpr int kAttnWavesWide = 12;
constexpr int kAttnQTileBf16Wide = 32 * PV_ATTN_QB * kAttnWavesWide;
constexpr int kAttnQTileF32 = 64;

// Per-row maps from per-image metadata (maps.hip):
//   rowinfo[g] = (image, row << 16 | col), msrc[t] = 4 source patch rows.
hipError_t build_maps(const ImageMeta* meta, int n_images, int n_patches, int out_rows,
                      int merge, int32_t* rowinfo, int32_t* msrc, hipStream_t s);
// rowinfo -> (row, col) pairs and cu_seqlens from meta (for the index-map entry).
hipError_t export_maps(const ImageMeta* meta, const int32_t* rowinfo, int n_images,
                       int n_patches, int32_t* cu_seqlens, int32_t* patch_rc, hipStream_t s);

// fp32 -> bf16 copy (no-merge output of the bf16 path).
hipError_t f32_to_bf16(const float* x, void* y, size_t n, hipStream_t s);
// Operand preparation (bf16 hi | lo halves of fp32 A operands):
//   im2col_split: out [N][2 Kp] = im2col(pixels) as hi | lo, k >= K zero
//   pad_rows:     out [rows][Kp] = w [rows][K] zero-padded (bf16)
hipError_t im2col_split(const float* pixels, const DevMaps& maps, void* out, int n_patches, int K, int Kp,
                        hipStream_t s);
// Resize + normalisation of uint8 H x W x 3 images: value = raw * mul[c] +
// add[c] after a half-pixel-centre bilinear resample to the plan's size.
struct NormAff {
  float mul[3], add[3];
};
//   im2col_u8_split: as im2col_split, with the pixels sampled from the uint8
//                    sources src[] (device, one per plan image)
//   resize_norm_u8:  the tH x tW window at (sm.y0, sm.x0) of the source
//                    `image` resized to sm.RH x sm.RW -> fp32 planes [3][tH][tW]
hipError_t im2col_u8_split(const uint8_t* images, const SrcImage* src, const DevMaps& maps, const NormAff& aff,
                           void* out, int n_patches, int K, int Kp, hipStream_t s);
hipError_t resize_norm_u8(const uint8_t* image, const SrcImage& sm, int tH, int tW, const NormAff& aff, float* out,
                          hipStream_t s);
hipError_t pad_rows(const void* w, void* out, int rows, int K, int Kp, hipStream_t s);
//   quant_rows_fp8: rows [row0, row0 + rows) of dst8 [.][K] = the bf16 src
//                 [rows][K] in fp8 e4m3, scales[(k/128)*srows + row][(k/32)%4]
//                 one E8M0 byte per 32 k (K a multiple of 128)
hipError_t quant_rows_fp8(const void* src, int rows, int K, void* dst8, void* scales, int srows, int row0,
                          hipStream_t s);
//   gateup_fp8:   b8 [2F][D] fp8 e4m3 = the gate/up weights in the GEMM's
//                 interleaved row order, bs [D/128][2F][4] scale bytes
hipError_t gateup_fp8(const void* w_gate, const void* w_up, void* b8, void* bs, int F, int D, hipStream_t s);
//   rows_fp4:     a bf16 [rows][K] matrix in packed fp4 e2m1, b4 [rows][K/2],
//                 bs [K/256][rows][8] scale bytes (K a multiple of 256)
hipError_t rows_fp4(const void* w, int rows, int K, void* b4, void* bs, hipStream_t s);
//   copy_f16:     n bf16 values -> fp16 (round to nearest even, saturated to
//                 +-65504); n a multiple of 8, both pointers 16-byte aligned
hipError_t copy_f16(const void* src, long long n, void* h16, hipStream_t s);
// Content keys of uint8 images (two 64-bit lanes per image, keys [n][2]
// device); offsets[i] (host) is image i's byte offset from `images`, which
// must be 4-byte aligned; src_hw host; ws: image_keys_workspace_bytes(n)
// bytes (the accumulators).
size_t image_keys_workspace_bytes(int n);
hipError_t image_keys(const uint8_t* images, const int32_t* src_hw, const uint64_t* offsets, int n, uint64_t* keys,
                      void* ws, hipStream_t s);
// Masked scatter: the k-th position p with ids[p] == token takes row k of src
// (k < rows); status[0] = (placeholder count == rows) ? 0 : 1.  ws: a list of
// n positions + the count (scatter_workspace_bytes(n) bytes).
size_t scatter_workspace_bytes(int64_t n);
hipError_t scatter_rows(const int32_t* ids, int64_t n, int32_t token, const void* src, int64_t rows, void* dst,
                        int64_t row_bytes, int32_t* status, void* ws, hipStream_t s);

}  // namespace pv
