// Host planner of a tower call: validates image sizes, derives per-image
// metadata, the attention work list and the device workspace layout.
// Pure host C++ (no HIP), so it is testable without a GPU.
//
// Per-image counts follow "Mistral 3" (KerasFormers), Mistral3VisionModel
// (all images packed into one patch sequence) and "Several images in one
// conversation" (each image keeps its own patch count); without merge each
// patch is one output row ("Pixtral-12B-2409", VISION TOKENS).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace pv {

// Uploaded to the device as is (32 bytes, read by the kernels).
struct ImageMeta {
  int32_t H, W;            // pixels
  int32_t Hp, Wp;          // patches
  int32_t patch_base;      // first patch row of this image in the packed sequence
  int32_t tok_base;        // first output row (merged token) of this image
  uint32_t pix_lo, pix_hi; // 64-bit element offset of the image in the pixel buffer
};
static_assert(sizeof(ImageMeta) == 32, "ImageMeta layout");

// Source of one plan image (a whole resized image, or one tile of it) in the
// uint8 input (H x W x 3, channel fastest), for the resize in the patch
// embedding's A load; uploaded after the rotary table (32 bytes).
struct SrcImage {
  int32_t H, W;             // source pixels
  int32_t RH, RW;           // size of the resized image the plan image is cut from
  int32_t y0, x0;           // origin of the plan image in the resized image
  uint32_t off_lo, off_hi;  // 64-bit byte offset of the source in the uint8 buffer
};
static_assert(sizeof(SrcImage) == 32, "SrcImage layout");

// Largest source or resized side the resize accepts (its tap arithmetic is
// 32-bit), and the largest tile cap.
constexpr int32_t kMaxSrcSide = 32768;
constexpr int32_t kMaxTiles = 65536;

// One attention work item: q-tile starting at local query q0 of an image.
struct AttnItem {
  int32_t image;
  int32_t q0;
};

struct PlanParams {
  int32_t patch = 14;
  int32_t merge = 2;
  int32_t max_side = 1540;
  int32_t hidden = 1024;
  int32_t mlp = 4096;
  int32_t out_dim = 5120;
  int32_t elem_bytes = 2;   // 2 = bf16 activations, 4 = fp32
  int32_t q_tile = 256;     // queries per attention work item
  // bf16 attention: a wider item (q_tile_wide queries, one workgroup per
  // CU) is chosen per call when it fills the rounds of the chip better at no
  // more padding (0: never); heads and slots size the rounds
  int32_t q_tile_wide = 0;
  int32_t heads = 16;
  int32_t slots = 512;       // workgroups of q_tile queries the chip holds at once
  int32_t slots_wide = 256;  // the same for q_tile_wide
  int32_t rope_pairs = 16;  // rotation pairs per axis (head_dim / 4)
  bool fp8 = false;         // bf16 tower whose per-block linear maps run in fp8
  // the tower's derived weight copies (padded patch weights, fp4 / fp8 copies
  // of the block matrices) live in caller memory written once: the workspace
  // then holds no region for them
  bool prepared = false;
  // deeper projector: its out_dim-wide GELU output ([out_rows][out_dim] bf16)
  // goes through the big region (0: plain merge)
  int32_t deep_out = 0;
  // bf16 tower with merge == 2: rows of merge_w (out_dim, or D for the deeper
  // projector), whose fp4 copy the merger multiplies with its input's low
  // part; 0 otherwise
  int32_t merge_rows = 0;
};

// Byte offsets of a tower's derived weight copies in the memory that one
// preparation fills (bf16 tower; every region 256-byte aligned):
//   wpad  [D][Kp] bf16, the patch weights zero-padded to Kp
//   per layer l, at layer0 + l * layer_stride:
//     fp16 copies (bf16 tower): b8 [2F][D] fp16, the gate rows then the up
//       rows (bs empty), wd8 [D][F] fp16, the down weights (wds empty)
//     fp8 copies (fp8 variant): wq8 [3D][D] + wqs [D/128][3D][4], wo8 [D][D] +
//       wos [D/128][D][4], b8 [2F][D] + bs8 [D/128][2F][4], wd8 [D][F] + wds
//       [F/128][D][4]
//   after the layers (merge_rows > 0): mw4 [merge_rows][2D] the merge weights
//     in fp4, mws [4D/256][merge_rows][8] scale bytes
struct PrepLayout {
  size_t wpad = 0;
  size_t layer0 = 0, layer_stride = 0;
  // offsets within a layer's region
  size_t b8 = 0, bs = 0, wq8 = 0, wqs = 0, wo8 = 0, wos = 0, wd8 = 0, wds = 0;
  size_t mw4 = 0, mws = 0;
  size_t total = 0;
};
PrepLayout prep_layout(int32_t patch, int32_t hidden, int32_t mlp, int32_t layers, bool fp8, int32_t merge_rows);

// Bytes of the merge weights' fp4 copy and of its scale bytes (K = 4D).
inline size_t merge_fp4_bytes(int32_t merge_rows, int32_t hidden) { return size_t(merge_rows) * 2 * size_t(hidden); }
inline size_t merge_fp4_scale_bytes(int32_t merge_rows, int32_t hidden) {
  return size_t(hidden) / 64 * size_t(merge_rows) * 8;
}

// Rows of the MLP input's fp8 scale blocks: the patches plus one tile of
// padding (a GEMM tile reads the scale bytes of 256 consecutive rows).
inline int64_t a8_scale_rows(int64_t patches) { return patches + 256; }

// K of the patch embedding's bf16 GEMM: 3 p^2 zero-padded to a multiple of 64.
inline int32_t patch_kp(int32_t patch) { return (3 * patch * patch + 63) / 64 * 64; }

// Byte offsets into the device workspace (all 256-byte aligned).
struct Layout {
  size_t meta = 0, items = 0, rope = 0, src = 0, rowinfo = 0, msrc = 0;
  size_t r = 0, y = 0, big = 0;
  size_t wpad = 0;          // bf16 tower: patch weights zero-padded to [D][Kp]
  // bf16 tower, unprepared: b8 holds this layer's gate/up weights in fp16
  // [2F][D] (bs empty) and wd8 its down weights in fp16 [D][F]; fp8
  // variant: a8/as hold every fp8 GEMM input, up to [N][max(D, F)], and
  // b8/bs this layer's gate/up weights in fp8
  size_t a8 = 0, as = 0, b8 = 0, bs = 0;
  // bf16 tower with merge == 2: the merger input's low part goes through
  // a8 / as ([T][2D] fp4 in merged-token order, [4D/256][T + 256][8] scale
  // bytes); unprepared, mw4 / mws hold the merge weights' fp4 copy
  size_t mw4 = 0, mws = 0;
  // fp8 variant: this layer's q|k|v, out-projection and down weights in fp8
  // (wd8 / wds; the bf16 tower's fp16 down weights above use wd8 alone)
  size_t wq8 = 0, wqs = 0, wo8 = 0, wos = 0, wd8 = 0, wds = 0;
  size_t upload_bytes = 0;  // [0, upload_bytes) is filled by one host->device copy
  size_t total = 0;
};

struct Plan {
  int32_t n_images = 0;
  int64_t n_patches = 0;
  int64_t out_rows = 0;
  int32_t max_patches = 0;
  int32_t rope_maxpos = 0;  // positions per axis in the rotary table
  std::vector<ImageMeta> meta;
  std::vector<int32_t> cu;  // n_images + 1
  std::vector<AttnItem> items;
  int32_t q_tile = 0;  // queries per attention work item chosen for this call
  std::vector<SrcImage> src;  // uint8 input only (else empty; the region is zeroed)
  Layout ws;
};

// Target size of the resize onto the patch grid: if max(h, w) > longest_edge
// each side becomes floor(side * longest_edge / max(h, w)) (at least 1;
// images are never enlarged), then is rounded up to a multiple of `grid`,
// capped at the largest multiple of `grid` within longest_edge.  Exact
// integer arithmetic.  Returns 0, -1 (grid < 1 or longest_edge < grid) or -2
// (a side outside [1, kMaxSrcSide]) with *err set.
int resize_target(int32_t h, int32_t w, int32_t longest_edge, int32_t grid, int32_t* th, int32_t* tw,
                  std::string* err);

// Tile layout of one image: the image is scaled by s = min(1, max over tile
// grids r x c with r * c <= max_num_tiles of min(r*tile/h, c*tile/w)) (exact
// fractions), each side becoming max(1, floor(s * side)) rounded up to a
// multiple of `grid`; the tiles are tile x tile, row-major, the last row and
// column keeping the remainder.  Writes the resized size and the grid.
// Returns 0, -1 (grid < 1, tile not a multiple of grid, max_num_tiles outside
// [1, kMaxTiles]) or -2 (a side outside [1, kMaxSrcSide]) with *err set.
int tile_layout(int32_t h, int32_t w, int32_t tile, int32_t grid, int32_t max_num_tiles, int32_t* rh,
                int32_t* rw, int32_t* rows, int32_t* cols, std::string* err);

// Returns 0 on success, -1 (argument) or -2 (shape) with *err set.
int build_plan(const PlanParams& p, const int32_t* image_hw, int32_t n_images, Plan* out,
               std::string* err);

// Host reference of the index maps (cu_seqlens [n+1], patch_rc [N][2],
// merge_src [T][4]; merge_src may be null).
void host_index_maps(const Plan& plan, int merge, int32_t* cu_seqlens, int32_t* patch_rc,
                     int32_t* merge_src);

// Rotary cos/sin table, built in double and rounded to float:
// table[((axis * maxpos) + pos) * pairs + m] = (cos, sin)(pos * omega_m),
// omega_m = theta^(-2m / (2 * pairs)), axis 0 = patch row, 1 = patch column;
// interleaved: columns take omega_m = theta^(-(2m + 1) / (2 * pairs)).
void build_rope_table(double theta, int32_t pairs, int32_t maxpos, bool interleaved, std::vector<float>* out);

}  // namespace pv
