// Host planner; see plan.h.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <numeric>

namespace pv {

namespace {
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace
// Queries per attention work item.  The wide item is taken when the work
// items of all heads fill the chip's rounds of workgroups at least 0.1
// better (by count) and pad the images' query ranges no more: at 1540^2,
// 768 items of 256 queries leave the second of two rounds of 512 half
// empty, while 512 items of 384 fill two rounds of 256 (measured 2% faster);
// mixed small images keep the 256-query items (less padding).
static int32_t choose_q_tile(const PlanParams& p, const std::vector<int32_t>& cu) {
  if (p.q_tile_wide <= 0) return p.q_tile;
  auto stats = [&](int32_t q, int32_t slots, double& fill, int64_t& padded) {
    int64_t items = 0;
    padded = 0;
    for (size_t i = 0; i + 1 < cu.size(); ++i) {
      const int64_t n = cu[i + 1] - cu[i], k = (n + q - 1) / q;
      items += k;
      padded += k * q;
    }
    items *= p.heads;
    const int64_t rounds = (items + slots - 1) / slots;
    fill = rounds > 0 ? double(items) / double(rounds * slots) : 1.0;
  };
  double f_n, f_w;
  int64_t pad_n, pad_w;
  stats(p.q_tile, p.slots, f_n, pad_n);
  stats(p.q_tile_wide, p.slots_wide, f_w, pad_w);
  return (f_w >= f_n + 0.1 && pad_w <= pad_n) ? p.q_tile_wide : p.q_tile;
}

int build_plan(const PlanParams& p, const int32_t* image_hw, int32_t n_images, Plan* out,
               std::string* err) {
  if (!image_hw || !out) {
    *err = "image_hw and plan must not be null";
    return -1;
  }
  if (n_images < 1) {
    *err = "n_images must be >= 1 (the tower runs only on image input)";
    return -1;
  }
  const int64_t grid = int64_t(p.patch) * p.merge;
  Plan& pl = *out;
  pl = Plan();
  pl.n_images = n_images;
  pl.meta.resize(n_images);
  pl.cu.assign(n_images + 1, 0);
  int64_t patches = 0, toks = 0, pix = 0;
  int32_t maxp = 0, maxside_p = 0;
  for (int32_t i = 0; i < n_images; ++i) {
    const int32_t H = image_hw[2 * i], W = image_hw[2 * i + 1];
    if (H <= 0 || W <= 0 || H % grid || W % grid || H > p.max_side || W > p.max_side) {
      *err = "image " + std::to_string(i) + " is " + std::to_string(H) + "x" + std::to_string(W) +
             ": each side must be a positive multiple of " + std::to_string(grid) +
             " and at most " + std::to_string(p.max_side);
      return -2;
    }
    ImageMeta& m = pl.meta[i];
    m.H = H;
    m.W = W;
    m.Hp = H / p.patch;
    m.Wp = W / p.patch;
    m.patch_base = int32_t(patches);
    m.tok_base = int32_t(toks);
    m.pix_lo = uint32_t(uint64_t(pix) & 0xffffffffu);
    m.pix_hi = uint32_t(uint64_t(pix) >> 32);
    const int64_t n = int64_t(m.Hp) * m.Wp;
    patches += n;
    toks += (p.merge == 2) ? (n / 4) : n;
    pix += int64_t(3) * H * W;
    maxp = std::max<int32_t>(maxp, int32_t(n));
    maxside_p = std::max(maxside_p, std::max(m.Hp, m.Wp));
    pl.cu[i + 1] = int32_t(patches);
    if (patches > (int64_t(1) << 30)) {
      *err = "too many patches in one call (limit 2^30)";
      return -2;
    }
  }
  pl.n_patches = patches;
  pl.out_rows = toks;
  pl.max_patches = maxp;
  pl.rope_maxpos = std::max(1, p.max_side / p.patch);

  // Attention work list: q-tiles of every image, longest images first so the
  // heaviest work items start earliest (longest-processing-time order).
  std::vector<int32_t> order(n_images);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return (pl.cu[a + 1] - pl.cu[a]) > (pl.cu[b + 1] - pl.cu[b]);
  });
  pl.q_tile = choose_q_tile(p, pl.cu);
  for (int32_t i : order) {
    const int32_t n = pl.cu[i + 1] - pl.cu[i];
    for (int32_t q0 = 0; q0 < n; q0 += pl.q_tile) pl.items.push_back({i, q0});
  }

  // Workspace layout.
  Layout& L = pl.ws;
  size_t off = 0;
  L.meta = off;
  off = align256(off + sizeof(ImageMeta) * n_images);
  // (sized for the larger of the two item counts, so that the workspace of
  // a subset of the images never exceeds that of the whole set)
  size_t items_cap = pl.items.size();
  for (int32_t q : {p.q_tile, p.q_tile_wide}) {
    if (q <= 0) continue;
    size_t k = 0;
    for (int32_t i = 0; i < n_images; ++i) k += size_t((pl.cu[i + 1] - pl.cu[i] + q - 1) / q);
    items_cap = std::max(items_cap, k);
  }
  L.items = off;
  off = align256(off + sizeof(AttnItem) * items_cap);
  L.rope = off;
  off = align256(off + sizeof(float) * 2 * 2 * size_t(pl.rope_maxpos) * p.rope_pairs);
  L.src = off;
  off = align256(off + sizeof(SrcImage) * n_images);
  L.upload_bytes = off;
  L.rowinfo = off;
  off = align256(off + sizeof(int32_t) * 2 * size_t(patches));
  L.msrc = off;
  off = align256(off + (p.merge == 2 ? sizeof(int32_t) * 4 * size_t(toks) : 0));
  const size_t N = size_t(patches), D = size_t(p.hidden);
  L.r = off;
  off = align256(off + N * D * 4);
  L.y = off;
  off = align256(off + N * D * p.elem_bytes);
  L.big = off;  // also: im2col hi | lo [N][2 Kp] and the final residual's hi | lo [N][2D] (bf16 tower)
  size_t big_row = std::max(3 * D, size_t(p.mlp)) * p.elem_bytes;
  if (p.elem_bytes == 2) big_row = std::max(big_row, std::max(size_t(4) * patch_kp(p.patch), 4 * D));
  // fp32 tower from uint8 input: the resized, normalised planes (3 p^2 fp32 per patch)
  if (p.elem_bytes == 4) big_row = std::max(big_row, size_t(12) * p.patch * p.patch);
  size_t big_bytes = N * big_row;
  if (p.deep_out > 0) big_bytes = std::max(big_bytes, size_t(toks) * size_t(p.deep_out) * 2);
  off = align256(off + big_bytes);
  L.wpad = off;
  off = align256(off + (p.elem_bytes == 2 && !p.prepared ? D * size_t(patch_kp(p.patch)) * 2 : 0));
  if (p.elem_bytes == 2) {
    // fp8 variant: every fp8 GEMM input (up to [N][max(D, F)]) and its scale
    // bytes; merge == 2: the merger input's fp4 low part [T][2D] and its scale
    // bytes
    size_t a8_bytes = 0, as_bytes = 0;
    if (p.fp8) {
      const size_t KA = std::max(D, size_t(p.mlp));
      a8_bytes = N * KA;
      as_bytes = (KA / 128) * size_t(a8_scale_rows(int64_t(N))) * 4;
    }
    if (p.merge_rows > 0) {
      a8_bytes = std::max(a8_bytes, size_t(toks) * 2 * D);
      as_bytes = std::max(as_bytes, (D / 64) * size_t(a8_scale_rows(int64_t(toks))) * 8);
    }
    L.a8 = off;
    off = align256(off + a8_bytes);
    L.as = off;
    off = align256(off + as_bytes);
  }
  if (p.elem_bytes == 2 && !p.prepared && p.merge_rows > 0) {
    L.mw4 = off;
    off = align256(off + merge_fp4_bytes(p.merge_rows, p.hidden));
    L.mws = off;
    off = align256(off + merge_fp4_scale_bytes(p.merge_rows, p.hidden));
  }
  if (p.elem_bytes == 2 && !p.prepared) {
    // this layer's gate/up weights: fp16 [2F][D] (bf16 tower), or fp8 [2F][D]
    // and its scale bytes (fp8 variant); bf16 tower: the down weights in
    // fp16 [D][F]
    const size_t F = size_t(p.mlp), F2 = 2 * F;
    L.b8 = off;
    off = align256(off + F2 * D * (p.fp8 ? 1 : 2));
    L.bs = off;
    off = align256(off + (p.fp8 ? (D / 128) * F2 * 4 : 0));
    if (!p.fp8) {
      L.wd8 = off;
      off = align256(off + D * F * 2);
      L.wds = off;
    }
    if (p.fp8) {
      L.wq8 = off;
      off = align256(off + 3 * D * D);
      L.wqs = off;
      off = align256(off + (D / 128) * 3 * D * 4);
      L.wo8 = off;
      off = align256(off + D * D);
      L.wos = off;
      off = align256(off + (D / 128) * D * 4);
      L.wd8 = off;
      off = align256(off + D * F);
      L.wds = off;
      off = align256(off + (F / 128) * D * 4);
    }
  }
  L.total = off;
  return 0;
}

PrepLayout prep_layout(int32_t patch, int32_t hidden, int32_t mlp, int32_t layers, bool fp8, int32_t merge_rows) {
  PrepLayout P;
  const size_t D = size_t(hidden), F = size_t(mlp), F2 = 2 * F;
  size_t off = 0;
  P.wpad = off;
  off = align256(off + D * size_t(patch_kp(patch)) * 2);
  P.layer0 = off;
  size_t lo = 0;
  if (fp8) {
    P.wq8 = lo;
    lo = align256(lo + 3 * D * D);
    P.wqs = lo;
    lo = align256(lo + (D / 128) * 3 * D * 4);
    P.wo8 = lo;
    lo = align256(lo + D * D);
    P.wos = lo;
    lo = align256(lo + (D / 128) * D * 4);
    P.b8 = lo;
    lo = align256(lo + F2 * D);
    P.bs = lo;
    lo = align256(lo + (D / 128) * F2 * 4);
    P.wd8 = lo;
    lo = align256(lo + D * F);
    P.wds = lo;
    lo = align256(lo + (F / 128) * D * 4);
  } else {  // fp16: gate rows, then up rows; the down weights
    P.b8 = lo;
    lo = align256(lo + F2 * D * 2);
    P.bs = lo;
    P.wd8 = lo;
    lo = align256(lo + D * F * 2);
    P.wds = lo;
  }
  P.layer_stride = lo;
  off += size_t(layers > 0 ? layers : 0) * lo;
  if (merge_rows > 0) {
    P.mw4 = off;
    off = align256(off + merge_fp4_bytes(merge_rows, hidden));
    P.mws = off;
    off = align256(off + merge_fp4_scale_bytes(merge_rows, hidden));
  }
  P.total = off;
  return P;
}

int resize_target(int32_t h, int32_t w, int32_t longest_edge, int32_t grid, int32_t* th, int32_t* tw,
                  std::string* err) {
  if (grid < 1 || longest_edge < grid) {
    *err = "grid must be >= 1 and longest_edge >= grid";
    return -1;
  }
  if (h < 1 || w < 1 || h > kMaxSrcSide || w > kMaxSrcSide) {
    *err = "source image " + std::to_string(h) + "x" + std::to_string(w) + ": each side must be in [1, " +
           std::to_string(kMaxSrcSide) + "]";
    return -2;
  }
  const int64_t L = longest_edge, g = grid, m = std::max(h, w);
  int64_t a = h, b = w;
  if (m > L) {  // fit: shrink so the longest side is longest_edge
    a = std::max<int64_t>(1, a * L / m);
    b = std::max<int64_t>(1, b * L / m);
  }
  const int64_t cap = L / g * g;  // then onto the grid
  *th = int32_t(std::min((a + g - 1) / g * g, cap));
  *tw = int32_t(std::min((b + g - 1) / g * g, cap));
  return 0;
}

int tile_layout(int32_t h, int32_t w, int32_t tile, int32_t grid, int32_t max_num_tiles, int32_t* rh,
                int32_t* rw, int32_t* rows, int32_t* cols, std::string* err) {
  if (grid < 1 || tile < grid || tile % grid || tile > kMaxSrcSide || max_num_tiles < 1 ||
      max_num_tiles > kMaxTiles) {
    *err = "tile must be a multiple of grid (>= 1, <= " + std::to_string(kMaxSrcSide) +
           ") and max_num_tiles in [1, " + std::to_string(kMaxTiles) + "]";
    return -1;
  }
  if (h < 1 || w < 1 || h > kMaxSrcSide || w > kMaxSrcSide) {
    *err = "source image " + std::to_string(h) + "x" + std::to_string(w) + ": each side must be in [1, " +
           std::to_string(kMaxSrcSide) + "]";
    return -2;
  }
  // best scale as a fraction num / den: for each row count r the widest
  // grid r x floor(M / r) is the best one with r rows
  int64_t num = 0, den = 1;
  for (int64_t r = 1; r <= max_num_tiles; ++r) {
    const int64_t c = max_num_tiles / r;
    int64_t n = r * tile, d = h;                       // r * tile / h
    if (c * tile * int64_t(h) < n * int64_t(w)) {      // c * tile / w is smaller
      n = c * tile;
      d = w;
    }
    if (n * den > num * d) {
      num = n;
      den = d;
    }
  }
  if (num >= den) {  // never enlarged
    num = 1;
    den = 1;
  }
  const int64_t g = grid;
  const int64_t a = std::max<int64_t>(1, int64_t(h) * num / den);
  const int64_t b = std::max<int64_t>(1, int64_t(w) * num / den);
  *rh = int32_t((a + g - 1) / g * g);
  *rw = int32_t((b + g - 1) / g * g);
  *rows = (*rh + tile - 1) / tile;
  *cols = (*rw + tile - 1) / tile;
  return 0;
}

void host_index_maps(const Plan& pl, int merge, int32_t* cu, int32_t* rc, int32_t* msrc) {
  for (int32_t i = 0; i <= pl.n_images; ++i) cu[i] = pl.cu[i];
  for (int32_t i = 0; i < pl.n_images; ++i) {
    const ImageMeta& m = pl.meta[i];
    for (int32_t j = 0; j < m.Hp * m.Wp; ++j) {
      rc[2 * (int64_t(m.patch_base) + j)] = j / m.Wp;
      rc[2 * (int64_t(m.patch_base) + j) + 1] = j % m.Wp;
    }
    if (merge == 2 && msrc) {
      const int32_t hw = m.Wp / 2;
      for (int32_t t = 0; t < (m.Hp / 2) * hw; ++t) {
        const int32_t R = t / hw, C = t % hw;
        int32_t* s = msrc + 4 * (int64_t(m.tok_base) + t);
        s[0] = m.patch_base + (2 * R) * m.Wp + 2 * C;
        s[1] = s[0] + 1;
        s[2] = s[0] + m.Wp;
        s[3] = s[2] + 1;
      }
    }
  }
}

void build_rope_table(double theta, int32_t pairs, int32_t maxpos, bool interleaved, std::vector<float>* out) {
  out->assign(size_t(2) * 2 * maxpos * pairs, 0.f);
  for (int axis = 0; axis < 2; ++axis)
    for (int32_t pos = 0; pos < maxpos; ++pos)
      for (int32_t m = 0; m < pairs; ++m) {
        // step j of the ladder theta^(-j / (2 pairs)): 2m on both axes, or 2m
        // on rows and 2m + 1 on columns (interleaved)
        const int j = 2 * m + (interleaved && axis == 1 ? 1 : 0);
        const double omega = std::pow(theta, -double(j) / (2.0 * pairs));
        const double a = double(pos) * omega;
        const size_t idx = ((size_t(axis) * maxpos + pos) * pairs + m) * 2;
        (*out)[idx] = float(std::cos(a));
        (*out)[idx + 1] = float(std::sin(a));
      }
}

}  // namespace pv
