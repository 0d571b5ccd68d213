// Per-row index maps of a packed batch, built on the device from the per-image
// metadata the host uploads ("Mistral 3" (KerasFormers), Mistral3VisionModel:
// all images in one patch sequence; "Several images in one conversation":
// each image keeps its own patch count).  These are the maps every hot kernel
// reads: the patch embedding's im2col rows, the rotary positions and the 2x2
// merge gather.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

// Largest image index i with key(i) <= x (key non-decreasing, key(0) = 0).
template <typename Key>
__device__ __forceinline__ int find_image(int n, int x, Key key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (key(mid) <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void rowinfo_kernel(const ImageMeta* __restrict__ meta, int n_images,
                                                      int n_patches, int32_t* __restrict__ rowinfo) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= n_patches) return;
  // an image with zero patches cannot occur (sides are >= one patch), so the
  // search over patch_base is exact
  const int i = find_image(n_images, g, [&](int k) { return meta[k].patch_base; });
  const int j = g - meta[i].patch_base;
  const int wp = meta[i].Wp;
  const int r = j / wp, c = j - r * wp;
  rowinfo[2 * g] = i;
  rowinfo[2 * g + 1] = (r << 16) | c;
}

__global__ __launch_bounds__(256) void msrc_kernel(const ImageMeta* __restrict__ meta, int n_images,
                                                   int out_rows, int32_t* __restrict__ msrc) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= out_rows) return;
  const int i = find_image(n_images, t, [&](int k) { return meta[k].tok_base; });
  const ImageMeta m = meta[i];
  const int local = t - m.tok_base;
  const int hw = m.Wp >> 1;
  const int R = local / hw, C = local - R * hw;
  const int s0 = m.patch_base + (2 * R) * m.Wp + 2 * C;
  int4 v;
  v.x = s0;
  v.y = s0 + 1;
  v.z = s0 + m.Wp;
  v.w = s0 + m.Wp + 1;
  reinterpret_cast<int4*>(msrc)[t] = v;
}

__global__ __launch_bounds__(256) void export_kernel(const ImageMeta* __restrict__ meta,
                                                     const int32_t* __restrict__ rowinfo, int n_images,
                                                     int n_patches, int32_t* __restrict__ cu,
                                                     int32_t* __restrict__ rc) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g <= n_images && g >= 0) cu[g] = (g == n_images) ? n_patches : meta[g].patch_base;
  if (g < n_patches) {
    const int v = rowinfo[2 * g + 1];
    rc[2 * g] = v >> 16;
    rc[2 * g + 1] = v & 0xffff;
  }
}

}  // namespace

hipError_t build_maps(const ImageMeta* meta, int n_images, int n_patches, int out_rows, int merge,
                      int32_t* rowinfo, int32_t* msrc, hipStream_t s) {
  hipLaunchKernelGGL(rowinfo_kernel, dim3((n_patches + 255) / 256), dim3(256), 0, s, meta, n_images, n_patches,
                     rowinfo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || merge != 2 || out_rows == 0) return e;
  hipLaunchKernelGGL(msrc_kernel, dim3((out_rows + 255) / 256), dim3(256), 0, s, meta, n_images, out_rows, msrc);
  return hipGetLastError();
}

hipError_t export_maps(const ImageMeta* meta, const int32_t* rowinfo, int n_images, int n_patches,
                       int32_t* cu_seqlens, int32_t* patch_rc, hipStream_t s) {
  const int n = (n_patches > n_images + 1 ? n_patches : n_images + 1);
  hipLaunchKernelGGL(export_kernel, dim3((n + 255) / 256), dim3(256), 0, s, meta, rowinfo, n_images, n_patches,
                     cu_seqlens, patch_rc);
  return hipGetLastError();
}

}  // namespace pv
