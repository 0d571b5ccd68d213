// RMSNorm passes of the tower ("Mistral 3" (KerasFormers),
// Mistral3VisionModel: RMS pre-norm after the patch embedding and pre-norm
// blocks): y = x / sqrt(mean(x^2) + eps) * g.
//
// One wavefront per row; each lane holds D/64 values as float4 chunks laid
// out so one load instruction covers 1 KiB of contiguous row.  The residual
// stream x is fp32; y is bf16 (or fp32 for the fp32 tower).  These passes are
// HBM-bound: 4 bytes read + 2 (4) bytes written per element, 8 + 2 (4) for the
// dual pass.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

template <int NC>
__device__ __forceinline__ float sumsq(const floatx4 (&v)[NC]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) s += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
  return wave_sum(s);
}

template <int NC, bool YF32>
__device__ __forceinline__ void store_row(void* y, size_t row, int D, int lane, const floatx4 (&v)[NC]) {
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const size_t o = row * D + size_t(i * 64 + lane) * 4;
    if constexpr (YF32) {
      *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(y) + o) = v[i];
    } else {
      u32x2 p;
      p[0] = pack_bf16x2(v[i][0], v[i][1]);
      p[1] = pack_bf16x2(v[i][2], v[i][3]);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(y) + o) = p;
    }
  }
}

// bf16 hi and lo = bf16(v - hi) of a row, stored as [hi (D) | lo (D)]: a
// product over both halves carries about 16 significant bits of v.
template <int NC>
__device__ __forceinline__ void store_row_split(void* y, size_t row, int D, int lane, const floatx4 (&v)[NC]) {
  uint16_t* yr = reinterpret_cast<uint16_t*>(y) + row * 2 * D;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const size_t o = size_t(i * 64 + lane) * 4;
    u32x2 hi, lo;
    hi[0] = pack_bf16x2(v[i][0], v[i][1]);
    hi[1] = pack_bf16x2(v[i][2], v[i][3]);
    lo[0] = pack_bf16x2(v[i][0] - lo_bf16(hi[0]), v[i][1] - hi_bf16(hi[0]));
    lo[1] = pack_bf16x2(v[i][2] - lo_bf16(hi[1]), v[i][3] - hi_bf16(hi[1]));
    *reinterpret_cast<u32x2*>(yr + o) = hi;
    *reinterpret_cast<u32x2*>(yr + D + o) = lo;
  }
}

template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_split_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                            void* __restrict__ y, int rows, float eps) {
  constexpr int D = NC * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const floatx4* xr = reinterpret_cast<const floatx4*>(x + size_t(row) * D);
  const floatx4* gr = reinterpret_cast<const floatx4*>(g);
  floatx4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = xr[i * 64 + lane];
  const float inv = rsqrtf(sumsq<NC>(v) * (1.f / D) + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = v[i] * inv * gr[i * 64 + lane];
  store_row_split<NC>(y, row, D, lane, v);
}

template <int NC, bool YF32>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                      void* __restrict__ y, int rows, float eps) {
  constexpr int D = NC * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const floatx4* xr = reinterpret_cast<const floatx4*>(x + size_t(row) * D);
  const floatx4* gr = reinterpret_cast<const floatx4*>(g);
  floatx4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = xr[i * 64 + lane];
  const float inv = rsqrtf(sumsq<NC>(v) * (1.f / D) + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = v[i] * inv * gr[i * 64 + lane];
  store_row<NC, YF32>(y, row, D, lane, v);
}

template <int NC, bool YF32>
__global__ __launch_bounds__(256) void rmsnorm_dual_kernel(float* __restrict__ x, const float* __restrict__ g1,
                                                           const float* __restrict__ g2, void* __restrict__ y,
                                                           int rows, float eps) {
  constexpr int D = NC * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  floatx4* xr = reinterpret_cast<floatx4*>(x + size_t(row) * D);
  const floatx4* g1r = reinterpret_cast<const floatx4*>(g1);
  const floatx4* g2r = reinterpret_cast<const floatx4*>(g2);
  floatx4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = xr[i * 64 + lane];
  const float inv1 = rsqrtf(sumsq<NC>(v) * (1.f / D) + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    v[i] = v[i] * inv1 * g1r[i * 64 + lane];
    xr[i * 64 + lane] = v[i];
  }
  const float inv2 = rsqrtf(sumsq<NC>(v) * (1.f / D) + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = v[i] * inv2 * g2r[i * 64 + lane];
  store_row<NC, YF32>(y, row, D, lane, v);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ x, uint32_t* __restrict__ y,
                                                          size_t npairs) {
  for (size_t i = blockIdx.x * size_t(256) + threadIdx.x; i < npairs; i += size_t(gridDim.x) * 256) {
    const float2 v = reinterpret_cast<const float2*>(x)[i];
    y[i] = pack_bf16x2(v.x, v.y);
  }
}

}  // namespace

#define PV_NORM_CASES(MACRO) MACRO(1) MACRO(2) MACRO(3) MACRO(4) MACRO(6) MACRO(8)

hipError_t rmsnorm(const float* x, const float* g, void* y, int rows, int D, float eps, bool y_f32,
                   hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
#define PV_CASE(NC)                                                                               \
  if (D == NC * 256) {                                                                            \
    if (y_f32) hipLaunchKernelGGL((rmsnorm_kernel<NC, true>), grid, block, 0, s, x, g, y, rows, eps); \
    else hipLaunchKernelGGL((rmsnorm_kernel<NC, false>), grid, block, 0, s, x, g, y, rows, eps);     \
    return hipGetLastError();                                                                     \
  }
  PV_NORM_CASES(PV_CASE)
#undef PV_CASE
  return hipErrorInvalidValue;
}

hipError_t rmsnorm_split(const float* x, const float* g, void* y, int rows, int D, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
#define PV_CASE(NC)                                                                       \
  if (D == NC * 256) {                                                                    \
    hipLaunchKernelGGL((rmsnorm_split_kernel<NC>), grid, block, 0, s, x, g, y, rows, eps); \
    return hipGetLastError();                                                             \
  }
  PV_NORM_CASES(PV_CASE)
#undef PV_CASE
  return hipErrorInvalidValue;
}

hipError_t rmsnorm_dual(float* x, const float* g1, const float* g2, void* y, int rows, int D, float eps,
                        bool y_f32, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
#define PV_CASE(NC)                                                                                         \
  if (D == NC * 256) {                                                                                      \
    if (y_f32) hipLaunchKernelGGL((rmsnorm_dual_kernel<NC, true>), grid, block, 0, s, x, g1, g2, y, rows, eps); \
    else hipLaunchKernelGGL((rmsnorm_dual_kernel<NC, false>), grid, block, 0, s, x, g1, g2, y, rows, eps);     \
    return hipGetLastError();                                                                               \
  }
  PV_NORM_CASES(PV_CASE)
#undef PV_CASE
  return hipErrorInvalidValue;
}

hipError_t f32_to_bf16(const float* x, void* y, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t pairs = n / 2;  // n is a multiple of 256 here
  const size_t blocks = (pairs + 255) / 256;
  const unsigned grid = unsigned(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(grid), dim3(256), 0, s, x, reinterpret_cast<uint32_t*>(y), pairs);
  return hipGetLastError();
}

}  // namespace pv
