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

// Power-of-two scale of a block of 32 values for fp8 e4m3 (max normal 448):
// the exponent X = floor(log2(max|x|)) - 7 puts the block maximum in
// [128, 256), clear of the top of the range.  Returns the E8M0 byte X + 127
// and sets mul = 2^-X.
__device__ __forceinline__ uint32_t mx_scale(float amax, float& mul) {
  const int e = int((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xff);  // biased exponent of the max
  int x = e - 127 - 7;
  x = x < -120 ? -120 : (x > 120 ? 120 : x);
  mul = __builtin_bit_cast(float, uint32_t(127 - x) << 23);
  return uint32_t(x + 127);
}

// Four fp32 values -> four fp8 e4m3 bytes (round to nearest even).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return uint32_t(r);
}

// The MLP input: y = norm(x) * g as bf16 hi [N][D], and its low part y - hi
// as packed fp4 [N][D/2] (low nibble = even column) with one scale byte per
// 32 columns, scale bytes step-major: ys[(col / 256) * srows + row][(col / 32) % 8].
template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_hi_lo4_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                             uint16_t* __restrict__ yh, uint8_t* __restrict__ y4,
                                                             uint8_t* __restrict__ ys, int rows, int srows, float eps) {
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
  for (int i = 0; i < NC; ++i) {
    v[i] = v[i] * inv * gr[i * 64 + lane];
    const int col = (i * 64 + lane) * 4;
    u32x2 hi;
    hi[0] = pack_bf16x2(v[i][0], v[i][1]);
    hi[1] = pack_bf16x2(v[i][2], v[i][3]);
    *reinterpret_cast<u32x2*>(yh + size_t(row) * D + col) = hi;
    const float l0 = v[i][0] - lo_bf16(hi[0]), l1 = v[i][1] - hi_bf16(hi[0]);
    const float l2 = v[i][2] - lo_bf16(hi[1]), l3 = v[i][3] - hi_bf16(hi[1]);
    // block of 32 columns = 8 consecutive lanes
    float amax = fmaxf(fmaxf(fabsf(l0), fabsf(l1)), fmaxf(fabsf(l2), fabsf(l3)));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    float scale;
    const uint32_t sbyte = mx_scale4(amax, scale);
    *reinterpret_cast<uint16_t*>(y4 + size_t(row) * (D / 2) + col / 2) = uint16_t(pack_fp4x4(l0, l1, l2, l3, scale));
    if ((lane & 7) == 0) {
      const int blk = col / 32;
      ys[(size_t(blk / 8) * srows + row) * 8 + (blk & 7)] = uint8_t(sbyte);
    }
  }
}

// The input of an fp8 linear map: y = norm(x) * g as fp8 e4m3 [N][D] with
// one scale byte per 32 columns (same scale layout as above).
template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_fp8_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                          uint8_t* __restrict__ y8, uint8_t* __restrict__ ys, int rows,
                                                          int srows, float eps) {
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
  for (int i = 0; i < NC; ++i) {
    v[i] = v[i] * inv * gr[i * 64 + lane];
    const int col = (i * 64 + lane) * 4;
    float amax = fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    float mul;
    const uint32_t sbyte = mx_scale(amax, mul);
    *reinterpret_cast<uint32_t*>(y8 + size_t(row) * D + col) =
        pack_fp8x4(v[i][0] * mul, v[i][1] * mul, v[i][2] * mul, v[i][3] * mul);
    if ((lane & 7) == 0) {
      const int blk = col / 32;
      ys[(size_t(blk / 4) * srows + row) * 4 + (blk & 3)] = uint8_t(sbyte);
    }
  }
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

hipError_t rmsnorm_hi_lo4(const float* x, const float* g, void* yh, void* y4, void* ys, int rows, int srows, int D,
                          float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D % 256 || srows < rows) return hipErrorInvalidValue;
  const dim3 grid((rows + 3) / 4), block(256);
#define PV_CASE(NC)                                                                                    \
  if (D == NC * 256) {                                                                                 \
    hipLaunchKernelGGL((rmsnorm_hi_lo4_kernel<NC>), grid, block, 0, s, x, g, static_cast<uint16_t*>(yh), \
                       static_cast<uint8_t*>(y4), static_cast<uint8_t*>(ys), rows, srows, eps);           \
    return hipGetLastError();                                                                          \
  }
  PV_NORM_CASES(PV_CASE)
#undef PV_CASE
  return hipErrorInvalidValue;
}

hipError_t rmsnorm_fp8(const float* x, const float* g, void* y8, void* ys, int rows, int srows, int D, float eps,
                       hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D % 128 || srows < rows) return hipErrorInvalidValue;
  const dim3 grid((rows + 3) / 4), block(256);
#define PV_CASE(NC)                                                                                   \
  if (D == NC * 256) {                                                                                \
    hipLaunchKernelGGL((rmsnorm_fp8_kernel<NC>), grid, block, 0, s, x, g, static_cast<uint8_t*>(y8),    \
                       static_cast<uint8_t*>(ys), rows, srows, eps);                                  \
    return hipGetLastError();                                                                         \
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
