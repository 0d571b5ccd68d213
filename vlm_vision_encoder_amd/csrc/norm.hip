// RMSNorm passes of the tower ("Mistral 3" (KerasFormers),
// Mistral3VisionModel: RMS pre-norm after the patch embedding and pre-norm
// blocks): y = x / sqrt(mean(x^2) + eps) * g.
//
// One wavefront per row; each lane holds D/64 values as float4 chunks laid
// out so one load instruction covers 1 KiB of contiguous row.  The residual
// stream x is fp32; y is bf16 (fp16 for the MLP input of the bf16 tower,
// fp32 for the fp32 tower).  These passes are HBM-bound: 4 bytes read + 2 (4)
// bytes written per element, 8 + 2 (4) for the dual pass.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

// Sum over the 64 lanes, in every lane: DPP moves inside each 16-lane row
// (quad permutes [1,0,3,2] and [2,3,0,1], half-row mirror, row mirror: no
// LDS traffic, a few cycles each), then two lane exchanges across rows.
__device__ __forceinline__ float row_sum64(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

template <int NC>
__device__ __forceinline__ float sumsq(const floatx4 (&v)[NC]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) s += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
  return row_sum64(s);
}

// Output element types of the norm passes.
enum NormOut { OUT_BF16 = 0, OUT_F32 = 1, OUT_F16 = 2 };

template <int NC, int YT>
__device__ __forceinline__ void store_row(void* y, size_t row, int D, int lane, const floatx4 (&v)[NC]) {
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const size_t o = row * D + size_t(i * 64 + lane) * 4;
    if constexpr (YT == OUT_F32) {
      *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(y) + o) = v[i];
    } else if constexpr (YT == OUT_F16) {
      u32x2 p;
      p[0] = pack_f16x2_sat(v[i][0], v[i][1]);
      p[1] = pack_f16x2_sat(v[i][2], v[i][3]);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(y) + o) = p;
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

// Maximum over the 8 lanes of v's aligned 8-lane group, by DPP moves (no
// LDS traffic): quad permutes [1,0,3,2] and [2,3,0,1], then the half-row
// mirror (lane i of 8 takes lane 7 - i, pairing the two quads).
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)));
  return v;
}

// Four consecutive 32-column scale bytes (lanes 8b..8b+7 hold block b's
// byte) combined into one little-endian word, valid in lanes 0 and 32 (and
// every lane of their 32-lane half).
__device__ __forceinline__ uint32_t scale_word(uint32_t sbyte, int lane) {
  uint32_t w = (sbyte & 0xffu) << (8 * ((lane >> 3) & 3));
  w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x128, 0xF, 0xF, true));  // row_ror:8 (lane ^ 8 in a 16-lane row)
  w |= uint32_t(__shfl_xor(int(w), 16, 64));
  return w;
}

// The merger's input (the final residual, fp32 [N][D]) as bf16 hi rows plus
// the low part x - hi in fp4 e2m1, the low part already in the merged
// tokens' order: workgroup t (one merged token), wave j (window slot j)
// takes source row src = msrc[t][j] and writes
//   yh [src][D]                     bf16 hi (row-major per patch: the GEMM's
//                                   2x2 gather reads it)
//   y4 [t][4D/2], k = j D + col     fp4 low part, low nibble = even k
//   ys [(4D/256)][srows][8]         one E8M0 byte per 32 k, step-major
// so that the low-part operand of the merge GEMM is dense [T][4D].
template <int NC>
__global__ __launch_bounds__(256) void merge_hi_lo4_kernel(const float* __restrict__ x, const int32_t* __restrict__ msrc,
                                                           uint16_t* __restrict__ yh, uint8_t* __restrict__ y4,
                                                           uint8_t* __restrict__ ys, int tokens, int srows) {
  constexpr int D = NC * 256;
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int t = blockIdx.x;
  if (t >= tokens) return;
  const int src = msrc[4 * t + j];
  const floatx4* xr = reinterpret_cast<const floatx4*>(x + size_t(src) * D);
  // all of the row's loads first: one memory round trip per wave instead of
  // one per 256 columns
  floatx4 vr[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) vr[i] = xr[i * 64 + lane];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const floatx4 v = vr[i];
    const int col = (i * 64 + lane) * 4;
    u32x2 hi;
    hi[0] = pack_bf16x2(v[0], v[1]);
    hi[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(yh + size_t(src) * D + col) = hi;
    const float l0 = v[0] - lo_bf16(hi[0]), l1 = v[1] - hi_bf16(hi[0]);
    const float l2 = v[2] - lo_bf16(hi[1]), l3 = v[3] - hi_bf16(hi[1]);
    const float amax = max8(fmaxf(fmaxf(fabsf(l0), fabsf(l1)), fmaxf(fabsf(l2), fabsf(l3))));
    float scale;
    const uint32_t sbyte = mx_scale4(amax, scale);
    *reinterpret_cast<uint16_t*>(y4 + size_t(t) * (2 * D) + (j * D + col) / 2) =
        uint16_t(pack_fp4x4(l0, l1, l2, l3, scale));
    const uint32_t w = scale_word(sbyte, lane);
    if ((lane & 31) == 0)
      *reinterpret_cast<uint32_t*>(ys + (size_t(j * NC + i) * srows + t) * 8 + (lane >> 3)) = w;
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
  floatx4 v[NC], gv[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = xr[i * 64 + lane];
#pragma unroll
  for (int i = 0; i < NC; ++i) gv[i] = gr[i * 64 + lane];
  const float inv = rsqrtf(sumsq<NC>(v) * (1.f / D) + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    v[i] = v[i] * inv * gv[i];
    const int col = (i * 64 + lane) * 4;
    const float amax = max8(fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3]))));
    float mul;
    const uint32_t sbyte = mx_scale(amax, mul);
    *reinterpret_cast<uint32_t*>(y8 + size_t(row) * D + col) =
        pack_fp8x4(v[i][0] * mul, v[i][1] * mul, v[i][2] * mul, v[i][3] * mul);
    // the 4 scale bytes of each 128-column step as one word: lanes 0-31
    // hold step 2i, lanes 32-63 step 2i + 1
    const uint32_t w = scale_word(sbyte, lane);
    if ((lane & 31) == 0) *reinterpret_cast<uint32_t*>(ys + (size_t(2 * i + (lane >> 5)) * srows + row) * 4) = w;
  }
}

// One row per wave; YT: NormOut.
template <int NC, int YT>
__device__ __forceinline__ void rmsnorm_rows(const float* __restrict__ x, const float* __restrict__ g,
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
  store_row<NC, YT>(y, row, D, lane, v);
}

template <int NC, bool YF32>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                      void* __restrict__ y, int rows, float eps) {
  rmsnorm_rows<NC, YF32 ? OUT_F32 : OUT_BF16>(x, g, y, rows, eps);
}

// The MLP input of the bf16 tower in fp16 (saturated to +-65504: |y| is at
// most sqrt(D) max|g|, since no value of a row exceeds sqrt(D) times its RMS).
template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_f16_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                          void* __restrict__ y, int rows, float eps) {
  rmsnorm_rows<NC, OUT_F16>(x, g, y, rows, eps);
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
  store_row<NC, YF32 ? OUT_F32 : OUT_BF16>(y, row, D, lane, v);
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

hipError_t rmsnorm_f16(const float* x, const float* g, void* y, int rows, int D, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
#define PV_CASE(NC)                                                                        \
  if (D == NC * 256) {                                                                     \
    hipLaunchKernelGGL((rmsnorm_f16_kernel<NC>), grid, block, 0, s, x, g, y, rows, eps); \
    return hipGetLastError();                                                              \
  }
  PV_NORM_CASES(PV_CASE)
#undef PV_CASE
  return hipErrorInvalidValue;
}

hipError_t merge_hi_lo4(const float* x, const int32_t* msrc, void* yh, void* y4, void* ys, int tokens, int srows,
                        int D, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  if (D % 256 || srows < tokens) return hipErrorInvalidValue;
#define PV_CASE(NC)                                                                                     \
  if (D == NC * 256) {                                                                                  \
    hipLaunchKernelGGL((merge_hi_lo4_kernel<NC>), dim3(tokens), dim3(256), 0, s, x, msrc,               \
                       static_cast<uint16_t*>(yh), static_cast<uint8_t*>(y4), static_cast<uint8_t*>(ys), \
                       tokens, srows);                                                                  \
    return hipGetLastError();                                                                           \
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
