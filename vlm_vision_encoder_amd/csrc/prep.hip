// Operand preparation for the bf16 GEMMs whose A operand carries fp32
// values: each such value x goes to the MFMAs as two bf16 numbers, hi =
// bf16(x) and lo = bf16(x - hi), placed in two halves of the K range (row =
// [hi | lo]) that meet the same weights.  HBM-bound passes: 4 bytes read and
// 4 bytes written per value.
//   im2col_split: the patch embedding's A ("Mistral 3" (KerasFormers),
//                 Mistral3VisionModel: the convolution with stride = kernel =
//                 patch size, i.e. one GEMM row per patch), K order
//                 (channel, row, column) of the conv weight, zero-padded to Kp.
//   pad_rows:     copy of a bf16 matrix with its rows zero-padded (patch
//                 weights [D][3p^2] -> [D][Kp]).
//   im2col_u8_split: the same A operand straight from uint8 H x W x 3 images:
//                 each pixel of the resized image is a bilinear sample of the
//                 source ("Mistral 3" page: images are resized so the longest
//                 edge fits and the sides stay on the patch grid; pixel
//                 centres at half-integers, no antialiasing), then x / 255 and
//                 (x - mean_c) / std_c (Mistral3ImageProcessor table), folded
//                 into one multiply-add per channel.
//   resize_norm_u8: the same samples written out as fp32 planes.
//   copy_f16:     fp16 copy of a bf16 array (the gate, up and down weights
//                 of the MLP's fp16 products; bf16 values convert exactly
//                 inside fp16's normal range).
//   rows_fp4:     fp4 e2m1 copy of a matrix, one power-of-two scale per 32 k
//                 (the merge weights, against the merger input's low part).
//   gateup_fp8, quant_rows_fp8: fp8 e4m3 copies of weights and activations
//                 for the fp8 variant of the tower's linear maps.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

__device__ __forceinline__ void split8(const float (&f)[8], u32x4& hi, u32x4& lo) {
  float r[8];
  hi = pack8(f);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[2 * e] = f[2 * e] - lo_bf16(hi[e]);
    r[2 * e + 1] = f[2 * e + 1] - hi_bf16(hi[e]);
  }
  lo = pack8(r);
}

// Taps of output index t when n_in source pixels are resampled to n_out:
// the source coordinate is ((2t + 1) n_in - n_out) / (2 n_out), clamped below
// at 0; taps i0 = floor, i1 = min(i0 + 1, n_in - 1), weight f of i1.  The
// integer form picks the taps exactly (sides <= 32768 keep it in 32 bits).
__device__ __forceinline__ void bilinear_taps(uint32_t t, uint32_t n_in, uint32_t n_out, uint32_t& i0,
                                              uint32_t& i1, float& f) {
  const uint32_t num = (2u * t + 1u) * n_in, den = 2u * n_out;
  if (num <= n_out) {
    i0 = 0;
    f = 0.f;
  } else {
    const uint32_t e = num - n_out;
    i0 = e / den;
    f = float(e - i0 * den) / float(den);
  }
  i1 = i0 + 1 < n_in ? i0 + 1 : n_in - 1;
}

// Normalised value of channel c at pixel (ty, tx) of the sH x sW source
// resized to RH x RW.
__device__ __forceinline__ float sample_u8(const uint8_t* __restrict__ img, uint32_t sH, uint32_t sW, uint32_t RH,
                                           uint32_t RW, uint32_t ty, uint32_t tx, int c, float mul, float add) {
  uint32_t y0, y1, x0, x1;
  float fy, fx;
  bilinear_taps(ty, sH, RH, y0, y1, fy);
  bilinear_taps(tx, sW, RW, x0, x1, fx);
  const uint8_t* r0 = img + size_t(y0) * sW * 3 + c;
  const uint8_t* r1 = img + size_t(y1) * sW * 3 + c;
  const float a = r0[x0 * 3], b = r0[x1 * 3], cc = r1[x0 * 3], d = r1[x1 * 3];
  const float top = a + fx * (b - a), bot = cc + fx * (d - cc);
  return (top + fy * (bot - top)) * mul + add;
}

// Staged im2col: one workgroup per kStagePatches consecutive patches of the
// packed sequence.  Phase 1 reads, for every channel c and pixel row u of a
// patch, the p pixels of each of the workgroup's patches -- consecutive
// patches of one patch row sit side by side in the image, so a wave reads one
// contiguous run -- into LDS (element k = c p^2 + u p + x of patch q at
// stage[q * stride + k]).  Phase 2 writes every (patch, 8 k) chunk as
// bf16 hi | lo with 16-byte stores, k >= K zero.  Phase 1 takes one thread per
// pixel column of the workgroup's patches (16 p <= 256), so patches of up to
// 16 pixels use it (K <= 768 fits the stride); larger ones take the
// per-thread kernel below.
#ifndef PV_STAGE_PATCHES
#define PV_STAGE_PATCHES 16
#endif
#ifndef PV_STAGE_THREADS
#define PV_STAGE_THREADS 256
#endif
#ifndef PV_STAGE_WG_PER_CU
#define PV_STAGE_WG_PER_CU 2
#endif
constexpr int kStagePatches = PV_STAGE_PATCHES;
constexpr int kStageStride = 1040;  // floats, any patch up to 16 pixels; consecutive patches 16 banks apart
constexpr int kStageThreads = PV_STAGE_THREADS;
// per-patch LDS stride for a compile-time patch edge: K rounded up to 8, plus
// an offset that moves consecutive patches to other banks (P = 14: 600 floats,
// 24 banks apart; P = 16: 776, 8 apart), so that 4 (P = 14) or 3 (P = 16)
// workgroups fit a CU's LDS
template <int P>
constexpr int stage_stride() {
  return P == 14 ? 600 : P == 16 ? 776 : kStageStride;
}

// P: the patch edge as a compile-time constant (its 3 P loads of a thread are
// all issued before the LDS stores), or 0 (maps.patch, a loop).
//
// Persistent over chunks of kStagePatches patches (workgroup b takes chunks
// b, b + gridDim.x, ...): the pixels of a workgroup's next chunk are loaded
// into registers while it writes the current chunk's rows, so the reads of
// one chunk overlap the stores of the one before (a launch with one
// workgroup per chunk does all its reads, then all its writes).
template <int P>
__global__ __launch_bounds__(kStageThreads) void im2col_staged_kernel(const float* __restrict__ pixels, DevMaps maps,
                                                                      uint16_t* __restrict__ out, int n_patches,
                                                                      int K, int Kp) {
  constexpr int SS = stage_stride<P>();
  constexpr int NV = P > 0 ? 3 * P : 1;  // pixels a thread holds for the next chunk (P > 0)
  static_assert(P == 0 || SS >= 3 * P * P, "stage stride below K");
  __shared__ __attribute__((aligned(16))) float stage[kStagePatches * SS];
  const int p = P > 0 ? P : maps.patch, pp = p * p;
  const int t = threadIdx.x;
  const int n_chunks = (n_patches + kStagePatches - 1) / kStagePatches;
  // thread t owns pixel x of patch q in every (c, u) row of a chunk
  const int q = t / p, x = t - q * p;
  // pointer to pixel x of row 0, channel 0 of patch q of chunk c, its
  // image's plane size and width; false if the chunk has no such patch
  auto locate = [&](int c, const float*& src, long long& plane, int& w) {
    const int g = c * kStagePatches + q;
    if (q >= kStagePatches || g >= n_patches) return false;
    const int img = maps.rowinfo[2 * g], rc = maps.rowinfo[2 * g + 1];
    const ImageMeta mt = maps.meta[img];
    src = pixels + pix_offset(mt) + (long long)((rc >> 16) * p) * mt.W + (rc & 0xffff) * p + x;
    plane = (long long)mt.H * mt.W;
    w = mt.W;
    return true;
  };
  float v[NV];
  auto load = [&](int c) {  // P > 0: the chunk's pixels of this thread into v
    const float* src;
    long long plane;
    int w;
    if (!locate(c, src, plane, w)) return;
#pragma unroll
    for (int cc = 0; cc < 3; ++cc)
#pragma unroll
      for (int u = 0; u < P; ++u) v[cc * P + u] = src[cc * plane + (long long)u * w];
  };
  int c = blockIdx.x;
  if constexpr (P > 0) {
    if (c < n_chunks) load(c);
  }
  for (; c < n_chunks; c += gridDim.x) {
    const int g0 = c * kStagePatches;
    const int np = n_patches - g0 < kStagePatches ? n_patches - g0 : kStagePatches;
    __syncthreads();  // the previous chunk's rows are read out of the stage
    if (q < np) {
      float* dst = stage + q * SS + x;
      if constexpr (P > 0) {
#pragma unroll
        for (int cc = 0; cc < 3; ++cc)
#pragma unroll
          for (int u = 0; u < P; ++u) dst[cc * P * P + u * P] = v[cc * P + u];
      } else {
        const float* src;
        long long plane;
        int w;
        locate(c, src, plane, w);
        for (int cc = 0; cc < 3; ++cc) {
          const float* sc = src + cc * plane;
          float* dc = dst + cc * pp;
#pragma unroll 7
          for (int u = 0; u < p; ++u) dc[u * p] = sc[(long long)u * w];
        }
      }
    }
    __syncthreads();
    if constexpr (P > 0) {
      if (c + gridDim.x < n_chunks) load(c + gridDim.x);  // in flight during the writes below
    }
    // (patch, 8 k) chunks of the rows
    const int chunks = Kp / 8;
    for (int f = t; f < np * chunks; f += kStageThreads) {
      const int qq = f / chunks, k0 = (f - qq * chunks) * 8;
      float e8[8];
      if (k0 + 8 <= K) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(stage + qq * SS + k0);
        const floatx4 b = *reinterpret_cast<const floatx4*>(stage + qq * SS + k0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          e8[e] = a[e];
          e8[4 + e] = b[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = k0 + e < K ? stage[qq * SS + k0 + e] : 0.f;
      }
      u32x4 hi, lo;
      split8(e8, hi, lo);
      uint16_t* row = out + size_t(g0 + qq) * 2 * Kp;
      *reinterpret_cast<u32x4*>(row + k0) = hi;
      *reinterpret_cast<u32x4*>(row + Kp + k0) = lo;
    }
  }
}

// One thread per (patch g, 8 consecutive k).
__global__ __launch_bounds__(256) void im2col_split_kernel(const float* __restrict__ pixels, DevMaps maps,
                                                           uint16_t* __restrict__ out, int n_patches, int K, int Kp) {
  const int chunks = Kp / 8;
  const long long idx = blockIdx.x * 256ll + threadIdx.x;
  if (idx >= (long long)n_patches * chunks) return;
  const int g = int(idx / chunks), k0 = int(idx - (long long)g * chunks) * 8;
  const int img = maps.rowinfo[2 * g], rc = maps.rowinfo[2 * g + 1];
  const ImageMeta mt = maps.meta[img];
  const int p = maps.patch, pp = p * p;
  const int pr = rc >> 16, pc = rc & 0xffff;
  const float* base = pixels + pix_offset(mt) + size_t(pr * p) * mt.W + pc * p;
  const size_t plane = size_t(mt.H) * mt.W;
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + e;
    float v = 0.f;
    if (k < K) {
      const int ch = k / pp, rem = k - ch * pp;
      const int u = rem / p, x = rem - u * p;
      v = base[size_t(ch) * plane + size_t(u) * mt.W + x];
    }
    f[e] = v;
  }
  u32x4 hi, lo;
  split8(f, hi, lo);
  uint16_t* row = out + size_t(g) * 2 * Kp;
  *reinterpret_cast<u32x4*>(row + k0) = hi;
  *reinterpret_cast<u32x4*>(row + Kp + k0) = lo;
}

// One thread per (patch g, 8 consecutive k); the plan image (a resized image
// or a tile of one) is sampled from its uint8 source.
__global__ __launch_bounds__(256) void im2col_u8_split_kernel(const uint8_t* __restrict__ images,
                                                              const SrcImage* __restrict__ srcs, DevMaps maps,
                                                              NormAff aff, uint16_t* __restrict__ out,
                                                              int n_patches, int K, int Kp) {
  const int chunks = Kp / 8;
  const long long idx = blockIdx.x * 256ll + threadIdx.x;
  if (idx >= (long long)n_patches * chunks) return;
  const int g = int(idx / chunks), k0 = int(idx - (long long)g * chunks) * 8;
  const int img = maps.rowinfo[2 * g], rc = maps.rowinfo[2 * g + 1];
  const SrcImage sm = srcs[img];
  const uint8_t* src = images + ((uint64_t(sm.off_hi) << 32) | sm.off_lo);
  const int p = maps.patch, pp = p * p;
  const int pr = rc >> 16, pc = rc & 0xffff;
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + e;
    float v = 0.f;
    if (k < K) {
      const int ch = k / pp, rem = k - ch * pp;
      const int u = rem / p, x = rem - u * p;
      v = sample_u8(src, sm.H, sm.W, sm.RH, sm.RW, sm.y0 + pr * p + u, sm.x0 + pc * p + x, ch, aff.mul[ch],
                    aff.add[ch]);
    }
    f[e] = v;
  }
  u32x4 hi, lo;
  split8(f, hi, lo);
  uint16_t* row = out + size_t(g) * 2 * Kp;
  *reinterpret_cast<u32x4*>(row + k0) = hi;
  *reinterpret_cast<u32x4*>(row + Kp + k0) = lo;
}

// One thread per output pixel (all three channels) of the tH x tW window at
// (y0, x0) of the resized RH x RW image.
__global__ __launch_bounds__(256) void resize_norm_u8_kernel(const uint8_t* __restrict__ img, SrcImage sm, int tH,
                                                             int tW, NormAff aff, float* __restrict__ out) {
  const long long idx = blockIdx.x * 256ll + threadIdx.x;
  const long long plane = (long long)tH * tW;
  if (idx >= plane) return;
  const int ty = int(idx / tW), tx = int(idx - (long long)ty * tW);
#pragma unroll
  for (int c = 0; c < 3; ++c)
    out[c * plane + idx] =
        sample_u8(img, sm.H, sm.W, sm.RH, sm.RW, sm.y0 + ty, sm.x0 + tx, c, aff.mul[c], aff.add[c]);
}

__global__ __launch_bounds__(256) void pad_rows_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
                                                       int rows, int K, int Kp) {
  const long long idx = blockIdx.x * 256ll + threadIdx.x;
  if (idx >= (long long)rows * Kp) return;
  const int r = int(idx / Kp), k = int(idx - (long long)r * Kp);
  out[idx] = k < K ? w[size_t(r) * K + k] : uint16_t(0);
}

// 32 consecutive bf16 values -> 32 fp8 e4m3 bytes at dst and the block's
// E8M0 scale byte (returned): X = floor(log2(max |x|)) - 7 puts the block
// maximum in [128, 256) of e4m3.
__device__ __forceinline__ uint8_t quant_block32(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst) {
  float f[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 w = reinterpret_cast<const u32x4*>(src)[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[8 * c + 2 * e] = lo_bf16(w[e]);
      f[8 * c + 2 * e + 1] = hi_bf16(w[e]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(f[e]));
  // X = floor(log2(amax)) - 7: the block maximum lands in [128, 256) of e4m3
  const int ex = int((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xff);
  int x = ex - 127 - 7;
  x = x < -120 ? -120 : (x > 120 ? 120 : x);
  const float mul = __builtin_bit_cast(float, uint32_t(127 - x) << 23);
  u32x4 o[2];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * q] * mul, f[4 * q + 1] * mul, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * q + 2] * mul, f[4 * q + 3] * mul, r, true);
    o[q / 4][q % 4] = uint32_t(r);
  }
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  d[0] = o[0];
  d[1] = o[1];
  return uint8_t(x + 127);
}

// One thread per (row n of the interleaved gate/up matrix, block of 32 k).
// Row n: 32-row blocks alternate gate and up (rows [64j, 64j+32) -> gate
// rows [32j, +32), rows [64j+32, 64j+64) -> up rows [32j, +32)).
__global__ __launch_bounds__(256) void gateup_fp8_kernel(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                         uint8_t* __restrict__ b8, uint8_t* __restrict__ bs, int F,
                                                         int D) {
  const int blocks = D / 32;
  const long long idx = blockIdx.x * 256ll + threadIdx.x;
  if (idx >= 2ll * F * blocks) return;
  const int n = int(idx / blocks), blk = int(idx - (long long)n * blocks);
  const int src_row = (n >> 6) * 32 + (n & 31);
  const uint16_t* src = ((n & 32) ? wu : wg) + size_t(src_row) * D + blk * 32;
  bs[(size_t(blk / 4) * (2 * F) + n) * 4 + (blk & 3)] = quant_block32(src, b8 + size_t(n) * D + blk * 32);
}

// The same rows in packed fp4 for the MLP input's fp4 low part: b4
// [2F][D/2] (low nibble = even k), scales bs[(k/256) * 2F + n][(k/32) % 8].
// One 32-value block of bf16 weights -> 16 bytes of fp4 e2m1 (low nibble =
// even k) and its E8M0 scale byte.
__device__ __forceinline__ uint32_t fp4_block32(const uint16_t* __restrict__ src, u32x4& o) {
  float f[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 w = reinterpret_cast<const u32x4*>(src)[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[8 * c + 2 * e] = lo_bf16(w[e]);
      f[8 * c + 2 * e + 1] = hi_bf16(w[e]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(f[e]));
  float scale;
  const uint32_t sbyte = mx_scale4(amax, scale);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = pack_fp4x4(f[8 * q], f[8 * q + 1], f[8 * q + 2], f[8 * q + 3], scale) |
           (pack_fp4x4(f[8 * q + 4], f[8 * q + 5], f[8 * q + 6], f[8 * q + 7], scale) << 16);
  return sbyte;
}

// One thread per (row n, block of 32 columns) of a bf16 [rows][K] matrix:
// b4 [rows][K/2] fp4, bs [K/256][rows][8] scale bytes.
__global__ __launch_bounds__(256) void rows_fp4_kernel(const uint16_t* __restrict__ w, int rows, int K,
                                                       uint8_t* __restrict__ b4, uint8_t* __restrict__ bs) {
  const int blocks = K / 32;
  const long long idx = blockIdx.x * 256ll + threadIdx.x;
  if (idx >= (long long)rows * blocks) return;
  const int n = int(idx / blocks), blk = int(idx - (long long)n * blocks);
  u32x4 o;
  const uint32_t sbyte = fp4_block32(w + size_t(n) * K + blk * 32, o);
  *reinterpret_cast<u32x4*>(b4 + size_t(n) * (K / 2) + blk * 16) = o;
  bs[(size_t(blk / 8) * rows + n) * 8 + (blk & 7)] = uint8_t(sbyte);
}

// Eight values a thread (n8 16-byte chunks of bf16) to fp16.
__global__ __launch_bounds__(256) void copy_f16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ h16,
                                                       long long n8) {
  const long long i = blockIdx.x * 256ll + threadIdx.x;
  if (i >= n8) return;
  const u32x4 v = src[i];
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_f16x2_sat(lo_bf16(v[j]), hi_bf16(v[j]));
  h16[i] = o;
}

// One thread per (row r, block of 32 columns) of a bf16 [rows][K] matrix;
// output row row0 + r of dst8 [.][K] and of the scale bytes
// scales[(col / 128) * srows + row][(col / 32) % 4].
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint16_t* __restrict__ src, int rows, int K,
                                                             uint8_t* __restrict__ dst8, uint8_t* __restrict__ scales,
                                                             int srows, int row0) {
  const int blocks = K / 32;
  const long long idx = blockIdx.x * 256ll + threadIdx.x;
  if (idx >= (long long)rows * blocks) return;
  const int r = int(idx / blocks), blk = int(idx - (long long)r * blocks);
  const size_t row = size_t(row0) + r;
  scales[(size_t(blk / 4) * srows + row) * 4 + (blk & 3)] =
      quant_block32(src + size_t(r) * K + blk * 32, dst8 + row * K + blk * 32);
}

inline dim3 grid_for(long long threads) { return dim3(unsigned((threads + 255) / 256)); }

}  // namespace

hipError_t im2col_split(const float* pixels, const DevMaps& maps, void* out, int n_patches, int K, int Kp,
                        hipStream_t s) {
  if (n_patches <= 0) return hipSuccess;
  if (Kp % 8 || K > Kp) return hipErrorInvalidValue;
  if (K <= kStageStride && K == 3 * maps.patch * maps.patch && kStagePatches * maps.patch <= kStageThreads) {
    // PV_STAGE_WG_PER_CU workgroups per CU (each then takes several chunks),
    // or one per chunk (0)
    const int n_chunks = (n_patches + kStagePatches - 1) / kStagePatches;
    const int cap = PV_STAGE_WG_PER_CU > 0 ? PV_STAGE_WG_PER_CU * kNumCUs : n_chunks;
    const dim3 grid(n_chunks < cap ? n_chunks : cap), block(kStageThreads);
    uint16_t* o = static_cast<uint16_t*>(out);
    if (maps.patch == 14)
      hipLaunchKernelGGL(im2col_staged_kernel<14>, grid, block, 0, s, pixels, maps, o, n_patches, K, Kp);
    else if (maps.patch == 16)
      hipLaunchKernelGGL(im2col_staged_kernel<16>, grid, block, 0, s, pixels, maps, o, n_patches, K, Kp);
    else
      hipLaunchKernelGGL(im2col_staged_kernel<0>, grid, block, 0, s, pixels, maps, o, n_patches, K, Kp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(im2col_split_kernel, grid_for((long long)n_patches * (Kp / 8)), dim3(256), 0, s, pixels, maps,
                     static_cast<uint16_t*>(out), n_patches, K, Kp);
  return hipGetLastError();
}

hipError_t im2col_u8_split(const uint8_t* images, const SrcImage* src, const DevMaps& maps, const NormAff& aff,
                           void* out, int n_patches, int K, int Kp, hipStream_t s) {
  if (n_patches <= 0) return hipSuccess;
  if (Kp % 8 || K > Kp || K != 3 * maps.patch * maps.patch) return hipErrorInvalidValue;
  hipLaunchKernelGGL(im2col_u8_split_kernel, grid_for((long long)n_patches * (Kp / 8)), dim3(256), 0, s, images,
                     src, maps, aff, static_cast<uint16_t*>(out), n_patches, K, Kp);
  return hipGetLastError();
}

hipError_t resize_norm_u8(const uint8_t* image, const SrcImage& sm, int tH, int tW, const NormAff& aff, float* out,
                          hipStream_t s) {
  if (sm.H < 1 || sm.W < 1 || sm.H > kMaxSrcSide || sm.W > kMaxSrcSide || tH < 1 || tW < 1 || sm.y0 < 0 ||
      sm.x0 < 0 || sm.y0 + tH > sm.RH || sm.x0 + tW > sm.RW || sm.RH > 2 * kMaxSrcSide || sm.RW > 2 * kMaxSrcSide)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(resize_norm_u8_kernel, grid_for((long long)tH * tW), dim3(256), 0, s, image, sm, tH, tW, aff,
                     out);
  return hipGetLastError();
}


hipError_t gateup_fp8(const void* w_gate, const void* w_up, void* b8, void* bs, int F, int D, hipStream_t s) {
  if (F <= 0) return hipSuccess;
  if (D % 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gateup_fp8_kernel, grid_for(2ll * F * (D / 32)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
                     static_cast<uint8_t*>(b8), static_cast<uint8_t*>(bs), F, D);
  return hipGetLastError();
}

hipError_t quant_rows_fp8(const void* src, int rows, int K, void* dst8, void* scales, int srows, int row0,
                          hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K % 128 || row0 < 0 || row0 + rows > srows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, grid_for((long long)rows * (K / 32)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(src), rows, K, static_cast<uint8_t*>(dst8),
                     static_cast<uint8_t*>(scales), srows, row0);
  return hipGetLastError();
}

hipError_t copy_f16(const void* src, long long n, void* h16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 8 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(h16)) % 16)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_f16_kernel, grid_for(n / 8), dim3(256), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(h16), n / 8);
  return hipGetLastError();
}

hipError_t rows_fp4(const void* w, int rows, int K, void* b4, void* bs, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K % 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_fp4_kernel, grid_for((long long)rows * (K / 32)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w), rows, K, static_cast<uint8_t*>(b4), static_cast<uint8_t*>(bs));
  return hipGetLastError();
}

hipError_t pad_rows(const void* w, void* out, int rows, int K, int Kp, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K > Kp) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pad_rows_kernel, grid_for((long long)rows * Kp), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w), static_cast<uint16_t*>(out), rows, K, Kp);
  return hipGetLastError();
}

}  // namespace pv
