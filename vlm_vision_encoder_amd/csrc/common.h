// Device-side helpers shared by the gfx950 kernels: vector types, bf16 and
// fp16 conversion, MFMA wrappers, wavefront reductions and the
// kernel-argument structs.  CDNA4 only (wave64, MFMA 32x32x16 bf16 / fp16).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "plan.h"

namespace pv {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element offset of an image in the pixel buffer.
__device__ __forceinline__ int64_t pix_offset(const ImageMeta& m) {
  return int64_t((uint64_t(m.pix_hi) << 32) | uint64_t(m.pix_lo));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, uint32_t(b) << 16);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Largest finite fp16 value.
constexpr float kF16Max = 65504.f;

// Two floats -> packed fp16 pair, round to nearest even, saturated to the
// finite range (a value past +-65504 becomes +-65504, not infinity).
__device__ __forceinline__ uint32_t pack_f16x2_sat(float a, float b) {
  halfx2 v;
  v[0] = (_Float16)__builtin_amdgcn_fmed3f(a, -kF16Max, kF16Max);
  v[1] = (_Float16)__builtin_amdgcn_fmed3f(b, -kF16Max, kF16Max);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 r;
  r[0] = pack_bf16x2(f[0], f[1]);
  r[1] = pack_bf16x2(f[2], f[3]);
  r[2] = pack_bf16x2(f[4], f[5]);
  r[3] = pack_bf16x2(f[6], f[7]);
  return r;
}

__device__ __forceinline__ floatx16 mfma32x32x16(const u32x4& a, const u32x4& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// The same product on fp16 operands (8 fp16 values per lane and operand).
__device__ __forceinline__ floatx16 mfma32x32x16_f16(const u32x4& a, const u32x4& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                 __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// Value of the neighbouring lane (lane ^ 1) via DPP quad permute [1,0,3,2].
__device__ __forceinline__ float swap_adjacent(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}

// Max / sum of v over the lane pair (l, l ^ 32), through ds_bpermute.
// (The v_permlane32_swap builtin is not used: this compiler returns the same
// register for both of its results, losing the swapped upper half.)
__device__ __forceinline__ float pair_max32(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }
__device__ __forceinline__ float pair_sum32(float v) { return v + __shfl_xor(v, 32, 64); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Power-of-two block scale for fp4 e2m1 (0, 0.5, 1, 1.5, 2, 3, 4, 6):
// X = floor(log2(max |x|)) - 2 puts the block maximum in [4, 8) (past 6 it
// saturates); returns the E8M0 byte X + 127 and sets scale = 2^X.  The
// hardware conversion v_cvt_scalef32_pk_fp4_f32 divides by that scale and
// rounds to nearest even, two values per instruction.
__device__ __forceinline__ uint32_t mx_scale4(float amax, float& scale) {
  const int e = int((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xff);
  int x = e - 127 - 2;
  x = x < -120 ? -120 : (x > 120 ? 120 : x);
  scale = __builtin_bit_cast(float, uint32_t(x + 127) << 23);
  return uint32_t(x + 127);
}

// Four values / scale -> four fp4 nibbles (16 bits, first value lowest).
__device__ __forceinline__ uint32_t pack_fp4x4(float a, float b, float c, float d, float scale) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, scale, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c, d, scale, 1);
}

// ---------------------------------------------------------------------------
// Device view of the per-call maps (all in the workspace).
struct DevMaps {
  const ImageMeta* meta;
  const int32_t* rowinfo;  // [N][2]: image, (row << 16) | col
  const int32_t* msrc;     // [T][4]
  const float* rope;       // [2][maxpos][pairs][2]
  int32_t n_images;
  int32_t rope_maxpos;
  int32_t patch;
};

enum AMode { A_DENSE = 0, A_IM2COL = 1, A_MERGE = 2 };
enum BMode { B_ONE = 0, B_QKV = 1, B_GATEUP = 2 };
enum EMode { E_STORE = 0, E_STORE_F32 = 1, E_QKV_ROPE = 2, E_SILU_MUL = 3, E_ADD_F32 = 4, E_GELU = 5 };

struct GemmArgs {
  int32_t M, N, K;
  const void* A;      // A_DENSE: [M][lda]; A_MERGE: fp32 residual [*][hidden]
  int32_t lda;
  const float* pixels;  // A_IM2COL
  const void* B0;     // weights [N][K] (B_QKV: wq, wk, wv; B_GATEUP: gate, up)
  const void* B1;
  const void* B2;
  int32_t ldb;
  int32_t kb;         // K extent of B when A's K repeats it (hi | lo halves of A), else 0
  // low-precision k (after the bf16 K range, or alone): k8 more k of
  // A8 [M][k8] x B8 [N][k8] in fp8 e4m3 (low_fmt 8) or packed fp4 e2m1
  // (low_fmt 4, two values a byte, low nibble first), one power-of-two scale
  // per 32 k on both sides, scale bytes in step-major blocks
  // As [k8/kstep][as_rows][sb], Bs [k8/kstep][bs_rows][sb] with
  // (kstep, sb) = (128, 4) for fp8 and (256, 8) for fp4; k8 = 0: none
  const void* A8;
  const void* B8;
  const void* As;
  const void* Bs;
  int32_t k8, as_rows, bs_rows;
  int32_t low_fmt;
  int32_t f16;        // 1: A and B are fp16 (fp16 MFMAs for the 16-bit k range), else bf16
  void* C;
  int32_t ldc;
  int32_t hidden;     // D (QKV split, merge gather)
  int32_t heads;
  DevMaps maps;
};

}  // namespace pv
