// Content keys of uint8 images, for the multimodal embeddings cache (the
// inference-research record's note on an engine that keeps a per-model
// cache of multimodal embeddings).  A key is two 64-bit lanes s = 0, 1:
//   mix(z)  the output function of the SplitMix64 generator (Steele, Lea and
//           Flood, 2014, with Vigna's constants):
//           z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
//           z *= 0x94D049BB133111EB; z ^= z >> 31
//   w_i     the image's 3HW bytes as little-endian 64-bit words, the last
//           one zero-padded, i = 0 .. ceil(3HW / 8) - 1
//   acc_s = sum over i of mix(w_i + (i + 1) G_s)            (mod 2^64)
//   key_s = mix(acc_s + mix(((H << 32) | W) ^ G_s)),
//   G_0 = 0x9E3779B97F4A7C15, G_1 = 0xD1B54A32D192ED03.
// The sum makes the words independent work (one thread per word, integer
// adds in any order give the same result); the index term ties each word to
// its place.  Not a cryptographic hash: two different images collide with
// probability about 2^-128 unless chosen to.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

constexpr uint64_t kG0 = 0x9E3779B97F4A7C15ull, kG1 = 0xD1B54A32D192ED03ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(uint32_t(v), m), hi = __shfl_xor(uint32_t(v >> 32), m);
  return (uint64_t(hi) << 32) | lo;
}

__global__ void keys_zero_kernel(unsigned long long* acc, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < 2 * n) acc[i] = 0ull;
}

// One image: `base` is the 4-aligned dword at or below its first byte, `a`
// the first byte's offset in that dword, `len` its byte count.  Dwords past
// the one holding the last byte are never read.
__global__ __launch_bounds__(256) void keys_sum_kernel(const uint32_t* __restrict__ base, int a, uint64_t len,
                                                       unsigned long long* __restrict__ acc) {
  const uint64_t nwords = (len + 7) / 8;
  const uint64_t jlast = (uint64_t(a) + len - 1) >> 2;
  uint64_t s0 = 0, s1 = 0;
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < nwords; i += uint64_t(gridDim.x) * 256) {
    const uint64_t j = 2 * i;
    const uint64_t d0 = base[j];
    const uint64_t d1 = j + 1 <= jlast ? base[j + 1] : 0u;
    uint64_t v = (d1 << 32) | d0;
    if (a) {
      const uint64_t d2 = j + 2 <= jlast ? base[j + 2] : 0u;
      v = (v >> (8 * a)) | (d2 << (64 - 8 * a));
    }
    const uint64_t valid = len - 8 * i;
    if (valid < 8) v &= (uint64_t(1) << (8 * valid)) - 1;
    s0 += mix64(v + (i + 1) * kG0);
    s1 += mix64(v + (i + 1) * kG1);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    s0 += shfl_xor64(s0, m);
    s1 += shfl_xor64(s1, m);
  }
  __shared__ uint64_t part[2][4];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    part[0][w] = s0;
    part[1][w] = s1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&acc[0], (unsigned long long)(part[0][0] + part[0][1] + part[0][2] + part[0][3]));
    atomicAdd(&acc[1], (unsigned long long)(part[1][0] + part[1][1] + part[1][2] + part[1][3]));
  }
}

// key lanes of one image from its two accumulators
__global__ void keys_final_kernel(const unsigned long long* __restrict__ acc, uint64_t size,
                                  uint64_t* __restrict__ key) {
  const int s = threadIdx.x;
  if (s < 2) key[s] = mix64(uint64_t(acc[s]) + mix64(size ^ (s ? kG1 : kG0)));
}

}  // namespace

size_t image_keys_workspace_bytes(int n) { return (size_t(n) * 16 + 255) / 256 * 256; }

hipError_t image_keys(const uint8_t* images, const int32_t* src_hw, const uint64_t* offsets, int n, uint64_t* keys,
                      void* ws, hipStream_t s) {
  unsigned long long* acc = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL(keys_zero_kernel, dim3((2 * n + 255) / 256), dim3(256), 0, s, acc, n);
  for (int i = 0; i < n; ++i) {
    const uint64_t len = uint64_t(3) * uint32_t(src_hw[2 * i]) * uint32_t(src_hw[2 * i + 1]);
    const uint64_t o = offsets[i];
    const int a = int(o & 3);
    const uint64_t nwords = (len + 7) / 8;
    const uint64_t blocks = (nwords + 255) / 256;
    const unsigned grid = unsigned(blocks < 2048 ? blocks : 2048);
    hipLaunchKernelGGL(keys_sum_kernel, dim3(grid), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(images + (o - a)), a, len, acc + 2 * i);
    const uint64_t size = (uint64_t(uint32_t(src_hw[2 * i])) << 32) | uint32_t(src_hw[2 * i + 1]);
    hipLaunchKernelGGL(keys_final_kernel, dim3(1), dim3(64), 0, s, acc + 2 * i, size, keys + 2 * i);
  }
  return hipGetLastError();
}

}  // namespace pv
