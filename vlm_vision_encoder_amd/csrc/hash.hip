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
// The sum makes the words independent work (integer adds in any order give
// the same result); the index term ties each word to its place.  Not a cryptographic hash: two different images collide with
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

constexpr int kKeyBlocks = 1024;  // workgroups per image (grid-stride beyond)
constexpr int kKeyUnroll = 4;     // 16-byte loads in flight per thread

// Words 2p and 2p + 1 of the image from dwords j = 4p .. 4p + 4 (d[0..4]) of
// the 4-aligned view starting `a` bytes before the image, zero past the
// image's last byte; their mixed sums are added to s0 and s1.
__device__ __forceinline__ void add_pair(const uint32_t (&d)[5], int a, uint64_t p, uint64_t len, uint64_t& s0,
                                         uint64_t& s1) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t i = 2 * p + h;
    if (8 * i >= len) break;
    uint64_t v = (uint64_t(d[2 * h + 1]) << 32) | d[2 * h];
    if (a) v = (v >> (8 * a)) | (uint64_t(d[2 * h + 2]) << (64 - 8 * a));
    const uint64_t valid = len - 8 * i;
    if (valid < 8) v &= (uint64_t(1) << (8 * valid)) - 1;
    s0 += mix64(v + (i + 1) * kG0);
    s1 += mix64(v + (i + 1) * kG1);
  }
}

// One image: `base` is the 4-aligned dword at or below its first byte, `a`
// the first byte's offset in that dword, `len` its byte count.  Lane t of a
// step loads dwords [4p, 4p + 4) with one 16-byte access (a wave reads 1 KB
// contiguously) and takes dword 4p + 4 from the next lane; no dword past the
// one holding the image's last byte is read.  Each workgroup writes its two
// partial sums; keys_final_kernel adds them in a fixed order.
__global__ __launch_bounds__(256) void keys_sum_kernel(const uint32_t* __restrict__ base, int a, uint64_t len,
                                                       unsigned long long* __restrict__ partial) {
  const uint64_t nwords = (len + 7) / 8;
  const uint64_t npairs = (nwords + 1) / 2;
  const uint64_t jlast = (uint64_t(a) + len - 1) >> 2;
  const int lane = threadIdx.x & 63;
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  uint64_t s0 = 0, s1 = 0;
  for (uint64_t p0 = uint64_t(blockIdx.x) * 256 + threadIdx.x - lane; p0 < npairs; p0 += kKeyUnroll * stride) {
    uint32_t d[kKeyUnroll][5];
#pragma unroll
    for (int u = 0; u < kKeyUnroll; ++u) {
      const uint64_t j = 4 * (p0 + u * stride + lane);
      if (j + 3 <= jlast) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + j);
        d[u][0] = v[0];
        d[u][1] = v[1];
        d[u][2] = v[2];
        d[u][3] = v[3];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) d[u][c] = j + c <= jlast ? base[j + c] : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kKeyUnroll; ++u) {
      const uint64_t p = p0 + u * stride + lane;
      const uint64_t j = 4 * p;
      uint32_t nxt = __shfl_down(d[u][0], 1);
      if (lane == 63) nxt = j + 4 <= jlast ? base[j + 4] : 0u;
      d[u][4] = nxt;
      if (p < npairs) add_pair(d[u], a, p, len, s0, s1);
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    s0 += shfl_xor64(s0, m);
    s1 += shfl_xor64(s1, m);
  }
  __shared__ uint64_t part[2][4];
  const int w = threadIdx.x >> 6;
  if (lane == 0) {
    part[0][w] = s0;
    part[1][w] = s1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = part[0][0] + part[0][1] + part[0][2] + part[0][3];
    partial[2 * blockIdx.x + 1] = part[1][0] + part[1][1] + part[1][2] + part[1][3];
  }
}

// key lanes of one image from its workgroups' partial sums
__global__ __launch_bounds__(64) void keys_final_kernel(const unsigned long long* __restrict__ partial, int nparts,
                                                        uint64_t size, uint64_t* __restrict__ key) {
  uint64_t s0 = 0, s1 = 0;
  for (int b = threadIdx.x; b < nparts; b += 64) {
    s0 += partial[2 * b];
    s1 += partial[2 * b + 1];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    s0 += shfl_xor64(s0, m);
    s1 += shfl_xor64(s1, m);
  }
  if (threadIdx.x == 0) {
    key[0] = mix64(s0 + mix64(size ^ kG0));
    key[1] = mix64(s1 + mix64(size ^ kG1));
  }
}

}  // namespace

size_t image_keys_workspace_bytes(int n) { return size_t(n) * kKeyBlocks * 16; }

hipError_t image_keys(const uint8_t* images, const int32_t* src_hw, const uint64_t* offsets, int n, uint64_t* keys,
                      void* ws, hipStream_t s) {
  unsigned long long* partial = static_cast<unsigned long long*>(ws);
  for (int i = 0; i < n; ++i) {
    const uint64_t len = uint64_t(3) * uint32_t(src_hw[2 * i]) * uint32_t(src_hw[2 * i + 1]);
    const uint64_t o = offsets[i];
    const int a = int(o & 3);
    const uint64_t npairs = ((len + 7) / 8 + 1) / 2;
    const uint64_t blocks = (npairs + 256 * kKeyUnroll - 1) / (256 * kKeyUnroll);
    const int grid = int(blocks < kKeyBlocks ? blocks : kKeyBlocks);
    unsigned long long* part = partial + size_t(i) * kKeyBlocks * 2;
    hipLaunchKernelGGL(keys_sum_kernel, dim3(grid), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(images + (o - a)), a, len, part);
    const uint64_t size = (uint64_t(uint32_t(src_hw[2 * i])) << 32) | uint32_t(src_hw[2 * i + 1]);
    hipLaunchKernelGGL(keys_final_kernel, dim3(1), dim3(64), 0, s, part, grid, size, keys + 2 * i);
  }
  return hipGetLastError();
}

}  // namespace pv
