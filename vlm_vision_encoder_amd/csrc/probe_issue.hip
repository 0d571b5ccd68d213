// Microbenchmark: do MFMA and vector-ALU instructions of one gfx950 SIMD
// overlap?  Not part of the tower library; built next to it as an executable
// (probe_issue) and run by hand to measure the issue behaviour that the
// attention kernel's design depends on.
//
// Every kernel runs ITERS iterations of a fixed body per wave on all 256 CUs
// and is timed with HIP events (the second of two launches):
//   mfma   4 independent v_mfma_f32_32x32x16_bf16 accumulation chains
//   exp    16 independent v_exp_f32
//   fma    16 independent v_fma_f32
//   mfma+exp / mfma+fma   both bodies interleaved in the same wave
// with 1 or 2 waves per SIMD of one body, and with 8-wave workgroups whose
// waves 0-3 run one body and waves 4-7 another (wave w runs on SIMD w % 4, so
// each SIMD holds one wave of each).  If MFMA and VALU did not overlap, a
// mixed kernel would take the sum of its parts.
//
// Two more measurements:
//   LDS read throughput: every lane of 4, 8 or 12 waves per CU reads
//     conflict-free 16-byte (ds_read_b128) or 8-byte transposing
//     (ds_read_b64_tr_b16) chunks from a 64 KB LDS buffer, 16 reads in
//     flight per wave; reported as bytes per ns per CU
//   wave placement: the SIMD (HW_ID bits 5:4) of every wave of a 12-wave and
//     an 8-wave workgroup
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kIters = 20000;
constexpr int kCUs = 256;

enum Body { MFMA = 1, EXP = 2, MFMA_EXP = 3, FMA = 4, MFMA_FMA = 5 };

template <int M>
__device__ __forceinline__ void body(floatx16 (&acc)[4], bf16x8 a, bf16x8 b, float (&e)[16]) {
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (M & 1) acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
      if constexpr (M == EXP || M == MFMA_EXP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) e[4 * q + i] = __builtin_amdgcn_exp2f(e[4 * q + i]);
      }
      if constexpr (M == FMA || M == MFMA_FMA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) e[4 * q + i] = __builtin_fmaf(e[4 * q + i], 0.999f, 0.0001f);
      }
    }
  }
}

// waves [0, split) run body MA, the rest MB; sink keeps every result live
template <int MA, int MB, int THREADS>
__global__ __launch_bounds__(THREADS) void probe(int split, float* sink) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  floatx16 acc[4] = {};
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * float(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * float(i));
  }
  float e[16];
  for (int i = 0; i < 16; ++i) e[i] = -0.001f * float(threadIdx.x + i);
  if (wave < split) body<MA>(acc, a, b, e);
  else body<MB>(acc, a, b, e);
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i] + e[i];
  sink[blockIdx.x * THREADS + threadIdx.x] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kLdsIters = 4000;
constexpr int kLdsChunks = 4096;  // 16-byte chunks: 64 KB

// TR 0: ds_read_b128 of chunk (lane + 64 * (i + 16 * wave) + it) mod 4096 --
// a wave reads 1 KB of consecutive chunks per instruction (16 lanes of a
// pass cover all 64 banks once); TR 1: ds_read_b64_tr_b16 of the 8-byte
// chunk at the same index, 512 bytes per instruction
template <int TR, int THREADS>
__global__ __launch_bounds__(THREADS) void lds_probe(uint32_t* sink) {
  __shared__ u32x4 buf[kLdsChunks];
  for (int c = threadIdx.x; c < kLdsChunks; c += THREADS) buf[c] = u32x4{uint32_t(c), 1u, 2u, 3u};
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < kLdsIters; ++it) {
    u32x4 r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = (lane + 64 * (i + 16 * wave) + 64 * it) & (kLdsChunks - 1);
      if constexpr (TR == 0) {
        r[i] = buf[c];
      } else {
        const v4i16 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(reinterpret_cast<char*>(buf) + ((size_t(c) * 8) & (kLdsChunks * 16 - 1))));
        const uint2 w = __builtin_bit_cast(uint2, t);
        r[i] = u32x4{w.x, w.y, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= r[i];
  }
  sink[blockIdx.x * THREADS + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// SIMD of each wave: HW_ID (hardware register 4) bits 5:4
template <int THREADS>
__global__ __launch_bounds__(THREADS) void simd_of_wave(int* out) {
  const int simd = (__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4)) & 3;
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6)] = simd;
}

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

template <int MA, int MB, int THREADS>
float time_ms(int blocks, int split, float* sink) {
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "event");
  check(hipEventCreate(&e1), "event");
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {
    check(hipEventRecord(e0, nullptr), "record");
    hipLaunchKernelGGL((probe<MA, MB, THREADS>), dim3(blocks), dim3(THREADS), 0, nullptr, split, sink);
    check(hipGetLastError(), "launch");
    check(hipEventRecord(e1, nullptr), "record");
    check(hipEventSynchronize(e1), "sync");
    check(hipEventElapsedTime(&ms, e0, e1), "elapsed");
  }
  check(hipEventDestroy(e0), "event");
  check(hipEventDestroy(e1), "event");
  return ms;
}

template <int TR, int THREADS>
float lds_ms(uint32_t* sink) {
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "event");
  check(hipEventCreate(&e1), "event");
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {
    check(hipEventRecord(e0, nullptr), "record");
    hipLaunchKernelGGL((lds_probe<TR, THREADS>), dim3(kCUs), dim3(THREADS), 0, nullptr, sink);
    check(hipGetLastError(), "launch");
    check(hipEventRecord(e1, nullptr), "record");
    check(hipEventSynchronize(e1), "sync");
    check(hipEventElapsedTime(&ms, e0, e1), "elapsed");
  }
  check(hipEventDestroy(e0), "event");
  check(hipEventDestroy(e1), "event");
  return ms;
}

template <int THREADS>
void print_waves(int* dev) {
  constexpr int W = THREADS / 64, B = 4;
  hipLaunchKernelGGL((simd_of_wave<THREADS>), dim3(B), dim3(THREADS), 0, nullptr, dev);
  check(hipGetLastError(), "launch");
  int host[B * W];
  check(hipMemcpy(host, dev, sizeof(host), hipMemcpyDeviceToHost), "copy");
  for (int b = 0; b < B; ++b) {
    std::printf("  %2d-wave workgroup %d, SIMD of waves 0..%d:", W, b, W - 1);
    for (int w = 0; w < W; ++w) std::printf(" %d", host[b * W + w]);
    std::printf("\n");
  }
}

}  // namespace

int main() {
  float* sink = nullptr;
  // the largest launch: 2 * kCUs blocks of 256 threads, or kCUs blocks of 512
  check(hipMalloc(&sink, size_t(2) * kCUs * 256 * sizeof(float)), "hipMalloc");
  std::printf("%d iterations per wave; per iteration: 4 MFMA (32x32x16 bf16), 16 exp, or 16 fma\n", kIters);
  std::printf("%-44s %10s %10s\n", "kernel", "1 w/SIMD", "2 w/SIMD");
  auto row = [&](const char* name, float a, float b) { std::printf("%-44s %8.3f ms %8.3f ms\n", name, a, b); };
  row("mfma", time_ms<MFMA, MFMA, 256>(kCUs, 4, sink), time_ms<MFMA, MFMA, 256>(2 * kCUs, 4, sink));
  row("exp", time_ms<EXP, EXP, 256>(kCUs, 4, sink), time_ms<EXP, EXP, 256>(2 * kCUs, 4, sink));
  row("fma", time_ms<FMA, FMA, 256>(kCUs, 4, sink), time_ms<FMA, FMA, 256>(2 * kCUs, 4, sink));
  row("mfma+exp in the same wave", time_ms<MFMA_EXP, MFMA_EXP, 256>(kCUs, 4, sink),
      time_ms<MFMA_EXP, MFMA_EXP, 256>(2 * kCUs, 4, sink));
  row("mfma+fma in the same wave", time_ms<MFMA_FMA, MFMA_FMA, 256>(kCUs, 4, sink),
      time_ms<MFMA_FMA, MFMA_FMA, 256>(2 * kCUs, 4, sink));
  std::printf("%-44s %10s %10s\n", "8-wave workgroups, one per CU", "", "2 w/SIMD");
  row("mfma waves beside exp waves on each SIMD", 0.f, time_ms<MFMA, EXP, 512>(kCUs, 4, sink));
  row("mfma waves beside fma waves on each SIMD", 0.f, time_ms<MFMA, FMA, 512>(kCUs, 4, sink));
  check(hipFree(sink), "hipFree");

  // LDS read throughput (one workgroup per CU)
  uint32_t* lsink = nullptr;
  check(hipMalloc(&lsink, size_t(kCUs) * 768 * sizeof(uint32_t)), "hipMalloc");
  std::printf("LDS reads, one workgroup per CU, %d x 16 reads per wave\n", kLdsIters);
  auto lrow = [&](const char* name, int waves, int bytes_per_lane, float ms) {
    const double bytes = double(kCUs) * waves * 64 * kLdsIters * 16 * bytes_per_lane;
    std::printf("  %-22s %2d waves/CU %8.3f ms  %7.1f bytes/ns per CU\n", name, waves, ms, bytes / kCUs / (ms * 1e6));
  };
  lrow("ds_read_b128", 4, 16, lds_ms<0, 256>(lsink));
  lrow("ds_read_b128", 8, 16, lds_ms<0, 512>(lsink));
  lrow("ds_read_b128", 12, 16, lds_ms<0, 768>(lsink));
  lrow("ds_read_b64_tr_b16", 4, 8, lds_ms<1, 256>(lsink));
  lrow("ds_read_b64_tr_b16", 8, 8, lds_ms<1, 512>(lsink));
  lrow("ds_read_b64_tr_b16", 12, 8, lds_ms<1, 768>(lsink));
  check(hipFree(lsink), "hipFree");

  // wave placement
  int* wsink = nullptr;
  check(hipMalloc(&wsink, 4 * 12 * sizeof(int)), "hipMalloc");
  std::printf("wave placement (HW_ID SIMD field)\n");
  print_waves<768>(wsink);
  print_waves<512>(wsink);
  check(hipFree(wsink), "hipFree");
  std::printf("done\n");
  return 0;
}
