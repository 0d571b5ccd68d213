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
// More measurements:
//   LDS read throughput: every lane of 4, 8 or 12 waves per CU reads
//     conflict-free 16-byte (ds_read_b128) or 8-byte transposing
//     (ds_read_b64_tr_b16) chunks from a 64 KB LDS buffer, 16 reads in
//     flight per wave; reported as bytes per ns per CU
//   wave placement: the SIMD (HW_ID bits 5:4) of every wave of a 12-wave and
//     an 8-wave workgroup
//   softmax instruction mix: 12-wave workgroups (3 waves per SIMD), one per
//     CU, each wave running the vector work of one P.V step of the attention
//     kernel's key tile (32 scores per lane: exp2, bf16 packing, row sums by
//     v_dot2 or by fp32 adds, or one kind of instruction alone) with and
//     without the step's 8 MFMAs beside it, and the whole key tile (8 score
//     MFMAs, the softmax, 8 P.V MFMAs) serial or with the next tile's score
//     MFMAs interleaved into the softmax; operands live in registers
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kMixIters = 10000;

__device__ __forceinline__ floatx16 mfma_u(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float dot2_acc(uint32_t packed, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed), one, acc, false);
}

// Vector work of one P.V step, 32 scores per lane in 4 groups of 8.  K:
// exp2 + pack + v_dot2 row sums, exp2 + pack + fp32 adds, or one kind of
// instruction alone (the values not exponentiated are the scores
// themselves; what is not packed is xor-folded).  MF adds the step's 8
// MFMAs (2 accumulators, B operand = the packed group).
enum MixKind { MIX_EXP_PACK_DOT2 = 0, MIX_EXP_PACK_ADD, MIX_EXP, MIX_PACK, MIX_DOT2, MIX_FMA };

template <int K, bool MF>
__global__ __launch_bounds__(768) void mix_probe(float* sink) {
  const int t = threadIdx.x;
  u32x4 vf[4][2];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 2; ++j)
      vf[i][j] = u32x4{pack2(0.5f, 0.25f * j), pack2(0.1f * i, 0.f), pack2(1.f, -1.f), pack2(0.f, 0.5f)};
  floatx16 o0 = {}, o1 = {};
  floatx16 s[2];
  for (int u = 0; u < 2; ++u)
    for (int v = 0; v < 16; ++v) s[u][v] = -0.01f * float((t + v + u) & 31);
  float l = 0.f;
  for (int it = 0; it < kMixIters; ++it) {
    for (int ub = 0; ub < 2; ++ub) asm volatile("" : "+v"(s[ub]));  // fresh scores every step
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ub = q >> 1, sp = q & 1;
      float p[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float x = s[ub][8 * sp + v];
        if constexpr (K == MIX_FMA) p[v] = __builtin_fmaf(x, 0.999f, 0.001f);
        else if constexpr (K == MIX_PACK || K == MIX_DOT2) p[v] = x;
        else p[v] = __builtin_amdgcn_exp2f(x);
      }
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (K == MIX_EXP_PACK_DOT2 || K == MIX_EXP_PACK_ADD || K == MIX_PACK)
          pk[i] = pack2(p[2 * i], p[2 * i + 1]);
        else
          pk[i] = __builtin_bit_cast(uint32_t, p[2 * i]) ^ __builtin_bit_cast(uint32_t, p[2 * i + 1]);
      }
      if constexpr (K == MIX_EXP_PACK_DOT2 || K == MIX_DOT2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) l = dot2_acc(pk[i], l);
      } else if constexpr (K == MIX_EXP_PACK_ADD) {
        l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      }
      if constexpr (MF) {
        o0 = mfma_u(vf[q][0], pk, o0);
        o1 = mfma_u(vf[q][1], pk, o1);
      } else {
        o0[q] += __builtin_bit_cast(float, pk[0] ^ pk[1] ^ pk[2] ^ pk[3]);
      }
    }
  }
  float r = l;
  for (int v = 0; v < 16; ++v) r += o0[v] + o1[v] + s[0][v] + s[1][v];
  sink[blockIdx.x * 768 + t] = r;
}

// The step's 8 MFMAs alone.
__global__ __launch_bounds__(768) void mix_mfma_only(float* sink) {
  u32x4 vf[4][2], b = {0x3f003f00u, 0x3f003f00u, 0x3f003f00u, 0x3f003f00u};
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 2; ++j) vf[i][j] = u32x4{0x3f80u + i, 0x3f00u * j, 0x3e00u, 0x3c00u};
  floatx16 o0 = {}, o1 = {};
  for (int it = 0; it < kMixIters; ++it) {
    asm volatile("" : "+v"(b));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o0 = mfma_u(vf[q][0], b, o0);
      o1 = mfma_u(vf[q][1], b, o1);
    }
  }
  float r = 0.f;
  for (int v = 0; v < 16; ++v) r += o0[v] + o1[v];
  sink[blockIdx.x * 768 + threadIdx.x] = r;
}

// A whole key tile per step: 8 score MFMAs, the softmax (exp2, pack, row
// sums by v_dot2 (SUM 0) or fp32 adds (SUM 1)), 8 P.V MFMAs.  PIPE 0 runs
// them in that order; PIPE 1 computes the next tile's scores while the
// current tile's softmax and P.V run, the interleave pinned per group of 8
// scores (one MFMA, five vector instructions, four times).  Two steps per
// trip, so the score buffers swap roles without copies.
template <int PIPE, int SUM>
__global__ __launch_bounds__(768) void tile_probe(float* sink) {
  const int t = threadIdx.x;
  u32x4 vf[2][2], kf[2][2], qf[4];
  for (int i = 0; i < 4; ++i)
    qf[i] = u32x4{pack2(0.01f * (t & 7), 0.02f), pack2(0.01f, -0.01f), pack2(0.f, 0.01f), pack2(0.03f, 0.f)};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) {
      vf[i][j] = u32x4{pack2(0.5f, 0.25f * j), pack2(0.1f * i, 0.f), pack2(1.f, -1.f), pack2(0.f, 0.5f)};
      kf[i][j] = u32x4{pack2(0.1f, -0.2f * j), pack2(0.1f * i, 0.3f), pack2(-0.1f, 0.1f), pack2(0.2f, 0.5f)};
    }
  floatx16 o0 = {}, o1 = {};
  floatx16 sa[2], sb[2];
  for (int u = 0; u < 2; ++u)
    for (int v = 0; v < 16; ++v) sa[u][v] = -0.01f * float((t + v + u) & 31);
  float l0 = 0.f, l1 = 0.f;
  auto step = [&](floatx16(&cur)[2], floatx16(&nxt)[2]) __attribute__((always_inline)) {
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(kf[i][j]), "+v"(vf[i][j]));
    const floatx16 z = {};
    nxt[0] = z;
    nxt[1] = z;
    if constexpr (PIPE == 0) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int ub = 0; ub < 2; ++ub) nxt[ub] = mfma_u(kf[ks & 1][ub], qf[ks], nxt[ub]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ub = q >> 1, sp = q & 1;
      if constexpr (PIPE != 0) {
        nxt[0] = mfma_u(kf[q & 1][0], qf[q], nxt[0]);
        nxt[1] = mfma_u(kf[q & 1][1], qf[q], nxt[1]);
      }
      float p[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) p[v] = __builtin_amdgcn_exp2f((PIPE == 0 ? nxt : cur)[ub][8 * sp + v]);
      const u32x4 pk = {pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
      if constexpr (SUM == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) l0 = dot2_acc(pk[i], l0);
      } else {
        l0 += (p[0] + p[1]) + (p[2] + p[3]);
        l1 += (p[4] + p[5]) + (p[6] + p[7]);
      }
      o0 = mfma_u(vf[q & 1][0], pk, o0);
      o1 = mfma_u(vf[q & 1][1], pk, o1);
      if constexpr (PIPE != 0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, 5, 0);  // five vector / transcendental
        }
      }
    }
  };
  for (int it = 0; it < kMixIters; it += 2) {
    step(sa, sb);
    step(sb, sa);
  }
  float r = l0 + l1;
  for (int v = 0; v < 16; ++v) r += o0[v] + o1[v] + sa[0][v] + sa[1][v];
  sink[blockIdx.x * 768 + t] = r;
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

// ns per step of a 768-thread kernel on kCUs workgroups (second of two launches)
template <typename F>
float step_ns(F launch) {
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "event");
  check(hipEventCreate(&e1), "event");
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {
    check(hipEventRecord(e0, nullptr), "record");
    launch();
    check(hipGetLastError(), "launch");
    check(hipEventRecord(e1, nullptr), "record");
    check(hipEventSynchronize(e1), "sync");
    check(hipEventElapsedTime(&ms, e0, e1), "elapsed");
  }
  check(hipEventDestroy(e0), "event");
  check(hipEventDestroy(e1), "event");
  return ms * 1e6f / kMixIters;
}

template <int K>
void mix_row(const char* name, float* sink, float mfma_ns) {
  const float a = step_ns([&] { hipLaunchKernelGGL((mix_probe<K, false>), dim3(kCUs), dim3(768), 0, nullptr, sink); });
  const float b = step_ns([&] { hipLaunchKernelGGL((mix_probe<K, true>), dim3(kCUs), dim3(768), 0, nullptr, sink); });
  const float hidden = 100.f * (a + mfma_ns - b) / (a < mfma_ns ? a : mfma_ns);
  std::printf("  %-22s %7.1f ns alone %7.1f ns with the MFMAs  (%5.1f%% of the smaller hidden)\n", name, a, b, hidden);
}

template <int PIPE, int SUM>
void tile_row(const char* name, float* sink) {
  const float a = step_ns([&] { hipLaunchKernelGGL((tile_probe<PIPE, SUM>), dim3(kCUs), dim3(768), 0, nullptr, sink); });
  std::printf("  %-44s %7.1f ns per key tile\n", name, a);
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

  // softmax instruction mix beside MFMAs, 3 waves per SIMD
  float* msink = nullptr;
  check(hipMalloc(&msink, size_t(kCUs) * 768 * sizeof(float)), "hipMalloc");
  const float mf = step_ns([&] { hipLaunchKernelGGL(mix_mfma_only, dim3(kCUs), dim3(768), 0, nullptr, msink); });
  std::printf("softmax vector work of one P.V step (per SIMD: 3 waves x 32 scores per lane) beside its 8 MFMAs\n");
  std::printf("  %-22s %7.1f ns\n", "8 MFMAs alone", mf);
  mix_row<MIX_EXP_PACK_DOT2>("exp2 + pack + v_dot2", msink, mf);
  mix_row<MIX_EXP_PACK_ADD>("exp2 + pack + fp32 add", msink, mf);
  mix_row<MIX_EXP>("exp2", msink, mf);
  mix_row<MIX_PACK>("pack (cvt_pk_bf16)", msink, mf);
  mix_row<MIX_DOT2>("v_dot2", msink, mf);
  mix_row<MIX_FMA>("fma", msink, mf);
  std::printf("whole key tile (16 MFMAs + softmax) per SIMD, 3 waves\n");
  tile_row<0, 0>("serial, v_dot2 row sums", msink);
  tile_row<0, 1>("serial, fp32-add row sums", msink);
  tile_row<1, 0>("next scores interleaved, v_dot2 row sums", msink);
  tile_row<1, 1>("next scores interleaved, fp32-add row sums", msink);
  check(hipFree(msink), "hipFree");

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
