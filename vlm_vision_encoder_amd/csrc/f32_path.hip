// fp32 tower kernels: the same GEMM kinds (operand loaders and epilogues) and
// the same block-diagonal attention as the bf16 path, in plain fp32 FMA
// arithmetic on the vector ALUs.  This is the full-precision configuration of
// the tower (small inputs, tight tolerance); the bf16 MFMA kernels are the
// throughput path.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

// A[m][k] of each GEMM kind, fp32.
template <int AM>
__device__ __forceinline__ float a_elem(const GemmArgs& g, int m, int k) {
  if (k >= g.K) return 0.f;
  m = m < g.M ? m : g.M - 1;
  if constexpr (AM == A_DENSE) {
    return reinterpret_cast<const float*>(g.A)[size_t(m) * g.lda + k];
  } else if constexpr (AM == A_IM2COL) {
    const int img = g.maps.rowinfo[2 * m], rc = g.maps.rowinfo[2 * m + 1];
    const ImageMeta mt = g.maps.meta[img];
    const int p = g.maps.patch, pp = p * p;
    const int ch = k / pp, rem = k - ch * pp, u = rem / p, x = rem - u * p;
    const int pr = rc >> 16, pc = rc & 0xffff;
    return g.pixels[pix_offset(mt) + size_t(ch) * mt.H * mt.W + size_t(pr * p + u) * mt.W + pc * p + x];
  } else {
    const int D = g.hidden, q = k / D, ch = k - q * D;
    const int src = g.maps.msrc[4 * m + q];
    return reinterpret_cast<const float*>(g.A)[size_t(src) * D + ch];
  }
}

// B row n of each kind (global column n; gate/up interleaved in 32-row blocks).
template <int BMD>
__device__ __forceinline__ float b_elem(const GemmArgs& g, int n, int k) {
  if (k >= g.K) return 0.f;
  const float* b;
  int r;
  if constexpr (BMD == B_ONE) {
    b = reinterpret_cast<const float*>(g.B0);
    r = n < g.N ? n : g.N - 1;
  } else if constexpr (BMD == B_QKV) {
    const int which = n / g.hidden;
    r = n - which * g.hidden;
    b = reinterpret_cast<const float*>(which == 0 ? g.B0 : (which == 1 ? g.B1 : g.B2));
  } else {
    r = (n >> 6) * 32 + (n & 31);
    b = reinterpret_cast<const float*>((n & 32) ? g.B1 : g.B0);
  }
  return b[size_t(r) * g.ldb + k];
}

// T x T output tile (T = 64 or 32), 256 threads, (T/16)^2 outputs per
// thread, k-tiles of 16.  The 32 x 32 tiles give small products (few rows)
// four times as many workgroups.
template <int AM, int BMD, int EM, int T>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  static_assert(T == 64 || T == 32, "tile");
  static_assert(EM != E_SILU_MUL || T == 64, "silu-mul pairs the 32-column halves of a 64-column tile");
  constexpr int R = T / 16;  // outputs per thread along each side
  __shared__ float as[16][T + 4];
  __shared__ float bs[16][T + 4];
  __shared__ float cs[EM == E_SILU_MUL ? T : 1][T + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (BMD == B_GATEUP ? 2 * g.N : g.N) / T;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * T, n0 = tn * T;
  float acc[R][R] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < T * 16 / 256; ++i) {
      const int e = tid + 256 * i, r = e >> 4, kk = e & 15;
      as[kk][r] = a_elem<AM>(g, m0 + r, k0 + kk);
      bs[kk][r] = b_elem<BMD>(g, n0 + r, k0 + kk);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[R], bv[R];
#pragma unroll
      for (int i = 0; i < R; ++i) av[i] = as[kk][ty * R + i];
#pragma unroll
      for (int j = 0; j < R; ++j) bv[j] = bs[kk][tx * R + j];
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  if constexpr (EM == E_SILU_MUL) {
    // tile columns [0,32) are gate units, [32,64) the matching up units
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) cs[ty * R + i][tx * R + j] = acc[i][j];
    __syncthreads();
    for (int e = tid; e < 64 * 32; e += 256) {
      const int r = e >> 5, cc = e & 31, row = m0 + r;
      if (row >= g.M) continue;
      const float gt = cs[r][cc], up = cs[r][cc + 32];
      reinterpret_cast<float*>(g.C)[size_t(row) * g.ldc + n0 / 2 + cc] = gt / (1.f + expf(-gt)) * up;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = m0 + ty * R + i;
    if (row >= g.M) continue;
    int pr = 0, pc = 0;
    if constexpr (EM == E_QKV_ROPE) {
      const int rc = g.maps.rowinfo[2 * row + 1];
      pr = rc >> 16;
      pc = rc & 0xffff;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int col = n0 + tx * R + j;
      float x = acc[i][j];
      if constexpr (EM == E_QKV_ROPE) {
        if (col < 2 * g.hidden) {
          const int d = col & 63, pair = d >> 1, axis = pair >> 4, mm = pair & 15;
          const float2 csn = reinterpret_cast<const float2*>(g.maps.rope)[(axis * g.maps.rope_maxpos + (axis ? pc : pr)) * 16 + mm];
          const float x0 = acc[i][j & ~1], x1 = acc[i][j | 1];
          x = (d & 1) ? (x0 * csn.y + x1 * csn.x) : (x0 * csn.x - x1 * csn.y);
        }
      }
      const size_t o = size_t(row) * g.ldc + col;
      float* C = reinterpret_cast<float*>(g.C);
      if constexpr (EM == E_ADD_F32) C[o] += x;
      else C[o] = x;
    }
  }
}

// 64 x 64 tiles, or 32 x 32 where 64 x 64 tiles would not give every CU two
// workgroups (not for silu-mul, whose tiles pair gate and up columns)
template <int AM, int BMD, int EM>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  const int ncols = (BMD == B_GATEUP) ? 2 * g.N : g.N;
  if (ncols % 64) return hipErrorInvalidValue;
  const int tiles = ((g.M + 63) / 64) * (ncols / 64);
  if (EM != E_SILU_MUL && tiles < 2 * kNumCUs) {
    const int tiles32 = ((g.M + 31) / 32) * (ncols / 32);
    hipLaunchKernelGGL((gemm_f32_kernel<AM, BMD, EM, (EM == E_SILU_MUL ? 64 : 32)>), dim3(tiles32), dim3(256), 0, s,
                       g);
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<AM, BMD, EM, 64>), dim3(tiles), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

// One workgroup per (64 queries, head), four lanes per query: lane 4 q + j
// holds dims [16 j, 16 j + 16) of query q and of its output.  A key's score
// is the sum of the four lanes' partial dot products, formed by two DPP quad
// permutes (lane ^ 1, then lane ^ 2; the four lanes add the same two pairs,
// so they hold the same bits).  Keys staged through LDS 64 at a time, online
// softmax in fp32.
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v;
}

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  __shared__ float ks[64][65];
  __shared__ float vs[64][65];
  const int heads = a.heads;
  const int item = blockIdx.x / heads, head = blockIdx.x - item * heads;
  const AttnItem it = a.items[item];
  const ImageMeta mt = a.meta[it.image];
  const int n = mt.Hp * mt.Wp, base = mt.patch_base, D = a.hidden;
  const size_t ld = size_t(3) * D;
  const float* qkv = reinterpret_cast<const float*>(a.qkv);
  const int tid = threadIdx.x, d0 = 16 * (tid & 3);
  int t = it.q0 + (tid >> 2);
  const bool valid = t < n;
  t = valid ? t : n - 1;
  float q[16], o[16];
  for (int d = 0; d < 16; ++d) {
    q[d] = qkv[size_t(base + t) * ld + head * 64 + d0 + d] * 0.125f;
    o[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int k0 = 0; k0 < n; k0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 256) {
      const int r = e >> 6, d = e & 63;
      int u = k0 + r;
      u = u < n ? u : n - 1;
      ks[r][d] = qkv[size_t(base + u) * ld + D + head * 64 + d];
      vs[r][d] = qkv[size_t(base + u) * ld + 2 * D + head * 64 + d];
    }
    __syncthreads();
    const int cnt = (n - k0) < 64 ? (n - k0) : 64;
    for (int r = 0; r < cnt; ++r) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < 16; ++d) part = __builtin_fmaf(q[d], ks[r][d0 + d], part);
      const float sc = quad_sum(part);
      const float m_new = fmaxf(m_run, sc);
      const float alpha = expf(m_run - m_new);
      const float p = expf(sc - m_new);
      l_run = l_run * alpha + p;
#pragma unroll
      for (int d = 0; d < 16; ++d) o[d] = o[d] * alpha + p * vs[r][d0 + d];
      m_run = m_new;
    }
  }
  if (!valid) return;
  float* out = reinterpret_cast<float*>(a.out) + size_t(base + t) * D + head * 64 + d0;
  const float inv = 1.f / l_run;
  for (int d = 0; d < 16; ++d) out[d] = o[d] * inv;
}

}  // namespace

hipError_t gemm_f32(GemmKind kind, const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  switch (kind) {
    case GEMM_PATCH:  return launch<A_IM2COL, B_ONE, E_STORE_F32>(g, s);
    case GEMM_QKV:    return launch<A_DENSE, B_QKV, E_QKV_ROPE>(g, s);
    case GEMM_OPROJ:  return launch<A_DENSE, B_ONE, E_ADD_F32>(g, s);
    case GEMM_GATEUP: return launch<A_DENSE, B_GATEUP, E_SILU_MUL>(g, s);
    case GEMM_DOWN:   return launch<A_DENSE, B_ONE, E_ADD_F32>(g, s);
    case GEMM_MERGE:  return launch<A_MERGE, B_ONE, E_STORE>(g, s);
    case GEMM_PLAIN:  return launch<A_DENSE, B_ONE, E_STORE>(g, s);
    case GEMM_MERGE_F32: return launch<A_MERGE, B_ONE, E_STORE>(g, s);
    case GEMM_GELU:
    case GEMM_PLAIN_F32: return hipErrorInvalidValue;  // the deeper projector is bf16 only
  }
  return hipErrorInvalidValue;
}

hipError_t attention_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_items * a.heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pv
