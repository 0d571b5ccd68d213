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

// 64x64 output tile, 256 threads, 4x4 outputs per thread, k-tiles of 16.
template <int AM, int BMD, int EM>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float as[16][68];
  __shared__ float bs[16][68];
  __shared__ float cs[64][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (BMD == B_GATEUP ? 2 * g.N : g.N) / 64;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * 64, n0 = tn * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i, r = e >> 4, kk = e & 15;
      as[kk][r] = a_elem<AM>(g, m0 + r, k0 + kk);
      bs[kk][r] = b_elem<BMD>(g, n0 + r, k0 + kk);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  if constexpr (EM == E_SILU_MUL) {
    // tile columns [0,32) are gate units, [32,64) the matching up units
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) cs[ty * 4 + i][tx * 4 + j] = acc[i][j];
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
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= g.M) continue;
    int pr = 0, pc = 0;
    if constexpr (EM == E_QKV_ROPE) {
      const int rc = g.maps.rowinfo[2 * row + 1];
      pr = rc >> 16;
      pc = rc & 0xffff;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
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

template <int AM, int BMD, int EM>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  const int ncols = (BMD == B_GATEUP) ? 2 * g.N : g.N;
  if (ncols % 64) return hipErrorInvalidValue;
  const int tiles = ((g.M + 63) / 64) * (ncols / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<AM, BMD, EM>), dim3(tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

// One wave per (64 queries, head): each lane owns one query, keys staged
// through LDS 64 at a time, online softmax in fp32.
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float ks[64][65];
  __shared__ float vs[64][65];
  const int heads = a.heads;
  const int item = blockIdx.x / heads, head = blockIdx.x - item * heads;
  const AttnItem it = a.items[item];
  const ImageMeta mt = a.meta[it.image];
  const int n = mt.Hp * mt.Wp, base = mt.patch_base, D = a.hidden;
  const size_t ld = size_t(3) * D;
  const float* qkv = reinterpret_cast<const float*>(a.qkv);
  const int lane = threadIdx.x;
  int t = it.q0 + lane;
  const bool valid = t < n;
  t = valid ? t : n - 1;
  float q[64], o[64];
  for (int d = 0; d < 64; ++d) {
    q[d] = qkv[size_t(base + t) * ld + head * 64 + d] * 0.125f;
    o[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int k0 = 0; k0 < n; k0 += 64) {
    __syncthreads();
    for (int e = lane; e < 64 * 64; e += 64) {
      const int r = e >> 6, d = e & 63;
      int u = k0 + r;
      u = u < n ? u : n - 1;
      ks[r][d] = qkv[size_t(base + u) * ld + D + head * 64 + d];
      vs[r][d] = qkv[size_t(base + u) * ld + 2 * D + head * 64 + d];
    }
    __syncthreads();
    const int cnt = (n - k0) < 64 ? (n - k0) : 64;
    for (int r = 0; r < cnt; ++r) {
      float sc = 0.f;
      for (int d = 0; d < 64; ++d) sc = __builtin_fmaf(q[d], ks[r][d], sc);
      const float m_new = fmaxf(m_run, sc);
      const float alpha = expf(m_run - m_new);
      const float p = expf(sc - m_new);
      l_run = l_run * alpha + p;
      for (int d = 0; d < 64; ++d) o[d] = o[d] * alpha + p * vs[r][d];
      m_run = m_new;
    }
  }
  if (!valid) return;
  float* out = reinterpret_cast<float*>(a.out) + size_t(base + t) * D + head * 64;
  const float inv = 1.f / l_run;
  for (int d = 0; d < 64; ++d) out[d] = o[d] * inv;
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
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_items * a.heads), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pv
