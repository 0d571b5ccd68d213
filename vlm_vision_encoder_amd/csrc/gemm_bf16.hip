// bf16 GEMM family on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16):
//   C[M][N] = A[M][K] * B[N][K]^T  (fp32 accumulation)
// with three A-operand loaders and five epilogues, covering every linear map
// of the tower:
//   patch embedding   A = im2col(pixels) (fp32 -> bf16 in the load), C fp32
//   q,k,v             A = y, B rows from wq|wk|wv, epilogue rotates q and k
//   out-projection    A = attention output, epilogue adds into the residual
//   MLP gate/up       B rows interleave gate and up, epilogue silu(g) * u
//   MLP down          epilogue adds into the residual
//   merger            A = 2x2 gather of the residual (fp32 -> bf16 in the load)
// ("Mistral 3" (KerasFormers), Mistral3VisionModel and Mistral3Model table.)
//
// Tiling: BM x BN x 64 block tile, 256 threads = 4 waves in a 2 x 2 grid,
// each wave owns a (BM/2) x (BN/2) tile of 32x32 MFMA blocks.  A and B tiles
// are staged through registers into double-buffered LDS (one barrier per
// k-tile); rows are 128 bytes = 8 chunks of 16 bytes, and chunk c of row r is
// stored at c ^ (r & 7) so the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks.  Blocks are renumbered so each XCD (blocks b with the same
// b % 8) works on a contiguous range of output tiles, which keeps the A panel
// and the weights it shares in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

constexpr int BK = 64;

__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = nblocks >> 3, rem = nblocks & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

template <int AM>
struct ARow {
  const char* p0 = nullptr;  // A_DENSE: row pointer; A_IM2COL: image pixel base at the patch origin
  int32_t hw = 0, w = 0;     // A_IM2COL: plane stride, row stride (elements)
  int32_t src[4] = {0, 0, 0, 0};  // A_MERGE: source patch rows
};

// Loads the 8 bf16 values A[row][k0 .. k0+8) for one thread's chunk.
template <int AM>
__device__ __forceinline__ u32x4 load_a_chunk(const GemmArgs& g, const ARow<AM>& r, int k0) {
  if constexpr (AM == A_DENSE) {
    return *reinterpret_cast<const u32x4*>(r.p0 + size_t(k0) * 2);
  } else if constexpr (AM == A_IM2COL) {
    const int p = g.maps.patch, pp = p * p;
    const float* base = reinterpret_cast<const float*>(r.p0);
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e;
      float v = 0.f;
      if (k < g.K) {
        const int ch = k / pp, rem = k - ch * pp;
        const int u = rem / p, x = rem - u * p;
        v = base[size_t(ch) * r.hw + size_t(u) * r.w + x];
      }
      f[e] = v;
    }
    return pack8(f);
  } else {
    const int D = g.hidden;
    const int q = k0 / D, ch = k0 - q * D;
    const float* src = reinterpret_cast<const float*>(g.A) + size_t(r.src[q]) * D + ch;
    const floatx4 a = *reinterpret_cast<const floatx4*>(src);
    const floatx4 b = *reinterpret_cast<const floatx4*>(src + 4);
    float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return pack8(f);
  }
}

template <int AM>
__device__ __forceinline__ ARow<AM> a_row(const GemmArgs& g, int m) {
  ARow<AM> r;
  m = m < g.M ? m : g.M - 1;  // rows past M are computed but never stored
  if constexpr (AM == A_DENSE) {
    r.p0 = reinterpret_cast<const char*>(g.A) + size_t(m) * g.lda * 2;
  } else if constexpr (AM == A_IM2COL) {
    const int img = g.maps.rowinfo[2 * m];
    const int rc = g.maps.rowinfo[2 * m + 1];
    const ImageMeta mt = g.maps.meta[img];
    const int p = g.maps.patch;
    const int pr = rc >> 16, pc = rc & 0xffff;
    r.hw = mt.H * mt.W;
    r.w = mt.W;
    r.p0 = reinterpret_cast<const char*>(g.pixels + pix_offset(mt) + size_t(pr * p) * mt.W + pc * p);
  } else {
    const int4 s = reinterpret_cast<const int4*>(g.maps.msrc)[m];
    r.src[0] = s.x; r.src[1] = s.y; r.src[2] = s.z; r.src[3] = s.w;
  }
  return r;
}

// Row pointer of B-tile row n (global output column n of this GEMM).
template <int BMD>
__device__ __forceinline__ const char* b_row(const GemmArgs& g, int n) {
  if constexpr (BMD == B_ONE) {
    n = n < g.N ? n : g.N - 1;
    return reinterpret_cast<const char*>(g.B0) + size_t(n) * g.ldb * 2;
  } else if constexpr (BMD == B_QKV) {
    const int D = g.hidden;
    const int which = n / D, rr = n - which * D;
    const void* b = which == 0 ? g.B0 : (which == 1 ? g.B1 : g.B2);
    return reinterpret_cast<const char*>(b) + size_t(rr) * g.ldb * 2;
  } else {
    // 32-row blocks alternate gate, up: rows [64j, 64j+32) -> gate rows
    // [32j, 32j+32), rows [64j+32, 64j+64) -> up rows [32j, 32j+32).
    const int j = (n >> 6) * 32 + (n & 31);
    const void* b = (n & 32) ? g.B1 : g.B0;
    return reinterpret_cast<const char*>(b) + size_t(j) * g.ldb * 2;
  }
}

template <int BM, int BN, int AM, int BMD, int EM>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int AC = BM * 8 / 256;  // 16-byte A chunks per thread per k-tile
  constexpr int BC = BN * 8 / 256;
  static_assert(AC >= 1 && BC >= 1, "tile too small");
  static_assert(EM != E_SILU_MUL || (TN % 2) == 0, "silu-mul needs gate/up block pairs in a wave");

  __shared__ u32x4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (BMD == B_GATEUP ? 2 * g.N : g.N) / BN;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  // Per-thread global row descriptors (fixed across k-tiles).
  ARow<AM> arow[AC];
  const char* brow[BC];
#pragma unroll
  for (int i = 0; i < AC; ++i) arow[i] = a_row<AM>(g, m0 + ((tid + 256 * i) >> 3));
#pragma unroll
  for (int i = 0; i < BC; ++i) brow[i] = b_row<BMD>(g, n0 + ((tid + 256 * i) >> 3));
  const int cchunk = tid & 7;

  u32x4 ra[AC], rb[BC];
  auto gload = [&](int kt) {
    const int k0 = kt * BK + cchunk * 8;
#pragma unroll
    for (int i = 0; i < AC; ++i) ra[i] = load_a_chunk<AM>(g, arow[i], k0);
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      if constexpr (AM == A_IM2COL) {
        // patch kernel rows have 3 p^2 elements: ragged K and rows that are
        // only 2-byte aligned, so load element by element
        const uint16_t* src = reinterpret_cast<const uint16_t*>(brow[i]) + k0;
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (k0 + e < g.K) ? src[e] : uint16_t(0);
        u32x4 z;
        z[0] = h[0] | (uint32_t(h[1]) << 16);
        z[1] = h[2] | (uint32_t(h[3]) << 16);
        z[2] = h[4] | (uint32_t(h[5]) << 16);
        z[3] = h[6] | (uint32_t(h[7]) << 16);
        rb[i] = z;
      } else {
        rb[i] = *reinterpret_cast<const u32x4*>(brow[i] + size_t(k0) * 2);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int row = (tid + 256 * i) >> 3;
      lds[buf][row * 8 + (cchunk ^ (row & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int row = (tid + 256 * i) >> 3;
      lds[buf][(BM + row) * 8 + (cchunk ^ (row & 7))] = rb[i];
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = (g.K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const u32x4* sa = lds[buf];
    const u32x4* sb = lds[buf] + BM * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = 2 * ks + lhalf;
      u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + 32 * i + lrow;
        fa[i] = sa[row * 8 + (ch ^ (row & 7))];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + 32 * j + lrow;
        fb[j] = sb[row * 8 + (ch ^ (row & 7))];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // C layout of a 32x32 block: lane holds column (lane & 31) and rows
  // 8*(v/4) + 4*(lane/32) + (v%4), v = 0..15.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * lhalf + (v & 3);
      const bool ok = row < g.M;
      if constexpr (EM == E_SILU_MUL) {
#pragma unroll
        for (int jj = 0; jj < TN / 2; ++jj) {
          const float gt = acc[i][2 * jj][v], up = acc[i][2 * jj + 1][v];
          const float s = gt / (1.f + __expf(-gt)) * up;
          const int col = (n0 + wn * WN + 64 * jj) / 2 + lrow;
          if (ok) reinterpret_cast<bf16*>(g.C)[size_t(row) * g.ldc + col] = (bf16)s;
        }
      } else if constexpr (EM == E_QKV_ROPE) {
        int rc = 0;
        if (ok) rc = g.maps.rowinfo[2 * row + 1];
        const int pr = rc >> 16, pc = rc & 0xffff;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WN + 32 * j + lrow;
          float x = acc[i][j][v];
          const float xp = swap_adjacent(x);
          if (col < 2 * g.hidden) {
            const int d = col & 63, pair = d >> 1;
            const int axis = pair >> 4, m = pair & 15;
            const int pos = axis ? pc : pr;
            const float2 cs = reinterpret_cast<const float2*>(g.maps.rope)[(axis * g.maps.rope_maxpos + pos) * 16 + m];
            // even lane: x0 cos - x1 sin ; odd lane: x0 sin + x1 cos
            x = (d & 1) ? (xp * cs.y + x * cs.x) : (x * cs.x - xp * cs.y);
          }
          if (ok) reinterpret_cast<bf16*>(g.C)[size_t(row) * g.ldc + col] = (bf16)x;
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WN + 32 * j + lrow;
          if (!ok || col >= g.N) continue;
          const size_t o = size_t(row) * g.ldc + col;
          if constexpr (EM == E_STORE) {
            reinterpret_cast<bf16*>(g.C)[o] = (bf16)acc[i][j][v];
          } else if constexpr (EM == E_STORE_F32) {
            reinterpret_cast<float*>(g.C)[o] = acc[i][j][v];
          } else {
            reinterpret_cast<float*>(g.C)[o] += acc[i][j][v];
          }
        }
      }
    }
  }
}

template <int BM, int BN, int AM, int BMD, int EM>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  const int ncols = (BMD == B_GATEUP) ? 2 * g.N : g.N;
  if (ncols % BN) return hipErrorInvalidValue;
  const int tiles = ((g.M + BM - 1) / BM) * (ncols / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AM, BMD, EM>), dim3(tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16(GemmKind kind, const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  switch (kind) {
    case GEMM_PATCH:  return launch<128, 128, A_IM2COL, B_ONE, E_STORE_F32>(g, s);
    case GEMM_QKV:    return launch<128, 128, A_DENSE, B_QKV, E_QKV_ROPE>(g, s);
    case GEMM_OPROJ:  return launch<128, 128, A_DENSE, B_ONE, E_ADD_F32>(g, s);
    case GEMM_GATEUP: return launch<128, 128, A_DENSE, B_GATEUP, E_SILU_MUL>(g, s);
    case GEMM_DOWN:   return launch<128, 128, A_DENSE, B_ONE, E_ADD_F32>(g, s);
    case GEMM_MERGE:  return launch<128, 128, A_MERGE, B_ONE, E_STORE>(g, s);
    case GEMM_PLAIN:  return launch<128, 128, A_DENSE, B_ONE, E_STORE>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pv
