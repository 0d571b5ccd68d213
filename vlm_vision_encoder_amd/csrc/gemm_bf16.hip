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
// stored at c ^ ((r >> 1) & 7): the LDS has 64 four-byte banks and serves a
// 16-byte read for 16 lanes (16 consecutive rows) per pass, which then differ
// in (row parity, chunk) and hit distinct banks.  Blocks are renumbered so each XCD (blocks b with the same
// b % 8) works on a contiguous range of output tiles, which keeps the A panel
// and the weights it shares in that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 64;
constexpr int kNumCUs = 256;  // MI355X: 8 XCDs x 32 CUs
// tile rows per group of the persistent dense GEMM's tile order
#ifndef PV_GEMM_GM
#define PV_GEMM_GM 4
#endif
#ifndef PV_GEMM_SCHED
#define PV_GEMM_SCHED 1
#endif

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
// The same for rows of CH chunks (CH = 8: 128-byte rows, as swz; CH = 4:
// 64-byte rows, where four consecutive rows already span the 64 banks, so the
// 16 rows of a pass must differ in (row % 4, chunk): chunk ^ ((row >> 2) & 3)).
template <int CH>
__device__ __forceinline__ int swzc(int row) {
  static_assert(CH == 8 || CH == 4, "row width");
  if constexpr (CH == 8) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

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

// fp32 values -> bf16 hi and bf16 lo = bf16(x - hi): hi + lo carries about
// 16 mantissa bits, so a product over both halves keeps the fp32 operand's
// precision to within the accumulation error.
__device__ __forceinline__ void split8(const float* f, u32x4& hi, u32x4& lo) {
  hi = pack8(f);
  float r[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[2 * e] = f[2 * e] - lo_bf16(hi[e]);
    r[2 * e + 1] = f[2 * e + 1] - hi_bf16(hi[e]);
  }
  lo = pack8(r);
}

// Loads A[row][k0 .. k0+8) for one thread's chunk: bf16 rows are copied; the
// fp32 operands (pixels, residual) are split into bf16 hi and lo parts.
template <int AM>
__device__ __forceinline__ void load_a_chunk(const GemmArgs& g, const ARow<AM>& r, int k0, u32x4& hi, u32x4& lo) {
  if constexpr (AM == A_DENSE) {
    hi = *reinterpret_cast<const u32x4*>(r.p0 + size_t(k0) * 2);
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
    split8(f, hi, lo);
  } else {
    const int D = g.hidden;
    const int q = k0 / D, ch = k0 - q * D;
    const float* src = reinterpret_cast<const float*>(g.A) + size_t(r.src[q]) * D + ch;
    const floatx4 a = *reinterpret_cast<const floatx4*>(src);
    const floatx4 b = *reinterpret_cast<const floatx4*>(src + 4);
    float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    split8(f, hi, lo);
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

// Epilogue of one wave's TM x TN grid of 32x32 accumulator blocks whose
// top-left output element is (m_base, n_base).  C layout of a 32x32 block:
// lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + (v%4).
template <int EM, int TM, int TN>
__device__ __forceinline__ void epilogue(const GemmArgs& g, floatx16 (&acc)[TM][TN], int m_base, int n_base,
                                         int lrow, int lhalf) {
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m_base + 32 * i + 8 * (v >> 2) + 4 * lhalf + (v & 3);
      const bool ok = row < g.M;
      if constexpr (EM == E_SILU_MUL) {
#pragma unroll
        for (int jj = 0; jj < TN / 2; ++jj) {
          const float gt = acc[i][2 * jj][v], up = acc[i][2 * jj + 1][v];
          const float sv = gt / (1.f + __expf(-gt)) * up;
          const int col = (n_base + 64 * jj) / 2 + lrow;
          if (ok) reinterpret_cast<bf16*>(g.C)[size_t(row) * g.ldc + col] = (bf16)sv;
        }
      } else if constexpr (EM == E_QKV_ROPE) {
        int rc = 0;
        if (ok) rc = g.maps.rowinfo[2 * row + 1];
        const int pr = rc >> 16, pc = rc & 0xffff;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n_base + 32 * j + lrow;
          float x = acc[i][j][v];
          const float xp = swap_adjacent(x);
          if (col < 2 * g.hidden) {
            const int d = col & 63, pair = d >> 1;
            const int axis = pair >> 4, m = pair & 15;
            const int pos = axis ? pc : pr;
            const float2 cs = reinterpret_cast<const float2*>(g.maps.rope)[(axis * g.maps.rope_maxpos + pos) * 16 + m];
            // even lane: x0 cos - x1 sin ; odd lane: x0 sin + x1 cos
            x = (d & 1) ? (xp * cs.y + x * cs.x) : (x * cs.x - xp * cs.y);
            // q leaves in exp2 units of the attention softmax: times
            // log2(e)/sqrt(64), before its single rounding to bf16
            if (col < g.hidden) x *= 0.18033688011112042f;
          }
          if (ok) reinterpret_cast<bf16*>(g.C)[size_t(row) * g.ldc + col] = (bf16)x;
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n_base + 32 * j + lrow;
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
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int AC = BM * 8 / 256;  // 16-byte A chunks per thread per k-tile
  constexpr int BC = BN * 8 / 256;
  static_assert(AC >= 1 && BC >= 1, "tile too small");
  static_assert(EM != E_SILU_MUL || (TN % 2) == 0, "silu-mul needs gate/up block pairs in a wave");
  // fp32 A operands (pixels, residual) run as two bf16 products, hi and lo
  constexpr bool SPLIT = AM != A_DENSE;
  constexpr int AROWS = SPLIT ? 2 * BM : BM;  // LDS rows of the A tile(s)

  __shared__ u32x4 lds[2][(AROWS + BN) * 8];

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

  u32x4 ra[AC], ral[SPLIT ? AC : 1], rb[BC];
  auto gload = [&](int kt) {
    const int k0 = kt * BK + cchunk * 8;
#pragma unroll
    for (int i = 0; i < AC; ++i) load_a_chunk<AM>(g, arow[i], k0, ra[i], ral[SPLIT ? i : 0]);
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
      lds[buf][row * 8 + (cchunk ^ swz(row))] = ra[i];
      if constexpr (SPLIT) lds[buf][(BM + row) * 8 + (cchunk ^ swz(row))] = ral[i];
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int row = (tid + 256 * i) >> 3;
      lds[buf][(AROWS + row) * 8 + (cchunk ^ swz(row))] = rb[i];
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
    const u32x4* sb = lds[buf] + AROWS * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = 2 * ks + lhalf;
      u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + 32 * i + lrow;
        fa[i] = sa[row * 8 + (ch ^ swz(row))];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + 32 * j + lrow;
        fb[j] = sb[row * 8 + (ch ^ swz(row))];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
      if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = BM + wm * WM + 32 * i + lrow;
          fa[i] = sa[row * 8 + (ch ^ swz(row))];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
      }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  epilogue<EM, TM, TN>(g, acc, m0 + wm * WM, n0 + wn * WN, lrow, lhalf);
}


// Epilogue through LDS: each 32x32 accumulator block is written to a per-wave
// LDS scratch in row-major order and read back so that every lane owns 8
// consecutive outputs of one row (bf16: one 16-byte store) or 4 consecutive
// fp32 values, which turns 16 scattered 2/4-byte global accesses per lane and
// block into 2 (bf16) or 4 + 4 (fp32 read-modify-write) 16-byte ones.
//
// fp32 staging uses 32-float rows with row r stored at r ^ ((r >> 2) & 1):
// the MFMA layout writes rows R and R + 4 in one instruction, which then fall
// in opposite halves of the 64 banks; read-back lanes that share a 16-lane
// pass cover (row parity, 16-byte chunk) once each.
//
// RoPE (q and k columns) is applied after the read-back, where a lane holds 4
// consecutive rotation pairs of one patch: their cos/sin are 32 contiguous
// bytes of the table.  silu(gate) * up is applied in the MFMA layout, where
// gate and up of one unit sit in the same lane.
// scratch: LDS private to the wave, >= SR * 32 floats (fp32 outputs go
// through it SR = 32 or 16 rows at a time), >= 32 * 32 floats for the q,k,v
// epilogue and >= 32 * 20 floats for bf16 outputs.
__device__ __forceinline__ int stage_row(int r) { return r ^ ((r >> 2) & 1); }

// Read-back layout of the fp32 epilogue: pass h, iteration it of block
// (i, j) gives a lane row (lane >> 3) + 8 * it + h * SR, columns 4 * (lane & 7)
// .. +3.  load_residual fetches the residual values of those positions ahead
// of time (E_ADD_F32), so the read-modify-write does not wait for them.
template <int TM, int TN>
struct Residual {
  floatx4 v[TM][TN][4];
};
template <int TM, int TN>
__device__ __forceinline__ void load_residual(const GemmArgs& g, Residual<TM, TN>& res, int m_base, int n_base,
                                              int lane) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = m_base + 32 * i + (lane >> 3) + 8 * it, col = n_base + 32 * j + 4 * (lane & 7);
        const int rr = row < g.M ? row : g.M - 1;  // rows past M are loaded but never stored
        res.v[i][j][it] =
            *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(g.C) + size_t(rr) * g.ldc + col);
      }
}

template <int EM, int TM, int TN, int SR = 32>
__device__ __forceinline__ void epilogue_lds(const GemmArgs& g, floatx16 (&acc)[TM][TN], int m_base, int n_base,
                                             int lane, float* scratch, const Residual<TM, TN>* res = nullptr) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  if constexpr (EM == E_ADD_F32 || EM == E_STORE_F32) {
    static_assert(SR == 32 || SR == 16, "staging rows");
    constexpr int VP = SR / 2;  // accumulator values per lane and pass
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int h = 0; h < 32 / SR; ++h) {
#pragma unroll
          for (int v = 0; v < VP; ++v)
            scratch[stage_row(8 * (v >> 2) + 4 * lhalf + (v & 3)) * 32 + lrow] = acc[i][j][h * VP + v];
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
          for (int it = 0; it < SR / 8; ++it) {
            const int r = (lane >> 3) + 8 * it, c4 = 4 * (lane & 7);
            const floatx4 val = *reinterpret_cast<const floatx4*>(scratch + stage_row(r) * 32 + c4);
            const int row = m_base + 32 * i + h * SR + r, col = n_base + 32 * j + c4;
            if (row < g.M) {
              floatx4* dst = reinterpret_cast<floatx4*>(reinterpret_cast<float*>(g.C) + size_t(row) * g.ldc + col);
              if constexpr (EM == E_ADD_F32) {
                static_assert(EM != E_ADD_F32 || SR == 32, "prefetched residual assumes one pass per block");
                *dst = (res ? res->v[i][j][it] : *dst) + val;
              } else {
                *dst = val;
              }
            }
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass's writes
        }
  } else if constexpr (EM == E_QKV_ROPE) {
    const float4* rope = reinterpret_cast<const float4*>(g.maps.rope);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int rc[2];  // packed (row, col) of the patch of the two rows this lane stores
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int row = m_base + 32 * i + (lane >> 2) + 16 * it;
        rc[it] = row < g.M ? g.maps.rowinfo[2 * row + 1] : 0;
      }
#pragma unroll
      for (int jb = 0; jb < TN; ++jb) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          scratch[stage_row(8 * (v >> 2) + 4 * lhalf + (v & 3)) * 32 + lrow] = acc[i][jb][v];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int r = (lane >> 2) + 16 * it, c8 = 8 * (lane & 3);
          // the two 16-byte halves are read in the order that keeps a pass
          // conflict-free, then put back in column order
          const int f = (r >> 1) & 1;
          const float* src = scratch + stage_row(r) * 32 + c8;
          const floatx4 first = *reinterpret_cast<const floatx4*>(src + 4 * f);
          const floatx4 second = *reinterpret_cast<const floatx4*>(src + 4 * (1 - f));
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = f ? second[e] : first[e];
            x[4 + e] = f ? first[e] : second[e];
          }
          const int row = m_base + 32 * i + r, col0 = n_base + 32 * jb + c8;
          if (col0 < 2 * g.hidden) {
            // dims d0 .. d0+7 of a head = rotation pairs m0 .. m0+3 of one axis
            const int pair0 = (col0 & 63) >> 1;
            const int axis = pair0 >> 4, m0 = pair0 & 15;
            const int pos = axis ? (rc[it] & 0xffff) : (rc[it] >> 16);
            const float4* cs = rope + ((axis * g.maps.rope_maxpos + pos) * 16 + m0) / 2;
            const float4 c01 = cs[0], c23 = cs[1];  // {cos, sin} of pairs m0, m0+1 | m0+2, m0+3
            const float cv[4] = {c01.x, c01.z, c23.x, c23.z}, sv[4] = {c01.y, c01.w, c23.y, c23.w};
            // q leaves in exp2 units of the attention softmax: times
            // log2(e)/sqrt(64), before its single rounding to bf16
            const float sc = col0 < g.hidden ? 0.18033688011112042f : 1.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float x0 = x[2 * k], x1 = x[2 * k + 1];
              x[2 * k] = (x0 * cv[k] - x1 * sv[k]) * sc;
              x[2 * k + 1] = (x0 * sv[k] + x1 * cv[k]) * sc;
            }
          }
          if (row < g.M)
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + size_t(row) * g.ldc + col0) = pack8(x);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next block's writes
      }
    }
  } else {
    // bf16 outputs: one 32 x 32 bf16 block staged per round
    constexpr int LDH = 40;  // row stride (bf16 elements), 80 bytes
    uint16_t* sh = reinterpret_cast<uint16_t*>(scratch);
    constexpr int NB = (EM == E_SILU_MUL) ? TN / 2 : TN;  // output blocks per row of blocks
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        int ocol0;  // first output column of the block
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rib = 8 * (v >> 2) + 4 * lhalf + (v & 3);  // row in block
          float x;
          if constexpr (EM == E_SILU_MUL) {
            // silu(g) * u = g * u / (1 + e^-g); the approximate reciprocal
            // (1 ulp) is far inside the bf16 rounding that follows
            const float gt = acc[i][2 * jb][v], up = acc[i][2 * jb + 1][v];
            x = gt * up * __builtin_amdgcn_rcpf(1.f + __expf(-gt));
            ocol0 = (n_base + 64 * jb) / 2;
          } else {
            x = acc[i][jb][v];
            ocol0 = n_base + 32 * jb;
          }
          sh[rib * LDH + lrow] = __builtin_bit_cast(uint16_t, (bf16)x);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int r = (lane >> 2) + 16 * it, c8 = 8 * (lane & 3);
          const u32x4 val = *reinterpret_cast<const u32x4*>(sh + r * LDH + c8);
          const int row = m_base + 32 * i + r;
          if (row < g.M)
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + size_t(row) * g.ldc + ocol0 + c8) = val;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
      }
    }
  }
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Dense-A GEMM (q,k,v, out-projection, gate/up, down), persistent: each
// workgroup walks a fixed list of output tiles, and the global -> LDS load
// ring (global_load_lds_dwordx4, NS stages, no VGPR staging) runs over the
// flattened sequence of (tile, k-tile) steps, so the next tile's first
// k-tiles are already in flight while the current tile finishes and writes
// its epilogue.  The chunk swizzle is applied by choosing which chunk each
// lane fetches.  Waves are arranged WMW x WNW; each computes a
// (BM/WMW) x (BN/WNW) tile of 32x32 MFMA blocks.  Tiles are numbered so the
// workgroups of one XCD (blocks b with equal b % 8) share a contiguous range
// of tiles, grouped GM tile rows at a time, keeping the A and B panels they
// share in that XCD's L2.
template <int BM, int BN, int WMW, int WNW, int NS, int BKT, int BMD, int EM>
__global__ __launch_bounds__(WMW * WNW * 64) void gemm_dense_kernel(GemmArgs g) {
  constexpr int NW = WMW * WNW, NT = NW * 64;
  constexpr int CH = BKT / 8;                    // 16-byte chunks per tile row
  constexpr int TMW = BM / WMW, TNW = BN / WNW;  // wave tile
  constexpr int TM = TMW / 32, TN = TNW / 32;
  constexpr int A_LD = BM * CH / NT, B_LD = BN * CH / NT;  // global_load_lds per thread per k-tile
  constexpr int LDT = A_LD + B_LD;
  static_assert(A_LD >= 1 && B_LD >= 1 && (BM * CH) % NT == 0 && (BN * CH) % NT == 0, "tile/thread mismatch");
  static_assert(EM != E_SILU_MUL || (TN % 2) == 0, "silu-mul needs gate/up block pairs in a wave");
  static_assert((NS - 2) * LDT <= 63, "vmcnt range");

  __shared__ u32x4 lds[NS][(BM + BN) * CH];
  constexpr int kScratchFloats = (BM + BN) * CH * 4 / NW;  // per-wave slice of one stage
  constexpr int kEpiRows = kScratchFloats >= 32 * 32 ? 32 : 16;
  static_assert(kScratchFloats >= 16 * 32 && kScratchFloats >= 32 * 20 && (EM != E_QKV_ROPE || kScratchFloats >= 32 * 32),
                "epilogue scratch does not fit a stage");

  // the wave index is uniform: keeping it scalar puts the LDS destinations of
  // the direct loads (M0) on the scalar unit
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int tiles_n = (BMD == B_GATEUP ? 2 * g.N : g.N) / BN;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int ntiles = tiles_m * tiles_n;
  const int KT = g.K / BKT;
  // k-tiles of B: A's K may run over B's K twice (hi | lo halves of A)
  const int KTB = g.kb > 0 ? g.kb / BKT : KT;

  // this workgroup's tiles: the blocks b with equal x = b % 8 (one XCD, nx
  // of them populated) own tiles [lo_x, hi_x); the nb_x blocks of XCD x
  // (index j = b / 8) take every nb_x-th of them
  const int nblk = gridDim.x, b = blockIdx.x;
  const int nx = nblk < 8 ? nblk : 8;
  const int x = b & 7, j = b >> 3;
  const int nb_x = (nblk - x + 7) >> 3;
  const int lo_x = int((long long)ntiles * x / nx), hi_x = int((long long)ntiles * (x + 1) / nx);
  const int my_tiles = (hi_x - lo_x > j) ? (hi_x - lo_x - j + nb_x - 1) / nb_x : 0;
  const int steps = my_tiles * KT;
  // logical tile L -> (tm, tn) in groups of GM tile rows, column-major inside
  // a group: the ~32 consecutive tiles an XCD runs at once form a
  // GM x (32/GM) block, so L2 serves both their A and their B panels
  auto tile_of = [&](int i) { return lo_x + j + i * nb_x; };
  auto tile_mn = [&](int L, int& tm, int& tn) {
    const int per_group = PV_GEMM_GM * tiles_n;
    const int grp = L / per_group, first_m = grp * PV_GEMM_GM;
    const int rows = (tiles_m - first_m) < PV_GEMM_GM ? (tiles_m - first_m) : PV_GEMM_GM;
    const int r = L - grp * per_group;
    tm = first_m + r % rows;
    tn = r / rows;
  };

  // load plan: wave instruction q of this wave fills LDS slots
  // [(wave * X_LD + q) * 64, +64) of the A (B) tile; lane l takes slot p.
  const char* ga[A_LD];
  const char* gb[B_LD];
  auto set_rows = [&](int t) {
    int tm, tn;
    tile_mn(t, tm, tn);
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      const int p = (wave * A_LD + q) * 64 + lane;
      const int P = p / CH, gc = (p % CH) ^ swzc<CH>(P);
      int m = tm * BM + P;
      m = m < g.M ? m : g.M - 1;
      ga[q] = reinterpret_cast<const char*>(g.A) + (size_t(m) * g.lda + gc * 8) * 2;
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q) {
      const int p = (wave * B_LD + q) * 64 + lane;
      const int P = p / CH, gc = (p % CH) ^ swzc<CH>(P);
      gb[q] = b_row<BMD>(g, tn * BN + P) + gc * 16;
    }
  };
  // (the global source is passed as a uint16_t pointer: with a char pointer
  // the host pass drops the kernel's launch stub without a diagnostic)
  int is_step = 0, is_kt = 0, is_tile = 0;  // next step to issue
  auto issue_next = [&]() {
    if (is_kt == 0) set_rows(tile_of(is_tile));
    const int st = is_step % NS;
    const size_t koff = size_t(is_kt) * BKT * 2;
    const size_t koffb = size_t(is_kt < KTB ? is_kt : is_kt - KTB) * BKT * 2;
#pragma unroll
    for (int q = 0; q < A_LD; ++q)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(ga[q] + koff),
                                       (lds_void*)&lds[st][(wave * A_LD + q) * 64], 16, 0, 0);
#pragma unroll
    for (int q = 0; q < B_LD; ++q)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(gb[q] + koffb),
                                       (lds_void*)&lds[st][BM * CH + (wave * B_LD + q) * 64], 16, 0, 0);
    ++is_step;
    if (++is_kt == KT) {
      is_kt = 0;
      ++is_tile;
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jn = 0; jn < TN; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;

  for (int st = 0; st < NS - 1; ++st)
    if (is_step < steps) issue_next();

  int kt = 0, ti = 0;
  for (int step = 0; step < steps; ++step) {
    // step has landed once at most (steps issued after it) x LDT loads of
    // this thread are outstanding; the barrier makes every thread's part
    // visible and frees the stage read in the previous step
    if (step + NS - 2 < steps) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LDT));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
    if (is_step < steps) issue_next();
    // the residual of an accumulating epilogue is fetched while the tile's
    // last k-step runs
    Residual<TM, TN> res;
    if constexpr (EM == E_ADD_F32) {
      if (kt == KT - 1) {
        int tm, tn;
        tile_mn(tile_of(ti), tm, tn);
        load_residual<TM, TN>(g, res, tm * BM + wm * TMW, tn * BN + wn * TNW, lane);
      }
    }
    const u32x4* sa = lds[step % NS];
    const u32x4* sb = lds[step % NS] + BM * CH;
    // fragments of k-substep ks + 1 are read while the MFMAs of ks run
    constexpr int KS = BKT / 16;
    u32x4 fa[2][TM], fb[2][TN];
    auto read_frags = [&](int ks, u32x4 (&ra)[TM], u32x4 (&rb)[TN]) {
      const int ch = 2 * ks + lhalf;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * TMW + 32 * i + lrow;
        ra[i] = sa[row * CH + (ch ^ swzc<CH>(row))];
      }
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) {
        const int row = wn * TNW + 32 * jn + lrow;
        rb[jn] = sb[row * CH + (ch ^ swzc<CH>(row))];
      }
    };
    read_frags(0, fa[0], fb[0]);
    static_for<KS>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      if constexpr (ks + 1 < KS) read_frags(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) acc[i][jn] = mfma32x32x16(fa[ks & 1][i], fb[ks & 1][jn], acc[i][jn]);
    });
#if PV_GEMM_SCHED == 1
    // issue order: the first fragments, then per k-substep the next
    // fragments' reads spread between that substep's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
    static_for<KS>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      if constexpr (ks + 1 < KS) {
        constexpr int NMF = TM * TN, NRD = TM + TN, PAIRS = NMF < NRD ? NMF : NRD;
        static_for<PAIRS>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        if constexpr (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
        if constexpr (NRD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PAIRS, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
      }
    });
#endif
    if (++kt == KT) {
      int tm, tn;
      tile_mn(tile_of(ti), tm, tn);
      // the stage just consumed is free until the next step's loads (issued
      // after the next barrier): once every wave is done with it, each wave
      // uses its own slice of it to stage the output
      __syncthreads();
      float* scratch = reinterpret_cast<float*>(lds[step % NS]) + wave * kScratchFloats;
      epilogue_lds<EM, TM, TN, kEpiRows>(g, acc, tm * BM + wm * TMW, tn * BN + wn * TNW, lane, scratch,
                                         EM == E_ADD_F32 ? &res : nullptr);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;
      kt = 0;
      ++ti;
    }
  }
}

template <int BM, int BN, int WMW, int WNW, int NS, int BKT, int BMD, int EM>
hipError_t launch_dense(const GemmArgs& g, hipStream_t s) {
  const int ncols = (BMD == B_GATEUP) ? 2 * g.N : g.N;
  if (ncols % BN || g.K % BKT || g.kb % BKT) return hipErrorInvalidValue;
  if (g.kb > 0 && g.K != 2 * g.kb) return hipErrorInvalidValue;
  const int tiles = ((g.M + BM - 1) / BM) * (ncols / BN);
  // as many workgroups as fit on the chip at once: the LDS ring sets how
  // many a CU holds
  constexpr int kLdsBytes = NS * (BM + BN) * BKT * 2;
  constexpr int kPerCU = (160 * 1024) / kLdsBytes < 2 ? 1 : 2;
  const int grid = tiles < kNumCUs * kPerCU ? tiles : kNumCUs * kPerCU;
  hipLaunchKernelGGL((gemm_dense_kernel<BM, BN, WMW, WNW, NS, BKT, BMD, EM>), dim3(grid), dim3(WMW * WNW * 64), 0, s,
                     g);
  return hipGetLastError();
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

// Tile configurations (BM, BN, waves along M, waves along N, LDS stages, k
// depth of a stage) of the dense GEMMs: wide-N products and the N = hidden
// products.
#ifndef PV_GEMM_CFG_BIG
#define PV_GEMM_CFG_BIG 256, 256, 4, 2, 2, 64
#endif
#ifndef PV_GEMM_CFG_N1K
#define PV_GEMM_CFG_N1K 256, 128, 4, 2, 2, 64
#endif
// q,k,v: 192-column tiles (16 per row of tiles instead of 12) balance the
// 1540 x 1540 image's 48 rows of tiles evenly over the 256 CUs
#ifndef PV_GEMM_CFG_QKV
#define PV_GEMM_CFG_QKV 256, 192, 4, 2, 2, 64
#endif

hipError_t gemm_bf16(GemmKind kind, const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  switch (kind) {
    case GEMM_PATCH:  return launch<128, 128, A_IM2COL, B_ONE, E_STORE_F32>(g, s);
    case GEMM_QKV:    return launch_dense<PV_GEMM_CFG_QKV, B_QKV, E_QKV_ROPE>(g, s);
    case GEMM_OPROJ:  return launch_dense<PV_GEMM_CFG_N1K, B_ONE, E_ADD_F32>(g, s);
    case GEMM_GATEUP: return launch_dense<PV_GEMM_CFG_BIG, B_GATEUP, E_SILU_MUL>(g, s);
    case GEMM_DOWN:   return launch_dense<PV_GEMM_CFG_N1K, B_ONE, E_ADD_F32>(g, s);
    case GEMM_MERGE:  return launch<128, 128, A_MERGE, B_ONE, E_STORE>(g, s);
    case GEMM_PLAIN:  return launch_dense<PV_GEMM_CFG_N1K, B_ONE, E_STORE>(g, s);
    case GEMM_MERGE_F32: return launch<128, 128, A_MERGE, B_ONE, E_STORE_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pv
