// bf16 GEMM family on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16, and _f16 for
// the MLP gate/up product):
//   C[M][N] = A[M][K] * B[N][K]^T  (fp32 accumulation)
// covering every linear map of the tower ("Mistral 3" (KerasFormers),
// Mistral3VisionModel and Mistral3Model table):
//   patch embedding   A = im2col of the pixels as bf16 hi | lo, C fp32
//   q,k,v             A = y, B rows from wq|wk|wv, epilogue rotates q and k
//   out-projection    A = attention output, epilogue adds into the residual
//   MLP gate/up       A = y (fp16), B rows interleave fp16 copies of gate
//                     and up; epilogue silu(g) * u, written in fp16
//   MLP down          A = silu(g) * u (fp16) against an fp16 copy of the
//                     weights; epilogue adds into the residual
//   merger            A = 2x2 gather of the final residual's bf16 rows, done
//                     by the A-operand loads themselves, then its fp4 low
//                     part (gathered when it was written) against fp4 merge
//                     weights
// The pixels enter as two bf16 halves hi and lo = bf16(x - hi) over a K
// range twice as long, both against the same B rows (GemmArgs::kb): about
// 16 significant bits on bf16 MFMAs.  The final residual enters the merger
// as bf16 plus its low part x - bf16(x) in fp4 (the LOW steps below), and
// the MLP's two products take fp16 operands (the RMS-normalised input, the
// silu * up values and the weights sit well inside fp16's range): about 11
// significant bits either way, at the bf16 MFMA rate.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

// tile rows per group of the persistent dense GEMM's tile order
#ifndef PV_GEMM_GM
#define PV_GEMM_GM 4
#endif
#ifndef PV_GEMM_SCHED
#define PV_GEMM_SCHED 1
#endif

typedef int i32x8 __attribute__((ext_vector_type(8)));

// two 16-byte LDS chunks -> the 32-byte fp8 operand of a 32x32x64 MFMA
__device__ __forceinline__ i32x8 join8(const u32x4& x, const u32x4& y) {
  return i32x8{int(x[0]), int(x[1]), int(x[2]), int(x[3]), int(y[0]), int(y[1]), int(y[2]), int(y[3])};
}
// one 16-byte LDS chunk -> the fp4 operand (its upper 16 bytes unused)
__device__ __forceinline__ i32x8 widen4(const u32x4& x) {
  return i32x8{int(x[0]), int(x[1]), int(x[2]), int(x[3]), 0, 0, 0, 0};
}

// 16-byte chunk swizzle of LDS tile rows of CH chunks.  The LDS has 64
// four-byte banks and serves a 16-byte read for 16 lanes (16 consecutive
// rows) per pass.  CH = 8 (128-byte rows): chunk ^ ((row >> 1) & 7) makes
// those rows differ in (row parity, chunk); CH = 4 (64-byte rows): four
// consecutive rows already span the 64 banks, so they must differ in
// (row % 4, chunk): chunk ^ ((row >> 2) & 3).
template <int CH>
__device__ __forceinline__ int swzc(int row) {
  static_assert(CH == 8 || CH == 4, "row width");
  if constexpr (CH == 8) return (row >> 1) & 7;
  else return (row >> 2) & 3;
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
// Orders one wave's LDS staging writes and the read-back of other lanes'
// values: a compiler barrier only.  A wave's LDS instructions execute in
// issue order, so a read issued after a write sees it without a counter
// wait; the compiler waits for a read's data where the data is used.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ int stage_row(int r) { return r ^ ((r >> 2) & 1); }

// Read-back layout of the fp32 epilogue: pass h, iteration it of block
// (i, j) gives a lane row (lane >> 3) + 8 * it + h * SR, columns 4 * (lane & 7)
// .. +3.  load_residual fetches the residual values of those positions ahead
// of time (E_ADD_F32) for the first NB blocks (b = i * TN + j < NB), so the
// read-modify-write does not wait for them; the other blocks read theirs in
// the epilogue.
template <int NB>
struct Residual {
  floatx4 v[NB][4];
};
template <int TM, int TN, int B, int NB>
__device__ __forceinline__ void load_residual_block(const GemmArgs& g, Residual<NB>& res, int m_base, int n_base,
                                                    int lane) {
  constexpr int i = B / TN, j = B % TN;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = m_base + 32 * i + (lane >> 3) + 8 * it, col = n_base + 32 * j + 4 * (lane & 7);
    const int rr = row < g.M ? row : g.M - 1;  // rows past M are loaded but never stored
    res.v[B][it] = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(g.C) + size_t(rr) * g.ldc + col);
  }
}

// F16O: 16-bit outputs in fp16 (saturated to +-65504) instead of bf16
template <int EM, int TM, int TN, int SR, int NRB, bool F16O>
__device__ __forceinline__ void epilogue_lds(const GemmArgs& g, floatx16 (&acc)[TM][TN], int m_base, int n_base,
                                             int lane, float* scratch, const Residual<NRB>& res) {
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
          wave_lds_order();
#pragma unroll
          for (int it = 0; it < SR / 8; ++it) {
            const int r = (lane >> 3) + 8 * it, c4 = 4 * (lane & 7);
            const floatx4 val = *reinterpret_cast<const floatx4*>(scratch + stage_row(r) * 32 + c4);
            const int row = m_base + 32 * i + h * SR + r, col = n_base + 32 * j + c4;
            if (row < g.M) {
              floatx4* dst = reinterpret_cast<floatx4*>(reinterpret_cast<float*>(g.C) + size_t(row) * g.ldc + col);
              if constexpr (EM == E_ADD_F32) {
                static_assert(EM != E_ADD_F32 || SR == 32, "prefetched residual assumes one pass per block");
                const int b = i * TN + j;
                if (b < NRB) *dst = res.v[b < NRB ? b : 0][it] + val;
                else *dst = *dst + val;
              } else {
                *dst = val;
              }
            }
          }
          wave_lds_order();
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
        wave_lds_order();
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
        wave_lds_order();
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
          } else if constexpr (EM == E_GELU) {
            // GELU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2
            const float a = acc[i][jb][v];
            x = 0.5f * a * (1.f + erff(a * 0.70710678118654752f));
            ocol0 = n_base + 32 * jb;
          } else {
            x = acc[i][jb][v];
            ocol0 = n_base + 32 * jb;
          }
          if constexpr (F16O)
            sh[rib * LDH + lrow] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_fmed3f(x, -kF16Max, kF16Max));
          else
            sh[rib * LDH + lrow] = __builtin_bit_cast(uint16_t, (bf16)x);
        }
        wave_lds_order();
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int r = (lane >> 2) + 16 * it, c8 = 8 * (lane & 3);
          const u32x4 val = *reinterpret_cast<const u32x4*>(sh + r * LDH + c8);
          const int row = m_base + 32 * i + r;
          if (row < g.M)
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + size_t(row) * g.ldc + ocol0 + c8) = val;
        }
        wave_lds_order();
      }
    }
  }
}

// Persistent GEMM (every linear map of the bf16 tower): each
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
// A operand (AMD): A_DENSE, rows of A; A_MERGE, output row t of the merger
// is the concatenation of four residual rows msrc[t][0..3] (2x2 patch
// gather): the loads fetch straight from the [rows][2D] hi | lo copy of the
// residual, K = 8D = (hi: 4 gathered rows) | (lo: the same 4 rows).
// LOW (8 or 4): after the bf16 k-steps, more steps multiply low-precision
// copies of A and B -- fp8 e4m3 (LOW 8) or fp4 e2m1 (LOW 4), one scale byte
// per 32 k on each side (v_mfma_scale_f32_32x32x64_f8f6f4) -- into the same
// accumulators.  A step moves the same 128-byte tile rows and chunk swizzle
// as a bf16 step (128 fp8 or 256 fp4 k), plus the rows' scale bytes (4 or 8
// a row) behind the tiles.  MFMA operands: for fp8, lane l (half h = l / 32)
// holds row l % 32, k [16h, 16h + 16) and [32 + 16h, 32 + 16h + 16) of the
// 64 and supplies the scale of its row's 32-k block h (byte 0 of its scale
// operand); for fp4 the lane's 16 operand bytes are one 32-k block (k
// [32h, 32h + 32) of the 64) and its scale byte scales exactly those values.
template <int BM, int BN, int WMW, int WNW, int NS, int BKT, int AMD, int BMD, int EM, int LOW = 0, bool F16 = false>
__global__ __launch_bounds__(WMW * WNW * 64) __attribute__((amdgpu_waves_per_eu(WMW * WNW >= 8 ? 2 : 8 / (WMW * WNW))))
void gemm_dense_kernel(GemmArgs g) {
  static_assert(AMD == A_DENSE || AMD == A_MERGE, "A operand mode");
  constexpr int NW = WMW * WNW, NT = NW * 64;
  constexpr int CH = BKT / 8;                    // 16-byte chunks per tile row
  constexpr int TMW = BM / WMW, TNW = BN / WNW;  // wave tile
  constexpr int TM = TMW / 32, TN = TNW / 32;
  constexpr int A_LD = BM * CH / NT, B_LD = BN * CH / NT;  // global_load_lds per thread per k-tile
  constexpr int LDT = A_LD + B_LD;
  static_assert(A_LD >= 1 && B_LD >= 1 && (BM * CH) % NT == 0 && (BN * CH) % NT == 0, "tile/thread mismatch");
  static_assert(EM != E_SILU_MUL || (TN % 2) == 0, "silu-mul needs gate/up block pairs in a wave");
  static_assert((NS - 2) * (LDT + 1) <= 63, "vmcnt range");
  static_assert(LOW == 0 || LOW == 8 || LOW == 4, "low-precision format");
  constexpr bool LO8 = LOW != 0;               // has low-precision steps
  constexpr int SB = LOW == 4 ? 8 : 4;         // scale bytes per row and step
  constexpr int KSTEP = LOW == 4 ? 256 : 128;  // k per low-precision step
  constexpr int SCA = BM * SB / 16, SCB = BN * SB / 16;  // 16-byte scale chunks per step
  constexpr int WSA = (SCA + 63) / 64, WSB = (SCB + 63) / 64;  // waves that load them
  // (with A_MERGE the bf16 steps gather A and the low-precision steps read a
  // dense operand already in the merged rows' order)
  static_assert(!LO8 || (BM <= 256 && BN <= 256 && BKT == 64 && NS == 2 && WSA + WSB <= NW),
                "low-precision steps: tiles of at most 256 x 256, 64-k bf16 steps (128-byte rows)");

  // residual-adding epilogues fetch the residual of up to 4 blocks (64
  // values a lane) during the tile's last k-steps, one block per step, so
  // the reads overlap those steps' MFMAs (a step waits for all loads issued
  // in the one before)
  constexpr int kPreBlocks = TM * TN <= 4 ? TM * TN : 2;
  // scale bytes behind each stage's tiles
  constexpr int kStageU4 = (BM + BN) * CH + (LO8 ? SCA + SCB : 0);
  __shared__ u32x4 lds[NS][kStageU4];
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
  const int KT16 = g.K / BKT;                  // bf16 k-steps per tile
  const int KT = KT16 + (LO8 ? g.k8 / KSTEP : 0);  // all k-steps per tile
  // k-tiles of B: A's K may run over B's K twice (hi | lo halves of A)
  const int KTB = g.kb > 0 ? g.kb / BKT : KT16;

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
  // Every instruction reads rows of one matrix, so its address is a uniform
  // base (scalar registers; the k-step moves only that) plus a per-lane
  // 32-bit byte offset inside the tile: the loads cost no vector ALU work.
  // The instruction's rows are [P0, P0 + 64 / CH), P0 = (wave * X_LD + q) *
  // 64 / CH: inside one 32-row gate/up block and one q/k/v matrix.
  static_assert(64 % CH == 0 && 32 % (64 / CH) == 0, "rows per load instruction");
  const char* ga_b = nullptr;             // A_DENSE: this tile's first row of A
  uint32_t ga_o[A_LD];
  const char* ga[AMD == A_MERGE ? A_LD : 1];  // A_MERGE: per-lane row pointers
  const char* gb_b[B_LD];
  uint32_t gb_o[B_LD];
  int4 msrc4[AMD == A_MERGE ? A_LD : 1];  // A_MERGE: source rows of each load slot's row
  int a_gc[AMD == A_MERGE ? A_LD : 1];    // A_MERGE: chunk each load slot fetches
  int is_tm = 0, is_tn = 0;               // tile of the steps being issued
  auto set_rows = [&](int t) {
    int tm, tn;
    tile_mn(t, tm, tn);
    is_tm = tm;
    is_tn = tn;
    if constexpr (AMD == A_DENSE) ga_b = reinterpret_cast<const char*>(g.A) + size_t(tm) * BM * g.lda * 2;
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      const int p = (wave * A_LD + q) * 64 + lane;
      const int P = p / CH, gc = (p % CH) ^ swzc<CH>(P);
      int m = tm * BM + P;
      m = m < g.M ? m : g.M - 1;  // rows past M are computed but never stored
      if constexpr (AMD == A_DENSE) {
        ga_o[q] = uint32_t(((m - tm * BM) * g.lda + gc * 8) * 2);
      } else {
        msrc4[q] = reinterpret_cast<const int4*>(g.maps.msrc)[m];
        a_gc[q] = gc;
      }
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q) {
      const int p = (wave * B_LD + q) * 64 + lane;
      const int P = p / CH, gc = (p % CH) ^ swzc<CH>(P);
      const int P0 = (wave * B_LD + q) * (64 / CH);  // uniform: row of lane 0
      const int n0 = tn * BN + P0;
      const char* base;
      int r;  // row inside the base matrix, relative to the base
      if constexpr (BMD == B_ONE) {
        const int n0c = n0 < g.N ? n0 : g.N - 1, n = tn * BN + P;
        base = reinterpret_cast<const char*>(g.B0) + size_t(n0c) * g.ldb * 2;
        r = (n < g.N ? n : g.N - 1) - n0c;
      } else if constexpr (BMD == B_QKV) {
        const int which = n0 / g.hidden;
        const void* bm = which == 0 ? g.B0 : (which == 1 ? g.B1 : g.B2);
        base = reinterpret_cast<const char*>(bm) + size_t(n0 - which * g.hidden) * g.ldb * 2;
        r = P - P0;
      } else {
        // 32-row blocks alternate gate, up: rows [64j, 64j+32) -> gate rows
        // [32j, 32j+32), rows [64j+32, 64j+64) -> up rows [32j, 32j+32).
        const void* bm = (n0 & 32) ? g.B1 : g.B0;
        base = reinterpret_cast<const char*>(bm) + size_t((n0 >> 6) * 32 + (n0 & 31)) * g.ldb * 2;
        r = P - P0;
      }
      gb_b[q] = base;
      gb_o[q] = uint32_t(r * g.ldb * 2 + gc * 16);
    }
  };
  // the same for the low-precision operands (rows of k8 * LOW / 8 bytes)
  const size_t row8 = size_t(g.k8) * LOW / 8;
  auto set_rows8 = [&]() {
    ga_b = reinterpret_cast<const char*>(g.A8) + size_t(is_tm) * BM * row8;
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      const int p = (wave * A_LD + q) * 64 + lane;
      const int P = p / CH, gc = (p % CH) ^ swzc<CH>(P);
      int m = is_tm * BM + P;
      m = m < g.M ? m : g.M - 1;
      ga_o[q] = uint32_t((m - is_tm * BM) * row8 + gc * 16);
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q) {
      const int p = (wave * B_LD + q) * 64 + lane;
      const int P = p / CH, gc = (p % CH) ^ swzc<CH>(P);
      gb_b[q] = reinterpret_cast<const char*>(g.B8) + size_t(is_tn * BN) * row8;
      gb_o[q] = uint32_t(P * row8 + gc * 16);
    }
  };
  // (the global source is passed as a uint16_t pointer: with a char pointer
  // the host pass drops the kernel's launch stub without a diagnostic)
  int is_step = 0, is_kt = 0, is_tile = 0;  // next step to issue
  // A_MERGE: k-tiles per gathered row segment (D / BKT); segment s of K
  // takes part s / 4 (hi, lo) of source row msrc[t][s % 4]
  const int KTQ = AMD == A_MERGE ? g.hidden / BKT : 1;
  auto issue_next = [&]() {
    if (is_kt == 0) set_rows(tile_of(is_tile));
    const int st = is_step % NS;
    if constexpr (LO8) {
      if (is_kt >= KT16) {
        const int s8 = is_kt - KT16;
        if (s8 == 0) set_rows8();
        const size_t koff8 = size_t(s8) * 128;
#pragma unroll
        for (int q = 0; q < A_LD; ++q)
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(ga_b + koff8 + ga_o[q]),
                                           (lds_void*)&lds[st][(wave * A_LD + q) * 64], 16, 0, 0);
#pragma unroll
        for (int q = 0; q < B_LD; ++q)
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(gb_b[q] + koff8 + gb_o[q]),
                                           (lds_void*)&lds[st][BM * CH + (wave * B_LD + q) * 64], 16, 0, 0);
        // scale bytes of the tile's rows for this step (SB per row): A's BM
        // rows by waves [0, WSA), B's BN rows by the next WSB waves, placed
        // as A's rows then B's rows behind the tiles (rows past M read
        // padding rows)
        if (wave < WSA + WSB) {
          const bool isa = wave < WSA;
          const int c = (isa ? wave : wave - WSA) * 64 + lane;
          if (c < (isa ? SCA : SCB)) {
            const char* src = isa
                ? reinterpret_cast<const char*>(g.As) + (size_t(s8) * g.as_rows + is_tm * BM) * SB + c * 16
                : reinterpret_cast<const char*>(g.Bs) + (size_t(s8) * g.bs_rows + is_tn * BN) * SB + c * 16;
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const uint16_t*>(src),
                (lds_void*)&lds[st][(BM + BN) * CH + (isa ? wave * 64 : SCA + (wave - WSA) * 64)], 16, 0, 0);
          }
        }
        ++is_step;
        if (++is_kt == KT) {
          is_kt = 0;
          ++is_tile;
        }
        return;
      }
    }
    size_t koff = size_t(is_kt) * BKT * 2;
    if constexpr (AMD == A_MERGE) {
      const int seg = is_kt / KTQ, kin = is_kt - seg * KTQ;
      if (kin == 0) {
        const int part = seg >> 2, qi = seg & 3;
#pragma unroll
        for (int q = 0; q < A_LD; ++q) {
          const int4 m4 = msrc4[q];
          const int src = qi == 0 ? m4.x : (qi == 1 ? m4.y : (qi == 2 ? m4.z : m4.w));
          ga[q] = reinterpret_cast<const char*>(g.A) +
                  (size_t(src) * g.lda + size_t(part) * g.hidden + a_gc[q] * 8) * 2;
        }
      }
      koff = size_t(kin) * BKT * 2;
    }
    const size_t koffb = size_t(is_kt < KTB ? is_kt : is_kt - KTB) * BKT * 2;
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      const char* src;
      if constexpr (AMD == A_MERGE) src = ga[q] + koff;
      else src = ga_b + koff + ga_o[q];
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(src),
                                       (lds_void*)&lds[st][(wave * A_LD + q) * 64], 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(gb_b[q] + koffb + gb_o[q]),
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

  // step has landed once at most (steps issued after it) x (loads per step)
  // of this thread are outstanding (low-precision products run two stages,
  // so their extra scale loads never enter the count); the barrier makes
  // every thread's part visible and frees the stage read in the previous step
  static_assert(!LO8 || NS == 2, "low-precision steps use two stages");
  auto begin_step = [&](int step) {
    if (step + NS - 2 < steps) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LDT));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
    if (is_step < steps) issue_next();
  };
  // fragment offsets (16-byte units inside a stage).  A row's chunk swizzle
  // depends only on lrow here (wave tiles and 32-row blocks start at
  // multiples of 16 rows), so chunk c = 2k + lhalf of A fragment i sits at
  // fa_off[k] + 32 * i * CH (B: fb_off[k] + 32 * j * CH): one register per k
  // and an immediate offset per fragment.
  static_assert(TMW % 16 == 0 && TNW % 16 == 0, "row-independent chunk swizzle");
  int fa_off[CH / 2], fb_off[CH / 2];
#pragma unroll
  for (int k = 0; k < CH / 2; ++k) {
    const int c = (2 * k + lhalf) ^ swzc<CH>(lrow);
    fa_off[k] = (wm * TMW + lrow) * CH + c;
    fb_off[k] = BM * CH + (wn * TNW + lrow) * CH + c;
  }
  // one bf16 k-step: fragments of k-substep ks + 1 are read while the MFMAs
  // of ks run
  auto compute_bf16 = [&](int stage) {
    const u32x4* sl = lds[stage];
    constexpr int KS = BKT / 16;
    u32x4 fa[2][TM], fb[2][TN];
    auto read_frags = [&](int ks, u32x4 (&ra)[TM], u32x4 (&rb)[TN]) {
#pragma unroll
      for (int i = 0; i < TM; ++i) ra[i] = sl[fa_off[ks] + 32 * i * CH];
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) rb[jn] = sl[fb_off[ks] + 32 * jn * CH];
    };
    read_frags(0, fa[0], fb[0]);
    static_for<KS>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      if constexpr (ks + 1 < KS) read_frags(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) {
          if constexpr (F16) acc[i][jn] = mfma32x32x16_f16(fa[ks & 1][i], fb[ks & 1][jn], acc[i][jn]);
          else acc[i][jn] = mfma32x32x16(fa[ks & 1][i], fb[ks & 1][jn], acc[i][jn]);
        }
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
  };
  // one fp8 k-step (LO8): two 64-k scaled MFMAs; scale words: one dword per
  // tile row, byte b = 32-k block b of the step
  auto compute_fp8 = [&](int stage) {
    const u32x4* sl = lds[stage];
    const uint32_t* scl = reinterpret_cast<const uint32_t*>(lds[stage] + (BM + BN) * CH);
    uint32_t sa_w[TM], sb_w[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) sa_w[i] = scl[wm * TMW + 32 * i + lrow];
#pragma unroll
    for (int jn = 0; jn < TN; ++jn) sb_w[jn] = scl[BM + wn * TNW + 32 * jn + lrow];
    static_for<2>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      // chunks c0 = 4 ks + lhalf and c1 = c0 + 2 of each row; all A
      // fragments held, B fragments streamed one at a time
      i32x8 fa8[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa8[i] = join8(sl[fa_off[2 * ks] + 32 * i * CH], sl[fa_off[2 * ks + 1] + 32 * i * CH]);
      const int sh = 8 * (2 * ks + lhalf);
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) {
        const i32x8 fb8 = join8(sl[fb_off[2 * ks] + 32 * jn * CH], sl[fb_off[2 * ks + 1] + 32 * jn * CH]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][jn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa8[i], fb8, acc[i][jn], 0, 0, 0,
                                                                       int(sa_w[i] >> sh), 0, int(sb_w[jn] >> sh));
      }
    });
  };

  // one fp4 k-step (LOW 4): 256 k as four 64-k scaled MFMAs; the MFMA over
  // k [64m, 64m + 64) takes, for lane half h, 16-byte chunk c = 2m + h of the
  // row (32 fp4 k, one scale block) and that block's scale byte c of the
  // row's two scale dwords
  auto compute_fp4 = [&](int stage) {
    const u32x4* sl = lds[stage];
    const uint32_t* scl = reinterpret_cast<const uint32_t*>(lds[stage] + (BM + BN) * CH);
    static_for<4>([&](auto m_c) {
      constexpr int m = decltype(m_c)::value;
      const int c = 2 * m + lhalf, sh = 8 * (c & 3);
      i32x8 fa4[TM];
      int sav[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * TMW + 32 * i + lrow;
        fa4[i] = widen4(sl[fa_off[m] + 32 * i * CH]);
        sav[i] = int(scl[2 * row + (m >> 1)] >> sh);
      }
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) {
        const int row = wn * TNW + 32 * jn + lrow;
        const i32x8 fb4 = widen4(sl[fb_off[m] + 32 * jn * CH]);
        const int sbv = int(scl[2 * BM + 2 * row + (m >> 1)] >> sh);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][jn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa4[i], fb4, acc[i][jn], 4, 4, 0, sav[i], 0, sbv);
      }
    });
  };

  int step = 0;
  for (int ti = 0; ti < my_tiles; ++ti) {
    int tm, tn;
    tile_mn(tile_of(ti), tm, tn);
    Residual<kPreBlocks> res;
    for (int kt = 0; kt < KT16; ++kt, ++step) {
      begin_step(step);
      // an accumulating epilogue's residual: block b of the first
      // kPreBlocks is fetched in k-step KT16 - kPreBlocks + b (the other
      // blocks of larger wave tiles are read in the epilogue)
      if constexpr (EM == E_ADD_F32) {
        static_for<kPreBlocks>([&](auto b_c) {
          constexpr int b = decltype(b_c)::value;
          // products with low-precision steps take all blocks in the last
          // bf16 step (spreading them spills there)
          const int at = LO8 ? KT16 - 1 : (KT16 - kPreBlocks + b > 0 ? KT16 - kPreBlocks + b : 0);
          if (kt == at)
            load_residual_block<TM, TN, b, kPreBlocks>(g, res, tm * BM + wm * TMW, tn * BN + wn * TNW, lane);
        });
      }
      compute_bf16(step % NS);
    }
    if constexpr (LO8) {
      for (int kt = KT16; kt < KT; ++kt, ++step) {
        begin_step(step);
        // low-precision-only products (no bf16 steps) fetch the residual here
        if constexpr (EM == E_ADD_F32) {
          // (all blocks in the last step here: spreading them spills)
          if (KT16 == 0 && kt == KT - 1) {
            static_for<kPreBlocks>([&](auto b_c) {
              load_residual_block<TM, TN, decltype(b_c)::value, kPreBlocks>(g, res, tm * BM + wm * TMW,
                                                                             tn * BN + wn * TNW, lane);
            });
          }
        }
        if constexpr (LOW == 8) compute_fp8(step % NS);
        else compute_fp4(step % NS);
      }
    }
    // the stage just consumed is free until the next step's loads (issued
    // after the next barrier): once every wave is done with it, each wave
    // uses its own slice of it to stage the output
    __syncthreads();
    float* scratch = reinterpret_cast<float*>(lds[(step - 1) % NS]) + wave * kScratchFloats;
    epilogue_lds<EM, TM, TN, kEpiRows, kPreBlocks, F16>(g, acc, tm * BM + wm * TMW, tn * BN + wn * TNW, lane, scratch,
                                                   res);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jn = 0; jn < TN; ++jn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;
  }
}

template <int BM, int BN, int WMW, int WNW, int NS, int BKT, int AMD, int BMD, int EM, int LOW = 0, bool F16 = false>
hipError_t launch_dense(const GemmArgs& g, hipStream_t s) {
  constexpr bool LO8 = LOW != 0;
  constexpr int KSTEP = LOW == 4 ? 256 : 128, SB = LOW == 4 ? 8 : 4;
  const int ncols = (BMD == B_GATEUP) ? 2 * g.N : g.N;
  if (ncols % BN || g.K % BKT || g.kb % BKT) return hipErrorInvalidValue;
  if (g.kb > 0 && g.K != 2 * g.kb) return hipErrorInvalidValue;
  // A_MERGE: K = 8D over a hi | lo copy [rows][2D] (kb = 4D), or K = 4D over a
  // bf16 copy [rows][D] (kb = 0, low-precision steps may follow)
  if (AMD == A_MERGE && (g.hidden % BKT || !((g.K == 8 * g.hidden && g.kb == 4 * g.hidden) ||
                                              (g.K == 4 * g.hidden && g.kb == 0))))
    return hipErrorInvalidValue;
  if (LO8 && (g.k8 <= 0 || g.k8 % KSTEP || g.kb != 0 || g.as_rows < ((g.M + BM - 1) / BM) * BM || g.bs_rows < ncols))
    return hipErrorInvalidValue;
  const int tiles = ((g.M + BM - 1) / BM) * (ncols / BN);
  // as many workgroups as fit on the chip at once: the LDS ring sets how
  // many a CU holds
  constexpr int kLdsBytes = NS * ((BM + BN) * BKT * 2 + (LO8 ? (BM + BN) * SB : 0));
  constexpr int kPerCU = (160 * 1024) / kLdsBytes < 2 ? 1 : 2;
  const int grid = tiles < kNumCUs * kPerCU ? tiles : kNumCUs * kPerCU;
  hipLaunchKernelGGL((gemm_dense_kernel<BM, BN, WMW, WNW, NS, BKT, AMD, BMD, EM, LOW, F16>), dim3(grid),
                     dim3(WMW * WNW * 64), 0, s, g);
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
// N = hidden products with an fp32 output (out-projection, down, patch
// embedding): 128 x 128 tiles, 4 waves, two workgroups per CU -- at 1540^2
// the 760 tiles spread over 512 slots instead of 384 over 256 (measured
// 11% faster on down than 256 x 128)
#ifndef PV_GEMM_CFG_RES
#define PV_GEMM_CFG_RES 128, 128, 2, 2, 2, 64
#endif
// the same products in 192 x 256 tiles, 8 waves, one workgroup per CU:
// chosen per call when it needs enough fewer rounds of the chip (below)
#ifndef PV_GEMM_CFG_RES_WIDE
#define PV_GEMM_CFG_RES_WIDE 192, 256, 2, 4, 2, 64
#endif
// merger (a few thousand rows, N = 5120): 256 x 256 tiles, one round of
// 240 tiles at 1540^2; 256 x 128 when N is not a multiple of 256
#ifndef PV_GEMM_CFG_MERGE
#define PV_GEMM_CFG_MERGE PV_GEMM_CFG_BIG
#endif
// q,k,v: 384 x 192 tiles (16 per row of tiles) put the 1540 x 1540 image's
// 32 rows of tiles on the 256 CUs in exactly two rounds (measured 3.5%
// faster than 256 x 192 in three; on the packed 8-image batch, whose 384-row
// tiles leave a last round 70% full, 256 x 192 tiles were no faster), or
// 256 x 256 tiles per call (below); the fp8 variant keeps 256 x 192 (its
// scale blocks are padded for tiles of at most 256 rows)
#ifndef PV_GEMM_CFG_QKV
#define PV_GEMM_CFG_QKV 384, 192, 4, 2, 2, 64
#endif
#ifndef PV_GEMM_CFG_QKV8
#define PV_GEMM_CFG_QKV8 256, 192, 4, 2, 2, 64
#endif

// q,k,v (16-bit): a round of 256 x 256 tiles costs about 0.85 of a round of
// 384 x 192 tiles (fewer L2 bytes per output; measured on the four
// workloads), so they are taken when 0.85 x their rounds is below the
// 384-row rounds: the 16 tiles of 4,096 patches (12 rounds against 11:
// 0.441 -> 0.415 ms), not 1540^2 (3 against 2: 0.082 -> 0.096 ms) nor the
// packed 8- and 64-image batches (equal and 1.5% slower).
bool use_qkv_big(const GemmArgs& g) {
  if (g.N % 256) return false;
  const long long r384 = ((g.M + 383) / 384 * (g.N / 192) + kNumCUs - 1) / kNumCUs;
  const long long r256 = ((g.M + 255) / 256 * (g.N / 256) + kNumCUs - 1) / kNumCUs;
  return r256 * 17 < r384 * 20;
}

// N = hidden products (out-projection, down, patch embedding): 128 x 128
// tiles (two workgroups per CU), 192 x 256 (one per CU) or, for the 16-bit
// down product, 256 x 256 (one per CU), whichever needs the fewest rounds
// of the chip weighted by what a round costs.  Costs in 30ths of a 128 x
// 128 round, measured on the 1540^2, packed 8-image, 64-image and 16-tile
// workloads:
//   192 x 256: 39 for the patch embedding (a plain fp32 store; 16 tiles
//     0.306 -> 0.287 ms, packed 8-image batch 0.093 -> 0.097), 42 for the
//     16-bit down product (4096-deep k: the larger tile's fewer L2 bytes per
//     flop pay over the long k loop), 50 for the out-projection (1024-deep
//     k: the one workgroup's residual read-modify-write is not hidden behind
//     another's k loop) and the fp8 products (their k loop runs at twice the
//     rate);
//   256 x 256: 51 for the 16-bit down product (packed 8-image batch 0.305 ->
//     0.263 ms, 16 tiles 0.654 -> 0.548 ms, 64 images 0.559 -> 0.532 ms;
//     at 1540^2 its 192 tiles leave a quarter of the CUs idle, and 256
//     tiles of 192 x 256 fill one round); for the out-projection 256 x 256
//     tiles were slower (packed 8-image batch 0.096 -> 0.107 ms).
// Ties keep the smaller tile.
enum ResTile { TILE_RES, TILE_WIDE, TILE_BIG };
ResTile res_tile(const GemmArgs& g, long long c_wide, long long c_big) {
  if (g.N % 256) return TILE_RES;
  const long long rows128 = (g.M + 127) / 128, rows192 = (g.M + 191) / 192, rows256 = (g.M + 255) / 256;
  const long long r_res = (rows128 * (g.N / 128) + 2 * kNumCUs - 1) / (2 * kNumCUs);
  const long long r_wide = (rows192 * (g.N / 256) + kNumCUs - 1) / kNumCUs;
  const long long r_big = (rows256 * (g.N / 256) + kNumCUs - 1) / kNumCUs;
  ResTile t = TILE_RES;
  long long best = 30 * r_res;
  if (r_wide * c_wide < best) t = TILE_WIDE, best = r_wide * c_wide;
  if (c_big > 0 && r_big * c_big < best) t = TILE_BIG;
  return t;
}

hipError_t gemm_bf16(GemmKind kind, const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const ResTile rt = kind == GEMM_PATCH                                 ? res_tile(g, 39, 0)
                     : (kind == GEMM_DOWN && g.f16 && g.K >= 2048) ? res_tile(g, 42, 51)
                                                                   : res_tile(g, 50, 0);
  const bool wide = rt == TILE_WIDE;
  switch (kind) {
    case GEMM_PATCH:
      return wide ? launch_dense<PV_GEMM_CFG_RES_WIDE, A_DENSE, B_ONE, E_STORE_F32>(g, s)
                  : launch_dense<PV_GEMM_CFG_RES, A_DENSE, B_ONE, E_STORE_F32>(g, s);
    case GEMM_QKV:
      if (g.k8 > 0) return launch_dense<PV_GEMM_CFG_QKV8, A_DENSE, B_QKV, E_QKV_ROPE, 8>(g, s);
      return use_qkv_big(g) ? launch_dense<PV_GEMM_CFG_BIG, A_DENSE, B_QKV, E_QKV_ROPE>(g, s)
                            : launch_dense<PV_GEMM_CFG_QKV, A_DENSE, B_QKV, E_QKV_ROPE>(g, s);
    case GEMM_OPROJ:
    case GEMM_DOWN:
      if (g.f16) {
        if (g.k8 > 0) return hipErrorInvalidValue;
        if (rt == TILE_BIG) return launch_dense<PV_GEMM_CFG_BIG, A_DENSE, B_ONE, E_ADD_F32, 0, true>(g, s);
        return wide ? launch_dense<PV_GEMM_CFG_RES_WIDE, A_DENSE, B_ONE, E_ADD_F32, 0, true>(g, s)
                    : launch_dense<PV_GEMM_CFG_RES, A_DENSE, B_ONE, E_ADD_F32, 0, true>(g, s);
      }
      if (wide)
        return g.k8 > 0 ? launch_dense<PV_GEMM_CFG_RES_WIDE, A_DENSE, B_ONE, E_ADD_F32, 8>(g, s)
                        : launch_dense<PV_GEMM_CFG_RES_WIDE, A_DENSE, B_ONE, E_ADD_F32>(g, s);
      return g.k8 > 0 ? launch_dense<PV_GEMM_CFG_RES, A_DENSE, B_ONE, E_ADD_F32, 8>(g, s)
                      : launch_dense<PV_GEMM_CFG_RES, A_DENSE, B_ONE, E_ADD_F32>(g, s);
    case GEMM_GATEUP:
      if (g.f16) {
        if (g.k8 > 0) return hipErrorInvalidValue;
        return launch_dense<PV_GEMM_CFG_BIG, A_DENSE, B_GATEUP, E_SILU_MUL, 0, true>(g, s);
      }
      if (g.k8 <= 0) return launch_dense<PV_GEMM_CFG_BIG, A_DENSE, B_GATEUP, E_SILU_MUL>(g, s);
      if (g.low_fmt != 8) return hipErrorInvalidValue;
      return launch_dense<PV_GEMM_CFG_BIG, A_DENSE, B_GATEUP, E_SILU_MUL, 8>(g, s);
    case GEMM_MERGE:
      if (g.k8 > 0)
        return g.N % 256 == 0 ? launch_dense<PV_GEMM_CFG_MERGE, A_MERGE, B_ONE, E_STORE, 4>(g, s)
                              : launch_dense<PV_GEMM_CFG_N1K, A_MERGE, B_ONE, E_STORE, 4>(g, s);
      return g.N % 256 == 0 ? launch_dense<PV_GEMM_CFG_MERGE, A_MERGE, B_ONE, E_STORE>(g, s)
                            : launch_dense<PV_GEMM_CFG_N1K, A_MERGE, B_ONE, E_STORE>(g, s);
    case GEMM_PLAIN:  return launch_dense<PV_GEMM_CFG_N1K, A_DENSE, B_ONE, E_STORE>(g, s);
    case GEMM_MERGE_F32:
      if (g.k8 > 0)
        return g.N % 256 == 0 ? launch_dense<PV_GEMM_CFG_MERGE, A_MERGE, B_ONE, E_STORE_F32, 4>(g, s)
                              : launch_dense<PV_GEMM_CFG_N1K, A_MERGE, B_ONE, E_STORE_F32, 4>(g, s);
      return g.N % 256 == 0 ? launch_dense<PV_GEMM_CFG_MERGE, A_MERGE, B_ONE, E_STORE_F32>(g, s)
                            : launch_dense<PV_GEMM_CFG_N1K, A_MERGE, B_ONE, E_STORE_F32>(g, s);
    case GEMM_GELU:
      return launch_dense<PV_GEMM_CFG_N1K, A_DENSE, B_ONE, E_GELU>(g, s);
    case GEMM_PLAIN_F32:
      return launch_dense<PV_GEMM_CFG_N1K, A_DENSE, B_ONE, E_STORE_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pv
