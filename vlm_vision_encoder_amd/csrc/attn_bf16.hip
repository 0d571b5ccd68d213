// Block-diagonal multi-head attention over the packed patch sequence, bf16
// MFMA with fp32 online softmax ("Mistral 3" (KerasFormers),
// Mistral3VisionModel: attention over a packed variable-resolution sequence,
// every image its own block; head_dim 64, scale 1/8).  q and k arrive already
// rotated by the 2-D RoPE, which the q,k,v projection applies in its epilogue
// (once per element, instead of once per query tile that re-reads a key).
//
// Work item = (image, tile of 32*QB*WAVES queries) x head.  Each wave owns
// 32*QB queries (QB column blocks of 32) and walks all keys of its image in
// tiles of 64.
//
// * Scores are computed transposed, S^T = K Q^T, so a lane holds one query
//   column: row max and row sum are lane-local plus one exchange with lane^32,
//   and the probabilities P^T already sit in the B-operand layout of
//   O^T = V^T P^T.  For that match, LDS row P of the key tile holds key
//   sigma(P) (bits 2 and 3 swapped): the 8 probabilities a lane holds per
//   16-key step are then 8 consecutive keys.
// * Two LDS stages (tile kt in use, tile kt+1 in flight).  A three-stage
//   variant computes tile kt+1's scores during tile kt's softmax; it needs 32
//   more VGPRs, and the occupancy it costs outweighs the overlap it buys
//   (measured), so the two-stage form is the default.
// * K and V tiles go global -> LDS with global_load_lds_dwordx4 (no VGPR
//   staging); the swizzles are applied by choosing which 16-byte chunk each
//   lane fetches.  K chunks are XOR-swizzled by (row >> 1) & 7 for the
//   16-byte fragment reads (64 banks, 16 lanes per pass); V stays row-major and its V^T A-operand fragments come
//   from two ds_read_b64_tr_b16 transpose reads (each 16-lane group receives
//   a 4-key x 16-dim block transposed), with chunks XOR-swizzled by
//   2*(row & 3) so the four rows of a group hit distinct banks.
// * Online softmax in the exp2 domain with the 1/8 scale folded into one FMA.
//   The running max is only raised when a tile's max exceeds it by more than
//   8 (log2 units), so most tiles skip the O rescale; probabilities are then
//   bounded by 2^8.  Row sums use v_dot2 on the bf16 probabilities that feed
//   the MFMA.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int sigma_row(int r) {  // swap bits 2 and 3
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// K tile chunk swizzle: the LDS has 64 four-byte banks and serves a 16-byte
// read for 16 lanes per pass, so the 16 rows a pass touches must differ in
// (row parity, chunk): chunk ^ ((row >> 1) & 7) does that.
__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ float dot2_sum(uint32_t packed, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed), one, acc, false);
}

template <int QB, int WAVES, bool PIPE>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int SLOTS = 512;                 // 16-byte chunks per 64 x 64 bf16 tile
  constexpr int LPT = SLOTS / NT;            // global_load_lds per thread per tile (K and V each)
  // LDS stages.  PIPE: V(kt), K(kt+1) and tile kt+2 in flight, the scores of
  // tile kt+1 computed during tile kt's softmax.  Otherwise: tile kt and
  // tile kt+1 in flight.
  constexpr int NS = PIPE ? 3 : 2;
  static_assert(LPT >= 1 && SLOTS % NT == 0, "WAVES must divide 8");

  __shared__ u32x4 kl[NS][SLOTS];
  __shared__ u32x4 vl[NS][SLOTS];

  const int heads = a.heads;
  const int item = blockIdx.x / heads, head = blockIdx.x - item * heads;
  const AttnItem it = a.items[item];
  const ImageMeta mt = a.meta[it.image];
  const int n = mt.Hp * mt.Wp;
  const int base = mt.patch_base;
  const int D = a.hidden;
  const size_t ld = size_t(3) * D;
  const uint16_t* qkv = reinterpret_cast<const uint16_t*>(a.qkv);
  const int qoff = head * 64, koff = D + head * 64, voff = 2 * D + head * 64;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int wq0 = it.q0 + 32 * QB * wave;  // first query of this wave
  const bool active = wq0 < n;

  // ---- per-thread load plan: wave-instruction j covers slots
  // [(wave*LPT + j) * 64, +64); lane l fetches slot p = that + l.
  int k_row[LPT], k_chunk[LPT], v_row[LPT], v_chunk[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int p = (wave * LPT + j) * 64 + lane;
    const int P = p >> 3, pc = p & 7;
    k_row[j] = sigma_row(P);
    k_chunk[j] = pc ^ kswz(P);
    v_row[j] = P;
    v_chunk[j] = pc ^ (2 * (P & 3));
  }
  auto issue_loads = [&](int kt, int st) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      int uk = kt * 64 + k_row[j];
      uk = uk < n ? uk : n - 1;
      int uv = kt * 64 + v_row[j];
      uv = uv < n ? uv : n - 1;
      const uint16_t* gk = qkv + size_t(base + uk) * ld + koff + k_chunk[j] * 8;
      const uint16_t* gv = qkv + size_t(base + uv) * ld + voff + v_chunk[j] * 8;
      __builtin_amdgcn_global_load_lds(gk, (lds_void*)&kl[st][(wave * LPT + j) * 64], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(gv, (lds_void*)&vl[st][(wave * LPT + j) * 64], 16, 0, 0);
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T), kept for the whole loop
  u32x4 qf[QB][4];
#pragma unroll
  for (int tb = 0; tb < QB; ++tb) {
    int t = wq0 + 32 * tb + lrow;
    t = t < n ? t : n - 1;
    const uint16_t* qp = qkv + size_t(base + t) * ld + qoff + 8 * lhalf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[tb][ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
  }

  floatx16 o[2][QB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[i][j][v] = 0.f;
  float m_sc[QB], l_run[QB];
#pragma unroll
  for (int tb = 0; tb < QB; ++tb) {
    m_sc[tb] = -INFINITY;  // running max, in scaled (log2) units
    l_run[tb] = 0.f;
  }
  const float c = kLog2e * 0.125f;  // log2(e) / sqrt(64)

  // transposed-read addresses for the V^T fragments: 16-lane group g gets
  // dims D0 + (lane % 16), keys U..U+3 (and U+4..U+7 from the second read)
  const int g = lane >> 4, r16 = lane & 15;
  const int tr_row = 8 * (g >> 1) + (r16 >> 2);          // + ub*32 + sp*16 (+4)
  const int tr_col = 16 * (g & 1) + 4 * (r16 & 3);       // + db*32 (elements)

  // S^T block of one key tile (stage st)
  auto scores = [&](int st, floatx16 (&s)[2][QB]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int ub = 0; ub < 2; ++ub) {
        const int row = ub * 32 + lrow;
        const u32x4 kf = kl[st][row * 8 + ((2 * ks + lhalf) ^ kswz(row))];
#pragma unroll
        for (int tb = 0; tb < QB; ++tb) {
          if (ks == 0) {
            const floatx16 z = {};
            s[ub][tb] = mfma32x32x16(kf, qf[tb][ks], z);
          } else {
            s[ub][tb] = mfma32x32x16(kf, qf[tb][ks], s[ub][tb]);
          }
        }
      }
    }
  };

  const int nkt = (n + 63) / 64;
  issue_loads(0, 0);
  if (PIPE && nkt > 1) issue_loads(1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  floatx16 s_cur[2][QB];
  if (PIPE && active) scores(0, s_cur);

  for (int kt = 0; kt < nkt; ++kt) {
    const int st_v = kt % NS, st_k = (kt + 1) % NS;
    if (PIPE) {
      if (kt + 2 < nkt) issue_loads(kt + 2, (kt + 2) % NS);
    } else {
      if (kt + 1 < nkt) issue_loads(kt + 1, st_k);
    }
    if (active) {
      // ---- PIPE: next tile's scores, independent of this tile's softmax, so
      // their MFMAs can overlap the exp work below
      floatx16 s_nxt[2][QB];
      if (PIPE) {
        if (kt + 1 < nkt) scores(st_k, s_nxt);
      } else {
        scores(st_v, s_cur);
      }
      // ---- mask keys past the image (last tile only)
      if (kt * 64 + 64 > n) {
#pragma unroll
        for (int ub = 0; ub < 2; ++ub)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int u = kt * 64 + ub * 32 + 16 * (v >> 3) + 8 * lhalf + (v & 7);
            if (u >= n) {
#pragma unroll
              for (int tb = 0; tb < QB; ++tb) s_cur[ub][tb][v] = -INFINITY;
            }
          }
      }
      // ---- online softmax
      u32x4 pf[2][QB][2];
#pragma unroll
      for (int tb = 0; tb < QB; ++tb) {
        float mx = s_cur[0][tb][0];
#pragma unroll
        for (int ub = 0; ub < 2; ++ub)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s_cur[ub][tb][v]);
        mx = pair_max32(mx) * c;
        if (__any(mx > m_sc[tb] + kRescaleSlack)) {
          const float m_new = fmaxf(m_sc[tb], mx);
          float alpha = __builtin_amdgcn_exp2f(m_sc[tb] - m_new);
          // keeps the rescale a rarely-taken branch (otherwise it becomes an
          // unconditional multiply by a selected factor)
          asm volatile("" : "+v"(alpha));
          m_sc[tb] = m_new;
          l_run[tb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][tb][v] *= alpha;
        }
        const float mneg = -m_sc[tb];
#pragma unroll
        for (int ub = 0; ub < 2; ++ub) {
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            float p[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[ub][tb][8 * sp + v], c, mneg));
            const u32x4 pk = pack8(p);
            pf[ub][tb][sp] = pk;
            l_run[tb] = dot2_sum(pk[0], l_run[tb]);
            l_run[tb] = dot2_sum(pk[1], l_run[tb]);
            l_run[tb] = dot2_sum(pk[2], l_run[tb]);
            l_run[tb] = dot2_sum(pk[3], l_run[tb]);
          }
        }
      }
      // ---- O^T += V^T P^T
      const uint16_t* vb = reinterpret_cast<const uint16_t*>(vl[st_v]);
#pragma unroll
      for (int ub = 0; ub < 2; ++ub)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            u32x4 vf;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int row = ub * 32 + sp * 16 + tr_row + 4 * half;
              const int col = db * 32 + tr_col;  // element; chunk = col / 8
              const int pchunk = (col >> 3) ^ (2 * (row & 3));
              const uint16_t* addr = vb + row * 64 + pchunk * 8 + (col & 7);
              const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)addr);
              const u32x2 w = __builtin_bit_cast(u32x2, r);
              vf[2 * half] = w[0];
              vf[2 * half + 1] = w[1];
            }
#pragma unroll
            for (int tb = 0; tb < QB; ++tb) o[db][tb] = mfma32x32x16(vf, pf[ub][tb][sp], o[db][tb]);
          }
      if (PIPE) {
#pragma unroll
        for (int ub = 0; ub < 2; ++ub)
#pragma unroll
          for (int tb = 0; tb < QB; ++tb) s_cur[ub][tb] = s_nxt[ub][tb];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (!active) return;
  // ---- normalise and store: lane holds query column t, dims 8*(v/4)+4*half+(v%4)
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int tb = 0; tb < QB; ++tb) {
    const float inv = 1.f / pair_sum32(l_run[tb]);
    const int t = wq0 + 32 * tb + lrow;
    if (t < n) {
      uint16_t* orow = out + size_t(base + t) * D + qoff;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w;
          w[0] = pack_bf16x2(o[db][tb][4 * g4] * inv, o[db][tb][4 * g4 + 1] * inv);
          w[1] = pack_bf16x2(o[db][tb][4 * g4 + 2] * inv, o[db][tb][4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g4 + 4 * lhalf) = w;
        }
    }
  }
}

}  // namespace

hipError_t attention_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  static_assert(kAttnQTileBf16 == 32 * PV_ATTN_QB * PV_ATTN_WAVES, "q tile must match the kernel shape");
  hipLaunchKernelGGL((attn_bf16_kernel<PV_ATTN_QB, PV_ATTN_WAVES, PV_ATTN_PIPE != 0>), dim3(a.n_items * a.heads),
                     dim3(PV_ATTN_WAVES * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pv
