// Block-diagonal multi-head attention over the packed patch sequence, bf16
// MFMA with fp32 online softmax ("Mistral 3" (KerasFormers),
// Mistral3VisionModel: attention over a packed variable-resolution sequence,
// every image its own block; head_dim 64, scale 1/8).  q and k arrive already
// rotated by the 2-D RoPE, which the q,k,v projection applies in its epilogue
// (once per element, instead of once per query tile that re-reads a key).
//
// Work item = (image, tile of 64*WAVES queries) x head.  Each wave owns 64
// queries (two 32-column MFMA blocks) and walks all keys of its image in tiles
// of 64.  The scores are computed transposed, S^T = K Q^T, so a lane holds one
// query column: the row max and row sum are lane-local plus one exchange with
// lane ^ 32, and the probabilities P^T are already in the B-operand layout of
// the second product O^T = V^T P^T.  For that match the 64-key tile is stored
// in LDS with bits 2 and 3 of the row index swapped (rows sigma(u)), so the 8
// probabilities a lane holds per 16-key step are 8 consecutive keys.  V is
// transposed into LDS (rows = head dims, 16-byte chunks XOR-swizzled by
// d ^ (d >> 3)) so its A-operand fragments are single 16-byte reads.
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int sigma_row(int r) {  // swap bits 2 and 3
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int KCH = 512 / NT;  // K chunks (16 B) per thread per tile
  constexpr int VIT = 256 / NT;  // V row-pair items per thread per tile
  static_assert(KCH >= 1 && VIT >= 1, "WAVES must be 1, 2 or 4");

  __shared__ u32x4 kl[2][64 * 8];
  __shared__ u32x4 vt[2][64 * 8];

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
  const int wq0 = it.q0 + 64 * wave;  // first query of this wave
  const bool active = wq0 < n;

  // ---- Q fragments (B operand of S^T = K Q^T), kept for the whole loop
  u32x4 qf[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    int t = wq0 + 32 * tb + lrow;
    t = t < n ? t : n - 1;
    const uint16_t* qp = qkv + size_t(base + t) * ld + qoff + 8 * lhalf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[tb][ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
  }

  floatx16 o[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[i][j][v] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  const float c = kLog2e * 0.125f;  // log2(e) / sqrt(64)

  // ---- staging of one 64-key tile: registers <- global, LDS <- registers
  u32x4 rk[KCH], rv[VIT][2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + NT * i, row = id >> 3, ch = id & 7;
      int u = kt * 64 + row;
      u = u < n ? u : n - 1;
      rk[i] = *reinterpret_cast<const u32x4*>(qkv + size_t(base + u) * ld + koff + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int id = tid + NT * i, pr = id >> 3, ch = id & 7;
      int u0 = kt * 64 + 2 * pr, u1 = u0 + 1;
      u0 = u0 < n ? u0 : n - 1;
      u1 = u1 < n ? u1 : n - 1;
      rv[i][0] = *reinterpret_cast<const u32x4*>(qkv + size_t(base + u0) * ld + voff + ch * 8);
      rv[i][1] = *reinterpret_cast<const u32x4*>(qkv + size_t(base + u1) * ld + voff + ch * 8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + NT * i, row = id >> 3, ch = id & 7;
      const int srow = sigma_row(row);
      kl[buf][srow * 8 + (ch ^ (srow & 7))] = rk[i];
    }
    uint32_t* vw = reinterpret_cast<uint32_t*>(vt[buf]);
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int id = tid + NT * i, pr = id >> 3, ch = id & 7;
      // word (pr) of row d holds keys (2pr, 2pr+1) of head dim d
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = ch * 8 + j;
        const uint32_t w0 = rv[i][0][j >> 1], w1 = rv[i][1][j >> 1];
        const uint32_t lo = (j & 1) ? (w0 >> 16) : (w0 & 0xffffu);
        const uint32_t hi = (j & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
        const int pchunk = (pr >> 2) ^ vt_swz(d);
        vw[d * 32 + pchunk * 4 + (pr & 3)] = lo | hi;
      }
    }
  };

  const int nkt = (n + 63) / 64;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    if (active) {
      // ---- S^T = K Q^T
      floatx16 s[2][2];
#pragma unroll
      for (int ub = 0; ub < 2; ++ub)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int v = 0; v < 16; ++v) s[ub][tb][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int ub = 0; ub < 2; ++ub) {
          const int row = ub * 32 + lrow;
          const u32x4 kf = kl[buf][row * 8 + ((2 * ks + lhalf) ^ (row & 7))];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) s[ub][tb] = mfma32x32x16(kf, qf[tb][ks], s[ub][tb]);
        }
      }
      // ---- mask keys past the image (last tile only)
      if (kt * 64 + 64 > n) {
#pragma unroll
        for (int ub = 0; ub < 2; ++ub)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int u = kt * 64 + ub * 32 + 16 * (v >> 3) + 8 * lhalf + (v & 7);
            if (u >= n) {
              s[ub][0][v] = -INFINITY;
              s[ub][1][v] = -INFINITY;
            }
          }
      }
      // ---- online softmax (exp2 with the 1/8 scale folded in)
      u32x4 pf[2][2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float mx = s[0][tb][0];
#pragma unroll
        for (int ub = 0; ub < 2; ++ub)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[ub][tb][v]);
        mx = pair_max32(mx);
        const float m_new = fmaxf(m_run[tb], mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run[tb] - m_new) * c);
        m_run[tb] = m_new;
        l_run[tb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][tb][v] *= alpha;
        const float mc = m_new * c;
#pragma unroll
        for (int ub = 0; ub < 2; ++ub) {
          float p[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ub][tb][v], c, -mc));
            l_run[tb] += p[v];
          }
          pf[ub][tb][0] = pack8(p);
          pf[ub][tb][1] = pack8(p + 8);
        }
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int ub = 0; ub < 2; ++ub)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const int d = db * 32 + lrow;
            const u32x4 vf = vt[buf][d * 8 + ((4 * ub + 2 * sp + lhalf) ^ vt_swz(d))];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) o[db][tb] = mfma32x32x16(vf, pf[ub][tb][sp], o[db][tb]);
          }
    }
    if (kt + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  // ---- normalise and store: lane holds query column t, dims 8*(v/4)+4*half+(v%4)
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
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
  static_assert(kAttnQTileBf16 == 256, "q tile must match the kernel's 4 waves x 64 queries");
  hipLaunchKernelGGL(attn_bf16_kernel<4>, dim3(a.n_items * a.heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pv
