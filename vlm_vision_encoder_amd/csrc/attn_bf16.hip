// Block-diagonal multi-head attention over the packed patch sequence, bf16
// MFMA with an fp32 softmax ("Mistral 3" (KerasFormers), Mistral3VisionModel:
// attention over a packed variable-resolution sequence, every image its own
// block; head_dim 64, scale 1/8).  q and k arrive already rotated by the 2-D
// RoPE, which the q,k,v projection applies in its epilogue (once per element,
// instead of once per query tile that re-reads a key).
//
// Work item = (image, tile of 32*QB*WAVES queries) x head.  Each wave owns
// 32*QB queries (QB column blocks of 32) and walks all keys of its image in
// tiles of 64.
//
// * Scores are computed transposed, S^T = K Q^T, so a lane holds one query
//   column: row reductions are lane-local plus one exchange with lane^32,
//   and the probabilities P^T already sit in the B-operand layout of
//   O^T = V^T P^T.  For that match, LDS row P of the key tile holds key
//   sigma(P) (bits 2 and 3 swapped): the 8 probabilities a lane holds per
//   16-key step are then 8 consecutive keys.
// * K and V tiles go global -> LDS with global_load_lds_dwordx4 (no VGPR
//   staging), two stages; the swizzles are applied by choosing which 16-byte
//   chunk each lane fetches.  K chunks are XOR-swizzled by (row >> 1) & 7 for
//   the 16-byte fragment reads (64 banks, 16 lanes per pass); V stays
//   row-major and its V^T A-operand fragments come from two ds_read_b64_tr_b16
//   transpose reads (each 16-lane group receives a 4-key x 16-dim block
//   transposed), with chunks XOR-swizzled by 2*(row & 3).
// * Softmax.  At head_dim 64 a score costs 128 MACs of MFMA work and one
//   exp (a transcendental, two issue cycles); the waves of a work item run
//   their score MFMAs, softmax and P.V MFMAs in step, and the chip holds a
//   lower clock the more of the SIMD's cycles are busy (power), so the
//   per-score vector work is kept to exp + half a convert + one add:
//   - q arrives multiplied by log2(e)/8 (by the q,k,v projection's epilogue,
//     before its one rounding to bf16), so scores come out in exp2 units;
//   - softmax is unchanged by a per-query offset, so each query takes the
//     max of its first key tile as offset m0 and the score MFMAs start from
//     -m0 instead of zero: no per-score subtraction and no running max;
//   - row sums are fp32 adds of the probabilities (a tree per 8).  A
//     v_dot2 on the packed bf16 pairs would take half the instructions, but
//     it does not issue beside the MFMAs of the SIMD's other waves, while
//     adds, converts and exps largely do (measured by the probe).
//   The only risk of a fixed offset is range (a later score more than ~127
//   above m0 overflows, or every score far below it underflows).  Each work
//   item checks its sums and outputs for that and, if any is not finite,
//   reruns with an online softmax that tracks the running max (raised only
//   when a tile exceeds it by more than 2^8).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 units

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


// Four waves per SIMD (two work items per CU) is worth more than the few
// values the register cap moves to scratch outside the key loop (measured).
template <int QB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int SLOTS = 512;                 // 16-byte chunks per 64 x 64 bf16 tile
  // global_load_lds per thread per tile (K and V each); with more than 8
  // waves only the first 8 load
  constexpr int LPT = SLOTS / NT > 0 ? SLOTS / NT : 1;
  constexpr int LOAD_WAVES = SLOTS / (64 * LPT);
  static_assert(SLOTS % (64 * LPT) == 0 && (NT <= SLOTS ? SLOTS % NT == 0 : true), "load plan");

  __shared__ u32x4 kl[2][SLOTS];
  __shared__ u32x4 vl[2][SLOTS];

  // Workgroups reach the 8 XCDs round robin (block b on XCD b % 8).  With a
  // head count divisible by 8, XCD x takes heads x, x + 8, ...:
  // * images of one length (head_major): the XCD's list is cut into chunks
  //   of as many items as its CUs hold at once (32 CUs x the workgroups per
  //   CU), each chunk walked head by head, so the query tiles running
  //   together on an XCD are tiles of one head and stream that head's K and
  //   V through the XCD's 4 MB L2 once (at 1540^2 two heads' K and V, 6.2
  //   MB, do not fit: HBM fetch 124 -> 75 MB per launch, time unchanged);
  // * mixed lengths: item-major over the XCD's heads, so every XCD starts
  //   its longest items (the work list is longest-first) first -- walking a
  //   chunk head by head would start the second head's long items after the
  //   first head's short ones (packed 8-image batch 2.6% slower).
  // Otherwise item-major over all heads.
  constexpr int kChunk = 32 * (WAVES > 8 ? 1 : 2);
  const int heads = a.heads;
  int item, head;
  if ((heads & 7) == 0 && a.head_major) {
    const int hpx = heads >> 3, jx = blockIdx.x >> 3;
    const int c = jx / (kChunk * hpx), j = jx - c * kChunk * hpx;
    const int rest = a.n_items - c * kChunk, len = rest < kChunk ? rest : kChunk;
    const int hl = j / len;
    item = c * kChunk + (j - hl * len);
    head = (blockIdx.x & 7) + 8 * hl;
  } else if ((heads & 7) == 0) {
    const int hpx = heads >> 3, jx = blockIdx.x >> 3;
    item = jx / hpx;
    head = (blockIdx.x & 7) + 8 * (jx - item * hpx);
  } else {
    item = blockIdx.x / heads;
    head = blockIdx.x - item * heads;
  }
  const AttnItem it = a.items[item];
  const ImageMeta mt = a.meta[it.image];
  const int n = mt.Hp * mt.Wp;
  const int base = mt.patch_base;
  const int D = a.hidden;
  const size_t ld = size_t(3) * D;
  const uint16_t* qkv = reinterpret_cast<const uint16_t*>(a.qkv);
  const int qoff = head * 64, koff = D + head * 64, voff = 2 * D + head * 64;

  // uniform wave index (scalar): the LDS destinations of the direct loads
  // (M0) are then computed on the scalar unit
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  // Waves w, w + 4 and w + 8 share a SIMD; a fixed priority per wave of a
  // SIMD lets the first one run ahead, so the SIMD's waves drift apart in
  // phase and one's exps meet another's MFMAs (1-2% per launch)
  if (wave >= 8) __builtin_amdgcn_s_setprio(2);
  else if (wave >= 4) __builtin_amdgcn_s_setprio(1);
  const int wq0 = it.q0 + 32 * QB * wave;  // first query of this wave
  const bool active = wq0 < n;

  // ---- load plan: wave-instruction j covers slots [(wave*LPT + j) * 64, +64);
  // lane l fetches slot p = that + l.  A load's address is the key tile's
  // first row (uniform, scalar registers) plus a 32-bit lane offset.
  uint32_t k_lo[LPT], v_lo[LPT];
  int k_row[LPT], v_row[LPT], k_chunk[LPT], v_chunk[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int p = (wave * LPT + j) * 64 + lane;
    const int P = p >> 3, pc = p & 7;
    k_row[j] = sigma_row(P);
    k_chunk[j] = pc ^ kswz(P);
    v_row[j] = P;
    v_chunk[j] = pc ^ (2 * (P & 3));
    k_lo[j] = uint32_t((k_row[j] * ld + koff + k_chunk[j] * 8) * 2);
    v_lo[j] = uint32_t((v_row[j] * ld + voff + v_chunk[j] * 8) * 2);
  }
  // LDS stages as compile-time constants: the key loop runs two tiles per
  // trip (stage 1 then 0, or 0 then 1), so every fragment address is a
  // loop-invariant register plus an immediate offset
  const std::integral_constant<int, 0> S0;
  const std::integral_constant<int, 1> S1;
  auto issue_loads = [&](int kt, auto st_c) {
    constexpr int st = decltype(st_c)::value;
    if (WAVES > LOAD_WAVES && wave >= LOAD_WAVES) return;
    const bool partial = kt * 64 + 64 > n;  // rows past the image are clamped to its last row
    const char* tile0 = reinterpret_cast<const char*>(qkv + size_t(base + kt * 64) * ld);
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      uint32_t ok = k_lo[j], ov = v_lo[j];
      if (partial) {
        const int last = n - 1 - kt * 64;  // >= 0: the tile holds a key
        const int uk = k_row[j] < last ? k_row[j] : last, uv = v_row[j] < last ? v_row[j] : last;
        ok = uint32_t((uk * ld + koff + k_chunk[j] * 8) * 2);
        ov = uint32_t((uv * ld + voff + v_chunk[j] * 8) * 2);
      }
      const uint16_t* gk = reinterpret_cast<const uint16_t*>(tile0 + ok);
      const uint16_t* gv = reinterpret_cast<const uint16_t*>(tile0 + ov);
      // (the index is below SLOTS anyway; the mask lets the compiler see that
      // the load stays inside its stage, so reads of the other stage do not
      // wait for it)
      __builtin_amdgcn_global_load_lds(gk, (lds_void*)&kl[st][((wave * LPT + j) * 64) & (SLOTS - 1)], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(gv, (lds_void*)&vl[st][((wave * LPT + j) * 64) & (SLOTS - 1)], 16, 0, 0);
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T); the q,k,v projection stores
  // q already multiplied by log2(e)/8, so scores come out in exp2 units
  u32x4 qf[QB][4];
#pragma unroll
  for (int tb = 0; tb < QB; ++tb) {
    int t = wq0 + 32 * tb + lrow;
    t = t < n ? t : n - 1;
    const uint16_t* qp = qkv + size_t(base + t) * ld + qoff + 8 * lhalf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[tb][ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
  }
  // The fixed offset -m0 enters the scores of later tiles as the initial
  // accumulator of the score MFMAs: a lane's 16 scores all belong to its one
  // query column, so -m0 replicated in 16 registers, set once after the
  // first tile, serves every later tile at no instruction cost (an earlier
  // form, a 65th score dimension, took one more MFMA per 32 keys).
  floatx16 c_off[QB];
#pragma unroll
  for (int tb = 0; tb < QB; ++tb) c_off[tb] = floatx16{};

  // transposed-read addresses for the V^T fragments: 16-lane group g gets
  // dims D0 + (lane % 16), keys U..U+3 (and U+4..U+7 from the second read)
  const int g = lane >> 4, r16 = lane & 15;
  const int tr_row = 8 * (g >> 1) + (r16 >> 2);          // + ub*32 + sp*16 (+4)
  const int tr_col = 16 * (g & 1) + 4 * (r16 & 3);       // + db*32 (elements)

  floatx16 o[2][QB];
  float m_sc[QB], l_run[QB];
  const int nkt = (n + 63) / 64;

  // One key tile.  MODE 0: first tile of the fixed-offset pass (finds m0);
  // MODE 1: later tiles of that pass (offset folded into the MFMA); MODE 2:
  // online softmax with a running max (fallback pass).
  auto tile = [&](auto mode_c, int kt, auto st_c) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int st = decltype(st_c)::value;  // = kt & 1: LDS addresses are base + immediate
    // ---- S^T = K Q^T (minus the query offset in MODE 1)
    floatx16 s[2][QB];
#pragma unroll
    for (int ub = 0; ub < 2; ++ub)
#pragma unroll
      for (int tb = 0; tb < QB; ++tb) {
        const floatx16 z = {};
        if constexpr (MODE == 1) s[ub][tb] = c_off[tb];
        else s[ub][tb] = z;
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int ub = 0; ub < 2; ++ub) {
        const int row = ub * 32 + lrow;
        const u32x4 kf = kl[st][row * 8 + ((2 * ks + lhalf) ^ kswz(row))];
#pragma unroll
        for (int tb = 0; tb < QB; ++tb) s[ub][tb] = mfma32x32x16(kf, qf[tb][ks], s[ub][tb]);
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
#pragma unroll
            for (int tb = 0; tb < QB; ++tb) s[ub][tb][v] = -INFINITY;
          }
        }
    }
    // ---- probabilities
    u32x4 pf[2][QB][2];
#pragma unroll
    for (int tb = 0; tb < QB; ++tb) {
      float sub = 0.f;  // added to every score before exp2 (MODE 0 and 2)
      if constexpr (MODE != 1) {
        float mx = s[0][tb][0];
#pragma unroll
        for (int ub = 0; ub < 2; ++ub)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[ub][tb][v]);
        mx = pair_max32(mx);
        if constexpr (MODE == 0) {
          sub = -mx;
#pragma unroll
          for (int v = 0; v < 16; ++v) c_off[tb][v] = sub;
        } else {
          if (__any(mx > m_sc[tb] + kRescaleSlack)) {
            const float m_new = fmaxf(m_sc[tb], mx);
            float alpha = __builtin_amdgcn_exp2f(m_sc[tb] - m_new);
            // keeps the rescale a rarely-taken branch
            asm volatile("" : "+v"(alpha));
            m_sc[tb] = m_new;
            l_run[tb] *= alpha;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
              for (int v = 0; v < 16; ++v) o[db][tb][v] *= alpha;
          }
          sub = -m_sc[tb];
        }
      }
#pragma unroll
      for (int ub = 0; ub < 2; ++ub) {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float p[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            if constexpr (MODE == 1) p[v] = __builtin_amdgcn_exp2f(s[ub][tb][8 * sp + v]);
            else p[v] = __builtin_amdgcn_exp2f(s[ub][tb][8 * sp + v] + sub);
          }
          const u32x4 pk = pack8(p);
          pf[ub][tb][sp] = pk;
          l_run[tb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        }
      }
    }
    // ---- O^T += V^T P^T
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(vl[st]);
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
  };
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jq = 0; jq < QB; ++jq)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][jq][v] = 0.f;
#pragma unroll
    for (int tb = 0; tb < QB; ++tb) {
      m_sc[tb] = -INFINITY;
      l_run[tb] = 0.f;
    }
    issue_loads(0, S0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // loads of tile kt+1 (into stage st_next = (kt+1) & 1) behind tile kt's compute
  auto next = [&](int kt, auto st_next) {
    if (kt + 1 < nkt) issue_loads(kt + 1, st_next);
  };
  auto done = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  bool online = a.online_max != 0;
  if (!online) {
    // ---- fixed-offset pass
    reset();
    next(0, S1);
    if (active) tile(std::integral_constant<int, 0>(), 0, S0);
    done();
    int kt = 1;
    for (; kt + 1 < nkt; kt += 2) {  // two tiles per trip: stages 1, 0
      next(kt, S0);
      if (active) tile(std::integral_constant<int, 1>(), kt, S1);
      done();
      next(kt + 1, S1);
      if (active) tile(std::integral_constant<int, 1>(), kt + 1, S0);
      done();
    }
    if (kt < nkt) {
      next(kt, S0);
      if (active) tile(std::integral_constant<int, 1>(), kt, S1);
      done();
    }
    // ---- range check: rerun with a running max if any sum or output overflowed
    int bad = 0;
    if (active) {
#pragma unroll
      for (int tb = 0; tb < QB; ++tb) {
        const float l = pair_sum32(l_run[tb]);
        bad |= !(l > 0.f && l < INFINITY);
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) bad |= !__builtin_isfinite(o[db][tb][v]);
      }
    }
    online = __syncthreads_or(bad) != 0;
  }
  if (online) {
    reset();
    int kt = 0;
    for (; kt + 1 < nkt; kt += 2) {
      next(kt, S1);
      if (active) tile(std::integral_constant<int, 2>(), kt, S0);
      done();
      next(kt + 1, S0);
      if (active) tile(std::integral_constant<int, 2>(), kt + 1, S1);
      done();
    }
    if (kt < nkt) {
      next(kt, S1);
      if (active) tile(std::integral_constant<int, 2>(), kt, S0);
      done();
    }
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
  if (a.q_tile == kAttnQTileBf16) {
    hipLaunchKernelGGL((attn_bf16_kernel<PV_ATTN_QB, PV_ATTN_WAVES>), dim3(a.n_items * a.heads),
                       dim3(PV_ATTN_WAVES * 64), 0, s, a);
  } else if (a.q_tile == kAttnQTileBf16Wide) {
    hipLaunchKernelGGL((attn_bf16_kernel<PV_ATTN_QB, kAttnWavesWide>), dim3(a.n_items * a.heads),
                       dim3(kAttnWavesWide * 64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pv
