// Tower engine and the C ABI declared in include/pv_tower.h.
//
// A forward call: validate + plan on the host, one host->device copy of the
// per-image metadata, attention work list and rotary table into the head of
// the caller's workspace, one kernel that expands the per-row maps, then the
// layer loop
//   patch GEMM -> dual RMSNorm (ln_pre, first attn_norm)
//   L x [QKV GEMM (+RoPE) -> attention -> O GEMM (+= residual) -> RMSNorm
//        -> gate/up GEMM (silu * up) -> down GEMM (+= residual) -> RMSNorm]
//   -> merger GEMM with the 2x2 gather in its A load (or the no-merge copy).
// The residual stream stays fp32 for the whole tower.  Nothing synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/pv_tower.h"
#include "api.h"
#include "kernels.h"
#include "plan.h"

std::string& pv::last_error() {
  thread_local std::string msg;
  return msg;
}

namespace {

using pv::fail;

// A timed launch: event before/after when the tower is profiling.
#define PV_LAUNCH(kind, call)              \
  do {                                     \
    PV_HIP(prof_begin(t, (kind), s));      \
    PV_HIP(call);                          \
    PV_HIP(prof_end(t, s));                \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-channel (R, G, B) normalisation of the Mistral 3 image processor
// ("Mistral 3" (KerasFormers), Mistral3ImageProcessor table): on x / 255.
constexpr float kProcessorMean[3] = {0.48145466f, 0.4578275f, 0.40821073f};
constexpr float kProcessorStd[3] = {0.26862954f, 0.26130258f, 0.27577711f};

// mean_std: host [6] = mean (R, G, B), std (R, G, B), or null for the
// processor's values.  Folded as raw * mul + add (mul = 1 / (255 std),
// add = -mean / std), computed in double and rounded once.
bool norm_affine(const float* mean_std, pv::NormAff* a) {
  for (int c = 0; c < 3; ++c) {
    const double m = mean_std ? mean_std[c] : kProcessorMean[c];
    const double sd = mean_std ? mean_std[3 + c] : kProcessorStd[c];
    if (!(sd > 0.0) || !std::isfinite(m) || !std::isfinite(sd)) return false;
    a->mul[c] = float(1.0 / (255.0 * sd));
    a->add[c] = float(-m / sd);
  }
  return true;
}

// Where the patch embedding takes its pixels from: normalised fp32 planes, or
// uint8 H x W x 3 source images resized in the A-operand load.
struct PixelSource {
  const float* f32 = nullptr;
  const uint8_t* u8 = nullptr;
  pv::NormAff aff{};
};

}  // namespace

struct pv_tower {
  pv_config cfg;
  pv_weights w;
  std::vector<pv_layer_weights> layers;
  pv_projector_weights proj{};  // deeper projector (PV_FLAG_DEEP_PROJECTOR)
  std::vector<float> rope;  // host rotary table
  int32_t rope_maxpos = 0;
  // Staging of the per-call upload: a ring of pinned host buffers, each with
  // the event of its last copy and the bytes it holds.  A call whose upload
  // equals a slot's bytes copies from that slot as it is (no host write, so no
  // wait even while an earlier copy from it is in flight); otherwise it fills
  // the least recently used slot whose copy has completed, adds a slot while
  // fewer than kStagingSlots exist, and only then waits for the oldest copy.
  struct Staging {
    void* host = nullptr;
    size_t cap = 0, used = 0;
    hipEvent_t done = nullptr;
    bool pending = false;
    uint64_t last_use = 0;
  };
  static constexpr int kStagingSlots = 8;
  std::vector<Staging> staging;
  uint64_t uploads = 0;
  std::vector<char> upload_buf;  // the next upload, assembled in plain host memory
  // derived weight copies written by pv_tower_prepare (borrowed caller memory)
  char* prep = nullptr;
  pv::PrepLayout prep_layout;
  // profiling: (class, start, end) per recorded launch; events are pooled
  bool profiling = false;
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
};

namespace {

// Rows of merge_w whose fp4 copy the bf16 merger uses (0: no such copy).
int32_t merge_rows_of(const pv_config& c) {
  if (c.dtype != PV_BF16 || c.merge != 2) return 0;
  return (c.flags & PV_FLAG_DEEP_PROJECTOR) ? c.hidden : c.out_dim;
}

pv::PlanParams plan_params(const pv_tower* t) {
  pv::PlanParams p;
  p.patch = t->cfg.patch;
  p.merge = t->cfg.merge;
  p.max_side = t->cfg.max_side;
  p.hidden = t->cfg.hidden;
  p.mlp = t->cfg.mlp;
  p.out_dim = t->cfg.out_dim;
  p.elem_bytes = t->cfg.dtype == PV_BF16 ? 2 : 4;
  p.q_tile = t->cfg.dtype == PV_BF16 ? pv::kAttnQTileBf16 : pv::kAttnQTileF32;
  p.q_tile_wide = t->cfg.dtype == PV_BF16 ? pv::kAttnQTileBf16Wide : 0;
  p.heads = t->cfg.heads;
  p.slots = 2 * pv::kNumCUs;  // two 8-wave items per CU (registers: 4 waves per SIMD)
  p.slots_wide = pv::kNumCUs;
  p.rope_pairs = 16;
  p.fp8 = (t->cfg.flags & PV_FLAG_FP8) != 0;
  p.prepared = t->prep != nullptr;
  p.deep_out = (t->cfg.flags & PV_FLAG_DEEP_PROJECTOR) ? t->cfg.out_dim : 0;
  p.merge_rows = merge_rows_of(t->cfg);
  return p;
}

pv_status make_plan(const pv_tower* t, const int32_t* image_hw, int32_t n, pv::Plan* plan) {
  std::string err;
  const int rc = pv::build_plan(plan_params(t), image_hw, n, plan, &err);
  if (rc == -1) return fail(PV_ERR_ARG, err);
  if (rc == -2) return fail(PV_ERR_SHAPE, err);
  return PV_OK;
}

hipError_t take_event(pv_tower* t, hipEvent_t* e) {
  if (!t->pool.empty()) {
    *e = t->pool.back();
    t->pool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Records an event before a launch of class `kind` (no-op unless profiling).
hipError_t prof_begin(pv_tower* t, int kind, hipStream_t s) {
  if (!t->profiling) return hipSuccess;
  pv_tower::Rec r{kind, nullptr, nullptr};
  hipError_t e = take_event(t, &r.a);
  if (e == hipSuccess) e = take_event(t, &r.b);
  if (e == hipSuccess) e = hipEventRecord(r.a, s);
  if (e != hipSuccess) return e;
  t->recs.push_back(r);
  return hipSuccess;
}
hipError_t prof_end(pv_tower* t, hipStream_t s) {
  if (!t->profiling) return hipSuccess;
  return hipEventRecord(t->recs.back().b, s);
}

// A staging slot for an upload of `bytes` bytes whose content is t->upload_buf.
pv_status staging_slot(pv_tower* t, size_t bytes, pv_tower::Staging** out, bool* fill) {
  auto done = [&](pv_tower::Staging& st) -> pv_status {
    if (!st.pending) return PV_OK;
    const hipError_t q = hipEventQuery(st.done);
    if (q == hipSuccess) {
      st.pending = false;
    } else if (q != hipErrorNotReady) {
      PV_HIP(q);
    }
    return PV_OK;
  };
  // 1. a slot that already holds these bytes: copy from it as it is
  for (auto& st : t->staging)
    if (st.used == bytes && std::memcmp(st.host, t->upload_buf.data(), bytes) == 0) {
      *out = &st;
      *fill = false;
      return PV_OK;
    }
  // 2. the least recently used slot whose last copy has completed
  pv_tower::Staging* best = nullptr;
  for (auto& st : t->staging) {
    pv_status e = done(st);
    if (e != PV_OK) return e;
    if (!st.pending && (!best || st.last_use < best->last_use)) best = &st;
  }
  // 3. a new slot; 4. else wait for the oldest copy
  if (!best && int(t->staging.size()) < pv_tower::kStagingSlots) {
    t->staging.emplace_back();
    best = &t->staging.back();
    PV_HIP(hipEventCreateWithFlags(&best->done, hipEventDisableTiming));
  }
  if (!best) {
    for (auto& st : t->staging)
      if (!best || st.last_use < best->last_use) best = &st;
    PV_HIP(hipEventSynchronize(best->done));
    best->pending = false;
  }
  if (best->cap < bytes) {
    if (best->host) PV_HIP(hipHostFree(best->host));
    best->host = nullptr;
    best->cap = 0;
    best->used = 0;
    PV_HIP(hipHostMalloc(&best->host, bytes, hipHostMallocDefault));
    best->cap = bytes;
  }
  *out = best;
  *fill = true;
  return PV_OK;
}

// Host -> device upload of [meta | items | rope | src] and expansion of the row maps.
pv_status upload_and_maps(pv_tower* t, const pv::Plan& plan, char* ws, hipStream_t s) {
  const pv::Layout& L = plan.ws;
  std::vector<char>& h = t->upload_buf;
  h.assign(L.upload_bytes, 0);
  std::memcpy(h.data() + L.meta, plan.meta.data(), sizeof(pv::ImageMeta) * plan.meta.size());
  std::memcpy(h.data() + L.items, plan.items.data(), sizeof(pv::AttnItem) * plan.items.size());
  std::memcpy(h.data() + L.rope, t->rope.data(), sizeof(float) * t->rope.size());
  if (!plan.src.empty()) std::memcpy(h.data() + L.src, plan.src.data(), sizeof(pv::SrcImage) * plan.src.size());
  pv_tower::Staging* st = nullptr;
  bool fill = false;
  pv_status e = staging_slot(t, L.upload_bytes, &st, &fill);
  if (e != PV_OK) return e;
  if (fill) {
    std::memcpy(st->host, h.data(), L.upload_bytes);
    st->used = L.upload_bytes;
  }
  PV_HIP(hipMemcpyAsync(ws, st->host, L.upload_bytes, hipMemcpyHostToDevice, s));
  PV_HIP(hipEventRecord(st->done, s));
  st->pending = true;
  st->last_use = ++t->uploads;
  PV_LAUNCH(PV_K_MAPS, pv::build_maps(reinterpret_cast<const pv::ImageMeta*>(ws + L.meta), plan.n_images,
                                       int(plan.n_patches), int(plan.out_rows), t->cfg.merge,
                                       reinterpret_cast<int32_t*>(ws + L.rowinfo),
                                       reinterpret_cast<int32_t*>(ws + L.msrc), s));
  return PV_OK;
}

// Where a layer's derived weight copies are (fp4 gate/up of the bf16
// tower; every fp8 copy of the fp8 variant).
struct WeightCopies {
  void *wq8, *wqs, *wo8, *wos, *b8, *bs, *wd8, *wds;
};

WeightCopies prepared_copies(const pv_tower* t, int l) {
  const pv::PrepLayout& P = t->prep_layout;
  char* b = t->prep + P.layer0 + size_t(l) * P.layer_stride;
  return {b + P.wq8, b + P.wqs, b + P.wo8, b + P.wos, b + P.b8, b + P.bs, b + P.wd8, b + P.wds};
}

// The fp8 copies of one layer's matrices: q|k|v stacked, out-projection,
// gate/up interleaved, down.
hipError_t make_fp8_copies(const pv_layer_weights& lw, const WeightCopies& wc, int D, int F, hipStream_t s) {
  hipError_t e = pv::quant_rows_fp8(lw.wq, D, D, wc.wq8, wc.wqs, 3 * D, 0, s);
  if (e == hipSuccess) e = pv::quant_rows_fp8(lw.wk, D, D, wc.wq8, wc.wqs, 3 * D, D, s);
  if (e == hipSuccess) e = pv::quant_rows_fp8(lw.wv, D, D, wc.wq8, wc.wqs, 3 * D, 2 * D, s);
  if (e == hipSuccess) e = pv::quant_rows_fp8(lw.wo, D, D, wc.wo8, wc.wos, D, 0, s);
  if (e == hipSuccess) e = pv::gateup_fp8(lw.w_gate, lw.w_up, wc.b8, wc.bs, F, D, s);
  if (e == hipSuccess) e = pv::quant_rows_fp8(lw.w_down, D, F, wc.wd8, wc.wds, D, 0, s);
  return e;
}

struct StageStop {
  int32_t stage = -1;  // -1: run to the end
  int32_t layer = 0;
  void* dst = nullptr;
  int64_t dst_bytes = 0;
};

pv_status copy_stage(const StageStop& st, const void* src, size_t bytes, hipStream_t s) {
  if (st.dst_bytes < int64_t(bytes))
    return fail(PV_ERR_CAPACITY, "dst_bytes " + std::to_string(st.dst_bytes) + " < " + std::to_string(bytes));
  PV_HIP(hipMemcpyAsync(st.dst, src, bytes, hipMemcpyDeviceToDevice, s));
  return PV_OK;
}

pv_status run_tower(pv_tower* t, const PixelSource& px, const pv::Plan& plan, void* out, char* ws,
                    const StageStop& st, hipStream_t s) {
  const pv_config& c = t->cfg;
  const bool bf = c.dtype == PV_BF16;
  const bool f8 = bf && (c.flags & PV_FLAG_FP8);  // per-block linear maps in fp8
  const size_t es = bf ? 2 : 4;
  const pv::Layout& L = plan.ws;
  const int N = int(plan.n_patches), D = c.hidden, F = c.mlp;
  float* r = reinterpret_cast<float*>(ws + L.r);
  void* y = ws + L.y;
  void* big = ws + L.big;
  auto gemm = [&](pv::GemmKind k, const pv::GemmArgs& g) { return bf ? pv::gemm_bf16(k, g, s) : pv::gemm_f32(k, g, s); };

  pv::GemmArgs g{};
  g.maps.meta = reinterpret_cast<const pv::ImageMeta*>(ws + L.meta);
  g.maps.rowinfo = reinterpret_cast<const int32_t*>(ws + L.rowinfo);
  g.maps.msrc = reinterpret_cast<const int32_t*>(ws + L.msrc);
  g.maps.rope = reinterpret_cast<const float*>(ws + L.rope);
  g.maps.n_images = plan.n_images;
  g.maps.rope_maxpos = t->rope_maxpos;
  g.maps.patch = c.patch;
  g.hidden = D;
  g.heads = c.heads;

  // ---- patch embedding: X = im2col(pixels) W^T, fp32 into the residual buffer
  if (bf) {
    // pixels as bf16 hi | lo rows of im2col, against weights padded to Kp
    const int Kpatch = 3 * c.patch * c.patch, Kp = pv::patch_kp(c.patch);
    void* wpad = t->prep ? static_cast<void*>(t->prep + t->prep_layout.wpad) : static_cast<void*>(ws + L.wpad);
    if (!t->prep) PV_LAUNCH(PV_K_PATCH, pv::pad_rows(t->w.patch_w, wpad, D, Kpatch, Kp, s));
    if (px.u8)
      PV_LAUNCH(PV_K_OPERAND, pv::im2col_u8_split(px.u8, reinterpret_cast<const pv::SrcImage*>(ws + L.src), g.maps,
                                                 px.aff, big, N, Kpatch, Kp, s));
    else
      PV_LAUNCH(PV_K_OPERAND, pv::im2col_split(px.f32, g.maps, big, N, Kpatch, Kp, s));
    pv::GemmArgs a = g;
    a.M = N; a.N = D; a.K = 2 * Kp; a.kb = Kp;
    a.A = big; a.lda = 2 * Kp;
    a.B0 = wpad; a.ldb = Kp;
    a.C = r; a.ldc = D;
    PV_LAUNCH(PV_K_PATCH, gemm(pv::GEMM_PATCH, a));
  } else {
    const float* pixels = px.f32;
    if (px.u8) {  // resized, normalised planes of every image into the big buffer first
      float* planes = reinterpret_cast<float*>(big);
      for (int i = 0; i < plan.n_images; ++i) {
        const pv::ImageMeta& m = plan.meta[i];
        const pv::SrcImage& sm = plan.src[i];
        const size_t off = (size_t(m.pix_hi) << 32) | m.pix_lo;
        const size_t soff = (size_t(sm.off_hi) << 32) | sm.off_lo;
        PV_LAUNCH(PV_K_OPERAND, pv::resize_norm_u8(px.u8 + soff, sm, m.H, m.W, px.aff, planes + off, s));
      }
      pixels = planes;
    }
    pv::GemmArgs a = g;
    a.M = N; a.N = D; a.K = 3 * c.patch * c.patch;
    a.pixels = pixels;
    a.B0 = t->w.patch_w; a.ldb = a.K;
    a.C = r; a.ldc = D;
    PV_LAUNCH(PV_K_PATCH, gemm(pv::GEMM_PATCH, a));
  }
  if (st.stage == PV_STAGE_PATCH_EMBED) return copy_stage(st, r, size_t(N) * D * 4, s);
  const float eps = float(c.rms_eps);
  const int srows = int(pv::a8_scale_rows(N));
  char* a8 = ws + L.a8;  // fp8 variant: the input of every fp8 linear map
  char* as = ws + L.as;
  if (c.layers == 0 || f8) {
    PV_LAUNCH(PV_K_NORM, pv::rmsnorm(r, t->w.ln_pre, r, N, D, eps, true, s));  // in place, fp32 out
    if (st.stage == PV_STAGE_LN_PRE) return copy_stage(st, r, size_t(N) * D * 4, s);
    if (f8 && c.layers > 0)
      PV_LAUNCH(PV_K_NORM, pv::rmsnorm_fp8(r, t->layers[0].attn_norm, a8, as, N, srows, D, eps, s));
  } else {
    PV_LAUNCH(PV_K_NORM, pv::rmsnorm_dual(r, t->w.ln_pre, t->layers[0].attn_norm, y, N, D, eps, !bf, s));
    if (st.stage == PV_STAGE_LN_PRE) return copy_stage(st, r, size_t(N) * D * 4, s);
  }

  pv::AttnArgs at{};
  at.qkv = big;
  at.out = y;  // y is free once q,k,v are computed
  at.meta = g.maps.meta;
  at.items = reinterpret_cast<const pv::AttnItem*>(ws + L.items);
  at.n_items = int(plan.items.size());
  at.heads = c.heads;
  at.hidden = D;
  at.online_max = (c.flags & PV_FLAG_ATTN_ONLINE_MAX) ? 1 : 0;
  at.q_tile = plan.q_tile;
  at.head_major = 1;
  for (size_t i = 1; i + 1 < plan.cu.size(); ++i)
    if (plan.cu[i + 1] - plan.cu[i] != plan.cu[1] - plan.cu[0]) at.head_major = 0;

  for (int l = 0; l < c.layers; ++l) {
    const pv_layer_weights& lw = t->layers[l];
    const bool stop_here = st.layer == l;
    // fp8 variant: operand in fp8 with one power-of-two scale per 32 k
    auto use_fp8 = [&](pv::GemmArgs& a, int k, const void* b8, const void* bsc, int brows) {
      a.K = 0; a.kb = 0;
      a.A = a8; a.A8 = a8; a.As = as; a.as_rows = srows; a.k8 = k;
      a.B8 = b8; a.Bs = bsc; a.bs_rows = brows; a.low_fmt = 8;
    };
    // this layer's derived weight copies: prepared once, or made here per call
    const WeightCopies wc = t->prep ? prepared_copies(t, l)
                                    : WeightCopies{ws + L.wq8, ws + L.wqs, ws + L.wo8, ws + L.wos,
                                                   ws + L.b8,  ws + L.bs,  ws + L.wd8, ws + L.wds};
    if (f8 && !t->prep) {  // this layer's weights in fp8
      PV_LAUNCH(PV_K_QKV, make_fp8_copies(lw, wc, D, F, s));
    }
    {  // q,k,v with the 2-D rotary in the epilogue
      pv::GemmArgs a = g;
      a.M = N; a.N = 3 * D; a.K = D;
      a.A = y; a.lda = D;
      a.B0 = lw.wq; a.B1 = lw.wk; a.B2 = lw.wv; a.ldb = D;
      a.C = big; a.ldc = 3 * D;
      if (f8) use_fp8(a, D, wc.wq8, wc.wqs, 3 * D);
      PV_LAUNCH(PV_K_QKV, gemm(pv::GEMM_QKV, a));
    }
    if (stop_here && st.stage == PV_STAGE_QKV) return copy_stage(st, big, size_t(N) * 3 * D * es, s);
    PV_LAUNCH(PV_K_ATTN, bf ? pv::attention_bf16(at, s) : pv::attention_f32(at, s));
    if (stop_here && st.stage == PV_STAGE_ATTN) return copy_stage(st, y, size_t(N) * D * es, s);
    {  // out-projection added into the residual
      pv::GemmArgs a = g;
      a.M = N; a.N = D; a.K = D;
      a.A = y; a.lda = D;
      a.B0 = lw.wo; a.ldb = D;
      a.C = r; a.ldc = D;
      if (f8) {
        PV_LAUNCH(PV_K_OPROJ, pv::quant_rows_fp8(y, N, D, a8, as, srows, 0, s));
        use_fp8(a, D, wc.wo8, wc.wos, D);
      }
      PV_LAUNCH(PV_K_OPROJ, gemm(pv::GEMM_OPROJ, a));
    }
    if (stop_here && st.stage == PV_STAGE_ATTN_RESID) return copy_stage(st, r, size_t(N) * D * 4, s);
    // the MLP of the bf16 tower runs its two products on fp16 operands (the
    // input y, silu(gate) * up and fp16 copies of the weights): their bf16
    // rounding would otherwise be the two largest errors of the tower output
    if (f8) {
      PV_LAUNCH(PV_K_NORM_MLP, pv::rmsnorm_fp8(r, lw.ffn_norm, a8, as, N, srows, D, eps, s));
    } else if (bf) {
      if (!t->prep) {  // this layer's gate rows, then up rows, in fp16
        PV_LAUNCH(PV_K_GATEUP, pv::copy_f16(lw.w_gate, (long long)F * D, wc.b8, s));
        PV_LAUNCH(PV_K_GATEUP, pv::copy_f16(lw.w_up, (long long)F * D, static_cast<char*>(wc.b8) + size_t(F) * D * 2, s));
      }
      PV_LAUNCH(PV_K_NORM_MLP, pv::rmsnorm_f16(r, lw.ffn_norm, y, N, D, eps, s));
    } else {
      PV_LAUNCH(PV_K_NORM_MLP, pv::rmsnorm(r, lw.ffn_norm, y, N, D, eps, true, s));
    }
    {  // gate/up with silu(gate) * up in the epilogue
      pv::GemmArgs a = g;
      a.M = N; a.N = F; a.K = D;
      a.A = y; a.lda = D;
      a.B0 = lw.w_gate; a.B1 = lw.w_up; a.ldb = D;
      if (bf && !f8) {  // fp16 y against the fp16 copies (gate rows, then up rows)
        a.B0 = wc.b8; a.B1 = static_cast<char*>(wc.b8) + size_t(F) * D * 2;
        a.f16 = 1;
      }
      a.C = big; a.ldc = F;
      if (f8) use_fp8(a, D, wc.b8, wc.bs, 2 * F);
      PV_LAUNCH(PV_K_GATEUP, gemm(pv::GEMM_GATEUP, a));
    }
    if (stop_here && st.stage == PV_STAGE_MLP_HIDDEN) return copy_stage(st, big, size_t(N) * F * es, s);
    {  // down-projection added into the residual
      pv::GemmArgs a = g;
      a.M = N; a.N = D; a.K = F;
      a.A = big; a.lda = F;
      a.B0 = lw.w_down; a.ldb = F;
      a.C = r; a.ldc = D;
      if (bf && !f8) {  // fp16 silu * up against the fp16 copy of w_down
        if (!t->prep) PV_LAUNCH(PV_K_DOWN, pv::copy_f16(lw.w_down, (long long)D * F, wc.wd8, s));
        a.B0 = wc.wd8;
        a.f16 = 1;
      }
      if (f8) {
        PV_LAUNCH(PV_K_DOWN, pv::quant_rows_fp8(big, N, F, a8, as, srows, 0, s));
        use_fp8(a, F, wc.wd8, wc.wds, D);
      }
      PV_LAUNCH(PV_K_DOWN, gemm(pv::GEMM_DOWN, a));
    }
    if (stop_here && st.stage == PV_STAGE_BLOCK_OUT) return copy_stage(st, r, size_t(N) * D * 4, s);
    if (l + 1 < c.layers) {
      if (f8) PV_LAUNCH(PV_K_NORM, pv::rmsnorm_fp8(r, t->layers[l + 1].attn_norm, a8, as, N, srows, D, eps, s));
      else PV_LAUNCH(PV_K_NORM, pv::rmsnorm(r, t->layers[l + 1].attn_norm, y, N, D, eps, !bf, s));
    }
  }
  if (st.stage >= 0) return fail(PV_ERR_ARG, "stage/layer not reached");

  const bool out_bf16 = bf && c.out_dtype == PV_BF16;
  // bf16 merger: the final residual (or its norm) as bf16 rows in big,
  // which the A loads gather 2x2 (K = 4D), plus its low part in fp4, already
  // gathered in merged-token order (a8 / as), against the fp4 copy of
  // merge_w (prepared, else made here)
  auto merge_args = [&](pv::GemmArgs& a, const float* x, int rows_w) -> pv_status {
    const int T = int(plan.out_rows), srows = int(pv::a8_scale_rows(T));
    void* mw4 = t->prep ? static_cast<void*>(t->prep + t->prep_layout.mw4) : static_cast<void*>(ws + L.mw4);
    void* mws = t->prep ? static_cast<void*>(t->prep + t->prep_layout.mws) : static_cast<void*>(ws + L.mws);
    if (!t->prep) PV_LAUNCH(PV_K_MERGE, pv::rows_fp4(t->w.merge_w, rows_w, 4 * D, mw4, mws, s));
    PV_LAUNCH(PV_K_OPERAND, pv::merge_hi_lo4(x, g.maps.msrc, big, ws + L.a8, ws + L.as, T, srows, D, s));
    a.M = T; a.K = 4 * D; a.kb = 0;
    a.A = big; a.lda = D;
    a.B0 = t->w.merge_w; a.ldb = 4 * D;
    a.A8 = ws + L.a8; a.B8 = mw4; a.As = ws + L.as; a.Bs = mws;
    a.k8 = 4 * D; a.as_rows = srows; a.bs_rows = rows_w; a.low_fmt = 4;
    return PV_OK;
  };
  if (c.merge == 2 && bf && (c.flags & PV_FLAG_DEEP_PROJECTOR)) {
    // deeper projector: RMSNorm (in place, fp32) -> 2x2 gather and 4D -> D
    // (bf16 m in y) -> D -> out_dim with GELU (bf16 a in big) -> out_dim ->
    // out_dim into out
    PV_LAUNCH(PV_K_NORM, pv::rmsnorm(r, t->proj.norm, r, N, D, eps, true, s));
    const int T = int(plan.out_rows), O = c.out_dim;
    pv::GemmArgs a = g;
    const pv_status ms = merge_args(a, r, D);
    if (ms != PV_OK) return ms;
    a.N = D;
    a.C = y; a.ldc = D;
    PV_LAUNCH(PV_K_MERGE, gemm(pv::GEMM_MERGE, a));
    pv::GemmArgs b = g;
    b.M = T; b.N = O; b.K = D;
    b.A = y; b.lda = D;
    b.B0 = t->proj.w1; b.ldb = D;
    b.C = big; b.ldc = O;
    PV_LAUNCH(PV_K_MERGE, gemm(pv::GEMM_GELU, b));
    pv::GemmArgs o = g;
    o.M = T; o.N = O; o.K = O;
    o.A = big; o.lda = O;
    o.B0 = t->proj.w2; o.ldb = O;
    o.C = out; o.ldc = O;
    PV_LAUNCH(PV_K_MERGE, gemm(out_bf16 ? pv::GEMM_PLAIN : pv::GEMM_PLAIN_F32, o));
  } else if (c.merge == 2 && bf) {
    pv::GemmArgs a = g;
    const pv_status ms = merge_args(a, r, c.out_dim);
    if (ms != PV_OK) return ms;
    a.N = c.out_dim;
    a.C = out; a.ldc = c.out_dim;
    PV_LAUNCH(PV_K_MERGE, gemm(out_bf16 ? pv::GEMM_MERGE : pv::GEMM_MERGE_F32, a));
  } else if (c.merge == 2) {
    pv::GemmArgs a = g;
    a.M = int(plan.out_rows); a.N = c.out_dim; a.K = 4 * D;
    a.A = r; a.lda = D;
    a.B0 = t->w.merge_w; a.ldb = 4 * D;
    a.C = out; a.ldc = c.out_dim;
    PV_LAUNCH(PV_K_MERGE, gemm(pv::GEMM_MERGE_F32, a));
  } else if (out_bf16) {
    PV_LAUNCH(PV_K_OPERAND, pv::f32_to_bf16(r, out, size_t(N) * D, s));
  } else {
    PV_HIP(hipMemcpyAsync(out, r, size_t(N) * D * 4, hipMemcpyDeviceToDevice, s));
  }
  return PV_OK;
}

// Target sizes of uint8 source images for this tower (longest edge = max_side,
// grid = patch * merge), the plan of those sizes, and the source offsets.
pv_status make_plan_u8(const pv_tower* t, const int32_t* src_hw, int32_t n, pv::Plan* plan,
                       std::vector<int32_t>* dst_hw, const uint64_t* offsets = nullptr) {
  if (!src_hw) return fail(PV_ERR_ARG, "src_hw must not be null");
  if (n < 1) return fail(PV_ERR_ARG, "n_images must be >= 1 (the tower runs only on image input)");
  dst_hw->assign(size_t(2) * n, 0);
  std::string err;
  for (int32_t i = 0; i < n; ++i) {
    const int rc = pv::resize_target(src_hw[2 * i], src_hw[2 * i + 1], t->cfg.max_side, t->cfg.patch * t->cfg.merge,
                                     &(*dst_hw)[2 * i], &(*dst_hw)[2 * i + 1], &err);
    if (rc == -1) return fail(PV_ERR_ARG, err);
    if (rc == -2) return fail(PV_ERR_SHAPE, "image " + std::to_string(i) + ": " + err);
  }
  pv_status st = make_plan(t, dst_hw->data(), n, plan);
  if (st != PV_OK) return st;
  plan->src.resize(n);
  uint64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    pv::SrcImage& sm = plan->src[i];
    sm.H = src_hw[2 * i];
    sm.W = src_hw[2 * i + 1];
    sm.RH = (*dst_hw)[2 * i];
    sm.RW = (*dst_hw)[2 * i + 1];
    sm.y0 = sm.x0 = 0;
    const uint64_t o = offsets ? offsets[i] : off;
    sm.off_lo = uint32_t(o & 0xffffffffu);
    sm.off_hi = uint32_t(o >> 32);
    off += uint64_t(3) * uint64_t(sm.H) * uint64_t(sm.W);
  }
  return PV_OK;
}

// Tiles of uint8 source images for this tower (tile = max_side, grid =
// patch * merge): layout [n][4] = (resized H, W, tile rows, tile columns),
// then the plan over all tiles (row-major per image, images in order).
pv_status make_plan_tiles_u8(const pv_tower* t, const int32_t* src_hw, int32_t n, int32_t max_num_tiles,
                             pv::Plan* plan, std::vector<int32_t>* layout) {
  if (!src_hw) return fail(PV_ERR_ARG, "src_hw must not be null");
  if (n < 1) return fail(PV_ERR_ARG, "n_images must be >= 1 (the tower runs only on image input)");
  const int32_t tile = t->cfg.max_side, grid = t->cfg.patch * t->cfg.merge;
  if (tile % grid) return fail(PV_ERR_UNSUPPORTED, "the tile edge (max_side) must be a multiple of patch * merge");
  layout->assign(size_t(4) * n, 0);
  std::vector<int32_t> tile_hw;
  std::vector<pv::SrcImage> src;
  std::string err;
  uint64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t* L = &(*layout)[4 * i];
    const int rc = pv::tile_layout(src_hw[2 * i], src_hw[2 * i + 1], tile, grid, max_num_tiles, &L[0], &L[1], &L[2],
                                   &L[3], &err);
    if (rc == -1) return fail(PV_ERR_ARG, err);
    if (rc == -2) return fail(PV_ERR_SHAPE, "image " + std::to_string(i) + ": " + err);
    for (int32_t a = 0; a < L[2]; ++a)
      for (int32_t b = 0; b < L[3]; ++b) {
        pv::SrcImage sm;
        sm.H = src_hw[2 * i];
        sm.W = src_hw[2 * i + 1];
        sm.RH = L[0];
        sm.RW = L[1];
        sm.y0 = a * tile;
        sm.x0 = b * tile;
        sm.off_lo = uint32_t(off & 0xffffffffu);
        sm.off_hi = uint32_t(off >> 32);
        src.push_back(sm);
        tile_hw.push_back(std::min(tile, L[0] - sm.y0));
        tile_hw.push_back(std::min(tile, L[1] - sm.x0));
        if (src.size() > size_t(INT32_MAX / 2)) return fail(PV_ERR_SHAPE, "too many tiles");
      }
    off += uint64_t(3) * uint64_t(src_hw[2 * i]) * uint64_t(src_hw[2 * i + 1]);
  }
  pv_status st = make_plan(t, tile_hw.data(), int32_t(src.size()), plan);
  if (st != PV_OK) return st;
  plan->src = std::move(src);
  return PV_OK;
}

void fill_info(const pv_tower* t, const pv::Plan& plan, pv_plan_info* info) {
  info->n_patches = plan.n_patches;
  info->out_rows = plan.out_rows;
  info->out_cols = t->cfg.merge == 2 ? t->cfg.out_dim : t->cfg.hidden;
  info->workspace_bytes = int64_t(plan.ws.total);
  info->n_images = plan.n_images;
  info->max_patches = plan.max_patches;
  info->attn_q_tile = plan.q_tile;
}

pv_status check_call(const pv_tower* t, const float* pixels, const int32_t* image_hw, int32_t n, const void* dst,
                     const void* ws) {
  if (!t) return fail(PV_ERR_ARG, "tower is null");
  if (!pixels || !image_hw || !dst || !ws) return fail(PV_ERR_ARG, "pixels, image_hw, output and workspace must not be null");
  if (n < 1) return fail(PV_ERR_ARG, "n_images must be >= 1");
  if (!aligned(pixels, 4)) return fail(PV_ERR_ARG, "pixels must be 4-byte aligned");
  if (!aligned(dst, 16)) return fail(PV_ERR_ARG, "output must be 16-byte aligned");
  if (!aligned(ws, 256)) return fail(PV_ERR_ARG, "workspace must be 256-byte aligned");
  return PV_OK;
}

// uint8 forward: max_num_tiles == 0 resizes each image whole (the longest
// edge rule), else cuts it into tiles of max_side.
pv_status forward_u8_common(pv_tower* t, const uint8_t* images, const int32_t* src_hw, int32_t n_images,
                            int32_t max_num_tiles, const float* mean_std, void* out, int64_t out_rows_cap,
                            void* workspace, size_t ws_bytes, void* stream, const uint64_t* offsets = nullptr) {
  pv::last_error().clear();
  if (!t) return fail(PV_ERR_ARG, "tower is null");
  if (!images || !out || !workspace) return fail(PV_ERR_ARG, "images, output and workspace must not be null");
  if (!aligned(out, 16)) return fail(PV_ERR_ARG, "output must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(PV_ERR_ARG, "workspace must be 256-byte aligned");
  PixelSource px;
  px.u8 = images;
  if (!norm_affine(mean_std, &px.aff)) return fail(PV_ERR_ARG, "mean_std must be finite with std > 0");
  pv::Plan plan;
  std::vector<int32_t> hw;
  pv_status st = max_num_tiles > 0 ? make_plan_tiles_u8(t, src_hw, n_images, max_num_tiles, &plan, &hw)
                                   : make_plan_u8(t, src_hw, n_images, &plan, &hw, offsets);
  if (st != PV_OK) return st;
  if (out_rows_cap < plan.out_rows)
    return fail(PV_ERR_CAPACITY, "out_rows_cap " + std::to_string(out_rows_cap) + " < " + std::to_string(plan.out_rows));
  if (ws_bytes < plan.ws.total)
    return fail(PV_ERR_CAPACITY, "workspace " + std::to_string(ws_bytes) + " < " + std::to_string(plan.ws.total));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((st = upload_and_maps(t, plan, ws, s)) != PV_OK) return st;
  return run_tower(t, px, plan, out, ws, StageStop(), s);
}

}  // namespace

pv_status pv::u8_out_rows(const pv_tower* t, const int32_t* src_hw, int32_t n, std::vector<int64_t>* rows,
                          int64_t* row_bytes, int64_t* ws_bytes) {
  pv::Plan plan;
  std::vector<int32_t> hw;
  pv_status st = make_plan_u8(t, src_hw, n, &plan, &hw);
  if (st != PV_OK) return st;
  rows->resize(n);
  for (int32_t i = 0; i < n; ++i)
    (*rows)[i] = (i + 1 < n ? plan.meta[i + 1].tok_base : plan.out_rows) - plan.meta[i].tok_base;
  const int64_t cols = t->cfg.merge == 2 ? t->cfg.out_dim : t->cfg.hidden;
  const int64_t es = (t->cfg.dtype == PV_BF16 && t->cfg.out_dtype == PV_BF16) ? 2 : 4;
  *row_bytes = cols * es;
  *ws_bytes = int64_t(plan.ws.total);
  return PV_OK;
}

pv_status pv::forward_u8_at(pv_tower* t, const uint8_t* images, const int32_t* src_hw, const uint64_t* offsets,
                            int32_t n, const float* mean_std, void* out, int64_t out_rows_cap, void* workspace,
                            size_t ws_bytes, hipStream_t s) {
  return forward_u8_common(t, images, src_hw, n, 0, mean_std, out, out_rows_cap, workspace, ws_bytes, s, offsets);
}

extern "C" {

const char* pv_last_error(void) { return pv::last_error().c_str(); }

const char* pv_status_str(pv_status s) {
  switch (s) {
    case PV_OK: return "PV_OK";
    case PV_ERR_ARG: return "PV_ERR_ARG";
    case PV_ERR_SHAPE: return "PV_ERR_SHAPE";
    case PV_ERR_CAPACITY: return "PV_ERR_CAPACITY";
    case PV_ERR_HIP: return "PV_ERR_HIP";
    case PV_ERR_UNSUPPORTED: return "PV_ERR_UNSUPPORTED";
  }
  return "PV_ERR_UNKNOWN";
}

pv_status pv_tower_create(const pv_config* cfg, const pv_weights* w, pv_tower** out) {
  pv::last_error().clear();
  if (!cfg || !w || !out) return fail(PV_ERR_ARG, "cfg, weights and out must not be null");
  *out = nullptr;
  const pv_config& c = *cfg;
  if (c.dtype != PV_BF16 && c.dtype != PV_F32) return fail(PV_ERR_ARG, "dtype must be PV_BF16 or PV_F32");
  if (c.out_dtype != PV_BF16 && c.out_dtype != PV_F32) return fail(PV_ERR_ARG, "out_dtype must be PV_BF16 or PV_F32");
  if (c.flags & ~(PV_FLAG_ATTN_ONLINE_MAX | PV_FLAG_FP8 | PV_FLAG_DEEP_PROJECTOR | PV_FLAG_ROPE_INTERLEAVED))
    return fail(PV_ERR_ARG, "unknown bits in flags");
  if ((c.flags & PV_FLAG_FP8) && c.dtype != PV_BF16) return fail(PV_ERR_UNSUPPORTED, "PV_FLAG_FP8 needs the bf16 tower");
  const bool deep = (c.flags & PV_FLAG_DEEP_PROJECTOR) != 0;
  if (deep && (c.dtype != PV_BF16 || c.merge != 2))
    return fail(PV_ERR_UNSUPPORTED, "PV_FLAG_DEEP_PROJECTOR needs the bf16 tower with merge == 2");
  if (c.patch < 1 || c.patch > 64) return fail(PV_ERR_ARG, "patch must be in [1, 64]");
  if (c.merge != 1 && c.merge != 2) return fail(PV_ERR_ARG, "merge must be 1 or 2");
  if (c.layers < 0) return fail(PV_ERR_ARG, "layers must be >= 0");
  if (c.hidden <= 0 || c.heads <= 0 || c.mlp <= 0) return fail(PV_ERR_ARG, "hidden, heads and mlp must be > 0");
  if (c.max_side < c.patch * c.merge || c.max_side / c.patch > 32767)
    return fail(PV_ERR_ARG, "max_side must be >= patch*merge and < 32768 patches");
  if (!(c.rope_theta > 0.0) || !(c.rms_eps >= 0.0)) return fail(PV_ERR_ARG, "rope_theta must be > 0 and rms_eps >= 0");
  if (c.hidden % c.heads || c.hidden / c.heads != 64) return fail(PV_ERR_UNSUPPORTED, "head_dim must be 64");
  const int nc = c.hidden / 256;
  if (c.hidden % 256 || !(nc == 1 || nc == 2 || nc == 3 || nc == 4 || nc == 6 || nc == 8))
    return fail(PV_ERR_UNSUPPORTED, "hidden must be 256, 512, 768, 1024, 1536 or 2048");
  // (the GEMMs address a tile's rows of A by a 32-bit byte offset: at most
  // 384 rows of 2 * mlp bytes)
  if (c.mlp % 256 || c.mlp > (1 << 20)) return fail(PV_ERR_UNSUPPORTED, "mlp must be a multiple of 256, at most 2^20");
  if (c.merge == 2 && (c.out_dim <= 0 || c.out_dim % 128)) return fail(PV_ERR_UNSUPPORTED, "out_dim must be a positive multiple of 128");
  if (!w->patch_w || !w->ln_pre) return fail(PV_ERR_ARG, "patch_w and ln_pre must not be null");
  if (c.merge == 2 && !w->merge_w) return fail(PV_ERR_ARG, "merge_w must not be null when merge == 2");
  if (c.layers > 0 && !w->layers) return fail(PV_ERR_ARG, "layers must not be null");
  for (int l = 0; l < c.layers; ++l) {
    const pv_layer_weights& lw = w->layers[l];
    const void* ptrs[] = {lw.attn_norm, lw.wq, lw.wk, lw.wv, lw.wo, lw.ffn_norm, lw.w_gate, lw.w_up, lw.w_down};
    for (const void* p : ptrs) {
      if (!p) return fail(PV_ERR_ARG, "layer " + std::to_string(l) + " has a null weight pointer");
      if (!aligned(p, 16)) return fail(PV_ERR_ARG, "layer " + std::to_string(l) + " weight not 16-byte aligned");
    }
  }
  if (!aligned(w->ln_pre, 16) || (w->merge_w && !aligned(w->merge_w, 16)) || !aligned(w->patch_w, 4))
    return fail(PV_ERR_ARG, "weights must be 16-byte aligned (patch_w 4-byte)");
  if (deep) {
    if (!w->proj || !w->proj->norm || !w->proj->w1 || !w->proj->w2)
      return fail(PV_ERR_ARG, "PV_FLAG_DEEP_PROJECTOR needs proj weights (norm, w1, w2)");
    if (!aligned(w->proj->norm, 16) || !aligned(w->proj->w1, 16) || !aligned(w->proj->w2, 16))
      return fail(PV_ERR_ARG, "projector weights must be 16-byte aligned");
  }

  pv_tower* t = new (std::nothrow) pv_tower();
  if (!t) return fail(PV_ERR_ARG, "out of host memory");
  t->cfg = c;
  t->w = *w;
  if (c.layers > 0) t->layers.assign(w->layers, w->layers + c.layers);
  t->w.layers = t->layers.empty() ? nullptr : t->layers.data();
  if (deep) t->proj = *w->proj;
  t->w.proj = deep ? &t->proj : nullptr;
  t->rope_maxpos = std::max(1, c.max_side / c.patch);
  pv::build_rope_table(c.rope_theta, 16, t->rope_maxpos, (c.flags & PV_FLAG_ROPE_INTERLEAVED) != 0, &t->rope);
  *out = t;
  return PV_OK;
}

void pv_tower_destroy(pv_tower* t) {
  if (!t) return;
  for (auto& st : t->staging) {
    if (st.done) {
      (void)hipEventSynchronize(st.done);
      (void)hipEventDestroy(st.done);
    }
    if (st.host) (void)hipHostFree(st.host);
  }
  for (auto& r : t->recs) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : t->pool) (void)hipEventDestroy(e);
  delete t;
}

pv_status pv_tower_plan(const pv_tower* t, const int32_t* image_hw, int32_t n_images, pv_plan_info* info) {
  pv::last_error().clear();
  if (!t || !info) return fail(PV_ERR_ARG, "tower and info must not be null");
  pv::Plan plan;
  pv_status st = make_plan(t, image_hw, n_images, &plan);
  if (st != PV_OK) return st;
  fill_info(t, plan, info);
  return PV_OK;
}

pv_status pv_tower_prepared_bytes(const pv_tower* t, int64_t* bytes) {
  pv::last_error().clear();
  if (!t || !bytes) return fail(PV_ERR_ARG, "tower and bytes must not be null");
  const pv_config& c = t->cfg;
  *bytes = c.dtype == PV_BF16 ? int64_t(pv::prep_layout(c.patch, c.hidden, c.mlp, c.layers,
                                                        (c.flags & PV_FLAG_FP8) != 0, merge_rows_of(c))
                                           .total)
                               : 0;
  return PV_OK;
}

pv_status pv_tower_prepare(pv_tower* t, void* mem, int64_t mem_bytes, void* stream) {
  pv::last_error().clear();
  if (!t) return fail(PV_ERR_ARG, "tower is null");
  const pv_config& c = t->cfg;
  if (!mem) {  // detach: derive the copies per call again
    t->prep = nullptr;
    return PV_OK;
  }
  if (c.dtype != PV_BF16) return PV_OK;  // the fp32 tower uses its weights as given
  if (!aligned(mem, 256)) return fail(PV_ERR_ARG, "mem must be 256-byte aligned");
  const bool f8 = (c.flags & PV_FLAG_FP8) != 0;
  const pv::PrepLayout P = pv::prep_layout(c.patch, c.hidden, c.mlp, c.layers, f8, merge_rows_of(c));
  if (mem_bytes < int64_t(P.total))
    return fail(PV_ERR_CAPACITY, "mem_bytes " + std::to_string(mem_bytes) + " < " + std::to_string(P.total));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* m = static_cast<char*>(mem);
  const int D = c.hidden, F = c.mlp;
  t->prep = nullptr;  // a failed preparation leaves the tower deriving per call
  PV_HIP(pv::pad_rows(t->w.patch_w, m + P.wpad, D, 3 * c.patch * c.patch, pv::patch_kp(c.patch), s));
  for (int l = 0; l < c.layers; ++l) {
    const pv_layer_weights& lw = t->layers[l];
    char* b = m + P.layer0 + size_t(l) * P.layer_stride;
    const WeightCopies wc{b + P.wq8, b + P.wqs, b + P.wo8, b + P.wos, b + P.b8, b + P.bs, b + P.wd8, b + P.wds};
    if (f8)
      PV_HIP(make_fp8_copies(lw, wc, D, F, s));
    else
    {
      PV_HIP(pv::copy_f16(lw.w_gate, (long long)F * D, wc.b8, s));
      PV_HIP(pv::copy_f16(lw.w_up, (long long)F * D, static_cast<char*>(wc.b8) + size_t(F) * D * 2, s));
      PV_HIP(pv::copy_f16(lw.w_down, (long long)D * F, wc.wd8, s));
    }
  }
  if (P.mw4 || P.mws) PV_HIP(pv::rows_fp4(t->w.merge_w, merge_rows_of(c), 4 * D, m + P.mw4, m + P.mws, s));
  t->prep = m;
  t->prep_layout = P;
  return PV_OK;
}

pv_status pv_resize_target(const int32_t* src_hw, int32_t n_images, int32_t longest_edge, int32_t grid,
                           int32_t* dst_hw) {
  pv::last_error().clear();
  if (!src_hw || !dst_hw) return fail(PV_ERR_ARG, "src_hw and dst_hw must not be null");
  if (n_images < 1) return fail(PV_ERR_ARG, "n_images must be >= 1");
  std::string err;
  for (int32_t i = 0; i < n_images; ++i) {
    int32_t th = 0, tw = 0;
    const int rc = pv::resize_target(src_hw[2 * i], src_hw[2 * i + 1], longest_edge, grid, &th, &tw, &err);
    if (rc == -1) return fail(PV_ERR_ARG, err);
    if (rc == -2) return fail(PV_ERR_SHAPE, "image " + std::to_string(i) + ": " + err);
    dst_hw[2 * i] = th;
    dst_hw[2 * i + 1] = tw;
  }
  return PV_OK;
}

pv_status pv_tower_plan_u8(const pv_tower* t, const int32_t* src_hw, int32_t n_images, int32_t* dst_hw,
                           pv_plan_info* info) {
  pv::last_error().clear();
  if (!t || !info) return fail(PV_ERR_ARG, "tower and info must not be null");
  pv::Plan plan;
  std::vector<int32_t> hw;
  pv_status st = make_plan_u8(t, src_hw, n_images, &plan, &hw);
  if (st != PV_OK) return st;
  if (dst_hw) std::memcpy(dst_hw, hw.data(), sizeof(int32_t) * hw.size());
  fill_info(t, plan, info);
  return PV_OK;
}

pv_status pv_tower_forward_u8(pv_tower* t, const uint8_t* images, const int32_t* src_hw, int32_t n_images,
                              const float* mean_std, void* out, int64_t out_rows_cap, void* workspace,
                              size_t ws_bytes, void* stream) {
  return forward_u8_common(t, images, src_hw, n_images, 0, mean_std, out, out_rows_cap, workspace, ws_bytes, stream);
}

pv_status pv_tower_forward_tiles_u8(pv_tower* t, const uint8_t* images, const int32_t* src_hw, int32_t n_images,
                                    int32_t max_num_tiles, const float* mean_std, void* out, int64_t out_rows_cap,
                                    void* workspace, size_t ws_bytes, void* stream) {
  if (max_num_tiles < 1) {
    pv::last_error() = "max_num_tiles must be >= 1";
    return PV_ERR_ARG;
  }
  return forward_u8_common(t, images, src_hw, n_images, max_num_tiles, mean_std, out, out_rows_cap, workspace,
                           ws_bytes, stream);
}

pv_status pv_tile_layout(const int32_t* src_hw, int32_t n_images, int32_t tile, int32_t grid, int32_t max_num_tiles,
                         int32_t* layout) {
  pv::last_error().clear();
  if (!src_hw || !layout) return fail(PV_ERR_ARG, "src_hw and layout must not be null");
  if (n_images < 1) return fail(PV_ERR_ARG, "n_images must be >= 1");
  std::string err;
  for (int32_t i = 0; i < n_images; ++i) {
    int32_t* L = layout + 4 * i;
    const int rc = pv::tile_layout(src_hw[2 * i], src_hw[2 * i + 1], tile, grid, max_num_tiles, &L[0], &L[1], &L[2],
                                   &L[3], &err);
    if (rc == -1) return fail(PV_ERR_ARG, err);
    if (rc == -2) return fail(PV_ERR_SHAPE, "image " + std::to_string(i) + ": " + err);
  }
  return PV_OK;
}

pv_status pv_tower_plan_tiles_u8(const pv_tower* t, const int32_t* src_hw, int32_t n_images, int32_t max_num_tiles,
                                 int32_t* layout, pv_plan_info* info) {
  pv::last_error().clear();
  if (!t || !info) return fail(PV_ERR_ARG, "tower and info must not be null");
  pv::Plan plan;
  std::vector<int32_t> lay;
  pv_status st = make_plan_tiles_u8(t, src_hw, n_images, max_num_tiles, &plan, &lay);
  if (st != PV_OK) return st;
  if (layout) std::memcpy(layout, lay.data(), sizeof(int32_t) * lay.size());
  fill_info(t, plan, info);
  return PV_OK;
}

pv_status pv_quantize_fp8(const void* src, int64_t rows, int32_t K, void* codes, void* scales, void* stream) {
  pv::last_error().clear();
  if (!src || !codes || !scales) return fail(PV_ERR_ARG, "src, codes and scales must not be null");
  if (rows < 1 || rows > INT32_MAX || K < 128 || K % 128) return fail(PV_ERR_ARG, "rows must be >= 1 and K a positive multiple of 128");
  if (int64_t(rows) * K > (int64_t(1) << 40)) return fail(PV_ERR_ARG, "matrix too large");
  if (!aligned(src, 16) || !aligned(codes, 16)) return fail(PV_ERR_ARG, "src and codes must be 16-byte aligned");
  PV_HIP(pv::quant_rows_fp8(src, int(rows), K, codes, scales, int(rows), 0, static_cast<hipStream_t>(stream)));
  return PV_OK;
}

pv_status pv_config_preset(int32_t preset, int32_t dtype, pv_config* cfg) {
  pv::last_error().clear();
  if (!cfg) return fail(PV_ERR_ARG, "cfg must not be null");
  if (dtype != PV_BF16 && dtype != PV_F32) return fail(PV_ERR_ARG, "dtype must be PV_BF16 or PV_F32");
  pv_config c{};
  c.hidden = 1024;
  c.heads = 16;
  c.mlp = 4096;
  c.layers = 24;
  c.rope_theta = 1.0e4;
  c.rms_eps = 1.0e-5;
  c.dtype = dtype;
  c.out_dtype = dtype;
  c.flags = 0;
  if (preset == PV_PRESET_MISTRAL3) {
    c.patch = 14;
    c.merge = 2;
    c.out_dim = 5120;
    c.max_side = 1540;
  } else if (preset == PV_PRESET_PIXTRAL12B) {
    c.patch = 16;
    c.merge = 1;
    c.out_dim = 0;
    c.max_side = 1024;
  } else {
    return fail(PV_ERR_ARG, "unknown preset");
  }
  *cfg = c;
  return PV_OK;
}

pv_status pv_preprocess_u8(const uint8_t* images, const int32_t* src_hw, const int32_t* dst_hw, int32_t n_images,
                           const float* mean_std, float* out, void* stream) {
  pv::last_error().clear();
  if (!images || !src_hw || !dst_hw || !out) return fail(PV_ERR_ARG, "images, src_hw, dst_hw and out must not be null");
  if (n_images < 1) return fail(PV_ERR_ARG, "n_images must be >= 1");
  if (!aligned(out, 4)) return fail(PV_ERR_ARG, "out must be 4-byte aligned");
  pv::NormAff aff;
  if (!norm_affine(mean_std, &aff)) return fail(PV_ERR_ARG, "mean_std must be finite with std > 0");
  for (int32_t i = 0; i < n_images; ++i) {
    const int32_t v[4] = {src_hw[2 * i], src_hw[2 * i + 1], dst_hw[2 * i], dst_hw[2 * i + 1]};
    for (int32_t x : v)
      if (x < 1 || x > pv::kMaxSrcSide)
        return fail(PV_ERR_SHAPE, "image " + std::to_string(i) + ": every side must be in [1, " +
                                      std::to_string(pv::kMaxSrcSide) + "]");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  size_t soff = 0, doff = 0;
  for (int32_t i = 0; i < n_images; ++i) {
    const int32_t sH = src_hw[2 * i], sW = src_hw[2 * i + 1], tH = dst_hw[2 * i], tW = dst_hw[2 * i + 1];
    pv::SrcImage sm{};
    sm.H = sH;
    sm.W = sW;
    sm.RH = tH;
    sm.RW = tW;
    PV_HIP(pv::resize_norm_u8(images + soff, sm, tH, tW, aff, out + doff, s));
    soff += size_t(3) * sH * sW;
    doff += size_t(3) * tH * tW;
  }
  return PV_OK;
}

pv_status pv_tower_forward(pv_tower* t, const float* pixels, const int32_t* image_hw, int32_t n_images, void* out,
                           int64_t out_rows_cap, void* workspace, size_t ws_bytes, void* stream) {
  pv::last_error().clear();
  pv_status st = check_call(t, pixels, image_hw, n_images, out, workspace);
  if (st != PV_OK) return st;
  pv::Plan plan;
  if ((st = make_plan(t, image_hw, n_images, &plan)) != PV_OK) return st;
  if (out_rows_cap < plan.out_rows)
    return fail(PV_ERR_CAPACITY, "out_rows_cap " + std::to_string(out_rows_cap) + " < " + std::to_string(plan.out_rows));
  if (ws_bytes < plan.ws.total)
    return fail(PV_ERR_CAPACITY, "workspace " + std::to_string(ws_bytes) + " < " + std::to_string(plan.ws.total));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((st = upload_and_maps(t, plan, ws, s)) != PV_OK) return st;
  PixelSource px;
  px.f32 = pixels;
  return run_tower(t, px, plan, out, ws, StageStop(), s);
}

pv_status pv_tower_forward_stage(pv_tower* t, const float* pixels, const int32_t* image_hw, int32_t n_images,
                                 int32_t stage, int32_t layer, void* dst, int64_t dst_bytes, void* workspace,
                                 size_t ws_bytes, void* stream) {
  pv::last_error().clear();
  pv_status st = check_call(t, pixels, image_hw, n_images, dst, workspace);
  if (st != PV_OK) return st;
  if (stage < PV_STAGE_PATCH_EMBED || stage > PV_STAGE_BLOCK_OUT) return fail(PV_ERR_ARG, "unknown stage");
  if (stage >= PV_STAGE_QKV && (layer < 0 || layer >= t->cfg.layers)) return fail(PV_ERR_ARG, "layer out of range");
  pv::Plan plan;
  if ((st = make_plan(t, image_hw, n_images, &plan)) != PV_OK) return st;
  if (ws_bytes < plan.ws.total)
    return fail(PV_ERR_CAPACITY, "workspace " + std::to_string(ws_bytes) + " < " + std::to_string(plan.ws.total));
  const size_t es = t->cfg.dtype == PV_BF16 ? 2 : 4;
  const size_t N = size_t(plan.n_patches), D = size_t(t->cfg.hidden);
  size_t need = N * D * 4;
  if (stage == PV_STAGE_QKV) need = N * 3 * D * es;
  if (stage == PV_STAGE_ATTN) need = N * D * es;
  if (stage == PV_STAGE_MLP_HIDDEN) need = N * size_t(t->cfg.mlp) * es;
  if (dst_bytes < int64_t(need))
    return fail(PV_ERR_CAPACITY, "dst_bytes " + std::to_string(dst_bytes) + " < " + std::to_string(need));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((st = upload_and_maps(t, plan, ws, s)) != PV_OK) return st;
  StageStop stop;
  stop.stage = stage;
  stop.layer = stage >= PV_STAGE_QKV ? layer : -1;
  stop.dst = dst;
  stop.dst_bytes = dst_bytes;
  PixelSource px;
  px.f32 = pixels;
  return run_tower(t, px, plan, nullptr, ws, stop, s);
}

pv_status pv_tower_index_maps(pv_tower* t, const int32_t* image_hw, int32_t n_images, int32_t* cu_seqlens,
                              int32_t* patch_rc, int32_t* merge_src, int32_t on_device, void* workspace,
                              size_t ws_bytes, void* stream) {
  pv::last_error().clear();
  if (!t || !cu_seqlens || !patch_rc) return fail(PV_ERR_ARG, "tower, cu_seqlens and patch_rc must not be null");
  pv::Plan plan;
  pv_status st = make_plan(t, image_hw, n_images, &plan);
  if (st != PV_OK) return st;
  if (!on_device) {
    pv::host_index_maps(plan, t->cfg.merge, cu_seqlens, patch_rc, merge_src);
    return PV_OK;
  }
  if (!workspace) return fail(PV_ERR_ARG, "workspace must not be null when on_device != 0");
  if (!aligned(workspace, 256)) return fail(PV_ERR_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < plan.ws.total)
    return fail(PV_ERR_CAPACITY, "workspace " + std::to_string(ws_bytes) + " < " + std::to_string(plan.ws.total));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((st = upload_and_maps(t, plan, ws, s)) != PV_OK) return st;
  PV_HIP(pv::export_maps(reinterpret_cast<const pv::ImageMeta*>(ws + plan.ws.meta),
                         reinterpret_cast<const int32_t*>(ws + plan.ws.rowinfo), plan.n_images,
                         int(plan.n_patches), cu_seqlens, patch_rc, s));
  if (merge_src && t->cfg.merge == 2 && plan.out_rows > 0)
    PV_HIP(hipMemcpyAsync(merge_src, ws + plan.ws.msrc, size_t(plan.out_rows) * 16, hipMemcpyDeviceToDevice, s));
  return PV_OK;
}

size_t pv_scatter_workspace_bytes(int64_t seq_len) { return pv::scatter_workspace_bytes(seq_len); }

pv_status pv_scatter_image_embeddings(const int32_t* token_ids, int64_t seq_len, int32_t image_token_id,
                                      const void* image_emb, int64_t n_image_rows, void* text_emb, int32_t dim,
                                      int32_t elem_bytes, int32_t* status, void* workspace, size_t ws_bytes,
                                      void* stream) {
  pv::last_error().clear();
  pv_status st = pv::scatter_check(token_ids, seq_len, image_emb, n_image_rows, text_emb, dim, elem_bytes, status);
  if (st != PV_OK) return st;
  if (!workspace) return fail(PV_ERR_ARG, "workspace must not be null");
  if (!aligned(workspace, 256)) return fail(PV_ERR_ARG, "workspace must be 256-byte aligned");
  const size_t need = pv::scatter_workspace_bytes(seq_len);
  if (ws_bytes < need)
    return fail(PV_ERR_CAPACITY, "workspace " + std::to_string(ws_bytes) + " < " + std::to_string(need));
  PV_HIP(pv::scatter_rows(token_ids, seq_len, image_token_id, image_emb, n_image_rows, text_emb,
                          int64_t(dim) * elem_bytes, status, workspace, static_cast<hipStream_t>(stream)));
  return PV_OK;
}

}  // extern "C"

// Argument checks shared by the masked-scatter entry points (host only).
pv_status pv::scatter_check(const int32_t* token_ids, int64_t seq_len, const void* image_emb, int64_t n_image_rows,
                            const void* text_emb, int32_t dim, int32_t elem_bytes, const int32_t* status) {
  if (!status) return fail(PV_ERR_ARG, "status must not be null");
  if (seq_len < 0 || n_image_rows < 0) return fail(PV_ERR_ARG, "seq_len and n_image_rows must be >= 0");
  if (seq_len > INT32_MAX || n_image_rows > INT32_MAX) return fail(PV_ERR_ARG, "seq_len and n_image_rows must fit int32");
  if (dim < 1) return fail(PV_ERR_ARG, "dim must be >= 1");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(PV_ERR_ARG, "elem_bytes must be 2 (bf16) or 4 (fp32)");
  if ((int64_t(dim) * elem_bytes) % 16) return fail(PV_ERR_ARG, "rows must be a multiple of 16 bytes");
  if (seq_len > 0 && (!token_ids || !text_emb)) return fail(PV_ERR_ARG, "token_ids and text_emb must not be null");
  if (n_image_rows > 0 && !image_emb) return fail(PV_ERR_ARG, "image_emb must not be null");
  if (!aligned(image_emb, 16) || !aligned(text_emb, 16) || !aligned(token_ids, 4) || !aligned(status, 4))
    return fail(PV_ERR_ARG, "image_emb and text_emb must be 16-byte aligned, token_ids and status 4-byte aligned");
  return PV_OK;
}

extern "C" {

pv_status pv_tower_set_profiling(pv_tower* t, int32_t enable) {
  pv::last_error().clear();
  if (!t) return fail(PV_ERR_ARG, "tower is null");
  if (enable) {
    for (auto& r : t->recs) {
      PV_HIP(hipEventSynchronize(r.b));
      t->pool.push_back(r.a);
      t->pool.push_back(r.b);
    }
    t->recs.clear();
  }
  t->profiling = enable != 0;
  return PV_OK;
}

pv_status pv_tower_read_profile(pv_tower* t, double* ms, int64_t* launches, int32_t reset) {
  pv::last_error().clear();
  if (!t || !ms || !launches) return fail(PV_ERR_ARG, "tower, ms and launches must not be null");
  for (int k = 0; k < PV_K_COUNT; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  for (auto& r : t->recs) {
    PV_HIP(hipEventSynchronize(r.b));
    float e = 0.f;
    PV_HIP(hipEventElapsedTime(&e, r.a, r.b));
    ms[r.kind] += e;
    launches[r.kind] += 1;
  }
  if (reset) {
    for (auto& r : t->recs) {
      t->pool.push_back(r.a);
      t->pool.push_back(r.b);
    }
    t->recs.clear();
  }
  return PV_OK;
}

}  // extern "C"
