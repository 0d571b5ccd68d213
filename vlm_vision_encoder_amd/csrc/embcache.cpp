// Multimodal embeddings cache: the tower's output rows of uint8 images, kept
// in caller-owned device memory and keyed by image content, so an image seen
// before skips the tower (the inference-research record names a per-model
// multimodal embeddings cache, next to an encoder side stream, as an
// engine's answer to encoder cost).
//
// Storage is a ring of output rows.  A call's missed images are computed by
// one tower forward straight into a contiguous run of rows at the ring head
// (wrapping to row 0 when the run does not fit before the end); entries whose
// rows that run overlaps are evicted, so the oldest insertions go first.
// Every image's rows are then copied from the cache into the caller's
// output.  All work is enqueued on the caller's stream in this order: the
// copies of hits, the forward of the misses, the copies of the misses, so a
// hit evicted by the same call is read before it is overwritten.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <new>
#include <utility>
#include <vector>

#include "../../include/pv_tower.h"
#include "api.h"
#include "kernels.h"
#include "plan.h"

struct pv_embcache {
  pv_tower* tower = nullptr;
  char* mem = nullptr;
  int64_t capacity_rows = 0;
  int64_t row_bytes = 0;
  bool has_ms = false;
  float mean_std[6] = {};
  struct Entry {
    int64_t row0, rows;
  };
  using Key = std::pair<uint64_t, uint64_t>;
  std::map<Key, Entry> entries;
  std::map<int64_t, Key> by_row;  // first row -> key, to find what a new run overlaps
  int64_t head = 0;
  int64_t rows_used = 0;
  int64_t hits = 0, misses = 0;
  void* pinned = nullptr;  // device keys land here when the cache computes them
  size_t pinned_bytes = 0;
};

namespace {

using pv::fail;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

void evict_overlapping(pv_embcache* c, int64_t lo, int64_t hi) {
  auto it = c->by_row.upper_bound(lo);
  if (it != c->by_row.begin()) --it;
  while (it != c->by_row.end() && it->first < hi) {
    const auto e = c->entries.find(it->second);
    const int64_t r0 = e->second.row0, r1 = r0 + e->second.rows;
    if (r1 > lo) {
      c->rows_used -= e->second.rows;
      c->entries.erase(e);
      it = c->by_row.erase(it);
    } else {
      ++it;
    }
  }
}

// Workspace of a cached call: device keys + their accumulators, then the
// tower's own workspace for all n images.
pv_status cached_layout(const pv_embcache* c, const int32_t* src_hw, int32_t n, std::vector<int64_t>* rows,
                        size_t* keys_off, size_t* acc_off, size_t* tower_off, size_t* total) {
  int64_t row_bytes = 0, tower_ws = 0;
  pv_status st = pv::u8_out_rows(c->tower, src_hw, n, rows, &row_bytes, &tower_ws);
  if (st != PV_OK) return st;
  *keys_off = 0;
  *acc_off = align256(size_t(n) * 16);
  *tower_off = *acc_off + pv::image_keys_workspace_bytes(n);
  *total = *tower_off + size_t(tower_ws);
  return PV_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

size_t pv_image_keys_workspace_bytes(int32_t n_images) {
  return n_images > 0 ? pv::image_keys_workspace_bytes(n_images) : 0;
}

pv_status pv_image_keys_u8(const uint8_t* images, const int32_t* src_hw, int32_t n_images, uint64_t* keys,
                           void* workspace, size_t ws_bytes, void* stream) {
  pv::last_error().clear();
  if (!images || !src_hw || !keys || !workspace) return fail(PV_ERR_ARG, "images, src_hw, keys and workspace must not be null");
  if (n_images < 1) return fail(PV_ERR_ARG, "n_images must be >= 1");
  if (!aligned(images, 4) || !aligned(keys, 8) || !aligned(workspace, 256))
    return fail(PV_ERR_ARG, "images must be 4-byte, keys 8-byte and workspace 256-byte aligned");
  std::vector<uint64_t> off(n_images);
  uint64_t o = 0;
  for (int32_t i = 0; i < n_images; ++i) {
    const int32_t H = src_hw[2 * i], W = src_hw[2 * i + 1];
    if (H < 1 || W < 1 || H > pv::kMaxSrcSide || W > pv::kMaxSrcSide)
      return fail(PV_ERR_SHAPE, "image " + std::to_string(i) + ": each side must be in [1, 32768]");
    off[i] = o;
    o += uint64_t(3) * uint64_t(H) * uint64_t(W);
  }
  if (ws_bytes < pv::image_keys_workspace_bytes(n_images)) return fail(PV_ERR_CAPACITY, "workspace too small");
  PV_HIP(pv::image_keys(images, src_hw, off.data(), n_images, keys, workspace, static_cast<hipStream_t>(stream)));
  return PV_OK;
}

pv_status pv_embcache_create(pv_tower* t, const float* mean_std, void* cache_mem, int64_t cache_bytes,
                             pv_embcache** out) {
  pv::last_error().clear();
  if (!t || !cache_mem || !out) return fail(PV_ERR_ARG, "tower, cache_mem and out must not be null");
  *out = nullptr;
  if (!aligned(cache_mem, 16)) return fail(PV_ERR_ARG, "cache_mem must be 16-byte aligned");
  const int32_t one[2] = {1, 1};
  std::vector<int64_t> rows;
  int64_t row_bytes = 0, ws = 0;
  pv_status st = pv::u8_out_rows(t, one, 1, &rows, &row_bytes, &ws);
  if (st != PV_OK) return st;
  if (cache_bytes < row_bytes) return fail(PV_ERR_CAPACITY, "cache_bytes holds no output row");
  if (mean_std)
    for (int c = 0; c < 6; ++c)
      if (!(mean_std[c] == mean_std[c]) || (c >= 3 && !(mean_std[c] > 0.f)))
        return fail(PV_ERR_ARG, "mean_std must be finite with std > 0");
  pv_embcache* c = new (std::nothrow) pv_embcache();
  if (!c) return fail(PV_ERR_ARG, "out of host memory");
  c->tower = t;
  c->mem = static_cast<char*>(cache_mem);
  c->row_bytes = row_bytes;
  c->capacity_rows = cache_bytes / row_bytes;
  if (mean_std) {
    c->has_ms = true;
    std::memcpy(c->mean_std, mean_std, sizeof(c->mean_std));
  }
  *out = c;
  return PV_OK;
}

void pv_embcache_destroy(pv_embcache* c) {
  if (!c) return;
  if (c->pinned) (void)hipHostFree(c->pinned);
  delete c;
}

pv_status pv_embcache_clear(pv_embcache* c) {
  pv::last_error().clear();
  if (!c) return fail(PV_ERR_ARG, "cache is null");
  c->entries.clear();
  c->by_row.clear();
  c->head = 0;
  c->rows_used = 0;
  return PV_OK;
}

pv_status pv_embcache_stats(const pv_embcache* c, int64_t* stats) {
  pv::last_error().clear();
  if (!c || !stats) return fail(PV_ERR_ARG, "cache and stats must not be null");
  stats[0] = int64_t(c->entries.size());
  stats[1] = c->rows_used;
  stats[2] = c->capacity_rows;
  stats[3] = c->hits;
  stats[4] = c->misses;
  return PV_OK;
}

pv_status pv_embcache_workspace_bytes(const pv_embcache* c, const int32_t* src_hw, int32_t n_images,
                                      int64_t* bytes) {
  pv::last_error().clear();
  if (!c || !src_hw || !bytes) return fail(PV_ERR_ARG, "cache, src_hw and bytes must not be null");
  if (n_images < 1) return fail(PV_ERR_ARG, "n_images must be >= 1");
  std::vector<int64_t> rows;
  size_t ko, ao, to, total;
  pv_status st = cached_layout(c, src_hw, n_images, &rows, &ko, &ao, &to, &total);
  if (st != PV_OK) return st;
  *bytes = int64_t(total);
  return PV_OK;
}

pv_status pv_tower_forward_cached_u8(pv_embcache* c, const uint8_t* images, const int32_t* src_hw,
                                     int32_t n_images, const uint64_t* keys, void* out, int64_t out_rows_cap,
                                     void* workspace, size_t ws_bytes, void* stream, int32_t* hit) {
  pv::last_error().clear();
  if (!c || !images || !src_hw || !out || !workspace)
    return fail(PV_ERR_ARG, "cache, images, src_hw, output and workspace must not be null");
  if (n_images < 1) return fail(PV_ERR_ARG, "n_images must be >= 1");
  if (!aligned(out, 16) || !aligned(workspace, 256))
    return fail(PV_ERR_ARG, "output must be 16-byte and workspace 256-byte aligned");
  if (!keys && !aligned(images, 4)) return fail(PV_ERR_ARG, "images must be 4-byte aligned to be hashed");
  std::vector<int64_t> rows;
  size_t keys_off, acc_off, tower_off, total;
  pv_status st = cached_layout(c, src_hw, n_images, &rows, &keys_off, &acc_off, &tower_off, &total);
  if (st != PV_OK) return st;
  if (ws_bytes < total)
    return fail(PV_ERR_CAPACITY, "workspace " + std::to_string(ws_bytes) + " < " + std::to_string(total));
  int64_t out_total = 0;
  std::vector<int64_t> out_row0(n_images);
  for (int32_t i = 0; i < n_images; ++i) {
    out_row0[i] = out_total;
    out_total += rows[i];
  }
  if (out_rows_cap < out_total)
    return fail(PV_ERR_CAPACITY, "out_rows_cap " + std::to_string(out_rows_cap) + " < " + std::to_string(out_total));
  std::vector<uint64_t> off(n_images);
  uint64_t o = 0;
  for (int32_t i = 0; i < n_images; ++i) {
    off[i] = o;
    o += uint64_t(3) * uint64_t(src_hw[2 * i]) * uint64_t(src_hw[2 * i + 1]);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);

  // keys: the caller's, or hashed on the device and read back (synchronises)
  const uint64_t* k = keys;
  if (!k) {
    const size_t need = size_t(n_images) * 16;
    if (c->pinned_bytes < need) {
      if (c->pinned) PV_HIP(hipHostFree(c->pinned));
      c->pinned = nullptr;
      c->pinned_bytes = 0;
      PV_HIP(hipHostMalloc(&c->pinned, need, hipHostMallocDefault));
      c->pinned_bytes = need;
    }
    uint64_t* dkeys = reinterpret_cast<uint64_t*>(ws + keys_off);
    PV_HIP(pv::image_keys(images, src_hw, off.data(), n_images, dkeys, ws + acc_off, s));
    PV_HIP(hipMemcpyAsync(c->pinned, dkeys, need, hipMemcpyDeviceToHost, s));
    PV_HIP(hipStreamSynchronize(s));
    k = static_cast<const uint64_t*>(c->pinned);
  }

  // hits, first occurrences of misses, and repeats of a miss in this call
  std::vector<int32_t> src_of(n_images, -1);  // repeat: the earlier image it copies
  std::vector<int32_t> miss;
  std::map<pv_embcache::Key, int32_t> first_miss;
  std::vector<char> is_hit(n_images, 0);
  int64_t miss_rows = 0;
  for (int32_t i = 0; i < n_images; ++i) {
    const pv_embcache::Key key{k[2 * i], k[2 * i + 1]};
    if (c->entries.count(key)) {
      is_hit[i] = 1;
      continue;
    }
    auto fm = first_miss.find(key);
    if (fm != first_miss.end()) {
      src_of[i] = fm->second;
      continue;
    }
    first_miss.emplace(key, i);
    miss.push_back(i);
    miss_rows += rows[i];
  }
  if (miss_rows > c->capacity_rows)
    return fail(PV_ERR_CAPACITY, "the missed images need " + std::to_string(miss_rows) + " rows; the cache holds " +
                                     std::to_string(c->capacity_rows));

  // 1. copies of the hits (before anything can overwrite their rows)
  for (int32_t i = 0; i < n_images; ++i) {
    if (!is_hit[i] || rows[i] == 0) continue;
    const auto& e = c->entries.at({k[2 * i], k[2 * i + 1]});
    PV_HIP(hipMemcpyAsync(static_cast<char*>(out) + out_row0[i] * c->row_bytes, c->mem + e.row0 * c->row_bytes,
                          size_t(rows[i]) * c->row_bytes, hipMemcpyDeviceToDevice, s));
  }
  // 2. one forward of the misses into a contiguous run at the ring head
  std::vector<int64_t> slot(n_images, -1);
  if (!miss.empty()) {
    if (c->head + miss_rows > c->capacity_rows) c->head = 0;
    const int64_t run0 = c->head;
    evict_overlapping(c, run0, run0 + miss_rows);
    std::vector<int32_t> sub_hw;
    std::vector<uint64_t> sub_off;
    int64_t r = run0;
    for (int32_t i : miss) {
      sub_hw.push_back(src_hw[2 * i]);
      sub_hw.push_back(src_hw[2 * i + 1]);
      sub_off.push_back(off[i]);
      slot[i] = r;
      r += rows[i];
    }
    if (miss_rows > 0) {
      st = pv::forward_u8_at(c->tower, images, sub_hw.data(), sub_off.data(), int32_t(miss.size()),
                             c->has_ms ? c->mean_std : nullptr, c->mem + run0 * c->row_bytes, miss_rows,
                             ws + tower_off, ws_bytes - tower_off, s);
      if (st != PV_OK) return st;
    }
    for (int32_t i : miss) {
      const pv_embcache::Key key{k[2 * i], k[2 * i + 1]};
      c->entries[key] = {slot[i], rows[i]};
      c->by_row[slot[i]] = key;
      c->rows_used += rows[i];
    }
    c->head = run0 + miss_rows;
  }
  // 3. copies of the misses and of their repeats
  for (int32_t i = 0; i < n_images; ++i) {
    if (is_hit[i] || rows[i] == 0) continue;
    const int32_t from = src_of[i] >= 0 ? src_of[i] : i;
    PV_HIP(hipMemcpyAsync(static_cast<char*>(out) + out_row0[i] * c->row_bytes, c->mem + slot[from] * c->row_bytes,
                          size_t(rows[i]) * c->row_bytes, hipMemcpyDeviceToDevice, s));
  }
  for (int32_t i = 0; i < n_images; ++i) {
    const bool served = is_hit[i] || src_of[i] >= 0;
    if (hit) hit[i] = served ? 1 : 0;
    if (served) ++c->hits;
    else ++c->misses;
  }
  return PV_OK;
}

}  // extern "C"
