// Masked scatter of merged image embeddings into a text-embedding sequence
// ("Mistral 3" (KerasFormers) model page, Mistral3Model argument table:
// image_token_id, the placeholder the processor expands per image; "Several
// images in one conversation"): the k-th placeholder position of the
// sequence takes row k of the image embeddings.  Two memory-bound passes:
//   scan: one workgroup compacts the placeholder positions (in sequence
//         order) into a list and counts them;
//   copy: one workgroup per image row moves the row (16-byte accesses).
#include <mutex>
#include <string>

#include "api.h"
#include "common.h"
#include "kernels.h"

namespace pv {

namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scatter_scan_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                    int32_t token, int32_t* __restrict__ pos,
                                                                    int32_t* __restrict__ count) {
  __shared__ int32_t part[kScanThreads];
  const int t = threadIdx.x;
  const int64_t chunk = (n + kScanThreads - 1) / kScanThreads;
  const int64_t lo = t * chunk, hi = lo + chunk < n ? lo + chunk : n;
  int32_t c = 0;
  for (int64_t p = lo; p < hi; ++p) c += ids[p] == token;
  part[t] = c;
  __syncthreads();
  // inclusive scan of the per-thread counts (Hillis-Steele over LDS)
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t k = part[t] - c;  // exclusive prefix: first list slot of this chunk
  for (int64_t p = lo; p < hi; ++p)
    if (ids[p] == token) pos[k++] = int32_t(p);
  if (t == kScanThreads - 1) count[0] = part[t];
}

__global__ __launch_bounds__(256) void scatter_copy_kernel(const int32_t* __restrict__ pos,
                                                           const int32_t* __restrict__ count,
                                                           const u32x4* __restrict__ src, int64_t rows,
                                                           u32x4* __restrict__ dst, int chunks,
                                                           int32_t* __restrict__ status) {
  const int64_t k = blockIdx.x;
  const int32_t cnt = count[0];
  if (k == 0 && threadIdx.x == 0) status[0] = int64_t(cnt) == rows ? 0 : 1;
  if (k >= rows || k >= cnt) return;
  const u32x4* s = src + k * chunks;
  u32x4* d = dst + int64_t(pos[k]) * chunks;
  for (int c = threadIdx.x; c < chunks; c += 256) d[c] = s[c];
}

}  // namespace

size_t scatter_workspace_bytes(int64_t seq_len) {
  const size_t list = (size_t(seq_len > 0 ? seq_len : 0) * 4 + 255) / 256 * 256;
  return list + 256;  // + the count
}

hipError_t scatter_rows(const int32_t* ids, int64_t n, int32_t token, const void* src, int64_t rows, void* dst,
                        int64_t row_bytes, int32_t* status, void* ws, hipStream_t s) {
  int32_t* pos = static_cast<int32_t*>(ws);
  int32_t* count = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + scatter_workspace_bytes(n) - 256);
  hipLaunchKernelGGL(scatter_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, ids, n, token, pos, count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = rows > 0 ? rows : 1;
  hipLaunchKernelGGL(scatter_copy_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, pos, count,
                     static_cast<const u32x4*>(src), rows, static_cast<u32x4*>(dst), int(row_bytes / 16), status);
  return hipGetLastError();
}

// ---- allocation-free variant: the scratch (position list + count) lives in
// a file-scope device array of a fixed size instead of a caller workspace.
namespace {

// longest token sequence the allocation-free scatter takes
constexpr int64_t kScratchMaxSeq = int64_t(1) << 20;
// scatter_workspace_bytes(kScratchMaxSeq) bytes: the list of up to
// kScratchMaxSeq positions, then 256 bytes holding the count
constexpr size_t kScratchBytes = (size_t(kScratchMaxSeq) * 4 + 255) / 256 * 256 + 256;
static __device__ __align__(256) int32_t scratch[kScratchBytes / 4];

// Device address of `scratch` per device: the host-side name is only a
// stand-in, so it is looked up once per device (with that device current)
// and the address is passed to the kernels.
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

pv_status scratch_of_current_device(void** out) {
  int dev = 0;
  PV_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(PV_ERR_HIP, "device index " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    PV_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(PV_ERR_HIP, "no device address for the scatter scratch");
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PV_OK;
}

}  // namespace

}  // namespace pv

extern "C" pv_status pv_scatter_image_embeddings_noalloc(const int32_t* token_ids, int64_t seq_len,
                                                         int32_t image_token_id, const void* image_emb,
                                                         int64_t n_image_rows, void* text_emb, int32_t dim,
                                                         int32_t elem_bytes, int32_t* status, void* stream) {
  pv::last_error().clear();
  pv_status st = pv::scatter_check(token_ids, seq_len, image_emb, n_image_rows, text_emb, dim, elem_bytes, status);
  if (st != PV_OK) return st;
  if (seq_len > pv::kScratchMaxSeq)
    return pv::fail(PV_ERR_CAPACITY, "seq_len " + std::to_string(seq_len) + " exceeds the allocation-free scatter's "
                                     "maximum of " + std::to_string(pv::kScratchMaxSeq) + " positions");
  void* ws = nullptr;
  if ((st = pv::scratch_of_current_device(&ws)) != PV_OK) return st;
  PV_HIP(pv::scatter_rows(token_ids, seq_len, image_token_id, image_emb, n_image_rows, text_emb,
                          int64_t(dim) * elem_bytes, status, ws, static_cast<hipStream_t>(stream)));
  return PV_OK;
}
