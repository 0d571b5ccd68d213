// Internal glue between the C ABI translation units (tower.cpp,
// embcache.cpp): the thread-local error message and the tower entry points
// the embeddings cache drives.  Host C++ only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pv_tower.h"

namespace pv {

// Thread-local message returned by pv_last_error().
std::string& last_error();

inline pv_status fail(pv_status s, const std::string& msg) {
  last_error() = msg;
  return s;
}

#define PV_HIP(call)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return ::pv::fail(PV_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_));     \
  } while (0)

// Output rows of each uint8 source image under the tower's resize rule, the
// output row size in bytes, and the workspace a forward of all of them needs.
pv_status u8_out_rows(const pv_tower* t, const int32_t* src_hw, int32_t n, std::vector<int64_t>* rows,
                      int64_t* row_bytes, int64_t* ws_bytes);

// pv_tower_forward_u8 over images whose bytes start at explicit offsets
// (offsets[i] bytes from `images`) instead of back to back.
pv_status forward_u8_at(pv_tower* t, const uint8_t* images, const int32_t* src_hw, const uint64_t* offsets,
                        int32_t n, const float* mean_std, void* out, int64_t out_rows_cap, void* workspace,
                        size_t ws_bytes, hipStream_t s);

// Argument checks of the masked scatter shared by its entry points (null,
// range, element size, row size, alignment): PV_OK or PV_ERR_ARG.
pv_status scatter_check(const int32_t* token_ids, int64_t seq_len, const void* image_emb, int64_t n_image_rows,
                        const void* text_emb, int32_t dim, int32_t elem_bytes, const int32_t* status);

}  // namespace pv
