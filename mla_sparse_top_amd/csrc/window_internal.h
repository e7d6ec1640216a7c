// Internal interface between the window-variant host layer (window_host.cpp) and its pre-pass
// kernel (window_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sfa {

struct WindowPrepArgs {
  const int32_t* cmp_indices;  // (T, topk_cmp) or null when topk_cmp == 0
  const int32_t* bt_ori;       // (batch, mb_ori)
  const int32_t* bt_cmp;       // (batch, mb_cmp) or null when mb_cmp == 0
  const int32_t* ori_len;      // (batch)
  const int32_t* cmp_len;      // (batch) or null when topk_cmp == 0
  int32_t* idx;                // out: (T, window + topk_cmp) logical positions, -1 masked
  int32_t* bt;                 // out: (batch, mb_ori + mb_cmp)
  int32_t* act;                // out: (batch)
  int32_t batch, s1, window, topk_cmp, mb_ori, mb_cmp;
};

hipError_t launch_window_prep(const WindowPrepArgs& a, hipStream_t stream);

}  // namespace sfa
