// Pre-pass of the sliding-window + compressed-cache attention variants (SWA, CFA, SCFA of "NPU
// DeepSeek-V4 model PyPTO fused-operator optimisation", section "FA-class operators"): it turns
// the two row sources of a query token into one gather list over one combined block table, so
// that the sparse attention kernel runs on them unchanged.
//
// The combined logical space of batch b puts the original cache first and the compressed cache
// after it: logical block i < mb_ori is block_table_ori[b][i], block mb_ori + i is
// block_table_cmp[b][i]. A query at position p = ori_len[b] - s1 + s lists its window positions
// max(0, p - window + 1) .. p as themselves, and compressed entry c as mb_ori * 128 + c. The
// combined live length is mb_ori * 128 + cmp_len[b]: every window position lies below
// mb_ori * 128, and a compressed entry is live iff c < cmp_len[b], the sparse kernel's own
// validity rule. Work is one thread per list slot and one per table entry; it is a few hundred
// KB of int32 writes, bound by launch latency.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "window_internal.h"

namespace sfa {
namespace {

constexpr int kPrepThreads = 256;

__global__ void __launch_bounds__(kPrepThreads) window_prep_kernel(const WindowPrepArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x;
  const int k_all = a.window + a.topk_cmp;
  const int64_t n_slots = (int64_t)a.batch * a.s1 * k_all;
  const int mb = a.mb_ori + a.mb_cmp;
  const int64_t ori_span = (int64_t)a.mb_ori * 128;
  if (tid < n_slots) {
    const int t = (int)(tid / k_all);
    const int k = (int)(tid - (int64_t)t * k_all);
    const int b = t / a.s1;
    int out = -1;
    if (k < a.window) {
      const int p = a.ori_len[b] - a.s1 + t % a.s1;  // the query's position
      const int j = p - a.window + 1 + k;
      if (j >= 0 && j <= p && j < ori_span) out = j;
    } else {
      const int c = a.cmp_indices[(int64_t)t * a.topk_cmp + (k - a.window)];
      if (c >= 0 && c < a.cmp_len[b] && c < (int64_t)a.mb_cmp * 128) out = (int)(ori_span + c);
    }
    a.idx[tid] = out;
  }
  const int64_t n_bt = (int64_t)a.batch * mb;
  if (tid < n_bt) {
    const int b = (int)(tid / mb);
    const int i = (int)(tid - (int64_t)b * mb);
    a.bt[tid] = i < a.mb_ori ? a.bt_ori[(int64_t)b * a.mb_ori + i] : a.bt_cmp[(int64_t)b * a.mb_cmp + (i - a.mb_ori)];
  }
  if (tid < a.batch) {
    const int cl = a.topk_cmp > 0 ? a.cmp_len[tid] : 0;
    const int64_t cap = (int64_t)a.mb_cmp * 128;
    a.act[tid] = (int)(ori_span + (cl < 0 ? 0 : (cl < cap ? cl : cap)));
  }
}

}  // namespace

hipError_t launch_window_prep(const WindowPrepArgs& a, hipStream_t stream) {
  const int64_t n_slots = (int64_t)a.batch * a.s1 * (a.window + a.topk_cmp);
  const int64_t n_bt = (int64_t)a.batch * (a.mb_ori + a.mb_cmp);
  int64_t n = n_slots > n_bt ? n_slots : n_bt;
  if (n < a.batch) n = a.batch;
  const int grid = (int)((n + kPrepThreads - 1) / kPrepThreads);
  hipLaunchKernelGGL(window_prep_kernel, dim3(grid), dim3(kPrepThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfa
