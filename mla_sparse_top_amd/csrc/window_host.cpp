// C-ABI entry points of the sliding-window + compressed-cache attention variants in libsfa.so:
// synchronous validation, workspace layout, the pre-pass launch, then sfa_decode on the
// combined gather list. Declarations and contracts are in include/sfa.h.

#include <math.h>
#include <stdint.h>

#include "sfa.h"
#include "window_internal.h"

namespace {

using namespace sfa;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a0 = (uintptr_t)p, a1 = a0 + n, b0 = (uintptr_t)q, b1 = b0 + m;
  return a0 < b1 && b0 < a1;
}

int check_window_dims(const sfa_window_dims* d) {
  if (!d) return SFA_ERR_NULL;
  if (d->window < 0 || d->topk_cmp < 0 || d->window + (int64_t)d->topk_cmp < 1) return SFA_ERR_DIMS;
  if (d->max_blocks_ori < 1 || d->max_blocks_cmp < 0) return SFA_ERR_DIMS;
  if (d->topk_cmp > 0 && d->max_blocks_cmp < 1) return SFA_ERR_DIMS;
  if ((int64_t)d->max_blocks_ori + d->max_blocks_cmp > (1 << 23)) return SFA_ERR_DIMS;
  return SFA_OK;
}

// The sfa_dims of the sparse attention over the combined gather list.
sfa_dims combined_dims(const sfa_window_dims* d) {
  sfa_dims c{};
  c.batch = d->batch;
  c.s1 = d->s1;
  c.n_q = d->n_q;
  c.n_kv = d->n_kv;
  c.kv_lora_rank = d->kv_lora_rank;
  c.rope_dim = d->rope_dim;
  c.block_size = d->block_size;
  c.topk = d->window + d->topk_cmp;
  c.max_blocks_per_batch = d->max_blocks_ori + (d->topk_cmp > 0 ? d->max_blocks_cmp : 0);
  c.num_cache_rows = d->num_cache_rows;
  c.kv_dtype = d->kv_dtype;
  c.num_splits = d->num_splits;
  return c;
}

struct Layout {
  size_t idx, bt, act, attn, total, attn_bytes;
};

int layout(const sfa_window_dims* d, Layout* L) {
  const sfa_dims c = combined_dims(d);
  size_t attn = 0;
  const int st = sfa_workspace_size(&c, 0, &attn);
  if (st != SFA_OK) return st;
  const size_t tokens = (size_t)d->batch * d->s1;
  L->idx = 0;
  L->bt = align_up(L->idx + tokens * (size_t)c.topk * 4);
  L->act = align_up(L->bt + (size_t)d->batch * c.max_blocks_per_batch * 4);
  L->attn = align_up(L->act + (size_t)d->batch * 4);
  L->attn_bytes = attn;
  L->total = L->attn + attn;
  return SFA_OK;
}

}  // namespace

extern "C" {

int sfa_window_workspace_size(const sfa_window_dims* dims, size_t* bytes_out) {
  const int st = check_window_dims(dims);
  if (st != SFA_OK) return st;
  if (!bytes_out) return SFA_ERR_NULL;
  Layout L{};
  const int s = layout(dims, &L);
  if (s != SFA_OK) return s;
  *bytes_out = L.total;
  return SFA_OK;
}

int sfa_window_decode(const sfa_window_dims* dims, const void* query_nope, const void* query_rope,
                      const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
                      const int32_t* cmp_indices, const int32_t* block_table_ori, const int32_t* block_table_cmp,
                      const int32_t* ori_len, const int32_t* cmp_len, float softmax_scale, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  const int st = check_window_dims(dims);
  if (st != SFA_OK) return st;
  Layout L{};
  const int ls = layout(dims, &L);  // also validates the shared attention dims
  if (ls != SFA_OK) return ls;
  // Everything sfa_decode checks is checked here too, before the pre-pass is queued, so that a
  // failing call queues nothing.
  const bool cmp = dims->topk_cmp > 0;
  const bool int8 = dims->kv_dtype == SFA_KV_INT8;
  if (!query_nope || !query_rope || !key_nope_2d || !key_rope_2d || !out || !block_table_ori || !ori_len)
    return SFA_ERR_NULL;
  if (cmp && (!cmp_indices || !block_table_cmp || !cmp_len)) return SFA_ERR_NULL;
  if (int8 && !k_nope_scales) return SFA_ERR_SCALES;
  if (!aligned16(query_nope) || !aligned16(query_rope) || !aligned16(key_nope_2d) || !aligned16(key_rope_2d) ||
      !aligned16(out) || (int8 && !aligned16(k_nope_scales)) || !aligned16(block_table_ori) || !aligned16(ori_len) ||
      (cmp && (!aligned16(cmp_indices) || !aligned16(block_table_cmp) || !aligned16(cmp_len))))
    return SFA_ERR_ALIGN;
  if (!isfinite(softmax_scale)) return SFA_ERR_SCALE_VALUE;
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace % kAlign) != 0) return SFA_ERR_WORKSPACE;
  const int64_t tokens = (int64_t)dims->batch * dims->s1;
  {
    const size_t rows = (size_t)dims->num_cache_rows;
    const size_t out_bytes = (size_t)tokens * dims->n_q * SFA_KV_LORA_RANK * 2;
    const void* ins[] = {query_nope, query_rope, key_nope_2d, key_rope_2d, int8 ? k_nope_scales : nullptr,
                         cmp ? cmp_indices : nullptr, block_table_ori, cmp ? block_table_cmp : nullptr, ori_len,
                         cmp ? cmp_len : nullptr, workspace};
    const size_t sizes[] = {(size_t)tokens * dims->n_q * SFA_KV_LORA_RANK * 2,
                            (size_t)tokens * dims->n_q * SFA_ROPE_DIM * 2,
                            rows * SFA_KV_LORA_RANK * (int8 ? 1 : 2),
                            rows * SFA_ROPE_DIM * 2,
                            int8 ? rows * 4 * sizeof(float) : 0,
                            (size_t)tokens * dims->topk_cmp * 4,
                            (size_t)dims->batch * dims->max_blocks_ori * 4,
                            (size_t)dims->batch * dims->max_blocks_cmp * 4,
                            (size_t)dims->batch * 4,
                            (size_t)dims->batch * 4,
                            L.total};
    for (int i = 0; i < 11; ++i)
      if (overlaps(out, out_bytes, ins[i], sizes[i])) return SFA_ERR_ALIAS;
  }
  if (tokens == 0) return SFA_OK;
  char* ws = static_cast<char*>(workspace);
  WindowPrepArgs a{};
  a.cmp_indices = cmp ? cmp_indices : nullptr;
  a.bt_ori = block_table_ori;
  a.bt_cmp = cmp ? block_table_cmp : nullptr;
  a.ori_len = ori_len;
  a.cmp_len = cmp ? cmp_len : nullptr;
  a.idx = reinterpret_cast<int32_t*>(ws + L.idx);
  a.bt = reinterpret_cast<int32_t*>(ws + L.bt);
  a.act = reinterpret_cast<int32_t*>(ws + L.act);
  a.batch = dims->batch;
  a.s1 = dims->s1;
  a.window = dims->window;
  a.topk_cmp = dims->topk_cmp;
  a.mb_ori = dims->max_blocks_ori;
  a.mb_cmp = cmp ? dims->max_blocks_cmp : 0;
  if (launch_window_prep(a, stream) != hipSuccess) return SFA_ERR_HIP;
  const sfa_dims c = combined_dims(dims);
  return sfa_decode(&c, query_nope, query_rope, key_nope_2d, key_rope_2d, k_nope_scales, a.idx, a.bt, a.act,
                    softmax_scale, out, L.attn_bytes ? ws + L.attn : nullptr, L.attn_bytes, stream);
}

}  // extern "C"
