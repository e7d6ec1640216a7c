// C-ABI entry points of the Lightning Indexer in libsfa.so: synchronous argument validation and
// kernel launch. Declarations and contracts are in include/sfa.h.

#include <stdint.h>

#include "indexer_internal.h"
#include "sfa.h"

namespace {

using namespace sfa;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a0 = (uintptr_t)p, a1 = a0 + n, b0 = (uintptr_t)q, b1 = b0 + m;
  return a0 < b1 && b0 < a1;
}

int check_dims(const sfa_indexer_dims* d) {
  if (!d) return SFA_ERR_NULL;
  if (d->batch < 0 || d->s1 < 0 || (int64_t)d->batch * d->s1 > INT32_MAX / 64) return SFA_ERR_DIMS;
  if (d->n_heads != kIdxHeads || d->head_dim != kIdxDim || d->block_size != kIdxBlock) return SFA_ERR_DIMS;
  if (d->max_blocks_per_batch < 1 || (int64_t)d->max_blocks_per_batch * kIdxBlock > (1 << 24)) return SFA_ERR_DIMS;
  if (d->num_cache_rows < 0 || d->num_cache_rows > ((int64_t)1 << 40)) return SFA_ERR_DIMS;
  if (d->topk < 1 || d->topk > (1 << 24)) return SFA_ERR_DIMS;
  return SFA_OK;
}

IndexerArgs base_args(const sfa_indexer_dims* d) {
  IndexerArgs a{};
  a.num_rows = d->num_cache_rows;
  a.batch = d->batch;
  a.s1 = d->s1;
  a.mb = d->max_blocks_per_batch;
  a.n_pos = d->max_blocks_per_batch * kIdxBlock;
  a.chunks = (d->s1 + kIdxTokenChunk - 1) / kIdxTokenChunk;
  a.topk = d->topk;
  // about four workgroups per CU over the whole grid, each running a few pages so that its
  // staged queries serve several pages of keys
  const int64_t pages = (int64_t)a.batch * a.chunks * a.mb;
  a.pages_per_wg = (int)(pages / 1024 < 1 ? 1 : (pages / 1024 > kIdxMaxPagesPerWg ? kIdxMaxPagesPerWg : pages / 1024));
  return a;
}

}  // namespace

extern "C" {

int sfa_indexer_scores(const sfa_indexer_dims* dims, const void* q_index, const void* k_index_cache,
                       const float* weights, const int32_t* block_table, const int32_t* kv_act_seqs,
                       float* scores, hipStream_t stream) {
  const int st = check_dims(dims);
  if (st != SFA_OK) return st;
  if (!q_index || !k_index_cache || !weights || !block_table || !kv_act_seqs || !scores) return SFA_ERR_NULL;
  if (!aligned16(q_index) || !aligned16(k_index_cache) || !aligned16(weights) || !aligned16(block_table) ||
      !aligned16(kv_act_seqs) || !aligned16(scores))
    return SFA_ERR_ALIGN;
  const int64_t tokens = (int64_t)dims->batch * dims->s1;
  const size_t score_bytes = (size_t)tokens * dims->max_blocks_per_batch * kIdxBlock * sizeof(float);
  const void* ins[] = {q_index, k_index_cache, weights, block_table, kv_act_seqs};
  const size_t sizes[] = {(size_t)tokens * kIdxHeads * kIdxDim * 2, (size_t)dims->num_cache_rows * kIdxDim * 2,
                          (size_t)tokens * kIdxHeads * sizeof(float),
                          (size_t)dims->batch * dims->max_blocks_per_batch * sizeof(int32_t),
                          (size_t)dims->batch * sizeof(int32_t)};
  for (int i = 0; i < 5; ++i)
    if (overlaps(scores, score_bytes, ins[i], sizes[i])) return SFA_ERR_ALIAS;
  if (tokens == 0) return SFA_OK;
  IndexerArgs a = base_args(dims);
  a.q = static_cast<const uint16_t*>(q_index);
  a.k = static_cast<const uint16_t*>(k_index_cache);
  a.w = weights;
  a.block_table = block_table;
  a.act = kv_act_seqs;
  a.scores = scores;
  return launch_indexer_scores(a, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

int sfa_topk_select(const sfa_indexer_dims* dims, const float* scores, const int32_t* kv_act_seqs,
                    int32_t* topk_indices, hipStream_t stream) {
  const int st = check_dims(dims);
  if (st != SFA_OK) return st;
  if (!scores || !kv_act_seqs || !topk_indices) return SFA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(kv_act_seqs) || !aligned16(topk_indices)) return SFA_ERR_ALIGN;
  const int64_t tokens = (int64_t)dims->batch * dims->s1;
  const size_t out_bytes = (size_t)tokens * dims->topk * sizeof(int32_t);
  if (overlaps(topk_indices, out_bytes, scores, (size_t)tokens * dims->max_blocks_per_batch * kIdxBlock * 4) ||
      overlaps(topk_indices, out_bytes, kv_act_seqs, (size_t)dims->batch * 4))
    return SFA_ERR_ALIAS;
  if (tokens == 0) return SFA_OK;
  IndexerArgs a = base_args(dims);
  a.scores = const_cast<float*>(scores);
  a.act = kv_act_seqs;
  a.topk_out = topk_indices;
  return launch_topk_select(a, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

}  // extern "C"
