// C-ABI entry point of the cache write in libsfa.so: synchronous argument validation and kernel
// launch. Declaration and contract are in include/sfa.h.

#include <stdint.h>

#include "cache_internal.h"
#include "sfa.h"

namespace {

using namespace sfa;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a0 = (uintptr_t)p, a1 = a0 + n, b0 = (uintptr_t)q, b1 = b0 + m;
  return a0 < b1 && b0 < a1;
}

// Only the fields the write uses are checked; n_q, n_kv, topk and num_splits are ignored.
// rope_dim 0: 512-wide rows with the rotary channels inside, no rope part.
int check_write_dims(const sfa_dims* d) {
  if (!d) return SFA_ERR_NULL;
  if (d->kv_lora_rank != SFA_KV_LORA_RANK || (d->rope_dim != SFA_ROPE_DIM && d->rope_dim != 0) ||
      d->block_size != SFA_BLOCK_SIZE)
    return SFA_ERR_DIMS;
  if (d->batch < 0 || d->s1 < 0 || (int64_t)d->batch * d->s1 > (1 << 26)) return SFA_ERR_DIMS;
  if (d->max_blocks_per_batch < 1 || d->max_blocks_per_batch > (1 << 23)) return SFA_ERR_DIMS;
  if (d->num_cache_rows < 0 || d->num_cache_rows > INT32_MAX) return SFA_ERR_DIMS;
  if (d->kv_dtype != SFA_KV_BF16 && d->kv_dtype != SFA_KV_INT8) return SFA_ERR_DIMS;
  return SFA_OK;
}

}  // namespace

extern "C" int sfa_cache_write(const sfa_dims* dims, const void* new_nope, const void* new_rope,
                               const int32_t* positions, const int32_t* block_table, void* key_nope_2d,
                               void* key_rope_2d, float* k_nope_scales, hipStream_t stream) {
  const int st = check_write_dims(dims);
  if (st != SFA_OK) return st;
  const bool int8 = dims->kv_dtype == SFA_KV_INT8;
  const bool rope = dims->rope_dim > 0;  // otherwise new_rope and key_rope_2d are not used
  if (!rope) new_rope = key_rope_2d = nullptr;
  if (!new_nope || (rope && !new_rope) || !positions || !block_table || !key_nope_2d || (rope && !key_rope_2d))
    return SFA_ERR_NULL;
  if (int8 && !k_nope_scales) return SFA_ERR_SCALES;
  if (!aligned16(new_nope) || !aligned16(new_rope) || !aligned16(positions) || !aligned16(block_table) ||
      !aligned16(key_nope_2d) || !aligned16(key_rope_2d) || (int8 && !aligned16(k_nope_scales)))
    return SFA_ERR_ALIGN;
  const int64_t tokens = (int64_t)dims->batch * dims->s1;
  const size_t rows = (size_t)dims->num_cache_rows;
  const void* ins[] = {new_nope, new_rope, positions, block_table};
  const size_t in_sizes[] = {(size_t)tokens * SFA_KV_LORA_RANK * 2, (size_t)tokens * dims->rope_dim * 2,
                             (size_t)tokens * 4, (size_t)dims->batch * dims->max_blocks_per_batch * 4};
  const void* outs[] = {key_nope_2d, key_rope_2d, int8 ? (const void*)k_nope_scales : nullptr};
  const size_t out_sizes[] = {rows * SFA_KV_LORA_RANK * (int8 ? 1 : 2), rows * dims->rope_dim * 2,
                              int8 ? rows * 4 * sizeof(float) : 0};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[o], out_sizes[o], ins[i], in_sizes[i])) return SFA_ERR_ALIAS;
    for (int p = o + 1; p < 3; ++p)
      if (overlaps(outs[o], out_sizes[o], outs[p], out_sizes[p])) return SFA_ERR_ALIAS;
  }
  if (tokens == 0 || rows == 0) return SFA_OK;
  CacheWriteArgs a{};
  a.new_nope = static_cast<const uint16_t*>(new_nope);
  a.new_rope = static_cast<const uint16_t*>(new_rope);
  a.positions = positions;
  a.block_table = block_table;
  a.key_nope = key_nope_2d;
  a.key_rope = static_cast<uint16_t*>(key_rope_2d);
  a.scales = k_nope_scales;
  a.num_rows = dims->num_cache_rows;
  a.n_tokens = (int32_t)tokens;
  a.s1 = dims->s1;
  a.mb = dims->max_blocks_per_batch;
  return launch_cache_write(a, int8, rope, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}
