// C-ABI entry point of the compressor in libsfa.so: synchronous argument validation and kernel
// launch. Declaration and contract are in include/sfa.h.

#include <math.h>
#include <stdint.h>

#include "compress_internal.h"
#include "sfa.h"

namespace {

using namespace sfa;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a0 = (uintptr_t)p, a1 = a0 + n, b0 = (uintptr_t)q, b1 = b0 + m;
  return a0 < b1 && b0 < a1;
}

int check_compress_dims(const sfa_compress_dims* d, float eps) {
  if (!d) return SFA_ERR_NULL;
  const bool cache_row = d->channels == SFA_KV_LORA_RANK + SFA_ROPE_DIM;
  if ((!cache_row && d->channels != SFA_KV_LORA_RANK && d->channels != 128) || d->block_size != SFA_BLOCK_SIZE)
    return SFA_ERR_DIMS;
  if (d->rotate != 0 && (d->rotate != 1 || d->channels != 128)) return SFA_ERR_DIMS;  // Hadamard: 128 channels
  if (d->batch < 0 || d->s1 < 0 || (int64_t)d->batch * d->s1 > (1 << 26)) return SFA_ERR_DIMS;
  if (d->batch > (1 << 20)) return SFA_ERR_DIMS;
  if (d->ratio < 1 || d->ratio > 1024) return SFA_ERR_DIMS;
  if (d->rope_positions < 0) return SFA_ERR_DIMS;
  if (d->max_blocks < 1 || d->max_blocks > (1 << 23)) return SFA_ERR_DIMS;
  if (d->num_cache_rows < 0 || d->num_cache_rows > INT32_MAX) return SFA_ERR_DIMS;
  if (!(eps >= 0.0f) || !isfinite(eps)) return SFA_ERR_DIMS;
  return SFA_OK;
}

}  // namespace

extern "C" int sfa_compress(const sfa_compress_dims* dims, const float* kv, const float* score, const float* ape,
                            const float* gamma, float eps, const float* rope_cos, const float* rope_sin,
                            const int32_t* start_pos, float* kv_state, float* score_state,
                            const int32_t* block_table_cmp, void* key_nope_2d, void* key_rope_2d,
                            hipStream_t stream) {
  const int st = check_compress_dims(dims, eps);
  if (st != SFA_OK) return st;
  if ((int64_t)dims->batch * dims->s1 == 0) return SFA_OK;  // no token: nothing is read or written
  const bool cache_row = dims->channels == SFA_KV_LORA_RANK + SFA_ROPE_DIM;
  if (!kv || !score || !ape || !gamma || !rope_cos || !rope_sin || !start_pos || !kv_state || !score_state ||
      !block_table_cmp || !key_nope_2d || (cache_row && !key_rope_2d))
    return SFA_ERR_NULL;
  if (!cache_row) key_rope_2d = nullptr;  // a 512- or 128-channel row goes whole to key_nope_2d
  const void* ins[] = {kv, score, ape, gamma, rope_cos, rope_sin, start_pos, block_table_cmp};
  void* outs[] = {kv_state, score_state, key_nope_2d, key_rope_2d};
  for (const void* p : ins)
    if (!aligned16(p)) return SFA_ERR_ALIGN;
  for (const void* p : outs)
    if (p && !aligned16(p)) return SFA_ERR_ALIGN;
  const size_t C = (size_t)dims->channels;
  const size_t tokens = (size_t)dims->batch * dims->s1;
  const size_t rows = (size_t)dims->num_cache_rows;
  const size_t state = (size_t)dims->batch * dims->ratio * C * 4;
  const size_t in_sizes[] = {tokens * C * 4, tokens * C * 4, (size_t)dims->ratio * C * 4, C * 4,
                             (size_t)dims->rope_positions * 32 * 4, (size_t)dims->rope_positions * 32 * 4,
                             (size_t)dims->batch * 4, (size_t)dims->batch * dims->max_blocks * 4};
  const size_t out_sizes[] = {state, state, rows * (cache_row ? SFA_KV_LORA_RANK : C) * 2,
                              cache_row ? rows * SFA_ROPE_DIM * 2 : 0};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlaps(outs[o], out_sizes[o], ins[i], in_sizes[i])) return SFA_ERR_ALIAS;
    for (int q = o + 1; q < 4; ++q)
      if (overlaps(outs[o], out_sizes[o], outs[q], out_sizes[q])) return SFA_ERR_ALIAS;
  }
  CompressArgs a{};
  a.kv = kv;
  a.score = score;
  a.ape = ape;
  a.gamma = gamma;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.start_pos = start_pos;
  a.kv_state = kv_state;
  a.score_state = score_state;
  a.block_table = block_table_cmp;
  a.key_nope = static_cast<uint16_t*>(key_nope_2d);
  a.key_rope = static_cast<uint16_t*>(key_rope_2d);
  a.num_rows = dims->num_cache_rows;
  a.eps = eps;
  a.batch = dims->batch;
  a.s1 = dims->s1;
  a.ratio = dims->ratio;
  a.rope_positions = dims->rope_positions;
  a.mb = dims->max_blocks;
  a.channels = dims->channels;
  a.rotate = dims->rotate;
  return launch_compress(a, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}
