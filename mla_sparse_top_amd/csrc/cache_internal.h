// Internal interface between the cache-write host layer (cache_host.cpp) and its kernel
// (cache_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sfa {

constexpr int kCwWaves = 4;         // waves per workgroup
constexpr int kCwRowsPerWave = 4;   // new tokens one wave writes (their loads are issued together)
constexpr int kCwTokensPerWg = kCwWaves * kCwRowsPerWave;

struct CacheWriteArgs {
  const uint16_t* new_nope;     // bf16 bits (T, 512)
  const uint16_t* new_rope;     // bf16 bits (T, 64); unused for 512-wide rows
  const int32_t* positions;     // (T) logical position of each new token in its batch
  const int32_t* block_table;   // (batch, mb)
  void* key_nope;               // bf16 bits or int8 (rows, 512)
  uint16_t* key_rope;           // bf16 bits (rows, 64); unused for 512-wide rows
  float* scales;                // (rows, 4) for an INT8 cache
  int64_t num_rows;
  int32_t n_tokens, s1, mb;
};

hipError_t launch_cache_write(const CacheWriteArgs& a, bool int8_cache, bool rope, hipStream_t stream);

}  // namespace sfa
