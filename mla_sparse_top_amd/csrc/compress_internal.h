// Internal interface between the compressor's host layer (compress_host.cpp) and its kernel
// (compress_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sfa {


struct CompressArgs {
  const float* kv;              // (T, C), C = channels
  const float* score;           // (T, C)
  const float* ape;             // (ratio, C)
  const float* gamma;           // (C)
  const float* rope_cos;        // (rope_positions, 32)
  const float* rope_sin;        // (rope_positions, 32)
  const int32_t* start_pos;     // (batch)
  float* kv_state;              // (batch, ratio, C)
  float* score_state;           // (batch, ratio, C)
  const int32_t* block_table;   // (batch, mb)
  uint16_t* key_nope;           // bf16 bits (rows, 512) for C = 576 or 512, or (rows, 128) for C = 128
  uint16_t* key_rope;           // bf16 bits (rows, 64) for C = 576; unused otherwise
  int64_t num_rows;
  float eps;
  int32_t batch, s1, ratio, rope_positions, mb;
  int32_t channels;             // 576, 512 or 128
  int32_t rotate;               // 128 channels: the Hadamard transform after RoPE
};

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);

}  // namespace sfa
