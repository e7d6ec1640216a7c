// Internal interface between the compressor's host layer (compress_host.cpp) and its kernel
// (compress_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sfa {

constexpr int kCmpChannels = 576;            // 512 nope + 64 rope
constexpr int kCmpThreads = 192;             // three waves; thread i owns channels i, i+192, i+384
constexpr int kCmpPerThread = kCmpChannels / kCmpThreads;

struct CompressArgs {
  const float* kv;              // (T, 576)
  const float* score;           // (T, 576)
  const float* ape;             // (ratio, 576)
  const float* gamma;           // (576)
  const float* rope_cos;        // (rope_positions, 32)
  const float* rope_sin;        // (rope_positions, 32)
  const int32_t* start_pos;     // (batch)
  float* kv_state;              // (batch, ratio, 576)
  float* score_state;           // (batch, ratio, 576)
  const int32_t* block_table;   // (batch, mb)
  uint16_t* key_nope;           // bf16 bits (rows, 512)
  uint16_t* key_rope;           // bf16 bits (rows, 64)
  int64_t num_rows;
  float eps;
  int32_t batch, s1, ratio, rope_positions, mb;
};

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);

}  // namespace sfa
