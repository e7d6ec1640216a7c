// Internal interface between the Lightning Indexer host layer (indexer_host.cpp) and its kernels
// (indexer_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sfa {

constexpr int kIdxHeads = 64;      // index heads
constexpr int kIdxDim = 128;       // index head dim
constexpr int kIdxBlock = 128;     // cache rows per page (shared with the latent cache)
constexpr int kIdxTokenChunk = 8;  // query tokens of one batch per score workgroup

struct IndexerArgs {
  const uint16_t* q;            // bf16 bits (T*64, 128), row t*64 + h
  const uint16_t* k;            // bf16 bits (rows, 128)
  const float* w;               // (T, 64)
  const int32_t* block_table;   // (batch, mb)
  const int32_t* act;           // (batch)
  float* scores;                // (T, mb*128)
  int32_t* topk_out;            // (T, topk)
  int64_t num_rows;
  int32_t batch, s1, mb, n_pos, chunks, topk;
};

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t stream);
hipError_t launch_topk_select(const IndexerArgs& a, hipStream_t stream);

}  // namespace sfa
