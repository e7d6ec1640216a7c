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
constexpr int kIdxTokenChunk = 4;  // query tokens of one batch per score workgroup (16 KB of LDS each)
constexpr int kIdxMaxPagesPerWg = 4;  // upper bound of IndexerArgs::pages_per_wg
constexpr int kIdxSelCache = 32768;  // positions per token whose keys the selection holds in LDS

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
  int32_t pages_per_wg;         // pages of one batch each score workgroup runs
};

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t stream);
hipError_t launch_topk_select(const IndexerArgs& a, hipStream_t stream);

}  // namespace sfa
