// Internal interface between the C-ABI host layer (sfa_host.cpp) and the kernels
// (sfa_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sfa {

constexpr int kNope = 512;          // kv_lora_rank
constexpr int kRope = 64;           // qk_rope_dim
constexpr int kBlock = 128;         // rows per cache page
constexpr int kTile = 32;           // top-k slots per inner tile
constexpr int kWaves = 4;           // waves per workgroup, one per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWave = 32;   // each wave owns 32 heads over the whole 576-wide d
constexpr int kMaxHeads = kWaves * kHeadsPerWave;  // one workgroup covers every head of a token
constexpr int kMaxSlots = 2048;     // slots one workgroup compacts (topk partition size cap)
constexpr int kMaxSplits = 16;      // top-k partitions per token
constexpr int kMaxTopk = kMaxSlots * kMaxSplits;
// Partial output of one (token, partition): the register image of the O^T accumulators,
// 4 waves x 16 blocks of 32 columns x 4 row quads x 64 lanes x float4 (256 KB)
constexpr size_t kPartialBytes = (size_t)kWaves * 16 * 4 * 64 * 16;
constexpr size_t kPartialMlBytes = kMaxHeads * 2 * sizeof(float);
// The spread merge: up to this many partitions share a token's merge, one output unit (a wave's
// heads x 128 columns) each at most.
constexpr int kMaxSpread = kWaves * 4;
// 64-bit counter words per token in the workspace, each tagged with the call's generation:
// partitions arrived, partials counted ready, the spread merge's published flags (partition x
// wave) and the merging partition's decision for each output unit (wave x 128-column block)
constexpr int kCntArrive = 0, kCntReady = 1, kCntPublished = 2, kCntDecision = 2 + kMaxSpread * kWaves;
constexpr int kCounterWords = kCntDecision + kWaves * 4;

struct KernelArgs {
  const uint16_t* q_nope;     // bf16 bits (T*n_q, 512)
  const uint16_t* q_rope;     // bf16 bits (T*n_q, 64)
  const void* k_nope;         // bf16 bits or int8 (rows, 512)
  const uint16_t* k_rope;     // bf16 bits (rows, 64)
  const float* k_scales;      // (rows, 4) for int8
  const int32_t* topk_idx;    // (T, topk)
  const int32_t* block_table; // (batch, mb)
  const int32_t* act;         // (batch)
  uint16_t* out;              // bf16 bits (T, n_q, 512)
  float* part_o;              // (T, splits) x kPartialBytes
  float* part_ml;             // (T, splits, 128, 2): running max and sum per head
  uint64_t* counters;         // (T, kCounterWords), tagged with the call's generation
  uint64_t gen;               // this call's generation: 48 bits, never 0
  // 2 to 16 partitions whose workgroups are all resident: the spread merge, with an early
  // arrival's wait for the others bounded by this many wall-clock ticks; 0: the last arrival
  // merges everything.
  int64_t merge_wait_ticks;
  int64_t num_rows;
  int32_t n_tokens, s1, n_q, topk, mb, n_splits, chunk, reverse;
  // 1, or 2 when a token's heads are split over two workgroups of 64 heads (one partition only)
  int32_t head_groups;
  float scale_log2;           // softmax_scale * log2(e)
  // Window variants (the kernel instantiated with its window flag): slot g < window of token
  // t = b*s1 + s is original-cache position act[b] - s1 + s - window + 1 + g, through
  // block_table / act / mb; slot g >= window is compressed entry topk_idx[t][g - window] (row
  // length topk - window), live iff below act_cmp[b], through block_table_cmp / mb_cmp.
  const int32_t* block_table_cmp;
  const int32_t* act_cmp;
  int32_t mb_cmp, window;
};

struct ResolveArgs {
  const int32_t* topk_idx;
  const int32_t* block_table;
  const int32_t* act;
  int32_t* rows_out;
  int64_t num_rows;
  int32_t n_tokens, s1, topk, mb;
};

hipError_t launch_attention(const KernelArgs& a, bool int8_cache, bool window_slots, bool rope, hipStream_t stream);
hipError_t launch_resolve(const ResolveArgs& a, hipStream_t stream);

}  // namespace sfa
