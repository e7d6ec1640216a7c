// Internal interface between the MLA prolog's C-ABI layer (prolog_host.cpp) and its kernels
// (prolog_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sfa {

constexpr int kPrLatent = 512;      // latent row (kv_lora_rank)
constexpr int kPrRope = 64;         // rotary channels
constexpr int kPrTokBlock = 128;    // tokens per workgroup (4 MFMA blocks of 32)
// 32-feature MFMA blocks per workgroup of each GEMM: the down-projections (64 features; with
// their k split, 33 tiles x 7 splits at hidden 7168), the query up-projection (96 features: 256
// tiles at 128 heads), the absorption (256 of a head's 512 channels: 256 tiles at 128 heads)
// and the V4 query up-projection (256 features: 256 tiles at 128 heads of 512 channels)
constexpr int kPrFb0 = 2, kPrFb1 = 3, kPrFb2 = 8, kPrFb3 = 8;
constexpr int prolog_feat_blocks(int mode) {
  return mode == 0 ? kPrFb0 : mode == 1 ? kPrFb1 : mode == 2 ? kPrFb2 : kPrFb3;
}

// One launch of the weight-streaming GEMM: out[t, f] = sum over k of W[f, k] * B[t, k] for the
// workgroup's features, tokens and k range; the epilogue depends on the mode.
struct PrologGemmArgs {
  const uint16_t* w0;        // bf16 (rows, k): features [0, f_split)
  const uint16_t* w1;        // bf16 (rows, k): features [f_split, n_feat), row f - f_split
  const uint16_t* b_hi;      // bf16 activations, token row stride b_stride elements
  const uint16_t* b_lo;      // low halves (hi + lo carries the fp32 value), or null
  int64_t b_stride;
  int32_t f_split, n_feat, k, tokens, n_split, k_chunk, tok_blocks;
  // modes 0 and 3: fp32 partial sums (n_split, tokens, n_feat)
  float* part;
  // mode 1: per-head nope part as hi/lo bf16 (tokens, n_q, dn); rotary part -> q_rope
  uint16_t* qn_hi;
  uint16_t* qn_lo;
  uint16_t* q_rope;          // bf16 (tokens * n_q, 64)
  // mode 2: absorbed query
  uint16_t* q_nope;          // bf16 (tokens * n_q, 512)
  const int32_t* positions;  // (tokens)
  const float* rope_cos;     // (rope_positions, 32)
  const float* rope_sin;
  int32_t rope_positions, n_q, dn;
};

// The per-token vector step after the down-projections: sums the partials, RMSNorm of the
// query part (hi/lo bf16 out) and of the latent row (bf16 out), RoPE of the rotary key.
struct PrologNormArgs {
  const float* part;         // (n_split, tokens, q_rank + 576)
  int32_t n_split, tokens, q_rank;
  const uint16_t* gamma_cq;  // bf16 (q_rank)
  const uint16_t* gamma_ckv; // bf16 (512)
  float eps;
  uint16_t* cq_hi;           // bf16 (tokens, q_rank)
  uint16_t* cq_lo;
  uint16_t* kv_nope;         // bf16 (tokens, 512)
  uint16_t* kv_rope;         // bf16 (tokens, 64)
  uint16_t* cq_out;          // bf16 (tokens, q_rank), or null: cq rounded to bf16
  const int32_t* positions;
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_positions;
  // V4 form: the latent row is 512 channels normalised whole (no separate rotary key), its last
  // 64 channels rotated in place; part then holds q_rank + 512 features per token
  int32_t kv_inside;
};

// The V4 query heads after their up-projection: RMSNorm with unit weight per head, RoPE in
// place on the head's last 64 channels.
struct PrologV4HeadArgs {
  const float* part;         // (n_split, tokens, n_feat), n_feat = n_q * 512
  int32_t n_split, tokens, n_q, n_feat;
  float eps;
  const int32_t* positions;
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_positions;
  uint16_t* q;               // bf16 (tokens * n_q, 512)
};

// The indexer prolog's per-token step: sums the split partials of the index query (n_heads x
// 128 per token) and of the key and weight projections (128 + n_heads), then LayerNorm of the
// key, RoPE on the second half of every 128-wide vector, the optional Hadamard transform, and
// the weights' scale.
struct IndexerFinishArgs {
  const float* part_q;       // (split_q, tokens, n_heads * 128)
  const float* part_kw;      // (split_kw, tokens, 128 + n_heads)
  int32_t split_q, split_kw, tokens, n_heads, rotate;
  const uint16_t* ln_gamma;  // bf16 (128)
  const uint16_t* ln_beta;   // bf16 (128)
  float eps, w_scale;
  const int32_t* positions;
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_positions;
  uint16_t* q_index;         // bf16 (tokens * n_heads, 128)
  uint16_t* k_index;         // bf16 (tokens, 128)
  float* weights;            // fp32 (tokens, n_heads)
};

hipError_t launch_prolog_gemm(const PrologGemmArgs& a, int mode, hipStream_t stream);
hipError_t launch_indexer_finish(const IndexerFinishArgs& a, hipStream_t stream);
hipError_t launch_prolog_norm(const PrologNormArgs& a, hipStream_t stream);
hipError_t launch_prolog_v4_head(const PrologV4HeadArgs& a, hipStream_t stream);

}  // namespace sfa
