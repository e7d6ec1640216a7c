// C-ABI entry points of the MLA prolog (sfa_mla_prolog_workspace_size, sfa_mla_prolog) and of
// the indexer prolog (sfa_indexer_prolog_workspace_size, sfa_indexer_prolog): synchronous
// argument validation, the k splits of the projections, workspace layouts, and the launches.
// Declarations and contracts are in include/sfa.h.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "prolog_internal.h"
#include "sfa.h"

namespace {

using namespace sfa;

constexpr size_t kAlign = 256;
constexpr int kTargetWorkgroups = 256;  // one per compute unit of the MI355X

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a0 = (uintptr_t)p, a1 = a0 + n, b0 = (uintptr_t)q, b1 = b0 + m;
  return a0 < b1 && b0 < a1;
}

int check(const sfa_prolog_dims* d) {
  if (!d) return SFA_ERR_NULL;
  if (d->tokens < 0 || d->tokens > (1 << 20)) return SFA_ERR_DIMS;
  // the GEMMs walk k in chunks of 64
  if (d->hidden < 64 || d->hidden > (1 << 16) || d->hidden % 64) return SFA_ERR_DIMS;
  if (d->q_lora_rank < 64 || d->q_lora_rank > 4096 || d->q_lora_rank % 64) return SFA_ERR_DIMS;
  if (d->n_q < 1 || d->n_q > SFA_MAX_HEADS) return SFA_ERR_DIMS;
  if (d->qk_nope_dim < 64 || d->qk_nope_dim > 512 || d->qk_nope_dim % 64) return SFA_ERR_DIMS;
  if (d->rope_positions < 1) return SFA_ERR_DIMS;
  if (!(d->eps >= 0.0f) || !isfinite(d->eps)) return SFA_ERR_DIMS;
  return SFA_OK;
}

// k splits of the down-projections: as many as keep the launch within one workgroup per
// compute unit (a second round of workgroups would run on an almost idle GPU), each split a
// whole number of 64-wide chunks
int down_splits(const sfa_prolog_dims* d) {
  const int feat = 32 * kPrFb0;
  const int64_t tiles = (d->q_lora_rank + kPrLatent + kPrRope + feat - 1) / feat;
  const int64_t tok_blocks = (d->tokens + kPrTokBlock - 1) / kPrTokBlock;
  const int units = d->hidden / 64;
  int best = 1;
  for (int s = 1; s <= units; ++s)
    if (units % s == 0 && tiles * tok_blocks * s <= kTargetWorkgroups) best = s;
  return best;
}

struct Layout {
  size_t part, cq_hi, cq_lo, qn_hi, qn_lo, total;
};

Layout layout(const sfa_prolog_dims* d, int splits) {
  const size_t t = (size_t)d->tokens;
  Layout l{};
  size_t o = 0;
  l.part = o;
  o += align_up((size_t)splits * t * (d->q_lora_rank + kPrLatent + kPrRope) * 4, kAlign);
  l.cq_hi = o;
  o += align_up(t * d->q_lora_rank * 2, kAlign);
  l.cq_lo = o;
  o += align_up(t * d->q_lora_rank * 2, kAlign);
  l.qn_hi = o;
  o += align_up(t * d->n_q * d->qk_nope_dim * 2, kAlign);
  l.qn_lo = o;
  o += align_up(t * d->n_q * d->qk_nope_dim * 2, kAlign);
  l.total = t ? o : 0;
  return l;
}

// ---- the V4 form of the MLA prolog

int check_v4(const sfa_prolog_v4_dims* d) {
  if (!d) return SFA_ERR_NULL;
  if (d->tokens < 0 || d->tokens > (1 << 20)) return SFA_ERR_DIMS;
  if (d->hidden < 64 || d->hidden > (1 << 16) || d->hidden % 64) return SFA_ERR_DIMS;
  if (d->q_lora_rank < 64 || d->q_lora_rank > 4096 || d->q_lora_rank % 64) return SFA_ERR_DIMS;
  if (d->n_q < 1 || d->n_q > SFA_MAX_HEADS) return SFA_ERR_DIMS;
  if (d->head_dim != kPrLatent) return SFA_ERR_DIMS;
  if (d->rope_positions < 1) return SFA_ERR_DIMS;
  if (!(d->eps >= 0.0f) || !isfinite(d->eps)) return SFA_ERR_DIMS;
  return SFA_OK;
}

// k splits of a weight-streaming GEMM over `feat_total` features: as many as keep the launch
// within one workgroup per compute unit, each a whole number of 64-wide chunks of k
int gemm_splits(int64_t feat_total, int mode, int64_t tokens, int k) {
  const int feat = 32 * prolog_feat_blocks(mode);
  const int64_t tiles = (feat_total + feat - 1) / feat;
  const int64_t tok_blocks = (tokens + kPrTokBlock - 1) / kPrTokBlock;
  const int units = k / 64;
  int best = 1;
  for (int s = 1; s <= units; ++s)
    if (units % s == 0 && tiles * tok_blocks * s <= kTargetWorkgroups) best = s;
  return best;
}

struct V4Layout {
  size_t part_down, cq_hi, cq_lo, part_up, total;
  int split_down, split_up;
};

V4Layout v4_layout(const sfa_prolog_v4_dims* d) {
  const size_t t = (size_t)d->tokens, q = (size_t)d->q_lora_rank, nf = (size_t)d->n_q * kPrLatent;
  V4Layout l{};
  l.split_down = gemm_splits((int64_t)q + kPrLatent, 0, d->tokens, d->hidden);
  l.split_up = gemm_splits((int64_t)nf, 3, d->tokens, d->q_lora_rank);
  size_t o = 0;
  l.part_down = o;
  o += align_up((size_t)l.split_down * t * (q + kPrLatent) * 4, kAlign);
  l.cq_hi = o;
  o += align_up(t * q * 2, kAlign);
  l.cq_lo = o;
  o += align_up(t * q * 2, kAlign);
  l.part_up = o;
  o += align_up((size_t)l.split_up * t * nf * 4, kAlign);
  l.total = t ? o : 0;
  return l;
}

// ---- indexer prolog

constexpr int kIpDim = 128;  // index head width (the Lightning Indexer's)

int check_ip(const sfa_indexer_prolog_dims* d) {
  if (!d) return SFA_ERR_NULL;
  if (d->tokens < 0 || d->tokens > (1 << 20)) return SFA_ERR_DIMS;
  if (d->hidden < 256 || d->hidden > (1 << 16) || d->hidden % 64) return SFA_ERR_DIMS;
  if (d->q_lora_rank < 256 || d->q_lora_rank > 4096 || d->q_lora_rank % 64) return SFA_ERR_DIMS;
  if (d->n_heads != 64 || d->head_dim != kIpDim) return SFA_ERR_DIMS;
  if (d->rope_positions < 1 || (d->rotate != 0 && d->rotate != 1)) return SFA_ERR_DIMS;
  if (!(d->eps >= 0.0f) || !isfinite(d->eps)) return SFA_ERR_DIMS;
  return SFA_OK;
}

// k splits of one of the indexer prolog's projections: the largest that keeps the launch
// within one round of workgroups and every split at least 4 chunks of 64
int ip_splits(int64_t tiles, int64_t tok_blocks, int k) {
  const int units = k / 64;
  int best = 1;
  for (int s = 1; s <= units; ++s)
    if (units % s == 0 && units / s >= 4 && tiles * tok_blocks * s <= kTargetWorkgroups) best = s;
  return best;
}

struct IpLayout {
  size_t part_q, part_kw, total;
  int split_q, split_kw;
};

IpLayout ip_layout(const sfa_indexer_prolog_dims* d) {
  const int64_t t = d->tokens, tok_blocks = (t + kPrTokBlock - 1) / kPrTokBlock;
  const int feat = 32 * kPrFb0;
  const int64_t nq = (int64_t)d->n_heads * kIpDim, nkw = kIpDim + d->n_heads;
  IpLayout l{};
  l.split_q = ip_splits((nq + feat - 1) / feat, tok_blocks, d->q_lora_rank);
  l.split_kw = ip_splits((nkw + feat - 1) / feat, tok_blocks, d->hidden);
  l.part_q = 0;
  l.part_kw = align_up((size_t)l.split_q * t * nq * 4, kAlign);
  l.total = t ? l.part_kw + align_up((size_t)l.split_kw * t * nkw * 4, kAlign) : 0;
  return l;
}

}  // namespace

extern "C" {

int sfa_mla_prolog_workspace_size(const sfa_prolog_dims* dims, size_t* bytes_out) {
  if (!bytes_out) return SFA_ERR_NULL;
  const int st = check(dims);
  if (st != SFA_OK) return st;
  *bytes_out = layout(dims, down_splits(dims)).total;
  return SFA_OK;
}

int sfa_mla_prolog(const sfa_prolog_dims* dims, const void* x, const void* w_dq, const void* gamma_cq,
                   const void* w_uq_qr, const void* w_uk, const void* w_dkv_kr, const void* gamma_ckv,
                   const int32_t* positions, const float* rope_cos, const float* rope_sin, void* q_nope,
                   void* q_rope, void* kv_nope, void* kv_rope, void* cq_out, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  const int st = check(dims);
  if (st != SFA_OK) return st;
  if (dims->tokens == 0) return SFA_OK;  // nothing to read or write; pointers may be NULL
  const void* ins[] = {x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos, rope_sin};
  void* outs[] = {q_nope, q_rope, kv_nope, kv_rope};
  for (const void* p : ins)
    if (!p) return SFA_ERR_NULL;
  for (const void* p : outs)
    if (!p) return SFA_ERR_NULL;
  for (const void* p : ins)
    if (!aligned16(p)) return SFA_ERR_ALIGN;
  for (const void* p : outs)
    if (!aligned16(p)) return SFA_ERR_ALIGN;
  if (cq_out && !aligned16(cq_out)) return SFA_ERR_ALIGN;
  const int splits = down_splits(dims);
  const Layout lay = layout(dims, splits);
  if (lay.total > 0 && (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace % kAlign) != 0))
    return SFA_ERR_WORKSPACE;

  const size_t t = (size_t)dims->tokens, h = (size_t)dims->hidden, q = (size_t)dims->q_lora_rank;
  const size_t n = (size_t)dims->n_q, dn = (size_t)dims->qk_nope_dim, np = (size_t)dims->rope_positions;
  const size_t in_bytes[] = {t * h * 2, q * h * 2, q * 2, n * (dn + kPrRope) * q * 2, n * kPrLatent * dn * 2,
                             (size_t)(kPrLatent + kPrRope) * h * 2, kPrLatent * 2, t * 4, np * 32 * 4, np * 32 * 4};
  const size_t out_bytes[] = {t * n * kPrLatent * 2, t * n * kPrRope * 2, t * kPrLatent * 2, t * kPrRope * 2};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 10; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return SFA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return SFA_ERR_ALIAS;
    if (overlaps(outs[i], out_bytes[i], workspace, lay.total)) return SFA_ERR_ALIAS;
    if (overlaps(outs[i], out_bytes[i], cq_out, t * q * 2)) return SFA_ERR_ALIAS;
  }
  for (int j = 0; j < 10; ++j) {
    if (overlaps(cq_out, t * q * 2, ins[j], in_bytes[j])) return SFA_ERR_ALIAS;
    if (overlaps(workspace, lay.total, ins[j], in_bytes[j])) return SFA_ERR_ALIAS;  // written by the kernels
  }
  if (overlaps(cq_out, t * q * 2, workspace, lay.total)) return SFA_ERR_ALIAS;
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + lay.part);
  uint16_t* cq_hi = reinterpret_cast<uint16_t*>(ws + lay.cq_hi);
  uint16_t* cq_lo = reinterpret_cast<uint16_t*>(ws + lay.cq_lo);
  uint16_t* qn_hi = reinterpret_cast<uint16_t*>(ws + lay.qn_hi);
  uint16_t* qn_lo = reinterpret_cast<uint16_t*>(ws + lay.qn_lo);
  const int tok_blocks = (int)((t + kPrTokBlock - 1) / kPrTokBlock);

  PrologGemmArgs g;
  memset(&g, 0, sizeof(g));
  g.tokens = (int32_t)t;
  g.tok_blocks = tok_blocks;
  g.positions = positions;
  g.rope_cos = rope_cos;
  g.rope_sin = rope_sin;
  g.rope_positions = dims->rope_positions;
  g.n_q = dims->n_q;
  g.dn = dims->qk_nope_dim;

  // 1. both down-projections, k split into `splits` ranges: fp32 partial sums
  PrologGemmArgs g1 = g;
  g1.w0 = static_cast<const uint16_t*>(w_dq);
  g1.w1 = static_cast<const uint16_t*>(w_dkv_kr);
  g1.f_split = (int32_t)q;
  g1.n_feat = (int32_t)(q + kPrLatent + kPrRope);
  g1.k = (int32_t)h;
  g1.n_split = splits;
  g1.k_chunk = (int32_t)(h / splits);
  g1.b_hi = static_cast<const uint16_t*>(x);
  g1.b_stride = (int64_t)h;
  g1.part = part;
  if (launch_prolog_gemm(g1, 0, stream) != hipSuccess) return SFA_ERR_HIP;

  // 2. partial sums, RMSNorms, the key's RoPE
  PrologNormArgs nm{};
  nm.part = part;
  nm.n_split = splits;
  nm.tokens = (int32_t)t;
  nm.q_rank = (int32_t)q;
  nm.gamma_cq = static_cast<const uint16_t*>(gamma_cq);
  nm.gamma_ckv = static_cast<const uint16_t*>(gamma_ckv);
  nm.eps = dims->eps;
  nm.cq_hi = cq_hi;
  nm.cq_lo = cq_lo;
  nm.kv_nope = static_cast<uint16_t*>(kv_nope);
  nm.kv_rope = static_cast<uint16_t*>(kv_rope);
  nm.cq_out = static_cast<uint16_t*>(cq_out);
  nm.positions = positions;
  nm.rope_cos = rope_cos;
  nm.rope_sin = rope_sin;
  nm.rope_positions = dims->rope_positions;
  if (launch_prolog_norm(nm, stream) != hipSuccess) return SFA_ERR_HIP;

  // 3. query up-projection: nope parts (hi/lo) and rotated rope parts
  PrologGemmArgs g2 = g;
  g2.w0 = static_cast<const uint16_t*>(w_uq_qr);
  g2.w1 = g2.w0;
  g2.n_feat = (int32_t)(n * (dn + kPrRope));
  g2.f_split = g2.n_feat;
  g2.k = (int32_t)q;
  g2.n_split = 1;
  g2.k_chunk = (int32_t)q;
  g2.b_hi = cq_hi;
  g2.b_lo = cq_lo;
  g2.b_stride = (int64_t)q;
  g2.qn_hi = qn_hi;
  g2.qn_lo = qn_lo;
  g2.q_rope = static_cast<uint16_t*>(q_rope);
  if (launch_prolog_gemm(g2, 1, stream) != hipSuccess) return SFA_ERR_HIP;

  // 4. absorption into the 512 latent channels per head
  PrologGemmArgs g3 = g;
  g3.w0 = static_cast<const uint16_t*>(w_uk);
  g3.w1 = g3.w0;
  g3.n_feat = kPrLatent;
  g3.f_split = kPrLatent;
  g3.k = (int32_t)dn;
  g3.n_split = 1;
  g3.k_chunk = (int32_t)dn;
  g3.b_hi = qn_hi;
  g3.b_lo = qn_lo;
  g3.b_stride = (int64_t)(n * dn);
  g3.q_nope = static_cast<uint16_t*>(q_nope);
  if (launch_prolog_gemm(g3, 2, stream) != hipSuccess) return SFA_ERR_HIP;
  return SFA_OK;
}

int sfa_mla_prolog_v4_workspace_size(const sfa_prolog_v4_dims* dims, size_t* bytes_out) {
  if (!bytes_out) return SFA_ERR_NULL;
  const int st = check_v4(dims);
  if (st != SFA_OK) return st;
  *bytes_out = v4_layout(dims).total;
  return SFA_OK;
}

int sfa_mla_prolog_v4(const sfa_prolog_v4_dims* dims, const void* x, const void* w_dq, const void* gamma_cq,
                      const void* w_uq, const void* w_dkv, const void* gamma_ckv, const int32_t* positions,
                      const float* rope_cos, const float* rope_sin, void* q, void* kv, void* cq_out,
                      void* workspace, size_t workspace_bytes, hipEvent_t kv_ready, hipStream_t stream) {
  const int st = check_v4(dims);
  if (st != SFA_OK) return st;
  if (dims->tokens == 0) return SFA_OK;  // nothing to read or write; pointers may be NULL
  const void* ins[] = {x, w_dq, gamma_cq, w_uq, w_dkv, gamma_ckv, positions, rope_cos, rope_sin};
  void* outs[] = {q, kv};
  for (const void* p : ins)
    if (!p) return SFA_ERR_NULL;
  for (const void* p : outs)
    if (!p) return SFA_ERR_NULL;
  for (const void* p : ins)
    if (!aligned16(p)) return SFA_ERR_ALIGN;
  for (const void* p : outs)
    if (!aligned16(p)) return SFA_ERR_ALIGN;
  if (cq_out && !aligned16(cq_out)) return SFA_ERR_ALIGN;
  const V4Layout lay = v4_layout(dims);
  if (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace % kAlign) != 0) return SFA_ERR_WORKSPACE;

  const size_t t = (size_t)dims->tokens, h = (size_t)dims->hidden, qr = (size_t)dims->q_lora_rank;
  const size_t n = (size_t)dims->n_q, np = (size_t)dims->rope_positions;
  const size_t in_bytes[] = {t * h * 2, qr * h * 2, qr * 2, n * kPrLatent * qr * 2, (size_t)kPrLatent * h * 2,
                             kPrLatent * 2, t * 4, np * 32 * 4, np * 32 * 4};
  const size_t out_bytes[] = {t * n * kPrLatent * 2, t * kPrLatent * 2, cq_out ? t * qr * 2 : 0};
  const void* all_outs[] = {q, kv, cq_out};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 9; ++j)
      if (overlaps(all_outs[i], out_bytes[i], ins[j], in_bytes[j])) return SFA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(all_outs[i], out_bytes[i], all_outs[j], out_bytes[j])) return SFA_ERR_ALIAS;
    if (overlaps(all_outs[i], out_bytes[i], workspace, lay.total)) return SFA_ERR_ALIAS;
  }
  for (int j = 0; j < 9; ++j)
    if (overlaps(workspace, lay.total, ins[j], in_bytes[j])) return SFA_ERR_ALIAS;  // written by the kernels
  char* ws = static_cast<char*>(workspace);
  float* part_down = reinterpret_cast<float*>(ws + lay.part_down);
  uint16_t* cq_hi = reinterpret_cast<uint16_t*>(ws + lay.cq_hi);
  uint16_t* cq_lo = reinterpret_cast<uint16_t*>(ws + lay.cq_lo);
  float* part_up = reinterpret_cast<float*>(ws + lay.part_up);
  const int tok_blocks = (int)((t + kPrTokBlock - 1) / kPrTokBlock);

  PrologGemmArgs g;
  memset(&g, 0, sizeof(g));
  g.tokens = (int32_t)t;
  g.tok_blocks = tok_blocks;
  g.positions = positions;
  g.rope_cos = rope_cos;
  g.rope_sin = rope_sin;
  g.rope_positions = dims->rope_positions;
  g.n_q = dims->n_q;

  // 1. both down-projections (query rank, then the 512-wide latent row), k split: fp32 partials
  PrologGemmArgs g1 = g;
  g1.w0 = static_cast<const uint16_t*>(w_dq);
  g1.w1 = static_cast<const uint16_t*>(w_dkv);
  g1.f_split = (int32_t)qr;
  g1.n_feat = (int32_t)(qr + kPrLatent);
  g1.k = (int32_t)h;
  g1.n_split = lay.split_down;
  g1.k_chunk = (int32_t)(h / lay.split_down);
  g1.b_hi = static_cast<const uint16_t*>(x);
  g1.b_stride = (int64_t)h;
  g1.part = part_down;
  if (launch_prolog_gemm(g1, 0, stream) != hipSuccess) return SFA_ERR_HIP;

  // 2. partial sums, the query-rank RMSNorm (cq as hi/lo), the latent row's RMSNorm and RoPE
  PrologNormArgs nm{};
  nm.part = part_down;
  nm.n_split = lay.split_down;
  nm.tokens = (int32_t)t;
  nm.q_rank = (int32_t)qr;
  nm.gamma_cq = static_cast<const uint16_t*>(gamma_cq);
  nm.gamma_ckv = static_cast<const uint16_t*>(gamma_ckv);
  nm.eps = dims->eps;
  nm.cq_hi = cq_hi;
  nm.cq_lo = cq_lo;
  nm.kv_nope = static_cast<uint16_t*>(kv);
  nm.kv_rope = nullptr;
  nm.cq_out = static_cast<uint16_t*>(cq_out);
  nm.positions = positions;
  nm.rope_cos = rope_cos;
  nm.rope_sin = rope_sin;
  nm.rope_positions = dims->rope_positions;
  nm.kv_inside = 1;
  if (launch_prolog_norm(nm, stream) != hipSuccess) return SFA_ERR_HIP;
  if (kv_ready && hipEventRecord(kv_ready, stream) != hipSuccess) return SFA_ERR_HIP;  // kv and cq final

  // 3. query up-projection over cq (hi and lo): fp32 sums per head channel
  PrologGemmArgs g2 = g;
  g2.w0 = static_cast<const uint16_t*>(w_uq);
  g2.w1 = g2.w0;
  g2.n_feat = (int32_t)(n * kPrLatent);
  g2.f_split = g2.n_feat;
  g2.k = (int32_t)qr;
  g2.n_split = lay.split_up;
  g2.k_chunk = (int32_t)(qr / lay.split_up);
  g2.b_hi = cq_hi;
  g2.b_lo = cq_lo;
  g2.b_stride = (int64_t)qr;
  g2.part = part_up;
  if (launch_prolog_gemm(g2, 3, stream) != hipSuccess) return SFA_ERR_HIP;

  // 4. per head: RMSNorm with unit weight, RoPE on its last 64 channels, bf16 rows
  PrologV4HeadArgs hd{};
  hd.part = part_up;
  hd.n_split = lay.split_up;
  hd.tokens = (int32_t)t;
  hd.n_q = dims->n_q;
  hd.n_feat = g2.n_feat;
  hd.eps = dims->eps;
  hd.positions = positions;
  hd.rope_cos = rope_cos;
  hd.rope_sin = rope_sin;
  hd.rope_positions = dims->rope_positions;
  hd.q = static_cast<uint16_t*>(q);
  return launch_prolog_v4_head(hd, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

int sfa_indexer_prolog_workspace_size(const sfa_indexer_prolog_dims* dims, size_t* bytes_out) {
  if (!bytes_out) return SFA_ERR_NULL;
  const int st = check_ip(dims);
  if (st != SFA_OK) return st;
  *bytes_out = ip_layout(dims).total;
  return SFA_OK;
}

int sfa_indexer_prolog(const sfa_indexer_prolog_dims* dims, const void* x, const void* qr, const void* w_idx_qb,
                       const void* w_idx_k, const void* ln_gamma_k, const void* ln_beta_k, const void* w_idx_proj,
                       const int32_t* positions, const float* rope_cos, const float* rope_sin, void* q_index,
                       void* k_index, float* weights, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_ip(dims);
  if (st != SFA_OK) return st;
  if (dims->tokens == 0) return SFA_OK;  // nothing to read or write; pointers may be NULL
  const void* ins[] = {x, qr, w_idx_qb, w_idx_k, ln_gamma_k, ln_beta_k, w_idx_proj, positions, rope_cos, rope_sin};
  void* outs[] = {q_index, k_index, weights};
  for (const void* p : ins)
    if (!p) return SFA_ERR_NULL;
  for (const void* p : outs)
    if (!p) return SFA_ERR_NULL;
  for (const void* p : ins)
    if (!aligned16(p)) return SFA_ERR_ALIGN;
  for (const void* p : outs)
    if (!aligned16(p)) return SFA_ERR_ALIGN;
  const IpLayout lay = ip_layout(dims);
  if (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace % kAlign) != 0) return SFA_ERR_WORKSPACE;
  const size_t t = (size_t)dims->tokens, h = (size_t)dims->hidden, q = (size_t)dims->q_lora_rank;
  const size_t nh = (size_t)dims->n_heads, np = (size_t)dims->rope_positions;
  const size_t in_bytes[] = {t * h * 2, t * q * 2, nh * kIpDim * q * 2, kIpDim * h * 2, kIpDim * 2, kIpDim * 2,
                             nh * h * 2, t * 4, np * 32 * 4, np * 32 * 4};
  const size_t out_bytes[] = {t * nh * kIpDim * 2, t * kIpDim * 2, t * nh * 4};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 10; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return SFA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return SFA_ERR_ALIAS;
    if (overlaps(outs[i], out_bytes[i], workspace, lay.total)) return SFA_ERR_ALIAS;
  }
  for (int j = 0; j < 10; ++j)
    if (overlaps(workspace, lay.total, ins[j], in_bytes[j])) return SFA_ERR_ALIAS;  // written by the kernels
  char* ws = static_cast<char*>(workspace);
  float* part_q = reinterpret_cast<float*>(ws + lay.part_q);
  float* part_kw = reinterpret_cast<float*>(ws + lay.part_kw);

  PrologGemmArgs g;
  memset(&g, 0, sizeof(g));
  g.tokens = (int32_t)t;
  g.tok_blocks = (int)((t + kPrTokBlock - 1) / kPrTokBlock);

  // index query: qr . W_qb^T, fp32 partial sums over `split_q` k ranges
  PrologGemmArgs g1 = g;
  g1.w0 = static_cast<const uint16_t*>(w_idx_qb);
  g1.w1 = g1.w0;
  g1.n_feat = (int32_t)(nh * kIpDim);
  g1.f_split = g1.n_feat;
  g1.k = (int32_t)q;
  g1.n_split = lay.split_q;
  g1.k_chunk = (int32_t)(q / lay.split_q);
  g1.b_hi = static_cast<const uint16_t*>(qr);
  g1.b_stride = (int64_t)q;
  g1.part = part_q;
  if (launch_prolog_gemm(g1, 0, stream) != hipSuccess) return SFA_ERR_HIP;

  // key and weight projections of x: rows of W_k, then of W_proj
  PrologGemmArgs g2 = g;
  g2.w0 = static_cast<const uint16_t*>(w_idx_k);
  g2.w1 = static_cast<const uint16_t*>(w_idx_proj);
  g2.f_split = kIpDim;
  g2.n_feat = (int32_t)(kIpDim + nh);
  g2.k = (int32_t)h;
  g2.n_split = lay.split_kw;
  g2.k_chunk = (int32_t)(h / lay.split_kw);
  g2.b_hi = static_cast<const uint16_t*>(x);
  g2.b_stride = (int64_t)h;
  g2.part = part_kw;
  if (launch_prolog_gemm(g2, 0, stream) != hipSuccess) return SFA_ERR_HIP;

  IndexerFinishArgs f;
  f.part_q = part_q;
  f.part_kw = part_kw;
  f.split_q = lay.split_q;
  f.split_kw = lay.split_kw;
  f.tokens = (int32_t)t;
  f.n_heads = (int32_t)nh;
  f.rotate = dims->rotate;
  f.ln_gamma = static_cast<const uint16_t*>(ln_gamma_k);
  f.ln_beta = static_cast<const uint16_t*>(ln_beta_k);
  f.eps = dims->eps;
  f.w_scale = (float)(1.0 / sqrt((double)nh * kIpDim));
  f.positions = positions;
  f.rope_cos = rope_cos;
  f.rope_sin = rope_sin;
  f.rope_positions = dims->rope_positions;
  f.q_index = static_cast<uint16_t*>(q_index);
  f.k_index = static_cast<uint16_t*>(k_index);
  f.weights = weights;
  return launch_indexer_finish(f, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

}  // extern "C"
