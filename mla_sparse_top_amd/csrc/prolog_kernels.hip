// MLA prolog: HIP kernels for gfx950 (CDNA4).
//
// What is computed ("CANN DeepSeek Indexer attention optimisation", section "MLA Prolog", with
// its parameter list; "NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section
// "MlaProlog", computation steps): for each new token with hidden row x,
//   cq      = RMSNorm(x . w_dq^T) * gamma_cq
//   u       = cq . w_uq_qr^T, per head h: nope part qn_h (dn channels), rotary part qp_h (64)
//   q_nope  = qn_h . w_uk[h]^T (weight absorption: 512 channels per head)
//   q_rope  = RoPE(qp_h)
//   kv      = x . w_dkv_kr^T: latent row RMSNorm(kv[:512]) * gamma_ckv, rotary key RoPE(kv[512:])
// RoPE rotates adjacent channel pairs by the angle of the token's position (caller's tables).
//
// How it is computed here (four launches on one stream):
//   1. prolog_gemm_kernel<0>: both down-projections as one weight-streaming GEMM over the
//      features of w_dq then w_dkv_kr. Weights go from HBM straight into the A operand of
//      v_mfma_f32_32x32x16_bf16 (32 features x 16 k per instruction), activations into the B
//      operand (32 tokens). A workgroup owns 64 features x 128 tokens x one k range; its four
//      waves split that range and sum their accumulators through LDS; the k ranges of one
//      feature tile are separate workgroups that write fp32 partial sums.
//   2. prolog_norm_kernel: one workgroup per token sums the partials, applies both RMSNorms
//      and the key's RoPE, and writes cq as a bf16 hi + lo pair (hi = bf16(v), lo = bf16(v -
//      hi): about 16 significant bits, so cq is not rounded to bf16 between the steps).
//   3. prolog_gemm_kernel<1>: the query up-projection over cq (two MFMAs per step, hi and lo).
//      Its epilogue writes each head's nope part as a hi + lo pair and rotates the rotary part.
//   4. prolog_gemm_kernel<2>: the absorption, per head a 512 x dn weight over the nope part
//      (hi and lo), each wave owning 64 of a workgroup's 256 output channels.
// Loads use buffer descriptors whose range ends at the last token, so the rows of a partial
// token block read zeros and are never stored.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "prolog_internal.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kFm = 2;     // 32-feature MFMA blocks per wave
constexpr int kTn = 4;     // 32-token MFMA blocks per wave
constexpr int kDepth = 4;  // k-steps whose loads are in flight ahead of the MFMAs
constexpr int kTiles = kFm * kTn;
constexpr int kNormMaxChunks = 5;  // float4 chunks per thread in the norm step: q_rank <= 4096

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8 load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// two floats -> two bf16 (round to nearest even) in one dword, first in the low half
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_value(__bf16 b) { return (float)b; }

// v as a bf16 pair: hi = bf16(v), lo = bf16(v - hi) (v - hi is exact in fp32)
__device__ __forceinline__ void split4(const floatx4 v, u32x2& hi, u32x2& lo) {
  bf16x2 h0, h1;
  h0[0] = (__bf16)v[0];
  h0[1] = (__bf16)v[1];
  h1[0] = (__bf16)v[2];
  h1[1] = (__bf16)v[3];
  hi = u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
  lo = u32x2{pack2(v[0] - (float)h0[0], v[1] - (float)h0[1]), pack2(v[2] - (float)h1[0], v[3] - (float)h1[1])};
}

// Rotates the pairs (v0, v1) and (v2, v3) by table columns i and i + 1 of position p (zeros
// when p is outside the tables) and packs them as four bf16.
__device__ __forceinline__ u32x2 rope4(const floatx4 v, int p, int np, const float* cs, const float* sn, int i) {
  if (p < 0 || p >= np) return u32x2{0u, 0u};
  const float c0 = cs[(size_t)p * 32 + i], s0 = sn[(size_t)p * 32 + i];
  const float c1 = cs[(size_t)p * 32 + i + 1], s1 = sn[(size_t)p * 32 + i + 1];
  return u32x2{pack2(v[0] * c0 - v[1] * s0, v[0] * s0 + v[1] * c0),
               pack2(v[2] * c1 - v[3] * s1, v[2] * s1 + v[3] * c1)};
}

// Mode 0: down-projections (fp32 partials). Mode 1: query up-projection (B = cq hi/lo).
// Mode 2: absorption (B = the heads' nope parts hi/lo).
template <int kMode>
__global__ void __launch_bounds__(kThreads, 1) prolog_gemm_kernel(const PrologGemmArgs a) {
  constexpr bool kLo = kMode != 0;
  constexpr bool kSplitWaves = kMode != 2;
  __shared__ floatx4 red[kSplitWaves ? 4 : 1][kTiles * 4][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31, hb = lane >> 5;

  // workgroup -> (token block, feature tile / head, k split)
  int id = blockIdx.x;
  int split = 0, head = 0, f0;
  if (kMode == 2) {
    const int half = id % (kPrLatent / kPrAbsTile);
    id /= kPrLatent / kPrAbsTile;
    head = id % a.n_q;
    id /= a.n_q;
    f0 = half * kPrAbsTile + wave * (kFm * 32);
  } else {
    split = id % a.n_split;
    id /= a.n_split;
    const int tiles = (a.n_feat + kPrFeatTile - 1) / kPrFeatTile;
    f0 = (id % tiles) * kPrFeatTile;
    id /= tiles;
  }
  const int tb0 = id * kPrTokBlock;
  const int rows = min(kPrTokBlock, a.tokens - tb0);

  // weights of this tile: rows f0 .. f0 + 63 (mode 2: head's 512 x dn block)
  const uint16_t* wbase;
  uint32_t wrows;
  if (kMode == 2) {
    wbase = a.w0 + ((size_t)head * kPrLatent + f0) * a.k;
    wrows = kFm * 32;
  } else if (f0 < a.f_split) {
    wbase = a.w0 + (size_t)f0 * a.k;
    wrows = min(kPrFeatTile, a.f_split - f0);
  } else {
    wbase = a.w1 + (size_t)(f0 - a.f_split) * a.k;
    wrows = min(kPrFeatTile, a.n_feat - f0);
  }
  const __amdgpu_buffer_rsrc_t rw = rsrc(wbase, wrows * (uint32_t)a.k * 2u);
  const size_t boff = (size_t)tb0 * a.b_stride + (kMode == 2 ? (size_t)head * a.dn : 0);
  const uint32_t bbytes = (uint32_t)(((size_t)(rows - 1) * a.b_stride + a.k) * 2);
  const __amdgpu_buffer_rsrc_t rbh = rsrc(a.b_hi + boff, bbytes);
  const __amdgpu_buffer_rsrc_t rbl = rsrc(kLo ? a.b_lo + boff : a.b_hi + boff, bbytes);

  // this wave's k range
  const int kw = kSplitWaves ? a.k_chunk / 4 : a.k;
  const int kw0 = kSplitWaves ? split * a.k_chunk + wave * kw : 0;
  const int steps = kw / 16;

  uint32_t voa[kFm], vob[kTn];
#pragma unroll
  for (int fm = 0; fm < kFm; ++fm) voa[fm] = (uint32_t)(((32 * fm + r) * a.k + 8 * hb) * 2);
#pragma unroll
  for (int tb = 0; tb < kTn; ++tb) vob[tb] = (uint32_t)(((size_t)(32 * tb + r) * a.b_stride + 8 * hb) * 2);

  floatx16 acc[kFm][kTn];
#pragma unroll
  for (int fm = 0; fm < kFm; ++fm)
#pragma unroll
    for (int tb = 0; tb < kTn; ++tb) acc[fm][tb] = floatx16{};

  bf16x8 ra[kDepth][kFm], rb[kDepth][kTn], rl[kDepth][kLo ? kTn : 1];
  auto load = [&](int slot, int s) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)(kw0 + 16 * s) * 2u;
#pragma unroll
    for (int fm = 0; fm < kFm; ++fm) ra[slot][fm] = load8(rw, voa[fm], kb);
#pragma unroll
    for (int tb = 0; tb < kTn; ++tb) {
      rb[slot][tb] = load8(rbh, vob[tb], kb);
      if (kLo) rl[slot][tb] = load8(rbl, vob[tb], kb);
    }
  };
  auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int fm = 0; fm < kFm; ++fm)
#pragma unroll
      for (int tb = 0; tb < kTn; ++tb) {
        acc[fm][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[slot][fm], rb[slot][tb], acc[fm][tb], 0, 0, 0);
        if (kLo)
          acc[fm][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[slot][fm], rl[slot][tb], acc[fm][tb], 0, 0, 0);
      }
  };
  // steps >= kDepth (the host keeps every wave's k range at least kDepth * 16 long): the loads
  // of kDepth steps are in flight while a step's MFMAs run; the main loop has no branches, so
  // each step waits only for its own loads
#pragma unroll
  for (int j = 0; j < kDepth; ++j) load(j, j);
  int s = 0;
  for (; s + 2 * kDepth <= steps; s += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      mfmas(j);
      load(j, s + j + kDepth);
    }
  }
#pragma unroll
  for (int j = 0; j < kDepth; ++j) {
    mfmas(j);
    if (s + j + kDepth < steps) load(j, s + j + kDepth);
  }
  s += kDepth;
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (s + j < steps) mfmas(j);

  // Output tile (fm, tb): lane holds token 32*tb + r and, in register 4*g + e, feature
  // 32*fm + 8*g + 4*hb + e.
  auto epilogue = [&](int fm, int tb, const floatx4 (&v)[4]) __attribute__((always_inline)) {
    const int t = tb0 + 32 * tb + r;
    if (t >= a.tokens) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + 32 * fm + 8 * g + 4 * hb;
      if (kMode == 0) {
        *reinterpret_cast<floatx4*>(a.part + ((size_t)split * a.tokens + t) * a.n_feat + f) = v[g];
      } else if (kMode == 1) {
        if (f >= a.n_feat) continue;
        const int per = a.dn + kPrRope;
        const int h = f / per, j = f - h * per;
        const size_t row = (size_t)t * a.n_q + h;
        if (j < a.dn) {
          u32x2 hi, lo;
          split4(v[g], hi, lo);
          *reinterpret_cast<u32x2*>(a.qn_hi + row * a.dn + j) = hi;
          *reinterpret_cast<u32x2*>(a.qn_lo + row * a.dn + j) = lo;
        } else {
          const int jr = j - a.dn;
          *reinterpret_cast<u32x2*>(a.q_rope + row * kPrRope + jr) =
              rope4(v[g], a.positions[t], a.rope_positions, a.rope_cos, a.rope_sin, jr >> 1);
        }
      } else {
        const size_t row = (size_t)t * a.n_q + head;
        *reinterpret_cast<u32x2*>(a.q_nope + row * kPrLatent + f) =
            u32x2{pack2(v[g][0], v[g][1]), pack2(v[g][2], v[g][3])};
      }
    }
  };

  if (kSplitWaves) {
    // sum the four waves' partial tiles: every wave stores its tiles, then wave w sums tiles
    // 2w and 2w + 1 over the four copies and runs their epilogue
#pragma unroll
    for (int i = 0; i < kTiles; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx16& x = acc[i / kTn][i % kTn];
        red[wave][i * 4 + g][lane] = floatx4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
      }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = 2 * wave + q;
      floatx4 v[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v[g] = red[0][i * 4 + g][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) v[g] += red[w][i * 4 + g][lane];
      }
      epilogue(i / kTn, i % kTn, v);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
      const floatx16& x = acc[i / kTn][i % kTn];
      floatx4 v[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) v[g] = floatx4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
      epilogue(i / kTn, i % kTn, v);
    }
  }
}

// Sum of x over the workgroup (256 threads); every thread gets the result.
__device__ __forceinline__ float block_sum(float x, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  const float s = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return s;
}

__global__ void __launch_bounds__(kThreads) prolog_norm_kernel(const PrologNormArgs a) {
  __shared__ float sh[4];
  const int t = blockIdx.x;
  const int nf = a.q_rank + kPrLatent + kPrRope;
  const int nq4 = a.q_rank / 4, nkv4 = nq4 + kPrLatent / 4, nch = nf / 4;
  floatx4 v[kNormMaxChunks];
  float ssq = 0.f, skv = 0.f;
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = threadIdx.x + i * kThreads;
    v[i] = floatx4{};
    if (c < nch) {
      for (int s = 0; s < a.n_split; ++s)
        v[i] += *reinterpret_cast<const floatx4*>(a.part + ((size_t)s * a.tokens + t) * nf + 4 * c);
      const float sq = v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
      if (c < nq4)
        ssq += sq;
      else if (c < nkv4)
        skv += sq;
    }
  }
  const float inv_q = 1.0f / sqrtf(block_sum(ssq, sh) / (float)a.q_rank + a.eps);
  const float inv_kv = 1.0f / sqrtf(block_sum(skv, sh) / (float)kPrLatent + a.eps);
  const int p = a.positions[t];
  const __bf16* gq = reinterpret_cast<const __bf16*>(a.gamma_cq);
  const __bf16* gk = reinterpret_cast<const __bf16*>(a.gamma_ckv);
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c >= nch) continue;
    if (c < nq4) {
      floatx4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = v[i][e] * inv_q * bf16_value(gq[4 * c + e]);
      u32x2 hi, lo;
      split4(y, hi, lo);
      *reinterpret_cast<u32x2*>(a.cq_hi + (size_t)t * a.q_rank + 4 * c) = hi;
      *reinterpret_cast<u32x2*>(a.cq_lo + (size_t)t * a.q_rank + 4 * c) = lo;
    } else if (c < nkv4) {
      const int j = 4 * (c - nq4);
      floatx4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = v[i][e] * inv_kv * bf16_value(gk[j + e]);
      *reinterpret_cast<u32x2*>(a.kv_nope + (size_t)t * kPrLatent + j) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
    } else {
      const int j = 4 * (c - nkv4);
      *reinterpret_cast<u32x2*>(a.kv_rope + (size_t)t * kPrRope + j) =
          rope4(v[i], p, a.rope_positions, a.rope_cos, a.rope_sin, j >> 1);
    }
  }
}

}  // namespace

hipError_t launch_prolog_gemm(const PrologGemmArgs& a, int mode, hipStream_t stream) {
  int grid;
  if (mode == 2)
    grid = a.tok_blocks * a.n_q * (kPrLatent / kPrAbsTile);
  else
    grid = a.tok_blocks * ((a.n_feat + kPrFeatTile - 1) / kPrFeatTile) * a.n_split;
  if (mode == 0)
    hipLaunchKernelGGL(prolog_gemm_kernel<0>, dim3(grid), dim3(kThreads), 0, stream, a);
  else if (mode == 1)
    hipLaunchKernelGGL(prolog_gemm_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(prolog_gemm_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prolog_norm(const PrologNormArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prolog_norm_kernel, dim3(a.tokens), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfa
