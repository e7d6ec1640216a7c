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
//      features of w_dq then w_dkv_kr: weights in the A operand of v_mfma_f32_32x32x16_bf16
//      (32 features x 16 k), activations in the B operand (32 tokens), both staged through
//      LDS. A workgroup owns 64 features x 128 tokens x one k range; the k ranges of one
//      feature tile are separate workgroups that write fp32 partial sums.
//   2. prolog_norm_kernel: one workgroup per token sums the partials, applies both RMSNorms
//      and the key's RoPE, and writes cq as a bf16 hi + lo pair (hi = bf16(v), lo = bf16(v -
//      hi): about 16 significant bits, so cq is not rounded to bf16 between the steps).
//   3. prolog_gemm_kernel<1>: the query up-projection over cq (two MFMAs per step, hi and lo).
//      Its epilogue writes each head's nope part as a hi + lo pair and rotates the rotary part.
//   4. prolog_gemm_kernel<2>: the absorption, per head a 512 x dn weight over the nope part
//      (hi and lo), in tiles of 64 output channels.
// The V4 form (same page section, its own layout: 512-wide query heads and latent row with the
// rotary part inside, no absorption) runs four launches too: the down-projections (query rank
// and the 512-wide latent row) as step 1; the norm kernel with the latent row normalised whole
// and its last 64 channels rotated in place; prolog_gemm_kernel<3>, the up-projection over cq
// hi + lo into fp32 sums, 256 features per workgroup (one round of 256 workgroups at 128 heads,
// each reading cq once); and prolog_v4_head_kernel, per head RMSNorm with unit weight and RoPE
// in place on the head's last 64 channels.
// Operands reach LDS through buffer descriptors whose range ends at the last token (or weight
// row), so the rows of a partial block read zeros, and their outputs are never stored.

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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kNormMaxChunks = 5;  // float4 chunks per thread in the norm step: q_rank <= 4096

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

// Buffer resource over [base, base + bytes): loads at or past the end read zeros.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  // dword 2: the size in bytes; dword 3: raw-buffer configuration (32-bit data format, no
  // swizzle, no stride)
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, 0x00020000u};
}

// LDS-DMA: lane L's 16 bytes from the buffer at voff + soff land at LDS address lds + 16 * L.
// M0 is saved and restored around the instruction and needs one wait state after its write.
// Issued from inline asm so that the compiler does not wait for the whole vector-memory queue
// before LDS reads; completion is waited for explicitly (wait_vmcnt), visibility to the other
// waves comes from the barrier after that wait.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most n groups of kPer vector-memory instructions are outstanding (n <= 6).
template <int kPer>
__device__ __forceinline__ void wait_groups(int n) {
  if (n >= 6)
    wait_vmcnt<6 * kPer>();
  else if (n == 5)
    wait_vmcnt<5 * kPer>();
  else if (n == 4)
    wait_vmcnt<4 * kPer>();
  else if (n == 3)
    wait_vmcnt<3 * kPer>();
  else if (n == 2)
    wait_vmcnt<2 * kPer>();
  else if (n == 1)
    wait_vmcnt<kPer>();
  else
    wait_vmcnt<0>();
}

// Workgroup barrier that orders LDS traffic only: outstanding DMA stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
}

typedef __attribute__((address_space(3))) char lds_char_t;

__device__ __forceinline__ bf16x8 lds16(const lds_char_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// Mode 0: down-projections (fp32 partials). Mode 1: query up-projection (B = cq hi/lo).
// Mode 2: absorption (B = the heads' nope parts hi/lo). Mode 3: the V4 query up-projection
// (B = cq hi/lo, fp32 sums out, normalised per head by prolog_v4_head_kernel).
//
// A workgroup owns 32 * kFb features x 128 tokens and walks its k range in chunks of 64 (one
// 128-byte line per row). Wave w owns tokens 32w .. 32w + 31 and all the workgroup's features,
// so its accumulators are whole sums. Weight rows and token rows reach LDS by LDS-DMA, eight
// rows x 128 bytes per instruction, the 16-byte piece p of row r stored at position
// p ^ ((r >> 1) & 7) so that the operand reads are free of bank conflicts: a 16-byte-per-lane
// LDS read is served 16 lanes at a time over 64 banks (256 bytes), and its 16 lanes read 16
// consecutive rows, whose row pairs fill the two 128-byte halves and take 8 distinct positions
// in each. Waves 0 and 1 issue the weights' DMA
// (from HBM, through a deep ring), waves 2 and 3 the token rows' (from L2, a shallow ring):
// a wave's loads complete in issue order, so a wave that waits for one stream never waits
// for the other. The outputs are staged through LDS and stored as whole rows.
template <int kMode, int kFb>
struct GemmShape {
  static constexpr bool kLo = kMode != 0;
  static constexpr int kFeat = 32 * kFb;
  static constexpr int kWBytes = kFeat * 128;                  // weight rows of a chunk
  static constexpr int kABytes = kPrTokBlock * 128;            // token rows of a chunk (hi or lo)
  static constexpr int kAStage = kABytes * (kLo ? 2 : 1);
  static constexpr int kTStages = kMode == 2 || kMode == 3 ? 2 : 3;
  static constexpr int kWFit = (152 * 1024 - kTStages * kAStage) / kWBytes;
  static constexpr int kWStages = kWFit > 8 ? 8 : kWFit;
  static constexpr int kLdsBytes = kWStages * kWBytes + kTStages * kAStage;
  static constexpr int kWDma = 2 * kFb;                        // per weight wave and chunk
  static constexpr int kTDma = 16 * (kLo ? 2 : 1) / 2;         // per token wave and chunk
  // output staging: 128 token rows of the workgroup's features (fp32 partials, bf16 q_nope),
  // each row padded by 16 bytes so that the 32 rows a store instruction touches spread over
  // the LDS banks
  static constexpr bool kF32Out = kMode == 0 || kMode == 3;    // fp32 partial sums out
  static constexpr int kOutRow = kFeat * (kF32Out ? 4 : 2);
  static constexpr int kOutStride = kOutRow + 16;
  static_assert(kWStages >= 2 && kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(kMode == 1 || kMode == 3 || kPrTokBlock * kOutStride <= kLdsBytes, "output staging fits");
  static_assert(kWDma * (kWStages - 2) <= 63 && kTDma * (kTStages - 2) <= 63, "vmcnt range");
};

template <int kMode, int kFb>
__global__ void __launch_bounds__(kThreads, 1) prolog_gemm_kernel(const PrologGemmArgs a) {
  using G = GemmShape<kMode, kFb>;
  constexpr bool kLo = G::kLo;
  constexpr int kFeat = G::kFeat, kWBytes = G::kWBytes, kABytes = G::kABytes, kAStage = G::kAStage;
  constexpr int kWStages = G::kWStages, kTStages = G::kTStages;
  __shared__ __attribute__((aligned(1024))) char smem[G::kLdsBytes];
  const lds_char_t* lds = (const lds_char_t*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const uint32_t abase = lds_base + kWStages * kWBytes;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, hb = lane >> 5;

  // workgroup -> (token block, feature tile or head and tile, k split)
  int id = blockIdx.x;
  int split = 0, head = 0, f0;
  if (kMode == 2) {
    constexpr int per_head = kPrLatent / kFeat;
    f0 = (id % per_head) * kFeat;
    id /= per_head;
    head = id % a.n_q;
    id /= a.n_q;
  } else {
    split = id % a.n_split;
    id /= a.n_split;
    const int tiles = (a.n_feat + kFeat - 1) / kFeat;
    f0 = (id % tiles) * kFeat;
    id /= tiles;
  }
  const int tb0 = id * kPrTokBlock;
  const int rows = min(kPrTokBlock, a.tokens - tb0);

  // weights of this tile: kFeat rows (features f0 ..) of k elements
  const uint16_t* wbase;
  uint32_t wrows;
  if (kMode == 2) {
    wbase = a.w0 + ((size_t)head * kPrLatent + f0) * a.k;
    wrows = kFeat;
  } else if (f0 < a.f_split) {
    wbase = a.w0 + (size_t)f0 * a.k;
    wrows = min(kFeat, a.f_split - f0);
  } else {
    wbase = a.w1 + (size_t)(f0 - a.f_split) * a.k;
    wrows = min(kFeat, a.n_feat - f0);
  }
  const int kc0 = kMode == 2 ? 0 : split * a.k_chunk;
  const int nch = (kMode == 2 ? a.k : a.k_chunk) / 64;

  // DMA lane geometry: lane L carries row (L >> 3) of an 8-row group starting at row 8j and
  // stores its piece at position L & 7, so it loads piece (L & 7) ^ (L >> 4) ^ 4 (j & 1) of its
  // row (row >> 1 is 4j + (L >> 4))
  const uint32_t drow = (uint32_t)(lane >> 3);
  const uint32_t dpiece = 16u * ((uint32_t)(lane & 7) ^ (drow >> 1));
  const bool w_wave = wave < 2;
  u32x4 rs0, rs1;
  uint32_t row_bytes;
  if (w_wave) {
    rs0 = make_rsrc(wbase, wrows * (uint32_t)a.k * 2u);
    rs1 = rs0;
    row_bytes = (uint32_t)a.k * 2u;
  } else {
    const size_t boff = (size_t)tb0 * a.b_stride + (kMode == 2 ? (size_t)head * a.dn : 0);
    const uint32_t bbytes = (uint32_t)(((size_t)(rows - 1) * a.b_stride + a.k) * 2);
    rs0 = make_rsrc(a.b_hi + boff, bbytes);
    rs1 = make_rsrc(kLo ? a.b_lo + boff : a.b_hi + boff, bbytes);
    row_bytes = (uint32_t)a.b_stride * 2u;
  }
  const int half = wave & 1;  // which half of the rows this wave's DMA covers

  // chunk c's DMA share of this wave: weight waves take 8-row groups half, half + 2, ... of the
  // kFeat weight rows; token waves take token rows 64 * half .. + 63 (hi, then lo)
  auto issue = [&](int c) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)(kc0 + 64 * c) * 2u;
    if (w_wave) {
      const uint32_t st = lds_base + (uint32_t)((c % kWStages) * kWBytes);
#pragma unroll
      for (int i = 0; i < 2 * kFb; ++i) {
        const uint32_t row0 = (uint32_t)(8 * (half + 2 * i));  // group half + 2i: odd for wave 1
        dma16(rs0, (row0 + drow) * row_bytes + (dpiece ^ (64u * (uint32_t)half)), kb, st + row0 * 128u);
      }
    } else {
      const uint32_t st = abase + (uint32_t)((c % kTStages) * kAStage);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t row0 = (uint32_t)(64 * half + 8 * i);  // group 8 half + i
        const uint32_t pc = dpiece ^ (64u * (uint32_t)(i & 1));
        dma16(rs0, (row0 + drow) * row_bytes + pc, kb, st + row0 * 128u);
        if (kLo) dma16(rs1, (row0 + drow) * row_bytes + pc, kb, st + kABytes + row0 * 128u);
      }
    }
  };
  const int depth = w_wave ? kWStages : kTStages;
  // wait for this wave's DMA of chunk c, leaving the later chunks it has issued in flight
  auto wait_for = [&](int c) __attribute__((always_inline)) {
    const int ahead = min(depth - 2, nch - 1 - c);
    if (w_wave)
      wait_groups<G::kWDma>(ahead);
    else
      wait_groups<G::kTDma>(ahead);
  };

  floatx16 acc[kFb];
#pragma unroll
  for (int fb = 0; fb < kFb; ++fb) acc[fb] = floatx16{};

  for (int c = 0; c < depth - 1; ++c)
    if (c < nch) issue(c);
  const int wave_row = 32 * wave + r;
  const uint32_t rsw = 16u * (uint32_t)((r >> 1) & 7);  // rows 32 fb + r and 32 w + r
  for (int c = 0; c < nch; ++c) {
    wait_for(c);
    lds_barrier();  // chunk c visible to every wave; chunk c - 1's slots free again
    if (c + depth - 1 < nch) issue(c + depth - 1);
    const lds_char_t* ws = lds + (c % kWStages) * kWBytes;
    const lds_char_t* as = lds + kWStages * kWBytes + (c % kTStages) * kAStage + wave_row * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t pos = (16u * (uint32_t)(2 * s + hb)) ^ rsw;
      const bf16x8 bv = lds16(as + pos);
      bf16x8 lv;
      if (kLo) lv = lds16(as + kABytes + pos);
#pragma unroll
      for (int fb = 0; fb < kFb; ++fb) {
        const bf16x8 av = lds16(ws + (32 * fb + r) * 128 + pos);
        acc[fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[fb], 0, 0, 0);
        if (kLo) acc[fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, lv, acc[fb], 0, 0, 0);
      }
    }
  }

  // Output block fb: lane holds token 32 * wave + r and, in register 4 * g + e, feature
  // 32 * fb + 8 * g + 4 * hb + e.
  if (kMode == 1) {
    const int t = tb0 + wave_row;
    if (t >= a.tokens) return;
#pragma unroll
    for (int fb = 0; fb < kFb; ++fb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 v = floatx4{acc[fb][4 * g], acc[fb][4 * g + 1], acc[fb][4 * g + 2], acc[fb][4 * g + 3]};
        const int f = f0 + 32 * fb + 8 * g + 4 * hb;
        if (f >= a.n_feat) continue;
        const int per = a.dn + kPrRope;
        const int h = f / per, j = f - h * per;
        const size_t row = (size_t)t * a.n_q + h;
        if (j < a.dn) {
          u32x2 hi, lo;
          split4(v, hi, lo);
          *reinterpret_cast<u32x2*>(a.qn_hi + row * a.dn + j) = hi;
          *reinterpret_cast<u32x2*>(a.qn_lo + row * a.dn + j) = lo;
        } else {
          const int jr = j - a.dn;
          *reinterpret_cast<u32x2*>(a.q_rope + row * kPrRope + jr) =
              rope4(v, a.positions[t], a.rope_positions, a.rope_cos, a.rope_sin, jr >> 1);
        }
      }
    }
    return;
  }

  if (kMode == 3) {
    // fp32 sums straight from the accumulators: 16 bytes per lane, the 8 pieces of a token's
    // 128-byte feature block come from one instruction's lanes
    const int t = tb0 + wave_row;
    if (t >= a.tokens) return;
    float* dst = a.part + ((size_t)split * a.tokens + t) * a.n_feat;
#pragma unroll
    for (int fb = 0; fb < kFb; ++fb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = f0 + 32 * fb + 8 * g + 4 * hb;
        if (f < a.n_feat)
          *reinterpret_cast<floatx4*>(dst + f) =
              floatx4{acc[fb][4 * g], acc[fb][4 * g + 1], acc[fb][4 * g + 2], acc[fb][4 * g + 3]};
      }
    return;
  }

  // modes 0 and 2: stage the wave's 32 token rows in LDS (its own rows: no other wave reads
  // them), then store whole rows, 16 bytes per lane
  wait_vmcnt<0>();
  lds_barrier();  // every wave is done with the operand slots
  constexpr int kRow = G::kOutRow, kStride = G::kOutStride;
  char* orow = smem + (size_t)wave * 32 * kStride;
#pragma unroll
  for (int fb = 0; fb < kFb; ++fb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int fl = 32 * fb + 8 * g + 4 * hb;  // feature within the tile
      if (G::kF32Out)
        *reinterpret_cast<floatx4*>(orow + r * kStride + fl * 4) =
            floatx4{acc[fb][4 * g], acc[fb][4 * g + 1], acc[fb][4 * g + 2], acc[fb][4 * g + 3]};
      else
        *reinterpret_cast<u32x2*>(orow + r * kStride + fl * 2) =
            u32x2{pack2(acc[fb][4 * g], acc[fb][4 * g + 1]), pack2(acc[fb][4 * g + 2], acc[fb][4 * g + 3])};
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are done before its reads
  constexpr int kPieces = kRow / 16;   // 16-byte pieces per row
  const int nvalid = G::kF32Out ? min(kFeat, a.n_feat - f0) * 4 / 16 : kPieces;
#pragma unroll
  for (int i = 0; i < 32 * kPieces / 64; ++i) {
    const int idx = i * 64 + lane;
    const int rr = idx / kPieces, pc = idx % kPieces;
    const int t = tb0 + 32 * wave + rr;
    if (t >= a.tokens || pc >= nvalid) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(orow + rr * kStride + pc * 16);
    char* dst;
    if (G::kF32Out)
      dst = reinterpret_cast<char*>(a.part + ((size_t)split * a.tokens + t) * a.n_feat + f0) + pc * 16;
    else
      dst = reinterpret_cast<char*>(a.q_nope + ((size_t)t * a.n_q + head) * kPrLatent + f0) + pc * 16;
    *reinterpret_cast<u32x4*>(dst) = v;
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
  // the V4 form: a 512-wide latent row, normalised whole, its last 64 channels rotated in place
  const int nf = a.q_rank + kPrLatent + (a.kv_inside ? 0 : kPrRope);
  const int nq4 = a.q_rank / 4, nkv4 = nq4 + kPrLatent / 4, nch = nf / 4;
  floatx4 v[kNormMaxChunks];
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) v[i] = floatx4{};
  // the splits' partials: the chunks' loads of one split are independent, and the split loop
  // is unrolled, so all of them are in flight together
#pragma unroll 4
  for (int s = 0; s < a.n_split; ++s) {
    const float* src = a.part + ((size_t)s * a.tokens + t) * nf;
#pragma unroll
    for (int i = 0; i < kNormMaxChunks; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (c < nch) v[i] += *reinterpret_cast<const floatx4*>(src + 4 * c);
    }
  }
  float ssq = 0.f, skv = 0.f;
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = threadIdx.x + i * kThreads;
    const float sq = v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    if (c < nq4)
      ssq += sq;
    else if (c < nkv4)
      skv += sq;
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
      if (a.cq_out) *reinterpret_cast<u32x2*>(a.cq_out + (size_t)t * a.q_rank + 4 * c) = hi;
    } else if (c < nkv4) {
      const int j = 4 * (c - nq4);
      floatx4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = v[i][e] * inv_kv * bf16_value(gk[j + e]);
      const int jr = j - (kPrLatent - kPrRope);  // V4: the row's own rotary channels
      *reinterpret_cast<u32x2*>(a.kv_nope + (size_t)t * kPrLatent + j) =
          a.kv_inside && jr >= 0 ? rope4(y, p, a.rope_positions, a.rope_cos, a.rope_sin, jr >> 1)
                                 : u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
    } else {
      const int j = 4 * (c - nkv4);
      *reinterpret_cast<u32x2*>(a.kv_rope + (size_t)t * kPrRope + j) =
          rope4(v[i], p, a.rope_positions, a.rope_cos, a.rope_sin, j >> 1);
    }
  }
}

// One 128-wide vector per wave pass: lane L holds channels L and L + 64. Channel 64 + 2i and
// 65 + 2i (lanes 2i and 2i + 1, second register) turn by the angle of column i of row p (zeros
// outside the tables); then, with rotate, the Sylvester Hadamard transform scaled by
// 1/sqrt(128): the stride-64 butterfly within the lane, the strides 32 .. 1 across lanes.
__device__ __forceinline__ void rope_hadamard128(float (&y)[2], int lane, int p, const IndexerFinishArgs& a) {
  const float partner = __shfl_xor(y[1], 1, 64);
  if (p < 0 || p >= a.rope_positions) {
    y[1] = 0.0f;
  } else {
    const int i = lane >> 1;
    const float co = a.rope_cos[(size_t)p * 32 + i], si = a.rope_sin[(size_t)p * 32 + i];
    y[1] = (lane & 1) ? fmaf(partner, si, y[1] * co) : fmaf(-partner, si, y[1] * co);
  }
  if (a.rotate) {
    const float u0 = y[0] + y[1], u1 = y[0] - y[1];
    y[0] = u0;
    y[1] = u1;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float q = __shfl_xor(y[k], d, 64);
        y[k] = (lane & d) ? q - y[k] : y[k] + q;
      }
    }
    y[0] *= 0.08838834764831845f;  // 1/sqrt(128)
    y[1] *= 0.08838834764831845f;
  }
}

__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// One workgroup (4 waves) per token: wave w takes heads w, w + 4, ... of the query; wave 0 then
// the key (LayerNorm over its 128 channels), wave 1 the head weights.
// One wave per job of a token: n_heads query heads, then the key, then the head weights (jobs
// t * (n_heads + 2) + j), so that the token's 64 transforms run on 64 waves instead of one
// workgroup's four; no job shares data with another.
__global__ void __launch_bounds__(kThreads) indexer_finish_kernel(const IndexerFinishArgs a) {
  const int lane = threadIdx.x & 63;
  const int per_token = a.n_heads + 2;
  const int64_t item = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (item >= (int64_t)a.tokens * per_token) return;  // whole waves only
  const int t = (int)(item / per_token);
  const int j = (int)(item - (int64_t)t * per_token);
  const int p = a.positions[t];
  const int nq = a.n_heads * 128;
  const int nkw = 128 + a.n_heads;
  if (j < a.n_heads) {
    const int h = j;
    float y[2] = {0.0f, 0.0f};
    for (int s = 0; s < a.split_q; ++s) {
      const float* src = a.part_q + ((size_t)s * a.tokens + t) * nq + h * 128;
      y[0] += src[lane];
      y[1] += src[64 + lane];
    }
    rope_hadamard128(y, lane, p, a);
    uint16_t* dst = a.q_index + ((size_t)t * a.n_heads + h) * 128;
    dst[lane] = bf16_bits(y[0]);
    dst[64 + lane] = bf16_bits(y[1]);
  } else if (j == a.n_heads) {
    float y[2] = {0.0f, 0.0f};
    for (int s = 0; s < a.split_kw; ++s) {
      const float* src = a.part_kw + ((size_t)s * a.tokens + t) * nkw;
      y[0] += src[lane];
      y[1] += src[64 + lane];
    }
    float sum = y[0] + y[1];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
    const float mu = sum * (1.0f / 128.0f);
    const float d0 = y[0] - mu, d1 = y[1] - mu;
    float sq = d0 * d0 + d1 * d1;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sq += __shfl_xor(sq, d, 64);
    const float inv = 1.0f / sqrtf(sq * (1.0f / 128.0f) + a.eps);
    const __bf16* g = reinterpret_cast<const __bf16*>(a.ln_gamma);
    const __bf16* b = reinterpret_cast<const __bf16*>(a.ln_beta);
    y[0] = d0 * inv * (float)g[lane] + (float)b[lane];
    y[1] = d1 * inv * (float)g[64 + lane] + (float)b[64 + lane];
    rope_hadamard128(y, lane, p, a);
    a.k_index[(size_t)t * 128 + lane] = bf16_bits(y[0]);
    a.k_index[(size_t)t * 128 + 64 + lane] = bf16_bits(y[1]);
  } else {
    for (int h = lane; h < a.n_heads; h += 64) {
      float w = 0.0f;
      for (int s = 0; s < a.split_kw; ++s) w += a.part_kw[((size_t)s * a.tokens + t) * nkw + 128 + h];
      a.weights[(size_t)t * a.n_heads + h] = w * a.w_scale;
    }
  }
}

// The V4 query heads: one wave per (token, head) sums the up-projection's k-split partials of
// the head's 512 channels (lane L holds channels 8L .. 8L + 7), normalises them with unit weight
// (the page's second RMSNorm), rotates the last 64 channels in place (lanes 56 .. 63: lane L's
// pairs are table columns 4(L - 56) .. + 3) and stores the row as bf16, 16 bytes per lane.
__global__ void __launch_bounds__(kThreads) prolog_v4_head_kernel(const PrologV4HeadArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);  // t * n_q + h
  if (item >= (int64_t)a.tokens * a.n_q) return;  // whole waves only
  const int t = (int)(item / a.n_q), h = (int)(item - (int64_t)t * a.n_q);
  floatx4 v0 = floatx4{}, v1 = floatx4{};
  for (int s = 0; s < a.n_split; ++s) {
    const float* src = a.part + ((size_t)s * a.tokens + t) * a.n_feat + (size_t)h * kPrLatent + 8 * lane;
    v0 += *reinterpret_cast<const floatx4*>(src);
    v1 += *reinterpret_cast<const floatx4*>(src + 4);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += v0[e] * v0[e] + v1[e] * v1[e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.0f / sqrtf(ss / (float)kPrLatent + a.eps);
  v0 *= inv;
  v1 *= inv;
  u32x4 out;
  if (lane >= (kPrLatent - kPrRope) / 8) {
    const int p = a.positions[t];
    const int i = 4 * (lane - (kPrLatent - kPrRope) / 8);
    const u32x2 r0 = rope4(v0, p, a.rope_positions, a.rope_cos, a.rope_sin, i);
    const u32x2 r1 = rope4(v1, p, a.rope_positions, a.rope_cos, a.rope_sin, i + 2);
    out = u32x4{r0[0], r0[1], r1[0], r1[1]};
  } else {
    out = u32x4{pack2(v0[0], v0[1]), pack2(v0[2], v0[3]), pack2(v1[0], v1[1]), pack2(v1[2], v1[3])};
  }
  *reinterpret_cast<u32x4*>(a.q + (size_t)item * kPrLatent + 8 * lane) = out;
}

}  // namespace

hipError_t launch_indexer_finish(const IndexerFinishArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.tokens * (a.n_heads + 2);
  const int per = kThreads / 64;
  hipLaunchKernelGGL(indexer_finish_kernel, dim3((unsigned)((waves + per - 1) / per)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prolog_gemm(const PrologGemmArgs& a, int mode, hipStream_t stream) {
  const int feat = 32 * prolog_feat_blocks(mode);
  int grid;
  if (mode == 2)
    grid = a.tok_blocks * a.n_q * (kPrLatent / feat);
  else
    grid = a.tok_blocks * ((a.n_feat + feat - 1) / feat) * a.n_split;
  if (mode == 0)
    hipLaunchKernelGGL((prolog_gemm_kernel<0, kPrFb0>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (mode == 1)
    hipLaunchKernelGGL((prolog_gemm_kernel<1, kPrFb1>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (mode == 2)
    hipLaunchKernelGGL((prolog_gemm_kernel<2, kPrFb2>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((prolog_gemm_kernel<3, kPrFb3>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prolog_v4_head(const PrologV4HeadArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.tokens * a.n_q;
  const int per = kThreads / 64;
  hipLaunchKernelGGL(prolog_v4_head_kernel, dim3((unsigned)((waves + per - 1) / per)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prolog_norm(const PrologNormArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prolog_norm_kernel, dim3(a.tokens), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfa
