// Sparse flash attention over a paged MLA latent cache: HIP kernels for gfx950 (CDNA4).
//
// What is computed is the operation described in "DeepSeek V3/V2 Sparse Flash Attention with
// Quantization" (sections "Algorithm overview", "Implementation notes: compute pipeline", "INT8
// quantisation path", "Flash online softmax update"): for every query token, gather the top-k
// latent rows through the block table, S = [q_nope|q_rope] . [k_nope|k_rope]^T, softmax of
// scale*S, times V = k_nope. How it is computed here is a gfx950 design of its own:
//
//   * A workgroup of 4 waves owns one (token, top-k partition, head group). A head group is 64
//     of the query heads that share the single latent KV head; each wave holds 16 of them. The
//     two head groups of a 128-head token are adjacent work items, so they run on the same XCD
//     and the second one's gather mostly hits that XCD's L2.
//   * Resolve + compaction: the partition's slots are resolved (index -> block_table -> row),
//     masked slots are dropped and the valid rows are packed in order into an LDS list. Tiles
//     are then dense: padding costs no loads and no MFMA, and a tile of invalid slots never runs.
//   * Gather: each 32-row tile is fetched with LDS-DMA (global_load_lds_dwordx4). One wave
//     instruction moves one 1 KB nope row, or eight 128 B rope rows, fully coalesced, with no
//     VGPR staging. Four LDS stages keep three tiles in flight while a fourth is computed. INT8
//     rows are fetched to registers a tile ahead instead, dequantised (fp32 multiply by the
//     group scale, round-to-nearest-even to bf16) and written into the same bf16 LDS layout.
//   * S^T = K . Q^T with v_mfma_f32_16x16x32_bf16: keys on M, heads on N, d as the reduction.
//     Q sits in registers for the whole partition. Each lane then holds one head and 8 of a
//     tile's 32 keys, so the softmax row max and row sum need two cross-lane steps.
//   * Online softmax over tiles (running max / running sum). The running max is only moved
//     when a tile's max exceeds it by more than 2^8 (exp2 domain), so O is rescaled rarely; the
//     final O / l is unchanged.
//   * O^T += V^T . P^T, again 16x16x32 MFMA. P^T comes straight from the S^T accumulator
//     registers (no shuffle). V^T fragments are read from the row-major K tile with
//     ds_read_b64_tr_b16 (LDS transpose read), so no transposed copy exists. P is split into
//     bf16 hi + lo parts, two MFMAs on the same V fragment, so it keeps about 16 significant
//     bits instead of 8: a single bf16 P does not meet the 5e-3 / 1e-4 accuracy standard when
//     few keys carry the weight.
//   * Partitions of one (token, head group) merge in the same kernel: each writes its
//     unnormalised O, its running max and its running sum. The last to arrive (counted with a
//     device-scope atomic) combines all of them in partition order, so the result does not
//     depend on arrival order: O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j. This is the
//     prefill update rule applied across partitions.
//   * Work items are mapped so that consecutive logical ids land on the same XCD and share its
//     L2: the hardware deals workgroups to the 8 XCDs round-robin.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sfa_internal.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4_t;

// LDS layout of one pipeline stage (one 32-row tile):
//   nope: 32 rows x 1024 B. The 16-byte chunk c of row k sits at chunk c ^ nope_swz(k) (the XOR
//         only touches the low 4 bits of the chunk index). With this swizzle, neither the
//         16-byte reads of the QK^T operand (16 rows, same chunk) nor the 8-byte transpose
//         reads of the PV operand (8 rows x 2 chunks) repeat a bank within one LDS cycle.
//   rope: 32 rows x 128 B, chunk c of row k at c ^ rope_swz(k). One DMA instruction fills eight
//         consecutive rope rows.
constexpr int kNopeRowBytes = kNope * 2;
constexpr int kRopeRowBytes = kRope * 2;
constexpr int kNopeTileBytes = kTile * kNopeRowBytes;
constexpr int kRopeTileBytes = kTile * kRopeRowBytes;
constexpr int kStageBytes = kNopeTileBytes + kRopeTileBytes;
constexpr int kStagesBf16 = 4;
constexpr int kStagesInt8 = 2;
constexpr int kDmaPerTile = 9;             // per wave: 8 nope rows + 1 rope instruction
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p stays <= 256 between rescales
constexpr int kQSteps = (kNope + kRope) / 32;  // 18 MFMA k-steps over d
// LDS operand loads kept in flight ahead of the MFMA that consumes them
constexpr int kQkDepth = 6;
constexpr int kPvDepth = 4;

__device__ __forceinline__ int nope_swz(int key) { return ((key & 7) << 1) | ((key >> 3) & 1); }
__device__ __forceinline__ int rope_swz(int key) { return (key >> 1) & 7; }

// LDS-DMA of 16 bytes per lane: lane L's bytes land at lds_addr + 16*L. lds_addr must be
// wave-uniform (it goes through M0). Issued from inline asm so that the compiler does not
// wait for the whole vector-memory queue before every LDS read. Completion is tracked
// explicitly with wait_vmcnt, and cross-wave visibility with lds_barrier.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(lds_addr)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS traffic only. Outstanding global loads (register prefetch,
// LDS-DMA into other stages) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ shortx4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(lds_char_t*)p);
}

template <bool kInt8>
__global__ void __launch_bounds__(kThreads, 1) sfa_attention_kernel(const KernelArgs a) {
  constexpr int kStages = kInt8 ? kStagesInt8 : kStagesBf16;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  __shared__ int32_t s_rows[kMaxSlots];
  __shared__ int32_t s_wcnt[kWaves];
  __shared__ int32_t s_last;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;  // row (A operand) or column (B operand, result) of the 16x16 MFMA
  const int kg = lane >> 4; // k-group of an operand / row quad of a result

  // ---- work item: XCD-aware remap of the workgroup id, then (token, partition, head group)
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int per_xcd = nwg >> 3;
  int lid = bid;
  if (per_xcd > 0 && bid < (per_xcd << 3)) lid = (bid & 7) * per_xcd + (bid >> 3);
  const int hg = lid % a.head_groups;
  lid /= a.head_groups;
  int t = lid / a.n_splits;
  const int sp = lid - t * a.n_splits;
  if (a.reverse) t = a.n_tokens - 1 - t;
  const int b = t / a.s1;

  const int h0 = hg * kHeadsPerGroup + wave * kHeadsPerWave;  // first head of this wave
  const bool wave_active = h0 < a.n_q;                         // wave-uniform
  const int h = h0 + n;                                         // this lane's head
  const bool head_ok = h < a.n_q;

  // ---- Q^T fragments (B operand, k = d): lane (n, kg) holds d in [32c + 8kg, 32c + 8kg + 8).
  // Issued first so that their latency overlaps the slot resolution below.
  bf16x8 qf[kQSteps];
  {
    const bf16x8 zero = {};
    const int64_t qrow = (int64_t)t * a.n_q + (head_ok ? h : 0);
    const bf16x8* qn = reinterpret_cast<const bf16x8*>(a.q_nope + qrow * kNope);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(a.q_rope + qrow * kRope);
#pragma unroll
    for (int c = 0; c < 16; ++c) qf[c] = head_ok ? qn[4 * c + kg] : zero;
#pragma unroll
    for (int c = 0; c < 2; ++c) qf[16 + c] = head_ok ? qr[4 * c + kg] : zero;
    // Q is only ever an MFMA B operand, which may come from AGPRs: pin it there and leave the
    // architectural VGPRs to the in-flight LDS operands of the MFMA pipelines.
#pragma unroll
    for (int c = 0; c < kQSteps; ++c) asm volatile("" : "+a"(qf[c]));
  }

  // ---- resolve this partition's slots and compact the valid rows into s_rows, in slot order.
  // Thread T owns the contiguous slots [8T, 8T+8) of the partition (a partition holds at most
  // 2048 = 256 x 8 slots): all index loads are issued together, then all block-table loads,
  // then one workgroup-wide exclusive scan of the per-thread valid counts places the rows.
  static_assert(kMaxSlots == kThreads * 8, "one pass of 8 slots per thread covers a partition");
  const int lim = min(a.act[b], a.mb * kBlock);
  const int k0 = sp * a.chunk;
  const int nslot = max(0, min(a.topk, k0 + a.chunk) - k0);
  const int32_t* idx = a.topk_idx + (int64_t)t * a.topk + k0;
  const int32_t* btab = a.block_table + (int64_t)b * a.mb;
  int jv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = 8 * tid + i;
    jv[i] = k < nslot ? idx[k] : -1;
  }
  int rowv[8];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = jv[i];
    const bool in = j >= 0 && j < lim;
    const int blk = in ? btab[j >> 7] : -1;
    const int64_t r = (int64_t)blk * kBlock + (j & (kBlock - 1));
    const bool v = in && blk >= 0 && r < a.num_rows;
    rowv[i] = v ? (int)r : -1;
    cnt += v ? 1 : 0;
  }
  // inclusive scan of cnt across the wave, then across waves through LDS
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  if (lane == 63) s_wcnt[wave] = incl;
  lds_barrier();
  int off = incl - cnt, n_valid = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_wcnt[w];
    off += (w < wave) ? c : 0;
    n_valid += c;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (rowv[i] >= 0) s_rows[off++] = rowv[i];
  }
  lds_barrier();
  const int ntiles = (n_valid + kTile - 1) / kTile;

  floatx4 oacc[32];  // O^T block db: lane (n, kg) holds d = 16*db + 4*kg + r of head h
#pragma unroll
  for (int db = 0; db < 32; ++db) oacc[db] = floatx4{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const uint32_t smem_lds = (uint32_t)(uintptr_t)((lds_char_t*)smem);

  // ---- loaders
  // rope: lane L fetches chunk ((L & 7) ^ rope_swz(key)) of key = 8*wave + L/8.
  auto issue_rope = [&](int tile, int stage) __attribute__((always_inline)) {
    const int key = wave * 8 + (lane >> 3);
    const int slot = min(tile * kTile + key, n_valid - 1);
    const int row = s_rows[slot];
    const char* src = reinterpret_cast<const char*>(a.k_rope) + (int64_t)row * kRopeRowBytes +
                      16 * ((lane & 7) ^ rope_swz(key));
    dma16(src, __builtin_amdgcn_readfirstlane(smem_lds + stage * kStageBytes + kNopeTileBytes +
                                              wave * 8 * kRopeRowBytes));
  };
  // bf16 nope: wave w moves rows 8w..8w+7 of the tile, one 1 KB row per instruction; lane L
  // fills physical chunk L, i.e. fetches logical chunk L ^ nope_swz(key). Slots past n_valid
  // repeat the last valid row; their scores are masked to -inf, so they contribute exactly zero.
  auto issue_nope_bf16 = [&](int tile, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int key = wave * 8 + k;
      const int slot = min(tile * kTile + key, n_valid - 1);
      const int row = s_rows[slot];
      const char* src = reinterpret_cast<const char*>(a.k_nope) + (int64_t)row * kNopeRowBytes +
                        16 * (lane ^ nope_swz(key));
      dma16(src, __builtin_amdgcn_readfirstlane(smem_lds + stage * kStageBytes + key * kNopeRowBytes));
    }
  };
  // int8 nope: lane L holds columns [8L, 8L+8) of rows 8w..8w+7 and the scale of group L/16.
  uint2 q8[8];
  float sc8[8];
  auto load_nope_int8 = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int key = wave * 8 + k;
      const int slot = min(tile * kTile + key, n_valid - 1);
      const int row = s_rows[slot];
      q8[k] = *reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(a.k_nope) +
                                              (int64_t)row * kNope + 8 * lane);
      sc8[k] = a.k_scales[(int64_t)row * 4 + (lane >> 4)];
    }
  };
  // Dequant: code -> fp32 (exact), times the fp32 group scale (RNE), -> bf16 (RNE); the
  // 16-byte chunk of columns [8L, 8L+8) is chunk L of the row, stored swizzled.
  auto store_nope_int8 = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int key = wave * 8 + k;
      const uint32_t lo = q8[k].x, hi = q8[k].y;
      const float s = sc8[k];
      uint4 v;
      v.x = pack_bf16x2((float)(int8_t)(lo)*s, (float)(int8_t)(lo >> 8) * s);
      v.y = pack_bf16x2((float)(int8_t)(lo >> 16) * s, (float)(int8_t)(lo >> 24) * s);
      v.z = pack_bf16x2((float)(int8_t)(hi)*s, (float)(int8_t)(hi >> 8) * s);
      v.w = pack_bf16x2((float)(int8_t)(hi >> 16) * s, (float)(int8_t)(hi >> 24) * s);
      *reinterpret_cast<uint4*>(smem + stage * kStageBytes + key * kNopeRowBytes + 16 * (lane ^ nope_swz(key))) = v;
    }
  };

  // ---- one tile: S^T = K Q^T, online softmax, O^T += V^T P^T
  // QK^T A operand: lane (n, kg) reads key 16*kb + n, logical chunk 4c + kg.
  // PV A operand (transpose read, instruction half hh): lane (kg, j = n) points at key
  // 16*hh + 4*kg + j/4 and column 16*db + 4*(j & 3); it receives column 16*db + j of keys
  // 16*hh + 4*kg + 0..3, which are exactly the keys its P^T operand holds.
  const int tr_key = 4 * kg + (n >> 2);
  const int tr_swz = nope_swz(tr_key);  // the same for tr_key + 16
  const int tr_sub = (n & 3);           // 4-column group inside the 16-column block

  auto compute_tile = [&](int tile, int stage) __attribute__((always_inline)) {
    const char* ks = smem + stage * kStageBytes;
    const char* rs = ks + kNopeTileBytes;
    floatx4 s[2] = {floatx4{}, floatx4{}};
    // A operand of step c (= 2*kstep + kb): key 16*kb + n, logical chunk 4*kstep + kg. Loads run
    // two MFMAs ahead of their use, and each step is fenced so the scheduler keeps that shape.
    auto qk_operand = [&](int c) __attribute__((always_inline)) -> bf16x8 {
      const int kstep = c >> 1, kb = c & 1;
      const int key = 16 * kb + n;
      if (kstep < 16)
        return *reinterpret_cast<const bf16x8*>(ks + key * kNopeRowBytes + 16 * ((4 * kstep + kg) ^ nope_swz(key)));
      return *reinterpret_cast<const bf16x8*>(rs + key * kRopeRowBytes + 16 * ((4 * (kstep - 16) + kg) ^ rope_swz(key)));
    };
    constexpr int kQkOps = 2 * kQSteps;
    bf16x8 qa[kQkDepth];
#pragma unroll
    for (int c = 0; c < kQkDepth; ++c) qa[c] = qk_operand(c);
#pragma unroll
    for (int c = 0; c < kQkOps; ++c) {
      const bf16x8 cur = qa[c % kQkDepth];
      if (c + kQkDepth < kQkOps) qa[c % kQkDepth] = qk_operand(c + kQkDepth);
      s[c & 1] = mfma16(cur, qf[c >> 1], s[c & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // result s[kb][r] holds key 16*kb + 4*kg + r of the tile, head h
    const int nk = n_valid - tile * kTile;
    float p[8];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * kb + 4 * kg + r;
        const float x = key < nk ? s[kb][r] * a.scale_log2 : -INFINITY;
        p[4 * kb + r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = mt > m_run + kRescaleThreshold;
    if (__any(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        oacc[db] *= alpha;  // one block at a time keeps the AGPR<->VGPR round trip short
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run *= alpha;
      m_run = m_new;
    }
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(p[i] - m_run);
      ls += p[i];
    }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run += ls;

    // P^T operand: lane (n, kg) element i is key 4kg + i (i < 4) or 16 + 4kg + (i - 4).
    // hi = bf16(p), lo = bf16(p - hi).
    bf16x8 ph, pl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 hb = (__bf16)p[i];
      ph[i] = hb;
      pl[i] = (__bf16)(p[i] - (float)hb);
    }

    auto pv_operand = [&](int db) __attribute__((always_inline)) -> bf16x8 {
      const int chunk = 2 * db + (tr_sub >> 1);
      const int off = 16 * (chunk ^ tr_swz) + 8 * (tr_sub & 1);
      const shortx4 v0 = lds_tr16(ks + tr_key * kNopeRowBytes + off);
      const shortx4 v1 = lds_tr16(ks + (tr_key + 16) * kNopeRowBytes + off);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 va[kPvDepth];
#pragma unroll
    for (int db = 0; db < kPvDepth; ++db) va[db] = pv_operand(db);
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const bf16x8 cur = va[db % kPvDepth];
      if (db + kPvDepth < 32) va[db % kPvDepth] = pv_operand(db + kPvDepth);
      oacc[db] = mfma16(cur, ph, oacc[db]);
      oacc[db] = mfma16(cur, pl, oacc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop over tiles
  if (ntiles > 0) {
    if constexpr (!kInt8) {
#pragma unroll
      for (int j = 0; j < kStages - 1; ++j) {
        if (j < ntiles) {
          issue_nope_bf16(j, j);
          issue_rope(j, j);
        }
      }
      for (int i = 0; i < ntiles; ++i) {
        // tile i has landed once at most (tiles queued after it) x kDmaPerTile loads remain
        const int younger = min(kStages - 2, ntiles - 1 - i);
        if (younger >= 2)
          wait_vmcnt<2 * kDmaPerTile>();
        else if (younger == 1)
          wait_vmcnt<kDmaPerTile>();
        else
          wait_vmcnt<0>();
        lds_barrier();  // every wave's part of tile i is in LDS; tile i-1's stage is free
        if (i + kStages - 1 < ntiles) {
          issue_nope_bf16(i + kStages - 1, (i + kStages - 1) % kStages);
          issue_rope(i + kStages - 1, (i + kStages - 1) % kStages);
        }
        if (wave_active) compute_tile(i, i % kStages);
      }
    } else {
      issue_rope(0, 0);
      load_nope_int8(0);
      for (int i = 0; i < ntiles; ++i) {
        wait_vmcnt<0>();
        store_nope_int8(i & 1);
        lds_barrier();
        if (i + 1 < ntiles) {
          issue_rope(i + 1, (i + 1) & 1);
          load_nope_int8(i + 1);
        }
        if (wave_active) compute_tile(i, i & 1);
      }
    }
  }

  // ---- epilogue: oacc[db][r] is column d = 16*db + 4*kg + r of head h
  if (a.n_splits == 1) {
    if (wave_active && head_ok) {
      const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
      uint16_t* o = a.out + ((int64_t)t * a.n_q + h) * kNope + 4 * kg;
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        uint2 v;
        v.x = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
        v.y = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * db) = v;
      }
    }
    return;
  }

  // Partial of (t, hg, sp) in register-image order: [wave][db][lane] float4.
  const int S = a.n_splits;
  const int64_t grp_item = (int64_t)t * a.head_groups + hg;  // (token, head group)
  floatx4* part = reinterpret_cast<floatx4*>(a.part_o);
  if (wave_active) {
    floatx4* po = part + ((grp_item * S + sp) * kWaves + wave) * (32 * 64);
#pragma unroll
    for (int db = 0; db < 32; ++db) po[db * 64 + lane] = oacc[db];
    if (kg == 0) {
      float* ml = a.part_ml + ((grp_item * S + sp) * kHeadsPerGroup + wave * kHeadsPerWave + n) * 2;
      ml[0] = m_run;
      ml[1] = l_run;
    }
  }
  __threadfence();  // release: this partition's partial is visible device-wide
  lds_barrier();
  if (tid == 0) s_last = (atomicAdd(a.counters + grp_item, 1) == S - 1) ? 1 : 0;
  lds_barrier();
  if (!s_last) return;
  __threadfence();  // acquire: the other partitions' partials

  if (wave_active) {
    float ws[kMaxSplits];
    float mmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      if (s < S) mmax = fmaxf(mmax, a.part_ml[((grp_item * S + s) * kHeadsPerGroup + wave * kHeadsPerWave + n) * 2]);
    }
    float lsum = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      ws[s] = 0.f;
      if (s < S) {
        const float* ml = a.part_ml + ((grp_item * S + s) * kHeadsPerGroup + wave * kHeadsPerWave + n) * 2;
        const float ms = ml[0];
        const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mmax);
        ws[s] = w;
        lsum += w * ml[1];
      }
    }
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    uint16_t* o = a.out + ((int64_t)t * a.n_q + h) * kNope + 4 * kg;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      floatx4 acc = {};
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) {
        if (s < S) {
          const floatx4 v = (s == sp) ? oacc[db] : part[((grp_item * S + s) * kWaves + wave) * (32 * 64) + db * 64 + lane];
          acc += ws[s] * v;
        }
      }
      if (head_ok) {
        uint2 v;
        v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * db) = v;
      }
    }
  }
}

// Clears the per-(token, head group) arrival counters before an attention launch that merges
// partitions. A fill kernel rather than a memset, so that the call can be recorded in a graph.
__global__ void __launch_bounds__(256) sfa_zero_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// rows_out[t, k] = physical row of slot k, or -1. The same predicate as the attention
// kernel's compaction step.
__global__ void __launch_bounds__(256) sfa_resolve_kernel(const ResolveArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_tokens * a.topk) return;
  const int t = (int)(i / a.topk);
  const int b = t / a.s1;
  const int lim = min(a.act[b], a.mb * kBlock);
  const int j = a.topk_idx[i];
  int out = -1;
  if (j >= 0 && j < lim) {
    const int blk = a.block_table[(int64_t)b * a.mb + (j >> 7)];
    const int64_t r = (int64_t)blk * kBlock + (j & (kBlock - 1));
    if (blk >= 0 && r < a.num_rows) out = (int)r;
  }
  a.rows_out[i] = out;
}

}  // namespace

hipError_t launch_attention(const KernelArgs& a, bool int8_cache, hipStream_t stream) {
  if (a.n_splits > 1) {
    const int64_t n = (int64_t)a.n_tokens * a.head_groups;
    int32_t* counters = a.counters;
    int64_t count = n;
    void* zargs[] = {&counters, &count};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&sfa_zero_kernel),
                                         dim3((unsigned)((n + 255) / 256)), dim3(256), zargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(a.n_tokens * a.n_splits * a.head_groups));
  const dim3 block(kThreads);
  KernelArgs copy = a;
  void* args[] = {&copy};
  const void* fn = int8_cache ? reinterpret_cast<const void*>(&sfa_attention_kernel<true>)
                              : reinterpret_cast<const void*>(&sfa_attention_kernel<false>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_resolve(const ResolveArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.n_tokens * a.topk;
  const dim3 grid((unsigned)((total + 255) / 256));
  const dim3 block(256);
  ResolveArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&sfa_resolve_kernel), grid, block, args, 0, stream);
}

}  // namespace sfa
