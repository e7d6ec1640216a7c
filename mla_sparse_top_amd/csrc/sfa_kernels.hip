// Sparse flash attention over a paged MLA latent cache: HIP kernels for gfx950 (CDNA4).
//
// What is computed is the operation described in "DeepSeek V3/V2 Sparse Flash Attention with
// Quantization" (sections "Algorithm overview", "Implementation notes: compute pipeline", "INT8
// quantisation path", "Flash online softmax update"): for every query token, gather the top-k
// latent rows through the block table, S = [q_nope|q_rope] . [k_nope|k_rope]^T, softmax of
// scale*S, times V = k_nope. How it is computed here is a gfx950 design of its own:
//
//   * A workgroup of 4 waves owns one (token, top-k partition, head group). A head group is 64
//     of the query heads that share the single latent KV head. The waves form two pairs; a pair
//     owns 32 heads, and its two waves split the work along d: wave "half" h computes the part
//     of the scores over its 288 columns of [nope|rope] (nope 256h..256h+255, rope 32h..32h+31)
//     and accumulates the output columns 256h..256h+255. The two partial score tiles are
//     summed through LDS, so both waves of a pair see the same scores and run the same softmax.
//     Every 32-key tile of K and V is thus read from LDS once per pair instead of once per wave,
//     and the MFMA is the 32x32x16 shape (32 keys x 32 heads).
//   * The two head groups of a 128-head token are adjacent work items, so they run on the same
//     XCD and the second one's gather mostly hits that XCD's L2.
//   * Resolve + compaction: the partition's slots are resolved (index -> block_table -> row),
//     masked slots are dropped and the valid rows are packed in order into an LDS list. Tiles
//     are then dense: padding costs no loads and no MFMA, and a tile of invalid slots never runs.
//   * Gather: each 32-row tile is fetched with LDS-DMA (global_load_lds_dwordx4) into one of
//     three LDS stages. One wave instruction moves one 1 KB nope row, or eight 128 B rope rows,
//     fully coalesced, with no VGPR staging. INT8 rows are fetched to registers instead,
//     dequantised (fp32 multiply by the group scale, round-to-nearest-even to bf16) and written
//     into the same bf16 LDS layout.
//   * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: keys on M, heads on N, d as the reduction.
//     Q sits in registers for the whole partition. Each lane then holds one head and 16 of a
//     tile's 32 keys, so the softmax row max and row sum need one cross-lane step.
//   * Online softmax over tiles (running max / running sum). The running max is only moved
//     when a tile's max exceeds it by more than 2^8 (exp2 domain), so O is rescaled rarely; the
//     final O / l is unchanged.
//   * O^T += V^T . P^T, again 32x32x16 MFMA. P^T comes straight from the S^T accumulator
//     registers (no shuffle). V^T fragments are read from the row-major K tile with
//     ds_read_b64_tr_b16 (LDS transpose read), so no transposed copy exists. P is split into
//     bf16 hi + lo parts, two MFMAs on the same V fragment, so it keeps about 16 significant
//     bits instead of 8: a single bf16 P does not meet the 5e-3 / 1e-4 accuracy standard when
//     few keys carry the weight.
//   * The loop is software-pipelined: while the MFMAs of the next tile's S^T run, the VALU
//     computes the current tile's softmax, and then the current tile's PV MFMAs run. One
//     workgroup barrier per tile.
//   * Partitions of one (token, head group) merge in the same kernel: each writes its
//     unnormalised O, its running max and its running sum. The last to arrive (counted with a
//     device-scope atomic) combines all of them in partition order, so the result does not
//     depend on arrival order: O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j. This is the
//     prefill update rule applied across partitions.
//   * Work items are mapped so that consecutive logical ids land on the same XCD and share its
//     L2: the hardware deals workgroups to the 8 XCDs round-robin.
//
// The MFMAs are issued from inline assembly so that the O accumulators stay in AGPRs and the
// score accumulators in VGPRs without register-file copies. The compiler does not look inside
// inline assembly for hazards, so the required wait states are written out next to each use.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "sfa_internal.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4_t;

// LDS layout of one pipeline stage (one 32-row tile):
//   nope: 32 rows x 1024 B. The 16-byte chunk c of row k sits at chunk c ^ nope_swz(k) (the XOR
//         only touches the low 4 bits of the chunk index). With this swizzle, neither the
//         16-byte reads of the QK^T operand (16 rows, same chunk) nor the 8-byte transpose
//         reads of the PV operand (4 rows x 2 chunks per 16 lanes) repeat a bank.
//   rope: 32 rows x 128 B, chunk c of row k at c ^ rope_swz(k).
constexpr int kNopeRowBytes = kNope * 2;
constexpr int kRopeRowBytes = kRope * 2;
constexpr int kNopeTileBytes = kTile * kNopeRowBytes;
constexpr int kRopeTileBytes = kTile * kRopeRowBytes;
constexpr int kStageBytes = kNopeTileBytes + kRopeTileBytes;
constexpr int kStages = 3;
constexpr int kXBytes = 64 * 16 * 4;           // one wave's partial S^T tile (64 lanes x 16 fp32)
constexpr float kRescaleThreshold = 8.0f;      // log2 units: p stays <= 256 between rescales
constexpr int kQkSteps = (kNope + kRope) / 32;  // 18 k-steps of 16 over a wave's 288 columns
constexpr int kQkDepth = 8;                    // LDS operand loads in flight ahead of the MFMA
constexpr int kPvDepth = 4;

static_assert(kStages * kStageBytes + 2 * kWaves * kXBytes + kMaxSlots * 4 + 64 <= 160 * 1024,
              "LDS budget of one workgroup");

__device__ __forceinline__ int nope_swz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }
__device__ __forceinline__ int rope_swz(int key) { return (key >> 1) & 7; }

// LDS-DMA of 16 bytes per lane: lane L's bytes land at lds_addr + 16*L. lds_addr must be
// wave-uniform (it goes through M0, which the asm saves and restores; M0 needs one wait state
// between its write and the DMA). Issued from inline asm so that the compiler does not wait
// for the whole vector-memory queue before every LDS read. Completion is tracked explicitly
// with wait_vmcnt, and cross-wave visibility with lds_barrier.
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

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset: used for the
// nope rows, where one instruction reads one whole cache row.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory");
}

// The same through a buffer resource (base, byte size): a cache row's byte offset fits in the
// 32-bit scalar offset whenever the pool is below 4 GiB, which saves the 64-bit address
// arithmetic per row. Up to three nope rows per call, with one M0 save and restore around them;
// the shift of the next row's offset fills the wait state after each M0 write.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint64_t nbytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  // dword 2: the size in bytes (callers keep it below 4 GiB); dword 3: the raw-buffer
  // configuration (32-bit data format, no swizzle, no stride)
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, (uint32_t)nbytes, 0x00020000u};
}
// Rows k0, k0 + 1, k0 + 2 of this wave's block of the tile: row k lands at lds_base + k * 1 KB.
template <int kK0>
__device__ __forceinline__ void dma16_rows3(const u32x4& rsrc, int r0, int r1, int r2, uint32_t v0, uint32_t v1,
                                            uint32_t v2, uint32_t lds_base) {
  uint32_t saved, o0, o1, o2;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_lshl_b32 %1, %8, 10\n\t"
      "s_add_u32 m0, %11, %12\n\t"
      "s_lshl_b32 %2, %9, 10\n\t"
      "buffer_load_dwordx4 %4, %7, %1 offen lds\n\t"
      "s_add_u32 m0, %11, %13\n\t"
      "s_lshl_b32 %3, %10, 10\n\t"
      "buffer_load_dwordx4 %5, %7, %2 offen lds\n\t"
      "s_add_u32 m0, %11, %14\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %6, %7, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved), "=&s"(o0), "=&s"(o1), "=&s"(o2)
      : "v"(v0), "v"(v1), "v"(v2), "s"(rsrc), "s"(r0), "s"(r1), "s"(r2), "s"(lds_base), "n"(kK0 * 1024),
        "n"((kK0 + 1) * 1024), "n"((kK0 + 2) * 1024)
      : "memory");
}
template <int kK0>
__device__ __forceinline__ void dma16_rows2(const u32x4& rsrc, int r0, int r1, uint32_t v0, uint32_t v1,
                                            uint32_t lds_base) {
  uint32_t saved, o0, o1;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_lshl_b32 %1, %6, 10\n\t"
      "s_add_u32 m0, %8, %9\n\t"
      "s_lshl_b32 %2, %7, 10\n\t"
      "buffer_load_dwordx4 %3, %5, %1 offen lds\n\t"
      "s_add_u32 m0, %8, %10\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %4, %5, %2 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved), "=&s"(o0), "=&s"(o1)
      : "v"(v0), "v"(v1), "s"(rsrc), "s"(r0), "s"(r1), "s"(lds_base), "n"(kK0 * 1024), "n"((kK0 + 1) * 1024)
      : "memory");
}
// One DMA instruction with a per-lane byte offset into the buffer (the rope rows: eight rows
// per instruction).
__device__ __forceinline__ void dma16_voff(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS traffic only. Outstanding global loads (the register
// staging of later tiles) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  // s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maximum, written as the builtin so
  // that the compiler's wait-count tracking knows the LDS queue is empty after it
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// S^T += K . Q^T steps: the accumulator in VGPRs, the K fragment in VGPRs (fresh from LDS), the
// Q^T fragment in AGPRs. Consecutive steps accumulate into the same registers, which the
// hardware chains back to back (an exactly overlapping accumulator needs no wait states); the
// chain starts from 0. The first step's leading pad covers a VALU write of an operand right
// before it. The later steps read only LDS-loaded K fragments, the Q registers (written once)
// and the chained accumulator, so they carry no pad; the build checks the generated code for a
// VALU write of an MFMA operand within two instructions before an unpadded MFMA.
__device__ __forceinline__ void mfma_qk_first(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_qk(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
// Before anything else reads the chain's result: a 32x32x16 result needs 12 wait states before
// a VALU or LDS read of it; this gives 20.
__device__ __forceinline__ void mfma_qk_drain(floatx16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
}

// O^T += V^T . P^T step on an AGPR-resident accumulator, tied in place, with no pad: its V^T
// operand comes from LDS or from register copies made before the tile barrier, and its P^T
// operands are converted several instructions ahead (the assembly test holds this).
__device__ __forceinline__ void mfma_pv(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// O *= alpha on the AGPR-resident accumulators, in place: each element is read to a VGPR,
// scaled and written back by inline asm, so no compiler-generated VALU ever touches O (which
// would make the compiler keep O in VGPRs and copy it around every tile). Pads: the last MFMA
// that wrote O needs 12 wait states before an AGPR read (20 given); the MFMA that next reads O
// as its accumulator needs 2 after the AGPR write (4 given).
template <int N>
__device__ __forceinline__ void rescale_agprs(floatx16 (&acc)[N], float alpha) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int d = 0; d < N; ++d) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float tmp;
      asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                   : "+a"(acc[d][r]), "=&v"(tmp)
                   : "v"(alpha));
    }
  }
  asm volatile("s_nop 3" ::: "memory");
}

// Pins the O accumulators to AGPRs at a point of the program (where O is carried from one tile
// to the next); without it the register allocator may carry O in VGPRs and copy it around.
template <int N>
__device__ __forceinline__ void pin_agprs(floatx16 (&acc)[N]) {
#pragma unroll
  for (int d = 0; d < N; ++d) asm volatile("" : "+a"(acc[d]));
}

// Before compiler-generated code reads O after the MFMAs: 20 wait states after the last write.
template <int N>
__device__ __forceinline__ void mfma_pv_drain(floatx16 (&acc)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
  pin_agprs(acc);
}

__device__ __forceinline__ shortx4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(lds_char_t*)p);
}

// Lanes l and l ^ 32 hold the same head: combine their values. v_permlane32_swap hands each lane
// its partner's value; both results are the same in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// An INT8 tile's nope rows on their way from HBM to LDS: this wave's 8 rows and their scales.
struct StagedInt8 {
  uint2 nope[8];
  float scale[8];
};

// kBufDma: cache rows (nope, rope, INT8 scales) are fetched through buffer resources with
// 32-bit byte offsets (pools below 4 Mi rows); otherwise through 64-bit global addresses.
// kWindow: the window variants' slot list (see KernelArgs), resolved here instead of read from
// topk_indices; the rest of the kernel is the same.
template <bool kInt8, bool kBufDma, bool kWindow>
__global__ void __launch_bounds__(kThreads, 1) sfa_attention_kernel(const KernelArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) char xbuf[2 * kWaves * kXBytes];
  __shared__ __attribute__((aligned(16))) int32_t s_rows[kMaxSlots];
  __shared__ int32_t s_wcnt[kWaves];
  __shared__ int32_t s_last;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int lane = tid & 63;
  const int n = lane & 31;  // row (A operand) or column (B operand, result) of the 32x32 MFMA
  const int g = lane >> 5;  // k-group of an operand / row-quad parity of a result
  const int pair = wave >> 1;
  const int half = wave & 1;

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

  const int hp0 = hg * kHeadsPerGroup + pair * kHeadsPerPair;  // first head of this pair
  const bool pair_active = hp0 < a.n_q;                         // wave-uniform
  const int h = hp0 + n;                                         // this lane's head
  const bool head_ok = h < a.n_q;

  // The scores are used as fma(S, c, -m) with c = |scale * log2 e|. A negative scale is moved
  // into Q by flipping the sign bits of its bf16 elements, which is exact.
  // Masked keys carry a score of -inf, which c * (-inf) keeps at -inf only for c > 0. A zero
  // scale is therefore raised to 1e-30: every |c * (x - m)| then stays far below 2^-24 for any
  // finite score, so each valid key still gets p = exp2(0) = 1 exactly, as with c = 0.
  const float c_scale = fmaxf(fabsf(a.scale_log2), 1e-30f);
  const uint32_t q_sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // ---- resolve this partition's slots and compact the valid rows into s_rows, in slot order.
  // Thread T owns the contiguous slots [8T, 8T+8) of the partition (a partition holds at most
  // 2048 = 256 x 8 slots): all index loads are issued together, then all block-table loads,
  // then one workgroup-wide exclusive scan of the per-thread valid counts places the rows.
  static_assert(kMaxSlots == kThreads * 8, "one pass of 8 slots per thread covers a partition");
  const int lim = min(a.act[b], a.mb * kBlock);
  const int k0 = sp * a.chunk;
  const int nslot = max(0, min(a.topk, k0 + a.chunk) - k0);
  const int32_t* btab = a.block_table + (int64_t)b * a.mb;
  int jv[8];
  bool livev[8];  // the slot names a live position of its cache
  int blkv[8];
  if constexpr (!kWindow) {
    const int32_t* idx = a.topk_idx + (int64_t)t * a.topk + k0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * tid + i;
      jv[i] = k < nslot ? idx[k] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = jv[i];
      livev[i] = j >= 0 && j < lim;
      blkv[i] = btab[livev[i] ? (j >> 7) : 0];
    }
  } else {
    // slot g < window: original-cache position p - window + 1 + g of the query at position
    // p = act[b] - s1 + s (negative when the window reaches below 0); slot g >= window:
    // compressed entry topk_idx[t][g - window] through the compressed block table
    const int p = a.act[b] - a.s1 + (t - b * a.s1);
    const int topk_cmp = a.topk - a.window;
    const int32_t* cidx = a.topk_idx + (int64_t)t * topk_cmp;
    const int lim_c = a.mb_cmp > 0 ? min(a.act_cmp[b], a.mb_cmp * kBlock) : 0;
    const int32_t* btab_c = a.block_table_cmp + (int64_t)b * a.mb_cmp;
    bool cmpv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * tid + i;
      const int gs = k0 + k;
      cmpv[i] = gs >= a.window;
      jv[i] = k >= nslot ? -1 : (cmpv[i] ? cidx[gs - a.window] : p - a.window + 1 + gs);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = jv[i];
      livev[i] = j >= 0 && j < (cmpv[i] ? lim_c : lim);
      blkv[i] = livev[i] ? (cmpv[i] ? btab_c : btab)[j >> 7] : -1;
    }
  }
  // ---- Q^T fragments (B operand, k = d): step c < 16 covers nope chunks 32*half + 2c + {0, 1},
  // steps 16 and 17 rope chunks 4*half + 2(c - 16) + {0, 1}; lane (n, g) holds chunk +g.
  // Issued after the index and block-table loads: load completion is counted in issue order,
  // so Q's 147 KB per token must not sit in front of the two dependent index round trips.
  // The loads are unconditional (a lane past n_q reads head 0's row) and the zeroing of such
  // lanes happens after the compaction: a conditional load would make the compaction's wait for
  // its own loads also wait for Q.
  uint4 qv[kQkSteps];
  {
    const int64_t qrow = (int64_t)t * a.n_q + (head_ok ? h : 0);
    const uint4* qn = reinterpret_cast<const uint4*>(a.q_nope + qrow * kNope);
    const uint4* qr = reinterpret_cast<const uint4*>(a.q_rope + qrow * kRope);
#pragma unroll
    for (int c = 0; c < 16; ++c) qv[c] = qn[32 * half + 2 * c + g];
#pragma unroll
    for (int c = 0; c < 2; ++c) qv[16 + c] = qr[4 * half + 2 * c + g];
  }
  int rowv[8];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = jv[i];
    const bool in = livev[i];
    const int blk = blkv[i];
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
  const int ntiles = (n_valid + kTile - 1) / kTile;
  int last_row = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (rowv[i] >= 0) {
      s_rows[off++] = rowv[i];
      last_row = rowv[i];
    }
  }
  // The thread that placed the last valid row repeats it up to the end of the last tile, so
  // every tile reads 32 real rows; the scores of the repeats are masked out.
  if (cnt > 0 && off == n_valid) {
    for (int q = n_valid; q < ntiles * kTile; ++q) s_rows[q] = last_row;
  }
  lds_barrier();

  bf16x8 qf[kQkSteps];
  {
    const uint32_t keep = head_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int c = 0; c < kQkSteps; ++c) {
      const uint4 v = {(qv[c].x ^ q_sign) & keep, (qv[c].y ^ q_sign) & keep, (qv[c].z ^ q_sign) & keep,
                       (qv[c].w ^ q_sign) & keep};
      qf[c] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // Q is only ever an MFMA B operand, which may come from AGPRs: keep it there and leave the
  // VGPRs to the in-flight LDS operands and the softmax.
#pragma unroll
  for (int c = 0; c < kQkSteps; ++c) asm volatile("" : "+a"(qf[c]));

  // O^T block dc: reg r holds column d = 256*half + 32*dc + 8*(r/4) + 4g + (r%4) of head h
  floatx16 oacc[8];
#pragma unroll
  for (int dc = 0; dc < 8; ++dc) oacc[dc] = floatx16{};
  pin_agprs(oacc);
  float m_run = -INFINITY;  // running max (exp2 domain) that p and O are currently relative to
  float l_run = 0.f;

  // ---- loaders: wave w carries rows 8w..8w+7 of each tile
  const uint32_t smem_lds = (uint32_t)(uintptr_t)((lds_char_t*)smem);
  // rope: lane L fetches chunk ((L & 7) ^ rope_swz(key)) of key = 8*wave + L/8.
  const u32x4 rs_nope = make_rsrc(a.k_nope, (uint64_t)a.num_rows * kNopeRowBytes);
  const u32x4 rs_rope = make_rsrc(a.k_rope, (uint64_t)a.num_rows * kRopeRowBytes);
  auto issue_rope = [&](int tile, uint32_t stage_off) __attribute__((always_inline)) {
    const int key = wave * 8 + (lane >> 3);
    const int row = s_rows[tile * kTile + key];
    const uint32_t chunk = 16 * ((lane & 7) ^ rope_swz(key));
    const uint32_t lds = smem_lds + stage_off + kNopeTileBytes + wave * 8 * kRopeRowBytes;
    if constexpr (kBufDma) {
      dma16_voff(rs_rope, (uint32_t)row * kRopeRowBytes + chunk, lds);
    } else {
      dma16(reinterpret_cast<const char*>(a.k_rope) + (int64_t)row * kRopeRowBytes + chunk, lds);
    }
  };
  // The wave's 8 rows of a tile, as wave-uniform values (one 32-byte broadcast read).
  auto tile_rows = [&](int tile, int (&rows)[8]) __attribute__((always_inline)) {
    const int4* rp = reinterpret_cast<const int4*>(s_rows + tile * kTile + wave * 8);
    const int4 r0 = rp[0], r1 = rp[1];
    rows[0] = __builtin_amdgcn_readfirstlane(r0.x);
    rows[1] = __builtin_amdgcn_readfirstlane(r0.y);
    rows[2] = __builtin_amdgcn_readfirstlane(r0.z);
    rows[3] = __builtin_amdgcn_readfirstlane(r0.w);
    rows[4] = __builtin_amdgcn_readfirstlane(r1.x);
    rows[5] = __builtin_amdgcn_readfirstlane(r1.y);
    rows[6] = __builtin_amdgcn_readfirstlane(r1.z);
    rows[7] = __builtin_amdgcn_readfirstlane(r1.w);
  };
  // bf16 nope: one 1 KB row per instruction; lane L fills physical chunk L, i.e. fetches
  // logical chunk L ^ nope_swz(key).
  // Rows [k0, k1) of the wave's eight; nope_voff[k] is lane L's physical chunk offset in row k.
  uint32_t nope_voff[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) nope_voff[k] = (uint32_t)(16 * (lane ^ nope_swz(wave * 8 + k)));
  auto issue_nope_rows = [&](const int (&rows)[8], uint32_t stage_off, int k0, int k1) __attribute__((always_inline)) {
    const uint32_t lds_base = smem_lds + stage_off + wave * 8 * kNopeRowBytes;
    if constexpr (kBufDma) {
      static_assert(kNopeRowBytes == 1024, "row offsets are formed as row << 10");
      if (k0 == 0 && k1 == 3) dma16_rows3<0>(rs_nope, rows[0], rows[1], rows[2], nope_voff[0], nope_voff[1], nope_voff[2], lds_base);
      if (k0 == 3 && k1 == 6) dma16_rows3<3>(rs_nope, rows[3], rows[4], rows[5], nope_voff[3], nope_voff[4], nope_voff[5], lds_base);
      if (k0 == 6 && k1 == 8) dma16_rows2<6>(rs_nope, rows[6], rows[7], nope_voff[6], nope_voff[7], lds_base);
    } else {
#pragma unroll
      for (int k = k0; k < k1; ++k) {
        const char* base = reinterpret_cast<const char*>(a.k_nope) + (int64_t)rows[k] * kNopeRowBytes;
        dma16_sbase(base, nope_voff[k], lds_base + k * kNopeRowBytes);
      }
    }
  };
  auto issue_nope_bf16 = [&](int tile, uint32_t stage_off) __attribute__((always_inline)) {
    int rows[8];
    tile_rows(tile, rows);
    issue_nope_rows(rows, stage_off, 0, 3);
    issue_nope_rows(rows, stage_off, 3, 6);
    issue_nope_rows(rows, stage_off, 6, 8);
  };
  // int8 nope: lane L holds columns [8L, 8L+8) of each row and the scale of their group L/16.
  StagedInt8 st8;
  // lane L loads bytes [8L, 8L+8) of the row and the scale of group L/16
  const __amdgpu_buffer_rsrc_t rb_code = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.k_nope), 0, kInt8 ? (int)(a.num_rows * kNope) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb_scale = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.k_scales), 0, kInt8 ? (int)(a.num_rows * 16) : 0, 0x00020000);
  auto load_int8_row = [&](int k, int row) __attribute__((always_inline)) {
    if constexpr (kBufDma) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rb_code, 8 * lane, row << 9, 0);
      st8.nope[k] = uint2{v[0], v[1]};
      st8.scale[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb_scale, 4 * (lane >> 4), row << 4, 0));
    } else {
      st8.nope[k] = *reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(a.k_nope) +
                                                    (int64_t)row * kNope + 8 * lane);
      st8.scale[k] = a.k_scales[(int64_t)row * 4 + (lane >> 4)];
    }
  };
  auto load_nope_int8 = [&](int tile) __attribute__((always_inline)) {
    int rows[8];
    tile_rows(tile, rows);
#pragma unroll
    for (int k = 0; k < 8; ++k) load_int8_row(k, rows[k]);
  };
  // Dequant: code -> fp32 (exact), times the fp32 group scale (RNE), -> bf16 (RNE); the 16-byte
  // chunk of columns [8L, 8L+8) is chunk L of the row, stored swizzled.
  auto store_nope_int8 = [&](uint32_t stage_off) __attribute__((always_inline)) {
    char* base = smem + stage_off;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int key = wave * 8 + k;
      const uint32_t lo = st8.nope[k].x, hi = st8.nope[k].y;
      const float sc = st8.scale[k];
      uint4 v;
      v.x = pack_bf16x2((float)(int8_t)(lo)*sc, (float)(int8_t)(lo >> 8) * sc);
      v.y = pack_bf16x2((float)(int8_t)(lo >> 16) * sc, (float)(int8_t)(lo >> 24) * sc);
      v.z = pack_bf16x2((float)(int8_t)(hi)*sc, (float)(int8_t)(hi >> 8) * sc);
      v.w = pack_bf16x2((float)(int8_t)(hi >> 16) * sc, (float)(int8_t)(hi >> 24) * sc);
      *reinterpret_cast<uint4*>(base + key * kNopeRowBytes + 16 * (lane ^ nope_swz(key))) = v;
    }
  };
  // Starts the fetch of a tile into a stage (INT8: the nope part into registers, written to the
  // stage by finish_tile).
  auto start_tile = [&](int tile, uint32_t stage_off) __attribute__((always_inline)) {
    if constexpr (kInt8) {
      load_nope_int8(tile);
    } else {
      issue_nope_bf16(tile, stage_off);
    }
    issue_rope(tile, stage_off);
  };
  // The same in three parts, so that it can be spread between MFMAs.
  int rows_next[8];
  auto start_tile_part = [&](int tile, uint32_t stage_off, int part) __attribute__((always_inline)) {
    if (part == 0) tile_rows(tile, rows_next);
    if constexpr (kInt8) {
#pragma unroll
      for (int k = 3 * part; k < min(8, 3 * part + 3); ++k) load_int8_row(k, rows_next[k]);
    } else {
      issue_nope_rows(rows_next, stage_off, 3 * part, min(8, 3 * part + 3));
    }
    if (part == 2) issue_rope(tile, stage_off);
  };
  // Completes it: waits for this wave's loads of the tile (INT8: and writes it to the stage).
  auto finish_tile = [&](uint32_t stage_off) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    if constexpr (kInt8) store_nope_int8(stage_off);
  };

  // ---- per-lane LDS offsets of the MFMA operands. The swizzle XOR only touches the low 4 bits
  // of a chunk index, so the QK^T operand of step c < 16 is qk_off[c & 7] + 256*(c >> 3) and the
  // PV operand of (dc, kb, q) is pv_off[q][dc & 3] + 256*(dc >> 2) + 16 KB*kb.
  // QK^T A operand: lane (n, g) reads key n, logical chunk 32*half + 2c + g.
  // PV A operand via transpose reads: lane (G = lane/16, j = lane%16) of read q points at key
  // 16*kb + 8*q + 4*g + j/4 and column 256*half + 32*dc + 16*(G & 1) + 4*(j & 3); it receives
  // column 32*dc + n of keys 16*kb + 8*q + 4*g + 0..3: the keys its P^T operand holds.
  int qk_off[8], rope_off[2], pv_off[2][4];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) qk_off[cc] = n * kNopeRowBytes + 512 * half + 16 * ((2 * cc + g) ^ nope_swz(n));
#pragma unroll
  for (int c = 0; c < 2; ++c)
    rope_off[c] = kNopeTileBytes + n * kRopeRowBytes + 16 * ((4 * half + 2 * c + g) ^ rope_swz(n));
  {
    const int j = lane & 15;
    const int tr_key = 4 * g + (j >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (j & 3);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int dl = 0; dl < 4; ++dl) {
        const int key = tr_key + 8 * q;
        const int col = 32 * dl + tr_col;  // inside the 128-column group, wave half added below
        pv_off[q][dl] = key * kNopeRowBytes + 512 * half + 16 * ((col >> 3) ^ nope_swz(key)) + 2 * (col & 7);
      }
    }
  }

  const char* smem_c = smem;
  auto qk_operand = [&](uint32_t stage_off, int c) __attribute__((always_inline)) -> bf16x8 {
    const char* ks = smem_c + stage_off;
    if (c < 16) return *reinterpret_cast<const bf16x8*>(ks + qk_off[c & 7] + 256 * (c >> 3));
    return *reinterpret_cast<const bf16x8*>(ks + rope_off[c - 16]);
  };
  // u = 8*kb + dc
  auto pv_operand = [&](uint32_t stage_off, int u) __attribute__((always_inline)) -> bf16x8 {
    const int dc = u & 7, kb = u >> 3;
    const char* ks = smem_c + stage_off + 256 * (dc >> 2) + 16 * kNopeRowBytes * kb;
    const shortx4 v0 = lds_tr16(ks + pv_off[0][dc & 3]);
    const shortx4 v1 = lds_tr16(ks + pv_off[1][dc & 3]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // The partial S^T tile exchange: [parity][wave][row quad][lane] float4.
  auto x_write = [&](int parity, const floatx16& s) __attribute__((always_inline)) {
    floatx4* xp = reinterpret_cast<floatx4*>(xbuf + (parity * kWaves + wave) * kXBytes) + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) xp[64 * q] = floatx4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
  };

  // S^T(tile) over this wave's half of d, into s
  auto qk_tile = [&](uint32_t stage_off, floatx16& s) __attribute__((always_inline)) {
    bf16x8 qa[kQkDepth];
#pragma unroll
    for (int c = 0; c < kQkDepth; ++c) qa[c] = qk_operand(stage_off, c);
#pragma unroll
    for (int c = 0; c < kQkSteps; ++c) {
      const bf16x8 cur = qa[c % kQkDepth];
      if (c + kQkDepth < kQkSteps) qa[c % kQkDepth] = qk_operand(stage_off, c + kQkDepth);
      if (c == 0)
        mfma_qk_first(s, cur, qf[0]);
      else
        mfma_qk(s, cur, qf[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  floatx16 s_own;  // this wave's partial S^T of the tile whose softmax runs next
  // LDS offsets of the three stages: tile ti (PV), tile ti + 1 (S^T), and the free one that
  // receives tile ti + 2. They rotate every tile.
  uint32_t off_cur = 0, off_next = kStageBytes, off_free = 2 * kStageBytes;
  // The last kTail PV steps of a tile run after the barrier that ends its interval, between the
  // next interval's S^T steps. Their V operands are read into registers before that barrier, so
  // the stage they came from may be refilled right after it.
  constexpr int kTail = kPvDepth;
  bf16x8 tail_v[kTail];
  bf16x8 tail_ph, tail_pl;  // P^T of key half 1, which those steps use
  auto tail_step = [&](int j) __attribute__((always_inline)) {
    mfma_pv(oacc[(16 - kTail + j) & 7], tail_v[j], tail_ph);
    mfma_pv(oacc[(16 - kTail + j) & 7], tail_v[j], tail_pl);
  };

  // One tile interval:
  //   1. LDS reads of the partner's partial S^T(ti) and of the first S^T(ti + 1) operands;
  //   2. the DMA issue of tile ti + 2 into the free stage;
  //   3. the S^T MFMAs of tile ti + 1 interleaved with the PV tail of tile ti - 1 and the
  //      softmax of tile ti;
  //   4. the PV MFMAs of tile ti up to its tail, with the exchange write of S^T(ti + 1) in
  //      between;
  //   5. wait for this wave's DMA of tile ti + 2, barrier.
  // After the last tile the S^T of a nonexistent tile is computed on stale LDS and thrown away,
  // which keeps a single copy of this code.
  auto interval = [&](int ti) __attribute__((always_inline)) {
    pin_agprs(oacc);
    const bool do_dma = ti >= 1 && ti + 2 < ntiles;
    const bool do_tail = ti >= 1 && pair_active;
    floatx4 xq[4];
    bf16x8 qa[kQkDepth];
    if (pair_active) {
      const floatx4* xp =
          reinterpret_cast<const floatx4*>(xbuf + ((ti & 1) * kWaves + (wave ^ 1)) * kXBytes) + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) xq[q] = xp[64 * q];
#pragma unroll
      for (int c = 0; c < kQkDepth; ++c) qa[c] = qk_operand(off_next, c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (do_dma) start_tile_part(ti + 2, off_free, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (pair_active) {
      floatx16 s_next;
      // A deferred rescale of O (decided with the tile max) waits for the PV tail of the
      // previous tile, which is still relative to the old running max.
      bool rescale = false;
      float alpha = 1.0f;
      constexpr int kRescaleAfter = kTail - 1 > 3 ? kTail - 1 : 3;  // after the decision at step 2
      // S^T step c of tile ti + 1, then (c < kTail) PV tail step c of tile ti - 1: the tail's
      // operands are in registers, so its MFMAs fill the MFMA pipe while the S^T steps wait on
      // LDS.
      auto qk_step = [&](int c) __attribute__((always_inline)) {
        const bf16x8 cur = qa[c % kQkDepth];
        if (c + kQkDepth < kQkSteps) qa[c % kQkDepth] = qk_operand(off_next, c + kQkDepth);
        if (c == 0)
          mfma_qk_first(s_next, cur, qf[0]);
        else
          mfma_qk(s_next, cur, qf[c]);
        if (c < kTail && do_tail) tail_step(c);
        if (c == kRescaleAfter && rescale) rescale_agprs(oacc, alpha);
      };

      // s[r] is key 8*(r/4) + 4g + (r%4) of the tile, head h
      const int nk = n_valid - ti * kTile;
      const bool tail = nk < kTile;  // wave-uniform: only the last tile has masked keys
      float x[16];
      qk_step(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s_own[r] + xq[r >> 2][r & 3];
      __builtin_amdgcn_sched_barrier(0);
      qk_step(1);
      float mx = -INFINITY;
      if (!tail) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[r]);
      } else {
        // keys past the partition's last valid row: -inf scores, so their p is exactly 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x[r] = (8 * (r >> 2) + 4 * g + (r & 3)) < nk ? x[r] : -INFINITY;
          mx = fmaxf(mx, x[r]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      qk_step(2);
      const float mt = pair_max(mx) * c_scale;  // the tile max in the exp2 domain
      if (ti == 0) {
        m_run = mt;  // first tile: O and l are still zero, nothing to rescale
      } else if (__any(mt > m_run + kRescaleThreshold)) {
        const bool need = mt > m_run + kRescaleThreshold;
        alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
        if (need) m_run = mt;
        l_run *= alpha;
        rescale = true;
      }
      __builtin_amdgcn_sched_barrier(0);
      // p = 2^(c*x - m). Key half 0 (p[0..7]) is finished here, two values per S^T step, so
      // that its PV steps can start; key half 1 (p[8..15]) is computed under the first PV
      // steps, whose MFMAs leave the VALU idle.
      float p[16];
      auto exp_pair = [&](int r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) p[r + i] = __builtin_amdgcn_exp2f(fmaf(x[r + i], c_scale, -m_run));
      };
      // P^T operands: hi = p truncated to bf16 (exact), lo = bf16(p - hi) (round to nearest
      // even), so hi + lo carries about 16 significant bits. For key half kb, element i of lane
      // (n, g) is result reg 8*kb + i.
      uint32_t hw[2][4], lw[2][4];
      auto split_pair = [&](int kb, int i) __attribute__((always_inline)) {
        const float p0 = p[8 * kb + 2 * i], p1 = p[8 * kb + 2 * i + 1];
        const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
        hw[kb][i] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
        lw[kb][i] = pack_bf16x2(p0 - __uint_as_float(u0 & 0xffff0000u), p1 - __uint_as_float(u1 & 0xffff0000u));
      };
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        qk_step(3 + 2 * qq);
        exp_pair(2 * qq);
        __builtin_amdgcn_sched_barrier(0);
        qk_step(4 + 2 * qq);
        split_pair(0, qq);
        __builtin_amdgcn_sched_barrier(0);
      }
      qk_step(11);
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) ls += p[r];
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 ph[2], pl[2];
      ph[0] = __builtin_bit_cast(bf16x8, uint4{hw[0][0], hw[0][1], hw[0][2], hw[0][3]});
      pl[0] = __builtin_bit_cast(bf16x8, uint4{lw[0][0], lw[0][1], lw[0][2], lw[0][3]});
#pragma unroll
      for (int c = 12; c < kQkSteps; ++c) {
        qk_step(c);
        __builtin_amdgcn_sched_barrier(0);
      }

      // PV(ti) up to its tail, key half 0 then 1; the exchange write of S^T(ti + 1) once its
      // chain has drained; key half 1's p and P^T operands under the key-half-0 steps.
      static_assert(16 - kTail >= 8, "key half 1's operands are completed by PV step 7");
      bf16x8 va[kPvDepth];
#pragma unroll
      for (int u = 0; u < kPvDepth; ++u) va[u] = pv_operand(off_cur, u);
#pragma unroll
      for (int u = 0; u < 16 - kTail; ++u) {
        const bf16x8 cur = va[u % kPvDepth];
        if (u + kPvDepth < 16) va[u % kPvDepth] = pv_operand(off_cur, u + kPvDepth);
        mfma_pv(oacc[u & 7], cur, ph[u >> 3]);
        mfma_pv(oacc[u & 7], cur, pl[u >> 3]);
        if (u == 1) {
          mfma_qk_drain(s_next);
          x_write((ti + 1) & 1, s_next);
        }
        if (u < 4) exp_pair(8 + 2 * u);
        if (u >= 4 && u < 8) split_pair(1, u - 4);
        if (u == 7) {
          ph[1] = __builtin_bit_cast(bf16x8, uint4{hw[1][0], hw[1][1], hw[1][2], hw[1][3]});
          pl[1] = __builtin_bit_cast(bf16x8, uint4{lw[1][0], lw[1][1], lw[1][2], lw[1][3]});
#pragma unroll
          for (int r = 8; r < 16; ++r) ls += p[r];
          l_run += pair_sum(ls);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < kTail; ++j) tail_v[j] = va[(16 - kTail + j) % kPvDepth];
      tail_ph = ph[1];
      tail_pl = pl[1];
      s_own = s_next;
    }
    pin_agprs(oacc);
    // tile ti + 2 must be in LDS for the next interval's S^T MFMAs
    if (ti + 2 < ntiles) finish_tile(off_free);
    lds_barrier();
    const uint32_t o = off_cur;
    off_cur = off_next;
    off_next = off_free;
    off_free = o;
  };

  // ---- prologue: tiles 0 and 1 in LDS, tile 2 on its way, S^T(0) exchanged.
  // DMA instructions per tile and wave on the bf16 path: 8 nope rows (one each) and one for the
  // wave's 8 rope rows, on both the buffer-resource and the 64-bit path.
  constexpr int kDmaPerTile = 9;
  if (ntiles > 0) {
    if constexpr (kInt8) {
      // one register buffer: each tile's nope is written to LDS before the next is loaded
      start_tile(0, 0);
      finish_tile(0);
      if (ntiles > 1) {
        start_tile(1, kStageBytes);
        finish_tile(kStageBytes);
      }
    } else {
      // Tiles 0, 1 and 2 are fetched together, and S^T(0) waits for tile 0 alone: a wave issues
      // kDmaPerTile DMA instructions per tile, and vector-memory loads complete in issue order.
      start_tile(0, 0);
      if (ntiles > 1) start_tile(1, kStageBytes);
      if (ntiles > 2) start_tile(2, 2 * kStageBytes);
      if (ntiles > 2)
        wait_vmcnt<2 * kDmaPerTile>();
      else if (ntiles > 1)
        wait_vmcnt<kDmaPerTile>();
      else
        wait_vmcnt<0>();
    }
    if (kInt8 && ntiles > 2) start_tile(2, 2 * kStageBytes);
    lds_barrier();
    if (pair_active) {
      qk_tile(0, s_own);
      mfma_qk_drain(s_own);
      x_write(0, s_own);
    }
    // tile 1 must be in LDS for the first interval's S^T; tile 2 may still be on its way
    if constexpr (!kInt8) {
      if (ntiles > 2)
        wait_vmcnt<kDmaPerTile>();
      else
        wait_vmcnt<0>();
    }
    lds_barrier();
    for (int ti = 0; ti < ntiles; ++ti) interval(ti);
    // the PV tail of the last tile
    if (pair_active) {
#pragma unroll
      for (int j = 0; j < kTail; ++j) tail_step(j);
    }
  }
  mfma_pv_drain(oacc);

  // ---- epilogue: oacc[dc][4*rq + e] is column d = 256*half + 32*dc + 8*rq + 4*g + e of head h
  if (a.n_splits == 1) {
    // The normalised bf16 O of this wave (32 heads x 256 columns) goes through LDS, so that each
    // store instruction writes two whole 512-byte rows instead of 32 scattered 16-byte pieces.
    // Layout: 16 KB per wave, row = head, 16-byte chunk c of a row at chunk c ^ row (no bank
    // conflicts on the row-wise read back). The stages are free once every wave is here.
    lds_barrier();
    char* ob = smem + wave * (kHeadsPerPair * 512);
    if (pair_active) {
      const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          uint2 v;
          v.x = pack_bf16x2(oacc[dc][4 * rq] * inv, oacc[dc][4 * rq + 1] * inv);
          v.y = pack_bf16x2(oacc[dc][4 * rq + 2] * inv, oacc[dc][4 * rq + 3] * inv);
          const int c = 4 * dc + rq;  // columns 8c .. 8c + 7 of the wave's 256
          *reinterpret_cast<uint2*>(ob + n * 512 + ((c ^ n) & 31) * 16 + 8 * g) = v;
        }
      }
      // read back (the wave's own LDS accesses complete in order): lane L takes chunk L % 32 of
      // row 2i + L / 32. The stores are non-temporal: the output is not read again here, and
      // all workgroups store it in one burst at the end (measured ~2 % of the decode call).
      const int j = lane & 31;
      uint16_t* orow = a.out + ((int64_t)t * a.n_q + hp0) * kNope + 256 * half + 8 * j;
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 2 * i + g;
        const uint4 v = *reinterpret_cast<const uint4*>(ob + r * 512 + ((j ^ r) & 31) * 16);
        if (hp0 + r < a.n_q)
          __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(orow + (int64_t)r * kNope));
      }
    }
    return;
  }

  // Partial of (t, hg, sp) in register-image order: [wave][dc][rq][lane] float4. Both waves of a
  // pair hold the same running max and sum; the half-0 wave records them.
  //
  // Publication without an L2 write-back: every partial is written with agent-scope stores (the
  // sc1 form of the store, which the L2 of this XCD writes through instead of holding dirty), so
  // once this wave's stores are acknowledged (vmcnt 0) they are visible to every XCD, and the
  // arrival count that follows needs no release fence. (A release fence would write back this
  // XCD's whole L2, which measured as the dominant cost of the merge.) The last arriver still
  // takes an agent-scope acquire fence, which drops stale lines from its own L2.
  const int S = a.n_splits;
  const int64_t grp_item = (int64_t)t * a.head_groups + hg;  // (token, head group)
  floatx4* part = reinterpret_cast<floatx4*>(a.part_o);
  constexpr int kWaveImage = 8 * 4 * 64;  // float4s per wave
  if (pair_active) {
    floatx4* po = part + ((grp_item * S + sp) * kWaves + wave) * kWaveImage + lane;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const floatx4 v{oacc[dc][4 * rq], oacc[dc][4 * rq + 1], oacc[dc][4 * rq + 2], oacc[dc][4 * rq + 3]};
        asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(po + (dc * 4 + rq) * 64), "v"(v) : "memory");
      }
    }
    if (half == 0 && g == 0) {
      uint64_t* ml = reinterpret_cast<uint64_t*>(a.part_ml) + (grp_item * S + sp) * kHeadsPerGroup +
                     pair * kHeadsPerPair + n;
      const uint64_t bits = (uint64_t)__float_as_uint(m_run) | ((uint64_t)__float_as_uint(l_run) << 32);
      __hip_atomic_store(ml, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
  lds_barrier();
  if (tid == 0) s_last = (atomicAdd(a.counters + grp_item, 1) == S - 1) ? 1 : 0;
  lds_barrier();
  if (!s_last || !pair_active) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other partitions' partials

  // The last arriver combines all S partials (its own included, re-read from memory so that O's
  // registers are free): the (m, l) of every partition for this lane's head are loaded in one
  // batch, then O in two halves of 16 float4 per partition, each half's loads issued together.
  const float2* mlp = reinterpret_cast<const float2*>(a.part_ml) + grp_item * S * kHeadsPerGroup +
                      pair * kHeadsPerPair + n;
  float2 mlv[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) mlv[s] = mlp[(s < S ? s : S - 1) * kHeadsPerGroup];
  float mmax = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) mmax = s < S ? fmaxf(mmax, mlv[s].x) : mmax;
  float wv[kMaxSplits];
  float lsum = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    wv[s] = (s < S && mlv[s].x != -INFINITY) ? __builtin_amdgcn_exp2f(mlv[s].x - mmax) : 0.f;
    lsum += wv[s] * mlv[s].y;
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint16_t* o = a.out + ((int64_t)t * a.n_q + h) * kNope + 256 * half + 4 * g;
  const floatx4* pbase = part + (grp_item * S * kWaves + wave) * kWaveImage + lane;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    floatx4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma nounroll
    for (int s = 0; s < S; ++s) {
      float w = 0.f;
#pragma unroll
      for (int u = 0; u < kMaxSplits; ++u) w = (u == s) ? wv[u] : w;
      const floatx4* ps = pbase + (int64_t)s * kWaves * kWaveImage + hh * 16 * 64;
      floatx4 buf[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) buf[i] = ps[i * 64];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += w * buf[i];
    }
    if (head_ok) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dc = 4 * hh + i / 4, rq = i % 4;
        uint2 v;
        v.x = pack_bf16x2(acc[i][0] * inv, acc[i][1] * inv);
        v.y = pack_bf16x2(acc[i][2] * inv, acc[i][3] * inv);
        *reinterpret_cast<uint2*>(o + 32 * dc + 8 * rq) = v;
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

hipError_t launch_attention(const KernelArgs& a, bool int8_cache, bool window_slots, hipStream_t stream) {
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
  // 32-bit byte offsets (and buffer sizes) cover every cache row while the pool holds fewer
  // than 4 Mi rows (4 GiB of bf16 nope)
  const bool buf = a.num_rows < (int64_t{1} << 22);
  const void* fn;
  if (window_slots)
    fn = int8_cache ? (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<true, true, true>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<true, false, true>))
                    : (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<false, true, true>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<false, false, true>));
  else
    fn = int8_cache ? (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<true, true, false>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<true, false, false>))
                    : (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<false, true, false>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<false, false, false>));
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
