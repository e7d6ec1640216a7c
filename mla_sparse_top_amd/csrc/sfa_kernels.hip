// Sparse flash attention over a paged MLA latent cache: HIP kernels for gfx950 (CDNA4).
//
// What is computed is the operation described in "DeepSeek V3/V2 Sparse Flash Attention with
// Quantization" (sections "Algorithm overview", "Implementation notes: compute pipeline", "INT8
// quantisation path", "Flash online softmax update"): for every query token, gather the top-k
// latent rows through the block table, S = [q_nope|q_rope] . [k_nope|k_rope]^T, softmax of
// scale*S, times V = k_nope. The window variants ("NPU DeepSeek-V4 model PyPTO fused-operator
// optimisation", FA-class operators) also take 512-wide rows with the rotary channels inside the
// row (its D = 512): no rope part, S = q . k^T over the 512 channels, V = the row. How it is
// computed here is a gfx950 design of its own:
//
//   * A workgroup of 4 waves (one per SIMD) owns one (token, top-k partition) and every query
//     head of the token (or 64 of them, with two head groups): wave w owns heads 32w..32w+31
//     over the whole 576-wide d, so no wave waits on another's partial scores, and every
//     gathered 32-row tile feeds all the workgroup's heads: 36 S^T steps and 64 P.V steps of the
//     32x32x16 MFMA per wave and tile.
//   * Registers: the wave's Q (32 heads x 576, the B operand of S^T = K . Q^T) stays in 144
//     VGPRs, its O^T (32 heads x 512 fp32) in all 256 AGPRs.
//   * Resolve + compaction: the partition's slots are resolved (index -> block_table -> row),
//     masked slots are dropped and the valid rows are packed in order into an LDS list. Tiles
//     are then dense: padding costs no loads and no MFMA, and a tile of invalid slots never runs.
//   * Gather: bf16 tiles go HBM -> LDS by DMA (buffer_load ... lds), one 1 KB nope row per wave
//     instruction and eight 128 B rope rows per instruction, into four LDS stages, so a tile is
//     requested three tile intervals before its S^T runs; a tile's DMA goes out in five pieces
//     spread over the interval. INT8 codes and scales go by DMA into two code buffers; each wave
//     dequantises the 8 rows it fetched (int8 -> fp32, times the fp32 group scale,
//     round-to-nearest-even to bf16) into the bf16 tile layout, in small steps between the S^T
//     MFMAs of the interval (three bf16 stages).
//   * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: keys on M, heads on N, d as the reduction.
//     Each lane then holds one head and 16 of a tile's 32 keys, so the softmax row max and row
//     sum need one cross-lane step (v_permlane32_swap).
//   * Online softmax over tiles (running max / running sum). The running max is only moved
//     when a tile's max exceeds it by more than 2^8 (exp2 domain), so O is rescaled rarely; the
//     final O / l is unchanged.
//   * O^T += V^T . P^T, again 32x32x16 MFMA. P^T comes straight from the S^T accumulator
//     registers (no shuffle). V^T fragments are read from the row-major K tile with
//     ds_read_b64_tr_b16 (LDS transpose read), so no transposed copy exists. P is split into
//     bf16 hi + lo parts, two MFMAs on the same V fragment, so it keeps about 16 significant
//     bits instead of 8: a single bf16 P does not meet the 5e-3 / 1e-4 accuracy standard when
//     few keys carry the weight.
//   * Software pipeline, one barrier per tile interval: the 36 S^T steps of tile i+1 alternate
//     with the P.V steps of tile i's first 16 keys; then tile i's last 16 keys' P.V steps run
//     while the VALU computes tile i+1's softmax, so MFMA and VALU work overlap in every phase.
//   * Partitions of one token merge in the same kernel: each takes an arrival ticket and
//     publishes the unnormalised O, running max and running sum other partitions need; with 2
//     to 16 resident partitions each output unit (a wave's heads x 128 columns) is merged by one
//     of them (the merge spread over the token's workgroups), otherwise all by the last to
//     arrive. Whoever merges combines all partitions in partition order, so the result does not
//     depend on arrival order: O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j, the prefill
//     update rule applied across partitions.
//   * Work items are mapped so that consecutive logical ids land on the same XCD and share its
//     L2 (the hardware deals workgroups to the 8 XCDs round-robin): the partitions of a token,
//     and the tokens of one sequence, which draw on the same rows.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4_t;

// LDS layout of one pipeline stage (one 32-row tile):
//   nope: 32 rows x 1024 B. The 16-byte chunk c of row k sits at chunk c ^ nope_swz(k) (the XOR
//         only touches the low 4 bits of the chunk index). With this swizzle, neither the
//         16-byte reads of the QK^T operand (32 rows, same chunk) nor the 8-byte transpose
//         reads of the PV operand (4 rows x 2 chunks per 16 lanes) repeat a bank.
//   rope: 32 rows x 128 B, chunk c of row k at c ^ rope_swz(k).
// An INT8 code buffer holds one tile's codes (wave w's rows 8w..8w+7 in its own 4 KB, row-major
// 512 B rows) and scales (wave w's 8 rows x 4 fp32 at 256 B per wave).
constexpr int kNopeRowBytes = kNope * 2;
constexpr int kRopeRowBytes = kRope * 2;
constexpr int kNopeTileBytes = kTile * kNopeRowBytes;
constexpr int kRopeTileBytes = kTile * kRopeRowBytes;
constexpr int kStageBytes = kNopeTileBytes + kRopeTileBytes;
constexpr int kCodeTileBytes = kTile * kNope;        // 16 KB
constexpr int kCodeBufBytes = kCodeTileBytes + kWaves * 256;
constexpr float kRescaleThreshold = 8.0f;           // log2 units: p stays <= 256 between rescales
constexpr int kQkDepthBf16 = 4;
constexpr int kPvDepthBf16 = 3;
constexpr int kOutWaveBytes = kHeadsPerWave * kNopeRowBytes;  // a wave's bf16 output rows (32 KB)
// Per-token counters of the partition merge: 64-bit words holding (generation << 16) | count.
// Every call carries its own 48-bit generation, so a word left by another call, or any other
// contents of the workspace, carries another generation and counts as zero: the workspace needs
// no clearing before a call. tagged_add returns the count before its increment.
__device__ __forceinline__ uint64_t tagged_count(uint64_t* p, uint64_t gen) {
  const uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (v >> 16) == gen ? (v & 0xffffu) : 0;
}
__device__ __forceinline__ uint64_t tagged_add(uint64_t* p, uint64_t gen) {
  uint64_t old = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const uint64_t cnt = (old >> 16) == gen ? (old & 0xffffu) : 0;
    if (__hip_atomic_compare_exchange_strong(p, &old, (gen << 16) | (cnt + 1), __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return cnt;
  }
}

// Bound on the last arriver's wait for the other partitions' partials (each try sleeps ~128
// clocks): far beyond the time a partial takes to be stored.
constexpr int kSpinLimit = 1 << 24;
// A merging partition's decision on the heads of one of its waves (spread merge).
constexpr uint64_t kMergedByFirst = 1, kPublishedByFirst = 2;

template <bool kInt8>
struct Lds {
  static constexpr int kStages = kInt8 ? 3 : 4;
  static constexpr int kCodesOff = kStages * kStageBytes;
  static constexpr int kBytes = kCodesOff + (kInt8 ? 2 * kCodeBufBytes : 0);
};
static_assert(Lds<false>::kBytes + kMaxSlots * 4 + 64 <= 160 * 1024, "LDS budget (bf16)");
static_assert(Lds<true>::kBytes + kMaxSlots * 4 + 64 <= 160 * 1024, "LDS budget (INT8)");
static_assert(Lds<false>::kBytes >= kWaves * kOutWaveBytes && Lds<true>::kBytes >= kWaves * kOutWaveBytes,
              "the output staging reuses the stage memory");

__device__ __forceinline__ int nope_swz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }
__device__ __forceinline__ int rope_swz(int key) { return (key >> 1) & 7; }

__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint64_t nbytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  // dword 2: the size in bytes (callers keep it below 4 GiB); dword 3: the raw-buffer
  // configuration (32-bit data format, no swizzle, no stride)
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, (uint32_t)nbytes, 0x00020000u};
}

// LDS-DMA: lane L's bytes land at M0 + 16*L (dwordx4) or M0 + 4*L (dword). M0 is saved and
// restored around each use; it needs one wait state between its write and the DMA. Issued from
// inline asm so that the compiler does not wait for the whole vector-memory queue before every
// LDS read. Completion is tracked explicitly with wait_vmcnt, cross-wave visibility with a
// barrier.
//
// Four whole nope rows, one per instruction, through a buffer resource: row rK's byte offset
// (rK << 10) goes in the scalar offset, lane L's 16-byte piece in its VGPR offset, and row kK0+i
// lands at lds_base + (kK0+i) * 1 KB.
template <int kK0>
__device__ __forceinline__ void dma_rows4(const u32x4& rsrc, int r0, int r1, int r2, int r3, uint32_t v0,
                                          uint32_t v1, uint32_t v2, uint32_t v3, uint32_t lds_base) {
  uint32_t saved, o0, o1, o2, o3;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_lshl_b32 %1, %10, 10\n\t"
      "s_add_u32 m0, %14, %15\n\t"
      "s_lshl_b32 %2, %11, 10\n\t"
      "buffer_load_dwordx4 %5, %9, %1 offen lds\n\t"
      "s_add_u32 m0, %14, %16\n\t"
      "s_lshl_b32 %3, %12, 10\n\t"
      "buffer_load_dwordx4 %6, %9, %2 offen lds\n\t"
      "s_add_u32 m0, %14, %17\n\t"
      "s_lshl_b32 %4, %13, 10\n\t"
      "buffer_load_dwordx4 %7, %9, %3 offen lds\n\t"
      "s_add_u32 m0, %14, %18\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %8, %9, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved), "=&s"(o0), "=&s"(o1), "=&s"(o2), "=&s"(o3)
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(rsrc), "s"(r0), "s"(r1), "s"(r2), "s"(r3), "s"(lds_base),
        "n"(kK0 * 1024), "n"((kK0 + 1) * 1024), "n"((kK0 + 2) * 1024), "n"((kK0 + 3) * 1024)
      : "memory");
}
template <int kK0>
__device__ __forceinline__ void dma_rows2(const u32x4& rsrc, int r0, int r1, uint32_t v0, uint32_t v1, uint32_t lds_base) {
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
// One DMA instruction with a per-lane byte offset into the buffer.
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
__device__ __forceinline__ void dma4_voff(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory");
}
// 64-bit addressing (pools of 4 Mi rows and more): a per-lane global address.
__device__ __forceinline__ void dma16_g(const void* gaddr, uint32_t lds_addr) {
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
__device__ __forceinline__ void dma4_g(const void* gaddr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(lds_addr)
      : "memory");
}
// A wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset (one whole nope row).
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS traffic only. Outstanding DMA stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  // s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maximum, written as the builtin so
  // that the compiler's wait-count tracking knows the LDS queue is empty after it
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
}

// The lane id, recomputed where it is used (two VALU instructions): a volatile statement is
// not hoisted out of the tile loop, so values derived from it are not kept live (or spilled)
// across the loop.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// S^T += K . Q^T steps: the accumulator and both operands in VGPRs. Consecutive steps
// accumulate into the same registers, which the hardware chains back to back (an exactly
// overlapping accumulator needs no wait states); the chain starts from 0. The first step's
// leading pad covers a VALU write of an operand right before it. The later steps read only
// LDS-loaded K fragments, the Q registers (written once) and the chained accumulator, so they
// carry no pad; the build checks the generated code for a VALU write of an MFMA operand within
// two instructions before an unpadded MFMA.
__device__ __forceinline__ void mfma_qk_first(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// A chained step right after a branch target: the pad keeps the rule of two wait states before
// every MFMA whose predecessor cannot be seen in straight-line code.
__device__ __forceinline__ void mfma_qk_pad(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// The last step of a chain, with the pad its result needs before a VALU or LDS read (18 wait
// states for a 32x32x16 result; 20 given) in the same statement, so that no copy of the result
// can be scheduled between the MFMA and its pad.
__device__ __forceinline__ void mfma_qk_last(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+v"(acc)
               : "v"(a), "v"(b));
}
// Before anything else reads the chain's result: a 32x32x16 result needs 18 wait states before
// a VALU or LDS read of it; this gives 20.
__device__ __forceinline__ void mfma_drain(floatx16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
}

// O^T += V^T . P^T step on an AGPR-resident accumulator, tied in place, with no pad: its V^T
// operand comes from LDS, and its P^T operands are converted many instructions ahead (the
// assembly test holds this).
__device__ __forceinline__ void mfma_pv(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// O *= alpha on the AGPR-resident accumulators, in place: each element is read to a VGPR,
// scaled and written back by inline asm, so no compiler-generated VALU ever touches O (which
// would make the compiler keep O in VGPRs and copy it around every tile). Pads: the last MFMA
// that wrote O needs 18 wait states before an AGPR read (20 given); the MFMA that next reads O
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

// Four consecutive O elements of an AGPR-resident accumulator block, read into VGPRs by inline
// asm so that the compiler never copies the whole block (or all sixteen) out of the AGPRs. The
// caller has drained the MFMA pipe (mfma_pv_drain) before the first read.
__device__ __forceinline__ floatx4 agpr_quad(const floatx16& acc, int q) {
  floatx4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[4 * q + e]));
  return v;
}

__device__ __forceinline__ shortx4 lds_tr16(const lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)p);
}
__device__ __forceinline__ bf16x8 lds_b128(const lds_char_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
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

// kBufDma: cache rows (nope, rope, INT8 codes and scales) are fetched through buffer resources
// with 32-bit byte offsets (pools below 4 Mi rows); otherwise through 64-bit global addresses.
// kWindow: the window variants' slot list (see KernelArgs), resolved here instead of read from
// topk_indices; the rest of the kernel is the same.
// kRopeW: 64, rows of 512 nope + 64 rope channels (scores over both, V = nope); or 0, the
// 512-wide rows whose rotary channels sit inside the row (scores over the 512, V = the row).
template <bool kInt8, bool kBufDma, bool kWindow, int kRopeW>
__global__ void __launch_bounds__(kThreads, 1) sfa_attention_kernel(const KernelArgs a) {
  using L = Lds<kInt8>;
  static_assert(kRopeW == kRope || kRopeW == 0, "rows carry 64 rope channels or none");
  // S^T k-steps of 16 over the row (36 over 576 channels, 32 over 512); DMA pieces and INT8
  // dequantisation parts are spread over them at these strides
  constexpr int kQk = (kNope + kRopeW) / 16;
  constexpr int kPieceStride = kRopeW ? 7 : 6;
  constexpr int kDqStride = kRopeW ? 8 : 6;
  // S^T operand loads in flight ahead of the MFMA (INT8 keeps one fewer: its dequantisation
  // needs the registers)
  constexpr int kQkDepth = kInt8 ? 3 : kQkDepthBf16;
  constexpr int kPvDepth = kInt8 ? 2 : kPvDepthBf16;
  __shared__ __attribute__((aligned(1024))) char smem[L::kBytes];
  __shared__ __attribute__((aligned(16))) int32_t s_rows[kMaxSlots];
  __shared__ int32_t s_wcnt[kWaves];
  __shared__ int32_t s_rank;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int lane = tid & 63;
  const int n = lane & 31;  // row (A operand) or column (B operand, result) of the 32x32 MFMA
  const int g = lane >> 5;  // k-group of an operand / row-quad parity of a result
  // ---- work item: XCD-aware remap of the workgroup id, then (token, partition, head group)
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int per_xcd = nwg >> 3;
  int lid = bid;
  if (per_xcd > 0 && bid < (per_xcd << 3)) lid = (bid & 7) * per_xcd + (bid >> 3);
  const int per_token = a.n_splits * a.head_groups;
  int t = lid / per_token;
  const int sp = (lid - t * per_token) / a.head_groups;
  const int hg = lid - t * per_token - sp * a.head_groups;
  if (a.reverse) t = a.n_tokens - 1 - t;
  const int b = t / a.s1;
  // With two head groups a workgroup covers 64 heads: waves 0 and 1 compute them, and waves 2
  // and 3 only help gather the tiles.
  const int h0 = hg * (kMaxHeads / 2) + wave * kHeadsPerWave;  // first head of this wave
  const bool wave_active = (a.head_groups == 1 || wave < 2) && h0 < a.n_q;  // wave-uniform
  const int h = h0 + n;                 // this lane's head
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
  // ---- Q^T fragments (B operand, k = d): step c < 32 covers nope chunks 2c + {0, 1}, steps
  // 32..35 (with rope channels) rope chunks 2(c - 32) + {0, 1}; lane (n, g) holds chunk +g.
  // Issued after the index and block-table loads: load completion is counted in issue order,
  // so Q's 147 KB per token must not sit in front of the two dependent index round trips.
  // A lane past n_q reads head 0's row; its scores are computed and never stored.
  uint4 qv[kQk];
  {
    const int64_t qrow = (int64_t)t * a.n_q + (head_ok ? h : 0);
    const uint4* qn = reinterpret_cast<const uint4*>(a.q_nope + qrow * kNope);
#pragma unroll
    for (int c = 0; c < 32; ++c) qv[c] = qn[2 * c + g];
    if constexpr (kRopeW > 0) {
      const uint4* qr = reinterpret_cast<const uint4*>(a.q_rope + qrow * kRope);
#pragma unroll
      for (int c = 0; c < 4; ++c) qv[32 + c] = qr[2 * c + g];
    }
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

  // O^T block dc: reg r holds column d = 32*dc + 8*(r/4) + 4g + (r%4) of head h
  floatx16 oacc[16];
#pragma unroll
  for (int dc = 0; dc < 16; ++dc) oacc[dc] = floatx16{};
  pin_agprs(oacc);
  float m_run = -INFINITY;  // running max (exp2 domain) that p and O are currently relative to
  float l_run = 0.f;

  // ---- loaders. Wave w fetches rows 8w..8w+7 of each tile.
  const uint32_t smem_lds = (uint32_t)(uintptr_t)((lds_char_t*)smem);
  const lds_char_t* smem_p = (const lds_char_t*)smem;
  auto stage_of = [&](int tile) -> uint32_t { return (uint32_t)((tile % L::kStages) * kStageBytes); };
  auto codes_of = [&](int tile) -> uint32_t { return (uint32_t)(L::kCodesOff + (tile & 1) * kCodeBufBytes); };
  const u32x4 rs_nope = make_rsrc(a.k_nope, (uint64_t)a.num_rows * (kInt8 ? kNope : kNopeRowBytes));
  const u32x4 rs_rope = make_rsrc(a.k_rope, kRopeW ? (uint64_t)a.num_rows * kRopeRowBytes : 0);
  const u32x4 rs_scale = make_rsrc(a.k_scales, kInt8 ? (uint64_t)a.num_rows * 16 : 0);
  // lane L's row: key 8w + L/8 of the tile (rope DMA; its readlanes give the wave's 8 rows)
  auto lane_row = [&](int tile) -> int { return s_rows[tile * kTile + wave * 8 + (lane_id_here() >> 3)]; };
  // rope: lane L fetches chunk ((L & 7) ^ rope_swz(key)) of key = 8w + L/8
  auto issue_rope = [&](int row, uint32_t stage) __attribute__((always_inline)) {
    if constexpr (kRopeW == 0) return;
    const int ln = lane_id_here();
    const int key = wave * 8 + (ln >> 3);
    const uint32_t chunk = 16 * ((ln & 7) ^ rope_swz(key));
    const uint32_t lds = smem_lds + stage + kNopeTileBytes + wave * 8 * kRopeRowBytes;
    if constexpr (kBufDma) {
      dma16_voff(rs_rope, (uint32_t)row * kRopeRowBytes + chunk, lds);
    } else {
      dma16_g(reinterpret_cast<const char*>(a.k_rope) + (int64_t)row * kRopeRowBytes + chunk, lds);
    }
  };
  // bf16 nope: one 1 KB row per instruction; lane L fills physical chunk L, i.e. fetches
  // logical chunk L ^ nope_swz(key).
  auto issue_nope_bf16 = [&](int row, uint32_t stage) __attribute__((always_inline)) {
    int r[8];
    uint32_t vo[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      r[k] = __builtin_amdgcn_readlane(row, 8 * k);
      vo[k] = (uint32_t)(16 * lane) ^ (uint32_t)(16 * nope_swz(wave * 8 + k));
    }
    const uint32_t lds_base = smem_lds + stage + wave * 8 * kNopeRowBytes;
    if constexpr (kBufDma) {
      static_assert(kNopeRowBytes == 1024, "row offsets are formed as row << 10");
      dma_rows4<0>(rs_nope, r[0], r[1], r[2], r[3], vo[0], vo[1], vo[2], vo[3], lds_base);
      dma_rows4<4>(rs_nope, r[4], r[5], r[6], r[7], vo[4], vo[5], vo[6], vo[7], lds_base);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const char* base = reinterpret_cast<const char*>(a.k_nope) + (int64_t)r[k] * kNopeRowBytes;
        dma16_sbase(base, vo[k], lds_base + k * kNopeRowBytes);
      }
    }
  };
  // INT8 codes: instruction m moves the wave's rows 2m and 2m + 1 (lanes 0-31 and 32-63, 16
  // bytes each) into the wave's 4 KB of the code buffer; scales: lane L < 32 moves group L % 4 of
  // key L / 4 (lanes 32-63 repeat it into unused bytes).
  auto issue_int8 = [&](int row, int tile) __attribute__((always_inline)) {
    const uint32_t cb = smem_lds + codes_of(tile) + wave * 4096;
    const uint32_t sb = smem_lds + codes_of(tile) + kCodeTileBytes + wave * 256;
    const int srow = s_rows[tile * kTile + wave * 8 + ((lane & 31) >> 2)];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r0 = __builtin_amdgcn_readlane(row, 16 * m);       // key 2m
      const int r1 = __builtin_amdgcn_readlane(row, 16 * m + 8);   // key 2m + 1
      const int rr = g ? r1 : r0;
      if constexpr (kBufDma) {
        dma16_voff(rs_nope, (uint32_t)rr * kNope + 16 * n, cb + m * 1024);
      } else {
        dma16_g(reinterpret_cast<const int8_t*>(a.k_nope) + (int64_t)rr * kNope + 16 * n, cb + m * 1024);
      }
    }
    if constexpr (kBufDma) {
      dma4_voff(rs_scale, (uint32_t)srow * 16 + 4 * (lane & 3), sb);
    } else {
      dma4_g(reinterpret_cast<const char*>(a.k_scales) + (int64_t)srow * 16 + 4 * (lane & 3), sb);
    }
  };
  // DMA instructions per tile and wave: bf16 8 nope rows + 1 rope; INT8 4 code + 1 scale + 1 rope
  // (no rope instruction for rows without rope channels)
  constexpr int kDmaPerTile = (kInt8 ? 5 : 8) + (kRopeW ? 1 : 0);
  // The same DMA in five pieces, to be spread between MFMAs: piece k < 4 moves the wave's rows
  // 2k and 2k + 1 (bf16 nope rows, or INT8 codes), piece 4 the rope rows (and INT8 scales).
  auto issue_piece = [&](int tile, int row, int k) __attribute__((always_inline)) {
    const uint32_t stage = stage_of(tile);
    if (k == 4) {
      if constexpr (kInt8) {
        const uint32_t sb = smem_lds + codes_of(tile) + kCodeTileBytes + wave * 256;
        const int ln = lane_id_here();
        const int srow = s_rows[tile * kTile + wave * 8 + ((ln & 31) >> 2)];
        if constexpr (kBufDma) {
          dma4_voff(rs_scale, (uint32_t)srow * 16 + 4 * (ln & 3), sb);
        } else {
          dma4_g(reinterpret_cast<const char*>(a.k_scales) + (int64_t)srow * 16 + 4 * (ln & 3), sb);
        }
      }
      issue_rope(row, stage);
      return;
    }
    const int r0 = __builtin_amdgcn_readlane(row, 16 * k);      // key 2k of the wave's 8
    const int r1 = __builtin_amdgcn_readlane(row, 16 * k + 8);  // key 2k + 1
    const int ln = lane_id_here();
    if constexpr (kInt8) {
      const uint32_t cb = smem_lds + codes_of(tile) + wave * 4096;
      const int rr = (ln >> 5) ? r1 : r0;
      if constexpr (kBufDma) {
        dma16_voff(rs_nope, (uint32_t)rr * kNope + 16 * (ln & 31), cb + k * 1024);
      } else {
        dma16_g(reinterpret_cast<const int8_t*>(a.k_nope) + (int64_t)rr * kNope + 16 * (ln & 31), cb + k * 1024);
      }
    } else {
      const uint32_t lds_base = smem_lds + stage + wave * 8 * kNopeRowBytes;
      const uint32_t vo0 = (uint32_t)(16 * ln) ^ (uint32_t)(16 * nope_swz(wave * 8 + 2 * k));
      const uint32_t vo1 = (uint32_t)(16 * ln) ^ (uint32_t)(16 * nope_swz(wave * 8 + 2 * k + 1));
      if constexpr (kBufDma) {
        switch (k) {
          case 0: dma_rows2<0>(rs_nope, r0, r1, vo0, vo1, lds_base); break;
          case 1: dma_rows2<2>(rs_nope, r0, r1, vo0, vo1, lds_base); break;
          case 2: dma_rows2<4>(rs_nope, r0, r1, vo0, vo1, lds_base); break;
          default: dma_rows2<6>(rs_nope, r0, r1, vo0, vo1, lds_base); break;
        }
      } else {
        const char* kn = reinterpret_cast<const char*>(a.k_nope);
        dma16_sbase(kn + (int64_t)r0 * kNopeRowBytes, vo0, lds_base + 2 * k * kNopeRowBytes);
        dma16_sbase(kn + (int64_t)r1 * kNopeRowBytes, vo1, lds_base + (2 * k + 1) * kNopeRowBytes);
      }
    }
  };
  auto issue_tile = [&](int tile, int row) __attribute__((always_inline)) {
    if constexpr (kInt8) {
      issue_int8(row, tile);
    } else {
      issue_nope_bf16(row, stage_of(tile));
    }
    issue_rope(row, stage_of(tile));
  };
  // INT8 dequantisation of the wave's 8 rows of a tile, from its code buffer into the bf16
  // layout of the tile's stage: code -> fp32 (exact), times the fp32 group scale (one rounding:
  // fma((code + 128), s, -128 s) is the exact product rounded once), -> bf16 (RNE). Lane L takes
  // 16 codes of key 2m + L/32 per step m, which become logical chunks 2(L % 32) and +1 of its row.
  // The dequantisation of one tile runs in four parts (the wave's rows 2m and 2m + 1), each split
  // into a read of its codes and scale and two halves of 8 codes that are converted and stored,
  // so that the three can sit between different MFMAs.
  struct Int8Part {
    u32x4 c;        // lane L: codes 16(L % 32) .. +15 of key 2m + L / 32 of the wave's 8
    float sc;       // the scale of their group
    uint32_t dst;   // LDS byte address of logical chunk 2(L % 32) of that key's bf16 row
  };
  auto dq_load = [&](int tile, int m) __attribute__((always_inline)) -> Int8Part {
    const lds_char_t* cb = smem_p + codes_of(tile) + wave * 4096;
    const lds_char_t* sb = smem_p + codes_of(tile) + kCodeTileBytes + wave * 256;
    const int ln = lane_id_here();
    Int8Part q;
    q.c = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(cb + m * 1024 + 16 * ln);
    q.sc = *reinterpret_cast<const __attribute__((address_space(3))) float*>(sb + (2 * m + (ln >> 5)) * 16 +
                                                                              4 * ((ln & 31) >> 3));
    const int key = wave * 8 + 2 * m + (ln >> 5);
    // the row starts on a 1 KB boundary, so chunk 2(L % 32) + 1 is at dst ^ 16
    q.dst = stage_of(tile) + key * kNopeRowBytes + 16 * ((2 * (ln & 31)) ^ nope_swz(key));
    return q;
  };
  // Quarter qq: codes 16(L % 32) + 4qq .. +3 become two bf16 pairs of o; after the second
  // quarter of a half (qq odd) the 16-byte logical chunk 2(L % 32) + qq / 2 of the row is stored.
  auto dq_quarter = [&](int qq, const Int8Part& q, uint32_t (&o)[4]) __attribute__((always_inline)) {
    const uint32_t w = q.c[qq] ^ 0x80808080u;
    const float nb = -128.0f * q.sc;
    const float f0 = fmaf((float)(w & 0xffu), q.sc, nb);
    const float f1 = fmaf((float)((w >> 8) & 0xffu), q.sc, nb);
    const float f2 = fmaf((float)((w >> 16) & 0xffu), q.sc, nb);
    const float f3 = fmaf((float)(w >> 24), q.sc, nb);
    o[2 * (qq & 1)] = pack_bf16x2(f0, f1);
    o[2 * (qq & 1) + 1] = pack_bf16x2(f2, f3);
    if (qq & 1)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((lds_char_t*)smem_p + (q.dst ^ (16u * (qq >> 1)))) =
          u32x4{o[0], o[1], o[2], o[3]};
  };
  auto dequant_part = [&](int tile, int m) __attribute__((always_inline)) {
    const Int8Part q = dq_load(tile, m);
    uint32_t o[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) dq_quarter(qq, q, o);
  };
  auto dequant_tile = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 4; ++m) dequant_part(tile, m);
  };

  // ---- per-lane LDS offsets of the MFMA operands (the swizzle XOR only touches bits of the
  // chunk index, so each operand is a per-lane base XOR a constant, plus an immediate):
  //   QK^T nope step c: (kbase ^ 32*(c % 8)) + 256*(c / 8); lane (n, g) reads key n, logical
  //     chunk 2c + g.
  //   QK^T rope step r: rbase ^ 32r; key n, logical rope chunk 2r + g.
  //   PV (key half kb, column block dc), read q: (vbase[q] ^ 64*(dc % 4)) + 256*(dc / 4) +
  //     16 KB*kb. Lane (G = lane/16, j = lane%16) of read q points at key 16kb + 8q + 4g + j/4
  //     and column 32dc + 16*(G & 1) + 4*(j & 3); it receives column 32dc + n of keys
  //     16kb + 8q + 4g + 0..3, the keys its P^T operand holds.
  const uint32_t kbase = n * kNopeRowBytes + 16 * (g ^ nope_swz(n));
  const uint32_t rbase = kNopeTileBytes + n * kRopeRowBytes + 16 * (g ^ rope_swz(n));
  uint32_t vbase[2];
  {
    const int j = lane & 15;
    const int tcol = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int key = 8 * q + 4 * g + (j >> 2);
      vbase[q] = key * kNopeRowBytes + 16 * (tcol ^ nope_swz(key)) + 8 * (j & 1);
    }
  }
  auto qk_operand = [&](uint32_t kst, uint32_t rst, int c) __attribute__((always_inline)) -> bf16x8 {
    if (kRopeW == 0 || c < 32) return lds_b128(smem_p + ((kst ^ (32u * (c & 7))) + 256u * (c >> 3)));
    return lds_b128(smem_p + (rst ^ (32u * (c - 32))));
  };
  // u = 16*kb + dc
  auto pv_operand = [&](uint32_t v0, uint32_t v1, int u) __attribute__((always_inline)) -> bf16x8 {
    const int dc = u & 15, kb = u >> 4;
    const uint32_t add = 256u * (dc >> 2) + 16384u * kb;
    const shortx4 x0 = lds_tr16(smem_p + ((v0 ^ (64u * (dc & 3))) + add));
    const shortx4 x1 = lds_tr16(smem_p + ((v1 ^ (64u * (dc & 3))) + add));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  bf16x8 qf[kQk];
  // S^T(tile) in one piece (the prologue's first tile)
  auto qk_tile = [&](uint32_t stage, floatx16& s) __attribute__((always_inline)) {
    const uint32_t kst = kbase + stage, rst = rbase + stage;
    bf16x8 qa[kQkDepth];
#pragma unroll
    for (int c = 0; c < kQkDepth; ++c) qa[c] = qk_operand(kst, rst, c);
#pragma unroll
    for (int c = 0; c < kQk; ++c) {
      const bf16x8 cur = qa[c % kQkDepth];
      if (c + kQkDepth < kQk) qa[c % kQkDepth] = qk_operand(kst, rst, c + kQkDepth);
      if (c == 0)
        mfma_qk_first(s, cur, qf[0]);
      else
        mfma_qk(s, cur, qf[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The P^T operands of the tile whose P.V runs next (hi and lo per key half): the softmax of a
  // tile runs one interval before its P.V.
  bf16x8 ph[2], pl[2];
  // The softmax of one tile in 19 pieces, placed between MFMAs. Scores s[r] are key
  // 8*(r/4) + 4g + (r%4) of the tile, head h; nk = valid keys of the tile. Produces the P^T
  // operands (oh, ol), updates the running max and sum, and decides the O rescale (alpha).
  struct Soft {
    float x[16];
    float mx, ls;
    uint32_t hw[2][4], lw[2][4];
  };
  auto soft_piece = [&](int c, bool first, int nk, const floatx16& sc, Soft& st, bf16x8 (&oh)[2],
                        bf16x8 (&ol)[2], float& alpha, bool& rescale) __attribute__((always_inline)) {
    if (c == 0) {
      st.mx = -INFINITY;
      st.ls = 0.f;
      if (nk >= kTile) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          st.x[r] = sc[r];
          st.mx = fmaxf(st.mx, st.x[r]);
        }
      } else {
        // keys past the partition's last valid row: -inf scores, so their p is exactly 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          st.x[r] = (8 * (r >> 2) + 4 * g + (r & 3)) < nk ? sc[r] : -INFINITY;
          st.mx = fmaxf(st.mx, st.x[r]);
        }
      }
    } else if (c == 1) {
      const float mt = pair_max(st.mx) * c_scale;  // the tile max in the exp2 domain
      if (first) {
        m_run = mt;  // first tile: O and l are still zero, nothing to rescale
      } else if (__any(mt > m_run + kRescaleThreshold)) {
        const bool need = mt > m_run + kRescaleThreshold;
        alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
        if (need) m_run = mt;
        l_run *= alpha;
        rescale = true;
      }
    } else if (c >= 2 && c < 10) {
      // p = 2^(c*x - m), two per piece (in place of x)
      const int r = 2 * (c - 2);
      st.x[r] = __builtin_amdgcn_exp2f(fmaf(st.x[r], c_scale, -m_run));
      st.x[r + 1] = __builtin_amdgcn_exp2f(fmaf(st.x[r + 1], c_scale, -m_run));
    } else if (c >= 10 && c < 18) {
      // P^T operands: hi = p truncated to bf16 (exact), lo = bf16(p - hi) (round to nearest
      // even), so hi + lo carries about 16 significant bits. For key half kb, element i of
      // lane (n, g) is result reg 8*kb + i.
      const int kb = (c - 10) >> 2, i = (c - 10) & 3;
      const float p0 = st.x[8 * kb + 2 * i], p1 = st.x[8 * kb + 2 * i + 1];
      const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
      st.ls += p0 + p1;
      st.hw[kb][i] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
      st.lw[kb][i] = pack_bf16x2(p0 - __uint_as_float(u0 & 0xffff0000u), p1 - __uint_as_float(u1 & 0xffff0000u));
    } else if (c == 18) {
      l_run += pair_sum(st.ls);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        oh[kb] = __builtin_bit_cast(bf16x8, uint4{st.hw[kb][0], st.hw[kb][1], st.hw[kb][2], st.hw[kb][3]});
        ol[kb] = __builtin_bit_cast(bf16x8, uint4{st.lw[kb][0], st.lw[kb][1], st.lw[kb][2], st.lw[kb][3]});
      }
    }
  };
  constexpr int kSoftPieces = 19;

  // One tile interval (tile i: P.V; tile i + 1: S^T and softmax), with the LDS reads of the two
  // kinds of MFMA spread over the whole interval (S^T operands at full LDS rate and the P.V
  // transpose reads together need about as many LDS clocks as the MFMAs take):
  //   A. the 36 (without rope channels 32) S^T(i + 1) steps, each followed by one P.V(i) MFMA
  //      of key half 0 (32 of them), with the DMA of a later tile issued in five pieces between
  //      them (INT8: and the dequantisation of tile i + 2);
  //   B. the 32 P.V(i) MFMAs of key half 1 with the softmax of tile i + 1 between them;
  //   C. an O rescale when tile i + 1 moved the running max (rare), after the P.V MFMAs, which
  //      still use the old max;
  //   D. the wait for the DMA the next interval needs, and the barrier.
  // bf16 issues tile i + 3 into the stage tile i - 1 left; INT8 issues the codes of tile i + 3
  // into the code buffer tile i + 1 left, and its rope rows into tile i's stage, whose rope part
  // S^T(i) has finished with.
  auto interval = [&](auto has_next_tag, int ti) __attribute__((always_inline)) {
    constexpr bool kHasNext = decltype(has_next_tag)::value;
    pin_agprs(oacc);
    const bool do_dma = ti + 3 < ntiles;
    int row_dma = 0;
    if (do_dma) row_dma = lane_row(ti + 3);
    const uint32_t st_cur = stage_of(ti);
    const uint32_t v0 = vbase[0] + st_cur, v1 = vbase[1] + st_cur;
    bf16x8 va[kPvDepth];
    floatx16 s_next;
    // INT8: tile i + 2's codes (fetched in the previous interval) are dequantised in part A,
    // from step 10 on. Without a tile i + 2 the same code runs on stale codes into the stage
    // tile i + 2 would use, which nothing reads before it is refilled: the loop has no branch.
    if (wave_active) {
#pragma unroll
      for (int u = 0; u < kPvDepth; ++u) va[u] = pv_operand(v0, v1, u);
    }
    if (kHasNext && wave_active) {
      const uint32_t st_next = stage_of(ti + 1);
      const uint32_t kst = kbase + st_next, rst = rbase + st_next;
      bf16x8 qa[kQkDepth];
      Int8Part dq_part;
      uint32_t dq_out[4];
#pragma unroll
      for (int c = 0; c < kQkDepth; ++c) qa[c] = qk_operand(kst, rst, c);
      __builtin_amdgcn_sched_barrier(0);
      // part A: S^T step c, then P.V MFMA c of key half 0 (u = c / 2, hi for even c, lo for odd)
#pragma unroll
      for (int c = 0; c < kQk; ++c) {
        const bf16x8 cur = qa[c % kQkDepth];
        if (c + kQkDepth < kQk) qa[c % kQkDepth] = qk_operand(kst, rst, c + kQkDepth);
        if (c == 0)
          mfma_qk_first(s_next, cur, qf[0]);
        else if (c + 1 == kQk)
          mfma_qk_last(s_next, cur, qf[c]);
        else if (c % kPieceStride == 5)
          mfma_qk_pad(s_next, cur, qf[c]);  // follows the conditional DMA piece of step c - 1
        else
          mfma_qk(s_next, cur, qf[c]);
        if (c < 32) {
          const int u = c >> 1;
          const bf16x8 vcur = va[u % kPvDepth];
          if (c & 1) {
            mfma_pv(oacc[u], vcur, pl[0]);
            if (u + kPvDepth < 32) va[u % kPvDepth] = pv_operand(v0, v1, u + kPvDepth);
          } else {
            mfma_pv(oacc[u], vcur, ph[0]);
          }
        }
        if constexpr (kInt8) {
          // part m's codes are read at step 6 + kDqStride m and converted a quarter at a time at
          // steps 8 + kDqStride m .. 11 + kDqStride m
          if (c == 6) {
            // tile i + 2's codes and scales have landed once at most its rope instruction (its
            // last, if any) and this interval's first piece (one instruction, step 4) are in
            // flight
            if (do_dma)
              wait_vmcnt<kRopeW ? 2 : 1>();
            else
              wait_vmcnt<kRopeW ? 1 : 0>();
          }
          if (c >= 6 && (c - 6) % kDqStride == 0 && (c - 6) / kDqStride < 4)
            dq_part = dq_load(ti + 2, (c - 6) / kDqStride);
          if (c >= 8 && (c - 8) % kDqStride < 4 && (c - 8) / kDqStride < 4)
            dq_quarter((c - 8) % kDqStride, dq_part, dq_out);
        }
        if (do_dma && c % kPieceStride == 4) issue_piece(ti + 3, row_dma, c / kPieceStride);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // no S^T to overlap (the last interval, or a wave without heads): the INT8 dequantisation
      // of tile i + 2 first (no DMA of this interval is in flight yet), then this interval's DMA
      if constexpr (kInt8) {
        if (ti + 2 < ntiles) {
          wait_vmcnt<0>();
          dequant_tile(ti + 2);
        }
      }
      if (do_dma) {
#pragma unroll
        for (int k = 0; k < 5; ++k) issue_piece(ti + 3, row_dma, k);
      }
      if (wave_active) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const bf16x8 vcur = va[u % kPvDepth];
          if (u + kPvDepth < 32) va[u % kPvDepth] = pv_operand(v0, v1, u + kPvDepth);
          mfma_pv(oacc[u], vcur, ph[0]);
          mfma_pv(oacc[u], vcur, pl[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) {
      // part B: key half 1 of P.V(i), the softmax of tile i + 1 between its MFMAs
      Soft st;
      bf16x8 nh[2], nl[2];
      float alpha = 1.0f;
      bool rescale = false;
      const int nk = n_valid - (ti + 1) * kTile;
#pragma unroll
      for (int u = 16; u < 32; ++u) {
        const bf16x8 cur = va[u % kPvDepth];
        if (u + kPvDepth < 32) va[u % kPvDepth] = pv_operand(v0, v1, u + kPvDepth);
        mfma_pv(oacc[u & 15], cur, ph[1]);
        if (kHasNext) {
          const int c0 = 2 * (u - 16) - 1;  // pieces 2(u-16) - 1 and 2(u-16): 0 .. 18 over u = 16 .. 25
          if (c0 >= 0 && c0 < kSoftPieces) soft_piece(c0, false, nk, s_next, st, nh, nl, alpha, rescale);
        }
        mfma_pv(oacc[u & 15], cur, pl[1]);
        if (kHasNext) {
          const int c1 = 2 * (u - 16);
          if (c1 < kSoftPieces) soft_piece(c1, false, nk, s_next, st, nh, nl, alpha, rescale);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kHasNext) {
        ph[0] = nh[0];
        ph[1] = nh[1];
        pl[0] = nl[0];
        pl[1] = nl[1];
      }
      if (rescale) rescale_agprs(oacc, alpha);
    }
    pin_agprs(oacc);
    // tile i + 2 must be in LDS for the next interval's S^T MFMAs (INT8: its rope rows; its nope
    // part this wave wrote itself)
    if (ti + 2 < ntiles) {
      if (do_dma)
        wait_vmcnt<kDmaPerTile>();
      else
        wait_vmcnt<0>();
    }
    lds_barrier();
  };

  // ---- prologue: the first tiles in flight; Q to bf16 operands; S^T(0) and its softmax.
  if (ntiles > 0) {
    if constexpr (kInt8) {
      // tiles 0 and 1 by DMA, dequantised in order; then tile 2's DMA
      issue_tile(0, lane_row(0));
      if (ntiles > 1) {
        issue_tile(1, lane_row(1));
        wait_vmcnt<kDmaPerTile>();
      } else {
        wait_vmcnt<0>();
      }
      dequant_tile(0);
      if (ntiles > 1) {
        wait_vmcnt<0>();
        dequant_tile(1);
      }
      if (ntiles > 2) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // the code reads of tile 0 are done before the refill
        issue_tile(2, lane_row(2));
      }
    } else {
      issue_tile(0, lane_row(0));
      if (ntiles > 1) issue_tile(1, lane_row(1));
      if (ntiles > 2) issue_tile(2, lane_row(2));
    }
  }
  {
    const uint32_t keep = head_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int c = 0; c < kQk; ++c) {
      const uint4 v = {(qv[c].x ^ q_sign) & keep, (qv[c].y ^ q_sign) & keep, (qv[c].z ^ q_sign) & keep,
                       (qv[c].w ^ q_sign) & keep};
      qf[c] = __builtin_bit_cast(bf16x8, v);
    }
  }
#pragma unroll
  for (int c = 0; c < kQk; ++c) asm volatile("" : "+v"(qf[c]));

  if (ntiles > 0) {
    if constexpr (!kInt8) {
      // tiles 0 and 1 must be in LDS (tile 2 may still be on its way)
      if (ntiles > 2)
        wait_vmcnt<kDmaPerTile>();
      else
        wait_vmcnt<0>();
    }
    lds_barrier();
    if (wave_active) {
      floatx16 s0;
      qk_tile(stage_of(0), s0);
      mfma_drain(s0);
      Soft st;
      float alpha = 1.0f;
      bool rescale = false;
#pragma unroll
      for (int c = 0; c < kSoftPieces; ++c) soft_piece(c, true, n_valid, s0, st, ph, pl, alpha, rescale);
    }
    // INT8 refills tile 0's rope rows (with tile 3) in the first interval: every wave must be
    // done with S^T(0) first
    if constexpr (kInt8) lds_barrier();
    int ti = 0;
    for (; ti + 1 < ntiles; ++ti) interval(std::integral_constant<bool, true>{}, ti);
    interval(std::integral_constant<bool, false>{}, ti);
  }
  mfma_pv_drain(oacc);

  // ---- epilogue: oacc[dc][4*rq + e] is column d = 32*dc + 8*rq + 4*g + e of head h.
  // The normalised bf16 O of a wave (32 heads x 512 columns) goes through LDS, so that each store
  // instruction writes one whole 1 KB output row instead of 64 scattered 8-byte pieces. Layout:
  // 32 KB per wave, row = head, 16-byte chunk c of a row at chunk c ^ row.
  lds_char_t* ob = (lds_char_t*)smem_p + wave * kOutWaveBytes;
  auto put_out = [&](int dc, int rq, const floatx4& v) __attribute__((always_inline)) {
    const u32x2 w{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    const int c = 4 * dc + rq;  // columns 8c .. 8c + 7
    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(ob + n * kNopeRowBytes + ((c ^ n) & 63) * 16 + 8 * g) = w;
  };
  // read back (the wave's own LDS accesses complete in order): lane L takes chunk L of row r.
  // The stores are non-temporal: the output is not read again here.
  // Only the 128-column blocks set in `blocks` are stored (lane L holds columns 8L .. 8L + 7).
  auto flush_out = [&](int blocks) __attribute__((always_inline)) {
    uint16_t* orow = a.out + ((int64_t)t * a.n_q + h0) * kNope + 8 * lane;
    const bool mine = (blocks >> (lane >> 4)) & 1;
#pragma unroll 8
    for (int r = 0; r < kHeadsPerWave; ++r) {
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          ob + r * kNopeRowBytes + ((lane ^ r) & 63) * 16);
      if (h0 + r < a.n_q && mine) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(orow + (int64_t)r * kNope));
    }
  };

  if (a.n_splits == 1) {
    lds_barrier();  // the stages are free once every wave is here
    if (wave_active) {
      const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
      for (int dc = 0; dc < 16; ++dc) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          put_out(dc, rq, agpr_quad(oacc[dc], rq) * inv);
      }
      flush_out(0xf);
    }
    return;
  }

  // Partitions of one token: each takes an arrival ticket (its arrival rank), and whoever merges
  // a head combines all partitions' partials of it in partition order, with one arithmetic shape,
  // so the result does not depend on the arrival order or on who merges. Two protocols:
  //
  // Spread (up to 16 partitions, every workgroup of the grid resident at once): the output is cut
  // into 16 units, (wave w, block hh of 128 columns), and unit (w, hh) is merged by the partition
  // whose arrival rank is w mod S (S <= 4: whole waves) or (w + 4 hh) mod S (S > 4). A partition
  // publishes each wave partial (64 KB) that another partition needs, so the merge is spread over
  // all S workgroups instead of funnelled through the last. A merging wave waits for the other
  // partitions' partials of its wave; partitions that arrived later may not be running, so an
  // early arrival's wait is bounded, and on a time-out it publishes its own partial and leaves
  // its units to the last arrival, which waits for that decision (every earlier arrival is
  // running, so the last arrival's waits end).
  //
  // Otherwise: all but the last publish their whole partial (unnormalised O in register-image
  // order [wave][dc][rq][lane] float4, and the running max and sum per head) and count
  // themselves ready; the last waits for that count and merges, with its own partial still in
  // registers. That wait is safe too: every partition it waits for has taken its ticket. A spin
  // limit still bounds every wait.
  //
  // Publication without an L2 write-back: the partials are written with agent-scope stores (the
  // sc1 form, which the L2 of this XCD writes through instead of holding dirty), so once this
  // wave's stores are acknowledged (vmcnt 0) they are visible to every XCD, and the flag or
  // count that follows needs no release fence. (A release fence would write back this XCD's
  // whole L2.) A merging wave takes an agent-scope acquire fence, which drops stale lines from
  // its own L2, before it reads a partial.
  const int S = a.n_splits;
  uint64_t* const cw = a.counters + (int64_t)t * kCounterWords;
  uint64_t* arrive = cw + kCntArrive;
  uint64_t* ready = cw + kCntReady;
  if (tid == 0) s_rank = (int)tagged_add(arrive, a.gen);
  lds_barrier();
  const int rank = s_rank;
  floatx4* part = reinterpret_cast<floatx4*>(a.part_o);
  constexpr int kWaveImage = 16 * 4 * 64;  // float4s per wave
  // this wave's partial: its O image and its heads' running max and sum
  auto publish = [&]() __attribute__((always_inline)) {
    floatx4* po = part + (((int64_t)t * S + sp) * kWaves + wave) * kWaveImage + lane;
#pragma unroll
    for (int dc = 0; dc < 16; ++dc) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const floatx4 v = agpr_quad(oacc[dc], rq);
        // A VALU write of a 128-bit store's data registers needs a wait state after the store;
        // the compiler does not see the store inside the asm, so the pad is part of it.
        asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(po + (dc * 4 + rq) * 64), "v"(v)
                     : "memory");
      }
    }
    if (g == 0) {
      uint64_t* ml = reinterpret_cast<uint64_t*>(a.part_ml) + ((int64_t)t * S + sp) * kMaxHeads + h;
      const uint64_t bits = (uint64_t)__float_as_uint(m_run) | ((uint64_t)__float_as_uint(l_run) << 32);
      __hip_atomic_store(ml, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
  };
  // O = sum_s w_s O_s / sum_s w_s l_s for this wave's heads, w_s = 2^(m_s - M), in partition
  // order as fused multiply-adds from zero, with this partition's own partial from its registers
  // and the others' from the workspace: the (m, l) of every partition first, then O four column
  // blocks at a time, each batch of loads issued together.
  auto merge = [&](int blocks) __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other partitions' partials
    const float2* mlp = reinterpret_cast<const float2*>(a.part_ml) + (int64_t)t * S * kMaxHeads + h;
    if (S == 2) {
      // the operations of the general case below for two partitions, with the other partition's
      // partial read in two batches of 32 loads per lane (two column blocks each)
      const float2 other = mlp[(1 - sp) * kMaxHeads];
      const float2 ml0 = sp == 0 ? make_float2(m_run, l_run) : other;
      const float2 ml1 = sp == 0 ? other : make_float2(m_run, l_run);
      const float mmax = fmaxf(ml0.x, ml1.x);
      const float w0 = ml0.x != -INFINITY ? __builtin_amdgcn_exp2f(ml0.x - mmax) : 0.f;
      const float w1 = ml1.x != -INFINITY ? __builtin_amdgcn_exp2f(ml1.x - mmax) : 0.f;
      const float lsum = __builtin_fmaf(w1, ml1.y, __builtin_fmaf(w0, ml0.y, 0.f));
      const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
      const floatx4* ps = part + (((int64_t)t * 2 + (1 - sp)) * kWaves + wave) * kWaveImage + lane;
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        if (!((blocks >> (2 * hp)) & 3)) continue;
        floatx4 buf[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) buf[i] = ps[(32 * hp + i) * 64];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int dc = 8 * hp + (i >> 2), rq = i & 3;
          const floatx4 own = agpr_quad(oacc[dc], rq);
          const floatx4 o0 = sp == 0 ? own : buf[i], o1 = sp == 0 ? buf[i] : own;
          floatx4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w1, o1[e], __builtin_fmaf(w0, o0[e], 0.f));
          put_out(dc, rq, acc * inv);
        }
      }
      flush_out(blocks);
      return;
    }
    float2 mlv[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      mlv[s] = s == sp ? make_float2(m_run, l_run) : s < S ? mlp[s * kMaxHeads] : make_float2(-INFINITY, 0.f);
    float mmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) mmax = s < S ? fmaxf(mmax, mlv[s].x) : mmax;
    float wv[kMaxSplits];
    float lsum = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      wv[s] = (s < S && mlv[s].x != -INFINITY) ? __builtin_amdgcn_exp2f(mlv[s].x - mmax) : 0.f;
      if (s < S) lsum = __builtin_fmaf(wv[s], mlv[s].y, lsum);
    }
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    const floatx4* pbase = part + ((int64_t)t * S * kWaves + wave) * kWaveImage + lane;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {  // column blocks 4hh .. 4hh + 3
      if (!((blocks >> hh) & 1)) continue;
      floatx4 acc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma nounroll
      for (int s = 0; s < S; ++s) {
        float w = 0.f;
#pragma unroll
        for (int u = 0; u < kMaxSplits; ++u) w = (u == s) ? wv[u] : w;
        // acc = fma(w, O_s, acc) in partition order, the same operations whether O_s comes from
        // this partition's registers or from memory
        if (s == sp) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int dc = 4 * hh + (i >> 2), rq = i & 3;
            const floatx4 o = agpr_quad(oacc[dc], rq);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][e] = __builtin_fmaf(w, o[e], acc[i][e]);
          }
        } else {
          const floatx4* ps = pbase + (int64_t)s * kWaves * kWaveImage + 16 * hh * 64;
          floatx4 buf[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) buf[i] = ps[i * 64];
#pragma unroll
          for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][e] = __builtin_fmaf(w, buf[i][e], acc[i][e]);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) put_out(4 * hh + (i >> 2), i & 3, acc[i] * inv);
    }
    flush_out(blocks);
  };
  // Lane 0 polls a tagged word until it is set (or, with a deadline, until the wall clock passes
  // it); the wave gets lane 0's last reading.
  auto poll = [&](uint64_t* p, uint64_t deadline) __attribute__((always_inline)) -> int {
    int v = 0;
    if (lane == 0) {
      for (int spin = 0; spin < kSpinLimit; ++spin) {
        v = (int)tagged_count(p, a.gen);
        if (v != 0 || (deadline != 0 && wall_clock64() > deadline)) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    return __builtin_amdgcn_readlane(v, 0);
  };
  auto set_word = [&](uint64_t* p, uint64_t v) __attribute__((always_inline)) {
    if (lane == 0) __hip_atomic_store(p, (a.gen << 16) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  if (S <= kMaxSpread && a.merge_wait_ticks > 0) {
    if (!wave_active) return;
    const bool last = rank == S - 1;
    int mine = 0, others = 0;  // this wave's column blocks merged here / by other partitions
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int m = S <= kWaves ? wave % S : (wave + kWaves * hh) % S;
      if (m == rank)
        mine |= 1 << hh;
      else
        others |= 1 << hh;
    }
    uint64_t* pub_mine = cw + kCntPublished + sp * kWaves + wave;
    uint64_t* decision = cw + kCntDecision + wave * 4;  // + hh
    // every other partition's partial of this wave (a bounded wait for an early arrival)
    auto others_published = [&](uint64_t deadline) __attribute__((always_inline)) -> bool {
      for (int q = 0; q < S; ++q)
        if (q != sp && poll(cw + kCntPublished + q * kWaves + wave, deadline) == 0) return false;
      return true;
    };
    if (others) {
      publish();
      set_word(pub_mine, 1);
    }
    int todo = 0;
    if (mine) {
      if (others_published(last ? 0 : wall_clock64() + (uint64_t)a.merge_wait_ticks)) {
        todo = mine;
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
          if ((mine >> hh) & 1) set_word(decision + hh, kMergedByFirst);
      } else {
        // a later partition has not published: leave these blocks to the last arrival
        if (!others) {
          publish();
          set_word(pub_mine, 1);
        }
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
          if ((mine >> hh) & 1) set_word(decision + hh, kPublishedByFirst);
      }
    }
    if (last && others) {
      // the mergers of the other blocks arrived earlier and are running: they decide, one word
      // per block, all of a merger's blocks at once (so one reading per merger)
      int left = 0, asked = 0;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        if (!((others >> hh) & 1) || ((asked >> hh) & 1)) continue;
        const int m = S <= kWaves ? wave % S : (wave + kWaves * hh) % S;
        int same = 0;  // the blocks of this wave that merger m takes
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if ((S <= kWaves ? wave % S : (wave + kWaves * k) % S) == m) same |= 1 << k;
        asked |= same;
        if (poll(decision + hh, 0) == (int)kPublishedByFirst) left |= same;
      }
      if (left && !mine) others_published(0);
      todo |= left;
    }
    if (todo) merge(todo);
    return;
  }

  if (rank != S - 1) {
    if (wave_active) publish();
    lds_barrier();
    if (tid == 0) tagged_add(ready, a.gen);
    return;
  }
  if (tid == 0) {
    for (int spin = 0; spin < kSpinLimit; ++spin) {
      if (tagged_count(ready, a.gen) >= (uint64_t)(S - 1)) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  lds_barrier();
  if (!wave_active) return;
  merge(0xf);
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

hipError_t launch_attention(const KernelArgs& a, bool int8_cache, bool window_slots, bool rope, hipStream_t stream) {
  const dim3 grid((unsigned)(a.n_tokens * a.n_splits * a.head_groups));
  const dim3 block(kThreads);
  KernelArgs copy = a;
  void* args[] = {&copy};
  // 32-bit byte offsets (and buffer sizes) cover every cache row while the pool holds fewer
  // than 4 Mi rows (4 GiB of bf16 nope)
  const bool buf = a.num_rows < (int64_t{1} << 22);
  const void* fn;
  // rows without rope channels come only through the window variants
  if (window_slots && !rope)
    fn = int8_cache ? (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<true, true, true, 0>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<true, false, true, 0>))
                    : (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<false, true, true, 0>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<false, false, true, 0>));
  else if (window_slots)
    fn = int8_cache ? (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<true, true, true, kRope>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<true, false, true, kRope>))
                    : (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<false, true, true, kRope>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<false, false, true, kRope>));
  else
    fn = int8_cache ? (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<true, true, false, kRope>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<true, false, false, kRope>))
                    : (buf ? reinterpret_cast<const void*>(&sfa_attention_kernel<false, true, false, kRope>)
                           : reinterpret_cast<const void*>(&sfa_attention_kernel<false, false, false, kRope>));
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
