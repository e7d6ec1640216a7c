// Cache write of the paged MLA latent cache: HIP kernel for gfx950 (CDNA4).
//
// What is computed ("DeepSeek V3/V2 Sparse Flash Attention with Quantization", sections
// "Algorithm overview" (PagedAttention) and "INT8 quantisation rule"): each new token's latent
// row (512 nope + 64 rope, bf16) lands at the physical row that its logical position maps to
// through block_table. For an INT8 cache the nope part is quantised in groups of 128 elements:
// scale = absmax / 127 in fp32, code = round-half-even(x / scale) clamped to [-128, 127], with
// scale 0 and codes 0 for an all-zero group. The rope part (and a bf16 cache's nope part) is
// copied. Rows of the 512-wide layout ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation",
// D = 512: the rotary channels inside the row) have no rope part; the row is the 512 channels.
//
// How: the operation is a streaming copy with a little arithmetic, bound by HBM. A wave writes
// four new tokens: lane L holds the 16-byte chunk L of a 1 KB nope row, so a 128-element group
// is 16 consecutive lanes and its absolute maximum is a 4-step butterfly inside the group. The
// wave issues the loads of all four rows before it resolves where they go, so the position ->
// block-table round trips overlap the row reads (measured: 289 -> 181 us for 524,288 INT8 rows
// against resolving first; 8 or 16 tokens per wave measured slower than 4). Stores are whole 512-byte code rows
// (8 bytes per lane), whole 1 KB bf16 rows, 128-byte rope rows and one 16-byte scale quad per
// row, all coalesced.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cache_internal.h"

namespace sfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kNopeBytes = 1024;  // bf16 nope row
constexpr int kRopeBytes = 128;   // bf16 rope row
constexpr int kCodeBytes = 512;   // int8 nope row

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// code = clamp(round-half-even(fp32(x / scale)), -128, 127) as a byte. x / scale is the IEEE
// fp32 division (correctly rounded; fp32 denormals are kept) and rintf rounds ties to even. The
// division's VALU work hides under the memory traffic: a multiply by a reciprocal with an exact
// fallback near ties measured no faster.
__device__ __forceinline__ uint32_t code_byte(float x, float scale) {
  const float q = fminf(fmaxf(rintf(x / scale), -128.0f), 127.0f);
  return (uint32_t)(int32_t)q & 0xffu;
}

template <bool kInt8, bool kRope>
__global__ void __launch_bounds__(kCwWaves * 64) cache_write_kernel(const CacheWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * kCwWaves + wave) * kCwRowsPerWave;

  // ---- lane i < kCwRowsPerWave resolves token t0 + i: its position is loaded first; the new
  // rows, which do not depend on where they go, are loaded next; then the block-table entry. Vector loads
  // complete in issue order, so the block-table read waits only for the position, and its round
  // trip overlaps the row reads.
  static_assert(kCwRowsPerWave <= 64 && (kCwRowsPerWave & (kCwRowsPerWave - 1)) == 0, "one lane per token of the wave");
  const int ti = t0 + (lane & (kCwRowsPerWave - 1));
  const bool tok_lane = lane < kCwRowsPerWave && ti < a.n_tokens;
  const int pos = tok_lane ? a.positions[ti] : -1;
  u32x4 nv[kCwRowsPerWave], rv[kCwRowsPerWave];
#pragma unroll
  for (int i = 0; i < kCwRowsPerWave; ++i) {
    const int64_t t = min(t0 + i, a.n_tokens - 1);
    nv[i] = reinterpret_cast<const u32x4*>(a.new_nope + t * 512)[lane];
    if constexpr (kRope) rv[i] = reinterpret_cast<const u32x4*>(a.new_rope + t * 64)[lane & 7];
  }
  const bool pos_ok = pos >= 0 && pos < a.mb * 128;
  const int blk = pos_ok ? a.block_table[(int64_t)(ti / a.s1) * a.mb + (pos >> 7)] : -1;
  const int64_t row_l = (int64_t)blk * 128 + (pos & 127);
  const int32_t row_lane = (blk >= 0 && row_l < a.num_rows) ? (int32_t)row_l : -1;  // rows < 2^31
  int64_t row[kCwRowsPerWave];
#pragma unroll
  for (int i = 0; i < kCwRowsPerWave; ++i) row[i] = __builtin_amdgcn_readlane(row_lane, i);

#pragma unroll
  for (int i = 0; i < kCwRowsPerWave; ++i) {
    if (row[i] < 0) continue;
    const int64_t r = row[i];
    if (kRope && lane < 8) reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.key_rope) + r * kRopeBytes)[lane] = rv[i];
    if constexpr (!kInt8) {
      reinterpret_cast<u32x4*>(static_cast<char*>(a.key_nope) + r * kNopeBytes)[lane] = nv[i];
    } else {
      const uint32_t w[4] = {nv[i][0], nv[i][1], nv[i][2], nv[i][3]};
      float x[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_lo(w[k]);
        x[2 * k + 1] = bf16_hi(w[k]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
      // the group is lanes 16g .. 16g+15: butterfly over the low four lane bits
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
      const float scale = amax / 127.0f;
      uint32_t lo = 0, hi = 0;
      if (scale != 0.0f) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo |= code_byte(x[k], scale) << (8 * k);
          hi |= code_byte(x[4 + k], scale) << (8 * k);
        }
      }
      reinterpret_cast<u32x2*>(static_cast<char*>(a.key_nope) + r * kCodeBytes)[lane] = u32x2{lo, hi};
      if ((lane & 15) == 0) a.scales[r * 4 + (lane >> 4)] = scale;
    }
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, bool int8_cache, bool rope, hipStream_t stream) {
  const int grid = (a.n_tokens + kCwTokensPerWg - 1) / kCwTokensPerWg;
  const dim3 block(kCwWaves * 64);
  if (int8_cache && rope)
    hipLaunchKernelGGL((cache_write_kernel<true, true>), dim3(grid), block, 0, stream, a);
  else if (int8_cache)
    hipLaunchKernelGGL((cache_write_kernel<true, false>), dim3(grid), block, 0, stream, a);
  else if (rope)
    hipLaunchKernelGGL((cache_write_kernel<false, true>), dim3(grid), block, 0, stream, a);
  else
    hipLaunchKernelGGL((cache_write_kernel<false, false>), dim3(grid), block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfa
