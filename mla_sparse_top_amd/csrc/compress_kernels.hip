// Compressor of the compressed latent cache: HIP kernel for gfx950 (CDNA4).
//
// What is computed ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section
// "Compressor", its computation steps): the projections kv and score (score already holding
// X W_gate, to which the slot's position embedding ape is added here) of each new token refresh
// the sequence's state; when position p + 1 is a multiple of the compression ratio, the state
// is pooled into one compressed entry. Per channel, the softmax over the state's slots of the
// scores weights the kv values; the weighted sum is RMS-normalised over its 576 channels (times
// gamma), its last 64 channels are rotated in adjacent pairs by the RoPE angle of position p,
// and the row is stored as bf16 at the entry's row of the compressed pool.
//
// How: one workgroup per sequence, three waves, each thread owning three channels, so every
// per-channel step (refresh, online softmax over the slots, scaling) runs in registers with no
// communication; the RMS needs one block reduction, and RoPE pairs are adjacent lanes of the
// third wave (one xor shuffle). The tokens of a sequence are taken in order. A slot written
// earlier in the same call is read from the token's inputs rather than from the state, and only
// each slot's last writer stores it, so no address is both written and read in one call.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "compress_internal.h"

namespace sfa {
namespace {

constexpr int kNope = 512;
constexpr int kRope = 64;

// fp32 -> bf16 bits, rounded to nearest with ties to even (a NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ void __launch_bounds__(kCmpThreads) compress_kernel(const CompressArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  __shared__ float part[kCmpThreads / 64];

  const int64_t p0 = a.start_pos[b];
  // tokens with 0 <= p < rope_positions: a contiguous range of s
  const int64_t s_lo = p0 < 0 ? -p0 : 0;
  const int64_t s_hi = min((int64_t)a.s1, (int64_t)a.rope_positions - p0);
  const int64_t C = kCmpChannels;

  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int p = (int)(p0 + s);
    const int64_t t = (int64_t)b * a.s1 + s;
    const int slot = p % a.ratio;
    float kv_t[kCmpPerThread], sc_t[kCmpPerThread];
#pragma unroll
    for (int k = 0; k < kCmpPerThread; ++k) {
      const int c = tid + k * kCmpThreads;
      kv_t[k] = a.kv[t * C + c];
      sc_t[k] = a.score[t * C + c] + a.ape[(int64_t)slot * C + c];
    }
    if (s + a.ratio >= s_hi) {  // no later token of this call refreshes this slot
      const int64_t o = ((int64_t)b * a.ratio + slot) * C;
#pragma unroll
      for (int k = 0; k < kCmpPerThread; ++k) {
        a.kv_state[o + tid + k * kCmpThreads] = kv_t[k];
        a.score_state[o + tid + k * kCmpThreads] = sc_t[k];
      }
    }
    if ((p + 1) % a.ratio != 0) continue;  // uniform over the workgroup

    // ---- pool: online softmax over the slots, per channel
    float m[kCmpPerThread], l[kCmpPerThread], acc[kCmpPerThread];
#pragma unroll
    for (int k = 0; k < kCmpPerThread; ++k) {
      m[k] = sc_t[k];
      l[k] = 1.0f;
      acc[k] = kv_t[k];
    }
    for (int r = 0; r < a.ratio; ++r) {
      if (r == slot) continue;
      const int64_t back = (slot - r + a.ratio) % a.ratio;  // slot r was last refreshed at p - back
      const int64_t sp = s - back;
      float kr[kCmpPerThread], sr[kCmpPerThread];
      if (sp >= s_lo) {  // by a token of this call: take its inputs
        const int64_t tp = (int64_t)b * a.s1 + sp;
#pragma unroll
        for (int k = 0; k < kCmpPerThread; ++k) {
          const int c = tid + k * kCmpThreads;
          kr[k] = a.kv[tp * C + c];
          sr[k] = a.score[tp * C + c] + a.ape[(int64_t)r * C + c];
        }
      } else {           // before this call: the stored state, which this call has not written
        const int64_t o = ((int64_t)b * a.ratio + r) * C;
#pragma unroll
        for (int k = 0; k < kCmpPerThread; ++k) {
          kr[k] = a.kv_state[o + tid + k * kCmpThreads];
          sr[k] = a.score_state[o + tid + k * kCmpThreads];
        }
      }
#pragma unroll
      for (int k = 0; k < kCmpPerThread; ++k) {
        const float mn = fmaxf(m[k], sr[k]);
        const float e_old = expf(m[k] - mn), e_new = expf(sr[k] - mn);
        l[k] = l[k] * e_old + e_new;
        acc[k] = acc[k] * e_old + e_new * kr[k];
        m[k] = mn;
      }
    }
    float x[kCmpPerThread], ss = 0.0f;
#pragma unroll
    for (int k = 0; k < kCmpPerThread; ++k) {
      x[k] = acc[k] / l[k];
      ss += x[k] * x[k];
    }

    // ---- RMSNorm over the 576 channels
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    const float total = part[0] + part[1] + part[2];
    __syncthreads();  // part is rewritten by the next entry
    const float inv = 1.0f / sqrtf(total / (float)kCmpChannels + a.eps);
    float y[kCmpPerThread];
#pragma unroll
    for (int k = 0; k < kCmpPerThread; ++k) y[k] = x[k] * inv * a.gamma[tid + k * kCmpThreads];

    // ---- RoPE: channel 512 + j is y[2] of thread 128 + j (the third wave); pair j/2 rotates by
    // the angle of column j/2 of row p.
    const float partner = __shfl_xor(y[2], 1, 64);
    if (wave == 2) {
      const int i = lane >> 1;
      const float co = a.rope_cos[(int64_t)p * (kRope / 2) + i], si = a.rope_sin[(int64_t)p * (kRope / 2) + i];
      y[2] = (lane & 1) ? fmaf(partner, si, y[2] * co) : fmaf(-partner, si, y[2] * co);
    }

    // ---- store at the entry's row
    const int64_t c_entry = (p + 1) / a.ratio - 1;
    if (c_entry >= (int64_t)a.mb * 128) continue;
    const int blk = a.block_table[(int64_t)b * a.mb + (c_entry >> 7)];
    if (blk < 0) continue;
    const int64_t row = (int64_t)blk * 128 + (c_entry & 127);
    if (row >= a.num_rows) continue;
    a.key_nope[row * kNope + tid] = bf16_rne(y[0]);
    a.key_nope[row * kNope + tid + kCmpThreads] = bf16_rne(y[1]);
    if (wave < 2)
      a.key_nope[row * kNope + tid + 2 * kCmpThreads] = bf16_rne(y[2]);
    else
      a.key_rope[row * kRope + lane] = bf16_rne(y[2]);
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(compress_kernel, dim3(a.batch), dim3(kCmpThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfa
