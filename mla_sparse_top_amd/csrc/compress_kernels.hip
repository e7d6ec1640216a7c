// Compressor of the compressed latent cache: HIP kernel for gfx950 (CDNA4).
//
// What is computed ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section
// "Compressor", its computation steps): the projections kv and score (score already holding
// X W_gate, to which the slot's position embedding ape is added here) of each new token refresh
// the sequence's state; when position p + 1 is a multiple of the compression ratio, the state
// is pooled into one compressed entry. Per channel, the softmax over the state's slots of the
// scores weights the kv values; the weighted sum is RMS-normalised over its channels (times
// gamma), its last 64 channels are rotated in adjacent pairs by the RoPE angle of position p,
// with rotate = true the row then goes through the Sylvester Hadamard transform scaled by
// 1/sqrt(n), and the row is stored as bf16 at the entry's row of the compressed pool. Rows are
// 576 channels (the attention cache row: 512 to key_nope, 64 to key_rope), 512 (the same row in
// the page's D = 512 layout, rotary channels inside, whole to key_nope) or 128 (an index-key
// row, the page's D = 128 configuration, whole to key_nope).
//
// How: one workgroup per sequence, each thread owning a few channels, so every per-channel step
// (refresh, online softmax over the slots, scaling) runs in registers with no communication;
// the RMS needs one block reduction, RoPE pairs are adjacent lanes of the last wave (one xor
// shuffle), and the Hadamard transform's butterflies are xor shuffles across one wave. With a
// long window (ratio 10 and up) the workgroup holds several such channel groups, each taking a
// share of the slots with its own running max, sum and weighted sum, merged through LDS, so
// that the slot loads of a pooling go out several groups at a time. The tokens of a sequence
// are taken in order. A slot written earlier in the same call is read from
// the token's inputs rather than from the state, and only each slot's last writer stores it, so
// no address is both written and read in one call; every load can therefore be issued early, and
// the loads of a chunk of tokens, and of a batch of slots, go out together. The work is a few
// dependent memory round trips per sequence, not bandwidth: more workgroups would not shorten it.

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

// kC channels: 576 (the attention cache row, three waves, thread i owning channels i, i + 192,
// i + 384), 512 (two waves, thread i owning channels i + 128k, k < 4) or 128 (an index-key row,
// one wave, lane i owning channels i and i + 64). The rotary channels, the last 64, are the last
// register of the last wave's lanes in all three.
template <int kC>
constexpr int compress_threads() {
  return kC == 576 ? 192 : kC == 512 ? 128 : 64;
}
// kSplit channel groups of compress_threads<kC>() threads each: group g pools the slot batches
// g, g + kSplit, g + 2 kSplit, ... (all groups then hold the same merged row; group 0 stores).
template <int kC, bool kRotate, int kSplit>
__global__ void __launch_bounds__(compress_threads<kC>() * kSplit) compress_kernel(const CompressArgs a) {
  static_assert(!kRotate || kC == 128, "the Hadamard transform is built for 128 channels");
  constexpr int kT = compress_threads<kC>();  // threads of a channel group
  constexpr int kPer = kC / kT;             // channels per thread
  constexpr int kWaves = kT / 64;
  const int b = blockIdx.x;
  const int sg = threadIdx.x / kT;          // channel group
  const int tid = threadIdx.x - sg * kT;    // thread within the group
  const int lane = tid & 63;
  const int wave = tid >> 6;
  __shared__ float part[kSplit][kWaves];
  // the groups' running max, sum and weighted sum per channel, for the merge
  __shared__ float mrg[kSplit > 1 ? 3 * kSplit * kC : 1];

  const int64_t p0 = a.start_pos[b];
  // tokens with 0 <= p < rope_positions: a contiguous range of s
  const int64_t s_lo = p0 < 0 ? -p0 : 0;
  const int64_t s_hi = min((int64_t)a.s1, (int64_t)a.rope_positions - p0);
  const int64_t C = kC;

  // Tokens are taken in chunks: the inputs of a chunk are loaded together, and the slots a
  // pooling reads are loaded kSlotBatch at a time, so that a call waits on few memory round
  // trips (each load's address depends on nothing loaded).
  constexpr int kTokChunk = 4;
  constexpr int kSlotBatch = kSplit > 1 ? 4 : 8;  // the groups supply the rest of the parallelism
  for (int64_t s0 = s_lo; s0 < s_hi; s0 += kTokChunk) {
    float kv_c[kTokChunk][kPer], sc_c[kTokChunk][kPer];
#pragma unroll
    for (int j = 0; j < kTokChunk; ++j) {
      if (s0 + j >= s_hi) break;
      const int64_t t = (int64_t)b * a.s1 + s0 + j;
      const int slot = (int)((p0 + s0 + j) % a.ratio);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int c = tid + k * kT;
        kv_c[j][k] = a.kv[t * C + c];
        sc_c[j][k] = a.score[t * C + c] + a.ape[(int64_t)slot * C + c];
      }
    }
#pragma unroll
    for (int j = 0; j < kTokChunk; ++j) {
      const int64_t s = s0 + j;
      if (s >= s_hi) break;
      const int p = (int)(p0 + s);
      const int slot = p % a.ratio;
      const float* kv_t = kv_c[j];
      const float* sc_t = sc_c[j];
      if (sg == 0 && s + a.ratio >= s_hi) {  // no later token of this call refreshes this slot
        const int64_t o = ((int64_t)b * a.ratio + slot) * C;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          a.kv_state[o + tid + k * kT] = kv_t[k];
          a.score_state[o + tid + k * kT] = sc_t[k];
        }
      }
      if ((p + 1) % a.ratio != 0) continue;  // uniform over the workgroup

      // ---- pool: online softmax over the slots, per channel (group 0 starts from the token's
      // own slot, the others from nothing)
      float m[kPer], l[kPer], acc[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        m[k] = sg == 0 ? sc_t[k] : -INFINITY;
        l[k] = sg == 0 ? 1.0f : 0.0f;
        acc[k] = sg == 0 ? kv_t[k] : 0.0f;
      }
      // the other slots r = slot + 1 .. slot + ratio - 1 (mod ratio), kSlotBatch at a time, the
      // batches dealt to the groups in turn
      for (int r0 = 1 + sg * kSlotBatch; r0 < a.ratio; r0 += kSlotBatch * kSplit) {
        float kr[kSlotBatch][kPer], sr[kSlotBatch][kPer];
#pragma unroll
        for (int i = 0; i < kSlotBatch; ++i) {
          if (r0 + i >= a.ratio) break;
          const int r = (slot + r0 + i) % a.ratio;
          const int64_t back = a.ratio - r0 - i;  // slot r was last refreshed at p - back
          const int64_t sp = s - back;
          if (sp >= s_lo) {  // by a token of this call: take its inputs
            const int64_t tp = (int64_t)b * a.s1 + sp;
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
              const int c = tid + k * kT;
              kr[i][k] = a.kv[tp * C + c];
              sr[i][k] = a.score[tp * C + c] + a.ape[(int64_t)r * C + c];
            }
          } else {           // before this call: the stored state, which this call has not written
            const int64_t o = ((int64_t)b * a.ratio + r) * C;
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
              kr[i][k] = a.kv_state[o + tid + k * kT];
              sr[i][k] = a.score_state[o + tid + k * kT];
            }
          }
        }
#pragma unroll
        for (int i = 0; i < kSlotBatch; ++i) {
          if (r0 + i >= a.ratio) break;
#pragma unroll
          for (int k = 0; k < kPer; ++k) {
            const float mn = fmaxf(m[k], sr[i][k]);
            const float e_old = expf(m[k] - mn), e_new = expf(sr[i][k] - mn);
            l[k] = l[k] * e_old + e_new;
            acc[k] = acc[k] * e_old + e_new * kr[i][k];
            m[k] = mn;
          }
        }
      }
      if constexpr (kSplit > 1) {
        // merge the groups' partial poolings in group order: M = max m_g, L = sum l_g 2^.., A = ..
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int c = tid + k * kT;
          mrg[(0 * kSplit + sg) * kC + c] = m[k];
          mrg[(1 * kSplit + sg) * kC + c] = l[k];
          mrg[(2 * kSplit + sg) * kC + c] = acc[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int c = tid + k * kT;
          float mx = mrg[c];
#pragma unroll 4
          for (int g = 1; g < kSplit; ++g) mx = fmaxf(mx, mrg[g * kC + c]);
          float lt = 0.0f, at = 0.0f;
#pragma unroll 4
          for (int g = 0; g < kSplit; ++g) {
            const float e = expf(mrg[g * kC + c] - mx);  // 0 for a group that saw no slot
            lt = fmaf(mrg[(kSplit + g) * kC + c], e, lt);
            at = fmaf(mrg[(2 * kSplit + g) * kC + c], e, at);
          }
          l[k] = lt;
          acc[k] = at;
        }
        __syncthreads();  // mrg is rewritten by the next entry
      }
      float x[kPer], ss = 0.0f;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        x[k] = acc[k] / l[k];
        ss += x[k] * x[k];
      }

      // ---- RMSNorm over the kC channels
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
      float total = ss;
      if (kWaves > 1) {
        if (lane == 0) part[sg][wave] = ss;
        __syncthreads();
        total = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += part[sg][w];
        __syncthreads();  // part is rewritten by the next entry
      }
      const float inv = 1.0f / sqrtf(total / (float)kC + a.eps);
      float y[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) y[k] = x[k] * inv * a.gamma[tid + k * kT];

      // ---- RoPE: channel kC - 64 + j is the last register of lane j of the last wave; pair j/2
      // rotates by the angle of column j/2 of row p.
      const float partner = __shfl_xor(y[kPer - 1], 1, 64);
      if (wave == kWaves - 1) {
        const int i = lane >> 1;
        const float co = a.rope_cos[(int64_t)p * (kRope / 2) + i], si = a.rope_sin[(int64_t)p * (kRope / 2) + i];
        y[kPer - 1] = (lane & 1) ? fmaf(partner, si, y[kPer - 1] * co) : fmaf(-partner, si, y[kPer - 1] * co);
      }

      // ---- Hadamard transform (128 channels): the stride-64 butterfly is within a lane (channels
      // lane and lane + 64), the strides 32 .. 1 between lanes; then the 1/sqrt(128) scale.
      if (kRotate) {
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
#pragma unroll
        for (int k = 0; k < 2; ++k) y[k] *= 0.08838834764831845f;  // 1/sqrt(128)
      }

      // ---- store at the entry's row (group 0)
      if (sg != 0) continue;
      const int64_t c_entry = (p + 1) / a.ratio - 1;
      if (c_entry >= (int64_t)a.mb * 128) continue;
      const int blk = a.block_table[(int64_t)b * a.mb + (c_entry >> 7)];
      if (blk < 0) continue;
      const int64_t row = (int64_t)blk * 128 + (c_entry & 127);
      if (row >= a.num_rows) continue;
      if (kC == 576) {
        a.key_nope[row * kNope + tid] = bf16_rne(y[0]);
        a.key_nope[row * kNope + tid + kT] = bf16_rne(y[1]);
        if (wave < 2)
          a.key_nope[row * kNope + tid + 2 * kT] = bf16_rne(y[kPer - 1]);
        else
          a.key_rope[row * kRope + lane] = bf16_rne(y[kPer - 1]);
      } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k) a.key_nope[row * kC + tid + k * kT] = bf16_rne(y[k]);
      }
    }
  }
}

}  // namespace

template <int kC, bool kRotate>
void launch_one(const CompressArgs& a, hipStream_t stream) {
  // slot groups for a long window: up to 8 channel groups, within 1024 threads
  constexpr int kT = compress_threads<kC>();
  constexpr int kMaxSplit = kT <= 128 ? 8 : 4;
  if (a.ratio >= 10)
    hipLaunchKernelGGL((compress_kernel<kC, kRotate, kMaxSplit>), dim3(a.batch), dim3(kT * kMaxSplit), 0, stream, a);
  else
    hipLaunchKernelGGL((compress_kernel<kC, kRotate, 1>), dim3(a.batch), dim3(kT), 0, stream, a);
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  if (a.channels == 576)
    launch_one<576, false>(a, stream);
  else if (a.channels == 512)
    launch_one<512, false>(a, stream);
  else if (a.rotate)
    launch_one<128, true>(a, stream);
  else
    launch_one<128, false>(a, stream);
  return hipGetLastError();
}

}  // namespace sfa
