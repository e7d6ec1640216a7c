// Lightning Indexer scores and top-k selection: HIP kernels for gfx950 (CDNA4).
//
// What is computed ("CANN DeepSeek Indexer attention optimisation", sections "Lightning
// Indexer" and "Sparse Flash Attention"): for query token i and cache position j,
// I[i, j] = sum over the 64 index heads h of w[i, h] * ReLU(q_index[i, h] . k_index[j]); then
// the k positions with the largest I[i, :] are the token's top-k set for sparse attention.
// How it is computed here:
//
//   * Scores: a workgroup owns one 128-position page of one batch and up to 8 of its query
//     tokens. Each wave takes 32 positions. Their index keys (32 rows x 256 bytes, one
//     contiguous run of the page) are loaded straight into the B operand layout of
//     v_mfma_f32_32x32x16_bf16 and stay in registers while the wave runs the tokens: per token,
//     S^T = Q . K^T with the 64 heads on M (two 32-head blocks) and the positions on N, 8
//     k-steps over the 128 dims. Each lane then holds one position and 16 heads of each block,
//     so the ReLU, the head weighting and the sum over heads are in-lane, plus one cross-lane
//     add. Positions past the live length (and whole dead pages) score -inf.
//   * Top-k: one workgroup per token runs a most-significant-digit-first radix select over the
//     scores' order-preserving 32-bit keys: four 8-bit histogram passes in LDS find the k-th
//     largest key exactly and how many of the keys equal to it belong to the top k. A last pass
//     writes the positions above that key, then the first of the equal ones in position
//     order, at offsets from block-wide prefix sums. The output is unsorted.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "indexer_internal.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kScoreThreads = 256;  // 4 waves x 32 positions = one page
constexpr int kSelectThreads = 256;

__global__ void __launch_bounds__(kScoreThreads) indexer_scores_kernel(const IndexerArgs a) {
  const int jb = blockIdx.x;                  // logical page
  const int b = blockIdx.y / a.chunks;
  const int c = blockIdx.y - b * a.chunks;
  const int t0 = b * a.s1 + c * kIdxTokenChunk;
  const int t1 = min(b * a.s1 + a.s1, t0 + kIdxTokenChunk);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;  // position within the wave's 32 (B operand column, result column)
  const int g = lane >> 5;  // k-group of the operands / row-quad parity of the result
  const int pos = jb * kIdxBlock + wave * 32 + n;
  const int lim = min(a.act[b], a.n_pos);

  int blk = -1;
  if (jb * kIdxBlock < lim) blk = a.block_table[(int64_t)b * a.mb + jb];
  if (blk < 0 || (int64_t)(blk + 1) * kIdxBlock > a.num_rows) {
    // a page with no live position (or an invalid block-table entry): every score is -inf
    for (int t = t0; t < t1; ++t)
      if (g == 0) a.scores[(int64_t)t * a.n_pos + pos] = -INFINITY;
    return;
  }

  // K^T operand (B[k][n]): lane (n, g) holds dims 16*ks + 8*g .. +7 of this position's key
  const uint4* krow = reinterpret_cast<const uint4*>(a.k + ((int64_t)blk * kIdxBlock + wave * 32 + n) * kIdxDim);
  bf16x8 kop[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kop[ks] = __builtin_bit_cast(bf16x8, krow[2 * ks + g]);

  for (int t = t0; t < t1; ++t) {
    // Q operand (A[m][k]): lane (n, g) holds dims 16*ks + 8*g .. +7 of head 32*hb + n
    const uint4* q0 = reinterpret_cast<const uint4*>(a.q + ((int64_t)t * kIdxHeads + n) * kIdxDim);
    const uint4* q1 = q0 + 32 * kIdxDim / 8;
    floatx16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q0[2 * ks + g]), kop[ks], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q1[2 * ks + g]), kop[ks], acc1, 0, 0, 0);
    }
    // acc_hb[r] is head 32*hb + 8*(r/4) + 4*g + (r%4) at this lane's position
    const float4* wr = reinterpret_cast<const float4*>(a.w + (int64_t)t * kIdxHeads);
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 w0 = wr[2 * q + g];      // heads 8q + 4g .. +3
      const float4 w1 = wr[8 + 2 * q + g];  // heads 32 + 8q + 4g .. +3
      s += w0.x * fmaxf(acc0[4 * q], 0.f) + w0.y * fmaxf(acc0[4 * q + 1], 0.f) +
           w0.z * fmaxf(acc0[4 * q + 2], 0.f) + w0.w * fmaxf(acc0[4 * q + 3], 0.f);
      s += w1.x * fmaxf(acc1[4 * q], 0.f) + w1.y * fmaxf(acc1[4 * q + 1], 0.f) +
           w1.z * fmaxf(acc1[4 * q + 2], 0.f) + w1.w * fmaxf(acc1[4 * q + 3], 0.f);
    }
    s += __shfl_xor(s, 32);  // the other 32 heads of each block sit in the partner lane
    if (g == 0) a.scores[(int64_t)t * a.n_pos + pos] = pos < lim ? s : -INFINITY;
  }
}

// Order-preserving map of a float onto uint32: a larger float gives a larger key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum of v over the workgroup (kSelectThreads threads); `tmp` holds 4 ints.
__device__ __forceinline__ int block_inclusive_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(v, d);
    if (lane >= d) v += up;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int w = 0; w < kSelectThreads / 64; ++w) add += (w < wave) ? tmp[w] : 0;
  __syncthreads();
  return v + add;
}

__global__ void __launch_bounds__(kSelectThreads) topk_select_kernel(const IndexerArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int scan_tmp[kSelectThreads / 64];
  __shared__ uint32_t s_digit;
  __shared__ int s_remaining;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = t / a.s1;
  const int n = max(0, min(a.act[b], a.n_pos));
  const int K = a.topk;
  int32_t* out = a.topk_out + (int64_t)t * K;
  const float* sc = a.scores + (int64_t)t * a.n_pos;

  if (n <= K) {  // every live position is selected
    for (int i = tid; i < K; i += kSelectThreads) out[i] = i < n ? i : -1;
    return;
  }

  // k-th largest key, digit by digit from the top
  uint32_t prefix = 0, mask = 0;
  int remaining = K;  // how many still to take among keys matching the prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelectThreads) {
      const uint32_t key = order_key(sc[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread tid looks at digit 255 - tid: its inclusive sum counts the keys at or above it
    const int h = (int)hist[255 - tid];
    const int incl = block_inclusive_scan(h, scan_tmp);
    if (incl >= remaining && incl - h < remaining) {
      s_digit = 255u - (uint32_t)tid;
      s_remaining = remaining - (incl - h);
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    remaining = s_remaining;
    __syncthreads();
  }
  // prefix is the k-th largest key; `remaining` of the keys equal to it are taken, the first
  // ones in position order, after the K - remaining keys above it
  const uint32_t kth = prefix;
  const int need = remaining;
  const int chunk = (n + kSelectThreads - 1) / kSelectThreads;
  const int i0 = min(n, tid * chunk), i1 = min(n, i0 + chunk);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = order_key(sc[i]);
    gt += key > kth ? 1 : 0;
    eq += key == kth ? 1 : 0;
  }
  int off_gt = block_inclusive_scan(gt, scan_tmp) - gt;
  int off_eq = block_inclusive_scan(eq, scan_tmp) - eq;
  const int base_eq = K - need;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = order_key(sc[i]);
    if (key > kth) {
      out[off_gt++] = i;
    } else if (key == kth) {
      if (off_eq < need) out[base_eq + off_eq] = i;
      ++off_eq;
    }
  }
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.mb, (unsigned)(a.batch * a.chunks));
  IndexerArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&indexer_scores_kernel), grid, dim3(kScoreThreads), args, 0,
                         stream);
}

hipError_t launch_topk_select(const IndexerArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.batch * a.s1));
  IndexerArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&topk_select_kernel), grid, dim3(kSelectThreads), args, 0,
                         stream);
}

}  // namespace sfa
