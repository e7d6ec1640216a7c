// Lightning Indexer scores and top-k selection: HIP kernels for gfx950 (CDNA4).
//
// What is computed ("CANN DeepSeek Indexer attention optimisation", sections "Lightning
// Indexer" and "Sparse Flash Attention"): for query token i and cache position j,
// I[i, j] = sum over the 64 index heads h of w[i, h] * ReLU(q_index[i, h] . k_index[j]); then
// the k positions with the largest I[i, :] are the token's top-k set for sparse attention.
// How it is computed here:
//
//   * Scores: a workgroup owns up to 4 query tokens of one batch and a run of that batch's
//     128-position pages. It first copies the tokens' index queries (16 KB each) and head
//     weights into LDS. Each wave then takes 32 positions of every page: their index keys (32
//     rows x 256 bytes, one contiguous run of the page) are loaded straight into the B operand
//     layout of v_mfma_f32_32x32x16_bf16, the next page's keys in flight while this page runs.
//     Per token, S^T = Q . K^T has the 64 heads on M (two 32-head blocks, A operand read from
//     LDS) and the positions on N, 8 k-steps over the 128 dims. Each lane then holds one
//     position and 16 heads of each block, so the ReLU, the head weighting and the sum over
//     heads are in-lane, plus one cross-lane add. Positions past the live length (and whole
//     dead pages) score -inf.
//   * Top-k: one workgroup of 1024 threads per token runs a most-significant-digit-first radix
//     select over the scores' order-preserving 32-bit keys, held in LDS when a token has at most
//     32768 positions. Three histogram passes (12, 10 and 10 bits) find the k-th largest key
//     exactly and how many of the keys equal to it belong to the top k; when the k-th key's
//     12-bit bin holds at most 1024 keys, the last two passes run over that bin's keys alone. A
//     last pass writes the positions above that key, then the first of the equal ones in
//     position order, at offsets from block-wide prefix sums. The row is staged in LDS and stored
//     whole when topk <= 4096. The output is unsorted.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "indexer_internal.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kScoreThreads = 256;  // 4 waves x 32 positions = one page
constexpr int kRowPieces = kIdxDim * 2 / 16;  // 16-byte pieces of a 256-byte q or k row
constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;

// Buffer resource over the index keys of one page: 128 rows x 256 bytes from the page's first
// row, or an empty range (every load returns zeros) for a page that is not read.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* k, int blk) {
  const uint16_t* base = blk >= 0 ? k + (int64_t)blk * kIdxBlock * kIdxDim : k;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, blk >= 0 ? kIdxBlock * kIdxDim * 2 : 0,
                                           0x00020000);
}

// Index keys of one wave's 32 positions of a page, in the B operand layout: lane (n, g) holds
// dims 16*ks + 8*g .. +7 of position n's key in kop[ks].
__device__ __forceinline__ void load_keys(bf16x8 (&kop)[8], __amdgpu_buffer_rsrc_t r, int wave, int n, int g) {
  const int voff = (wave * 32 + n) * kIdxDim * 2 + g * 16;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    kop[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff + ks * 32, 0, 0));
}

// Physical block of logical page p, or -1 when the page holds no live position or the table
// entry does not name a block inside the cache.
__device__ __forceinline__ int page_block(const IndexerArgs& a, int b, int p, int lim) {
  const int blk = a.block_table[(int64_t)b * a.mb + p];  // p < mb: always inside the table
  return (p * kIdxBlock >= lim || blk < 0 || (int64_t)(blk + 1) * kIdxBlock > a.num_rows) ? -1 : blk;
}

// Scores of one page for the workgroup's NT tokens; q_s holds the tokens' queries with the
// 16-byte pieces of head h's row XOR-swizzled by (h & 15), w_s their head weights.
template <int NT>
__device__ __forceinline__ void score_page(const IndexerArgs& a, const bf16x8 (&kop)[8], bool live_page, int p,
                                           int t0, int lim, const uint4* q_s, const float4* w_s, int wave, int n,
                                           int g) {
  const int pos = p * kIdxBlock + wave * 32 + n;
  const bool live = live_page && pos < lim;
#pragma unroll
  for (int tok = 0; tok < NT; ++tok) {
    // one token and one 32-head block at a time: a single 16-register accumulator, and the
    // compiler can count the outstanding key loads exactly
    float v = 0.f;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      __builtin_amdgcn_sched_barrier(0);
      const uint4* qh = q_s + (tok * kIdxHeads + 32 * hb + n) * kRowPieces;  // head 32*hb + n
      floatx16 acc = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qh[(2 * ks + g) ^ (n & 15)]), kop[ks],
                                                      acc, 0, 0, 0);
      // acc[r] is head 32*hb + 8*(r/4) + 4*g + (r%4) at this lane's position
      const float4* wr = w_s + tok * (kIdxHeads / 4) + 8 * hb;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 w = wr[2 * q + g];  // heads 32*hb + 8q + 4g .. +3
        v += w.x * fmaxf(acc[4 * q], 0.f) + w.y * fmaxf(acc[4 * q + 1], 0.f) + w.z * fmaxf(acc[4 * q + 2], 0.f) +
             w.w * fmaxf(acc[4 * q + 3], 0.f);
      }
    }
    v += __shfl_xor(v, 32);  // the other 16 heads of each row quad sit in the partner lane
    if (g == 0) a.scores[(int64_t)(t0 + tok) * a.n_pos + pos] = live ? v : -INFINITY;
  }
}

template <int NT>
__device__ __forceinline__ void scores_body(const IndexerArgs& a, uint4* q_s, float4* w_s, const int (&blk)[kIdxMaxPagesPerWg],
                                            int t0, int p0, int p1, int lim) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;  // position within the wave's 32 (B operand column, result column)
  const int g = lane >> 5;  // k-group of the operands / row-quad parity of the result

  // The first batch of query pieces and the weights are requested before the first page's keys,
  // so that (loads return in order) staging them does not wait for the keys. Every thread loads
  // and stores a weight vector (clamped index, w_s has a slot per thread) so that the load is
  // unconditional and queues with the others.
  constexpr int kQ = NT * kIdxHeads * kRowPieces / kScoreThreads;  // 16-byte pieces per thread
  constexpr int kStep = kQ < 8 ? kQ : 8;                            // staged 8 at a time
  const uint4* qg = reinterpret_cast<const uint4*>(a.q) + (int64_t)t0 * kIdxHeads * kRowPieces;
  const float4 wv = reinterpret_cast<const float4*>(a.w + (int64_t)t0 * kIdxHeads)[min(tid, NT * kIdxHeads / 4 - 1)];
  bf16x8 kbuf[2][8];
#pragma unroll
  for (int j0 = 0; j0 < kQ; j0 += kStep) {
    uint4 qv[kStep];
#pragma unroll
    for (int j = 0; j < kStep; ++j) qv[j] = qg[tid + (j0 + j) * kScoreThreads];
    if (j0 == 0) load_keys(kbuf[0], page_rsrc(a.k, blk[0]), wave, n, g);
#pragma unroll
    for (int j = 0; j < kStep; ++j) {
      const int i = tid + (j0 + j) * kScoreThreads;
      const int h = (i / kRowPieces) & (kIdxHeads - 1);
      q_s[(i & ~(kRowPieces - 1)) | ((i & (kRowPieces - 1)) ^ (h & 15))] = qv[j];
    }
  }
  w_s[tid] = wv;
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kIdxMaxPagesPerWg; ++i) {
    if (p0 + i >= p1) break;
    if (i + 1 < kIdxMaxPagesPerWg) load_keys(kbuf[(i + 1) & 1], page_rsrc(a.k, blk[i + 1]), wave, n, g);
    score_page<NT>(a, kbuf[i & 1], blk[i] >= 0, p0 + i, t0, lim, q_s, w_s, wave, n, g);
  }
}

// Accumulators in arch VGPRs (no AGPRs) within a budget of four waves per SIMD (128 registers).
// Measured: a split VGPR/AGPR allocation of 148 registers ran only two waves per SIMD, where 154
// arch VGPRs ran three.
__global__ void __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) indexer_scores_kernel(const IndexerArgs a) {
  extern __shared__ uint4 q_s[];  // nt tokens x 64 heads x 16 pieces
  __shared__ float4 w_s[kScoreThreads];  // the first nt * 16 hold the tokens' head weights
  // Consecutive workgroups go to the 8 XCDs in turn. Renumber them so that each XCD runs whole
  // rows of the grid (all page runs of the same tokens): a token's queries then reach one XCD's
  // L2 instead of all eight.
  const unsigned n_wg = gridDim.x * gridDim.y;
  unsigned id = blockIdx.y * gridDim.x + blockIdx.x;
  if ((n_wg & 7u) == 0) id = (id & 7u) * (n_wg >> 3) + (id >> 3);
  const int row = (int)(id / gridDim.x);  // b * chunks + c
  const int b = row / a.chunks;
  const int c = row - b * a.chunks;
  const int t0 = b * a.s1 + c * kIdxTokenChunk;
  const int nt = min(kIdxTokenChunk, a.s1 - c * kIdxTokenChunk);
  const int p0 = (int)(id - (unsigned)row * gridDim.x) * a.pages_per_wg;
  const int p1 = min(a.mb, p0 + a.pages_per_wg);
  const int lim = min(a.act[b], a.n_pos);

  if (p0 * kIdxBlock >= lim) {  // nothing live in the whole run of pages
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int p = p0; p < p1; ++p)
      for (int tok = 0; tok < nt; ++tok)
        if (lane < 32) a.scores[(int64_t)(t0 + tok) * a.n_pos + p * kIdxBlock + wave * 32 + lane] = -INFINITY;
    return;
  }
  // every block number of the run is read up front (uniform loads, before any store), and the
  // page loop is unrolled, so that the loop never waits on a table read queued behind key loads
  int blk[kIdxMaxPagesPerWg];
#pragma unroll
  for (int i = 0; i < kIdxMaxPagesPerWg; ++i) blk[i] = p0 + i < p1 ? page_block(a, b, p0 + i, lim) : -1;
  switch (nt) {
    case 1: scores_body<1>(a, q_s, w_s, blk, t0, p0, p1, lim); break;
    case 2: scores_body<2>(a, q_s, w_s, blk, t0, p0, p1, lim); break;
    case 3: scores_body<3>(a, q_s, w_s, blk, t0, p0, p1, lim); break;
    default: scores_body<4>(a, q_s, w_s, blk, t0, p0, p1, lim); break;
  }
}

// Order-preserving map of a float onto uint32: a larger float gives a larger key, and -0.0 and
// +0.0 give the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum of v over the workgroup (kSelectThreads threads); `tmp` holds one int
// per wave.
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
  for (int w = 0; w < kSelectWaves; ++w) add += (w < wave) ? tmp[w] : 0;
  __syncthreads();
  return v + add;
}

struct SelectShared {
  uint32_t hist[4096];           // digit histogram; afterwards the output row is staged here
  uint32_t cand[kSelectThreads]; // keys of the k-th key's 12-bit bin, when it holds at most 1024
  int scan_tmp[kSelectWaves];
  uint32_t digit;
  int remaining;
  int bin_count;
  int n_cand;
};
constexpr int kSelectStage = 4096;  // rows with topk up to this are staged in LDS, then stored whole

template <bool kCached>
__global__ void __launch_bounds__(kSelectThreads) topk_select_kernel(const IndexerArgs a) {
  __shared__ SelectShared sh;
  __shared__ __attribute__((aligned(16))) uint32_t keys[kCached ? kIdxSelCache : 4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int b = t / a.s1;
  const int n = max(0, min(a.act[b], a.n_pos));
  const int K = a.topk;
  int32_t* out = a.topk_out + (int64_t)t * K;
  const float* sc = a.scores + (int64_t)t * a.n_pos;

  if (n <= K) {  // every live position is selected
    for (int i = tid; i < K; i += kSelectThreads) out[i] = i < n ? i : -1;
    return;
  }
  if (kCached) {  // rows are 512-byte aligned (n_pos is a multiple of 128)
    // the keys are staged in LDS and histogrammed on their top 12 bits (the first radix digit)
    // in the same pass
    for (int i = tid; i < 4096; i += kSelectThreads) sh.hist[i] = 0;
    __syncthreads();
    const float4* sc4 = reinterpret_cast<const float4*>(sc);
    for (int i = tid; i < (n + 3) / 4; i += kSelectThreads) {
      const float4 v = sc4[i];
      const uint4 k4 = uint4{order_key(v.x), order_key(v.y), order_key(v.z), order_key(v.w)};
      reinterpret_cast<uint4*>(keys)[i] = k4;
      atomicAdd(&sh.hist[k4.x >> 20], 1u);
      if (4 * i + 1 < n) atomicAdd(&sh.hist[k4.y >> 20], 1u);
      if (4 * i + 2 < n) atomicAdd(&sh.hist[k4.z >> 20], 1u);
      if (4 * i + 3 < n) atomicAdd(&sh.hist[k4.w >> 20], 1u);
    }
  }
  auto key_at = [&](int i) -> uint32_t { return kCached ? keys[i] : order_key(sc[i]); };

  // One most-significant-digit radix step: the digit at `shift` (nb bins) that holds the k-th
  // largest of the keys matching (prefix, mask), and how many keys of that digit are still to
  // be taken. The keys are all n positions, or the compacted candidates (one per thread).
  uint32_t prefix = 0, mask = 0;
  int remaining = K;  // how many still to take among keys matching the prefix (<= their count)
  auto radix_step = [&](int shift, int nb, bool from_cand, int nc, bool counted) {
    if (!counted) {
    for (int i = tid; i < nb; i += kSelectThreads) sh.hist[i] = 0;
    __syncthreads();
    if (from_cand) {
      if (tid < nc) {
        const uint32_t key = sh.cand[tid];
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    } else {
      for (int i = tid; i < n; i += kSelectThreads) {
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    }
    }
    __syncthreads();
    // thread tid takes digits nb-1-per*tid down to nb-per-per*tid; the inclusive scan of the
    // group sums counts every matching key at or above the group's lowest digit
    const int per = nb / kSelectThreads;
    const int top = nb - 1 - per * tid;
    int sum = 0;
    for (int j = 0; j < per; ++j) sum += (int)sh.hist[top - j];
    const int incl = block_inclusive_scan(sum, sh.scan_tmp);
    if (incl >= remaining && incl - sum < remaining) {
      int acc = incl - sum;
      for (int j = 0; j < per; ++j) {
        const int h = (int)sh.hist[top - j];
        if (acc + h >= remaining) {
          sh.digit = (uint32_t)(top - j);
          sh.remaining = remaining - acc;
          sh.bin_count = h;
          break;
        }
        acc += h;
      }
    }
    if (tid == 0) sh.n_cand = 0;
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    remaining = sh.remaining;
  };

  // Digit 1 (bits 31..20) over every key. When the k-th key's bin holds at most one key per
  // thread (the usual case), its keys are compacted and digits 2 and 3 (bits 19..10, 9..0) run
  // over them alone; otherwise over every key again.
  radix_step(20, 4096, false, 0, kCached);
  const bool compact = sh.bin_count <= kSelectThreads;
  __syncthreads();  // every thread has read sh before it is written again
  int nc = 0;
  if (compact) {
    // each thread's hits (positions tid, tid + 1024, ...) go to offsets from one block-wide scan
    int hits = 0;
    for (int i = tid; i < n; i += kSelectThreads) hits += (key_at(i) & 0xfff00000u) == prefix ? 1 : 0;
    const int incl = block_inclusive_scan(hits, sh.scan_tmp);
    int o = incl - hits;
    for (int i = tid; i < n; i += kSelectThreads) {
      const uint32_t key = key_at(i);
      if ((key & 0xfff00000u) == prefix) sh.cand[o++] = key;
    }
    if (tid == kSelectThreads - 1) sh.n_cand = incl;
    __syncthreads();
    nc = sh.n_cand;
  }
  radix_step(10, 1024, compact, nc, false);
  __syncthreads();
  radix_step(0, 1024, compact, nc, false);
  __syncthreads();

  // prefix is the k-th largest key; `remaining` of the keys equal to it are taken, the first
  // ones in position order, after the K - remaining keys above it
  const uint32_t kth = prefix;
  const int need = remaining;
  const bool stage = K <= kSelectStage;
  int32_t* const dst = stage ? reinterpret_cast<int32_t*>(sh.hist) : out;
  // contiguous runs of positions per thread, so that prefix sums over threads follow position
  // order; with fewer than 32768 positions both counts share one 32-bit scan
  const int chunk = (n + kSelectThreads - 1) / kSelectThreads;
  const int i0 = min(n, tid * chunk), i1 = min(n, i0 + chunk);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_at(i);
    gt += key > kth ? 1 : 0;
    eq += key == kth ? 1 : 0;
  }
  int off_gt, off_eq;
  if (n < 32768) {
    const int packed = (gt << 16) | eq;
    const int excl = block_inclusive_scan(packed, sh.scan_tmp) - packed;
    off_gt = excl >> 16;
    off_eq = excl & 0xffff;
  } else {
    off_gt = block_inclusive_scan(gt, sh.scan_tmp) - gt;
    off_eq = block_inclusive_scan(eq, sh.scan_tmp) - eq;
  }
  const int base_eq = K - need;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_at(i);
    if (key > kth) {
      dst[off_gt++] = i;
    } else if (key == kth) {
      if (off_eq < need) dst[base_eq + off_eq] = i;
      ++off_eq;
    }
  }
  if (stage) {
    __syncthreads();
    for (int i = tid; i < K; i += kSelectThreads) out[i] = dst[i];
  }
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t stream) {
  const int spans = (a.mb + a.pages_per_wg - 1) / a.pages_per_wg;
  const dim3 grid((unsigned)spans, (unsigned)(a.batch * a.chunks));
  const size_t lds = (size_t)min(a.s1, kIdxTokenChunk) * kIdxHeads * kRowPieces * sizeof(uint4);
  IndexerArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&indexer_scores_kernel), grid, dim3(kScoreThreads), args, lds,
                         stream);
}

hipError_t launch_topk_select(const IndexerArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.batch * a.s1));
  IndexerArgs copy = a;
  void* args[] = {&copy};
  const void* fn = a.n_pos <= kIdxSelCache ? reinterpret_cast<const void*>(&topk_select_kernel<true>)
                                           : reinterpret_cast<const void*>(&topk_select_kernel<false>);
  return hipLaunchKernel(fn, grid, dim3(kSelectThreads), args, 0, stream);
}

}  // namespace sfa
