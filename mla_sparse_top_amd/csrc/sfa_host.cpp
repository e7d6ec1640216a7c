// C-ABI entry points of libsfa.so: synchronous argument validation, partition choice,
// workspace layout, kernel launch. Declarations and contracts are in include/sfa.h.

#include "sfa.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "sfa_internal.h"

namespace {

using namespace sfa;

constexpr size_t kAlignWs = 256;
// Target number of workgroups for decode: the MI355X has 256 compute units and the attention
// kernel runs one workgroup per CU (its register and LDS footprint allow no more).
constexpr int kTargetWorkgroups = 256;
constexpr int kMaxAutoSplits = 8;
constexpr int kMinSlots = 256;  // top-k slots per partition at least, in the automatic choice

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// rope_dim 0 (512-wide rows with the rotary channels inside) is accepted for the window variants
int check_dims(const sfa_dims* d, bool allow_no_rope = false) {
  if (!d) return SFA_ERR_NULL;
  if (d->n_kv != 1 || d->kv_lora_rank != kNope || d->block_size != kBlock) return SFA_ERR_DIMS;
  if (d->rope_dim != kRope && !(allow_no_rope && d->rope_dim == 0)) return SFA_ERR_DIMS;
  if (d->n_q < 16 || d->n_q > SFA_MAX_HEADS || (d->n_q % 16) != 0) return SFA_ERR_DIMS;
  if (d->batch < 0 || d->s1 < 0) return SFA_ERR_DIMS;
  if ((int64_t)d->batch * d->s1 > (1 << 24)) return SFA_ERR_DIMS;
  if (d->topk < 1 || d->topk > kMaxTopk) return SFA_ERR_DIMS;
  if (d->max_blocks_per_batch < 1 || d->max_blocks_per_batch > (1 << 23)) return SFA_ERR_DIMS;
  if (d->num_cache_rows < 0 || d->num_cache_rows > INT32_MAX) return SFA_ERR_DIMS;
  if (d->kv_dtype != SFA_KV_BF16 && d->kv_dtype != SFA_KV_INT8) return SFA_ERR_DIMS;
  if (d->num_splits < 0 || d->num_splits > kMaxSplits) return SFA_ERR_DIMS;
  return SFA_OK;
}

int pick_splits(const sfa_dims* d, int is_prefill) {
  const int64_t tokens = (int64_t)d->batch * d->s1;
  const int min_s = (d->topk + kMaxSlots - 1) / kMaxSlots;  // each partition compacts <= 2048 slots
  int s;
  if (d->num_splits > 0) {
    s = d->num_splits;
  } else if (is_prefill) {
    s = 1;
  } else {
    // Enough (token, partition) work items to give every CU one, but at least kMinSlots slots
    // per partition and at most kMaxAutoSplits partitions: the merge moves a 256 KB partial per
    // partition through memory, which only pays for itself against a few hundred gathered rows
    // (measured with the spread merge: a 128-slot window runs in 20.6 us as one partition and
    // 32.2 us as two; 32 single-token sequences with top-k 2048 in 64.6 us with 4 partitions,
    // 60.9 us with 8).
    const int64_t items = tokens;
    const int64_t want = items > 0 ? (kTargetWorkgroups + items - 1) / items : 1;
    s = (int)(want < kMaxAutoSplits ? want : kMaxAutoSplits);
    const int by_len = d->topk / kMinSlots > 0 ? d->topk / kMinSlots : 1;
    if (s > by_len) s = by_len;
    if (s < 1) s = 1;
  }
  if (s < min_s) s = min_s;
  return s;
}

struct WsLayout {
  size_t part_o, part_ml, counters, total;
};

WsLayout ws_layout(const sfa_dims* d, int splits) {
  WsLayout w{0, 0, 0, 0};
  if (splits <= 1) return w;
  const size_t groups = (size_t)d->batch * d->s1;
  const size_t items = groups * splits;
  w.part_o = 0;
  w.part_ml = align_up(items * kPartialBytes, kAlignWs);
  w.counters = w.part_ml + align_up(items * kPartialMlBytes, kAlignWs);
  w.total = w.counters + align_up(kCounterWords * groups * sizeof(uint64_t), kAlignWs);
  return w;
}

// Compute units and wall-clock rate (kHz) of the device a stream belongs to, looked up once per
// device (0 when the runtime cannot tell).
struct DeviceInfo {
  int cus;
  int64_t clock_khz;
};
DeviceInfo device_info(hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int64_t> cache[kMaxDevices];  // cus << 40 | kHz, 0 = not looked up yet
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return DeviceInfo{0, 0};
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, khz = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || cus <= 0 || khz <= 0)
      return DeviceInfo{0, 0};
    v = ((int64_t)cus << 40) | khz;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return DeviceInfo{(int)(v >> 40), v & ((int64_t{1} << 40) - 1)};
}

// An early arrival's wait for the other partitions in the spread merge: long against the spread
// of equal partitions' finishing times (a few microseconds), short enough that a partner that is
// not running costs little. SFA_MERGE_WAIT_NS overrides it (nanoseconds; 0 turns the spread
// merge off), so that every outcome of the wait can be exercised.
constexpr int64_t kMergeWaitNanos = 50000;
int64_t merge_wait_nanos() {
  const char* e = getenv("SFA_MERGE_WAIT_NS");
  if (!e || !*e) return kMergeWaitNanos;
  char* end = nullptr;
  const long long v = strtoll(e, &end, 10);
  return (end && *end == 0 && v >= 0) ? (int64_t)v : kMergeWaitNanos;
}

// [p, p + n) overlaps [q, q + m)
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a0 = (uintptr_t)p, a1 = a0 + n, b0 = (uintptr_t)q, b1 = b0 + m;
  return a0 < b1 && b0 < a1;
}

// The second source of the window variants (sfa_window_decode); null for sfa_decode/prefill.
struct WindowSource {
  int32_t window, topk_cmp, mb_cmp;
  const int32_t* bt_cmp;
  const int32_t* cmp_len;
};

int run_attention(const sfa_dims* d, int is_prefill, const void* qn, const void* qr, const void* kn,
                  const void* kr, const float* scales, const int32_t* idx, const int32_t* bt,
                  const int32_t* act, float softmax_scale, void* out, void* ws, size_t ws_bytes,
                  hipStream_t stream, const WindowSource* win = nullptr) {
  int st = check_dims(d, win != nullptr);
  if (st != SFA_OK) return st;
  const int64_t tokens = (int64_t)d->batch * d->s1;
  // the window variants take no index list when they have no compressed source (SWA)
  const bool need_idx = !win || win->topk_cmp > 0;
  // rows without rope channels: query_rope and key_rope are not read (and may be null)
  const bool rope = d->rope_dim > 0;
  if (!rope) qr = kr = nullptr;
  if (!qn || (rope && !qr) || !kn || (rope && !kr) || (need_idx && !idx) || !bt || !act || !out) return SFA_ERR_NULL;
  if (win && win->topk_cmp > 0 && (!win->bt_cmp || !win->cmp_len)) return SFA_ERR_NULL;
  const bool int8 = d->kv_dtype == SFA_KV_INT8;
  if (int8 && !scales) return SFA_ERR_SCALES;
  if (!aligned16(qn) || !aligned16(qr) || !aligned16(kn) || !aligned16(kr) || !aligned16(idx) ||
      !aligned16(bt) || !aligned16(act) || !aligned16(out) || (int8 && !aligned16(scales)))
    return SFA_ERR_ALIGN;
  if (win && win->topk_cmp > 0 && (!aligned16(win->bt_cmp) || !aligned16(win->cmp_len))) return SFA_ERR_ALIGN;
  if (!isfinite(softmax_scale)) return SFA_ERR_SCALE_VALUE;

  const int splits = pick_splits(d, is_prefill);
  const WsLayout lay = ws_layout(d, splits);
  if (lay.total > 0) {
    if (!ws || ws_bytes < lay.total || ((uintptr_t)ws % kAlignWs) != 0) return SFA_ERR_WORKSPACE;
  }

  const size_t rows = (size_t)d->num_cache_rows;
  const size_t out_bytes = (size_t)tokens * d->n_q * kNope * 2;
  const int64_t idx_cols = win ? win->topk_cmp : d->topk;
  const void* ins[] = {qn, qr, kn, kr, scales, idx, bt, act, lay.total ? ws : nullptr,
                       win ? win->bt_cmp : nullptr, win ? win->cmp_len : nullptr};
  const size_t sizes[] = {(size_t)tokens * d->n_q * kNope * 2,
                          (size_t)tokens * d->n_q * d->rope_dim * 2,
                          rows * kNope * (int8 ? 1 : 2),
                          rows * d->rope_dim * 2,
                          int8 ? rows * 4 * sizeof(float) : 0,
                          (size_t)tokens * idx_cols * sizeof(int32_t),
                          (size_t)d->batch * d->max_blocks_per_batch * sizeof(int32_t),
                          (size_t)d->batch * sizeof(int32_t),
                          lay.total,
                          win ? (size_t)d->batch * win->mb_cmp * sizeof(int32_t) : 0,
                          win ? (size_t)d->batch * sizeof(int32_t) : 0};
  for (int i = 0; i < 11; ++i)
    if (overlaps(out, out_bytes, ins[i], sizes[i])) return SFA_ERR_ALIAS;
  // the kernels write the workspace: it must not hold an input either
  for (int i = 0; i < 11; ++i)
    if (i != 8 && overlaps(ins[8], sizes[8], ins[i], sizes[i])) return SFA_ERR_ALIAS;

  if (tokens == 0) return SFA_OK;

  KernelArgs a;
  memset(&a, 0, sizeof(a));
  a.q_nope = static_cast<const uint16_t*>(qn);
  a.q_rope = static_cast<const uint16_t*>(qr);
  a.k_nope = kn;
  a.k_rope = static_cast<const uint16_t*>(kr);
  a.k_scales = scales;
  a.topk_idx = idx;
  a.block_table = bt;
  a.act = act;
  a.out = static_cast<uint16_t*>(out);
  if (lay.total) {
    char* base = static_cast<char*>(ws);
    a.part_o = reinterpret_cast<float*>(base + lay.part_o);
    a.part_ml = reinterpret_cast<float*>(base + lay.part_ml);
    a.counters = reinterpret_cast<uint64_t*>(base + lay.counters);
  }
  // a generation of its own for every call (48 bits, never 0): the merge counters of earlier
  // calls, or any other workspace contents, do not count for this one
  static std::atomic<uint64_t> next_gen{1};
  uint64_t gen = next_gen.fetch_add(1, std::memory_order_relaxed) & ((uint64_t{1} << 48) - 1);
  if (gen == 0) gen = next_gen.fetch_add(1, std::memory_order_relaxed) & ((uint64_t{1} << 48) - 1);
  a.gen = gen;
  a.num_rows = d->num_cache_rows;
  a.n_tokens = (int32_t)tokens;
  a.s1 = d->s1;
  a.n_q = d->n_q;
  a.topk = d->topk;
  a.mb = d->max_blocks_per_batch;
  a.n_splits = splits;
  a.chunk = (d->topk + splits - 1) / splits;
  a.reverse = is_prefill ? 1 : 0;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);  // log2(e)
  // One partition with fewer than half as many tokens as CUs: two workgroups of 64 heads per
  // token instead of one of 128, so that twice as many CUs gather and compute; it needs no
  // merge. (Short slot lists, such as a 128-position window, do not pay for partitions.)
  a.head_groups = 1;
  {
    const DeviceInfo di = device_info(stream);
    if (splits == 1 && d->n_q > kMaxHeads / 2 && di.cus > 0 && 2 * tokens <= di.cus) a.head_groups = 2;
  }
  if (splits >= 2 && splits <= kMaxSpread) {
    // the spread merge needs the partitions of a token running at once: every workgroup of the
    // grid (one per compute unit) resident
    const DeviceInfo di = device_info(stream);
    const int64_t ns = merge_wait_nanos();
    if (di.cus > 0 && splits * tokens <= di.cus && ns > 0) {
      const int64_t ticks = di.clock_khz * ns / 1000000;
      a.merge_wait_ticks = ticks > 0 ? ticks : 1;
    }
  }
  if (win) {
    a.window = win->window;
    a.mb_cmp = win->topk_cmp > 0 ? win->mb_cmp : 0;
    a.block_table_cmp = win->topk_cmp > 0 ? win->bt_cmp : nullptr;
    a.act_cmp = win->topk_cmp > 0 ? win->cmp_len : nullptr;
  }
  return launch_attention(a, int8, win != nullptr, rope, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

int check_window_dims(const sfa_window_dims* d) {
  if (!d) return SFA_ERR_NULL;
  if (d->window < 0 || d->topk_cmp < 0 || d->window + (int64_t)d->topk_cmp < 1) return SFA_ERR_DIMS;
  if (d->max_blocks_ori < 1 || d->max_blocks_cmp < 0) return SFA_ERR_DIMS;
  if (d->topk_cmp > 0 && (d->max_blocks_cmp < 1 || d->max_blocks_cmp > (1 << 23))) return SFA_ERR_DIMS;
  return SFA_OK;
}

// The attention dims of a window call: its slots are the window followed by the compressed list.
sfa_dims window_attention_dims(const sfa_window_dims* w) {
  sfa_dims c{};
  c.batch = w->batch;
  c.s1 = w->s1;
  c.n_q = w->n_q;
  c.n_kv = w->n_kv;
  c.kv_lora_rank = w->kv_lora_rank;
  c.rope_dim = w->rope_dim;
  c.block_size = w->block_size;
  c.topk = (int32_t)((int64_t)w->window + w->topk_cmp > INT32_MAX ? INT32_MAX : w->window + w->topk_cmp);
  c.max_blocks_per_batch = w->max_blocks_ori;
  c.num_cache_rows = w->num_cache_rows;
  c.kv_dtype = w->kv_dtype;
  c.num_splits = w->num_splits;
  return c;
}

}  // namespace

extern "C" {

int sfa_window_workspace_size(const sfa_window_dims* dims, size_t* bytes_out) {
  if (!bytes_out) return SFA_ERR_NULL;
  int st = check_window_dims(dims);
  if (st != SFA_OK) return st;
  const sfa_dims c = window_attention_dims(dims);
  st = check_dims(&c, true);
  if (st != SFA_OK) return st;
  *bytes_out = ws_layout(&c, pick_splits(&c, 0)).total;
  return SFA_OK;
}

int sfa_window_decode(const sfa_window_dims* dims, const void* query_nope, const void* query_rope,
                      const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
                      const int32_t* cmp_indices, const int32_t* block_table_ori, const int32_t* block_table_cmp,
                      const int32_t* ori_len, const int32_t* cmp_len, float softmax_scale, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  const int st = check_window_dims(dims);
  if (st != SFA_OK) return st;
  const sfa_dims c = window_attention_dims(dims);
  WindowSource w{dims->window, dims->topk_cmp, dims->max_blocks_cmp, block_table_cmp, cmp_len};
  return run_attention(&c, 0, query_nope, query_rope, key_nope_2d, key_rope_2d, k_nope_scales,
                       dims->topk_cmp > 0 ? cmp_indices : nullptr, block_table_ori, ori_len, softmax_scale, out,
                       workspace, workspace_bytes, stream, &w);
}

int sfa_workspace_size(const sfa_dims* dims, int is_prefill, size_t* bytes_out) {
  if (!bytes_out) return SFA_ERR_NULL;
  const int st = check_dims(dims);
  if (st != SFA_OK) return st;
  *bytes_out = ws_layout(dims, pick_splits(dims, is_prefill)).total;
  return SFA_OK;
}

int sfa_num_splits(const sfa_dims* dims, int is_prefill) {
  const int st = check_dims(dims);
  if (st != SFA_OK) return st;
  return pick_splits(dims, is_prefill);
}

int sfa_decode(const sfa_dims* dims, const void* query_nope, const void* query_rope,
               const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
               const int32_t* topk_indices, const int32_t* block_table, const int32_t* kv_act_seqs,
               float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  return run_attention(dims, 0, query_nope, query_rope, key_nope_2d, key_rope_2d, k_nope_scales,
                       topk_indices, block_table, kv_act_seqs, softmax_scale, out, workspace,
                       workspace_bytes, stream);
}

int sfa_prefill(const sfa_dims* dims, const void* query_nope, const void* query_rope,
                const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
                const int32_t* topk_indices, const int32_t* block_table, const int32_t* kv_act_seqs,
                float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return run_attention(dims, 1, query_nope, query_rope, key_nope_2d, key_rope_2d, k_nope_scales,
                       topk_indices, block_table, kv_act_seqs, softmax_scale, out, workspace,
                       workspace_bytes, stream);
}

int sfa_resolve_rows(const sfa_dims* dims, const int32_t* topk_indices, const int32_t* block_table,
                     const int32_t* kv_act_seqs, int32_t* rows_out, hipStream_t stream) {
  const int st = check_dims(dims);
  if (st != SFA_OK) return st;
  if (!topk_indices || !block_table || !kv_act_seqs || !rows_out) return SFA_ERR_NULL;
  if (!aligned16(topk_indices) || !aligned16(block_table) || !aligned16(kv_act_seqs) || !aligned16(rows_out))
    return SFA_ERR_ALIGN;
  const int64_t tokens = (int64_t)dims->batch * dims->s1;
  const size_t out_bytes = (size_t)tokens * dims->topk * sizeof(int32_t);
  if (overlaps(rows_out, out_bytes, topk_indices, out_bytes) ||
      overlaps(rows_out, out_bytes, block_table, (size_t)dims->batch * dims->max_blocks_per_batch * 4) ||
      overlaps(rows_out, out_bytes, kv_act_seqs, (size_t)dims->batch * 4))
    return SFA_ERR_ALIAS;
  if (tokens == 0) return SFA_OK;
  ResolveArgs a;
  a.topk_idx = topk_indices;
  a.block_table = block_table;
  a.act = kv_act_seqs;
  a.rows_out = rows_out;
  a.num_rows = dims->num_cache_rows;
  a.n_tokens = (int32_t)tokens;
  a.s1 = dims->s1;
  a.topk = dims->topk;
  a.mb = dims->max_blocks_per_batch;
  return launch_resolve(a, stream) == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

const char* sfa_status_string(int status) {
  switch (status) {
    case SFA_OK: return "ok";
    case SFA_ERR_NULL: return "a required pointer is NULL";
    case SFA_ERR_DIMS: return "unsupported dimensions (n_kv must be 1, kv_lora_rank 512, rope_dim 64, "
                              "block_size 128, n_q a multiple of 16 in [16,128], topk in [1,32768])";
    case SFA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case SFA_ERR_WORKSPACE: return "workspace missing, not 256-byte aligned, or smaller than sfa_workspace_size";
    case SFA_ERR_SCALES: return "INT8 cache requires k_nope_scales";
    case SFA_ERR_ALIAS: return "an output overlaps an input or the workspace, or the workspace overlaps an input";
    case SFA_ERR_SCALE_VALUE: return "softmax_scale is not finite";
    case SFA_ERR_HIP: return "a HIP runtime call failed";
    case SFA_ERR_SCRATCH_LIMIT: return "the call needs more workspace than sfa_decode_noalloc's fixed scratch "
                                       "(SFA_NOALLOC_SCRATCH_BYTES); lower num_splits or use sfa_decode";
    default: return "unknown status";
  }
}

}  // extern "C"
