// C entry points that touch the HIP runtime: planning on the current device, decode, merge.
// Argument checks run before any HIP call; see include/kv_attn.h for the contract.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "kv_attn_internal.h"

namespace kvattn {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

// Compute units of the current device, cached per device. Returns 0 on a HIP error.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices && cus > 0) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool debug_mode() {
  const char* e = getenv("KV_ATTN_DEBUG");
  return e != nullptr && strcmp(e, "1") == 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// KV_ATTN_DEBUG=1: copy the device-resident tables to the host and validate them.
kv_attn_status debug_validate(const int32_t* block_table, const int32_t* ctx_lens,
                              const kv_attn_params* p, hipStream_t stream) {
  std::vector<int32_t> ctx(p->batch);
  std::vector<int32_t> table;
  if (hipStreamSynchronize(stream) != hipSuccess) return KV_ATTN_ERR_HIP;
  if (hipMemcpy(ctx.data(), ctx_lens, sizeof(int32_t) * ctx.size(), hipMemcpyDeviceToHost) != hipSuccess)
    return KV_ATTN_ERR_HIP;
  if (block_table != nullptr) {
    table.resize(size_t(p->batch) * p->max_blocks_per_seq);
    if (hipMemcpy(table.data(), block_table, sizeof(int32_t) * table.size(), hipMemcpyDeviceToHost) !=
        hipSuccess)
      return KV_ATTN_ERR_HIP;
  }
  return kv_attn_validate_host(block_table != nullptr ? table.data() : nullptr, ctx.data(), p);
}

// Device scratch of kv_attn_decode_noalloc: one copy per device, held until the process ends.
// Host code never uses the array's name as an address; it uses the per-device pointer that
// hipGetSymbolAddress returns for the device that is current.
static __device__ __align__(256) unsigned char scratch[KV_ATTN_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // nullptr = not looked up yet on that device
std::mutex g_scratch_mutex;

// Address of the current device's copy of `scratch` (looked up once per device), or nullptr on
// a HIP error.
void* scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace
}  // namespace kvattn

extern "C" {

kv_attn_status kv_attn_get_plan(const kv_attn_params* p, int32_t num_cus, kv_attn_plan* plan) {
  if (p == nullptr || plan == nullptr) return KV_ATTN_ERR_NULL;
  if (num_cus < 0) return KV_ATTN_ERR_VALUE;
  const kv_attn_status st = kvattn::validate_params(p);
  if (st != KV_ATTN_OK) return st;
  int cus = num_cus;
  if (cus == 0) {
    if (kvattn::fault_injected("query")) return KV_ATTN_ERR_HIP;
    cus = kvattn::current_cu_count();
    if (cus <= 0) return KV_ATTN_ERR_HIP;
  }
  kvattn::Plan pl;
  const kv_attn_status ps = kvattn::make_plan(p, cus, &pl);
  if (ps != KV_ATTN_OK) return ps;
  plan->num_splits = pl.num_splits;
  plan->split_len = pl.split_tiles * kvattn::kTile;
  plan->grid_split = int32_t(pl.grid_split);
  plan->grid_merge = int32_t(pl.grid_merge);
  plan->kernel_variant = pl.variant;
  plan->group_padded = pl.group_padded;
  plan->num_cus = cus;
  plan->wave_heads = pl.wave_heads;
  plan->unit_order = pl.unit_order;
  plan->reserved = 0;
  plan->workspace_bytes = pl.workspace_bytes;
  plan->ml_offset = pl.num_splits > 1 ? pl.o_part_bytes : 0;
  plan->order_offset = pl.unit_order ? pl.order_bytes_offset : 0;
  return KV_ATTN_OK;
}

size_t kv_attn_workspace_size(const kv_attn_params* p) {
  kv_attn_plan plan;
  if (kv_attn_get_plan(p, 0, &plan) != KV_ATTN_OK) return 0;
  return size_t(plan.workspace_bytes);
}

}  // extern "C"

namespace kvattn {
namespace {

constexpr int kPassSplit = 1;
constexpr int kPassMerge = 2;
constexpr int kPassAppend = 4;

AppendArgs append_args(const kv_attn_params* p, const void* k_new, const void* v_new, void* k,
                       void* v, const int32_t* block_table, const int32_t* positions,
                       int32_t pos_offset) {
  const bool paged = block_table != nullptr;
  const int eb = p->kv_dtype == KV_ATTN_BF16 ? 2 : 4;
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k = k;
  a.v = v;
  a.block_table = block_table;
  a.positions = positions;
  a.k_sb = p->k_stride_block;
  a.k_st = p->k_stride_token;
  a.k_sh = p->k_stride_head;
  a.v_sb = p->v_stride_block;
  a.v_st = p->v_stride_token;
  a.v_sh = p->v_stride_head;
  a.h_kv = p->num_kv_heads;
  a.row_chunks = p->head_dim * eb / 16;
  a.elem_bytes = eb;
  a.bs_log2 = paged ? log2_exact(p->block_size) : 0;
  a.max_blocks = paged ? p->max_blocks_per_seq : 0;
  a.limit = paged ? int32_t(std::min<int64_t>(int64_t(p->max_blocks_per_seq) * p->block_size, 0x7fffffff))
                  : p->block_size;
  a.rows_per_seq = p->num_queries > 1 ? p->num_queries : 1;
  a.pos_offset = pos_offset;
  a.total = p->batch * a.rows_per_seq * p->num_kv_heads * a.row_chunks;
  return a;
}

// Score export (token_scores != nullptr): where the logits and row statistics go in the workspace.
struct ScoreLayout {
  uint64_t logits_offset, stats_offset, total;
  int64_t ld;
};

uint64_t round256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

ScoreLayout score_layout(const kv_attn_params* p, const Plan& plan) {
  ScoreLayout l;
  const int64_t rows = int64_t(p->batch) * p->num_q_heads;
  const int64_t ctx = p->max_ctx_len > 0 ? p->max_ctx_len : 1;
  l.ld = (ctx + kTile - 1) / kTile * kTile;
  l.logits_offset = round256(plan.workspace_bytes);
  l.stats_offset = l.logits_offset + round256(uint64_t(rows) * uint64_t(l.ld) * 4u);
  l.total = l.stats_offset + uint64_t(rows) * 8u;
  return l;
}

// Shared body of kv_attn_decode / _split / _merge / _append_decode / _decode_scores: validation,
// planning, then the passes in `passes`. Every host-side check runs before the first HIP call.
kv_attn_status decode_impl(int passes, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens, float* out,
                           const kv_attn_params* p, void* workspace, size_t workspace_bytes,
                           void* stream, const void* k_new = nullptr, const void* v_new = nullptr,
                           float* token_scores = nullptr, int32_t accumulate = 0) {
  if (p == nullptr || ctx_lens == nullptr || out == nullptr) return KV_ATTN_ERR_NULL;
  if ((passes & kPassSplit) && (q == nullptr || k_cache == nullptr || v_cache == nullptr))
    return KV_ATTN_ERR_NULL;
  if ((passes & kPassAppend) && (k_new == nullptr || v_new == nullptr)) return KV_ATTN_ERR_NULL;
  if ((passes & kPassAppend) && (!aligned16(k_new) || !aligned16(v_new))) return KV_ATTN_ERR_UNSUPPORTED;
  const bool paged = block_table != nullptr;
  kv_attn_status st = (passes & kPassSplit) ? validate_layout(p, paged) : validate_params(p);
  if (st != KV_ATTN_OK) return st;
  if ((passes & kPassSplit) &&
      (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)))
    return KV_ATTN_ERR_UNSUPPORTED;

  if (fault_injected("query")) return KV_ATTN_ERR_HIP;
  const int cus = current_cu_count();
  if (cus <= 0) return KV_ATTN_ERR_HIP;
  Plan plan;
  st = make_plan(p, cus, &plan);
  if (st != KV_ATTN_OK) return st;
  const bool scores = token_scores != nullptr;
  ScoreLayout sl = {};
  if (scores) {
    if (plan.num_queries > 1) return KV_ATTN_ERR_UNSUPPORTED;  // one query token per sequence
    // Score export is compiled for bf16 q and KV (matrix cores: the one-token kernel, or rows
    // mode with one block, which one token always fits) and for fp32 q and KV.
    const bool bf16_pair = p->q_dtype == KV_ATTN_BF16 && p->kv_dtype == KV_ATTN_BF16 &&
                           (plan.variant == 1 || (plan.variant == 2 && plan.row_blocks == 1));
    const bool f32_pair = p->q_dtype == KV_ATTN_F32 && p->kv_dtype == KV_ATTN_F32;
    if (!bf16_pair && !f32_pair) return KV_ATTN_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(token_scores) & 3u) != 0) return KV_ATTN_ERR_UNSUPPORTED;
    sl = score_layout(p, plan);
    // One (sequence, KV head)'s scores are addressed by a 31-bit byte offset.
    if (sl.ld * (p->num_q_heads / p->num_kv_heads) * 4 >= (int64_t(1) << 31)) return KV_ATTN_ERR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < sl.total) return KV_ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KV_ATTN_ERR_UNSUPPORTED;
  } else if (plan.num_splits > 1) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return KV_ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KV_ATTN_ERR_UNSUPPORTED;
  }
  if (fault_injected("launch")) return KV_ATTN_ERR_HIP;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((passes & kPassSplit) && debug_mode()) {
    st = debug_validate(block_table, ctx_lens, p, s);
    if (st != KV_ATTN_OK) return st;
  }
  float* logits = scores ? reinterpret_cast<float*>(static_cast<char*>(workspace) + sl.logits_offset)
                        : nullptr;
  float* row_stats = scores ? reinterpret_cast<float*>(static_cast<char*>(workspace) + sl.stats_offset)
                            : nullptr;
  float* o_part = plan.num_splits > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
  float* ml_part = plan.num_splits > 1
                       ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.o_part_bytes)
                       : nullptr;

  // The append fuses into the split kernel in the bf16 matrix-core variants (the tile holding
  // the new rows takes them from k_new / v_new and writes them into the cache); otherwise the
  // append kernel writes them first.
  const bool fused_append = (passes & kPassAppend) && (passes & kPassSplit) && !scores &&
                            (plan.variant == 2 || (plan.variant == 1 && plan.group_padded <= kAppendMaxGroup));
  if ((passes & kPassAppend) && !fused_append) {
    // The current token(s) are the last positions ctx_lens[b] counts: write them before reading.
    const int32_t nq = p->num_queries > 1 ? p->num_queries : 1;
    const AppendArgs ap = append_args(p, k_new, v_new, const_cast<void*>(k_cache),
                                      const_cast<void*>(v_cache), block_table, ctx_lens, -nq);
    if (launch_append(ap, stream) != 0) return KV_ATTN_ERR_HIP;
  }
  if (passes & kPassSplit) {
    SplitArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.block_table = block_table;
    a.ctx_lens = ctx_lens;
    a.out = out;
    a.o_part = o_part;
    a.ml_part = ml_part;
    a.k_sb = p->k_stride_block;
    a.k_st = p->k_stride_token;
    a.k_sh = p->k_stride_head;
    a.v_sb = p->v_stride_block;
    a.v_st = p->v_stride_token;
    a.v_sh = p->v_stride_head;
    a.h_q = p->num_q_heads;
    a.h_kv = p->num_kv_heads;
    a.group = p->num_q_heads / p->num_kv_heads;
    a.bs_log2 = paged ? log2_exact(p->block_size) : 0;
    a.max_blocks = paged ? p->max_blocks_per_seq : 0;
    a.max_ctx = p->max_ctx_len;
    a.split_tiles = plan.split_tiles;
    a.num_splits = plan.num_splits;
    a.window = p->window;
    a.num_sinks = p->num_sinks;
    a.num_queries = plan.num_queries;
    a.head_chunks = plan.head_chunks;
    a.wave_heads = plan.wave_heads;
    a.logits = logits;
    a.logits_ld = sl.ld;
    a.row_stats = plan.num_splits == 1 ? row_stats : nullptr;
    const double scale = p->scale != 0.0f ? double(p->scale) : 1.0 / sqrt(double(p->head_dim));
    a.scale_log2 = float(scale * 1.4426950408889634);  // log2(e)
    a.k_new = fused_append ? k_new : nullptr;
    a.v_new = fused_append ? v_new : nullptr;
    a.order = nullptr;
    if (plan.unit_order && !scores) {  // the score export keeps the split-by-split order
      int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.order_bytes_offset);
      OrderArgs oa;
      oa.ctx_lens = ctx_lens;
      oa.order = order;
      oa.batch = p->batch;
      oa.num_splits = plan.num_splits;
      oa.split_tiles = plan.split_tiles;
      oa.max_ctx = p->max_ctx_len;
      oa.window = p->window;
      oa.num_sinks = p->num_sinks;
      oa.num_queries = plan.num_queries;
      if (launch_order(oa, stream) != 0) return KV_ATTN_ERR_HIP;
      a.order = order;
    }
    if (launch_split(a, plan, p->head_dim, paged, p->q_dtype == KV_ATTN_BF16,
                     p->kv_dtype == KV_ATTN_BF16, stream) != 0)
      return KV_ATTN_ERR_HIP;
  }
  if ((passes & kPassMerge) && plan.num_splits > 1) {
    MergeArgs m;
    m.o_part = o_part;
    m.ml_part = ml_part;
    m.num_valid = nullptr;
    m.ctx_lens = ctx_lens;
    m.out = out;
    m.rows = p->batch * plan.num_queries * p->num_q_heads;
    m.num_splits = plan.num_splits;
    m.h_q = plan.num_queries * p->num_q_heads;
    m.split_tiles = plan.split_tiles;
    m.max_ctx = p->max_ctx_len;
    m.window = p->window;
    m.num_sinks = p->num_sinks;
    m.num_queries = plan.num_queries;
    m.row_stats = row_stats;
    if (launch_merge(m, p->head_dim, stream) != 0) return KV_ATTN_ERR_HIP;
  }
  if (scores && (passes & kPassMerge)) {
    ScoreArgs sa;
    sa.logits = logits;
    sa.row_stats = row_stats;
    sa.ctx_lens = ctx_lens;
    sa.scores = token_scores;
    sa.logits_ld = sl.ld;
    sa.scores_ld = p->max_ctx_len;
    sa.h_kv = p->num_kv_heads;
    sa.group = p->num_q_heads / p->num_kv_heads;
    sa.max_ctx = p->max_ctx_len;
    sa.window = p->window;
    sa.num_sinks = p->num_sinks;
    sa.accumulate = accumulate;
    sa.chunks = int32_t((int64_t(p->max_ctx_len) + kScoreChunk - 1) / kScoreChunk);
    if (launch_scores(sa, int64_t(p->batch) * p->num_kv_heads, stream) != 0) return KV_ATTN_ERR_HIP;
  }
  if (debug_mode()) {
    if (hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) return KV_ATTN_ERR_HIP;
  }
  return KV_ATTN_OK;
}

}  // namespace
}  // namespace kvattn

extern "C" {

kv_attn_status kv_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens, float* out,
                              const kv_attn_params* p, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return kvattn::decode_impl(kvattn::kPassSplit | kvattn::kPassMerge, q, k_cache, v_cache,
                             block_table, ctx_lens, out, p, workspace, workspace_bytes, stream);
}

kv_attn_status kv_attn_decode_split(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens, float* out,
                                    const kv_attn_params* p, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return kvattn::decode_impl(kvattn::kPassSplit, q, k_cache, v_cache, block_table, ctx_lens, out,
                             p, workspace, workspace_bytes, stream);
}

kv_attn_status kv_attn_decode_merge(const int32_t* ctx_lens, float* out, const kv_attn_params* p,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return kvattn::decode_impl(kvattn::kPassMerge, nullptr, nullptr, nullptr, nullptr, ctx_lens, out,
                             p, workspace, workspace_bytes, stream);
}

kv_attn_status kv_attn_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* block_table, const int32_t* positions,
                              const kv_attn_params* p, void* stream) {
  if (p == nullptr || k_new == nullptr || v_new == nullptr || k_cache == nullptr ||
      v_cache == nullptr || positions == nullptr)
    return KV_ATTN_ERR_NULL;
  const kv_attn_status st = kvattn::validate_layout(p, block_table != nullptr);
  if (st != KV_ATTN_OK) return st;
  if (!kvattn::aligned16(k_new) || !kvattn::aligned16(v_new) || !kvattn::aligned16(k_cache) ||
      !kvattn::aligned16(v_cache))
    return KV_ATTN_ERR_UNSUPPORTED;
  if (kvattn::fault_injected("launch")) return KV_ATTN_ERR_HIP;
  const kvattn::AppendArgs a =
      kvattn::append_args(p, k_new, v_new, k_cache, v_cache, block_table, positions, 0);
  if (kvattn::launch_append(a, stream) != 0) return KV_ATTN_ERR_HIP;
  if (kvattn::debug_mode()) {
    if (hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess ||
        hipGetLastError() != hipSuccess)
      return KV_ATTN_ERR_HIP;
  }
  return KV_ATTN_OK;
}

kv_attn_status kv_attn_append_decode(const void* q, const void* k_new, const void* v_new,
                                     void* k_cache, void* v_cache, const int32_t* block_table,
                                     const int32_t* ctx_lens, float* out, const kv_attn_params* p,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return kvattn::decode_impl(kvattn::kPassAppend | kvattn::kPassSplit | kvattn::kPassMerge, q,
                             k_cache, v_cache, block_table, ctx_lens, out, p, workspace,
                             workspace_bytes, stream, k_new, v_new);
}

size_t kv_attn_scores_workspace_size(const kv_attn_params* p) {
  if (p == nullptr || kvattn::validate_params(p) != KV_ATTN_OK) return 0;
  const int cus = kvattn::current_cu_count();
  if (cus <= 0) return 0;
  kvattn::Plan plan;
  if (kvattn::make_plan(p, cus, &plan) != KV_ATTN_OK || plan.num_queries > 1) return 0;
  return size_t(kvattn::score_layout(p, plan).total);
}

kv_attn_status kv_attn_decode_scores(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* ctx_lens, float* out,
                                     float* token_scores, int32_t accumulate,
                                     const kv_attn_params* p, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (token_scores == nullptr) return KV_ATTN_ERR_NULL;
  return kvattn::decode_impl(kvattn::kPassSplit | kvattn::kPassMerge, q, k_cache, v_cache,
                             block_table, ctx_lens, out, p, workspace, workspace_bytes, stream,
                             nullptr, nullptr, token_scores, accumulate);
}

kv_attn_status kv_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      float* out, const kv_attn_params* p, void* stream) {
  using namespace kvattn;
  // The host-side checks of kv_attn_decode come first (decode_impl repeats them, unchanged).
  if (p == nullptr || ctx_lens == nullptr || out == nullptr || q == nullptr || k_cache == nullptr ||
      v_cache == nullptr)
    return KV_ATTN_ERR_NULL;
  kv_attn_status st = validate_layout(p, block_table != nullptr);
  if (st != KV_ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return KV_ATTN_ERR_UNSUPPORTED;
  if (fault_injected("query")) return KV_ATTN_ERR_HIP;
  const int cus = current_cu_count();
  if (cus <= 0) return KV_ATTN_ERR_HIP;
  Plan plan;
  st = make_plan(p, cus, &plan);
  if (st != KV_ATTN_OK) return st;
  if (plan.workspace_bytes > uint64_t(KV_ATTN_NOALLOC_SCRATCH_BYTES)) return KV_ATTN_ERR_SCRATCH;
  void* ws = plan.num_splits > 1 ? scratch_for_current_device() : nullptr;
  if (plan.num_splits > 1 && ws == nullptr) return KV_ATTN_ERR_HIP;
  return decode_impl(kPassSplit | kPassMerge, q, k_cache, v_cache, block_table, ctx_lens, out, p,
                     ws, ws != nullptr ? size_t(KV_ATTN_NOALLOC_SCRATCH_BYTES) : 0, stream);
}

kv_attn_status kv_attn_merge(const float* o_partial, const float* ml_partial,
                             const int32_t* num_valid, float* out, int32_t rows,
                             int32_t num_splits, int32_t head_dim, void* stream) {
  if (o_partial == nullptr || ml_partial == nullptr || out == nullptr) return KV_ATTN_ERR_NULL;
  if (rows < 1 || num_splits < 1) return KV_ATTN_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return KV_ATTN_ERR_UNSUPPORTED;
  if (num_splits > kvattn::kMaxSplits) return KV_ATTN_ERR_UNSUPPORTED;
  if (kvattn::fault_injected("launch")) return KV_ATTN_ERR_HIP;
  kvattn::MergeArgs m;
  m.o_part = o_partial;
  m.ml_part = ml_partial;
  m.num_valid = num_valid;
  m.ctx_lens = nullptr;
  m.out = out;
  m.rows = rows;
  m.num_splits = num_splits;
  m.h_q = 1;
  m.split_tiles = 1;
  m.max_ctx = 0;
  m.window = 0;
  m.num_sinks = 0;
  m.num_queries = 1;
  m.row_stats = nullptr;
  if (kvattn::launch_merge(m, head_dim, stream) != 0) return KV_ATTN_ERR_HIP;
  if (kvattn::debug_mode()) {
    if (hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess ||
        hipGetLastError() != hipSuccess)
      return KV_ATTN_ERR_HIP;
  }
  return KV_ATTN_OK;
}

}  // extern "C"
