// Internal interfaces between the host layer and the kernels (not part of the C ABI).
#ifndef KV_ATTN_INTERNAL_H_
#define KV_ATTN_INTERNAL_H_

#include <stdint.h>

#include "kv_attn.h"

namespace kvattn {

// Positions per tile: one MFMA row block, and one 16-token block of a paged cache.
constexpr int kTile = 16;
// Waves per split workgroup; each wave streams every kWaves-th tile of the split (or, with
// SplitArgs::wave_heads, every tile of the split for its own KV head).
constexpr int kWaves = 4;
constexpr int kSplitThreads = 64 * kWaves;
// Merge pass: one workgroup of kMergeThreads per (sequence, query head) row.
constexpr int kMergeThreads = 256;
// Split planning constants (see make_plan).
constexpr int kMinSplitTiles = 16;     // a split spans at least 256 positions ...
constexpr int kMaxSplitTiles = 256;    // ... and at most 4096 positions with many units ...
constexpr int kMaxSplitTilesLong = 512;  // ... or 8192 with few units or several query tokens
constexpr int kMaxSplits = 4096;
constexpr int kMaxQueryRows = 32;      // rows mode: num_queries * group <= 32 (two MFMA blocks)
constexpr int kMaxQueries = 16;
constexpr int kRowsMinGroup = 4;      // one query token: rows mode from this group size on (bf16)
constexpr int kVectorMaxGroup = 8;    // vector path: query heads one workgroup holds
constexpr int kWaveHeadsMinTiles = 32; // wave heads: tiles per wave, at least, on a full device
constexpr int kAppendMaxGroup = 4;     // fused append: padded groups of variant 1 it serves
constexpr int kOrderMaxSplits = 256;   // unit order: splits per sequence, at most (one lane
                                       // of a wave scans 4 counters each)
constexpr int kOrderThreads = 256;    // unit order: the order kernel's one workgroup
constexpr int kOrderMinRounds = 4;     // unit order: split workgroups per split / CUs, at least
constexpr int kOrderBuckets = 256;     // unit order: partial-split lengths are ranked in 256 classes

// Everything the split kernel needs, by value.
struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;  // nullptr: contiguous cache
  const int32_t* ctx_lens;
  float* out;                  // final output (num_splits == 1)
  float* o_part;               // [B, h_q, S, d] unnormalised sums (num_splits > 1)
  float* ml_part;              // [B, h_q, S, 2] (m in base-2 units, l)
  int64_t k_sb, k_st, k_sh;    // element strides of the K cache
  int64_t v_sb, v_st, v_sh;
  int32_t h_q;
  int32_t h_kv;
  int32_t group;               // g = h_q / h_kv
  int32_t bs_log2;             // paged: log2(block_size); unused when contiguous
  int32_t max_blocks;          // paged: row length of block_table
  int32_t max_ctx;             // ctx_lens are clamped into [0, max_ctx]
  int32_t split_tiles;         // tiles per split
  int32_t num_splits;          // S
  float scale_log2;            // scale * log2(e)
  int32_t window;              // > 0: attend only the last `window` positions plus the sinks
  int32_t num_sinks;           // leading positions always attended when a window is set
  int32_t num_queries;         // query tokens per sequence (rows mode; 1 otherwise)
  int32_t head_chunks;         // workgroups per (sequence, KV head, split): 1, or 2 when the
                               // vector path serves a group above kVectorMaxGroup heads
  int32_t wave_heads;          // 1: a workgroup serves kWaves KV heads of one split, one per
                               // wave, each wave streaming every tile of the split (h_kv is a
                               // multiple of kWaves, head_chunks == 1); 0: one KV head, the
                               // waves sharing its tiles
  float* logits;               // nullptr, or [B * h_q, logits_ld]: base-2 scores of every visited
                               // position (one query token per sequence only)
  int64_t logits_ld;           // multiple of kTile, >= max_ctx rounded up to kTile
  float* row_stats;            // nullptr, or [B * h_q, 2]: final (m, l) per row (num_splits == 1)
  const void* k_new;           // nullptr, or the fused append's new K rows [B, nq, h_kv, d]
  const void* v_new;           // (bf16, matrix-core variants); k and v are then writable
  const int32_t* order;        // nullptr, or [B * S][2]: entry i = (b * S + split, clamped
                               // length of b) of the i-th (sequence, split) pair to serve, or
                               // (-1, 0) for an empty pair (head_chunks == 1); its workgroups
                               // are the next units-per-split indices
};

// The order kernel: a permutation of the B * S (sequence, split) pairs, longest first.
struct OrderArgs {
  const int32_t* ctx_lens;
  int32_t* order;              // [B * S][2]: the non-empty pairs longest first, then (-1, 0) each
  int32_t batch;
  int32_t num_splits;          // S <= kOrderMaxSplits
  int32_t split_tiles;
  int32_t max_ctx;
  int32_t window;
  int32_t num_sinks;
  int32_t num_queries;
};

struct MergeArgs {
  const float* o_part;         // [rows, S, d]
  const float* ml_part;        // [rows, S, 2]
  const int32_t* num_valid;    // [rows] or nullptr
  const int32_t* ctx_lens;     // decode path: valid splits = ceil(ctx / split_len) (nullptr otherwise)
  float* out;                  // [rows, d]
  int32_t rows;
  int32_t num_splits;
  int32_t h_q;                 // decode path: rows per sequence (row / h_q is the sequence)
  int32_t split_tiles;         // decode path: tiles per split
  int32_t max_ctx;             // decode path: clamp of ctx_lens
  int32_t window;              // decode path: as in SplitArgs
  int32_t num_sinks;
  int32_t num_queries;
  float* row_stats;            // nullptr, or [rows, 2]: the merged (m, l) of every row
};

// Per-position attention weights: for every (sequence, KV head, position) the sum over the
// group's query heads of 2^(s - m) / l, from the logits and row statistics the decode wrote.
struct ScoreArgs {
  const float* logits;         // [B * h_q, logits_ld]
  const float* row_stats;      // [B * h_q, 2]
  const int32_t* ctx_lens;
  float* scores;               // [B, h_kv, scores_ld]
  int64_t logits_ld;
  int64_t scores_ld;           // = max_ctx
  int32_t h_kv;
  int32_t group;
  int32_t max_ctx;
  int32_t window;
  int32_t num_sinks;
  int32_t accumulate;          // 0: write every entry (unattended ones 0); else add to attended ones
  int32_t chunks;              // position chunks of kScoreChunk per (sequence, KV head)
};
constexpr int kScoreChunk = 1024;

// Everything the append kernel needs: one new K/V row per (sequence, KV head) is stored at
// logical position positions[b] + pos_offset of sequence b.
struct AppendArgs {
  const void* k_new;           // [B, rows_per_seq, h_kv, d] contiguous
  const void* v_new;
  void* k;                     // caches (same layout rules as the split kernel)
  void* v;
  const int32_t* block_table;  // nullptr: contiguous cache
  const int32_t* positions;    // [B]
  int64_t k_sb, k_st, k_sh;
  int64_t v_sb, v_st, v_sh;
  int32_t h_kv;
  int32_t row_chunks;          // 16-byte pieces per row: d * elem_bytes / 16
  int32_t elem_bytes;
  int32_t bs_log2;             // paged only
  int32_t max_blocks;          // paged only
  int32_t limit;               // positions at or past it are not written
  int32_t pos_offset;          // 0, or -rows_per_seq when positions are context lengths
  int32_t rows_per_seq;        // new tokens per sequence, stored at positions[b] + pos_offset + i
  int32_t total;               // B * rows_per_seq * h_kv * row_chunks
};

struct Plan {
  int32_t num_splits;
  int32_t split_tiles;
  int32_t group_padded;
  int32_t variant;  // 0: vector fp32 path, 1: MFMA scores, 2: MFMA scores and P.V (rows mode)
  int32_t num_queries;  // query tokens per sequence (>= 1)
  int32_t row_blocks;   // rows mode: blocks of 16 query rows per (sequence, KV head)
  int32_t head_chunks;  // vector path: the group's query heads served by this many workgroups
  int32_t wave_heads;   // 1: each wave of a split workgroup serves its own KV head (SplitArgs)
  int32_t unit_order;   // 1: the order kernel lists the (sequence, split) pairs longest first
  int64_t grid_split;
  int64_t grid_merge;
  uint64_t workspace_bytes;
  uint64_t o_part_bytes;  // offset of ml_part inside the workspace
  uint64_t order_bytes_offset;  // offset of the order list (batch * S int32 pairs) when unit_order
};

// Host-only helpers (kv_attn_plan.cpp; no HIP calls).
kv_attn_status validate_params(const kv_attn_params* p);
// Checks that depend on whether the cache is paged (block_table present) or contiguous.
kv_attn_status validate_layout(const kv_attn_params* p, bool paged);
kv_attn_status make_plan(const kv_attn_params* p, int32_t num_cus, Plan* plan);
int32_t padded_group(int32_t g);
bool fault_injected(const char* where);  // KV_ATTN_FAULT=<where>: simulate a HIP failure

// Kernel launchers (kv_attn_kernels.hip); return a hipError_t value (0 = success).
int launch_split(const SplitArgs& a, const Plan& plan, int head_dim, bool paged, bool q_bf16,
                 bool kv_bf16, void* stream);
// The split kernel's instantiations, one family per file (kv_attn_split_*.hip).
int launch_split_mfma_d64(const SplitArgs& a, const Plan& plan, bool paged, void* stream);
int launch_split_mfma_d128(const SplitArgs& a, const Plan& plan, bool paged, void* stream);
int launch_split_vector_d64(const SplitArgs& a, const Plan& plan, bool q_bf16, bool kv_bf16,
                            void* stream);
int launch_split_vector_d128(const SplitArgs& a, const Plan& plan, bool q_bf16, bool kv_bf16,
                             void* stream);
int launch_split_rows(const SplitArgs& a, const Plan& plan, int head_dim, bool paged, void* stream);
int launch_merge(const MergeArgs& a, int head_dim, void* stream);
int launch_order(const OrderArgs& a, void* stream);
int launch_append(const AppendArgs& a, void* stream);
int launch_scores(const ScoreArgs& a, int64_t units, void* stream);

}  // namespace kvattn

#endif  // KV_ATTN_INTERNAL_H_
