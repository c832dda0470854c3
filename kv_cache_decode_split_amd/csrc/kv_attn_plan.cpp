// Host-only part of the library: argument validation, split planning, the host-side table
// validator and status strings. No HIP calls, so it builds and runs on a machine without a GPU.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "kv_attn_internal.h"

namespace kvattn {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int elem_bytes(int32_t dtype) { return dtype == KV_ATTN_BF16 ? 2 : 4; }

}  // namespace

int32_t padded_group(int32_t g) {
  int32_t G = 1;
  while (G < g) G <<= 1;
  return G;
}

bool fault_injected(const char* where) {
  const char* f = getenv("KV_ATTN_FAULT");
  return f != nullptr && strcmp(f, where) == 0;
}

kv_attn_status validate_params(const kv_attn_params* p) {
  if (p == nullptr) return KV_ATTN_ERR_NULL;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1) return KV_ATTN_ERR_SHAPE;
  if (p->num_q_heads % p->num_kv_heads != 0) return KV_ATTN_ERR_SHAPE;
  const int32_t g = p->num_q_heads / p->num_kv_heads;
  if (g > 16) return KV_ATTN_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return KV_ATTN_ERR_UNSUPPORTED;
  if ((p->q_dtype != KV_ATTN_F32 && p->q_dtype != KV_ATTN_BF16) ||
      (p->kv_dtype != KV_ATTN_F32 && p->kv_dtype != KV_ATTN_BF16))
    return KV_ATTN_ERR_UNSUPPORTED;
  if (p->max_ctx_len < 0 || p->num_splits < 0) return KV_ATTN_ERR_VALUE;
  if (p->window < 0 || p->num_sinks < 0 || p->num_queries < 0) return KV_ATTN_ERR_VALUE;
  if (p->num_queries > kMaxQueries) return KV_ATTN_ERR_UNSUPPORTED;
  if (!isfinite(p->scale)) return KV_ATTN_ERR_VALUE;
  if (p->block_size < 1 || p->num_blocks < 1) return KV_ATTN_ERR_SHAPE;
  const int64_t strides[6] = {p->k_stride_block, p->k_stride_token, p->k_stride_head,
                              p->v_stride_block, p->v_stride_token, p->v_stride_head};
  const int eb = elem_bytes(p->kv_dtype);
  for (int64_t s : strides) {
    if (s < 0) return KV_ATTN_ERR_SHAPE;
    // Every row starts 16-byte aligned so that each lane issues whole 128-bit loads.
    if ((s * eb) % 16 != 0) return KV_ATTN_ERR_UNSUPPORTED;
  }
  // Rows inside one 16-position tile are addressed with 32-bit byte offsets.
  if (p->k_stride_token * eb * kTile >= (int64_t(1) << 31) ||
      p->v_stride_token * eb * kTile >= (int64_t(1) << 31))
    return KV_ATTN_ERR_UNSUPPORTED;
  // The append kernel numbers its 16-byte pieces (sequence, query token, KV head, piece of a
  // row) with 32-bit indices.
  const int64_t pieces = int64_t(p->batch) * (p->num_queries > 1 ? p->num_queries : 1) *
                         p->num_kv_heads * (p->head_dim * eb / 16);
  if (pieces > int64_t(INT32_MAX)) return KV_ATTN_ERR_UNSUPPORTED;
  return KV_ATTN_OK;
}

kv_attn_status validate_layout(const kv_attn_params* p, bool paged) {
  const kv_attn_status st = validate_params(p);
  if (st != KV_ATTN_OK) return st;
  if (paged) {
    // Tiles of kTile positions must never straddle two blocks.
    if (!is_pow2(p->block_size) || p->block_size < kTile) return KV_ATTN_ERR_SHAPE;
    if (p->max_blocks_per_seq < 1) return KV_ATTN_ERR_SHAPE;
    if (int64_t(p->max_ctx_len) > int64_t(p->max_blocks_per_seq) * p->block_size)
      return KV_ATTN_ERR_SHAPE;
  } else {
    if (p->max_ctx_len > p->block_size) return KV_ATTN_ERR_SHAPE;
    if (p->num_blocks < p->batch) return KV_ATTN_ERR_SHAPE;
  }
  return KV_ATTN_OK;
}

int32_t num_queries(const kv_attn_params* p) { return p->num_queries > 1 ? p->num_queries : 1; }

// Tiles of kTile positions a sequence of at most max_ctx_len positions can visit. With a
// window W and n sinks that is at most ceil(min(n, T)/16) sink tiles plus the tiles that the
// W + gamma - 1 consecutive positions of the gamma query tokens' windows can touch, and never
// more than the whole sequence's tiles.
int64_t max_visited_tiles(const kv_attn_params* p) {
  const int64_t all = ceil_div(p->max_ctx_len > 0 ? p->max_ctx_len : 1, kTile);
  if (p->window <= 0) return all;
  const int64_t sinks = p->num_sinks < p->max_ctx_len ? p->num_sinks : p->max_ctx_len;
  const int64_t span = int64_t(p->window) + num_queries(p) - 1;
  const int64_t bounded = ceil_div(sinks, kTile) + ceil_div(span, kTile) + 1;
  return bounded < all ? bounded : all;
}

// Split planning. The visited tiles of one (sequence, KV head) pair are cut into S splits of
// split_tiles tiles; every split is one workgroup of kWaves waves. The grid is sized from the
// host-known max_ctx_len: workgroups whose split starts past their own sequence's tiles exit at
// once, so ragged batches need no host copy of ctx_lens.
kv_attn_status make_plan(const kv_attn_params* p, int32_t num_cus, Plan* plan) {
  const kv_attn_status st = validate_params(p);
  if (st != KV_ATTN_OK) return st;
  if (num_cus < 1) return KV_ATTN_ERR_VALUE;
  // Several query tokens: the rows-mode kernel takes bf16 q and KV and up to kMaxQueryRows
  // query rows per KV head.
  if (p->num_queries > 1) {
    if (p->q_dtype != KV_ATTN_BF16 || p->kv_dtype != KV_ATTN_BF16) return KV_ATTN_ERR_UNSUPPORTED;
    if (p->num_queries * (p->num_q_heads / p->num_kv_heads) > kMaxQueryRows)
      return KV_ATTN_ERR_UNSUPPORTED;
  }
  const int64_t tiles_max = max_visited_tiles(p);
  const int64_t units = int64_t(p->batch) * p->num_kv_heads;
  const bool force_vector = getenv("KV_ATTN_FORCE_VECTOR") != nullptr &&
                            strcmp(getenv("KV_ATTN_FORCE_VECTOR"), "1") == 0;
  const int32_t nq = num_queries(p);
  const int32_t g = p->num_q_heads / p->num_kv_heads;
  const bool bf16 = p->q_dtype == KV_ATTN_BF16 && p->kv_dtype == KV_ATTN_BF16 && !force_vector;
  plan->num_queries = nq;
  plan->row_blocks = 0;
  plan->head_chunks = 1;
  // Rows mode (variant 2) also serves one token once the group has kRowsMinGroup heads: P.V
  // then costs less on the matrix cores than as per-lane FMAs for every head (on MI355X the
  // C5 shape, group 8, went from 0.79 to 0.82 of peak, at the bandwidth of the loads alone).
  if (nq > 1 || (bf16 && g >= kRowsMinGroup)) {
    plan->variant = 2;
    plan->row_blocks = int32_t(ceil_div(int64_t(nq) * g, 16));
  } else {
    plan->variant = bf16 ? 1 : 0;
  }
  // The vector path (fp32 or mixed inputs) holds every head's query and output slices in
  // registers; above kVectorMaxGroup heads that spilled hundreds of registers to scratch, so
  // two workgroups then serve the halves of the group (each reading the KV head once).
  if (plan->variant == 0 && g > kVectorMaxGroup) plan->head_chunks = 2;
  // Wave heads: a split workgroup serves kWaves KV heads, one per wave, each wave streaming a
  // whole split, so that the rows of one position (token-major) or kWaves adjacent head slices of
  // one block (head-major) are read together. MI355X, split kernel, fraction of peak:
  //  * token-major: C5 0.72 -> 0.83, C2 0.74 -> 0.84, C3 0.82 -> 0.86, C3 with a 2048-position
  //    window 0.73 -> 0.82, C5 with 4 tokens 0.70 -> 0.77; C4 (1024 units, ragged) drops from
  //    0.80 to 0.68 at every split count tried, so kWaves * num_cus units or more keep one KV
  //    head per workgroup;
  //  * head-major, few units (long sequences split for parallelism): C5 0.824 -> 0.843, with
  //    groups 1 and 4 0.83 -> 0.85, with blocks in physical order 0.81 -> 0.86; C3 (512 units)
  //    unchanged, C2 (256 units, unsplit) 0.87 -> 0.84 and two-block rows mode (C5 with 4
  //    tokens) 0.80 -> 0.77, so head-major takes it only with few units, one row block and at
  //    least kWaves * kMaxSplitTiles tiles (16384 positions);
  //  * both: when a device's worth of such workgroups leaves each wave only a few tiles the
  //    step is latency-bound and the longer per-wave chains cost more than they gain (C5 with
  //    a 4096-position window, ~9 tiles per wave: 16.3 -> 19.2 us token-major, 15.0 -> 19.1 us
  //    head-major; C1 adds a merge pass), so each wave must get kWaveHeadsMinTiles tiles.
  const bool token_major = p->k_stride_head < p->k_stride_token && p->v_stride_head < p->v_stride_token;
  // KV_ATTN_WAVE_HEADS=0 / =1 overrides the choice (=1: whenever the shape allows it).
  const char* wh_env = getenv("KV_ATTN_WAVE_HEADS");
  const int wh_force = wh_env == nullptr ? -1 : strcmp(wh_env, "1") == 0 ? 1 : strcmp(wh_env, "0") == 0 ? 0 : -1;
  const int64_t per_cu = plan->row_blocks == 2 ? 2 : 1;  // split workgroups per CU (see below)
  const bool long_waves = tiles_max * (units / kWaves) >= int64_t(kWaveHeadsMinTiles) * num_cus * per_cu;
  const bool wave_heads_fit = token_major
      ? units < int64_t(kWaves) * num_cus
      : units * 2 < num_cus && plan->row_blocks < 2 && tiles_max >= int64_t(kWaves) * kMaxSplitTiles;
  const bool wave_heads_ok = p->num_kv_heads % kWaves == 0 && plan->head_chunks == 1;
  plan->wave_heads = wave_heads_ok && (wh_force >= 0 ? wh_force == 1 : wave_heads_fit && long_waves) ? 1 : 0;
  // Split workgroups per split.
  const int64_t work_units = plan->wave_heads ? units / kWaves : units * plan->head_chunks;

  int64_t S;
  if (p->num_splits > 0) {
    S = p->num_splits;
  } else {
    // About one split workgroup per CU (per_cu); two for two-block rows mode, which keeps one
    // tile in flight per wave and needs two waves per SIMD to keep enough loads outstanding.
    S = ceil_div(int64_t(num_cus) * per_cu, work_units);
    // Split length cap: 256 tiles keep a batch of many (sequence, KV head) units balanced when
    // its lengths are ragged; with few units (long sequences split for parallelism) or several
    // query tokens (heavier per-split epilogue and merge rows) 512 tiles stream faster. MI355X
    // sweeps: C4 (1024 units, ragged) best at 256; C5 (32 units, one KV head per workgroup)
    // 0.825 at 512 against 0.815;
    // C3 with 8 tokens 0.828 against 0.776, C5 with 4 tokens 0.807 against 0.755.
    const int64_t cap = (plan->wave_heads || nq > 1 || work_units * 2 < num_cus) ? kMaxSplitTilesLong
                                                                                 : kMaxSplitTiles;
    // Splits of >= 16 tiles (>= 4 per wave); with wave heads every wave streams the whole
    // split, so >= 4 tiles.
    const int64_t most = ceil_div(tiles_max, plan->wave_heads ? kMinSplitTiles / kWaves : kMinSplitTiles);
    const int64_t least = ceil_div(tiles_max, cap);
    if (S > most) S = most;
    if (S < least) S = least;
  }
  if (S > tiles_max) S = tiles_max;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  const int64_t split_tiles = ceil_div(tiles_max, S);
  S = ceil_div(tiles_max, split_tiles);

  plan->num_splits = int32_t(S);
  plan->split_tiles = int32_t(split_tiles);
  plan->group_padded = plan->head_chunks > 1 ? kVectorMaxGroup : padded_group(g);
  plan->grid_split = work_units * S;
  const int64_t rows = int64_t(p->batch) * nq * p->num_q_heads;
  plan->grid_merge = S > 1 ? rows : 0;
  // Unit order: when the split workgroups take several rounds of the device, the ones dispatched
  // last decide the tail; split by split, those are whatever pairs come last, often long ones.
  // Longest first leaves the short partial splits for the end (MI355X, C4's ragged batch: split
  // kernel 1397 -> 1334 us; a list-scheduling model of its measured per-tile times predicted
  // 1394 -> 1329). KV_ATTN_UNIT_ORDER=0 / =1 overrides the choice where the shape allows it.
  const char* uo_env = getenv("KV_ATTN_UNIT_ORDER");
  const int uo_force = uo_env == nullptr ? -1 : strcmp(uo_env, "1") == 0 ? 1 : strcmp(uo_env, "0") == 0 ? 0 : -1;
  const bool order_ok = S > 1 && S <= kOrderMaxSplits && plan->head_chunks == 1;
  const bool order_pays = work_units >= int64_t(kOrderMinRounds) * num_cus;
  plan->unit_order = order_ok && (uo_force >= 0 ? uo_force == 1 : order_pays) ? 1 : 0;
  plan->order_bytes_offset = 0;
  if (S > 1) {
    const uint64_t o_bytes = uint64_t(rows) * uint64_t(S) * uint64_t(p->head_dim) * 4u;
    const uint64_t o_aligned = (o_bytes + 255u) & ~uint64_t(255u);
    plan->o_part_bytes = o_aligned;
    plan->workspace_bytes = o_aligned + uint64_t(rows) * uint64_t(S) * 2u * 4u;
    if (plan->unit_order) {
      plan->order_bytes_offset = (plan->workspace_bytes + 255u) & ~uint64_t(255u);
      plan->workspace_bytes = plan->order_bytes_offset + uint64_t(p->batch) * uint64_t(S) * 8u;
    }
  } else {
    plan->o_part_bytes = 0;
    plan->workspace_bytes = 0;
  }
  if (plan->grid_split > 0x7fffffffLL || plan->grid_merge > 0x7fffffffLL) return KV_ATTN_ERR_SHAPE;
  return KV_ATTN_OK;
}

}  // namespace kvattn

extern "C" {

int32_t kv_attn_abi_version(void) { return KV_ATTN_ABI_VERSION; }

const char* kv_attn_status_string(int32_t status) {
  switch (status) {
    case KV_ATTN_OK: return "ok";
    case KV_ATTN_ERR_NULL: return "a required pointer is NULL";
    case KV_ATTN_ERR_SHAPE: return "inconsistent sizes";
    case KV_ATTN_ERR_UNSUPPORTED: return "unsupported head_dim, group size, dtype or alignment";
    case KV_ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_ATTN_ERR_HIP: return "HIP runtime error";
    case KV_ATTN_ERR_TABLE: return "ctx_lens or block_table content out of range";
    case KV_ATTN_ERR_VALUE: return "invalid scalar argument";
    case KV_ATTN_ERR_SCRATCH: return "problem needs more workspace than the fixed device scratch";
    default: return "unknown status";
  }
}

kv_attn_status kv_attn_validate_host(const int32_t* block_table, const int32_t* ctx_lens,
                                     const kv_attn_params* p) {
  const bool paged = block_table != nullptr;
  const kv_attn_status st = kvattn::validate_layout(p, paged);
  if (st != KV_ATTN_OK) return st;
  if (ctx_lens == nullptr) return KV_ATTN_ERR_NULL;
  for (int32_t b = 0; b < p->batch; ++b) {
    const int32_t len = ctx_lens[b];
    if (len < 0 || len > p->max_ctx_len) return KV_ATTN_ERR_TABLE;
    if (!paged) continue;
    const int64_t nblk = kvattn::ceil_div(len, p->block_size);
    if (nblk > p->max_blocks_per_seq) return KV_ATTN_ERR_TABLE;
    const int32_t* row = block_table + int64_t(b) * p->max_blocks_per_seq;
    for (int64_t i = 0; i < nblk; ++i)
      if (row[i] < 0 || row[i] >= p->num_blocks) return KV_ATTN_ERR_TABLE;
  }
  return KV_ATTN_OK;
}

}  // extern "C"
