/*
 * kv_attn.h — C ABI of the split-KV decode-attention library for MI355X (gfx950).
 *
 * One decode step of attention: for every sequence b and query head h,
 *
 *     out[b][h][:] = softmax(scale * q[b][h] . K_b^T) . V_b
 *
 * over the ctx_lens[b] positions held in the KV cache for the KV head that query head h reads.
 * This is the operation of one decode step in Ch. 19 "Inference Systems and Performance
 * Engineering" (第19章 推理系统与性能工程) §19.4.1, computed with the blockwise online-softmax
 * recurrence of §19.6.2 / §19.6.3 so the score row never leaves the chip. The cache may be
 * paged (§19.7.3: fixed-size blocks reached through a per-sequence block table). Query heads
 * share KV heads in groups (GQA) and each shared KV element is read from HBM once for the whole
 * group, the unique-KV assumption of Ch. 10 "System Model of Throughput and Latency"
 * (第十章 吞吐与延迟的系统模型) §4 and §5. The positions of a sequence are split across
 * workgroups; each split produces a running state (m, l, O) and a second pass merges them.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device pointers must point to device memory (or memory the device can
 *   read/write); host pointers to host memory. The library allocates nothing and frees
 *   nothing; the caller owns every buffer.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is enqueued
 *   asynchronously on it; no entry point synchronises unless the environment variable
 *   KV_ATTN_DEBUG=1 is set (then inputs are validated on the host and the stream is
 *   synchronised after the launch to report errors).
 * - Every argument the host can see is validated before any HIP call; on an invalid argument
 *   nothing is launched and the status says why. Contents of device-resident arrays (ctx_lens,
 *   block_table) are not validated on the fast path; see kv_attn_validate_host.
 * - Entry points are thread-safe: the only shared host state is a per-device cache of the
 *   compute unit count and one of the address of kv_attn_decode_noalloc's device scratch, each
 *   filled once (that scratch itself is shared by the calls on a device, see there).
 * - GQA grouping: with g = num_q_heads / num_kv_heads, query head h reads KV head h / g.
 * - ctx_lens[b] counts every position in the cache, the current token included (the caller has
 *   already appended it). Without a window every one of them is attended; ctx_lens[b] == 0
 *   gives an output row of zeros.
 * - Several query tokens (params.num_queries = gamma > 1): Ch. 19 §19.8 checks the gamma tokens
 *   a draft model proposed in one pass of the target model. Their K/V rows are already in the
 *   cache as its last gamma positions (ctx_lens[b] = T counts them), q and out are
 *   [batch, gamma, num_q_heads, head_dim], and query token j (0-based) attends causally to the
 *   first T - gamma + 1 + j positions (none if that is <= 0: a zero row). Every KV element is
 *   still read once for all gamma * g query rows of its KV head; scores and P.V then run on the
 *   matrix cores (P enters the product as the sum of two bf16 parts, about 16 significant
 *   bits). With a window, each token applies it to its own visible prefix. kv_attn_append_decode
 *   writes the gamma new rows at positions T - gamma .. T - 1 (nothing when T < gamma).
 * - Sliding window with attention sinks (params.window > 0): a sequence of length T attends
 *   only to its first min(num_sinks, T) positions and its last min(window, T) positions, each
 *   position once. Ch. 19 §19.4.3 bounds the cache of a long sequence by keeping only a recent
 *   window of tokens, and keeping the first few tokens as well (StreamingLLM's attention sinks)
 *   keeps the softmax stable; the positions outside the two ranges are neither read nor
 *   attended. The split kernel enumerates only the tiles of 16 positions that hold attended
 *   positions, so a step's HBM traffic follows the attended positions, not T.
 */
#ifndef KV_ATTN_H_
#define KV_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_ATTN_ABI_VERSION 5

/* Status codes. */
typedef enum kv_attn_status {
  KV_ATTN_OK = 0,
  KV_ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  KV_ATTN_ERR_SHAPE = 2,       /* inconsistent sizes (B, heads, block size, lengths) */
  KV_ATTN_ERR_UNSUPPORTED = 3, /* head_dim, group size, dtype or alignment not supported */
  KV_ATTN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the plan needs */
  KV_ATTN_ERR_HIP = 5,         /* the HIP runtime reported an error (launch or query) */
  KV_ATTN_ERR_TABLE = 6,       /* validator: ctx_lens / block_table content out of range */
  KV_ATTN_ERR_VALUE = 7,       /* an invalid scalar (non-finite scale, negative count) */
  KV_ATTN_ERR_SCRATCH = 8      /* kv_attn_decode_noalloc: the plan needs more workspace than
                                  the library's fixed device scratch holds */
} kv_attn_status;

/* Storage types of q and of the KV cache. */
typedef enum kv_attn_dtype {
  KV_ATTN_F32 = 0,
  KV_ATTN_BF16 = 1
} kv_attn_dtype;

/*
 * Problem description.
 *
 * q        : [batch, num_queries, num_q_heads, head_dim], contiguous, q_dtype (num_queries = 1:
 *            [batch, num_q_heads, head_dim]).
 * out      : the shape of q, contiguous, fp32.
 * k_cache,
 * v_cache  : element (block, token-in-block, kv_head, i) lives at
 *              base + block*stride_block + token*stride_token + kv_head*stride_head + i
 *            (elements of kv_dtype; the head_dim stride is 1). Both [blocks, block_size,
 *            h_kv, d] ("token major") and [blocks, h_kv, block_size, d] ("head major") are
 *            expressible; head major keeps the rows one (sequence, KV head) streams adjacent.
 * Paged cache (block_table != NULL): logical position t of sequence b is token
 *            t % block_size of physical block block_table[b * max_blocks_per_seq + t / block_size].
 *            Several sequences may point at the same physical block (prefix sharing); the cache
 *            is only read.
 * Contiguous cache (block_table == NULL): sequence b is "block" b and position t is token t;
 *            block_size is then the token capacity of one sequence slot.
 */
typedef struct kv_attn_params {
  int32_t batch;              /* B >= 1; B * gamma * h_kv * head_dim * elem_bytes / 16 < 2^31 */
  int32_t num_q_heads;        /* h_q >= 1 */
  int32_t num_kv_heads;       /* h_kv >= 1, h_q % h_kv == 0, 1 <= h_q / h_kv <= 16 */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t block_size;         /* paged: power of two >= 16; contiguous: slot capacity >= max_ctx_len */
  int32_t max_blocks_per_seq; /* paged: row length of block_table (>= 1); ignored if contiguous */
  int32_t max_ctx_len;        /* host-known upper bound of every ctx_lens[b] (>= 0); sizes the grid */
  int32_t num_splits;         /* 0 = automatic; > 0 requests that many splits per sequence */
  int32_t q_dtype;            /* kv_attn_dtype */
  int32_t kv_dtype;           /* kv_attn_dtype */
  float scale;                /* score scale; 0 means 1/sqrt(head_dim) */
  int32_t window;             /* 0 = attend every position; > 0 = sliding window of this many
                                 positions (plus the sinks), see the conventions above */
  int64_t num_blocks;         /* physical blocks in the caches (contiguous: batch); validator bound */
  int64_t k_stride_block, k_stride_token, k_stride_head; /* elements, >= 0 */
  int64_t v_stride_block, v_stride_token, v_stride_head; /* elements, >= 0 */
  int32_t num_sinks;          /* >= 0; leading positions attended as well when window > 0
                                 (ignored when window == 0) */
  int32_t num_queries;        /* query tokens per sequence, gamma (0 means 1); gamma > 1 is the
                                 verification step of speculative decoding, see below; needs
                                 bf16 q and KV and gamma * (num_q_heads / num_kv_heads) <= 32,
                                 gamma <= 16 */
} kv_attn_params;

/* The launch plan kv_attn_decode will use for a problem (split planning). */
typedef struct kv_attn_plan {
  int32_t num_splits;       /* S: splits per (sequence, KV head) */
  int32_t split_len;        /* positions per split, a multiple of 16 */
  int32_t grid_split;       /* workgroups of the split kernel: batch * num_kv_heads * S (times 2
                               when kernel_variant 0 serves a group above 8 heads in halves;
                               divided by 4 with wave_heads) */
  int32_t grid_merge;       /* workgroups of the merge kernel: batch * num_queries *
                               num_q_heads (0 when S == 1) */
  int32_t kernel_variant;   /* 0: fp32 vector path, 1: bf16 matrix-core (MFMA) scores,
                               2: bf16 MFMA scores and P.V ("rows mode": num_queries > 1, or
                               one token with a group of 4 or more query heads per KV head;
                               kv_attn_decode_scores runs the same variant) */
  int32_t group_padded;     /* compiled group width (power of two >= g; 8 for the halves above) */
  int32_t num_cus;          /* compute units the plan was made for */
  int32_t wave_heads;       /* 1: each split workgroup serves 4 KV heads, one per wave, every
                               wave streaming a whole split, so that a position's KV-head rows
                               (token-major) or 4 adjacent head slices of a block (head-major)
                               are read together. Needs num_kv_heads a multiple of 4 and no
                               halves; chosen for token-major caches (both stride_head <
                               stride_token) when batch * num_kv_heads < 4 * num_cus, and for
                               other layouts when batch * num_kv_heads < num_cus / 2, there
                               are at most 16 query rows per KV head and at least 1024 tiles
                               (16384 positions); in both cases only when tiles *
                               batch * num_kv_heads / 4 >= 32 * num_cus (64 * num_cus with 2
                               row blocks), i.e. every wave gets >= 32 tiles on a full device.
                               The automatic S then counts batch * num_kv_heads / 4 workgroups
                               per split and allows one split per 4 tiles. 0: one KV head per
                               workgroup. */
  int32_t unit_order;       /* 1: a one-workgroup order kernel first lists the (sequence, split)
                               pairs longest first (whole splits, then the sequences' last
                               partial splits by decreasing length; empty pairs last, as -1,
                               their workgroups leaving at once) and the split workgroups take
                               them in that order, so the last workgroups dispatched are the
                               shortest (on MI355X, C4's ragged batch: split kernel 1397 ->
                               1334 us). Chosen when S > 1, S <= 256, no halves
                               and batch * num_kv_heads (/ 4 with wave_heads) >= 4 * num_cus,
                               i.e. the split workgroups take several rounds of the device.
                               Not used by kv_attn_decode_scores. 0: workgroups take the pairs
                               split by split. */
  int32_t reserved;         /* 0 */
  uint64_t workspace_bytes; /* workspace kv_attn_decode needs (0 when S == 1) */
  uint64_t ml_offset;       /* byte offset of the (m, l) array inside the workspace (S > 1) */
  uint64_t order_offset;    /* byte offset of the order list (batch * S pairs of int32: the
                               pair's index b * S + split, or -1, and the sequence's clamped
                               length) inside the workspace when unit_order, else 0 */
} kv_attn_plan;

/* ABI version of the loaded library (KV_ATTN_ABI_VERSION it was built with). */
int32_t kv_attn_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* kv_attn_status_string(int32_t status);

/*
 * Plan the launch for `p` as if on a device with `num_cus` compute units (0 = query the
 * current HIP device). Validates `p` exactly as kv_attn_decode does (pointers aside). Split
 * planning: tiles of 16 positions; the splits per sequence are chosen so that the split
 * workgroups number at least about one per compute unit (two for kernel_variant 2 with more
 * than 16 query rows per KV head), there are at most ceil(tiles / 16) splits (ceil(tiles / 4)
 * with wave_heads), each spans at most
 * 256 tiles (512 when the split workgroups of one split are under half the compute units, or
 * with num_queries > 1 or wave_heads), and a
 * caller-given num_splits overrides the count. With a window the tiles counted are those a
 * sequence can visit: ceil(min(num_sinks, max_ctx_len) / 16) + ceil((window + gamma - 1) / 16)
 * + 1 at most, gamma being num_queries (the union of the gamma query tokens' windows).
 * Writes *plan only on KV_ATTN_OK.
 */
kv_attn_status kv_attn_get_plan(const kv_attn_params* p, int32_t num_cus, kv_attn_plan* plan);

/* Workspace bytes kv_attn_decode needs for `p` on the current device; 0 if none or if `p`
 * is invalid. */
size_t kv_attn_workspace_size(const kv_attn_params* p);

/*
 * Decode attention for one step (see the top of this file for the computation).
 *
 * q, k_cache, v_cache : device, layouts above, 16-byte aligned; every stride times the
 *                       element size must be a multiple of 16 bytes.
 * block_table         : device int32 [batch, max_blocks_per_seq], or NULL for a contiguous cache.
 *                       Entries past ceil(ctx_lens[b] / block_size) are never read.
 * ctx_lens            : device int32 [batch]; contract 0 <= ctx_lens[b] <= max_ctx_len (values
 *                       outside are clamped into that range).
 * out                 : device fp32 [batch, num_q_heads, head_dim] ([batch, gamma, num_q_heads,
 *                       head_dim] with gamma = num_queries > 1); must not alias any input.
 * workspace           : device scratch of at least kv_attn_workspace_size(p) bytes when the plan
 *                       has more than one split (may be NULL otherwise); contents need no
 *                       initialisation and are left unspecified.
 * Returns KV_ATTN_OK once the kernels are enqueued.
 */
kv_attn_status kv_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens, float* out,
                              const kv_attn_params* p, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The two passes of kv_attn_decode, separately (same arguments and checks; calling
 * kv_attn_decode_split then kv_attn_decode_merge with the same p, workspace and stream is
 * exactly kv_attn_decode).
 *
 * kv_attn_decode_split: the streaming pass. With a one-split plan it writes `out` and the merge
 * pass is a no-op. Otherwise it leaves every split's running state in the workspace: the
 * unnormalised sums O at byte offset 0 as fp32 [rows, S, head_dim] and (m, l) at byte offset
 * plan.ml_offset as fp32 [rows, S, 2], rows = batch * gamma * num_q_heads in the row order of
 * `out` (gamma = 1 for a single query token), m being a base-2 maximum (see
 * kv_attn_merge). Split s of sequence b covers positions [s * split_len, (s+1) * split_len) of
 * that sequence; splits starting at or past ctx_lens[b] are not written. With a window the
 * split covers the same number of 16-position tiles, counted over the visited tiles only (the
 * sink tiles first, then the window's), so that ceil(n_b / (split_len / 16)) splits are written,
 * n_b being the sequence's visited tiles.
 * kv_attn_decode_merge: the merge pass over a workspace the split pass filled; it merges, for
 * row (b, h), the first ceil(ctx_lens[b] / split_len) splits into out (with a window, the
 * splits the split pass wrote).
 */
kv_attn_status kv_attn_decode_split(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens, float* out,
                                    const kv_attn_params* p, void* workspace,
                                    size_t workspace_bytes, void* stream);
kv_attn_status kv_attn_decode_merge(const int32_t* ctx_lens, float* out, const kv_attn_params* p,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Merge per-split running states into outputs (the second pass of kv_attn_decode, exposed
 * for callers that produce split states elsewhere, e.g. position ranges held by different
 * devices). The merge rescales each state to the common maximum, as in the online-softmax
 * recurrence of Ch. 19 §19.6.2 applied with a whole split state in place of one block:
 *
 *     M = max_s m_s;  w_s = 2^(m_s - M);  out = (sum_s w_s O_s) / (sum_s w_s l_s)
 *
 * o_partial  : device fp32 [rows, num_splits, head_dim], unnormalised sums O_s.
 * ml_partial : device fp32 [rows, num_splits, 2] holding (m_s, l_s); m_s is a maximum of
 *              base-2 scaled scores (natural-log logits times log2(e)); a state with
 *              m_s = -inf and l_s = 0 is empty and is skipped.
 * num_valid  : device int32 [rows] (only the first num_valid[r] splits of row r are merged,
 *              clamped to [0, num_splits]) or NULL (all splits).
 * out        : device fp32 [rows, head_dim]; a row with no non-empty state is written as zeros.
 * head_dim   : 64 or 128; num_splits at most 4096.
 */
kv_attn_status kv_attn_merge(const float* o_partial, const float* ml_partial,
                             const int32_t* num_valid, float* out, int32_t rows,
                             int32_t num_splits, int32_t head_dim, void* stream);

/*
 * Append one token's K and V rows per sequence to the cache: the step that precedes attention
 * in every decode step (Ch. 10 §4 counts this new-KV write; Ch. 19 §19.7.3 grows a paged cache
 * block by block through the block table). With p->num_queries = n > 1, n consecutive tokens
 * per sequence (a speculative draft, Ch. 19 §19.8) at positions[b] .. positions[b] + n - 1.
 *
 * k_new, v_new : device, kv_dtype, contiguous [batch, num_kv_heads, head_dim] (n > 1:
 *                [batch, n, num_kv_heads, head_dim]), 16-byte aligned.
 * k_cache,
 * v_cache      : the caches described by p (strides, block_size, block_table as for decode);
 *                written in place at one slot per (sequence, KV head) and nowhere else.
 * positions    : device int32 [batch]: logical position written for sequence b, through
 *                block_table[b][pos / block_size] (paged) or slot pos of sequence b
 *                (contiguous). A negative position (idle sequence) or one at or past the
 *                capacity (max_blocks_per_seq * block_size, or block_size when contiguous) writes
 *                nothing. The block that holds the position must already be in the table.
 * Enqueued on `stream`; the rows of a sequence must not be read by other work in flight.
 */
kv_attn_status kv_attn_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* block_table, const int32_t* positions,
                              const kv_attn_params* p, void* stream);

/*
 * kv_attn_append then kv_attn_decode in one call: the new token of sequence b is the last
 * position ctx_lens[b] counts, so it is written at position ctx_lens[b] - 1 (nothing for an empty
 * sequence) and then attended together with the cached ones; with gamma = num_queries > 1 the
 * gamma new tokens are written at ctx_lens[b] - gamma .. ctx_lens[b] - 1 (nothing when
 * ctx_lens[b] < gamma). Arguments as for the two calls; every check of both runs before
 * anything is launched. With bf16 q and KV (kernel_variant 1 or 2) the append is fused into the
 * split kernel (Ch. 10 §4: the new K/V is written and used by the same step): the workgroup whose
 * tile holds a new row takes it from k_new / v_new and writes it into the cache, and no append
 * kernel is launched; the caches end up byte-identical to the two separate calls, and the output
 * equal up to rounding (that split visits its tiles in order). The fp32 vector path launches the
 * append kernel first.
 */
kv_attn_status kv_attn_append_decode(const void* q, const void* k_new, const void* v_new,
                                     void* k_cache, void* v_cache, const int32_t* block_table,
                                     const int32_t* ctx_lens, float* out, const kv_attn_params* p,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode with score export: kv_attn_decode, and in addition the attention weight every cached
 * position received, summed over the g query heads that share its KV head — the per-entry score
 * that eviction policies rank by (Ch. 19 §19.4.3: a few "heavy hitter" tokens collect most of
 * the attention; the eviction exercise takes one score per (layer, head, token)).
 *
 * token_scores : device fp32 [batch, num_kv_heads, max_ctx_len] contiguous. For every attended
 *                position t of sequence b (t < ctx_lens[b], and inside the window when one is
 *                set) entry (b, kvh, t) = sum over j < g of softmax weight of t for query head
 *                kvh*g + j; the weights of one query head sum to 1, so a sequence's entries per
 *                KV head sum to g. accumulate == 0 writes every entry (unattended ones 0);
 *                accumulate != 0 adds the weights to the attended entries and leaves the others
 *                (a running sum across decode steps, as H2O keeps). Must not alias any input.
 * workspace    : at least kv_attn_scores_workspace_size(p) bytes, 16-byte aligned, always
 *                required (the kernels keep the base-2 scores of every visited position and
 *                the final (m, l) of every query row there: the decode workspace, then
 *                4 * batch * num_q_heads * roundup(max_ctx_len, 16) + 8 * batch * num_q_heads
 *                bytes).
 * One query token per sequence, and q and KV both bf16 or both fp32 (otherwise
 * KV_ATTN_ERR_UNSUPPORTED). Other arguments, checks and errors as for kv_attn_decode.
 */
size_t kv_attn_scores_workspace_size(const kv_attn_params* p);
kv_attn_status kv_attn_decode_scores(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* ctx_lens, float* out,
                                     float* token_scores, int32_t accumulate,
                                     const kv_attn_params* p, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Host-side check of the device-resident inputs' contents (debug aid; runs on the CPU and
 * touches no device): every 0 <= ctx_lens[b] <= max_ctx_len and, for a paged cache
 * (block_table != NULL), every entry 0 <= block_table[b][i] < num_blocks for
 * i < ceil(ctx_lens[b] / block_size). Both arrays are host copies. Returns KV_ATTN_ERR_TABLE
 * on the first violation, KV_ATTN_OK otherwise (after validating `p` as kv_attn_get_plan does).
 */
kv_attn_status kv_attn_validate_host(const int32_t* block_table, const int32_t* ctx_lens,
                                     const kv_attn_params* p);

/*
 * kv_attn_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, checks and results as
 * kv_attn_decode (the same plan and kernels, so the output is bit-identical to it), but the
 * split states go to a device array the library holds itself, KV_ATTN_NOALLOC_SCRATCH_BYTES
 * bytes per device, kept until the process ends. Nothing is allocated or freed by the call.
 * Returns KV_ATTN_ERR_SCRATCH, before anything is launched, when the plan needs a larger
 * workspace than that (kv_attn_workspace_size(p) > KV_ATTN_NOALLOC_SCRATCH_BYTES). Every call
 * on a device uses that device's one array: calls that overlap on one device (other streams,
 * other threads, other graphs in flight) race on it and must be serialised by the caller. Its
 * contents need no initialisation (each call writes every state it reads) and are left
 * unspecified. The first call on a device looks up the array's address there (HIP error:
 * KV_ATTN_ERR_HIP); graph capture therefore works from the second call on a device.
 */
#define KV_ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
kv_attn_status kv_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      float* out, const kv_attn_params* p, void* stream);

/*
 * Measurement aid, not part of attention: the practical read ceiling of the device. Streams
 * `bytes` of device memory at `src` with the 16-byte nontemporal loads the split kernel uses for
 * its KV tiles, in the most favourable order measured (each 256-thread workgroup reads one
 * contiguous KV_ATTN_PROBE_CHUNK-byte range, four loads in flight per lane) and with no compute,
 * enqueued on `stream`; timing a few launches with device events gives the rate a bare read
 * stream reaches, against which the attention kernels' rates can be read as well as against the
 * published peak.
 * src   : device, 16-byte aligned, `bytes` readable (a positive multiple of 16; it is only read).
 * sink  : device uint32 (one word); it may be overwritten with a meaningless value (the kernel
 *         keeps its loads live with a store it practically never takes).
 * Returns KV_ATTN_ERR_NULL for a NULL pointer, KV_ATTN_ERR_UNSUPPORTED for a misaligned `src`,
 * a size that is 0 or not a multiple of 16, or more than 2^31 - 1 chunks, KV_ATTN_ERR_HIP if the
 * launch fails.
 */
#define KV_ATTN_PROBE_CHUNK (1u << 20)
kv_attn_status kv_attn_read_probe(const void* src, uint64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KV_ATTN_H_ */
