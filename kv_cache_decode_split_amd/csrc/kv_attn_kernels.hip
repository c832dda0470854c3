// Split-KV decode attention for gfx950: the merge kernel (second pass over the split states),
// the per-position score kernel, the append kernel, and the dispatch of the split kernel to the
// launcher that instantiates the right variant (kv_attn_split_*.hip; the kernel itself is in
// kv_attn_split.h).
#include "kv_attn_split.h"

namespace kvattn {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) x = fmaxf(x, lane_xor(x, mask));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) x += lane_xor(x, mask);
  return x;
}

// Second pass: one workgroup per (sequence, query head) row merges that row's split states,
// with the rescale-and-add step of the online-softmax recurrence applied to whole states:
// M = max_s m_s, w_s = 2^(m_s - M) (0 for an empty state), out = sum_s w_s O_s / sum_s w_s l_s.
// Threads first share the maxima and weights of all splits, then each output element is
// accumulated over kMergeThreads / D interleaved subsets of splits (independent loads in flight)
// and the subsets are added in a fixed order. The loads that depend on nothing (the row's
// length or valid count, the first split states and the first partial outputs) are all issued
// before any is used, so a row costs one memory round trip instead of three; entries past the
// valid count lie inside the workspace and are read but never used.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const MergeArgs a) {
  constexpr int SUB = kMergeThreads / D;
  constexpr int NW = kMergeThreads / 64;
  constexpr int PRE = 8;  // partial-output loads per thread issued up front
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[NW];
  __shared__ float s_acc[SUB][D];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = blockIdx.x;
  const int S = a.num_splits;
  const float* ml = a.ml_part + int64_t(row) * S * 2;
  const float* o = a.o_part + int64_t(row) * S * D;
  const int e = tid % D;
  const int sub = tid / D;

  int raw = S;
  if (a.num_valid != nullptr)
    raw = a.num_valid[row];
  else if (a.ctx_lens != nullptr)
    raw = a.ctx_lens[row / a.h_q];
  float m_first = neg_inf(), l_first = 0.f;
  if (tid < S) {
    m_first = ml[2 * tid];
    l_first = ml[2 * tid + 1];
  }
  float o_pre[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int s = sub + k * SUB;
    o_pre[k] = s < S ? o[int64_t(s) * D + e] : 0.f;
  }

  int nv = S;
  if (a.num_valid != nullptr) {
    nv = raw;
  } else if (a.ctx_lens != nullptr) {
    // Same tile enumeration as the split kernel: splits past the sequence's tiles hold nothing.
    const int ctx = raw < 0 ? 0 : (raw > a.max_ctx ? a.max_ctx : raw);
    int n_first = 0, win_tile0 = 0;
    if (a.window > 0) {
      n_first = (min(a.num_sinks, ctx) + kTile - 1) / kTile;
      win_tile0 = max(max(ctx - (a.num_queries - 1) - a.window, 0) / kTile, n_first);
    }
    const int ntiles = n_first + max((ctx + kTile - 1) / kTile - win_tile0, 0);
    nv = (ntiles + a.split_tiles - 1) / a.split_tiles;
  }
  nv = nv < 0 ? 0 : (nv > S ? S : nv);

  float m_loc = tid < nv ? m_first : neg_inf();
  for (int s = tid + kMergeThreads; s < nv; s += kMergeThreads) m_loc = fmaxf(m_loc, ml[2 * s]);
  m_loc = wave_max(m_loc);
  if (lane == 0) s_red[wave] = m_loc;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
  __syncthreads();

  float l_loc = 0.f;
  for (int s = tid; s < nv; s += kMergeThreads) {
    const float m = s == tid ? m_first : ml[2 * s];
    const float l = s == tid ? l_first : ml[2 * s + 1];
    const float w = (m == neg_inf()) ? 0.f : exp2_fast(m - M);
    s_w[s] = w;
    l_loc = fmaf(w, l, l_loc);
  }
  l_loc = wave_sum(l_loc);
  if (lane == 0) s_red[wave] = l_loc;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += s_red[w];

  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int s = sub + k * SUB;
    if (s < nv) acc = fmaf(s_w[s], o_pre[k], acc);
  }
  int s = sub + PRE * SUB;
  for (; s + 3 * SUB < nv; s += 4 * SUB) {
    const float o0 = o[int64_t(s) * D + e];
    const float o1 = o[int64_t(s + SUB) * D + e];
    const float o2 = o[int64_t(s + 2 * SUB) * D + e];
    const float o3 = o[int64_t(s + 3 * SUB) * D + e];
    acc = fmaf(s_w[s], o0, acc);
    acc = fmaf(s_w[s + SUB], o1, acc);
    acc = fmaf(s_w[s + 2 * SUB], o2, acc);
    acc = fmaf(s_w[s + 3 * SUB], o3, acc);
  }
  for (; s < nv; s += SUB) acc = fmaf(s_w[s], o[int64_t(s) * D + e], acc);
  s_acc[sub][e] = acc;
  __syncthreads();
  if (tid < D) {
    float total = s_acc[0][tid];
#pragma unroll
    for (int k = 1; k < SUB; ++k) total += s_acc[k][tid];
    a.out[int64_t(row) * D + tid] = L > 0.f ? total / L : 0.f;
  }
  if (a.row_stats != nullptr && tid == 0) {
    a.row_stats[int64_t(row) * 2 + 0] = M;
    a.row_stats[int64_t(row) * 2 + 1] = L;
  }
}

// Per-position attention weights (score export): one workgroup per (sequence, KV head, chunk of
// kScoreChunk positions), reading the split kernel's scores ([B*h_q, logits_ld], one row per
// query head). The weight of an attended position t for query row j is
// 2^(s_jt - m_j) / l_j with the row's final base-2 maximum m_j and sum l_j; the group's rows are
// summed. Unattended positions (past the length, or outside the window) get 0, or are left
// alone when accumulating.
__global__ __launch_bounds__(256) void score_kernel(const ScoreArgs a) {
  __shared__ float s_m[16], s_rl[16];
  const int unit = int(blockIdx.x) / a.chunks;  // b * h_kv + kvh
  const int chunk = int(blockIdx.x) - unit * a.chunks;
  const int b = unit / a.h_kv;
  const int64_t row0 = int64_t(unit) * a.group;  // first query row of the KV head
  if (int(threadIdx.x) < a.group) {
    const float l = a.row_stats[(row0 + threadIdx.x) * 2 + 1];
    s_m[threadIdx.x] = a.row_stats[(row0 + threadIdx.x) * 2 + 0];
    s_rl[threadIdx.x] = l > 0.f ? 1.f / l : 0.f;
  }
  __syncthreads();
  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  int sink_end = 0, win_start = 0;
  if (a.window > 0) {
    sink_end = min(a.num_sinks, ctx);
    win_start = max(ctx - a.window, 0);
  }
  float* dst = a.scores + int64_t(unit) * a.scores_ld;
  const int end = int(min(int64_t(chunk + 1) * kScoreChunk, a.scores_ld));
  for (int t = chunk * kScoreChunk + int(threadIdx.x); t < end; t += 256) {
    const bool attended = t < ctx && (t < sink_end || t >= win_start);
    if (!attended) {
      if (a.accumulate == 0) dst[t] = 0.f;
      continue;
    }
    float w = 0.f;
    for (int j = 0; j < a.group; ++j)
      w = fmaf(exp2_fast(a.logits[(row0 + j) * a.logits_ld + t] - s_m[j]), s_rl[j], w);
    dst[t] = a.accumulate != 0 ? dst[t] + w : w;
  }
}

// Append: one thread per 16-byte piece of a new K (and V) row. The destination follows the
// block-table translation of the new token's logical position, exactly as the split kernel reads
// it back; negative positions (idle sequences) and positions at or past the capacity are skipped.
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  const int idx = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (idx >= a.total) return;
  const int chunk = idx % a.row_chunks;
  const int row = idx / a.row_chunks;  // (b * rows_per_seq + i) * h_kv + kvh
  const int kvh = row % a.h_kv;
  const int token = row / a.h_kv;
  const int b = token / a.rows_per_seq;
  const int i = token - b * a.rows_per_seq;
  const int first = a.positions[b] + a.pos_offset;  // < 0: this sequence appends nothing
  if (first < 0) return;
  const int pos = first + i;
  if (pos < 0 || pos >= a.limit) return;
  int64_t blk, slot;
  if (a.block_table != nullptr) {
    blk = a.block_table[int64_t(b) * a.max_blocks + (pos >> a.bs_log2)];
    slot = pos & ((1 << a.bs_log2) - 1);
  } else {
    blk = b;
    slot = pos;
  }
  const int64_t src = (int64_t(row) * a.row_chunks + chunk) * 16;
  const int64_t kdst = (blk * a.k_sb + slot * a.k_st + int64_t(kvh) * a.k_sh) * a.elem_bytes + chunk * 16;
  const int64_t vdst = (blk * a.v_sb + slot * a.v_st + int64_t(kvh) * a.v_sh) * a.elem_bytes + chunk * 16;
  const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(a.k_new) + src);
  const u32x4_t vx = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(a.v_new) + src);
  *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(a.k) + kdst) = kx;
  *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(a.v) + vdst) = vx;
}

// Exclusive prefix sums of in[0..n) (n <= 256, in[n - 1 - i] when reverse) into out[0..n), by
// one wave (lane l takes entries 4l .. 4l+3); returns the total. Called by wave 0 alone.
__device__ unsigned int wave_scan256(const unsigned int* in, unsigned int* out, int n, bool reverse) {
  const int lane = int(threadIdx.x & 63);
  unsigned int x[4], sum = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * lane + i;
    x[i] = idx < n ? in[reverse ? n - 1 - idx : idx] : 0u;
    sum += x[i];
  }
  unsigned int inc = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  unsigned int run = inc - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * lane + i;
    if (idx < n) out[idx] = run;
    run += x[i];
  }
  return __shfl(inc, 63);
}

// The (sequence, split) pairs longest first, each listed with its sequence's clamped length:
// every whole split (split by split), then each sequence's last partial split by decreasing
// length (in 256 length classes), then -1 for each empty pair (its workgroups leave after one
// load). Every non-empty pair appears exactly once
// whatever the order within a class (positions within a class are taken with LDS atomics).
// One workgroup.
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const OrderArgs a) {
  __shared__ unsigned int s_full[kOrderMaxSplits + 1];    // sequences with exactly v whole splits
  __shared__ unsigned int s_efirst[kOrderMaxSplits + 1];  // sequences whose first empty split is v
  __shared__ unsigned int s_part[kOrderBuckets];          // partial splits per length class
  __shared__ unsigned int s_tmp[2][kOrderMaxSplits], s_cnt[2][kOrderMaxSplits];
  __shared__ unsigned int s_off_full[kOrderMaxSplits], s_off_empty[kOrderMaxSplits];
  __shared__ unsigned int s_off_part[kOrderBuckets];
  __shared__ unsigned int s_n_full, s_n_part;
  const int S = a.num_splits;
  const int st = a.split_tiles;
  const int t = int(threadIdx.x);
  auto clamp_len = [&](int ctx) { return ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx); };
  // Visited tiles of a sequence of length ctx, as the split kernel counts them.
  auto tiles_of = [&](int ctx) {
    ctx = clamp_len(ctx);
    int n_first = 0, win_tile0 = 0;
    if (a.window > 0) {
      const int sink_end = min(a.num_sinks, ctx);
      const int win_start = max(ctx - (a.num_queries - 1) - a.window, 0);
      n_first = (sink_end + kTile - 1) / kTile;
      win_tile0 = max(win_start / kTile, n_first);
    }
    return n_first + max((ctx + kTile - 1) / kTile - win_tile0, 0);
  };
  // This thread's first sequence is loaded before anything else and its tile count kept.
  const int ctx0 = t < a.batch ? a.ctx_lens[t] : 0;
  for (int i = t; i <= kOrderMaxSplits; i += kOrderThreads) {
    s_full[i] = 0u;
    s_efirst[i] = 0u;
  }
  for (int i = t; i < kOrderBuckets; i += kOrderThreads) s_part[i] = 0u;
  __syncthreads();
  const int nt0 = tiles_of(ctx0);
  auto class_of = [&](int len) { return int((int64_t(len) * kOrderBuckets - 1) / st); };  // 1..st-1 -> 0..255
  for (int b = t; b < a.batch; b += kOrderThreads) {
    const int nt = b == t ? nt0 : tiles_of(a.ctx_lens[b]);
    const int nf = min(nt / st, S);
    const int hp = nf < S && nt > nf * st ? 1 : 0;
    atomicAdd(&s_full[nf], 1u);
    if (hp) atomicAdd(&s_part[class_of(nt - nf * st)], 1u);
    atomicAdd(&s_efirst[nf + hp], 1u);
  }
  __syncthreads();
  // Offsets of the three classes, one wave each (their bases are added where they are used).
  const int wave = t >> 6;
  const int lane = t & 63;
  if (wave == 0) {  // whole splits: split s has B - #{nf <= s} of them
    wave_scan256(s_full, s_tmp[0], S, false);
    for (int s = lane; s < S; s += 64) s_cnt[0][s] = unsigned(a.batch) - s_tmp[0][s] - s_full[s];
    const unsigned int n = wave_scan256(s_cnt[0], s_off_full, S, false);
    if (lane == 0) s_n_full = n;
  } else if (wave == 1) {  // partial splits, longest class first
    const unsigned int n = wave_scan256(s_part, s_off_part, kOrderBuckets, true);
    if (lane == 0) s_n_part = n;
  } else if (wave == 2) {  // empty splits: split s is empty for #{first empty split <= s} sequences
    wave_scan256(s_efirst, s_tmp[1], S, false);
    for (int s = lane; s < S; s += 64) s_cnt[1][s] = s_tmp[1][s] + s_efirst[s];
    wave_scan256(s_cnt[1], s_off_empty, S, false);
  }
  __syncthreads();
  const unsigned int base_part = s_n_full;
  const unsigned int base_empty = s_n_full + s_n_part;
  int2* list = reinterpret_cast<int2*>(a.order);
  for (int b = t; b < a.batch; b += kOrderThreads) {
    const int len = clamp_len(b == t ? ctx0 : a.ctx_lens[b]);
    const int nt = b == t ? nt0 : tiles_of(len);
    const int nf = min(nt / st, S);
    const int hp = nf < S && nt > nf * st ? 1 : 0;
    const int32_t item0 = b * S;
    for (int s = 0; s < nf; ++s) list[atomicAdd(&s_off_full[s], 1u)] = int2{item0 + s, len};
    if (hp) {
      // s_off_part holds the classes in reverse: class c at index kOrderBuckets - 1 - c
      const int c = class_of(nt - nf * st);
      list[base_part + atomicAdd(&s_off_part[kOrderBuckets - 1 - c], 1u)] = int2{item0 + nf, len};
    }
    for (int s = nf + hp; s < S; ++s) list[base_empty + atomicAdd(&s_off_empty[s], 1u)] = int2{-1, 0};  // nothing to do
  }
}

}  // namespace

int launch_order(const OrderArgs& a, void* stream) {
  if (a.num_splits < 1 || a.num_splits > kOrderMaxSplits || a.split_tiles < 1) return int(hipErrorInvalidValue);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, s, a);
  return int(hipGetLastError());
}

int launch_split(const SplitArgs& a, const Plan& plan, int head_dim, bool paged, bool q_bf16,
                 bool kv_bf16, void* stream) {
  if (head_dim != 64 && head_dim != 128) return int(hipErrorInvalidValue);
  if (plan.variant == 2) return launch_split_rows(a, plan, head_dim, paged, stream);
  if (plan.variant == 1)
    return head_dim == 64 ? launch_split_mfma_d64(a, plan, paged, stream)
                          : launch_split_mfma_d128(a, plan, paged, stream);
  return head_dim == 64 ? launch_split_vector_d64(a, plan, q_bf16, kv_bf16, stream)
                        : launch_split_vector_d128(a, plan, q_bf16, kv_bf16, stream);
}

int launch_append(const AppendArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.total <= 0) return 0;
  const uint32_t grid = uint32_t((int64_t(a.total) + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(256), 0, s, a);
  return int(hipGetLastError());
}

int launch_scores(const ScoreArgs& a, int64_t units, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t grid = units * a.chunks;
  if (grid <= 0) return 0;
  hipLaunchKernelGGL(score_kernel, dim3(uint32_t(grid)), dim3(256), 0, s, a);
  return int(hipGetLastError());
}

int launch_merge(const MergeArgs& a, int head_dim, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.num_splits > kMaxSplits) return int(hipErrorInvalidValue);
  const uint32_t grid = uint32_t(a.rows);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kMergeThreads), 0, s, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kMergeThreads), 0, s, a);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace kvattn
