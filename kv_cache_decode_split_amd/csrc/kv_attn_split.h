// The split (streaming) kernel of split-KV decode attention for gfx950 (CDNA4, wave64): a
// template over head dim, group width, dtypes, data path and cache layout. Each
// kv_attn_split_*.hip file instantiates one family of it (so the families compile in
// parallel); kv_attn_kernels.hip holds the merge, score and append kernels and the dispatch.
//
// What is computed (Ch. 19 "Inference Systems and Performance Engineering" §19.4.1): for one
// new query token per sequence, out = softmax(scale * q . K^T) . V over the sequence's cached
// positions. The score row is never materialised: positions stream through in tiles and a
// running state (m, l, O) is updated per tile with the online-softmax recurrence of §19.6.2
// (new max, rescale factor c = 2^(m_old - m_new) applied to l and O, then the tile's
// exponentials added), as in the tiled forward pass of §19.6.3 specialised to one query row.
// Scores are kept in base-2 units (scale * log2 e folded in) so every exponential is a single
// v_exp_f32; the base cancels between numerator and denominator.
//
// Work decomposition. One workgroup (4 waves) per (sequence b, KV head, split). A split is a
// run of 16-position tiles; wave w streams tiles w, w+4, w+8, ... of the split with its own
// running state, so no barrier is needed inside the streaming loop. At the end the four wave
// states are merged through LDS (the same rescale-and-add step applied to whole states) and
// either the normalised output (one split) or the split's (m, l, O) goes to global memory; a
// second kernel merges splits. Every KV element of the group's KV head is loaded once and used
// by all g query heads that share it (the unique-KV reuse Ch. 10 §4 assumes for GQA).
//
// Per-tile data paths:
//  * bf16 q and KV (variant 1): scores come from the matrix cores. With A = the tile's 16 key
//    rows and B = the group's query rows (zero-padded to 16 heads), a 16x16x32 bf16 MFMA chain
//    over d produces S[token][head]; bf16 products are exact and accumulate in fp32.
//  * any other dtype mix (variant 0): each row of 16 lanes holds one key row, each lane a
//    d/16-element slice; partial dots are summed across the row with DPP.
//  * Both variants accumulate P.V in fp32 on the vector ALUs: lane (r, q4) owns elements
//    [r*d/16, (r+1)*d/16) of the value rows 4*q4 .. 4*q4+3 of the tile, and takes the
//    probabilities it needs by DPP row broadcast (variant 1) or directly (variant 0).
//  * rows mode (variant 2: several query tokens per sequence, or one token with a bf16 group
//    of 4 or more heads): up to 32 query rows per KV head in one or two blocks of 16 MFMA
//    columns; scores as in variant 1, and P.V on the matrix cores as well (see compute_rows).
//
// Loads are 64- to 128-bit per lane; the tile's key rows are 16 contiguous 64-byte pieces per
// instruction (MFMA operand layout), value rows are whole 256-byte rows per 16 lanes. Tiles
// are double-buffered in registers so the next tile's loads are in flight while the current
// one is computed (two-block rows mode keeps one tile in flight, to fit two waves per SIMD).
// Positions that are not attended are never read: their row index is redirected to an attended
// row of the same tile and the score is masked to -inf.
#ifndef KV_ATTN_SPLIT_H_
#define KV_ATTN_SPLIT_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kv_attn_internal.h"

namespace kvattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDepth = 2;  // tiles in flight per wave
// Rows mode with two blocks of query rows keeps one tile in flight per wave: its accumulators
// and query operand leave room for only one wave per SIMD with two tiles in flight, and two
// waves per SIMD with one tile each stream faster (C5 with 4 query tokens: 365 vs 400 us).
constexpr int kRows2Depth = 1;
constexpr int kBufferRsrcWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;      // rotate right by 4 within a row of 16 lanes
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowNewBcast0 = 0x150; // row_newbcast:n, lane n of each row to the whole row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a row; every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppRowRor8>(x);
  return x;
}

// Value of lane J of this lane's row.
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp<kDppRowNewBcast0 + J>(x);
}

__device__ __forceinline__ float lane_xor(float x, int mask) { return __shfl_xor(x, mask); }

// Combine each lane's value with lane ^ 16 (rows 0<->1, 2<->3) or lane ^ 32 (rows 0<->2,
// 1<->3) through the gfx950 row-swap permutes; both lanes of a pair compute the same
// expression in the same operand order, so they end with bit-identical results.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One 128-bit load of streamed (read-once) cache data.
__device__ __forceinline__ u32x4_t load_stream16(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Raw per-lane slice of one row: BYTES = 8, 16 or 32.
template <int BYTES>
struct Seg {
  uint32_t w[BYTES / 4];
};

template <int BYTES>
__device__ __forceinline__ Seg<BYTES> load_seg(const char* p) {
  Seg<BYTES> s;
  if constexpr (BYTES == 8) {
    const u32x2_t x = *reinterpret_cast<const u32x2_t*>(p);
    s.w[0] = x[0];
    s.w[1] = x[1];
  } else {
    static_for<0, BYTES / 16>([&](auto I) __attribute__((always_inline)) {
      const u32x4_t x = load_stream16(p + 16 * I());
      s.w[4 * I() + 0] = x[0];
      s.w[4 * I() + 1] = x[1];
      s.w[4 * I() + 2] = x[2];
      s.w[4 * I() + 3] = x[3];
    });
  }
  return s;
}

template <int BYTES>
__device__ __forceinline__ void store_seg(char* p, const Seg<BYTES>& s) {
  if constexpr (BYTES == 8) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{s.w[0], s.w[1]};
  } else {
    static_for<0, BYTES / 16>([&](auto I) __attribute__((always_inline)) {
      *reinterpret_cast<u32x4_t*>(p + 16 * I()) =
          u32x4_t{s.w[4 * I() + 0], s.w[4 * I() + 1], s.w[4 * I() + 2], s.w[4 * I() + 3]};
    });
  }
}

// Exact widening of N stored elements to fp32 (bf16: the 16 bits become the high half).
template <int N, bool BF16, int BYTES>
__device__ __forceinline__ void widen(const Seg<BYTES>& s, float (&f)[N]) {
  if constexpr (BF16) {
    static_assert(BYTES * 8 == N * 16, "segment size");
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      f[2 * i] = __uint_as_float(s.w[i] << 16);
      f[2 * i + 1] = __uint_as_float(s.w[i] & 0xffff0000u);
    }
  } else {
    static_assert(BYTES == N * 4, "segment size");
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = __uint_as_float(s.w[i]);
  }
}

// PAGED: 0 contiguous, 1 paged, 2 decided at run time.
// R = 0: one query token per sequence (G = compiled group width). R > 0 ("rows" mode, variant 2:
// several query tokens per sequence, or one token with a bf16 group of 4 or more heads):
// num_queries tokens per sequence, the group's query rows (token-major, then head) packed into R
// blocks of 16 MFMA columns; scores and P.V both on the matrix cores (G unused).
// SCORES: score export (one query token): every visited position's base-2 score goes to
// a.logits and, with one split, each row's final (m, l) to a.row_stats. A separate
// instantiation, so that the kernels without it keep their register allocation.
template <int D, int G, bool Q_BF16, bool KV_BF16, bool MFMA, int PAGED, int R = 0,
          bool SCORES = false, bool APPEND = false>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(const SplitArgs a) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(!MFMA || (Q_BF16 && KV_BF16), "matrix-core scores need bf16 q and KV");
  static_assert(!APPEND || (MFMA && !SCORES), "the fused append serves the matrix-core variants");
  static_assert(R == 0 || MFMA, "rows mode runs on the matrix cores");
  static_assert(!(SCORES && R > 1), "score export takes one query token per sequence");
  constexpr bool ROWS = R > 0;
  constexpr int NR = ROWS ? 16 * R : G;       // query rows held per (sequence, KV head)
  constexpr int EPL = D / 16;                 // elements per lane of a 16-lane row
  constexpr int KVB = KV_BF16 ? 2 : 4;        // bytes per KV element
  constexpr int QB = Q_BF16 ? 2 : 4;
  constexpr int SEG = EPL * KVB;              // bytes per lane per row
  constexpr int KC = D / 32;                  // MFMA k-chunks (32 bf16 each)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int q4 = lane >> 4;

  // Workgroups are dealt to the eight XCDs round-robin by index. With the split index slowest,
  // consecutive indices are different (sequence, KV head) units of the same split, so every
  // XCD receives the same mix of early (always full) and late (often empty) splits; with the
  // split index fastest, XCD k would get split k of every unit and ragged batches would load
  // the XCDs very unevenly. Within a split the KV head is rotated by the split index: when
  // h_kv is a multiple of 8, XCD k would otherwise see only KV heads k, k+8, ..., and with a
  // head-major paged cache whose blocks a sequence holds in physical order each XCD would read
  // the same few 4 KiB slices of every block (measured on MI355X: 0.67 of peak instead of 0.79).
  //
  // A token-major cache ([.., position, KV head, d]) interleaves the KV heads' rows of every
  // position. Workgroups that each stream one KV head then read 1 / h_kv of every position's
  // row, and as they drift apart over a split the rows of a position are fetched at scattered
  // times (measured on MI355X, loads only: 0.79-0.84 of peak against 0.86 head-major). With
  // wave_heads a workgroup serves kWaves KV heads of one split instead, wave w taking KV head
  // kvh0 + w and every tile of the split, so the rows of each position are read together
  // (0.87 in the same measurement); each wave's state is then a split state of its own.
  const int S = a.num_splits;
  const int units = int(gridDim.x) / S;
  const int hcn = a.head_chunks;
  const bool wave_heads = a.wave_heads != 0;
  const int hpu = wave_heads ? kWaves : 1;      // KV heads per workgroup
  const int units_b = a.h_kv / hpu;             // workgroups per (sequence, split)
  int split, hc, b, kvh0;
  int ctx_listed = 0;  // unit order: the pair's clamped length, listed with it
  if (a.order != nullptr) {
    // Unit order (head_chunks == 1): the (sequence, split) pairs come longest first from the
    // order list, each served by units_b consecutive workgroups (so by every XCD when units_b is
    // 8 or more), the empty pairs last as -1; the KV head is rotated by the split index as below.
    const int2 entry = reinterpret_cast<const int2*>(a.order)[blockIdx.x / units_b];
    const int item = entry.x;
    if (item < 0) return;  // an empty pair (S > 1: its split state is never read)
    ctx_listed = entry.y;
    b = item / S;
    split = item - b * S;
    hc = 0;
    kvh0 = ((int(blockIdx.x % units_b) + split) % units_b) * hpu;
  } else {
    split = blockIdx.x / units;
    const int unit = blockIdx.x - split * units;
    // With head chunks (vector path, groups above G heads) consecutive units are the chunks of
    // one (sequence, KV head): chunk hc serves query heads h0 .. h0 + g - 1 of the group.
    hc = unit % hcn;
    const int unit_kv = unit / hcn;
    // The XCD of a workgroup is fixed by its index modulo 8. With fewer than 8 workgroups per
    // (sequence, split) (wave heads, or h_kv < 8) every split of a sequence would land on the
    // XCDs of the same residues and a ragged batch would load the XCDs unevenly, so unit u of
    // split s then serves unit (u + s * units_b) mod (units per split): the sequence index
    // advances by one per split. MI355X, C4's ragged lengths, split kernel: h_kv = 4 / 2 / 1
    // 0.759 / 0.685 / 0.595 -> 0.779 / 0.723 / 0.612 of peak, C4 with wave heads 0.69 -> 0.74.
    // (With 8 or more per split every XCD already serves every sequence; there the shift cost
    // C3 0.7 %.)
    const int units_kv = units / hcn;
    const int ukv = units_b < 8 ? int((int64_t(unit_kv) + int64_t(split) * units_b) % units_kv) : unit_kv;
    b = ukv / units_b;
    kvh0 = ((ukv - b * units_b + split) % units_b) * hpu;
  }
  const int kvh = kvh0 + (wave_heads ? wave : 0);  // this wave's KV head
  const int h0 = hc * G;
  const int g = hcn > 1 ? min(G, a.group - h0) : a.group;  // query heads this workgroup serves
  const bool paged = PAGED == 2 ? (a.block_table != nullptr) : (PAGED == 1);

  int ctx = a.order != nullptr ? ctx_listed : a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int nq = ROWS ? a.num_queries : 1;  // query tokens per sequence (the last nq positions)
  // Fused append: the nq new tokens' K/V rows sit at positions new0 .. ctx - 1 (none when
  // ctx < nq). The tile that holds them takes those rows from k_new / v_new instead of the cache
  // and writes them into the cache (no other workgroup reads them in this launch).
  const int new0 = (APPEND && ctx >= nq) ? ctx - nq : -1;
  // Attended positions: all of [0, ctx), or with a window W the sinks [0, sink_end) and the
  // recent positions [win_start, ctx) (with nq query tokens, the union of their windows). Their
  // tiles are enumerated as "visited" tiles: the n_first tiles of the sink range, then the tiles
  // from win_tile0 to the last tile (a tile is never visited twice when the two ranges meet).
  // Without a window sink_end = win_start = 0.
  int sink_end = 0, win_start = 0, n_first = 0, win_tile0 = 0;
  if (a.window > 0) {
    sink_end = min(a.num_sinks, ctx);
    win_start = max(ctx - (nq - 1) - a.window, 0);
    n_first = (sink_end + kTile - 1) / kTile;
    win_tile0 = max(win_start / kTile, n_first);
  }
  const int ntiles = n_first + max((ctx + kTile - 1) / kTile - win_tile0, 0);
  const int t_begin = split * a.split_tiles;
  const int rows = nq * g;  // query rows of this (sequence, KV head): token-major, then head
  // Global row of query row rho of KV head kv: token rho / g of sequence b, head kv * g + rho % g.
  auto out_row_of = [&](int kv, int rho) __attribute__((always_inline)) {
    if constexpr (ROWS)
      return (int64_t(b) * nq + rho / g) * a.h_q + int64_t(kv) * g + rho % g;
    else
      return int64_t(b) * a.h_q + int64_t(kv) * a.group + h0 + rho;
  };
  auto out_row = [&](int rho) __attribute__((always_inline)) { return out_row_of(kvh, rho); };
  if (t_begin >= ntiles) {
    // Only an empty sequence reaches here with one split: its rows are defined as zeros.
    if (S == 1) {
      for (int idx = threadIdx.x; idx < hpu * rows * D; idx += kSplitThreads) {
        const int r = idx / D;
        a.out[out_row_of(kvh0 + r / rows, r % rows) * D + idx % D] = 0.f;
      }
      if (SCORES && a.row_stats != nullptr && threadIdx.x < hpu * rows) {
        const int64_t row = out_row_of(kvh0 + threadIdx.x / rows, threadIdx.x % rows);
        a.row_stats[row * 2 + 0] = neg_inf();
        a.row_stats[row * 2 + 1] = 0.f;
      }
    }
    return;
  }
  const int t_end = min(t_begin + a.split_tiles, ntiles);
  const int wstride = wave_heads ? 1 : kWaves;  // tiles between this wave's consecutive tiles
  const int woff = wave_heads ? 0 : wave;
  const int first = t_begin + woff;                                   // this wave's first tile
  const int n_w = first < t_end ? (t_end - first + wstride - 1) / wstride : 0;
  // Tile k of this wave is tile (woff + wstride*k + rot) mod span of the split. The splits of a
  // sequence all start at once; in a paged cache whose blocks a sequence holds in physical order
  // they would then read addresses a fixed power-of-two stride apart at every step and crowd the
  // same memory channels. A split-dependent start (an odd multiple of the split index) breaks
  // that alignment: C5 with blocks in physical order 0.75 -> 0.80 of peak on MI355X, random
  // order and contiguous caches unchanged. The visiting order inside a split only changes the
  // rounding of the running state.
  const int span = t_end - t_begin;
  // Fused append: the split whose last visited tile holds new rows keeps its tiles in order, so
  // the tiles with new rows are the last ones each wave visits.
  const int last_tile = t_end - 1 < n_first ? t_end - 1 : win_tile0 + (t_end - 1 - n_first);
  const bool split_has_new = APPEND && new0 >= 0 && span > 0 && (last_tile + 1) * kTile > new0;
  const int rot = span > 0 && !split_has_new ? int((int64_t(split) * 61) % span) : 0;
  auto visit = [&](int k) __attribute__((always_inline)) {
    int j = woff + wstride * k + rot;
    if (j >= span) j -= span;
    return t_begin + j;
  };

  // ---- query rows, loaded once ------------------------------------------------------------
  constexpr int RB = ROWS ? R : 1;
  // Tiles in flight. The vector path with fp32 KV, 8 heads and d = 128 holds 64 query and 64
  // output registers per lane besides 64 per tile in flight; with two tiles in flight it no
  // longer fits the register file, so it keeps one.
  constexpr int DEPTH = (ROWS && R == 2) ? kRows2Depth : (!MFMA && !KV_BF16 && G * EPL >= 64) ? 1 : kDepth;
  bf16x8_t qb[RB][KC];  // MFMA B operand of block cb: query row 16*cb + r16, elements c*32 + q4*8 .. +8
  float qf[G][EPL];     // vector path: every head, elements r16*EPL .. +EPL
  if constexpr (MFMA) {
    const char* qbase = reinterpret_cast<const char*>(a.q);
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
      const int rho = 16 * cb + r16;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (rho < rows)
          x = *reinterpret_cast<const u32x4_t*>(qbase + (out_row(rho) * D + c * 32 + q4 * 8) * 2);
        qb[cb][c] = __builtin_bit_cast(bf16x8_t, x);
      }
    }
  } else {
    const char* qbase = reinterpret_cast<const char*>(a.q);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (j < g) {
        const Seg<EPL * QB> s = load_seg<EPL * QB>(qbase + (out_row(j) * D + r16 * EPL) * QB);
        widen<EPL, Q_BF16>(s, qf[j]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[j][e] = 0.f;
      }
    }
  }

  // ---- running state -------------------------------------------------------------------------
  // Variant 1: m_run / l_run belong to head r16 (l_run summed over this lane's 4 positions).
  // Variant 0: per head arrays, uniform across the wave (m) or across the row (l).
  float m_run = neg_inf(), l_run = 0.f;
  float m_v[G], l_v[G];
  float O[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_v[j] = neg_inf();
    l_v[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[j][e] = 0.f;
  }
  // Rows mode: per block cb, this lane's query row rho = 16*cb + r16 keeps (m, l) and the
  // transposed output block O^T[d][rho] of 4*EPL elements (d = EPL*(4*q4 + r) + dc, held in
  // oT[cb][dc][r]). Token j = rho / g sees positions below lim = ctx - nq + 1 + j; with a window,
  // those below the sinks or at or past lim - W. Padding rows see nothing.
  float m_r[RB], l_r[RB];
  f32x4_t oT[RB][EPL];
  int lim[RB], wst[RB];
  const int snk = a.window > 0 ? a.num_sinks : 0;
#pragma unroll
  for (int cb = 0; cb < RB; ++cb) {
    m_r[cb] = neg_inf();
    l_r[cb] = 0.f;
#pragma unroll
    for (int dc = 0; dc < EPL; ++dc) oT[cb][dc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int rho = 16 * cb + r16;
    lim[cb] = rho < rows ? ctx - nq + 1 + rho / g : -1;
    wst[cb] = a.window > 0 ? lim[cb] - a.window : -1;
  }

  // ---- tile addressing -------------------------------------------------------------------------
  // A tile's rows sit at a uniform base (scalar arithmetic) plus per-lane 32-bit byte offsets
  // that are the same for every tile whose 16 positions are all attended. A partial tile (the
  // sequence's last tile, or a tile at an edge of the sink or window range) recomputes them
  // with every unattended row redirected to an attended row of the same tile, so no lane ever
  // addresses a position that is not attended (such rows are masked out of the scores).
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int64_t k_head = int64_t(kvh) * a.k_sh;
  const int64_t v_head = int64_t(kvh) * a.v_sh;
  struct LaneOffsets {
    int k;        // variant 1: key row r16, elements q4*8 (the first 32-element chunk)
    int kr[4];    // variant 0: key rows 4*q4+i, elements r16*EPL
    int v[4];     // value rows 4*q4+i, elements r16*EPL
  };
  // Tile row m (position p0 + m) is attended iff it lies below ctx and is a sink or in the window.
  auto attended_at = [&](int p0, int m) __attribute__((always_inline)) {
    const int pos = p0 + m;
    return pos < ctx && (pos < sink_end || pos >= win_start);
  };
  // row_of(m) is the row a lane loads for tile row m.
  auto lane_offsets = [&](auto row_of) __attribute__((always_inline)) {
    LaneOffsets o;
    o.k = (row_of(r16) * int(a.k_st) + q4 * 8) * KVB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row_of(4 * q4 + i);
      o.kr[i] = (row * int(a.k_st) + r16 * EPL) * KVB;
      o.v[i] = (row * int(a.v_st) + r16 * EPL) * KVB;
    }
    return o;
  };
  const LaneOffsets full = lane_offsets([](int m) { return m; });

  auto logical_tile = [&](int vt) __attribute__((always_inline)) {
    return vt < n_first ? vt : win_tile0 + (vt - n_first);
  };

  // Paged caches: the block ids of this wave's tiles k0 .. k0+63 sit one per lane in bt_vec and
  // are read with a (scalar) lane read. Consuming the register right after it is loaded makes the
  // compiler wait for that load there, so the tile loads in the streaming loop never wait on it.
  int bt_vec = 0, bt_base = 0;
  auto fetch_block_ids = [&](int k0) __attribute__((always_inline)) {
    const int kk = k0 + lane;
    int blk = 0;
    if (kk < n_w)
      blk = a.block_table[int64_t(b) * a.max_blocks + ((logical_tile(visit(kk)) * kTile) >> a.bs_log2)];
    bt_vec = blk;
    bt_base = k0;
    asm volatile("" ::"v"(bt_vec));
  };

  struct Frag {
    u32x4_t kc[KC];      // variant 1: key row r16, 32-element chunks
    Seg<SEG> kr[4];      // variant 0: key rows 4*q4+i
    Seg<SEG> vr[4];      // value rows 4*q4+i
    const char* kt;      // fused append: the tile's K and V rows in the cache (row 0)
    const char* vt;
  };
  // Fused append: element offset of new row j (position new0 + j) of this KV head in k_new /
  // v_new ([B, nq, h_kv, D]).
  auto new_row = [&](int j) __attribute__((always_inline)) {
    return ((int64_t(b) * nq + j) * a.h_kv + kvh) * D;
  };

  // patch (fused append only, set for a wave's last tiles): the tile may hold new rows.
  auto load_tile = [&](int k, Frag& f, auto patch) __attribute__((always_inline)) {
    const int tile = logical_tile(visit(k));
    const int p0 = tile * kTile;
    int64_t koff, voff;             // element offset of tile row 0
    if (paged) {
      if (k - bt_base >= 64) fetch_block_ids(k & ~63);
      const int blk = __builtin_amdgcn_readlane(bt_vec, k - bt_base);
      const int slot0 = p0 & ((1 << a.bs_log2) - 1);
      koff = int64_t(blk) * a.k_sb + int64_t(slot0) * a.k_st + k_head;
      voff = int64_t(blk) * a.v_sb + int64_t(slot0) * a.v_st + v_head;
    } else {
      koff = int64_t(b) * a.k_sb + int64_t(p0) * a.k_st + k_head;
      voff = int64_t(b) * a.v_sb + int64_t(p0) * a.v_st + v_head;
    }
    const char* kt = kbase + koff * KVB;
    const char* vt = vbase + voff * KVB;
    // Every visited tile holds at least one attended row: row 0 if it is a sink row, else the
    // first row at or past the window start.
    const bool whole = p0 + kTile <= ctx && (p0 + kTile <= sink_end || p0 >= win_start);
    const int anchor = p0 < sink_end ? 0 : max(win_start - p0, 0);
    const LaneOffsets o = whole ? full : lane_offsets([&](int m) __attribute__((always_inline)) {
      return attended_at(p0, m) ? m : anchor;
    });
    if constexpr (MFMA) {
#pragma unroll
      for (int c = 0; c < KC; ++c) f.kc[c] = load_stream16(kt + o.k + c * 64);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) f.kr[i] = load_seg<SEG>(kt + o.kr[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) f.vr[i] = load_seg<SEG>(vt + o.v[i]);
    if constexpr (APPEND && decltype(patch)::value) {
      f.kt = kt;
      f.vt = vt;
      if (new0 >= 0 && p0 + kTile > new0) {
        // Every row a lane loaded from a new position (its own row, or the attended row an
        // unattended one was redirected to) comes from k_new / v_new: the cache does not hold it
        // yet, and a value row must be finite even where its probability is 0.
        auto loaded = [&](int m) __attribute__((always_inline)) {
          return whole || attended_at(p0, m) ? m : anchor;
        };
        const char* kn = reinterpret_cast<const char*>(a.k_new);
        const char* vn = reinterpret_cast<const char*>(a.v_new);
        const int mk = loaded(r16);
        if (p0 + mk >= new0) {
#pragma unroll
          for (int c = 0; c < KC; ++c)
            f.kc[c] = *reinterpret_cast<const u32x4_t*>(kn + (new_row(p0 + mk - new0) + c * 32 + q4 * 8) * 2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mv = loaded(4 * q4 + i);
          if (p0 + mv >= new0) f.vr[i] = load_seg<SEG>(vn + (new_row(p0 + mv - new0) + r16 * EPL) * 2);
        }
      }
    }
  };
  // Fused append: the lanes holding an attended new row write it into the cache once its data
  // has arrived (at compute time, so that no earlier load in flight is waited for).
  auto store_new_rows = [&](const Frag& f, int p0) __attribute__((always_inline)) {
    if (new0 < 0 || p0 + kTile <= new0) return;
    char* kw = const_cast<char*>(f.kt);  // the caller's writable caches in append mode
    char* vw = const_cast<char*>(f.vt);
    if (p0 + r16 >= new0 && attended_at(p0, r16)) {
#pragma unroll
      for (int c = 0; c < KC; ++c) *reinterpret_cast<u32x4_t*>(kw + full.k + c * 64) = f.kc[c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (p0 + 4 * q4 + i >= new0 && attended_at(p0, 4 * q4 + i)) store_seg<SEG>(vw + full.v[i], f.vr[i]);
  };

  // Score export: the scores of positions pos .. pos+3 for query head j of this (sequence, KV
  // head) go to row b*h_q + kvh*g + j of a.logits ([B*h_q, logits_ld]). Every lane issues one
  // bounds-checked 16-byte buffer store, padding heads (j >= g) with an offset past the end that
  // the hardware drops: a branch around the stores would hide them from the wait counts on the
  // path that skips them, and the loads of the next tiles would then be waited for too early on
  // the path that takes them. (a.logits is null outside the score-export instantiations; the
  // descriptor is then unused.)
  const __amdgpu_buffer_rsrc_t score_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      SCORES ? a.logits + (int64_t(b) * a.h_q + int64_t(kvh) * a.group + h0) * a.logits_ld : a.logits, 0,
      SCORES ? int(a.logits_ld * g * 4) : 0, kBufferRsrcWord3);
  auto store_scores = [&](f32x4_t v, int pos, int j) __attribute__((always_inline)) {
    const uint32_t off = j < g ? uint32_t((int64_t(j) * a.logits_ld + pos) * 4) : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), score_rsrc, off, 0, 0);
  };

  auto compute_tile = [&](int k, const Frag& f) __attribute__((always_inline)) {
    const int p0 = logical_tile(visit(k)) * kTile;
    auto attended = [&](int m) __attribute__((always_inline)) { return attended_at(p0, m); };
    float p[4][G];                          // variant 0: probabilities of rows 4*q4+i
    float pm[4];                            // variant 1: probability of (row 4*q4+i, head r16)
    bool rescale;
    if constexpr (MFMA) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.kc[c]), qb[0][c],
                                                      acc, 0, 0, 0);
      // acc[r] = score of tile row 4*q4 + r for head r16.
      float s[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = attended(4 * q4 + r) ? acc[r] * a.scale_log2 : neg_inf();
      if constexpr (SCORES)  // score export: positions p0 + 4*q4 .. +3 of head r16
        store_scores(f32x4_t{s[0], s[1], s[2], s[3]}, p0 + 4 * q4, r16);
      float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mt = max_xor32(max_xor16(mt));
      const float m_new = fmaxf(m_run, mt);
      const float c = exp2_fast(m_run - m_new);  // 0 on the first tile (m_run = -inf)
#pragma unroll
      for (int r = 0; r < 4; ++r) pm[r] = exp2_fast(s[r] - m_new);
      l_run = c * l_run + ((pm[0] + pm[1]) + (pm[2] + pm[3]));
      m_run = m_new;
      rescale = __any(r16 < G && c != 1.0f);
      if (rescale) {
        static_for<0, G>([&](auto J) __attribute__((always_inline)) {
          const float cj = row_bcast<J()>(c);
#pragma unroll
          for (int e = 0; e < EPL; ++e) O[J()][e] *= cj;
        });
      }
    } else {
      float s[4][G];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float kf[EPL];
        widen<EPL, KV_BF16>(f.kr[i], kf);
        const bool valid = attended(4 * q4 + i);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float x = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) x = fmaf(qf[j][e], kf[e], x);
          x = row_sum16(x);
          s[i][j] = valid ? x * a.scale_log2 : neg_inf();
        }
      }
      if constexpr (SCORES) {  // score export: lane r16 writes head r16's four positions
        f32x4_t v = {s[0][0], s[1][0], s[2][0], s[3][0]};
        static_for<1, G>([&](auto J) __attribute__((always_inline)) {
          if (r16 == J()) v = f32x4_t{s[0][J()], s[1][J()], s[2][J()], s[3][J()]};
        });
        store_scores(v, p0 + 4 * q4, r16);
      }
      bool any_change = false;
      float cv[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float mt = fmaxf(fmaxf(s[0][j], s[1][j]), fmaxf(s[2][j], s[3][j]));
        mt = max_xor32(max_xor16(mt));
        const float m_new = fmaxf(m_v[j], mt);
        cv[j] = exp2_fast(m_v[j] - m_new);
        m_v[j] = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i][j] = exp2_fast(s[i][j] - m_new);
        l_v[j] = cv[j] * l_v[j] + ((p[0][j] + p[1][j]) + (p[2][j] + p[3][j]));
        any_change |= cv[j] != 1.0f;
      }
      rescale = __any(any_change);
      if (rescale) {
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int e = 0; e < EPL; ++e) O[j][e] *= cv[j];
      }
    }
    // P.V for value rows 4*q4 .. 4*q4+3, elements r16*EPL .. +EPL, every head of the group.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vf[EPL];
      widen<EPL, KV_BF16>(f.vr[i], vf);
      static_for<0, G>([&](auto J) __attribute__((always_inline)) {
        float pj;
        if constexpr (MFMA)
          pj = row_bcast<J()>(pm[i]);
        else
          pj = p[i][J()];
#pragma unroll
        for (int e = 0; e < EPL; ++e) O[J()][e] = fmaf(pj, vf[e], O[J()][e]);
      });
    }
  };

  // Rows mode: scores S^T[key][row] = K Q^T and O^T[d][row] += V^T P^T, both on the matrix cores.
  // The score MFMA leaves, in lane (q4, r16), the scores of keys 4*q4 .. 4*q4+3 for query row
  // r16 of the block. The bf16 operand cannot hold P to fp32 accuracy (a lone probability near 1
  // would carry up to 2^-8 relative error into the output), so P is split into p_hi = bf16(p) and
  // p_lo = bf16(p - p_hi) (together within 2^-16 relative of p; l keeps the fp32 probabilities),
  // and both halves go through one 16x16x32 MFMA: its 32 k-slots hold the tile's 16 keys twice.
  // Lane (q4, r16) supplies k-slots 8*q4 .. 8*q4+7, taken as keys 4*q4 + (e & 3) of half e >> 2:
  // B gets (p_hi, p_lo) of its four keys, exactly the values the score MFMA left in the lane,
  // and A = V^T gets the same four value rows twice. For A the d index of output row m of block
  // dc is taken as EPL*m + dc, so that lane (q4, r16) needs V[4*q4 + i][EPL*r16 + dc], i = 0..3:
  // elements it already loaded (value rows 4*q4+i, elements EPL*r16 ..), repacked with no data
  // exchange between lanes. (On MI355X one 16x16x32 MFMA issues in about 1.14 times the cycles
  // of a 16x16x16 one, which the two halves would otherwise need twice.)
  auto compute_rows = [&](int k, const Frag& f) __attribute__((always_inline)) {
    const int p0 = logical_tile(visit(k)) * kTile;
    // Most tiles are attended by every query row at all 16 positions (below the first token's
    // limit, and all sinks or all at or past the last token's window start): they skip the
    // per-row masks. (Padding rows then see real scores of their zero query; they are never
    // written out.)
    const bool open = p0 + kTile <= ctx - nq + 1 &&
                      (a.window <= 0 || p0 >= ctx - a.window || p0 + kTile <= snk);
    bf16x8_t vt[EPL];
#pragma unroll
    for (int dc = 0; dc < EPL; ++dc) {
      const int w = dc >> 1;
      uint32_t lo, hi;
      if (dc & 1) {
        lo = (f.vr[0].w[w] >> 16) | (f.vr[1].w[w] & 0xffff0000u);
        hi = (f.vr[2].w[w] >> 16) | (f.vr[3].w[w] & 0xffff0000u);
      } else {
        lo = (f.vr[0].w[w] & 0xffffu) | (f.vr[1].w[w] << 16);
        hi = (f.vr[2].w[w] & 0xffffu) | (f.vr[3].w[w] << 16);
      }
      vt[dc] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo, hi, lo, hi});
    }
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.kc[c]),
                                                      qb[cb][c], acc, 0, 0, 0);
      float sc[4];
      if (open) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = acc[r] * a.scale_log2;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = p0 + 4 * q4 + r;
          const bool valid = pos < lim[cb] && (pos < snk || pos >= wst[cb]);
          sc[r] = valid ? acc[r] * a.scale_log2 : neg_inf();
        }
      }
      // Score export (one token, one block: query row r16 is head r16): the same lane layout as
      // the one-token kernel's scores, positions p0 + 4*q4 .. +3.
      if constexpr (SCORES) store_scores(f32x4_t{sc[0], sc[1], sc[2], sc[3]}, p0 + 4 * q4, r16);
      float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mt = max_xor32(max_xor16(mt));
      const float m_new = fmaxf(m_r[cb], mt);
      // A row that has seen nothing yet keeps m = -inf; exponentials then use 0 in its place,
      // so they are 0 instead of NaN.
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      const float c = exp2_fast(m_r[cb] - m_use);
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(sc[r] - m_use);
      l_r[cb] = c * l_r[cb] + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m_r[cb] = m_new;
      if (__any(16 * cb + r16 < rows && c != 1.0f)) {
#pragma unroll
        for (int dc = 0; dc < EPL; ++dc) oT[cb][dc] *= c;
      }
      const f32x4_t pf = {pr[0], pr[1], pr[2], pr[3]};
      const bf16x4_t p_hi = __builtin_convertvector(pf, bf16x4_t);
      const f32x4_t hi_f = __builtin_convertvector(p_hi, f32x4_t);
      const bf16x4_t p_lo = __builtin_convertvector(
          f32x4_t{pf[0] - hi_f[0], pf[1] - hi_f[1], pf[2] - hi_f[2], pf[3] - hi_f[3]}, bf16x4_t);
      const bf16x8_t p_b = __builtin_shufflevector(p_hi, p_lo, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int dc = 0; dc < EPL; ++dc)
        oT[cb][dc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[dc], p_b, oT[cb][dc], 0, 0, 0);
    }
  };
  auto compute = [&](int k, const Frag& f, auto patch) __attribute__((always_inline)) {
    if constexpr (APPEND && decltype(patch)::value) store_new_rows(f, logical_tile(visit(k)) * kTile);
    if constexpr (ROWS)
      compute_rows(k, f);
    else
      compute_tile(k, f);
  };
  constexpr std::false_type kPlain{};
  constexpr std::bool_constant<APPEND> kPatch{};

  // ---- streaming loop: DEPTH tiles in flight --------------------------------------------------
  // The steady-state loop issues its loads unconditionally, so the compiler's wait counts let
  // the DEPTH tiles behind the one being computed stay in flight; the last tiles are drained
  // with conditional loads outside it. With the fused append a wave's last kTail tiles (where
  // the new rows can be: the split that holds them is not rotated) stay out of the steady loop,
  // so that its code and wait counts are those of the plain kernel.
  constexpr int kTail = APPEND ? 2 : 0;
  Frag buf[DEPTH];
  if (paged && n_w > 0) fetch_block_ids(0);
  int k0 = 0;
  if (n_w >= 2 * DEPTH + kTail) {
    static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) { load_tile(P(), buf[P()], kPlain); });
    do {
      static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
        compute(k0 + P(), buf[P()], kPlain);
        load_tile(k0 + P() + DEPTH, buf[P()], kPlain);
      });
      k0 += DEPTH;
    } while (k0 + 2 * DEPTH + kTail <= n_w);
    if constexpr (APPEND) {
      // Tiles k0 .. k0+DEPTH-1 are in flight; at most DEPTH-1+kTail more remain after them.
      for (; k0 < n_w; k0 += DEPTH) {
        static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
          const int k = k0 + P();
          if (k < n_w) {
            compute(k, buf[P()], kPatch);
            if (k + DEPTH < n_w) load_tile(k + DEPTH, buf[P()], kPatch);
          }
        });
      }
    } else {
      // Tiles k0 .. k0+DEPTH-1 are in flight; at most DEPTH-1 more remain after them.
      static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
        const int k = k0 + P();
        compute(k, buf[P()], kPlain);
        if (k + DEPTH < n_w) load_tile(k + DEPTH, buf[P()], kPlain);
      });
      static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
        const int k = k0 + DEPTH + P();
        if (k < n_w) compute(k, buf[P()], kPlain);
      });
    }
  } else if constexpr (APPEND) {
    static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
      if (P() < n_w) load_tile(P(), buf[P()], kPatch);
    });
    for (; k0 < n_w; k0 += DEPTH) {
      static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
        const int k = k0 + P();
        if (k < n_w) {
          compute(k, buf[P()], kPatch);
          if (k + DEPTH < n_w) load_tile(k + DEPTH, buf[P()], kPatch);
        }
      });
    }
  } else {
    static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
      if (P() < n_w) load_tile(P(), buf[P()], kPlain);
    });
    static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
      if (P() < n_w) {
        compute(P(), buf[P()], kPlain);
        if (P() + DEPTH < n_w) load_tile(P() + DEPTH, buf[P()], kPlain);
      }
    });
    static_for<0, DEPTH>([&](auto P) __attribute__((always_inline)) {
      if (DEPTH + P() < n_w) compute(DEPTH + P(), buf[P()], kPlain);
    });
  }

  // ---- merge the four wave states through LDS ---------------------------------------------------
  constexpr int DP = ROWS ? D + 4 : D;  // rows mode: padded rows spread its stores over the banks
  __shared__ float sm_m[kWaves][NR];
  __shared__ float sm_l[kWaves][NR];
  __shared__ float sm_o[kWaves][NR][DP];
  if constexpr (ROWS) {
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
      const float lt = sum_xor32(sum_xor16(l_r[cb]));
      const int rho = 16 * cb + r16;
      if (q4 == 0) {
        sm_m[wave][rho] = m_r[cb];
        sm_l[wave][rho] = lt;
      }
#pragma unroll
      for (int dc = 0; dc < EPL; ++dc)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm_o[wave][rho][EPL * (4 * q4 + r) + dc] = oT[cb][dc][r];
    }
  } else if constexpr (MFMA) {
    const float lt = sum_xor32(sum_xor16(l_run));
    if (q4 == 0 && r16 < G) {
      sm_m[wave][r16] = m_run;
      sm_l[wave][r16] = lt;
    }
  } else {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float lt = sum_xor32(sum_xor16(l_v[j]));
      if (lane == 0) {
        sm_m[wave][j] = m_v[j];
        sm_l[wave][j] = lt;
      }
    }
  }
  if constexpr (!ROWS) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) O[j][e] = sum_xor32(sum_xor16(O[j][e]));
    }
    if (q4 == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sm_o[wave][j][r16 * EPL + e] = O[j][e];
      }
    }
  }
  __syncthreads();
  if (wave_heads) {
    // Every wave's state is a split state of its own KV head, kvh0 + w.
    for (int idx = threadIdx.x; idx < kWaves * rows * D; idx += kSplitThreads) {
      const int r = idx / D;
      const int e = idx % D;
      const int w = r / rows;
      const int j = r - w * rows;
      const float M = sm_m[w][j];
      const bool seen = M != neg_inf();  // a row that saw no position: L = 0, output 0
      const float L = seen ? sm_l[w][j] : 0.f;
      const float acc = seen ? sm_o[w][j][e] : 0.f;
      const int64_t row = out_row_of(kvh0 + w, j);
      if (S == 1) {
        a.out[row * D + e] = L > 0.f ? acc / L : 0.f;
        if (SCORES && a.row_stats != nullptr && e == 0) {
          a.row_stats[row * 2 + 0] = M;
          a.row_stats[row * 2 + 1] = L;
        }
      } else {
        const int64_t slot = row * S + split;
        a.o_part[slot * D + e] = acc;
        if (e == 0) {
          a.ml_part[slot * 2 + 0] = M;
          a.ml_part[slot * 2 + 1] = L;
        }
      }
    }
    return;
  }
  for (int idx = threadIdx.x; idx < rows * D; idx += kSplitThreads) {
    const int j = idx / D;
    const int e = idx % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][j];
      const float ww = (mw == neg_inf()) ? 0.f : exp2_fast(mw - M);  // empty wave: weight 0
      L = fmaf(ww, sm_l[w][j], L);
      acc = fmaf(ww, sm_o[w][j][e], acc);
    }
    const int64_t row = out_row(j);
    if (S == 1) {
      a.out[row * D + e] = L > 0.f ? acc / L : 0.f;  // L = 0: a query token that sees nothing
      if (SCORES && a.row_stats != nullptr && e == 0) {
        a.row_stats[row * 2 + 0] = M;
        a.row_stats[row * 2 + 1] = L;
      }
    } else {
      const int64_t slot = row * S + split;
      a.o_part[slot * D + e] = acc;
      if (e == 0) {
        a.ml_part[slot * 2 + 0] = M;
        a.ml_part[slot * 2 + 1] = L;
      }
    }
  }
}

template <int D, int G, bool QB, bool KB, bool MF, int PG, int R = 0, bool SC = false, bool AP = false>
int launch_one(const SplitArgs& a, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((split_kernel<D, G, QB, KB, MF, PG, R, SC, AP>), dim3(uint32_t(grid)),
                     dim3(kSplitThreads), 0, stream, a);
  return int(hipGetLastError());
}

// Variant 1 (bf16 q and KV, matrix-core scores, VALU P.V), cache layout compiled in; with
// a.logits set, the score-export instantiation; with a.k_new set, the fused append.
template <int D, int G>
int launch_mfma_group(const SplitArgs& a, const Plan& plan, bool paged, hipStream_t s) {
  if (a.logits != nullptr)
    return paged ? launch_one<D, G, true, true, true, 1, 0, true>(a, plan.grid_split, s)
                 : launch_one<D, G, true, true, true, 0, 0, true>(a, plan.grid_split, s);
  if (a.k_new != nullptr) {
    // Variant 1 serves groups of at most 3 heads (rows mode takes 4 or more), so G <= 4.
    if constexpr (G <= kAppendMaxGroup)
      return paged ? launch_one<D, G, true, true, true, 1, 0, false, true>(a, plan.grid_split, s)
                   : launch_one<D, G, true, true, true, 0, 0, false, true>(a, plan.grid_split, s);
    return int(hipErrorInvalidValue);
  }
  return paged ? launch_one<D, G, true, true, true, 1>(a, plan.grid_split, s)
               : launch_one<D, G, true, true, true, 0>(a, plan.grid_split, s);
}

template <int D>
int launch_mfma(const SplitArgs& a, const Plan& plan, bool paged, hipStream_t s) {
  switch (plan.group_padded) {
    case 1: return launch_mfma_group<D, 1>(a, plan, paged, s);
    case 2: return launch_mfma_group<D, 2>(a, plan, paged, s);
    case 4: return launch_mfma_group<D, 4>(a, plan, paged, s);
    case 8: return launch_mfma_group<D, 8>(a, plan, paged, s);
    case 16: return launch_mfma_group<D, 16>(a, plan, paged, s);
    default: return int(hipErrorInvalidValue);
  }
}

// Variant 0 (the vector path: any dtype mix, layout decided at run time), at most
// kVectorMaxGroup heads per workgroup; score export for fp32 q and KV.
template <int D, int G>
int launch_vector_group(const SplitArgs& a, const Plan& plan, bool q_bf16, bool kv_bf16,
                        hipStream_t s) {
  if (a.logits != nullptr) {
    if (!q_bf16 && !kv_bf16) return launch_one<D, G, false, false, false, 2, 0, true>(a, plan.grid_split, s);
    return int(hipErrorInvalidValue);
  }
  if (q_bf16 && kv_bf16) return launch_one<D, G, true, true, false, 2>(a, plan.grid_split, s);
  if (q_bf16) return launch_one<D, G, true, false, false, 2>(a, plan.grid_split, s);
  if (kv_bf16) return launch_one<D, G, false, true, false, 2>(a, plan.grid_split, s);
  return launch_one<D, G, false, false, false, 2>(a, plan.grid_split, s);
}

template <int D>
int launch_vector(const SplitArgs& a, const Plan& plan, bool q_bf16, bool kv_bf16, hipStream_t s) {
  static_assert(kVectorMaxGroup == 8, "vector group widths");
  switch (plan.group_padded) {
    case 1: return launch_vector_group<D, 1>(a, plan, q_bf16, kv_bf16, s);
    case 2: return launch_vector_group<D, 2>(a, plan, q_bf16, kv_bf16, s);
    case 4: return launch_vector_group<D, 4>(a, plan, q_bf16, kv_bf16, s);
    case 8: return launch_vector_group<D, 8>(a, plan, q_bf16, kv_bf16, s);
    default: return int(hipErrorInvalidValue);  // the planner serves larger groups in head chunks
  }
}

// Rows mode (several query tokens per sequence, or one token with a group of 4 or more): bf16
// only, 1 or 2 blocks of 16 query rows; score export (one token) in one block.
template <int D>
int launch_rows(const SplitArgs& a, const Plan& plan, bool paged, hipStream_t s) {
  if (a.logits != nullptr) {
    if (plan.row_blocks != 1 || plan.num_queries != 1) return int(hipErrorInvalidValue);
    return paged ? launch_one<D, 1, true, true, true, 1, 1, true>(a, plan.grid_split, s)
                 : launch_one<D, 1, true, true, true, 0, 1, true>(a, plan.grid_split, s);
  }
  if (a.k_new != nullptr) {  // the fused append
    switch (plan.row_blocks) {
      case 1: return paged ? launch_one<D, 1, true, true, true, 1, 1, false, true>(a, plan.grid_split, s)
                           : launch_one<D, 1, true, true, true, 0, 1, false, true>(a, plan.grid_split, s);
      case 2: return paged ? launch_one<D, 1, true, true, true, 1, 2, false, true>(a, plan.grid_split, s)
                           : launch_one<D, 1, true, true, true, 0, 2, false, true>(a, plan.grid_split, s);
      default: return int(hipErrorInvalidValue);
    }
  }
  switch (plan.row_blocks) {
    case 1: return paged ? launch_one<D, 1, true, true, true, 1, 1>(a, plan.grid_split, s)
                         : launch_one<D, 1, true, true, true, 0, 1>(a, plan.grid_split, s);
    case 2: return paged ? launch_one<D, 1, true, true, true, 1, 2>(a, plan.grid_split, s)
                         : launch_one<D, 1, true, true, true, 0, 2>(a, plan.grid_split, s);
    default: return int(hipErrorInvalidValue);
  }
}

}  // namespace
}  // namespace kvattn

#endif  // KV_ATTN_SPLIT_H_
