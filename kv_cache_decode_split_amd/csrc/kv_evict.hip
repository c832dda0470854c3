// Budgeted KV eviction selection for gfx950 (see include/kv_evict.h for the contract).
//
// What is computed (Ch. 19 "Inference Systems and Performance Engineering" §19.4.3, the eviction
// exercise): the current position of every (layer, head) row stays; every other entry competes
// in one global pool ranked by (-score, layer, head, position); the first K = M - L*H stay.
//
// Each pool entry gets a 64-bit key whose unsigned order is the pool's ranking reversed: the
// high word is the score's bits made order-preserving (negative values complemented, the sign
// set on the others, -0.0 folded onto +0.0), the low word is the complement of the flat index
// i = (l*H + h)*N + t, so a lower index wins a tie. The K entries that stay are exactly those
// whose key is at least k*, the K-th largest key. The scores are streamed once; kernel
// boundaries are the only grid-wide synchronisation:
//
//   init    eight workgroups each histogram the top 13-bit digit of a sample of the scores
//           (chunks of 256 consecutive entries spread over the array; every entry when the pool
//           is small) and write their histogram out whole, so nothing needs clearing first; the
//           other workgroups clear the band histogram;
//   pass1   every workgroup reads the sample histograms and derives the same band of top digits:
//           the digits holding the sample ranks of k* minus and plus eight standard deviations
//           of a sampled quantile (the exact digit of k* when every entry was sampled), at most
//           16 digits wide. It then streams every entry: top digit above the band 1, below it 0,
//           inside it 0 for now, with the key copied into list 1 (each workgroup into its own
//           region, so no global counter is needed) and counted in a histogram of (band digit,
//           next 10 bits); it also counts the entries above the band exactly;
//   list    every workgroup finds k*'s rank among the band entries from those exact counts, and
//           from the band histogram the top 23 bits of k*; then walks its share of list 1:
//           entries above those bits get a 1, entries sharing them go to list 2;
//   final   one workgroup ranks list 2 (directly when it holds at most 1024 keys, else by digit
//           passes over the remaining 41 bits) and gives a 1 to its entries at or above k*, and
//           to every row's current position.
//
// The sample only places the band; the counts that fix k* are exact. If k* turns out to lie
// outside the band (a sample unlike the rest of the scores, or a band clipped to 16 digits), the
// list pass says so and the final workgroup computes the whole selection exactly by itself,
// digit by digit over every entry (correct for any input, slow on large pools).
//
// Histograms are built in LDS per workgroup and added into one of several global replicas with
// device-scope atomics, skipping bins that stayed zero, so few workgroups contend for one
// address. No kernel uses a device-scope fence or a grid-wide arrival counter: on this chip each
// costs tens of nanoseconds per workgroup, serialised.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "kv_attn_internal.h"
#include "kv_evict.h"

namespace kvevict {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 1024;                 // threads of every workgroup
constexpr int kVec = 4;                              // floats per 128-bit load
constexpr int kSlabs = 4;                            // loads per thread per iteration
constexpr int kChunk = kStreamThreads * kVec * kSlabs;  // entries per workgroup iteration
constexpr int kGrid = 256;                           // workgroups of the full pass (at most)
constexpr int kLdsKeys = 6144;                       // list-2 entries the final kernel stages
constexpr int kBins = 8192;                          // 13-bit digits
constexpr int kGroups = 64;                          // coarse bins: 128 consecutive digits each
constexpr int kGroupBins = kBins / kGroups;
// Group counters sit one 128-byte line apart: device-scope atomics from many workgroups to words
// of one line serialise (packed, the 64 counters of a replica made a full pass 2.2x slower).
constexpr int kGroupStride = 32;
constexpr int kRep = kBins + kGroups * kGroupStride; // words per replica: bins, then groups
// Sample: kSampleWGs workgroups of kSampleGroups groups of four entries per thread; chunks of
// kSampleRun consecutive entries, or every entry of an array of at most kSampleAll entries.
constexpr int kSampleWGs = 16;
constexpr int kSampleGroups = 2;
constexpr int kSampleRun = 256;
constexpr int kSampleChunksPerWG = kStreamThreads * 4 * kSampleGroups / kSampleRun;
constexpr int kSampleChunks = kSampleWGs * kSampleChunksPerWG;
constexpr int64_t kSampleAll = int64_t(kSampleWGs) * kStreamThreads * 4 * kSampleGroups;
// Band histogram: kBandDigits top digits x 2^kSubBits sub-digits (the next bits of the key).
constexpr int kBandDigits = 16;
constexpr int kSubBits = 10;
constexpr int kSubBins = 1 << kSubBits;
constexpr int kPrefixShift = 51 - kSubBits;          // the band prefix is key >> 41 (23 bits)
constexpr int kBandRep = kBandDigits * kSubBins + kBandDigits * kGroupStride;
constexpr int kBandReplicas = 4;
constexpr size_t kStateBytes = 256;
constexpr size_t kSampleBytes = size_t(kSampleWGs) * kRep * 4;
constexpr size_t kBandBytes = size_t(kBandReplicas) * kBandRep * 4;
constexpr size_t kCountBytes = 4096;                 // per-region counts (above, list 1, list 2)
constexpr size_t kFixedBytes = kStateBytes + kSampleBytes + kBandBytes + kCountBytes;
constexpr int kClearPieces = int(kBandBytes / 16);   // 16-byte pieces of the band histogram
constexpr int kClearWGs = (kClearPieces + kStreamThreads - 1) / kStreamThreads;
static_assert(3 * kGrid * 4 <= int(kCountBytes), "per-region counts");
static_assert(kBins % kStreamThreads == 0, "bins per thread");
static_assert(kGroupBins == 2 * 64 && (kRep * 4) % 16 == 0, "a wave reads a group's bins in pairs");
static_assert(kSubBins == kStreamThreads, "band layout: thread t owns sub-bin t");
// A larger array is cut into kSampleChunks windows of at least kSampleRun entries each.
static_assert(kBandBytes % 16 == 0 && kSampleAll >= int64_t(kSampleChunks) * kSampleRun, "sizes");

// Digits of the full selection (the fallback): 13, 13, 13, 13 and 12 bits from the top.
__host__ __device__ constexpr int digit_shift(int pass) { return pass < 4 ? 51 - 13 * pass : 0; }
__host__ __device__ constexpr int digit_bits(int pass) { return pass < 4 ? 13 : 12; }
// Digits of the final workgroup below the band prefix: bits 40..28, 27..15, 14..2 and 1..0.
__host__ __device__ constexpr int tail_shift(int pass) { return pass < 3 ? 28 - 13 * pass : 0; }
__host__ __device__ constexpr int tail_bits(int pass) { return pass < 3 ? 13 : 2; }

struct State {
  int32_t d_lo, d_hi;            // band of top digits (pass1, workgroup 0)
  int32_t mode;                  // list pass: 0 = k* is in the band, 1 = the exact fallback runs
  int32_t pad;
  unsigned long long prefix;     // k*'s top 23 bits in place (list pass)
  unsigned long long k_rem;      // rank of k* (1 = largest) among the list-2 keys
};
static_assert(sizeof(State) <= kStateBytes, "state");

// Sizes that follow from the problem alone (the same on the host and in every kernel).
struct Geometry {
  int32_t grid;                  // workgroups of the full pass = list-1 regions
  int32_t list_grid;             // workgroups of the list pass = list-2 regions (= grid)
  int64_t cap1;                  // list-1 entries per region (the entries its workgroup visits)
  int64_t cap2;                  // list-2 entries per region (= cap1)
};

struct Args {
  const float* scores;
  uint8_t* keep;
  State* st;
  unsigned int* sample;          // [kSampleWGs][kRep]: top-digit histograms of the sample
  unsigned int* band;            // [kBandReplicas][kBandRep]: band digit x sub-digit, then totals
  unsigned int* count_above;     // [grid]: pool entries above the band, per workgroup (mod 2^32)
  unsigned int* count1;          // [grid]: list-1 entries in each region
  unsigned int* count2;          // [grid]: list-2 entries in each region
  unsigned long long* list1;     // [grid][cap1]
  unsigned long long* list2;     // [list_grid][cap2]
  int64_t row_stride;
  int64_t n;                     // L*H*N < 2^31
  int64_t pool;                  // L*H*(N-1)
  int64_t cap1, cap2;
  int32_t grid;
  int32_t list_grid;
  int32_t N;
  int32_t current;
  int32_t magic_shift;
  int32_t force_fallback;        // test aid: 1 makes the list pass take the exact fallback
  unsigned long long magic;      // row of flat index i: (i * magic) >> magic_shift
  unsigned long long k;          // K = M - L*H, 1 <= K < pool size
};

__device__ __forceinline__ int row_of(const Args& a, int64_t i) {
  return int((static_cast<unsigned long long>(i) * a.magic) >> a.magic_shift);
}

// The order-preserving bits of a score (the high word of its key).
__device__ __forceinline__ uint32_t ord_of(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0u) u = 0u;                        // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long make_key(float x, uint32_t idx) {
  return (static_cast<unsigned long long>(ord_of(x)) << 32) | static_cast<unsigned long long>(~idx);
}

__device__ __forceinline__ int top_digit(float x) { return int(ord_of(x) >> (digit_shift(0) - 32)); }

// Whether flat entry i is a row's current position (kept outside the pool).
__device__ __forceinline__ bool is_current(const Args& a, int64_t i) {
  return i - int64_t(row_of(a, i)) * a.N == a.current;
}

__device__ __forceinline__ float score_at(const Args& a, int64_t i) {
  const int row = row_of(a, i);
  return a.scores[int64_t(row) * a.row_stride + (i - int64_t(row) * a.N)];
}

// Four consecutive entries i0 .. i0+3 (i0 a multiple of 4, i0 >= 0) and whether each is inside
// the array. VEC: dense rows (row_stride == N) and n a multiple of 4, so the scores are one flat
// array read with aligned 128-bit loads and no row arithmetic. Otherwise each entry is addressed
// through its row. The loads are issued unconditionally (an entry past the end reads entry 0 and
// is marked invalid): a load under a branch hides it from the compiler's wait counts, which then
// wait for every load in flight, the next iteration's included.
template <bool VEC>
__device__ __forceinline__ void in_range4(const Args& a, int64_t i0, bool (&valid)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) valid[e] = VEC ? i0 < a.n : i0 + e < a.n;
}

template <bool VEC>
__device__ __forceinline__ void load4(const Args& a, int64_t i0, float (&x)[4], bool (&valid)[4]) {
  if constexpr (VEC) {
    const bool in = i0 < a.n;
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.scores + (in ? i0 : 0)));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      valid[e] = in;
      x[e] = v[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      valid[e] = i < a.n;
      x[e] = score_at(a, valid[e] ? i : 0);
    }
  }
}

// Writes the mask bytes of entries i0 .. i0+3 (only those inside the array).
template <bool VEC>
__device__ __forceinline__ void store4(const Args& a, int64_t i0, const uint32_t (&m)[4],
                                       const bool (&valid)[4]) {
  if constexpr (VEC) {
    if (valid[0]) *reinterpret_cast<uint32_t*>(a.keep + i0) = m[0] | (m[1] << 8) | (m[2] << 16) | (m[3] << 24);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (valid[e]) a.keep[i0 + e] = uint8_t(m[e]);
  }
}

// Sum over the workgroup (every thread gets the total; s_wave: kStreamThreads / 64 words).
__device__ __forceinline__ unsigned long long block_sum(unsigned long long x, unsigned long long* s_wave) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = x;
  __syncthreads();
  unsigned long long t = 0;
#pragma unroll
  for (int w = 0; w < kStreamThreads / 64; ++w) t += s_wave[w];
  __syncthreads();
  return t;
}

// Exclusive prefix sum over the workgroup's threads in thread order (s_wave: kStreamThreads/64).
__device__ __forceinline__ unsigned int block_exclusive_scan(unsigned int x, unsigned int* s_wave) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  unsigned int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  __syncthreads();
  return base + inc - x;
}

// Given a histogram of the digit (bits [shift, shift + bits)) over the keys that share k*'s
// higher bits (s_tot, in LDS), fix that digit: the bin, scanned from the top, in which the
// running count first reaches k_rem. Updates *prefix and *k_rem (LDS) for the whole workgroup.
__device__ void select_digit(const unsigned int* s_tot, int shift, int bits, unsigned long long* prefix,
                             unsigned long long* k_rem) {
  __shared__ unsigned int s_wave[kStreamThreads / 64];
  const int nb = 1 << bits;
  const int per = nb >= kStreamThreads ? nb / kStreamThreads : 1;
  const int first = nb - 1 - int(threadIdx.x) * per;  // this thread's bins: first, first-1, ...
  unsigned int local = 0;
  if (first >= 0)
    for (int j = 0; j < per; ++j) local += s_tot[first - j];
  const unsigned int before = block_exclusive_scan(local, s_wave);
  const unsigned long long k = *k_rem;
  __syncthreads();
  if (first >= 0 && before < k && k <= static_cast<unsigned long long>(before) + local) {
    unsigned long long acc = before;
    for (int j = 0; j < per; ++j) {
      const unsigned int c = s_tot[first - j];
      if (k <= acc + c) {
        *prefix |= static_cast<unsigned long long>(first - j) << shift;
        *k_rem = k - acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Sampled entries of thread t in sample workgroup w: kSampleGroups groups of four consecutive entries,
// group j starting at the flat index this returns (a multiple of 4; entries past the end of the
// thread's range are invalid). An array of at most kSampleAll entries is split into kSampleWGs
// contiguous ranges, every entry taken; a larger one is cut into kSampleChunks equal windows
// (a multiple of 4 entries each) and chunk c takes kSampleRun consecutive entries at a scattered
// offset inside window c, kSampleRun / (4 kSampleGroups) threads per chunk, each group of them
// reading consecutive bytes with each load.
__device__ __forceinline__ int64_t sample_group(const Args& a, int w, int t, int j, int64_t* end) {
  if (a.n <= kSampleAll) {
    const int64_t per = ((a.n + kSampleWGs - 1) / kSampleWGs + 3) & ~int64_t(3);
    const int64_t last = int64_t(w + 1) * per;
    *end = last < a.n ? last : a.n;
    return int64_t(w) * per + (int64_t(j) * kStreamThreads + t) * 4;  // per <= kStreamThreads * 4 * kSampleGroups
  }
  constexpr int kThreadsPerRun = kSampleRun / (4 * kSampleGroups);
  const int c = w * kSampleChunksPerWG + t / kThreadsPerRun;
  const int64_t window = (a.n / kSampleChunks) & ~int64_t(3);  // >= kSampleRun here
  const int64_t slack = window - kSampleRun;
  const int64_t jitter = int64_t((uint64_t(c) * 2654435761ull) % uint64_t(slack + 1)) & ~int64_t(3);
  const int64_t start = int64_t(c) * window + jitter;
  *end = start + kSampleRun;
  return start + (t % kThreadsPerRun) * 4 + j * (4 * kThreadsPerRun);
}

// Sample histograms (workgroups 0 .. kSampleWGs-1: each writes its whole histogram, pool entries
// only) and the clearing of the band histogram (the other workgroups).
template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void init_kernel(const Args a) {
  __shared__ unsigned int h[kBins];
  if (blockIdx.x >= kSampleWGs) {
    const int i = int(blockIdx.x - kSampleWGs) * kStreamThreads + int(threadIdx.x);
    if (i < kClearPieces) reinterpret_cast<u32x4_t*>(a.band)[i] = u32x4_t{0u, 0u, 0u, 0u};
    return;
  }
  for (int i = threadIdx.x; i < kBins; i += kStreamThreads) h[i] = 0u;
  __syncthreads();
  const int w = int(blockIdx.x);
  float x[kSampleGroups][4];
  bool valid[kSampleGroups][4];
  int64_t i0[kSampleGroups], end[kSampleGroups];
#pragma unroll
  for (int j = 0; j < kSampleGroups; ++j) {  // every load first, then the histogram
    i0[j] = sample_group(a, w, int(threadIdx.x), j, &end[j]);
    load4<VEC>(a, i0[j], x[j], valid[j]);
  }
#pragma unroll
  for (int j = 0; j < kSampleGroups; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (valid[j][e] && i0[j] + e < end[j] && !is_current(a, i0[j] + e)) atomicAdd(&h[top_digit(x[j][e])], 1u);
  __syncthreads();
  unsigned int* out = a.sample + size_t(w) * kRep;
  for (int i = threadIdx.x; i < kBins; i += kStreamThreads) out[i] = h[i];
  // Group totals: 16 consecutive lanes add 8 bins each and combine by shuffles.
  const int t = int(threadIdx.x);
  const int grp = t >> 4;
  const unsigned int* b = h + grp * kGroupBins + (t & 15) * 8;
  unsigned int c = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) c += b[j];
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) c += __shfl_xor(c, off, 16);
  if ((t & 15) == 0) out[kBins + grp * kGroupStride] = c;
}

// The one full pass: the band from the sample, the mask outside the band, list 1 and the band
// histogram inside it, and the exact count of entries above the band.
// The band [d_lo, d_hi] from the sample histograms (R replicas), by wave 0 in two memory round
// trips: the 64 group totals of every replica (one group per lane), from which the sample size m,
// the target ranks and their groups follow; then the 128 bins of both target groups (two bins
// per lane and group). Ranks count from the top (1 = largest). Results in *d_hi, *d_lo (LDS).
template <int R>
__device__ void sample_band(const Args& a, int* d_hi, int* d_lo) {
  if (threadIdx.x < 64) {
    const int lane = int(threadIdx.x);
    const unsigned int* h = a.sample;
    unsigned int c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) c += h[size_t(r) * kRep + kBins + lane * kGroupStride];
    unsigned int suf = c;  // counts in this lane's group and every higher one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned int y = __shfl_down(suf, off);
      if (lane + off < 64) suf += y;
    }
    const unsigned long long m = __shfl(suf, 0);  // the sampled pool entries (>= 1)
    // k*'s rank in the sample, r = K m / pool, and the ranks r -/+ delta: delta = 0 when the
    // whole pool was sampled (both ranks are then K and the band is k*'s digit), else eight
    // standard deviations of the sampled count above a fixed quantile, plus 32.
    const bool whole = a.n <= kSampleAll;
    const double f = double(a.k) / double(a.pool);
    const unsigned long long rk = whole ? a.k : (unsigned long long)(double(m) * f + 0.5);
    const unsigned long long delta =
        whole ? 0ull : (unsigned long long)(8.0 * sqrt(double(m) * f * (1.0 - f))) + 32ull;
    const unsigned long long lo_rank = rk > delta ? rk - delta : 1ull;
    const unsigned long long rank[2] = {lo_rank < m ? lo_rank : m, rk + delta < m ? rk + delta : m};
    const unsigned long long above = suf - c;
    int grp[2];
    unsigned long long k1[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const unsigned long long hit = __ballot(above < rank[q] && rank[q] <= above + c);
      grp[q] = hit != 0ull ? __ffsll(static_cast<long long>(hit)) - 1 : 0;
      k1[q] = rank[q] - static_cast<unsigned long long>(__shfl(suf - c, grp[q]));
    }
    unsigned int fa[2] = {0u, 0u}, fb[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int bin_a = grp[q] * kGroupBins + kGroupBins - 1 - 2 * lane;  // bins bin_a, bin_a - 1
#pragma unroll
      for (int r = 0; r < R; ++r) {
        fa[q] += h[size_t(r) * kRep + bin_a];
        fb[q] += h[size_t(r) * kRep + bin_a - 1];
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int bin_a = grp[q] * kGroupBins + kGroupBins - 1 - 2 * lane;
      const unsigned int local = fa[q] + fb[q];
      unsigned int inc = local;  // counts of this lane's bins and every higher one in the group
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      const unsigned long long before = inc - local;
      if (before < k1[q] && k1[q] <= before + local) {
        const int d = k1[q] <= before + fa[q] ? bin_a : bin_a - 1;
        if (q == 0) *d_hi = d; else *d_lo = d;
      }
    }
  }
  __syncthreads();
}

// The one full pass: the band from the sample, the mask outside the band, list 1 and the band
// histogram inside it, and the exact count of entries above the band. Each workgroup issues its
// first loads of scores before it reads the sample, so that they are in flight meanwhile.
template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void pass1_kernel(const Args a) {
  __shared__ unsigned int h2[kBandDigits * kSubBins];
  __shared__ unsigned int s_n;
  __shared__ int s_dhi, s_dlo;
  __shared__ unsigned long long s_wave[kStreamThreads / 64];
  const int64_t base0 = int64_t(blockIdx.x) * kChunk;
  const int64_t stride = int64_t(gridDim.x) * kChunk;
  // Validity is recomputed from the index where an entry is used rather than held across the
  // loop (held flags take scalar registers, two per entry and buffer).
  auto load_chunk = [&](int64_t base, float (&xs)[kSlabs][4]) {
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      bool unused[4];
      load4<VEC>(a, base + s * (kStreamThreads * kVec) + int(threadIdx.x) * kVec, xs[s], unused);
    }
  };
  // One chunk in flight while the band is read (a workgroup has about that much in flight at
  // most: a second chunk's loads only wait at issue).
  float x[kSlabs][4];
  load_chunk(base0, x);
  // Current positions are not pool entries, but the full pass below treats every entry alike (a
  // per-entry test would cost registers in its unrolled loop). Workgroup b takes the current
  // positions of rows b, b + grid, ... back out: from its count above the band and from its band
  // histogram. Its own counts may wrap below zero; their sums over the workgroups are exact. The
  // list pass skips current positions that entered list 1.
  const int64_t rows = a.n / a.N;
  const int64_t row0 = int64_t(blockIdx.x) + int64_t(threadIdx.x) * gridDim.x;
  const float x_cur = row0 < rows ? a.scores[row0 * a.row_stride + a.current] : 0.f;
  for (int i = threadIdx.x; i < kBandDigits * kSubBins; i += kStreamThreads) h2[i] = 0u;
  if (threadIdx.x == 0) {
    s_n = 0u;
    s_dhi = kBins - 1;
    s_dlo = 0;
  }
  __syncthreads();
  sample_band<kSampleWGs>(a, &s_dhi, &s_dlo);
  const int d_hi = s_dhi;
  const int d_lo = s_dlo > d_hi - (kBandDigits - 1) ? s_dlo : d_hi - (kBandDigits - 1);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.st->d_lo = d_lo;
    a.st->d_hi = d_hi;
  }
  unsigned int above = 0;
  for (int64_t row = row0; row < rows; row += int64_t(kStreamThreads) * gridDim.x) {
    const float xc = row == row0 ? x_cur : a.scores[row * a.row_stride + a.current];
    const int d = top_digit(xc);
    if (d > d_hi) {
      --above;
    } else if (d >= d_lo) {
      const uint32_t idx = uint32_t(row * a.N + a.current);
      atomicSub(&h2[(d - d_lo) * kSubBins + int((make_key(xc, idx) >> kPrefixShift) & (kSubBins - 1))], 1u);
    }
  }
  unsigned long long* region = a.list1 + int64_t(blockIdx.x) * a.cap1;
  auto process = [&](int64_t base, const float (&xs)[kSlabs][4]) {
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      const int64_t i0 = base + s * (kStreamThreads * kVec) + int(threadIdx.x) * kVec;
      bool vs[4];
      in_range4<VEC>(a, i0, vs);
      uint32_t mk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // Current positions get their 1 from the final kernel; in the band they enter list 1 like
        // any entry and the list pass drops them.
        const int d = top_digit(xs[s][e]);
        const bool up = vs[e] && d > d_hi;
        mk[e] = up ? 1u : 0u;
        above += up ? 1u : 0u;
        if (vs[e] && d >= d_lo && d <= d_hi) {
          const unsigned long long key = make_key(xs[s][e], uint32_t(i0 + e));
          region[atomicAdd(&s_n, 1u)] = key;
          atomicAdd(&h2[(d - d_lo) * kSubBins + int((key >> kPrefixShift) & (kSubBins - 1))], 1u);
        }
      }
      store4<VEC>(a, i0, mk, vs);
    }
  };
  // Two register buffers in turn: each chunk's loads are issued one chunk ahead of its use, and
  // no values move between the buffers (a move would wait for every load in flight).
  float xb[kSlabs][4];
  for (int64_t base = base0; base < a.n; base += 2 * stride) {
    load_chunk(base + stride, xb);
    process(base, x);
    load_chunk(base + 2 * stride, x);
    if (base + stride < a.n) process(base + stride, xb);
  }
  const unsigned int above_total = unsigned(block_sum(above, s_wave));  // mod 2^32
  if (threadIdx.x == 0) {
    a.count_above[blockIdx.x] = above_total;
    a.count1[blockIdx.x] = s_n;
  }
  // Add the band histogram into one replica: thread t takes sub-bin t of every band digit (so a
  // wave's atomics hit 64 consecutive words), skipping bins that stayed zero; each digit's total
  // is reduced per wave, summed over the waves in LDS and added one 128-byte line apart.
  __shared__ unsigned int s_tot[kStreamThreads / 64][kBandDigits];
  unsigned int* g = a.band + size_t(blockIdx.x % kBandReplicas) * kBandRep;
  const int nd = d_hi - d_lo + 1;
  const int wave = int(threadIdx.x >> 6);
  const int lane = int(threadIdx.x & 63);
  for (int j = 0; j < nd; ++j) {
    const unsigned int v = h2[j * kSubBins + threadIdx.x];
    if (v != 0u) __hip_atomic_fetch_add(g + j * kSubBins + threadIdx.x, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned int c = v;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) s_tot[wave][j] = c;
  }
  __syncthreads();
  if (int(threadIdx.x) < nd) {
    unsigned int c = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) c += s_tot[w][threadIdx.x];
    if (c != 0u)
      __hip_atomic_fetch_add(g + kBandDigits * kSubBins + threadIdx.x * kGroupStride, c, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// List pass: every workgroup fixes k*'s rank inside the band and its top 23 bits (identically),
// then walks the list-1 regions r = blockIdx.x, blockIdx.x + gridDim.x, ...: entries above those
// bits get a 1, entries sharing them go to this workgroup's list-2 region. When k* is not inside
// the band, workgroup 0 sets the fallback mode and every workgroup leaves.
__global__ __launch_bounds__(kStreamThreads) void list_kernel(const Args a) {
  __shared__ unsigned long long s_wave[kStreamThreads / 64];
  __shared__ unsigned int s_wave32[kStreamThreads / 64];
  __shared__ unsigned int s_n;
  __shared__ int s_j, s_sub;
  __shared__ unsigned long long s_k1, s_k2;
  const int t = int(threadIdx.x);
  constexpr int kPre = 4;  // list-1 keys per thread loaded before the prefix is known
  const unsigned long long* src = a.list1 + int64_t(blockIdx.x) * a.cap1;
  const unsigned int count = a.count1[blockIdx.x];
  // Every load that depends on nothing is issued first: this region's count, the state, the
  // per-region counts and the totals of every band digit (thread t < kBandDigits: band digit
  // kBandDigits - 1 - t; digits past the band stayed zero).
  const int d_lo = a.st->d_lo;
  const int d_hi = a.st->d_hi;
  unsigned long long up = 0;
  for (int r = t; r < a.grid; r += kStreamThreads) up += a.count_above[r];
  unsigned int c = 0;
  if (t < kBandDigits) {
#pragma unroll
    for (int r = 0; r < kBandReplicas; ++r)
      c += a.band[size_t(r) * kBandRep + kBandDigits * kSubBins + (kBandDigits - 1 - t) * kGroupStride];
  }
  unsigned long long pre[kPre];
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    const unsigned int i = unsigned(t) + unsigned(q) * kStreamThreads;
    pre[q] = i < count ? src[i] : 0ull;
  }
  // Pool entries above the band: the per-workgroup counts summed mod 2^32 (the true count is
  // below 2^31). Pool entries in the band: the band digits' totals.
  const unsigned long long pool_above = static_cast<uint32_t>(block_sum(up, s_wave));
  const unsigned long long band = block_sum(c, s_wave);
  // k*'s rank among the band entries is K - pool_above; outside [1, band]: not in the band.
  const bool in_band = a.force_fallback == 0 && pool_above < a.k && a.k - pool_above <= band;
  if (!in_band) {
    if (blockIdx.x == 0 && t == 0) a.st->mode = 1;
    return;
  }
  const unsigned long long k0 = a.k - pool_above;
  if (t == 0) {
    s_n = 0u;
    s_j = 0;
    s_sub = 0;
    s_k1 = 1;
    s_k2 = 1;
  }
  // The band digit holding rank k0, scanning from the top.
  unsigned int before = block_exclusive_scan(c, s_wave32);
  if (t < kBandDigits && before < k0 && k0 <= static_cast<unsigned long long>(before) + c) {
    s_j = kBandDigits - 1 - t;
    s_k1 = k0 - before;
  }
  __syncthreads();
  const int j = s_j;
  const unsigned long long k1 = s_k1;
  // Its sub-digit: bins 1023, 1022, ..., 0 of band digit j (thread t: bin 1023 - t).
  c = 0;
#pragma unroll
  for (int r = 0; r < kBandReplicas; ++r) c += a.band[size_t(r) * kBandRep + j * kSubBins + (kSubBins - 1 - t)];
  before = block_exclusive_scan(c, s_wave32);
  if (before < k1 && k1 <= static_cast<unsigned long long>(before) + c) {
    s_sub = kSubBins - 1 - t;
    s_k2 = k1 - before;
  }
  __syncthreads();
  const unsigned long long want = (static_cast<unsigned long long>(d_lo + j) << kSubBits) |
                                  static_cast<unsigned long long>(s_sub);
  if (blockIdx.x == 0 && t == 0) {
    a.st->mode = 0;
    a.st->prefix = want << kPrefixShift;
    a.st->k_rem = s_k2;
  }
  unsigned long long* region = a.list2 + int64_t(blockIdx.x) * a.cap2;
  auto classify = [&](unsigned long long key) {
    if (is_current(a, int64_t(~static_cast<uint32_t>(key)))) return;
    const unsigned long long top = key >> kPrefixShift;
    if (top > want)
      a.keep[~static_cast<uint32_t>(key)] = 1u;
    else if (top == want)
      region[atomicAdd(&s_n, 1u)] = key;
  };
#pragma unroll
  for (int q = 0; q < kPre; ++q)
    if (unsigned(t) + unsigned(q) * kStreamThreads < count) classify(pre[q]);
  for (unsigned int i = unsigned(t) + kPre * kStreamThreads; i < count; i += kStreamThreads) classify(src[i]);
  __syncthreads();
  if (t == 0) a.count2[blockIdx.x] = s_n;
}

// The exact selection by one workgroup when k* was not in the band: five digit passes over every
// pool key (LDS histograms), then the whole mask, current positions included.
template <bool VEC>
__device__ void fallback_select(const Args& a, unsigned int* s_tot, unsigned long long* s_prefix,
                                unsigned long long* s_k) {
  if (threadIdx.x == 0) {
    *s_prefix = 0ull;
    *s_k = a.k;
  }
  for (int pass = 0; pass < 5; ++pass) {
    for (int b = threadIdx.x; b < kBins; b += kStreamThreads) s_tot[b] = 0u;
    __syncthreads();
    const int hs = digit_shift(pass) + digit_bits(pass);  // bits above this digit
    const unsigned long long want = hs >= 64 ? 0ull : (*s_prefix >> hs);
    for (int64_t i0 = int64_t(threadIdx.x) * kVec; i0 < a.n; i0 += int64_t(kStreamThreads) * kVec) {
      float x[4];
      bool valid[4];
      load4<VEC>(a, i0, x, valid);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!valid[e] || is_current(a, i0 + e)) continue;
        const unsigned long long key = make_key(x[e], uint32_t(i0 + e));
        if (hs >= 64 || (key >> hs) == want)
          atomicAdd(&s_tot[int((key >> digit_shift(pass)) & ((1ull << digit_bits(pass)) - 1ull))], 1u);
      }
    }
    __syncthreads();
    select_digit(s_tot, digit_shift(pass), digit_bits(pass), s_prefix, s_k);
  }
  const unsigned long long kstar = *s_prefix;
  for (int64_t i0 = int64_t(threadIdx.x) * kVec; i0 < a.n; i0 += int64_t(kStreamThreads) * kVec) {
    float x[4];
    bool valid[4];
    load4<VEC>(a, i0, x, valid);
    uint32_t mk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      mk[e] = (is_current(a, i0 + e) || make_key(x[e], uint32_t(i0 + e)) >= kstar) ? 1u : 0u;
    store4<VEC>(a, i0, mk, valid);
  }
}

// One workgroup finishes: list 2 ranked (or, in fallback mode, the whole selection), then every
// row's current position gets its 1. List 2 is visited as one concatenated array: entry j lives
// in the region r with s_offs[r] <= j < s_offs[r + 1]; when it fits, it is first copied into LDS
// so that the digit passes do not wait on global memory.
template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void final_kernel(const Args a) {
  __shared__ unsigned int s_tot[kBins];
  __shared__ unsigned long long s_keys[kLdsKeys];
  __shared__ unsigned long long s_prefix, s_k;
  __shared__ unsigned int s_offs[kGrid + 1];
  __shared__ unsigned int s_wave[kStreamThreads / 64];
  if (a.st->mode != 0) {
    fallback_select<VEC>(a, s_tot, &s_prefix, &s_k);
    return;
  }
  const unsigned int c = int(threadIdx.x) < a.list_grid ? a.count2[threadIdx.x] : 0u;
  const unsigned int off = block_exclusive_scan(c, s_wave);
  if (int(threadIdx.x) < a.list_grid) s_offs[threadIdx.x] = off;
  if (int(threadIdx.x) == a.list_grid - 1) s_offs[a.list_grid] = off + c;
  if (threadIdx.x == 0) {
    s_prefix = a.st->prefix;
    s_k = a.st->k_rem;
  }
  __syncthreads();
  const unsigned int total = s_offs[a.list_grid];
  auto global_entry = [&](unsigned int j) {
    int lo = 0, hi = a.list_grid - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_offs[mid] <= j) lo = mid; else hi = mid - 1;
    }
    return a.list2[int64_t(lo) * a.cap2 + (j - s_offs[lo])];
  };
  const bool staged = total <= unsigned(kLdsKeys);
  if (staged) {
    for (unsigned int j = threadIdx.x; j < total; j += kStreamThreads) s_keys[j] = global_entry(j);
    __syncthreads();
  }
  auto entry = [&](unsigned int j) { return staged ? s_keys[j] : global_entry(j); };
  if (total <= unsigned(kStreamThreads)) {
    // A short list 2 (the usual case) is ranked directly: keys are distinct (each holds its
    // flat index), and a key is at or above k* exactly when fewer than k_rem keys of list 2
    // are larger, k_rem being k*'s rank among them. Every thread reads every key (LDS
    // broadcast) and counts those above its own.
    const unsigned long long k_rem = s_k;
    if (threadIdx.x < total) {
      const unsigned long long mine = s_keys[threadIdx.x];
      unsigned int above = 0;
      for (unsigned int j = 0; j < total; ++j) above += s_keys[j] > mine ? 1u : 0u;
      if (above < k_rem) a.keep[~static_cast<uint32_t>(mine)] = 1u;
    }
  } else {
    for (int pass = 0; pass < 4; ++pass) {
      for (int b = threadIdx.x; b < kBins; b += kStreamThreads) s_tot[b] = 0u;
      __syncthreads();
      const int hs = tail_shift(pass) + tail_bits(pass);  // bits above this digit
      const unsigned long long want = s_prefix >> hs;
      for (unsigned int j = threadIdx.x; j < total; j += kStreamThreads) {
        const unsigned long long key = entry(j);
        if ((key >> hs) == want)
          atomicAdd(&s_tot[int((key >> tail_shift(pass)) & ((1ull << tail_bits(pass)) - 1ull))], 1u);
      }
      __syncthreads();
      select_digit(s_tot, tail_shift(pass), tail_bits(pass), &s_prefix, &s_k);
    }
    const unsigned long long kstar = s_prefix;
    for (unsigned int j = threadIdx.x; j < total; j += kStreamThreads) {
      const unsigned long long key = entry(j);
      if (key >= kstar) a.keep[~static_cast<uint32_t>(key)] = 1u;
    }
  }
  // Rule 1: every row's current position stays (pass 1 gave it the value of its top digit).
  const int64_t rows = a.n / a.N;
  for (int64_t r = threadIdx.x; r < rows; r += kStreamThreads) a.keep[r * a.N + a.current] = 1u;
}

// The budget alone decides: all = 0 keeps only the current positions, all = 1 keeps everything.
__global__ __launch_bounds__(256) void fill_kernel(const Args a, int all) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < a.n; i += int64_t(gridDim.x) * 256) {
    const int row = row_of(a, i);
    const int t = int(i - int64_t(row) * a.N);
    a.keep[i] = (all != 0 || t == a.current) ? 1u : 0u;
  }
}

// kept_per_row[r] = number of ones in row r of the mask.
__global__ __launch_bounds__(256) void row_count_kernel(const uint8_t* keep, int32_t N, int32_t* out) {
  __shared__ unsigned int s_wave[4];
  const uint8_t* row = keep + int64_t(blockIdx.x) * N;
  unsigned int c = 0;
  for (int t = threadIdx.x; t < N; t += 256) c += row[t];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = int32_t(s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3]);
}

Geometry geometry(int64_t n) {
  Geometry g;
  const int64_t chunks = (n + kChunk - 1) / kChunk;
  g.grid = int32_t(chunks < kGrid ? chunks : kGrid);
  g.cap1 = ((chunks + g.grid - 1) / g.grid) * kChunk;  // entries one workgroup visits, at most
  g.list_grid = g.grid;  // one list-1 region per list workgroup
  g.cap2 = g.cap1;
  return g;
}

int ceil_log2(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

kv_attn_status check(const kv_evict_params* p) {
  if (p == nullptr) return KV_ATTN_ERR_NULL;
  if (p->num_layers < 1 || p->num_heads < 1 || p->num_tokens < 1) return KV_ATTN_ERR_SHAPE;
  if (p->current < 0 || p->current >= p->num_tokens) return KV_ATTN_ERR_SHAPE;
  if (p->row_stride < p->num_tokens) return KV_ATTN_ERR_SHAPE;
  if (p->budget < 0) return KV_ATTN_ERR_VALUE;
  const int64_t rows = int64_t(p->num_layers) * p->num_heads;
  if (rows * p->num_tokens > int64_t(INT32_MAX)) return KV_ATTN_ERR_UNSUPPORTED;
  return KV_ATTN_OK;
}

// Budget left for the pool, clamped: <= 0 keeps only the current positions.
int64_t free_slots(const kv_evict_params* p) {
  return p->budget - int64_t(p->num_layers) * p->num_heads;
}

int64_t pool_size(const kv_evict_params* p) {
  return int64_t(p->num_layers) * p->num_heads * (p->num_tokens - 1);
}

bool needs_ranking(const kv_evict_params* p) {
  const int64_t k = free_slots(p);
  return k > 0 && k < pool_size(p);
}

// KV_EVICT_FORCE_FALLBACK=1 (a test aid) sends every ranked call down the exact fallback path.
bool fallback_forced() {
  const char* e = getenv("KV_EVICT_FORCE_FALLBACK");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

}  // namespace
}  // namespace kvevict

extern "C" {

size_t kv_evict_workspace_size(const kv_evict_params* p) {
  using namespace kvevict;
  if (check(p) != KV_ATTN_OK || !needs_ranking(p)) return 0;
  const Geometry g = geometry(int64_t(p->num_layers) * p->num_heads * p->num_tokens);
  return kFixedBytes + 8u * size_t(int64_t(g.grid) * g.cap1 + int64_t(g.list_grid) * g.cap2);
}

kv_attn_status kv_evict_select(const float* scores, uint8_t* keep, int32_t* kept_per_row,
                               const kv_evict_params* p, void* workspace, size_t workspace_bytes,
                               void* stream) {
  using namespace kvevict;
  if (scores == nullptr || keep == nullptr || p == nullptr) return KV_ATTN_ERR_NULL;
  const kv_attn_status st = check(p);
  if (st != KV_ATTN_OK) return st;
  if (!aligned(scores, 4) || (kept_per_row != nullptr && !aligned(kept_per_row, 4)))
    return KV_ATTN_ERR_UNSUPPORTED;
  const bool rank = needs_ranking(p);
  if (rank) {
    if (workspace == nullptr || workspace_bytes < kv_evict_workspace_size(p))
      return KV_ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return KV_ATTN_ERR_UNSUPPORTED;
  }
  if (kvattn::fault_injected("launch")) return KV_ATTN_ERR_HIP;

  const int64_t rows = int64_t(p->num_layers) * p->num_heads;
  Args a = {};
  a.scores = scores;
  a.keep = keep;
  a.row_stride = p->row_stride;
  a.n = rows * p->num_tokens;
  a.pool = pool_size(p);
  a.N = p->num_tokens;
  a.current = p->current;
  a.force_fallback = fallback_forced() ? 1 : 0;
  // floor(i / N) = (i * ceil(2^s / N)) >> s for every i < 2^31 when s = 31 + ceil(log2 N):
  // the multiplier exceeds 2^s / N by less than 1, which adds less than i / 2^s < 1 / N to
  // the quotient, too little to reach the next integer.
  a.magic_shift = 31 + ceil_log2(p->num_tokens);
  a.magic = ((1ull << a.magic_shift) + uint64_t(p->num_tokens) - 1) / uint64_t(p->num_tokens);
  a.k = rank ? static_cast<unsigned long long>(free_slots(p)) : 0ull;
  const Geometry g = geometry(a.n);
  a.grid = g.grid;
  a.list_grid = g.list_grid;
  a.cap1 = g.cap1;
  a.cap2 = g.cap2;
  if (rank) {
    char* ws = static_cast<char*>(workspace);
    a.st = reinterpret_cast<State*>(ws);
    a.sample = reinterpret_cast<unsigned int*>(ws + kStateBytes);
    a.band = reinterpret_cast<unsigned int*>(ws + kStateBytes + kSampleBytes);
    a.count_above = reinterpret_cast<unsigned int*>(ws + kStateBytes + kSampleBytes + kBandBytes);
    a.count1 = a.count_above + kGrid;
    a.count2 = a.count1 + kGrid;
    a.list1 = reinterpret_cast<unsigned long long*>(ws + kFixedBytes);
    a.list2 = a.list1 + int64_t(g.grid) * g.cap1;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!rank) {
    const int all = free_slots(p) > 0 ? 1 : 0;  // K >= pool: everything stays
    const int64_t blocks = (a.n + 255) / 256;
    hipLaunchKernelGGL(fill_kernel, dim3(uint32_t(blocks < 2048 ? blocks : 2048)), dim3(256), 0, s,
                       a, all);
    if (hipGetLastError() != hipSuccess) return KV_ATTN_ERR_HIP;
  } else {
    const bool vec = p->row_stride == p->num_tokens && a.n % 4 == 0 && aligned(scores, 16) &&
                     aligned(keep, 4);
    if (vec) {
      hipLaunchKernelGGL(init_kernel<true>, dim3(kSampleWGs + kClearWGs), dim3(kStreamThreads), 0, s, a);
      hipLaunchKernelGGL(pass1_kernel<true>, dim3(g.grid), dim3(kStreamThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL(init_kernel<false>, dim3(kSampleWGs + kClearWGs), dim3(kStreamThreads), 0, s, a);
      hipLaunchKernelGGL(pass1_kernel<false>, dim3(g.grid), dim3(kStreamThreads), 0, s, a);
    }
    hipLaunchKernelGGL(list_kernel, dim3(g.list_grid), dim3(kStreamThreads), 0, s, a);
    if (vec)
      hipLaunchKernelGGL(final_kernel<true>, dim3(1), dim3(kStreamThreads), 0, s, a);
    else
      hipLaunchKernelGGL(final_kernel<false>, dim3(1), dim3(kStreamThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return KV_ATTN_ERR_HIP;
  }
  if (kept_per_row != nullptr) {
    hipLaunchKernelGGL(row_count_kernel, dim3(uint32_t(rows)), dim3(256), 0, s, keep, p->num_tokens,
                       kept_per_row);
    if (hipGetLastError() != hipSuccess) return KV_ATTN_ERR_HIP;
  }
  return KV_ATTN_OK;
}

}  // extern "C"
