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
// whose key is at least k*, the K-th largest key. k* is found digit by digit from the top (a
// radix selection, five digits of 13, 13, 13, 13 and 12 bits), with kernel boundaries as the
// only grid-wide synchronisation:
//
//   init    clears the histograms;
//   pass0   every entry: histogram of the top digit;
//   pass1   every workgroup first fixes k*'s top digit from that histogram (the same result in
//           each), then streams every entry again: writes the whole mask (current positions 1,
//           entries whose top digit is above k*'s 1, all others 0 for now) and copies the keys
//           that share k*'s top digit into list 1 (each workgroup into its own region, so no
//           global counter is needed), with a histogram of their second digit;
//   list    every workgroup first fixes k*'s second digit from pass 1's histogram, then walks
//           its share of list 1: entries above k*'s first two digits get a 1, those sharing
//           them go to list 2 (again one region per workgroup);
//   final   one workgroup fixes digits 2 to 4 over list 2 with LDS histograms and gives a 1 to
//           the list-2 entries at or above k*.
//
// The two full passes stream the scores with coalesced 128-bit loads (HBM-bound: 8 bytes read
// and 1 written per entry); list 1 is typically a small fraction of the pool and list 2 a few
// entries (all of the pool only if nearly every score is equal, when the single final
// workgroup becomes the slow part). Histograms are built in LDS per workgroup and added into
// one of several global replicas with device-scope atomics, skipping bins that stayed zero, so
// few workgroups contend for one address. No kernel uses a device-scope fence or a grid-wide
// arrival counter: on this chip each costs tens of nanoseconds per workgroup, serialised.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv_attn_internal.h"
#include "kv_evict.h"

namespace kvevict {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 1024;                 // threads of a full-pass workgroup
constexpr int kVec = 4;                              // floats per 128-bit load
constexpr int kSlabs = 4;                            // loads per thread per iteration
constexpr int kChunk = kStreamThreads * kVec * kSlabs;  // entries per workgroup iteration
constexpr int kGrid = 256;                           // workgroups of the full passes (at most)
constexpr int kListGrid = 64;                        // workgroups of the list pass (at most)
constexpr int kFinishThreads = 1024;                 // list-pass and final workgroups
constexpr int kLdsKeys = 6144;                       // list-2 entries the final kernel stages
constexpr int kBins = 8192;                          // 13-bit digits
constexpr int kGroups = 64;                          // coarse bins: 128 consecutive digits each
constexpr int kGroupBins = kBins / kGroups;
// Group counters sit one 128-byte line apart: device-scope atomics from many workgroups to words
// of one line serialise (packed, the 64 counters of a replica made pass 1 2.2x slower on MI355X).
constexpr int kGroupStride = 32;
constexpr int kRep = kBins + kGroups * kGroupStride; // words per replica: bins, then groups
constexpr int kReplicas0 = 8;                        // copies of the top digit's histogram
constexpr int kReplicas1 = 4;                        // copies of the second digit's histogram
constexpr size_t kStateBytes = 256;
constexpr size_t kHistBytes = size_t(kReplicas0 + kReplicas1) * kRep * 4;
constexpr size_t kCountBytes = 4096;                 // per-region list-1 and list-2 counts
constexpr size_t kFixedBytes = kStateBytes + kHistBytes + kCountBytes;
static_assert((kGrid + kListGrid) * 4 <= int(kCountBytes), "per-region counts");
static_assert(kBins % kStreamThreads == 0 && kBins % kFinishThreads == 0, "bins per thread");
static_assert(kGroupBins == 2 * 64 && (kRep * 4) % 16 == 0, "a wave reads a group's bins in pairs");

__host__ __device__ constexpr int digit_shift(int pass) { return pass < 4 ? 51 - 13 * pass : 0; }
__host__ __device__ constexpr int digit_bits(int pass) { return pass < 4 ? 13 : 12; }

struct State {
  unsigned long long prefix0;    // k*'s top digit, in place (written by pass1)
  unsigned long long k_rem0;     // rank of k* (1 = largest) among the keys sharing it
  unsigned long long prefix1;    // k*'s top two digits (written by the list pass)
  unsigned long long k_rem1;     // rank of k* among the keys sharing them
};
static_assert(sizeof(State) <= kStateBytes, "state");

// Sizes that follow from the problem alone (the same on the host and in every kernel).
struct Geometry {
  int32_t grid;                  // workgroups of the full passes = list-1 regions
  int32_t list_grid;             // workgroups of the list pass = list-2 regions
  int64_t cap1;                  // list-1 entries per region (the entries its workgroup visits)
  int64_t cap2;                  // list-2 entries per region (the list-1 regions it walks)
};

struct Args {
  const float* scores;
  uint8_t* keep;
  State* st;
  unsigned int* hist0;           // [kReplicas0][kRep]: top digit over the pool (bins, groups)
  unsigned int* hist1;           // [kReplicas1][kRep]: second digit over list 1
  unsigned int* count1;          // [grid]: list-1 entries in each region
  unsigned int* count2;          // [list_grid]: list-2 entries in each region
  unsigned long long* list1;     // [grid][cap1]
  unsigned long long* list2;     // [list_grid][cap2]
  int64_t row_stride;
  int64_t n;                     // L*H*N < 2^31
  int64_t cap1, cap2;
  int32_t grid;
  int32_t list_grid;
  int32_t N;
  int32_t current;
  int32_t magic_shift;
  unsigned long long magic;      // row of flat index i: (i * magic) >> magic_shift
  unsigned long long k;          // K = M - L*H, 1 <= K < pool size
};

__device__ __forceinline__ int row_of(const Args& a, int64_t i) {
  return int((static_cast<unsigned long long>(i) * a.magic) >> a.magic_shift);
}

__device__ __forceinline__ unsigned long long make_key(float x, uint32_t idx) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0u) u = 0u;                        // -0.0 ranks as +0.0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(ord) << 32) | static_cast<unsigned long long>(~idx);
}
static_assert(51 >= 32, "the top digit lies in the score word");

__device__ __forceinline__ int digit_of(unsigned long long key, int pass) {
  return int((key >> digit_shift(pass)) & ((1ull << digit_bits(pass)) - 1ull));
}

// Four consecutive entries i0 .. i0+3 (i0 a multiple of 4) and whether each is inside the array.
// VEC: dense rows (row_stride == N) and n a multiple of 4, so the scores are one flat array read
// with aligned 128-bit loads and no row arithmetic. Otherwise each entry is addressed through its
// row.
template <bool VEC>
__device__ __forceinline__ void load4(const Args& a, int64_t i0, float (&x)[4], bool (&valid)[4]) {
  if constexpr (VEC) {
    const bool in = i0 < a.n;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (in) v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.scores + i0));
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
      x[e] = 0.f;
      if (valid[e]) {
        const int row = row_of(a, i);
        x[e] = a.scores[int64_t(row) * a.row_stride + (i - int64_t(row) * a.N)];
      }
    }
  }
}

// The order-preserving top bits of a score (the high word of its key), without building the key.
__device__ __forceinline__ uint32_t ord_of(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int top_digit(float x) { return int(ord_of(x) >> (digit_shift(0) - 32)); }

// Whether flat entry i is a row's current position (kept outside the pool).
__device__ __forceinline__ bool is_current(const Args& a, int64_t i) {
  return i - int64_t(row_of(a, i)) * a.N == a.current;
}

// Add a workgroup's LDS histogram into one replica of a global histogram, bins and groups (bins
// and groups that stayed zero are skipped, so a workgroup touches only what its entries hit).
// Group sums: 16 consecutive lanes add 8 bins each and combine by shuffles.
template <int THREADS>
__device__ __forceinline__ void flush_hist(const unsigned int* h_lds, unsigned int* h_glob) {
  static_assert(THREADS % 64 == 0 && (kGroups * 16) % THREADS == 0, "whole waves per pass");
  for (int i = threadIdx.x; i < kBins; i += THREADS) {
    const unsigned int c = h_lds[i];
    if (c != 0u) __hip_atomic_fetch_add(h_glob + i, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int t = threadIdx.x; t < kGroups * 16; t += THREADS) {
    const int grp = t >> 4;
    const unsigned int* b = h_lds + grp * kGroupBins + (t & 15) * 8;
    unsigned int c = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) c += b[j];
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) c += __shfl_xor(c, off, 16);
    if ((t & 15) == 0 && c != 0u)
      __hip_atomic_fetch_add(h_glob + kBins + grp * kGroupStride, c, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Fixes digit `pass` of k* from a global histogram of R replicas (bins and groups of 128 bins):
// the bin, scanned from the top, in which the running count first reaches *k_rem. Wave 0 alone
// reads the 64 group totals (one per lane), finds the group, then reads that group's 128 bins
// (two per lane, the top ones in lane 0) and finds the bin; the other waves wait at the
// barrier. Updates *prefix and *k_rem (LDS) for the whole workgroup.
template <int R>
__device__ void select_digit_global(const unsigned int* h, int pass, unsigned long long* prefix,
                                    unsigned long long* k_rem) {
  if (threadIdx.x < 64) {
    const int lane = int(threadIdx.x);
    unsigned int v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = h[size_t(r) * kRep + kBins + lane * kGroupStride];
    unsigned int c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) c += v[r];
    // Counts above this lane's group: a suffix sum over the lanes.
    unsigned int suf = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned int y = __shfl_down(suf, off);
      if (lane + off < 64) suf += y;
    }
    const unsigned long long k = *k_rem;
    const unsigned long long above = suf - c;
    const unsigned long long hit = __ballot(above < k && k <= above + c);
    const int grp = hit != 0ull ? __ffsll(static_cast<long long>(hit)) - 1 : 0;
    const unsigned long long k1 = k - static_cast<unsigned long long>(__shfl(suf - c, grp));
    // Lane l holds bins top - 2l and top - 2l - 1 of the group.
    const int bin_a = grp * kGroupBins + kGroupBins - 1 - 2 * lane;
    unsigned int fa = 0, fb = 0;
    unsigned int wa[R], wb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wa[r] = h[size_t(r) * kRep + bin_a];
      wb[r] = h[size_t(r) * kRep + bin_a - 1];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      fa += wa[r];
      fb += wb[r];
    }
    const unsigned int local = fa + fb;
    unsigned int inc = local;  // counts of this lane's bins and every higher one in the group
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    const unsigned long long before = inc - local;
    if (hit != 0ull && before < k1 && k1 <= before + local) {
      const bool top = k1 <= before + fa;
      *prefix |= static_cast<unsigned long long>(top ? bin_a : bin_a - 1) << digit_shift(pass);
      *k_rem = top ? k1 - before : k1 - before - fa;
    }
  }
  __syncthreads();
}

// Exclusive prefix sum over the workgroup's threads in thread order (s_wave: THREADS/64 words).
template <int THREADS>
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

// Given the histogram of digit `pass` over the keys that share k*'s higher digits (s_tot, in
// LDS), fix that digit: it is the bin, scanned from the top, in which the running count first
// reaches k_rem. Updates *prefix and *k_rem (LDS) for the whole workgroup.
template <int THREADS>
__device__ void select_digit(const unsigned int* s_tot, int pass, unsigned long long* prefix,
                             unsigned long long* k_rem) {
  __shared__ unsigned int s_wave[THREADS / 64];
  const int nb = 1 << digit_bits(pass);
  const int per = nb / THREADS;
  const int first = nb - 1 - int(threadIdx.x) * per;  // this thread's bins: first, first-1, ...
  unsigned int local = 0;
  for (int j = 0; j < per; ++j) local += s_tot[first - j];
  const unsigned int before = block_exclusive_scan<THREADS>(local, s_wave);
  const unsigned long long k = *k_rem;
  __syncthreads();
  if (before < k && k <= static_cast<unsigned long long>(before) + local) {
    unsigned long long acc = before;
    for (int j = 0; j < per; ++j) {
      const unsigned int c = s_tot[first - j];
      if (k <= acc + c) {
        *prefix |= static_cast<unsigned long long>(first - j) << digit_shift(pass);
        *k_rem = k - acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Clears the histograms. The passes histogram every entry, current positions included; to leave
// the pool's histogram, workgroup 0 starts replica 0 of the top-digit histogram (bins and
// groups) at minus the current positions' counts (unsigned wrap-around cancels exactly once
// they are added).
__global__ __launch_bounds__(256) void init_kernel(const Args a) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ unsigned int h[kBins];
  __shared__ unsigned int hg[kGroups];
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < kBins; i += 256) h[i] = 0u;
    if (threadIdx.x < kGroups) hg[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t rows = a.n / a.N;
    for (int64_t r = threadIdx.x; r < rows; r += 256) {
      const int d = top_digit(a.scores[r * a.row_stride + a.current]);
      atomicAdd(&h[d], 1u);
      atomicAdd(&hg[d / kGroupBins], 1u);  // group totals counted directly: summing 128
                                            // LDS words a thread would conflict on one bank
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBins; i += 256) a.hist0[i] = 0u - h[i];
    if (threadIdx.x < kGroups) a.hist0[kBins + threadIdx.x * kGroupStride] = 0u - hg[threadIdx.x];
    return;
  }
  const int i = int(blockIdx.x - 1) * 256 + int(threadIdx.x);  // one 16-byte piece past replica 0
  constexpr int kPieces = (kReplicas0 + kReplicas1 - 1) * kRep / 4;
  if (i < kPieces) reinterpret_cast<u32x4_t*>(a.hist0 + kRep)[i] = u32x4_t{0u, 0u, 0u, 0u};
}

// Pass 0: histogram of the top digit over the whole pool.
template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void pass0_kernel(const Args a) {
  __shared__ unsigned int h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kStreamThreads) h[i] = 0u;
  __syncthreads();
  for (int64_t base = int64_t(blockIdx.x) * kChunk; base < a.n; base += int64_t(gridDim.x) * kChunk) {
    float x[kSlabs][4];
    bool valid[kSlabs][4];
#pragma unroll
    for (int s = 0; s < kSlabs; ++s)
      load4<VEC>(a, base + s * (kStreamThreads * kVec) + int(threadIdx.x) * kVec, x[s], valid[s]);
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid[s][e]) atomicAdd(&h[top_digit(x[s][e])], 1u);
    }
  }
  __syncthreads();
  flush_hist<kStreamThreads>(h, a.hist0 + size_t(blockIdx.x % kReplicas0) * kRep);
}

// Pass 1: fixes k*'s top digit (every workgroup, identically), then the whole mask, list 1 in
// this workgroup's region and the histogram of the second digit over it.
template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void pass1_kernel(const Args a) {
  __shared__ unsigned int h[kBins];
  __shared__ unsigned long long s_prefix, s_k;
  __shared__ unsigned int s_n;
  for (int i = threadIdx.x; i < kBins; i += kStreamThreads) h[i] = 0u;
  if (threadIdx.x == 0) {
    s_prefix = 0ull;
    s_k = a.k;
    s_n = 0u;
  }
  __syncthreads();
  select_digit_global<kReplicas0>(a.hist0, 0, &s_prefix, &s_k);
  const int d0 = digit_of(s_prefix, 0);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.st->prefix0 = s_prefix;
    a.st->k_rem0 = s_k;
  }
  unsigned long long* region = a.list1 + int64_t(blockIdx.x) * a.cap1;
  for (int64_t base = int64_t(blockIdx.x) * kChunk; base < a.n; base += int64_t(gridDim.x) * kChunk) {
    float x[kSlabs][4];
    bool valid[kSlabs][4];
#pragma unroll
    for (int s = 0; s < kSlabs; ++s)
      load4<VEC>(a, base + s * (kStreamThreads * kVec) + int(threadIdx.x) * kVec, x[s], valid[s]);
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      const int64_t i0 = base + s * (kStreamThreads * kVec) + int(threadIdx.x) * kVec;
      uint32_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // Current positions get their 1 from the final kernel; only the rare entries that share
        // k*'s top digit check whether they are one (and then stay out of the lists).
        const int d = top_digit(x[s][e]);
        m[e] = valid[s][e] && d > d0 ? 1u : 0u;
        if (valid[s][e] && d == d0 && !is_current(a, i0 + e)) {
          const unsigned long long key = make_key(x[s][e], uint32_t(i0 + e));
          region[atomicAdd(&s_n, 1u)] = key;
          atomicAdd(&h[digit_of(key, 1)], 1u);
        }
      }
      if constexpr (VEC) {
        if (valid[s][0])
          *reinterpret_cast<uint32_t*>(a.keep + i0) = m[0] | (m[1] << 8) | (m[2] << 16) | (m[3] << 24);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (valid[s][e]) a.keep[i0 + e] = uint8_t(m[e]);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.count1[blockIdx.x] = s_n;
  flush_hist<kStreamThreads>(h, a.hist1 + size_t(blockIdx.x % kReplicas1) * kRep);
}

// List pass: every workgroup fixes k*'s second digit (identically), then walks the list-1
// regions r = blockIdx.x, blockIdx.x + gridDim.x, ...: entries above k*'s first two digits get
// a 1, entries sharing them go to this workgroup's list-2 region.
__global__ __launch_bounds__(kFinishThreads) void list_kernel(const Args a) {
  __shared__ unsigned long long s_prefix, s_k;
  __shared__ unsigned int s_n;
  if (threadIdx.x == 0) {
    s_prefix = a.st->prefix0;
    s_k = a.st->k_rem0;
    s_n = 0u;
  }
  __syncthreads();
  select_digit_global<kReplicas1>(a.hist1, 1, &s_prefix, &s_k);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.st->prefix1 = s_prefix;
    a.st->k_rem1 = s_k;
  }
  const unsigned long long want = s_prefix >> digit_shift(1);
  unsigned long long* region = a.list2 + int64_t(blockIdx.x) * a.cap2;
  for (int r = blockIdx.x; r < a.grid; r += gridDim.x) {
    const unsigned int count = a.count1[r];
    const unsigned long long* src = a.list1 + int64_t(r) * a.cap1;
    for (unsigned int j = threadIdx.x; j < count; j += kFinishThreads) {
      const unsigned long long key = src[j];
      const unsigned long long top = key >> digit_shift(1);
      if (top > want)
        a.keep[~static_cast<uint32_t>(key)] = 1u;
      else if (top == want)
        region[atomicAdd(&s_n, 1u)] = key;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.count2[blockIdx.x] = s_n;
}

// One workgroup finishes: digits 2 to 4 over list 2 (LDS histograms), then the list-2 entries
// at or above k* get a 1. List 2 is visited as one concatenated array: entry j lives in the
// region r with s_offs[r] <= j < s_offs[r + 1]; when it fits, it is first copied into LDS so
// that the three digit passes do not wait on global memory.
__global__ __launch_bounds__(kFinishThreads) void final_kernel(const Args a) {
  __shared__ unsigned int s_tot[kBins];
  __shared__ unsigned long long s_keys[kLdsKeys];
  __shared__ unsigned long long s_prefix, s_k;
  __shared__ unsigned int s_offs[kListGrid + 1];
  __shared__ unsigned int s_wave[kFinishThreads / 64];
  const unsigned int c = int(threadIdx.x) < a.list_grid ? a.count2[threadIdx.x] : 0u;
  const unsigned int off = block_exclusive_scan<kFinishThreads>(c, s_wave);
  if (int(threadIdx.x) < a.list_grid) s_offs[threadIdx.x] = off;
  if (int(threadIdx.x) == a.list_grid - 1) s_offs[a.list_grid] = off + c;
  if (threadIdx.x == 0) {
    s_prefix = a.st->prefix1;
    s_k = a.st->k_rem1;
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
    for (unsigned int j = threadIdx.x; j < total; j += kFinishThreads) s_keys[j] = global_entry(j);
    __syncthreads();
  }
  auto entry = [&](unsigned int j) { return staged ? s_keys[j] : global_entry(j); };
  if (total <= unsigned(kFinishThreads)) {
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
    for (int pass = 2; pass < 5; ++pass) {
      for (int b = threadIdx.x; b < kBins; b += kFinishThreads) s_tot[b] = 0u;
      __syncthreads();
      const int sh = digit_shift(pass - 1);
      const unsigned long long want = s_prefix >> sh;
      for (unsigned int j = threadIdx.x; j < total; j += kFinishThreads) {
        const unsigned long long key = entry(j);
        if ((key >> sh) == want) atomicAdd(&s_tot[digit_of(key, pass)], 1u);
      }
      __syncthreads();
      select_digit<kFinishThreads>(s_tot, pass, &s_prefix, &s_k);
    }
    const unsigned long long kstar = s_prefix;
    for (unsigned int j = threadIdx.x; j < total; j += kFinishThreads) {
      const unsigned long long key = entry(j);
      if (key >= kstar) a.keep[~static_cast<uint32_t>(key)] = 1u;
    }
  }
  // Rule 1: every row's current position stays (pass 1 gave it the value of its top digit).
  const int64_t rows = a.n / a.N;
  for (int64_t r = threadIdx.x; r < rows; r += kFinishThreads) a.keep[r * a.N + a.current] = 1u;
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
  g.list_grid = g.grid < kListGrid ? g.grid : kListGrid;
  g.cap2 = int64_t((g.grid + g.list_grid - 1) / g.list_grid) * g.cap1;
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
  a.N = p->num_tokens;
  a.current = p->current;
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
    a.hist0 = reinterpret_cast<unsigned int*>(ws + kStateBytes);
    a.hist1 = a.hist0 + size_t(kReplicas0) * kRep;
    a.count1 = reinterpret_cast<unsigned int*>(ws + kStateBytes + kHistBytes);
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
    hipLaunchKernelGGL(init_kernel,
                       dim3(1 + ((kReplicas0 + kReplicas1 - 1) * kRep / 4 + 255) / 256), dim3(256),
                       0, s, a);
    if (vec) {
      hipLaunchKernelGGL(pass0_kernel<true>, dim3(g.grid), dim3(kStreamThreads), 0, s, a);
      hipLaunchKernelGGL(pass1_kernel<true>, dim3(g.grid), dim3(kStreamThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL(pass0_kernel<false>, dim3(g.grid), dim3(kStreamThreads), 0, s, a);
      hipLaunchKernelGGL(pass1_kernel<false>, dim3(g.grid), dim3(kStreamThreads), 0, s, a);
    }
    hipLaunchKernelGGL(list_kernel, dim3(g.list_grid), dim3(kFinishThreads), 0, s, a);
    hipLaunchKernelGGL(final_kernel, dim3(1), dim3(kFinishThreads), 0, s, a);
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
