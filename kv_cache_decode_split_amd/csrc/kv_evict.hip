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
// radix selection, five digits of 13, 13, 13, 13 and 12 bits):
//
//   pass 0  every entry: histogram of the top digit; the last workgroup to finish finds the
//           digit of k* and the rank of k* among the entries that share it;
//   pass 1  every entry: writes the whole mask (current positions 1, entries whose top digit is
//           above k*'s 1, all others 0 for now) and sets the entries that share k*'s top digit
//           aside (their keys, in a workspace list) while histogramming their second digit;
//   pass 2-4  the set-aside entries only: one digit each;
//   patch   the set-aside entries whose key is at least k* get a 1.
//
// The two full passes stream the scores with coalesced 128-bit loads (HBM-bound: 8 bytes read
// and 1 written per entry); the rest touches only the set-aside entries, typically a small
// fraction of the pool (all of it only if nearly every score is equal). No ranking of the whole
// pool is ever materialised. Histograms live in LDS per workgroup and are added into global
// memory with device-scope atomics (bins that stayed zero are skipped); the last workgroup of
// each pass, detected with an arrival counter, reads the global histogram and fixes the digit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv_attn_internal.h"
#include "kv_evict.h"

namespace kvevict {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kVec = 4;                              // floats per 128-bit load
constexpr int kSlabs = 4;                            // loads per thread per iteration
constexpr int kChunk = kThreads * kVec * kSlabs;     // entries per workgroup iteration
constexpr int kBins = 8192;                          // 13-bit digits
constexpr int kPasses = 5;
constexpr int kMaxGrid = 2048;
constexpr int kListGrid = 256;                       // workgroups of the passes over the list
constexpr size_t kStateBytes = 256;
constexpr size_t kHistBytes = size_t(kPasses) * kBins * 4;

__host__ __device__ constexpr int digit_shift(int pass) { return pass < 4 ? 51 - 13 * pass : 0; }
__host__ __device__ constexpr int digit_bits(int pass) { return pass < 4 ? 13 : 12; }

struct State {
  unsigned long long prefix;     // digits of k* found so far, in place (lower bits 0)
  unsigned long long k_rem;      // rank of k* (1 = largest) among the keys sharing those digits
  unsigned int list_count;       // entries set aside by pass 1
  unsigned int arrived[kPasses]; // workgroups that finished each pass
};
static_assert(sizeof(State) <= kStateBytes, "state");

struct Args {
  const float* scores;
  uint8_t* keep;
  State* st;
  unsigned int* hist;            // [kPasses][kBins]
  unsigned long long* list;      // set-aside keys
  int64_t row_stride;
  int64_t n;                     // L*H*N < 2^31
  unsigned long long magic;      // row of flat index i: (i * magic) >> magic_shift
  int32_t magic_shift;
  int32_t N;
  int32_t current;
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

__device__ __forceinline__ int digit_of(unsigned long long key, int pass) {
  return int((key >> digit_shift(pass)) & ((1ull << digit_bits(pass)) - 1ull));
}

__device__ __forceinline__ void atomic_add_agent(unsigned int* p, unsigned int v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned int load_agent(const unsigned int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Four consecutive entries i0 .. i0+3 (i0 a multiple of 4). VEC: the four share a row and one
// aligned 128-bit load reads them. valid: inside the array; pool: valid and not the current
// position.
template <bool VEC>
__device__ __forceinline__ void load4(const Args& a, int64_t i0, float (&x)[4], bool (&valid)[4],
                                      bool (&pool)[4]) {
  if constexpr (VEC) {
    const bool in = i0 < a.n;
#pragma unroll
    for (int e = 0; e < 4; ++e) valid[e] = in;
    if (in) {
      const int row = row_of(a, i0);
      const int t0 = int(i0 - int64_t(row) * a.N);
      const f32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t*>(a.scores + int64_t(row) * a.row_stride + t0));
      x[0] = v[0];
      x[1] = v[1];
      x[2] = v[2];
      x[3] = v[3];
#pragma unroll
      for (int e = 0; e < 4; ++e) pool[e] = t0 + e != a.current;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = 0.f;
        pool[e] = false;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      valid[e] = i < a.n;
      x[e] = 0.f;
      pool[e] = false;
      if (valid[e]) {
        const int row = row_of(a, i);
        const int t = int(i - int64_t(row) * a.N);
        x[e] = a.scores[int64_t(row) * a.row_stride + t];
        pool[e] = t != a.current;
      }
    }
  }
}

// Exclusive prefix sum over the workgroup's threads, in thread order.
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

// Run by the whole last workgroup of a pass: the digit of k* is the bin, scanned from the top,
// in which the running count first reaches k_rem.
__device__ void find_digit(const Args& a, int pass) {
  __shared__ unsigned int s_wave[kThreads / 64];
  const unsigned int* h = a.hist + size_t(pass) * kBins;
  const int nb = 1 << digit_bits(pass);
  const int per = nb / kThreads;
  const int first = nb - 1 - int(threadIdx.x) * per;  // this thread's bins: first, first-1, ...
  unsigned int local = 0;
  for (int j = 0; j < per; ++j) local += load_agent(h + (first - j));
  const unsigned int before = block_exclusive_scan(local, s_wave);
  const unsigned long long k = a.st->k_rem;
  if (before < k && k <= static_cast<unsigned long long>(before) + local) {
    unsigned long long acc = before;
    for (int j = 0; j < per; ++j) {
      const unsigned int c = load_agent(h + (first - j));
      if (k <= acc + c) {
        a.st->prefix |= static_cast<unsigned long long>(first - j) << digit_shift(pass);
        a.st->k_rem = k - acc;
        break;
      }
      acc += c;
    }
  }
}

// End of a histogram pass: publish this workgroup's counts, count arrivals; the last workgroup
// to arrive fixes the digit.
__device__ void finish_pass(const Args& a, int pass, const unsigned int* h_lds) {
  __shared__ unsigned int s_last;
  unsigned int* h = a.hist + size_t(pass) * kBins;
  const int nb = 1 << digit_bits(pass);
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    const unsigned int c = h_lds[i];
    if (c != 0u) atomic_add_agent(h + i, c);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int prev =
        __hip_atomic_fetch_add(&a.st->arrived[pass], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == gridDim.x - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0u) return;
  __threadfence();
  find_digit(a, pass);
}

__global__ __launch_bounds__(kThreads) void init_kernel(const Args a) {
  const int i = int(blockIdx.x) * kThreads + int(threadIdx.x);
  if (i < kPasses * kBins) a.hist[i] = 0u;
  if (i == 0) {
    a.st->prefix = 0ull;
    a.st->k_rem = a.k;
    a.st->list_count = 0u;
    for (int p = 0; p < kPasses; ++p) a.st->arrived[p] = 0u;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void pass0_kernel(const Args a) {
  __shared__ unsigned int h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
  __syncthreads();
  for (int64_t base = int64_t(blockIdx.x) * kChunk; base < a.n; base += int64_t(gridDim.x) * kChunk) {
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      const int64_t i0 = base + s * (kThreads * kVec) + int(threadIdx.x) * kVec;
      float x[4];
      bool valid[4], pool[4];
      load4<VEC>(a, i0, x, valid, pool);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pool[e]) atomicAdd(&h[digit_of(make_key(x[e], uint32_t(i0 + e)), 0)], 1u);
    }
  }
  __syncthreads();
  finish_pass(a, 0, h);
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void pass1_kernel(const Args a) {
  __shared__ unsigned int h[kBins];
  __shared__ unsigned long long s_list[kChunk];
  __shared__ unsigned int s_n, s_base;
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
  const int d0 = digit_of(a.st->prefix, 0);
  for (int64_t base = int64_t(blockIdx.x) * kChunk; base < a.n; base += int64_t(gridDim.x) * kChunk) {
    if (threadIdx.x == 0) s_n = 0u;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      const int64_t i0 = base + s * (kThreads * kVec) + int(threadIdx.x) * kVec;
      float x[4];
      bool valid[4], pool[4];
      load4<VEC>(a, i0, x, valid, pool);
      uint32_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = valid[e] ? 1u : 0u;  // current positions stay
        if (pool[e]) {
          const unsigned long long key = make_key(x[e], uint32_t(i0 + e));
          const int d = digit_of(key, 0);
          m[e] = d > d0 ? 1u : 0u;
          if (d == d0) {
            const unsigned int pos = atomicAdd(&s_n, 1u);
            s_list[pos] = key;
            atomicAdd(&h[digit_of(key, 1)], 1u);
          }
        }
      }
      if constexpr (VEC) {
        if (valid[0])
          *reinterpret_cast<uint32_t*>(a.keep + i0) = m[0] | (m[1] << 8) | (m[2] << 16) | (m[3] << 24);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (valid[e]) a.keep[i0 + e] = uint8_t(m[e]);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && s_n != 0u)
      s_base = __hip_atomic_fetch_add(&a.st->list_count, s_n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    for (unsigned int j = threadIdx.x; j < s_n; j += kThreads) a.list[s_base + j] = s_list[j];
    __syncthreads();
  }
  __syncthreads();
  finish_pass(a, 1, h);
}

// Passes 2..4: histogram of digit `pass` over the set-aside keys that still share k*'s digits.
__global__ __launch_bounds__(kThreads) void list_pass_kernel(const Args a, int pass) {
  __shared__ unsigned int h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
  __syncthreads();
  const int sh = digit_shift(pass - 1);
  const unsigned long long want = a.st->prefix >> sh;
  const unsigned int count = a.st->list_count;
  for (unsigned int j = blockIdx.x * kThreads + threadIdx.x; j < count; j += gridDim.x * kThreads) {
    const unsigned long long key = a.list[j];
    if ((key >> sh) == want) atomicAdd(&h[digit_of(key, pass)], 1u);
  }
  __syncthreads();
  finish_pass(a, pass, h);
}

// The set-aside entries at or above k* stay.
__global__ __launch_bounds__(kThreads) void patch_kernel(const Args a) {
  const unsigned long long kstar = a.st->prefix;
  const unsigned int count = a.st->list_count;
  for (unsigned int j = blockIdx.x * kThreads + threadIdx.x; j < count; j += gridDim.x * kThreads) {
    const unsigned long long key = a.list[j];
    if (key >= kstar) a.keep[~static_cast<uint32_t>(key)] = 1u;
  }
}

// The budget alone decides: all = 0 keeps only the current positions, all = 1 keeps everything.
__global__ __launch_bounds__(kThreads) void fill_kernel(const Args a, int all) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < a.n;
       i += int64_t(gridDim.x) * kThreads) {
    const int row = row_of(a, i);
    const int t = int(i - int64_t(row) * a.N);
    a.keep[i] = (all != 0 || t == a.current) ? 1u : 0u;
  }
}

// kept_per_row[r] = number of ones in row r of the mask.
__global__ __launch_bounds__(kThreads) void row_count_kernel(const uint8_t* keep, int32_t N,
                                                             int32_t* out) {
  __shared__ unsigned int s_wave[kThreads / 64];
  const uint8_t* row = keep + int64_t(blockIdx.x) * N;
  unsigned int c = 0;
  for (int t = threadIdx.x; t < N; t += kThreads) c += row[t];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned int total = 0;
    for (int w = 0; w < kThreads / 64; ++w) total += s_wave[w];
    out[blockIdx.x] = int32_t(total);
  }
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
  return kStateBytes + kHistBytes + size_t(pool_size(p)) * 8u;
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
  Args a;
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
  char* ws = static_cast<char*>(workspace);
  a.st = rank ? reinterpret_cast<State*>(ws) : nullptr;
  a.hist = rank ? reinterpret_cast<unsigned int*>(ws + kStateBytes) : nullptr;
  a.list = rank ? reinterpret_cast<unsigned long long*>(ws + kStateBytes + kHistBytes) : nullptr;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t chunks = (a.n + kChunk - 1) / kChunk;
  const uint32_t grid = uint32_t(chunks < kMaxGrid ? chunks : kMaxGrid);
  if (!rank) {
    const int all = free_slots(p) > 0 ? 1 : 0;  // K >= pool: everything stays
    const int64_t blocks = (a.n + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(fill_kernel, dim3(uint32_t(blocks < kMaxGrid ? blocks : kMaxGrid)),
                       dim3(kThreads), 0, s, a, all);
    if (hipGetLastError() != hipSuccess) return KV_ATTN_ERR_HIP;
  } else {
    const bool vec = p->num_tokens % 4 == 0 && p->row_stride % 4 == 0 && aligned(scores, 16) &&
                     aligned(keep, 4);
    hipLaunchKernelGGL(init_kernel, dim3((kPasses * kBins + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, s, a);
    if (vec) {
      hipLaunchKernelGGL(pass0_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL(pass1_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL(pass0_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL(pass1_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a);
    }
    for (int pass = 2; pass < kPasses; ++pass)
      hipLaunchKernelGGL(list_pass_kernel, dim3(kListGrid), dim3(kThreads), 0, s, a, pass);
    hipLaunchKernelGGL(patch_kernel, dim3(kListGrid), dim3(kThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return KV_ATTN_ERR_HIP;
  }
  if (kept_per_row != nullptr) {
    hipLaunchKernelGGL(row_count_kernel, dim3(uint32_t(rows)), dim3(kThreads), 0, s, keep,
                       p->num_tokens, kept_per_row);
    if (hipGetLastError() != hipSuccess) return KV_ATTN_ERR_HIP;
  }
  return KV_ATTN_OK;
}

}  // extern "C"
