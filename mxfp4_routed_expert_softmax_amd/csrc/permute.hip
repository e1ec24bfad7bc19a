// Bucketing of (token, slot) pairs by expert: a stable counting sort built
// from per-chunk counts and prefix sums, with no atomics anywhere, so the
// row order is a pure function of the ids. (The pages trace irreproducible
// runs to slot assignment that depends on I/O timing: ai.rs article on
// DeepSeek-V4.1-Flash, "What remains is the reference rounding itself".)
//
// Pairs are processed in chunks of kPermuteChunk. A workgroup sorts its
// chunk in LDS by the key (expert << 11 | index in chunk) with a bitonic
// network: keys are unique, so the order within an expert is pair order.
// An expert's pairs then sit in one run of the sorted chunk; the run's start
// and length give the chunk's count of that expert, and a pair's rank among
// the chunk's pairs of its expert is its distance from the run's start.
// Bucket bases come from a column prefix over chunks plus an exclusive scan
// over experts. Ids outside [0, E) sort after every valid key and own no row.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kPermThreads = 1024;  // >= E (E <= 1024)

// Sorts the chunk's keys into s_key[0..kPermuteChunk) (padding sorts last)
// and records in s_start[e] the sorted position where expert e's run starts
// and in s_cnt[e] its length (0 for experts absent from the chunk).
// Uniform control flow (barriers).
__device__ void sort_chunk(const int32_t* ids, int p0, int n, int E, uint32_t* s_key, int* s_start,
                           int* s_cnt) {
  for (int p = threadIdx.x; p < kPermuteChunk; p += blockDim.x) {
    uint32_t key = 0xffffffffu;
    if (p < n) {
      const int id = ids[p0 + p];
      const uint32_t e = (id < 0 || id >= E) ? (uint32_t)E : (uint32_t)id;
      key = (e << 11) | (uint32_t)p;
    }
    s_key[p] = key;
  }
  for (int e = threadIdx.x; e <= E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  for (int size = 2; size <= kPermuteChunk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < kPermuteChunk / 2; t += blockDim.x) {
        const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
        const uint32_t x = s_key[lo], y = s_key[hi];
        if ((x > y) == ((lo & size) == 0)) {
          s_key[lo] = y;
          s_key[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  // run boundaries of the valid experts
  for (int q = threadIdx.x; q < n; q += blockDim.x) {
    const int e = (int)(s_key[q] >> 11);
    if (e < E && (q == 0 || (int)(s_key[q - 1] >> 11) != e)) s_start[e] = q;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < n; q += blockDim.x) {
    const int e = (int)(s_key[q] >> 11);
    if (e < E && (q == n - 1 || (int)(s_key[q + 1] >> 11) != e)) s_cnt[e] = q + 1 - s_start[e];
  }
  __syncthreads();
}

// Writes the rows of the chunk's sorted valid pairs: pair p0 + p of expert e
// at sorted position q goes to row base_of(e) + q - s_start[e].
template <class Base>
__device__ __forceinline__ void scatter_sorted(const uint32_t* s_key, const int* s_start, int n,
                                               int E, int p0, int k, Base base_of,
                                               int32_t* row_token, int32_t* inv_row) {
  for (int q = threadIdx.x; q < n; q += blockDim.x) {
    const uint32_t key = s_key[q];
    const int e = (int)(key >> 11);
    if (e >= E) continue;
    const int gp = p0 + (int)(key & 2047u);
    const int pos = base_of(e) + q - s_start[e];
    row_token[pos] = gp / k;
    inv_row[gp] = pos;
  }
}

// Writes offsets[0..E], the active list and returns this thread's bucket
// base. Uniform control flow (contains barriers).
__device__ __forceinline__ int offsets_and_active(int e, int E, int total_e, int* s_tmp,
                                                  int32_t* offsets, int32_t* active) {
  int tot = 0;
  const int cnt = (e < E) ? total_e : 0;
  const int base = block_exclusive_scan(cnt, s_tmp, &tot);
  if (e < E) offsets[e] = base;
  if (e == 0) offsets[E] = tot;
  int n_active = 0;
  const int is_act = (e < E && cnt > 0) ? 1 : 0;
  const int slot = block_exclusive_scan(is_act, s_tmp, &n_active);
  if (active != nullptr && e < E) {
    if (is_act) active[slot] = e;
    if (e >= n_active) active[e] = -1;
  }
  return base;
}

// R <= kPermuteChunk: one workgroup does everything.
__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row, int32_t* __restrict__ active) {
  __shared__ uint32_t s_key[kPermuteChunk];
  __shared__ int s_start[1025], s_cnt[1025], s_base[1025];
  __shared__ int s_tmp[32];
  const int e = threadIdx.x;
  sort_chunk(ids, 0, R, E, s_key, s_start, s_cnt);
  const int base = offsets_and_active(e, E, e < E ? s_cnt[e] : 0, s_tmp, offsets, active);
  if (e < E) s_base[e] = base;
  __syncthreads();
  scatter_sorted(s_key, s_start, R, E, 0, k, [&](int ex) { return s_base[ex]; }, row_token,
                 inv_row);
  for (int p = threadIdx.x; p < R; p += blockDim.x) {
    const int id = ids[p];
    if (id < 0 || id >= E) inv_row[p] = -1;
  }
}

// Large R, pass 1: counts[c][e] of chunk c.
__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ counts) {
  __shared__ uint32_t s_key[kPermuteChunk];
  __shared__ int s_start[1025], s_cnt[1025];
  const int p0 = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, R - p0);
  sort_chunk(ids, p0, n, E, s_key, s_start, s_cnt);
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// Pass 2 (one workgroup): counts[c][e] <- global row where chunk c's rows of
// expert e start; offsets and the active list.
__global__ __launch_bounds__(kPermThreads) void permute_scan_kernel(
    int nchunks, int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active) {
  __shared__ int s_tmp[32];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      const int v = counts[(size_t)c * E + e];
      counts[(size_t)c * E + e] = run;
      run += v;
    }
  }
  const int base = offsets_and_active(e, E, run, s_tmp, offsets, active);
  if (e < E)
    for (int c = 0; c < nchunks; ++c) counts[(size_t)c * E + e] += base;
}

// Pass 3: every chunk sorts again and writes its rows.
__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, const int32_t* __restrict__ counts,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row) {
  __shared__ uint32_t s_key[kPermuteChunk];
  __shared__ int s_start[1025], s_cnt[1025];
  const int p0 = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, R - p0);
  sort_chunk(ids, p0, n, E, s_key, s_start, s_cnt);
  const int32_t* base = counts + (size_t)blockIdx.x * E;
  scatter_sorted(s_key, s_start, n, E, p0, k, [&](int ex) { return base[ex]; }, row_token, inv_row);
  for (int p = threadIdx.x; p < n; p += blockDim.x) {
    const int id = ids[p0 + p];
    if (id < 0 || id >= E) inv_row[p0 + p] = -1;
  }
}

size_t permute_ws_bytes(int T, int k, int E) {
  const long long R = (long long)T * k;
  if (R <= kPermuteChunk) return 0;
  const long long nchunks = (R + kPermuteChunk - 1) / kPermuteChunk;
  return (size_t)(nchunks * E * sizeof(int32_t));
}

void launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                    int32_t* row_token, int32_t* inv_row, int32_t* active, void* ws,
                    hipStream_t s) {
  const int R = T * k;
  if (R <= kPermuteChunk) {
    launch("permute_small_kernel", permute_small_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, R, k, E,
                       offsets, row_token, inv_row, active);
    return;
  }
  const int nchunks = (R + kPermuteChunk - 1) / kPermuteChunk;
  int32_t* counts = static_cast<int32_t*>(ws);
  launch("permute_count_kernel", permute_count_kernel, dim3(nchunks), dim3(kPermThreads), 0, s, ids, R, E,
                     counts);
  launch("permute_scan_kernel", permute_scan_kernel, dim3(1), dim3(kPermThreads), 0, s, nchunks, E, counts,
                     offsets, active);
  launch("permute_scatter_kernel", permute_scatter_kernel, dim3(nchunks), dim3(kPermThreads), 0, s, ids, R, k,
                     E, counts, row_token, inv_row);
}

}  // namespace moe
