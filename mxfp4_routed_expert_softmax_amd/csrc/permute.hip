// Bucketing of (token, slot) pairs by expert: a stable counting sort built
// from per-chunk counts and prefix sums, with no atomics anywhere, so the
// row order is a pure function of the ids. (The pages trace irreproducible
// runs to slot assignment that depends on I/O timing: ai.rs article on
// DeepSeek-V4.1-Flash, "What remains is the reference rounding itself".)
//
// Pairs are processed in chunks of kPermuteChunk. Thread e of a workgroup
// owns expert e: it counts the chunk's pairs with id e by walking the chunk
// in LDS (every thread reads the same word at once, an LDS broadcast), and
// later walks it again to write its rows in pair order. Bucket bases come
// from a column prefix over chunks plus an exclusive scan over experts.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kPermThreads = 1024;  // >= E (E <= 1024)

__device__ __forceinline__ int count_in_chunk(const int* s_ids, int n, int e) {
  int c = 0;
  const int n4 = n & ~3;
  for (int p = 0; p < n4; p += 4) {
    const int4 v = *reinterpret_cast<const int4*>(s_ids + p);
    c += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
  }
  for (int p = n4; p < n; ++p) c += (s_ids[p] == e);
  return c;
}

__device__ __forceinline__ void scatter_chunk(const int* s_ids, int n, int e, int pos, int base_p,
                                              int k, int32_t* row_token, int32_t* inv_row) {
  for (int p = 0; p < n; ++p) {
    if (s_ids[p] == e) {
      const int gp = base_p + p;
      row_token[pos] = gp / k;
      inv_row[gp] = pos;
      ++pos;
    }
  }
}

__device__ __forceinline__ void load_chunk(int* s_ids, const int32_t* ids, int p0, int n) {
  for (int p = threadIdx.x; p < n; p += blockDim.x) s_ids[p] = ids[p0 + p];
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

__device__ __forceinline__ void mark_invalid(const int* s_ids, int n, int E, int base_p,
                                             int32_t* inv_row) {
  for (int p = threadIdx.x; p < n; p += blockDim.x) {
    const int id = s_ids[p];
    if (id < 0 || id >= E) inv_row[base_p + p] = -1;
  }
}

// R <= kPermuteChunk: one workgroup does everything.
__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row, int32_t* __restrict__ active) {
  __shared__ __align__(16) int s_ids[kPermuteChunk];
  __shared__ int s_tmp[32];
  const int e = threadIdx.x;
  load_chunk(s_ids, ids, 0, R);
  __syncthreads();
  const int cnt = (e < E) ? count_in_chunk(s_ids, R, e) : 0;
  const int base = offsets_and_active(e, E, cnt, s_tmp, offsets, active);
  if (e < E && cnt > 0) scatter_chunk(s_ids, R, e, base, 0, k, row_token, inv_row);
  mark_invalid(s_ids, R, E, 0, inv_row);
}

// Large R, pass 1: counts[c][e] of chunk c.
__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ counts) {
  __shared__ __align__(16) int s_ids[kPermuteChunk];
  const int p0 = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, R - p0);
  load_chunk(s_ids, ids, p0, n);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    counts[(size_t)blockIdx.x * E + e] = count_in_chunk(s_ids, n, e);
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

// Pass 3: every chunk writes its rows.
__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, const int32_t* __restrict__ counts,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row) {
  __shared__ __align__(16) int s_ids[kPermuteChunk];
  const int p0 = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, R - p0);
  load_chunk(s_ids, ids, p0, n);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    scatter_chunk(s_ids, n, e, counts[(size_t)blockIdx.x * E + e], p0, k, row_token, inv_row);
  mark_invalid(s_ids, n, E, p0, inv_row);
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
