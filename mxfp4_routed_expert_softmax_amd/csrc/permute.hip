// Bucketing of (token, slot) pairs by expert: a stable counting sort built
// from per-chunk counts and prefix sums. No atomic decides an order (the
// chunk counts are LDS atomic adds, whose sums do not depend on their
// order), so the row order is a pure function of the ids. (The pages trace
// irreproducible runs to slot assignment that depends on I/O timing: ai.rs
// article on DeepSeek-V4.1-Flash, "What remains is the reference rounding
// itself".)
//
// Pairs are processed in chunks of kPermuteChunk; a wave takes 128
// consecutive pairs, two per lane (lane l holds pairs l and 64 + l of its
// 128). One ballot per bit of the expert ids (10 bits, E <= 1024) for each
// half lets every lane find the wave's pairs with its expert as the lanes
// that agree with it on every bit: their count below it is its rank among
// the wave's pairs of that expert, and their total the wave's count of it,
// stored in an LDS row of the wave's own. A column prefix over the waves
// then gives each wave's count of earlier pairs per expert, so a pair's
// rank in the chunk is that count plus its rank in the wave, in pair order.
// The scatter pass ranks each chunk in four parts of 512 pairs, one
// workgroup each, which add the counts of the chunk's earlier parts (an LDS
// histogram). Bucket bases come from a column prefix over chunks plus an
// exclusive scan over experts. Ids outside [0, E) own no row.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kPermThreads = 1024;  // >= E (E <= 1024); 16 waves of 128 pairs
constexpr int kPermWaves = kPermThreads / kWave;
static_assert(kPermWaves * 2 * kWave == kPermuteChunk, "two pairs per lane");
// The scatter pass ranks a chunk in kPermSub parts of 4 waves (512 pairs),
// each taking the counts of the chunk's earlier parts from an LDS histogram.
constexpr int kPermSub = 4;
constexpr int kPermSubWaves = kPermWaves / kPermSub;

// Ranks of the chunk's pairs p0 .. p0 + n - 1: lane l of wave w holds pairs
// 128 w + 64 i + l (i = 0, 1) with expert e[i] (-1 if invalid) and rank[i]
// among the chunk's earlier pairs of that expert. s_wc[w * (E + 1) + e]
// ends as the pairs of expert e in waves before w, s_cnt[e] as the chunk's
// count. NW waves (blockDim = 64 NW). Uniform control flow (barriers).
template <int NW>
__device__ void rank_chunk(const int32_t* ids, int p0, int n, int E, int* s_wc, int* s_cnt,
                           int (&e)[2], int (&rank)[2]) {
  const int lane = lane_id(), w = threadIdx.x / kWave, stride = E + 1;
  for (int q = threadIdx.x; q < NW * stride; q += blockDim.x) s_wc[q] = 0;
  __syncthreads();
  int* row = s_wc + w * stride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 2 * kWave * w + kWave * i + lane;
    int ex = -1;
    if (p < n) {
      const int id = ids[p0 + p];
      ex = (id < 0 || id >= E) ? -1 : id;
    }
    e[i] = ex;
    rank[i] = -1;
  }
  constexpr int kBits = 10;  // E <= 1024
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t val0 = __ballot(e[0] >= 0), val1 = __ballot(e[1] >= 0);
  uint64_t b0[kBits], b1[kBits];
#pragma unroll
  for (int b = 0; b < kBits; ++b) {
    b0[b] = __ballot((e[0] >> b) & 1);
    b1[b] = __ballot((e[1] >> b) & 1);
  }
  // the lanes of one half whose ids equal x
  auto match = [&](int x, const uint64_t (&bb)[kBits], uint64_t valid) {
    uint64_t m = valid;
#pragma unroll
    for (int b = 0; b < kBits; ++b) m &= ((x >> b) & 1) ? bb[b] : ~bb[b];
    return m;
  };
  if (e[0] >= 0) {
    const uint64_t m00 = match(e[0], b0, val0);
    rank[0] = __popcll(m00 & below);
    row[e[0]] = __popcll(m00) + __popcll(match(e[0], b1, val1));
  }
  if (e[1] >= 0) {
    const uint64_t m10 = match(e[1], b0, val0), m11 = match(e[1], b1, val1);
    rank[1] = __popcll(m10) + __popcll(m11 & below);
    row[e[1]] = __popcll(m10) + __popcll(m11);
  }
  __syncthreads();
  for (int x = threadIdx.x; x < E; x += blockDim.x) {
    int run = 0;
    for (int v = 0; v < NW; ++v) {
      const int c = s_wc[v * stride + x];
      s_wc[v * stride + x] = run;
      run += c;
    }
    s_cnt[x] = run;
  }
  __syncthreads();
}

// Writes the rows of the lane's two pairs: pair p0 + p of expert e goes to
// row base_of(e) + (its wave's earlier count) + rank; invalid pairs get
// inv_row -1.
template <class Base>
__device__ __forceinline__ void scatter_ranked(const int* s_wc, int E, int p0, int n, int k,
                                               const int (&e)[2], const int (&rank)[2],
                                               Base base_of, int32_t* row_token,
                                               int32_t* inv_row) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 2 * kWave * w + kWave * i + lane;
    if (p >= n) continue;
    const int gp = p0 + p;
    if (e[i] < 0) {
      inv_row[gp] = -1;
      continue;
    }
    const int pos = base_of(e[i]) + s_wc[w * (E + 1) + e[i]] + rank[i];
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

// LDS of the ranking: one row of E + 1 counts per wave, and the counts.
constexpr int kPermWcInts = kPermWaves * 1025;

// R <= kPermuteChunk: one workgroup does everything.
__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row, int32_t* __restrict__ active) {
  __shared__ int s_wc[kPermWcInts];
  __shared__ int s_cnt[1025], s_base[1025];
  __shared__ int s_tmp[32];
  const int x = threadIdx.x;
  int e[2], rank[2];
  rank_chunk<kPermWaves>(ids, 0, R, E, s_wc, s_cnt, e, rank);
  const int base = offsets_and_active(x, E, x < E ? s_cnt[x] : 0, s_tmp, offsets, active);
  if (x < E) s_base[x] = base;
  __syncthreads();
  scatter_ranked(s_wc, E, 0, R, k, e, rank, [&](int ex) { return s_base[ex]; }, row_token,
                 inv_row);
}

// Large R, pass 1: counts[c][e] of chunk c (an LDS histogram).
__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ counts) {
  __shared__ int s_cnt[1025];
  const int p0 = blockIdx.x * kPermuteChunk;
  const int n = min(kPermuteChunk, R - p0);
  for (int x = threadIdx.x; x < E; x += blockDim.x) s_cnt[x] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < n; p += blockDim.x) {
    const int id = ids[p0 + p];
    if (id >= 0 && id < E) atomicAdd(s_cnt + id, 1);
  }
  __syncthreads();
  for (int x = threadIdx.x; x < E; x += blockDim.x) counts[(size_t)blockIdx.x * E + x] = s_cnt[x];
}

// Pass 2 (one workgroup): counts[c][e] <- global row where chunk c's rows of
// expert e start; offsets and the active list.
__global__ __launch_bounds__(kPermThreads) void permute_scan_kernel(
    int nchunks, int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active) {
  __shared__ int s_tmp[32];
  const int e = threadIdx.x;
  // chunk counts are read 16 at a time, all 16 loads in flight together
  constexpr int kB = 16;
  int run = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) v[i] = c0 + i < nchunks ? counts[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kB; ++i) run += v[i];
    }
  }
  const int base = offsets_and_active(e, E, run, s_tmp, offsets, active);
  if (e < E) {
    int acc = base;
    for (int c0 = 0; c0 < nchunks; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) v[i] = c0 + i < nchunks ? counts[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        if (c0 + i < nchunks) counts[(size_t)(c0 + i) * E + e] = acc;
        acc += v[i];
      }
    }
  }
}

// Pass 3: part s of chunk c ranks its 512 pairs and writes their rows after
// the chunk's rows of the parts before it (counted in an LDS histogram).
__global__ __launch_bounds__(kPermSubWaves * kWave) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, const int32_t* __restrict__ counts,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row) {
  __shared__ int s_wc[kPermSubWaves * 1025];
  __shared__ int s_cnt[1025], s_pre[1025];
  const int c = blockIdx.x / kPermSub, sub = blockIdx.x % kPermSub;
  const int pc = c * kPermuteChunk, p0 = pc + sub * (kPermuteChunk / kPermSub);
  const int n = min(kPermuteChunk / kPermSub, R - p0);
  if (n <= 0) return;
  for (int x = threadIdx.x; x < E; x += blockDim.x) s_pre[x] = 0;
  __syncthreads();
  for (int p = pc + (int)threadIdx.x; p < p0; p += blockDim.x) {
    const int id = ids[p];
    if (id >= 0 && id < E) atomicAdd(s_pre + id, 1);
  }
  int e[2], rank[2];
  rank_chunk<kPermSubWaves>(ids, p0, n, E, s_wc, s_cnt, e, rank);  // its barriers cover s_pre
  const int32_t* base = counts + (size_t)c * E;
  scatter_ranked(s_wc, E, p0, n, k, e, rank, [&](int ex) { return base[ex] + s_pre[ex]; },
                 row_token, inv_row);
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
  launch("permute_scatter_kernel", permute_scatter_kernel, dim3(nchunks * kPermSub),
         dim3(kPermSubWaves * kWave), 0, s, ids, R, k, E, counts, row_token, inv_row);
}

}  // namespace moe
