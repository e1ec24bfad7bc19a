// The layer for a few tokens (decode, verification blocks). One token runs
// in two launches: the router rows, the routing wave, the shared expert and
// the routed gate/up stream share the first, and the routed down rows with
// the combine make the second. Verification blocks of 2-5 or 8 tokens run
// the block kernels further down, which follow the same plan over the
// union of the block's experts. Other counts up to 16 run the three-launch
// chain below, whose layout the other two forms grew from.
//
// Decode moves ~132 MB of expert weights per token, about 17 us of HBM time
// at 8 TB/s; the pages' own decode model is bandwidth over routed expert
// bytes per token (FreeToken issue #444, janit's comment, section 1), and a
// verification block pays for the union of its tokens' experts (ai.rs
// article on DeepSeek-V4.1-Flash, "The draft head that works and does not
// pay"). Every launch boundary costs a few microseconds, and inside a launch
// what costs is any chain of dependent round trips a workgroup waits
// through. So:
//
//   route   [router rows][routing][shared expert gate/up]
//   gate/up [routed gate/up items][shared expert down]
//   down    [routed down items; the last one per column also combines]
//
// The shared expert needs no routing, so its gate/up streams while the
// router and the top-k run, and its down streams with the routed gate/up.
// Within `route`, the routing workgroup waits for the router workgroups'
// flags; those have lower indices, and the dispatcher starts workgroups in
// index order, so they have started and finish: no deadlock whatever the
// occupancy. A flag holds a 48-bit tag unique to the call, so the
// workspace needs no initialisation; the wait is bounded (on timeout it
// records the failure in the workspace's status word and goes on with
// whatever logits it has, which cannot make an access go out of bounds;
// the call's last launch then fills the outputs with NaN and -1, so a
// timed-out call never returns plausible numbers). Data crossing
// workgroups inside a launch (logits, y rows for the combine) moves through
// agent-scope relaxed atomics, which are performed at the device coherence
// point, and a producer drains its stores (s_waitcnt) before it raises a
// flag or bumps a counter, so no cache-wide fence is needed. Data crossing a
// launch boundary uses plain loads and stores.
//
// Gate/up and down items are one-shot workgroups: weight loads first (one
// batch covers a whole row), then the activations, then the math; nothing
// waits for another workgroup. The down workgroup that finishes a column of
// 32 outputs last (a per-column counter, zeroed by `route`) sums that
// column's shared row and its k routed rows in the fixed order
// y_shared + w_0 y_0 + ... + w_{k-1} y_{k-1}.
//
// moe_expert_ffn_mxfp4 with few rows reuses the gate/up and down kernels
// behind a one-workgroup kernel that turns caller offsets into the slot
// table.
#include <unistd.h>

#include <atomic>
#include <chrono>

#include "moe_device.h"
#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMT = 4;          // token rows staged per pass
constexpr int kGuLanes = 32;    // gate/up: 32 lanes per row, 2 rows per wave
constexpr int kGuRows = 8;      // gate/up rows per item
constexpr int kGuU = 5;         // gate/up chunks per lane per batch (K = 5120 in one)
constexpr int kDnRows = 32;     // down: 8 lanes per row, 8 rows per wave
constexpr int kDnU = 9;         // down chunks per lane per batch (K = 2304 in one)
constexpr int kReplicas = 16;        // copies of the one-token routing table
constexpr int kReplicaWords = 512;   // 4 KB apart, so readers spread over channels
// Words of a replica: [0, k) the chosen ids, [kRepWeights, + 2k) the
// routing weights' low and high halves.
constexpr int kRepWeights = 64;
constexpr int kRouterV = 16;    // router: 16-byte vectors per lane (H <= 8192)
constexpr long kSpinLimit = 1L << 20;  // polls (with s_sleep) before giving up
// A tagged word: the call's 48-bit tag above a 16-bit payload. A reader
// takes a word as this call's only if it carries the tag, so a stale word
// from an earlier call (a different tag) or foreign bytes in a fresh
// workspace (a chance of 2^-48 per word) are never taken for new data.
constexpr int kTagShift = 16;
// Codes of the waits, recorded in the status word when one gives up.
constexpr uint32_t kWaitRouterFlags = 1;  // chain routing: router flags
constexpr uint32_t kWaitLogits = 2;       // routing: tagged logits
constexpr uint32_t kWaitTable = 3;        // one-token gate/up: routing table copy
constexpr uint32_t kWaitShared = 4;       // one-token shared down: shared gate/up flags
constexpr uint32_t kWaitGateup = 5;       // one-token routed down: the slot's gate/up items
constexpr uint32_t kWaitDown = 6;         // block combine: the routed y words
// Result word of a few-token call: this magic above the call's 48-bit tag.
// The call's status is the code of the status word when that word carries
// the same tag, else OK.
constexpr uint64_t kResultMagic = 0x5741u;

constexpr int kLdsGu = kMT * kGuLanes * kGuU * 64;  // bf16 x chunks
constexpr int kLdsDn = kMT * 8 * kDnU * 128;        // fp32 h chunks
constexpr int kLdsBytes = kLdsGu > kLdsDn ? kLdsGu : kLdsDn;

// Buffer loads through a resource that spans one weight matrix: 32-bit
// offsets with immediate strides, and offsets past the end return zero (so
// the tail of the last row needs no clamp or branch).
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t matrix_rsrc(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
// A whole 32-bit word (`off` a multiple of 4). In a loop whose loads run
// ahead of their use, byte loads make the compiler widen the byte right
// after the load, which waits for it; a word needs no widening, and the byte
// is taken out where it is used.
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// A wave-uniform value the compiler can see is one: buffer resources built
// from a value it cannot prove uniform become a loop around every load.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Coherent accessors for data handed between workgroups of one launch.
template <class V>
__device__ __forceinline__ V cld(const V* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class V>
__device__ __forceinline__ void cst(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copies `total` 16-byte elements into LDS in rounds of kStageB per thread:
// each round issues all its loads before any store (clamped indices repeat
// the last element, so there is no branch to sink the loads into).
constexpr int kStageB = 3;
template <class V, class Src, class Dst>
__device__ __forceinline__ void stage_rows(int total, Src src, Dst dst) {
  for (int base = 0; base < total; base += kStageB * kThreads) {
    V v[kStageB];
#pragma unroll
    for (int i = 0; i < kStageB; ++i) v[i] = src(min(base + (int)threadIdx.x + i * kThreads, total - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kStageB; ++i) dst(min(base + (int)threadIdx.x + i * kThreads, total - 1), v[i]);
  }
}

struct Slot {
  int e;      // expert slot in its bank
  int row0;   // first row of h / y
  int m;      // rows
  bool shared;
};

}  // namespace

struct DecodeArgs {
  const uint16_t* x;
  const uint16_t* wr;
  const float* bias;
  BankView routed, shared;
  int has_shared;
  const float* y_shared_ext;  // [T][H] shared rows from earlier launches, or null
  const uint8_t *sh8_gu_w, *sh8_gu_s, *sh8_d_w, *sh8_d_s;  // FP8 shared expert
  int shared_fp8;
  int T, H, I, E, k, R;
  const int32_t* offsets_in;    // FFN mode: caller's bucket offsets
  const int32_t* row_token_in;  // FFN mode (null = identity)
  float* out;
  int32_t* ids_out;
  float* w_out;
  float* logits;       // [T][E]
  float* route_w;      // [T][k]
  int32_t* tab;        // [1 + 3 * max_slots]: n_slots, expert[], row0[], m[]
  int32_t* row_token;  // [rows]
  int32_t* inv_row;    // [T][k]
  int32_t* row_pair;   // [R] the choice t k + j each bucket row holds
  float* h;            // [rows][I]
  float* y;            // [rows][H]
  uint64_t* flags;     // [nb_router] router flags (tagged words)
  uint64_t* tagged;    // tagged words (tag << 16 | 16-bit payload). One token:
                       // [2][E] logit halves (low, high), kReplicas routing
                       // tables, the shared items' flags; blocks: [T][2][E]
  uint64_t tag;        // this call's 48-bit tag (never 0)
  uint64_t wait_tag;   // the tag the routing's first wait expects: `tag`, or
                       // (test hook) one that no word carries
  long wait_limit;     // polls before the routing's first wait gives up
                       // (every other wait: kSpinLimit)
  uint64_t* wstat;     // [0] status word: tag << 16 | the code of a wait that
                       // gave up; [1] result word (kResultMagic << 48 | tag)
  int32_t* cnt_dn;     // [dn_items] down items finished per output column group
  uint64_t* hw;        // one token: [rows][I] routed h values as value words
  uint64_t* yw;        // one token: [rows][H] y values as value words
  int max_slots;       // routed slots
  int rows;            // rows of h and y (routed rows, then T shared rows)
  int nb_router, gu_items, dn_items;
};

namespace {

__device__ __forceinline__ int load_nslots(const DecodeArgs& a) {
  return min(max(a.tab[0], 0), a.max_slots);
}

// Slot s of the table, every field clamped so that it addresses only the
// bank and the h / y rows that exist, whatever the table holds.
__device__ __forceinline__ Slot load_slot(const DecodeArgs& a, int s) {
  const int32_t* t = a.tab + 1;
  const int e = min(max(t[s], 0), a.routed.E - 1);
  const int row0 = min(max(t[a.max_slots + s], 0), a.rows);
  const int m = min(max(t[2 * a.max_slots + s], 0), a.rows - row0);
  return Slot{e, row0, m, false};
}

__device__ __forceinline__ Slot shared_slot(const DecodeArgs& a) {
  return Slot{0, a.R, a.T, true};
}

__device__ __forceinline__ uint64_t tag_word(uint64_t tag, uint32_t payload) {
  return (tag << kTagShift) | (payload & 0xffffu);
}

// A bounded wait gave up: record it for the call's last launch.
// The store completes before the wave goes on, so any signal the wave gives
// afterwards (a flag, a count, a tagged word) is seen after it.
__device__ __forceinline__ void report_timeout(const DecodeArgs& a, uint32_t code) {
  cst(a.wstat, tag_word(a.tag, code));
  __builtin_amdgcn_s_waitcnt(0);
}

// A value word (the one-token launch's h and y, a block's routed y): the
// low 32 bits of the call's tag above an fp32 value. Like a tagged word, it shows by itself whether it
// holds this call's value (foreign bytes pass with a chance of 2^-32 per
// word), so its reader needs no flag and its writer no wait.
__device__ __forceinline__ uint64_t value_word(const DecodeArgs& a, float v) {
  return (a.tag << 32) | __float_as_uint(v);
}
__device__ __forceinline__ bool is_mine(const DecodeArgs& a, uint64_t w) {
  return (uint32_t)(w >> 32) == (uint32_t)a.tag;
}

__device__ __forceinline__ uint64_t result_word(const DecodeArgs& a) {
  return (kResultMagic << 48) | (a.tag & 0xffffffffffffull);
}

// The code of a wait of this call that gave up, or 0. Read where every wait
// the reader's results depend on has been passed (in a later launch, or
// after a count that those waits precede).
__device__ __forceinline__ uint32_t call_wait_code(const DecodeArgs& a) {
  const uint64_t v = cld(a.wstat);
  return (v >> kTagShift) == a.tag ? (uint32_t)(v & 0xffffu) : 0u;
}

// The last launch of a call whose wait gave up: NaN outputs, ids -1 and
// weights NaN (workgroup b of nb covers its share of out); workgroup 0
// records the call's result for moe_workspace_status.
__device__ void finish_call(const DecodeArgs& a, uint32_t code, int b, int nb) {
  if (code) {
    const long n = (long)a.T * a.H;
    for (long i = (long)b * kThreads + threadIdx.x; i < n; i += (long)nb * kThreads)
      a.out[i] = __builtin_nanf("");
    if (b == 0)
      for (int i = threadIdx.x; i < a.R; i += kThreads) {
        if (a.ids_out) a.ids_out[i] = -1;
        if (a.w_out) a.w_out[i] = __builtin_nanf("");
      }
  }
  if (b == 0 && threadIdx.x == 0) a.wstat[1] = result_word(a);
}

// ---------------------------------------------------------------------------
// Router rows: one wave per expert row, all row loads in flight at once.
// ---------------------------------------------------------------------------
__device__ void router_rows(const DecodeArgs& a, int b) {
  const int lane = lane_id();
  const int e = b * 4 + (threadIdx.x >> 6);
  if (e < a.E) {
    const int nv = a.H >> 3;
    const uint4* wrow = reinterpret_cast<const uint4*>(a.wr + (size_t)e * a.H);
    uint4 wv[kRouterV];
#pragma unroll
    for (int i = 0; i < kRouterV; ++i) wv[i] = wrow[min(lane + kWave * i, nv - 1)];
    const float bb = a.bias ? a.bias[e] : 0.0f;
    for (int t = 0; t < a.T; ++t) {
      const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)t * a.H);
      uint4 xv[kRouterV];
#pragma unroll
      for (int i = 0; i < kRouterV; ++i) xv[i] = xr[min(lane + kWave * i, nv - 1)];
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < kRouterV; ++i)
        if (lane + kWave * i < nv) acc = dot8_bf16(wv[i], xv[i], acc);
      acc = wave_sum(acc);
      if (lane == 0) cst(a.logits + (size_t)t * a.E + e, acc + bb);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) cst(a.flags + b, tag_word(a.tag, 1));
}

// ---------------------------------------------------------------------------
// Routing: top-k per token (one wave per token) and atomic-free bucketing.
// ---------------------------------------------------------------------------

// (topk_key_f64, wave_max_key_f64 and topk_row_f64: topk_wave.h)

template <int NK, int HALVES>
__device__ bool poll_tagged(const DecodeArgs& a, uint64_t expect, long limit, uint32_t code,
                            const uint64_t* src, int n, uint32_t* out);

// One token's logits, lane l holding experts l, l + 64, ...: polled as
// tagged words, which carry their own proof of being this launch's (the
// block path), or read once the router flags are up (the chain).
template <int NK, bool TAGGED>
__device__ __forceinline__ void row_logits(const DecodeArgs& a, int t, float (&lv)[NK]) {
  if constexpr (TAGGED) {
    uint32_t raw[NK];
    poll_tagged<NK, 2>(a, a.wait_tag, a.wait_limit, kWaitLogits, a.tagged + (size_t)t * 2 * a.E,
                       a.E, raw);
#pragma unroll
    for (int i = 0; i < NK; ++i) lv[i] = __uint_as_float(raw[i]);
  } else {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = lane + kWave * i;
      lv[i] = e < a.E ? cld(a.logits + (size_t)t * a.E + e) : 0.0f;
    }
  }
}

// Wave w takes tokens w, w + 4, ... one after the other (two tokens' rounds
// interleaved in one wave measured slower than the same rounds in turn, and
// polling both tokens' logits before either selection slower too: the
// router publishes token w + 4 after token w).
template <int NK, bool TAGGED>
__device__ void topk_block_rows(const DecodeArgs& a, int* s_ids, float* s_w) {
  for (int t = threadIdx.x >> 6; t < a.T; t += kThreads / kWave) {
    float lv[NK];
    row_logits<NK, TAGGED>(a, t, lv);
    topk_row_f64<NK>(lv, a.E, a.k, s_ids + t * a.k, s_w + t * a.k);
  }
}

// TAGGED: the block path, whose router publishes tagged logits (no flags);
// otherwise the chain, whose router raises one flag per workgroup.
template <bool TAGGED>
__device__ void routing(const DecodeArgs& a, char* lds) {
  // router flags, polled in parallel by this one workgroup
  for (long it = 0; !TAGGED; ++it) {
    bool ok = true;
    for (int i = threadIdx.x; i < a.nb_router; i += kThreads)
      ok &= cld(a.flags + i) == tag_word(a.wait_tag, 1);
    if (__syncthreads_and(ok)) break;
    if (it >= a.wait_limit) {
      if (threadIdx.x == 0) report_timeout(a, kWaitRouterFlags);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  const int R = a.R;
  int* s_ids = reinterpret_cast<int*>(lds);
  float* s_w = reinterpret_cast<float*>(s_ids + R);
  int* s_first = reinterpret_cast<int*>(s_w + R);
  int* s_tmp = s_first + R;
  if (a.E <= 6 * kWave)
    topk_block_rows<6, TAGGED>(a, s_ids, s_w);
  else
    topk_block_rows<16, TAGGED>(a, s_ids, s_w);
  __syncthreads();
  // Stable counting sort by ranks, no atomics: pair p (token p / k) of
  // expert e goes to row (#pairs with a smaller expert) + (#earlier pairs
  // with the same expert). The first pair of each expert owns its slot.
  int n_first = 0;
  for (int p = threadIdx.x; p < R; p += kThreads) {
    const int e = s_ids[p];
    int less = 0, before = 0, same = 0;
#pragma unroll 8
    for (int q = 0; q < R; ++q) {
      const int f = s_ids[q];
      less += f < e;
      same += f == e;
      before += (f == e) & (q < p);
    }
    const int row = less + before;
    a.row_token[row] = p / a.k;
    a.inv_row[p] = row;
    a.row_pair[row] = p;
    a.route_w[p] = s_w[p];
    if (a.ids_out) a.ids_out[p] = e;
    if (a.w_out) a.w_out[p] = s_w[p];
    s_first[p] = before == 0 ? (less << 11 | same) : -1;  // row0, count (R <= 1024)
    n_first += before == 0;
  }
  int n_act = 0;
  block_exclusive_scan(n_first, s_tmp, &n_act);
  int32_t* tex = a.tab + 1;
  for (int p = threadIdx.x; p < R; p += kThreads) {
    const int fp = s_first[p];
    if (fp < 0) continue;
    const int e = s_ids[p];
    int slot = 0;
#pragma unroll 8
    for (int q = 0; q < R; ++q) slot += (s_first[q] >= 0) & (s_ids[q] < e);
    tex[slot] = e;
    tex[a.max_slots + slot] = fp >> 11;
    tex[2 * a.max_slots + slot] = fp & 2047;
  }
  if (threadIdx.x == 0) a.tab[0] = n_act;
  for (int i = threadIdx.x; i < a.dn_items; i += kThreads) a.cnt_dn[i] = 0;
}

// Slot table from caller offsets (FFN mode). Thread i owns experts 4i..4i+3,
// so a block scan of per-thread counts gives slots in ascending expert order.
// Buckets are clamped to [0, R]; at most max_slots slots are written.
__global__ __launch_bounds__(kThreads) void ffn_table_kernel(DecodeArgs a) {
  __shared__ int s_tmp[32];
  int cnt[4], lo[4], act = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    int l = 0, h = 0;
    if (e < a.E) {
      if (a.offsets_in) {
        l = min(max(a.offsets_in[e], 0), a.R);
        h = min(max(a.offsets_in[e + 1], l), a.R);
      } else if (e == 0) {
        h = a.R;
      }
    }
    cnt[q] = h - l;
    lo[q] = l;
    act += h > l;
  }
  int n_act = 0;
  int s = block_exclusive_scan(act, s_tmp, &n_act);
  int32_t* tex = a.tab + 1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (cnt[q] > 0 && s < a.max_slots) {
      tex[s] = threadIdx.x * 4 + q;
      tex[a.max_slots + s] = lo[q];
      tex[2 * a.max_slots + s] = cnt[q];
      ++s;
    }
  }
  if (threadIdx.x == 0) a.tab[0] = min(n_act, a.max_slots);
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU item: 8 rows. 32 lanes per row (each wave-wide 16-byte
// load covers 2 rows x 512 contiguous bytes), so a K = 5120 row pair is one
// batch of 5 chunks per lane; weight loads are issued before the
// activations are staged. h is written with plain stores (read by a later
// launch).
// ---------------------------------------------------------------------------
// kCoherent: h is stored write-through, for readers in this same launch.
template <int MT, bool kCoherent = false>
__device__ void gateup_item(const DecodeArgs& a, const Slot& sd, int rb, uint4* s_x,
                            const int32_t* rtok) {
  const BankView bk = sd.shared ? a.shared : a.routed;
  const int H = a.H, I = a.I;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & (kGuLanes - 1);
  const int n = rb * kGuRows + wave * (kWave / kGuLanes) + lane / kGuLanes;
  const bool row_ok = n < I;
  const int nr = row_ok ? n : I - 1;
  const int kc = H >> 5;
  const uint32_t crow = (uint32_t)H >> 1, srow = (uint32_t)H >> 5;
  const uint8_t* gbase = bk.gu_codes + (size_t)sd.e * 2 * I * crow;
  const uint8_t* sbase = bk.gu_scales + (size_t)sd.e * 2 * I * srow;
  const __amdgpu_buffer_rsrc_t rg = matrix_rsrc(gbase, I * crow);
  const __amdgpu_buffer_rsrc_t ru = matrix_rsrc(gbase + (size_t)I * crow, I * crow);
  const __amdgpu_buffer_rsrc_t rgs = matrix_rsrc(sbase, I * srow);
  const __amdgpu_buffer_rsrc_t rus = matrix_rsrc(sbase + (size_t)I * srow, I * srow);
  constexpr int kStride = kGuLanes * kGuU * 4;  // uint4 per staged token row

  for (int t0 = 0; t0 < sd.m; t0 += MT) {
    const int nt = min(MT, sd.m - t0);
    float ag[MT], au[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ag[t] = au[t] = 0.0f;
    for (int c0 = 0; c0 < kc; c0 += kGuLanes * kGuU) {
      const int cn = min(kc - c0, kGuLanes * kGuU);
      uint4 wg[kGuU], wu[kGuU];
      uint32_t sg[kGuU], su[kGuU];
      // every lane loads (chunks past the row end are unused), so the loads
      // form one straight-line batch
      const int co = nr * crow + (c0 + j) * 16, so = nr * srow + c0 + j;
#pragma unroll
      for (int u = 0; u < kGuU; ++u) {
        wg[u] = bload16(rg, co + u * kGuLanes * 16);
        wu[u] = bload16(ru, co + u * kGuLanes * 16);
        sg[u] = bload8(rgs, so + u * kGuLanes);
        su[u] = bload8(rus, so + u * kGuLanes);
      }
      __syncthreads();
      stage_rows<uint4>(
          nt * cn * 4,
          [&](int idx) {
            const int t = idx / (cn * 4), q = idx - t * cn * 4;
            const int r = sd.row0 + t0 + t;
            int tok = sd.shared ? r - a.R : (rtok ? rtok[r] : r);
            tok = min(max(tok, 0), a.T - 1);
            return reinterpret_cast<const uint4*>(a.x + (size_t)tok * H + c0 * 32)[q];
          },
          [&](int idx, uint4 v) {
            // piece p of chunk c goes to p * K + c: lanes reading consecutive
            // chunks then read consecutive 16-byte words (no bank conflicts)
            const int t = idx / (cn * 4), q = idx - t * cn * 4;
            s_x[t * kStride + (q & 3) * (kGuLanes * kGuU) + (q >> 2)] = v;
          });
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kGuU; ++u) {
        const int c = kGuLanes * u + j;
        if (c < cn) {
          const float fg = e8m0_to_f32(sg[u]), fu = e8m0_to_f32(su[u]);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              const uint4* xv = s_x + t * kStride + c;
              constexpr int P = kGuLanes * kGuU;
              const uint4 x0 = xv[0], x1 = xv[P], x2 = xv[2 * P], x3 = xv[3 * P];
              float pg = dot8_fp4_bf16(wg[u].x, x0, 0.0f);
              pg = dot8_fp4_bf16(wg[u].y, x1, pg);
              pg = dot8_fp4_bf16(wg[u].z, x2, pg);
              pg = dot8_fp4_bf16(wg[u].w, x3, pg);
              float pu = dot8_fp4_bf16(wu[u].x, x0, 0.0f);
              pu = dot8_fp4_bf16(wu[u].y, x1, pu);
              pu = dot8_fp4_bf16(wu[u].z, x2, pu);
              pu = dot8_fp4_bf16(wu[u].w, x3, pu);
              ag[t] = fmaf(pg, fg, ag[t]);
              au[t] = fmaf(pu, fu, au[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float g = group_sum<kGuLanes>(ag[t]);
      const float u = group_sum<kGuLanes>(au[t]);
      if (row_ok && j == 0 && t < nt) {
        float* p = a.h + (size_t)(sd.row0 + t0 + t) * I + n;
        if (kCoherent)
          cst(p, silu_mul(g, u));
        else
          *p = silu_mul(g, u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down item: 32 output rows, 8 lanes per row (each wave-wide load covers 8
// whole 128-byte lines), K = 2304 in one batch of 9 chunks per lane; weight
// loads before the h rows are staged. `coherent` stores y for a consumer in
// the same launch.
// ---------------------------------------------------------------------------
template <int MT>
__device__ void down_item(const DecodeArgs& a, const Slot& sd, int rb, f32x4_t* s_h, float* y,
                          bool coherent) {
  const BankView bk = sd.shared ? a.shared : a.routed;
  const int H = a.H, I = a.I;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int n = rb * kDnRows + wave * 8 + (lane >> 3);
  const bool row_ok = n < H;
  const int nr = row_ok ? n : H - 1;
  const int kc = I >> 5;
  const uint32_t crow = (uint32_t)I >> 1, srow = (uint32_t)I >> 5;
  const __amdgpu_buffer_rsrc_t rd = matrix_rsrc(bk.d_codes + (size_t)sd.e * H * crow, H * crow);
  const __amdgpu_buffer_rsrc_t rds = matrix_rsrc(bk.d_scales + (size_t)sd.e * H * srow, H * srow);
  constexpr int kStride = 8 * kDnU * 8;  // f32x4_t per staged row

  for (int t0 = 0; t0 < sd.m; t0 += MT) {
    const int nt = min(MT, sd.m - t0);
    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (int c0 = 0; c0 < kc; c0 += 8 * kDnU) {
      const int cn = min(kc - c0, 8 * kDnU);
      uint4 wd[kDnU];
      uint32_t sd8[kDnU];
      const int co = nr * crow + (c0 + j) * 16, so = nr * srow + c0 + j;
#pragma unroll
      for (int u = 0; u < kDnU; ++u) {
        wd[u] = bload16(rd, co + u * 8 * 16);
        sd8[u] = bload8(rds, so + u * 8);
      }
      __syncthreads();
      stage_rows<f32x4_t>(
          nt * cn * 8,
          [&](int idx) {
            const int t = idx / (cn * 8), q = idx - t * cn * 8;
            return reinterpret_cast<const f32x4_t*>(a.h + (size_t)(sd.row0 + t0 + t) * I + c0 * 32)[q];
          },
          [&](int idx, f32x4_t v) {
            const int t = idx / (cn * 8), q = idx - t * cn * 8;
            s_h[t * kStride + (q & 7) * (8 * kDnU) + (q >> 3)] = v;
          });
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kDnU; ++u) {
        const int c = 8 * u + j;
        if (c < cn) {
          const float fd = e8m0_to_f32(sd8[u]);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              const f32x4_t* hv = s_h + t * kStride + c;
              constexpr int P = 8 * kDnU;
              float pd = dot8_fp4_f32(wd[u].x, hv[0], hv[P], 0.0f);
              pd = dot8_fp4_f32(wd[u].y, hv[2 * P], hv[3 * P], pd);
              pd = dot8_fp4_f32(wd[u].z, hv[4 * P], hv[5 * P], pd);
              pd = dot8_fp4_f32(wd[u].w, hv[6 * P], hv[7 * P], pd);
              acc[t] = fmaf(pd, fd, acc[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float v = group_sum<8>(acc[t]);
      if (row_ok && j == 0 && t < nt) {
        float* p = y + (size_t)(sd.row0 + t0 + t) * H + n;
        if (coherent)
          cst(p, v);
        else
          *p = v;
      }
    }
  }
}

// Combine of output columns [32c, 32c + 32): the shared row, then the k
// routed rows in slot order j = 0..k-1, one fp32 fma each (coherent loads:
// rows may have been written by other workgroups of this launch). `failed`:
// a wait of this call gave up, so the column is NaN.
__device__ void combine_column(const DecodeArgs& a, int c, bool failed) {
  const int n = c * kDnRows + (threadIdx.x & 31);
  if (n >= a.H) return;
  for (int t = threadIdx.x >> 5; t < a.T; t += kThreads / 32) {
    float v = a.y_shared_ext ? a.y_shared_ext[(size_t)t * a.H + n]
              : a.has_shared ? cld(a.y + (size_t)(a.R + t) * a.H + n) : 0.0f;
    for (int j0 = 0; j0 < a.k; j0 += 8) {  // 8 rows' loads in flight at a time
      float yv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = min(max(a.inv_row[t * a.k + min(j0 + u, a.k - 1)], 0), a.R - 1);
        yv[u] = cld(a.y + (size_t)r * a.H + n);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < a.k) v = fmaf(a.route_w[t * a.k + j0 + u], yv[u], v);
    }
    a.out[(size_t)t * a.H + n] = failed ? __builtin_nanf("") : v;
  }
}

// ---------------------------------------------------------------------------
// One token: streaming gate/up and down. Persistent workgroups walk the
// items b, b + G, b + 2G, ... with two register buffers, so the weights of
// the next item are in flight while the current one is computed and HBM
// never waits for a round of workgroups to finish. The single token row and
// the slot table are staged once per workgroup. (K = H <= 5120 for gate/up
// and K = I <= 2304 for down, one batch per row; larger shapes take the
// one-shot kernels.)
// ---------------------------------------------------------------------------
// The one-token gate/up stream gives each workgroup the same number of items,
// two (one pass of its two-buffer loop) wherever at most this many
// workgroups then cover the routed items.
constexpr int kGuStreamMax = 896;
// Down items (32-row groups) per workgroup of the one-token launch (1 or 2).
constexpr int kDnPerWg = 2;
// The last slots' down work goes one item per workgroup instead: their h
// flags come last (their gate/up workgroups are dispatched last), so halving
// the work behind each of those flags shortens the launch's tail. Measured
// at 6 slots: the last two slots single is 0.6-1 us faster than all pairs;
// the last three, four or six are slower (more workgroups behind the flags).
constexpr int kDnSingleSlots = 2;

// sg / su: the words holding the lane's scale bytes (byte lane % 4 of each).
struct GuRegs {
  uint4 g[kGuU], u[kGuU];
  uint32_t sg[kGuU], su[kGuU];
};

// `live` false: a padding issue of the fixed-trip loop. Its weight loads go
// through empty buffer resources, which return zeros without a memory access.
__device__ __forceinline__ void gu_issue(const DecodeArgs& a, const int* tab, int it, GuRegs& r,
                                         bool live = true) {
  const int s = it / a.gu_items, rb = it - s * a.gu_items;
  const int e = __builtin_amdgcn_readfirstlane(min(max(tab[1 + s], 0), a.routed.E - 1));
  live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & (kGuLanes - 1);
  const int nr = min(rb * kGuRows + wave * (kWave / kGuLanes) + lane / kGuLanes, a.I - 1);
  const uint32_t crow = (uint32_t)a.H >> 1, srow = (uint32_t)a.H >> 5;
  const uint8_t* gbase = uniform_ptr(a.routed.gu_codes + (size_t)e * 2 * a.I * crow);
  const uint8_t* sbase = uniform_ptr(a.routed.gu_scales + (size_t)e * 2 * a.I * srow);
  const uint32_t cb = live ? a.I * crow : 0u, sb = live ? a.I * srow : 0u;
  const __amdgpu_buffer_rsrc_t rg = matrix_rsrc(gbase, cb);
  const __amdgpu_buffer_rsrc_t ru = matrix_rsrc(gbase + (size_t)a.I * crow, cb);
  const __amdgpu_buffer_rsrc_t rgs = matrix_rsrc(sbase, sb);
  const __amdgpu_buffer_rsrc_t rus = matrix_rsrc(sbase + (size_t)a.I * srow, sb);
  // scale byte j + 32 u of a row is byte j % 4 of its word j / 4 + 8 u (rows
  // start on a word: H % 128 == 0)
  const int co = nr * crow + j * 16, so = nr * srow + (j & ~3);
#pragma unroll
  for (int u = 0; u < kGuU; ++u) {
    r.g[u] = bload16(rg, co + u * kGuLanes * 16);
    r.u[u] = bload16(ru, co + u * kGuLanes * 16);
    r.sg[u] = bload32(rgs, so + u * kGuLanes);
    r.su[u] = bload32(rus, so + u * kGuLanes);
  }
}

__device__ __forceinline__ void gu_compute(const DecodeArgs& a, const int* tab, int it,
                                           const GuRegs& r, const uint4* s_x) {
  const int s = it / a.gu_items, rb = it - s * a.gu_items;
  const int row = min(max(tab[1 + a.max_slots + s], 0), a.rows - 1);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & (kGuLanes - 1);
  const int n = rb * kGuRows + wave * (kWave / kGuLanes) + lane / kGuLanes;
  const int kc = a.H >> 5;
  const uint32_t sh = 8u * (j & 3);
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int u = 0; u < kGuU; ++u) {
    const int c = kGuLanes * u + j;
    if (c < kc) {
      const uint4* xv = s_x + c;
      constexpr int P = kGuLanes * kGuU;
      const uint4 x0 = xv[0], x1 = xv[P], x2 = xv[2 * P], x3 = xv[3 * P];
      float pg = dot8_fp4_bf16(r.g[u].x, x0, 0.0f);
      pg = dot8_fp4_bf16(r.g[u].y, x1, pg);
      pg = dot8_fp4_bf16(r.g[u].z, x2, pg);
      pg = dot8_fp4_bf16(r.g[u].w, x3, pg);
      float pu = dot8_fp4_bf16(r.u[u].x, x0, 0.0f);
      pu = dot8_fp4_bf16(r.u[u].y, x1, pu);
      pu = dot8_fp4_bf16(r.u[u].z, x2, pu);
      pu = dot8_fp4_bf16(r.u[u].w, x3, pu);
      ag = fmaf(pg, e8m0_to_f32(__builtin_amdgcn_ubfe(r.sg[u], sh, 8)), ag);
      au = fmaf(pu, e8m0_to_f32(__builtin_amdgcn_ubfe(r.su[u], sh, 8)), au);
    }
  }
  const float g = group_sum<kGuLanes>(ag), u = group_sum<kGuLanes>(au);
  if (j == 0 && n < a.I) cst(a.hw + (size_t)row * a.I + n, value_word(a, silu_mul(g, u)));
}

// Router rows for one token with x staged in LDS: a wave per expert row,
// the row's loads issued before the token is staged, so both are in flight
// together and only the weights live in registers. Each logit is published
// as one 64-bit word carrying the launch tag, so a reader knows a value is
// this launch's from the word itself (no flag, no ordering between words).
__device__ void router_rows_one(const DecodeArgs& a, int b, uint4* s_x) {
  const int lane = lane_id();
  const int e = min(b * 4 + (int)(threadIdx.x >> 6), a.E - 1);
  const int nv = a.H >> 3;
  const uint4* wrow = reinterpret_cast<const uint4*>(a.wr + (size_t)e * a.H);
  uint4 wv[kRouterV];
#pragma unroll
  for (int i = 0; i < kRouterV; ++i) wv[i] = wrow[min(lane + kWave * i, nv - 1)];
  stage_rows<uint4>(
      nv, [&](int idx) { return reinterpret_cast<const uint4*>(a.x)[idx]; },
      [&](int idx, uint4 v) { s_x[idx] = v; });
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kRouterV; ++i)
    if (lane + kWave * i < nv) acc = dot8_bf16(wv[i], s_x[lane + kWave * i], acc);
  acc = wave_sum(acc);
  if (lane == 0 && b * 4 + (int)(threadIdx.x >> 6) < a.E) {
    const uint32_t v = __float_as_uint(acc + (a.bias ? a.bias[e] : 0.0f));
    cst(a.tagged + e, tag_word(a.tag, v));
    cst(a.tagged + a.E + e, tag_word(a.tag, v >> 16));
  }
}

// Polls `n` values at `src` (lane i holds values i, i + 64, ...) until every
// word carries the tag `expect`; each value is HALVES tagged words, its
// 16-bit pieces at src + h n (h = 0 the low piece). Returns the values
// through `out` (NK per lane). Bounded: a timeout records `code` in the
// status word and returns false with what was read, which every consumer
// clamps.
template <int NK, int HALVES>
__device__ bool poll_tagged(const DecodeArgs& a, uint64_t expect, long limit, uint32_t code,
                            const uint64_t* src, int n, uint32_t* out) {
  const int lane = lane_id();
  for (long it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int q = lane + kWave * i;
      uint32_t val = 0;
#pragma unroll
      for (int h = 0; h < HALVES; ++h) {
        const uint64_t v = q < n ? cld(src + (size_t)h * n + q) : tag_word(expect, 0);
        val |= (uint32_t)(v & 0xffffu) << (16 * h);
        ok &= (v >> kTagShift) == expect;
      }
      out[i] = val;
    }
    if (__all(ok)) return true;
    if (it >= limit) {
      if (lane == 0) report_timeout(a, code);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Replica r of the one-token routing words.
__device__ __forceinline__ uint64_t* replica(const DecodeArgs& a, int r) {
  return a.tagged + 2 * a.E + (size_t)r * kReplicaWords;
}

// The one-token routing workgroup (wave 0): waits for the tagged logits,
// takes the top-k (descending logit, ties to the lower id) and publishes
// the chosen ids as tagged words in kReplicas copies, then the weights
// renormalised over the k as tagged words, for the workgroups of this
// launch; writes the ids and weights out (-1 and NaN if its wait gave up)
// and the call's result word.
template <int NK>
__device__ void route_token_tagged(const DecodeArgs& a) {
  const int lane = lane_id(), k = a.k;
  uint32_t raw[NK];
  if (lane == 0) a.wstat[1] = result_word(a);
  const bool ok = poll_tagged<NK, 2>(a, a.wait_tag, a.wait_limit, kWaitLogits, a.tagged, a.E, raw);
  // k rounds of: each lane's best remaining key, the wave's best of those
  // (fp64 max on the keys' bits), and that key taken out
  double key[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + kWave * i;
    key[i] = __longlong_as_double(e < a.E ? (long long)topk_key_f64(__uint_as_float(raw[i]), e) : 0);
  }
  float my_val = 0.0f, top = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    double best = key[0];
#pragma unroll
    for (int i = 1; i < NK; ++i) best = fmax(best, key[i]);
    const uint64_t win = wave_max_key_f64((uint64_t)__double_as_longlong(best));
    const uint32_t id = 0x7fffffffu - (uint32_t)(win & 0x7fffffffu);
    uint32_t bits = (uint32_t)(win >> 31);
    bits = (bits & 0x80000000u) ? (bits & 0x7fffffffu) : ~bits;
    const float val = __uint_as_float(bits);
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if ((uint64_t)__double_as_longlong(key[i]) == win) key[i] = 0.0;
    if (lane == j) {
      my_val = val;
      my_id = (int)min(id, (uint32_t)(a.E - 1));
    }
    if (j == 0) top = val;
  }
  // the gate/up workgroups wait on the ids alone: publish them before the
  // weights are worked out
  if (lane < k)
    for (int r = 0; r < kReplicas; ++r) cst(replica(a, r) + lane, tag_word(a.tag, (uint32_t)my_id));
  // weights from the k chosen lanes, read lane by lane (cheaper than
  // shuffles through LDS); the sum runs over j = 0..k-1 in order
  const float z = lane < k ? expf(my_val - top) : 0.0f;
  float zsum = 0.0f;
  for (int q = 0; q < k; ++q)
    zsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), q));
  const float wj = z / zsum;
  if (lane < k) {
    const uint32_t wb = __float_as_uint(wj);
    for (int r = 0; r < kReplicas; ++r) {
      uint64_t* ww = replica(a, r) + kRepWeights;
      cst(ww + lane, tag_word(a.tag, wb));
      cst(ww + k + lane, tag_word(a.tag, wb >> 16));
    }
    if (a.ids_out) a.ids_out[lane] = ok ? my_id : -1;
    if (a.w_out) a.w_out[lane] = ok ? wj : __builtin_nanf("");
  }
}

// A workgroup's copy of the routing, taken by one wave: polls replica `r`
// and builds the slot table in LDS (slot = rank of the expert id among the
// k, so slots ascend by expert id; one row per slot, row = slot), and
// (s_inv not null) the slot of each choice j.
__device__ void routing_copy(const DecodeArgs& a, int r, int* s_tab, int* s_inv) {
  const int k = a.k, ms = a.max_slots, lane = lane_id();
  uint32_t v[1];
  poll_tagged<1, 1>(a, a.tag, kSpinLimit, kWaitTable, replica(a, r), k, v);
  const int my_id = lane < k ? min(max((int)v[0], 0), a.E - 1) : 0x7fffffff;
  int slot = 0;
  for (int q = 0; q < k; ++q) slot += __builtin_amdgcn_readlane(my_id, q) < my_id;
  if (lane < k) {
    s_tab[1 + slot] = my_id;
    s_tab[1 + ms + slot] = slot;
    s_tab[1 + 2 * ms + slot] = 1;
    if (s_inv) s_inv[lane] = slot;
  }
  if (lane == 0) s_tab[0] = k;
}

__device__ void load_routing_tagged(const DecodeArgs& a, int r, int* s_tab) {
  if (threadIdx.x < kWave) routing_copy(a, r, s_tab, nullptr);
  __syncthreads();
}

// The k routing weights (one wave), from replica r's tagged words.
__device__ void routing_weights(const DecodeArgs& a, int r, float* s_w) {
  uint32_t v[1];
  poll_tagged<1, 2>(a, a.tag, kSpinLimit, kWaitTable, replica(a, r) + kRepWeights, a.k, v);
  if (lane_id() < a.k) s_w[lane_id()] = __uint_as_float(v[0]);
}

// sc: the words holding the lane's scale bytes (byte (lane % 8) % 4 of each).
struct DnRegs {
  uint4 w[kDnU];
  uint32_t sc[kDnU];
  f32x4_t h[3];  // this workgroup's share of the item's h row (I <= 3072)
};

// Down item `it`: items [0, nr) are (routed slot, 32-row group) pairs,
// slot-major; items [nr, nr + dn_items) are the shared expert's groups.
struct DnItem {
  const uint8_t* codes;   // the item's expert's down codes
  const uint8_t* scales;
  int row;                // h / y row
  int c;                  // 32-row group of the output
};

__device__ __forceinline__ DnItem dn_item(const DecodeArgs& a, const int* tab, int nr, int it) {
  const uint32_t crow = (uint32_t)a.I >> 1, srow = (uint32_t)a.I >> 5;
  if (it >= nr) {
    const int c = min(it - nr, a.dn_items - 1);
    return DnItem{a.shared.d_codes, a.shared.d_scales, min(a.R, a.rows - 1), c};
  }
  const int s = it / a.dn_items, c = it - s * a.dn_items;
  const int e = __builtin_amdgcn_readfirstlane(min(max(tab[1 + s], 0), a.routed.E - 1));
  const int row = min(max(tab[1 + a.max_slots + s], 0), a.rows - 1);
  return DnItem{a.routed.d_codes + (size_t)e * a.H * crow, a.routed.d_scales + (size_t)e * a.H * srow,
                row, c};
}

// The item's h row (I <= 3072: three float4 a thread). kCoherent: written
// by other workgroups of this launch, so read with coherent loads.
template <bool kCoherent>
__device__ __forceinline__ void dn_issue_h(const DecodeArgs& a, int row, DnRegs& r) {
  const int nv = a.I >> 2;
  if (kCoherent) {
    const uint64_t* hrow = reinterpret_cast<const uint64_t*>(a.h + (size_t)row * a.I);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = min((int)threadIdx.x + i * kThreads, nv - 1);
      const uint64_t lo = cld(hrow + 2 * f), hi = cld(hrow + 2 * f + 1);
      r.h[i] = f32x4_t{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                       __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
    }
  } else {
    const f32x4_t* hrow = reinterpret_cast<const f32x4_t*>(a.h + (size_t)row * a.I);
#pragma unroll
    for (int i = 0; i < 3; ++i) r.h[i] = hrow[min((int)threadIdx.x + i * kThreads, nv - 1)];
  }
}

// The item's weights and (with_h) its h row; `live` false reads no weights.
__device__ __forceinline__ void dn_issue(const DecodeArgs& a, const int* tab, int n_routed, int it,
                                         DnRegs& r, bool live = true, bool with_h = true) {
  const DnItem d = dn_item(a, tab, n_routed, it);
  const int c = d.c, row = d.row;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int nr = min(c * kDnRows + wave * 8 + (lane >> 3), a.H - 1);
  const uint32_t crow = (uint32_t)a.I >> 1, srow = (uint32_t)a.I >> 5;
  live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  const __amdgpu_buffer_rsrc_t rd = matrix_rsrc(uniform_ptr(d.codes), live ? a.H * crow : 0u);
  const __amdgpu_buffer_rsrc_t rds =
      matrix_rsrc(uniform_ptr(d.scales), live ? a.H * srow : 0u);
  // scale byte j + 8 u of a row is byte j % 4 of its word j / 4 + 2 u (rows
  // start on a word: I % 128 == 0)
  const int co = nr * crow + j * 16, so = nr * srow + 4 * (j >> 2);
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    r.w[u] = bload16(rd, co + u * 8 * 16);
    r.sc[u] = bload32(rds, so + u * 8);
  }
  if (with_h) dn_issue_h<false>(a, row, r);
}

__device__ __forceinline__ void dn_compute(const DecodeArgs& a, const int* tab, int nr, int it,
                                           const DnRegs& r, f32x4_t* s_h) {
  const int nv = a.I >> 2;
  __syncthreads();  // previous item's reads of s_h are done
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int f = min((int)threadIdx.x + i * kThreads, nv - 1);
    s_h[(f & 7) * (8 * kDnU) + (f >> 3)] = r.h[i];
  }
  __syncthreads();
  const DnItem d = dn_item(a, tab, nr, it);
  const int c = d.c, row = d.row;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int n = c * kDnRows + wave * 8 + (lane >> 3);
  const int kc = a.I >> 5;
  const uint32_t sh = 8u * (j & 3);
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    const int ch = 8 * u + j;
    if (ch < kc) {
      const f32x4_t* hv = s_h + ch;
      constexpr int P = 8 * kDnU;
      float pd = dot8_fp4_f32(r.w[u].x, hv[0], hv[P], 0.0f);
      pd = dot8_fp4_f32(r.w[u].y, hv[2 * P], hv[3 * P], pd);
      pd = dot8_fp4_f32(r.w[u].z, hv[4 * P], hv[5 * P], pd);
      pd = dot8_fp4_f32(r.w[u].w, hv[6 * P], hv[7 * P], pd);
      acc = fmaf(pd, e8m0_to_f32(__builtin_amdgcn_ubfe(r.sc[u], sh, 8)), acc);
    }
  }
  const float v = group_sum<8>(acc);
  if (j == 0 && n < a.H) cst(a.yw + (size_t)row * a.H + n, value_word(a, v));
}

// ---------------------------------------------------------------------------
// NVFP4 banks in the one-token launches (E2M1 codes, one E4M3 scale per 16
// codes, an fp32 scale per expert and matrix): the same items and register
// buffers as MXFP4, with a 32-code chunk's two scale bytes taken from one
// word (rows of K / 16 scale bytes start on a word), each 16-code half of
// the chunk's dot product multiplied by its own scale and the matrix scale
// applied to the row sums.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x2_t nv_scale_pair(uint32_t word, uint32_t sh) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((word >> sh) & 0xffffu, 1.0f, false);
}
__device__ __forceinline__ float nv_matrix_scale(const BankView& b, int e, int m) {
  return b.gscale ? b.gscale[e * 3 + m] : 1.0f;
}

// gate/up weights of 8-row group rb of the expert whose codes / scales
// start at gbase / sbase ([2][I][H/2], [2][I][H/16])
__device__ __forceinline__ void gu_issue_nv(const DecodeArgs& a, const uint8_t* gbase,
                                            const uint8_t* sbase, int rb, GuRegs& r, bool live) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & (kGuLanes - 1);
  const int nr = min(rb * kGuRows + wave * (kWave / kGuLanes) + lane / kGuLanes, a.I - 1);
  const uint32_t crow = (uint32_t)a.H >> 1, srow = (uint32_t)a.H >> 4;
  live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  gbase = uniform_ptr(gbase);
  sbase = uniform_ptr(sbase);
  const uint32_t cb = live ? a.I * crow : 0u, sb = live ? a.I * srow : 0u;
  const __amdgpu_buffer_rsrc_t rg = matrix_rsrc(gbase, cb);
  const __amdgpu_buffer_rsrc_t ru = matrix_rsrc(gbase + (size_t)a.I * crow, cb);
  const __amdgpu_buffer_rsrc_t rgs = matrix_rsrc(sbase, sb);
  const __amdgpu_buffer_rsrc_t rus = matrix_rsrc(sbase + (size_t)a.I * srow, sb);
  // chunk j + 32 u has scale bytes 2 j + 64 u and the next: half j % 2 of
  // the word at 4 (j / 2) + 64 u
  const int co = nr * crow + j * 16, so = nr * srow + 4 * (j >> 1);
#pragma unroll
  for (int u = 0; u < kGuU; ++u) {
    r.g[u] = bload16(rg, co + u * kGuLanes * 16);
    r.u[u] = bload16(ru, co + u * kGuLanes * 16);
    r.sg[u] = bload32(rgs, so + u * kGuLanes * 2);
    r.su[u] = bload32(rus, so + u * kGuLanes * 2);
  }
}

// kWord: h as value words (routed); otherwise coherent fp32 (shared)
template <bool kWord>
__device__ __forceinline__ void gu_compute_nv(const DecodeArgs& a, int rb, int row, float mg,
                                              float mu, const GuRegs& r, const uint4* s_x) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & (kGuLanes - 1);
  const int n = rb * kGuRows + wave * (kWave / kGuLanes) + lane / kGuLanes;
  const int kc = a.H >> 5;
  const uint32_t sh = 16u * (j & 1);
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int u = 0; u < kGuU; ++u) {
    const int c = kGuLanes * u + j;
    if (c < kc) {
      const uint4* xv = s_x + c;
      constexpr int P = kGuLanes * kGuU;
      const uint4 x0 = xv[0], x1 = xv[P], x2 = xv[2 * P], x3 = xv[3 * P];
      const f32x2_t fg = nv_scale_pair(r.sg[u], sh), fu = nv_scale_pair(r.su[u], sh);
      float g0 = dot8_fp4_bf16(r.g[u].x, x0, 0.0f);
      g0 = dot8_fp4_bf16(r.g[u].y, x1, g0);
      float g1 = dot8_fp4_bf16(r.g[u].z, x2, 0.0f);
      g1 = dot8_fp4_bf16(r.g[u].w, x3, g1);
      float u0 = dot8_fp4_bf16(r.u[u].x, x0, 0.0f);
      u0 = dot8_fp4_bf16(r.u[u].y, x1, u0);
      float u1 = dot8_fp4_bf16(r.u[u].z, x2, 0.0f);
      u1 = dot8_fp4_bf16(r.u[u].w, x3, u1);
      ag = fmaf(g1, fg.y, fmaf(g0, fg.x, ag));
      au = fmaf(u1, fu.y, fmaf(u0, fu.x, au));
    }
  }
  const float g = group_sum<kGuLanes>(ag) * mg, u = group_sum<kGuLanes>(au) * mu;
  if (j == 0 && n < a.I) {
    if (kWord)
      cst(a.hw + (size_t)row * a.I + n, value_word(a, silu_mul(g, u)));
    else
      cst(a.h + (size_t)row * a.I + n, silu_mul(g, u));
  }
}

// routed item `it` (slot-major over gu_items 8-row groups)
__device__ __forceinline__ void gu_issue_nv_routed(const DecodeArgs& a, const int* tab, int it,
                                                   GuRegs& r, bool live) {
  const int s = it / a.gu_items, rb = it - s * a.gu_items;
  const int e = __builtin_amdgcn_readfirstlane(min(max(tab[1 + s], 0), a.routed.E - 1));
  gu_issue_nv(a, a.routed.gu_codes + (size_t)e * 2 * a.I * (a.H >> 1),
              a.routed.gu_scales + (size_t)e * 2 * a.I * (a.H >> 4), rb, r, live);
}
__device__ __forceinline__ void gu_compute_nv_routed(const DecodeArgs& a, const int* tab, int it,
                                                     const GuRegs& r, const uint4* s_x) {
  const int s = it / a.gu_items, rb = it - s * a.gu_items;
  const int e = min(max(tab[1 + s], 0), a.routed.E - 1);
  const int row = min(max(tab[1 + a.max_slots + s], 0), a.rows - 1);
  gu_compute_nv<true>(a, rb, row, nv_matrix_scale(a.routed, e, 0), nv_matrix_scale(a.routed, e, 1),
                      r, s_x);
}

// down: item it of the routed slots (it < nr) or of the shared expert
struct DnItemNv {
  const uint8_t* codes;
  const uint8_t* scales;
  int row, c;
  float md;
};
__device__ __forceinline__ DnItemNv dn_item_nv(const DecodeArgs& a, const int* tab, int nr, int it) {
  const uint32_t crow = (uint32_t)a.I >> 1, srow = (uint32_t)a.I >> 4;
  if (it >= nr) {
    const int c = min(it - nr, a.dn_items - 1);
    return DnItemNv{a.shared.d_codes, a.shared.d_scales, min(a.R, a.rows - 1), c,
                    nv_matrix_scale(a.shared, 0, 2)};
  }
  const int s = it / a.dn_items, c = it - s * a.dn_items;
  const int e = __builtin_amdgcn_readfirstlane(min(max(tab[1 + s], 0), a.routed.E - 1));
  const int row = min(max(tab[1 + a.max_slots + s], 0), a.rows - 1);
  return DnItemNv{a.routed.d_codes + (size_t)e * a.H * crow,
                  a.routed.d_scales + (size_t)e * a.H * srow, row, c,
                  nv_matrix_scale(a.routed, e, 2)};
}

__device__ __forceinline__ void dn_issue_nv(const DecodeArgs& a, const int* tab, int n_routed,
                                            int it, DnRegs& r, bool live = true,
                                            bool with_h = true) {
  const DnItemNv d = dn_item_nv(a, tab, n_routed, it);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int nr = min(d.c * kDnRows + wave * 8 + (lane >> 3), a.H - 1);
  const uint32_t crow = (uint32_t)a.I >> 1, srow = (uint32_t)a.I >> 4;
  live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  const __amdgpu_buffer_rsrc_t rd = matrix_rsrc(uniform_ptr(d.codes), live ? a.H * crow : 0u);
  const __amdgpu_buffer_rsrc_t rds = matrix_rsrc(uniform_ptr(d.scales), live ? a.H * srow : 0u);
  // chunk j + 8 u has scale bytes 2 j + 16 u and the next: half j % 2 of
  // the word at 4 (j / 2) + 16 u
  const int co = nr * crow + j * 16, so = nr * srow + 4 * (j >> 1);
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    r.w[u] = bload16(rd, co + u * 8 * 16);
    r.sc[u] = bload32(rds, so + u * 16);
  }
  if (with_h) dn_issue_h<false>(a, d.row, r);
}

__device__ __forceinline__ void dn_compute_nv(const DecodeArgs& a, const int* tab, int nr, int it,
                                              const DnRegs& r, f32x4_t* s_h) {
  const int nv = a.I >> 2;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int f = min((int)threadIdx.x + i * kThreads, nv - 1);
    s_h[(f & 7) * (8 * kDnU) + (f >> 3)] = r.h[i];
  }
  __syncthreads();
  const DnItemNv d = dn_item_nv(a, tab, nr, it);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int n = d.c * kDnRows + wave * 8 + (lane >> 3);
  const int kc = a.I >> 5;
  const uint32_t sh = 16u * (j & 1);
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    const int ch = 8 * u + j;
    if (ch < kc) {
      const f32x4_t* hv = s_h + ch;
      constexpr int P = 8 * kDnU;
      const f32x2_t f = nv_scale_pair(r.sc[u], sh);
      float p0 = dot8_fp4_f32(r.w[u].x, hv[0], hv[P], 0.0f);
      p0 = dot8_fp4_f32(r.w[u].y, hv[2 * P], hv[3 * P], p0);
      float p1 = dot8_fp4_f32(r.w[u].z, hv[4 * P], hv[5 * P], 0.0f);
      p1 = dot8_fp4_f32(r.w[u].w, hv[6 * P], hv[7 * P], p1);
      acc = fmaf(p1, f.y, fmaf(p0, f.x, acc));
    }
  }
  const float v = group_sum<8>(acc) * d.md;
  if (j == 0 && n < a.H) cst(a.yw + (size_t)d.row * a.H + n, value_word(a, v));
}

// The slot's h row from its value words (all threads): reads until every
// word carries the call's tag. Bounded like poll_tagged.
__device__ void poll_h_words(const DecodeArgs& a, int row, DnRegs& r) {
  const int nv = a.I >> 2;
  const uint64_t* src = a.hw + (size_t)row * a.I;
  for (long it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = min((int)threadIdx.x + i * kThreads, nv - 1);
      uint64_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = cld(src + 4 * f + q);
        ok &= is_mine(a, w[q]);
      }
      r.h[i] = f32x4_t{__uint_as_float((uint32_t)w[0]), __uint_as_float((uint32_t)w[1]),
                       __uint_as_float((uint32_t)w[2]), __uint_as_float((uint32_t)w[3])};
    }
    if (__syncthreads_and(ok)) return;
    if (it >= kSpinLimit) {
      if (threadIdx.x == 0) report_timeout(a, kWaitGateup);
      return;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Output column groups c0 and (live1) c0 + 1 of the one token, by wave 0
// (lanes 0..31 and 32..63), each if all its parts have their y words: the
// shared row, then the k routed rows in order j, one fp32 fma each. Called
// by each part's writer once its own words have landed, so the writer
// whose words land last finds them all (another may too, and writes the
// same values). failed: a wait of the call gave up; the group is NaN.
__device__ void try_combine(const DecodeArgs& a, int c0, bool live1, const int* s_inv,
                            const float* s_w, bool failed) {
  const int lane = lane_id();
  const int n = (lane < 32 ? c0 : c0 + 1) * kDnRows + (lane & 31);
  const bool valid = (lane < 32 || live1) && n < a.H;
  const int nn = valid ? n : 0;
  bool ok = true;
  float v = 0.0f;
  if (a.y_shared_ext) {
    v = a.y_shared_ext[nn];
  } else if (a.has_shared) {
    const uint64_t w = cld(a.yw + (size_t)a.R * a.H + nn);
    ok &= is_mine(a, w);
    v = __uint_as_float((uint32_t)w);
  }
  for (int j0 = 0; j0 < a.k; j0 += 8) {  // 8 rows' loads in flight at a time
    uint64_t y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = min(max(s_inv[min(j0 + u, a.k - 1)], 0), a.R - 1);
      y[u] = cld(a.yw + (size_t)r * a.H + nn);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < a.k) {
        ok &= is_mine(a, y[u]);
        v = fmaf(s_w[j0 + u], __uint_as_float((uint32_t)y[u]), v);
      }
  }
  const uint64_t bad = __ballot(valid && !ok);
  const bool done = lane < 32 ? (uint32_t)bad == 0u : (uint32_t)(bad >> 32) == 0u;
  if (valid && done) a.out[n] = failed ? __builtin_nanf("") : v;
}

// Completion flags of the shared expert's gate/up items in the one-token
// launch: one tagged word per item, after the routing copies.
__device__ __forceinline__ uint64_t* shared_flags(const DecodeArgs& a) {
  return a.tagged + 2 * a.E + (size_t)kReplicas * kReplicaWords;
}

// LDS of a down workgroup of the one-token launch: the slot table, the slot
// and weight of each choice j (for the combine), then the staged h row.
struct DownLds {
  int* tab;
  int* inv;
  float* w;
  f32x4_t* h;
  __device__ DownLds(const DecodeArgs& a, char* lds)
      : tab(reinterpret_cast<int*>(lds)),
        inv(tab + 1 + 3 * a.max_slots),
        w(reinterpret_cast<float*>(inv + a.k)),
        h(reinterpret_cast<f32x4_t*>(lds + 1024 * sizeof(int))) {}
};

// The waits of a shared down workgroup, a wave each: the routing copy and
// the routing weights (for the combine) and the shared gate/up flags.
__device__ void shared_down_waits(const DecodeArgs& a, int n_sh, const DownLds& L) {
  const int wave = threadIdx.x >> 6;
  if (wave == 0) {
    uint32_t v[6];
    poll_tagged<6, 1>(a, a.tag, kSpinLimit, kWaitShared, shared_flags(a), n_sh, v);
  } else if (wave == 1) {
    routing_copy(a, blockIdx.x % kReplicas, L.tab, L.inv);
  } else if (wave == 2) {
    routing_weights(a, blockIdx.x % kReplicas, L.w);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// The shared expert in FP8 (E4M3 bytes, one E8M0 scale per 32 x 32 block),
// one token, inside the fused launch: the same item split, flags and
// dispatch slots as the MXFP4 shared expert, with twice the weight bytes per
// item. The gfx950 scaled FP8 conversions apply each block's power of two
// exactly (E4M3 x 2^s is representable in bf16 and fp32).
// ---------------------------------------------------------------------------
constexpr int kF8GuU = 10;  // gate/up: 32 lanes per column x 10 chunks of 16 B (K <= 5120)
constexpr int kF8DnU = 18;  // down: 8 lanes per row x 18 chunks of 16 B (K <= 2304)

__device__ __forceinline__ float dot16_fp8s_bf16(uint4 w, float sc, uint4 x0, uint4 x1, float acc) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  const uint32_t xx[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[i], sc, false),
                                          as_bf16x2(xx[2 * i]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[i], sc, true),
                                          as_bf16x2(xx[2 * i + 1]), acc, false);
  }
  return acc;
}

// Gate/up item: columns 8 item .. 8 item + 7 of the shared h row (2 per
// wave, 32 lanes per column); h stored write-through for the down items of
// this launch.
__device__ void fp8_shared_gu_item(const DecodeArgs& a, int item, uint4* s_x) {
  const int H = a.H, I = a.I;
  const int lane = lane_id(), wave = threadIdx.x >> 6, j = lane & 31;
  const int n = item * kGuRows + wave * 2 + (lane >> 5);
  const bool ok = n < I;
  const int nr = ok ? n : I - 1;
  const int nch = H >> 4, sb = H >> 5;
  const __amdgpu_buffer_rsrc_t rg = matrix_rsrc(a.sh8_gu_w, (uint32_t)I * H);
  const __amdgpu_buffer_rsrc_t ru = matrix_rsrc(a.sh8_gu_w + (size_t)I * H, (uint32_t)I * H);
  const __amdgpu_buffer_rsrc_t rs = matrix_rsrc(a.sh8_gu_s, (uint32_t)(2 * (I >> 5) * sb));
  uint4 wg[kF8GuU], wu[kF8GuU];
  uint32_t sg[kF8GuU], su[kF8GuU];
#pragma unroll
  for (int u = 0; u < kF8GuU; ++u) {
    const int c = j + 32 * u;
    wg[u] = bload16(rg, nr * H + c * 16);
    wu[u] = bload16(ru, nr * H + c * 16);
    sg[u] = bload8(rs, (nr >> 5) * sb + (c >> 1));
    su[u] = bload8(rs, ((I + nr) >> 5) * sb + (c >> 1));
  }
  stage_rows<uint4>(
      H >> 3, [&](int idx) { return reinterpret_cast<const uint4*>(a.x)[idx]; },
      [&](int idx, uint4 v) { s_x[idx] = v; });
  __syncthreads();
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int u = 0; u < kF8GuU; ++u) {
    const int c = j + 32 * u;
    if (c < nch) {
      const uint4 x0 = s_x[2 * c], x1 = s_x[2 * c + 1];
      ag = dot16_fp8s_bf16(wg[u], e8m0_to_f32(sg[u]), x0, x1, ag);
      au = dot16_fp8s_bf16(wu[u], e8m0_to_f32(su[u]), x0, x1, au);
    }
  }
  ag = group_sum<32>(ag);
  au = group_sum<32>(au);
  if (ok && j == 0) cst(a.h + (size_t)a.R * I + n, silu_mul(ag, au));
}

// Down item c: 32 output rows of the shared y row, 8 lanes per row. The
// weights are requested before the wait for the gate/up flags; h is read
// coherently once they are all up.
__device__ void fp8_shared_down_item(const DecodeArgs& a, int c, int n_sh, const DownLds& L) {
  const int H = a.H, I = a.I;
  const int q = threadIdx.x & 7;
  const int n = c * kDnRows + (threadIdx.x >> 3);
  const bool ok = n < H;
  const int nr = ok ? n : H - 1;
  const int nch = I >> 4, sb = I >> 5;
  const __amdgpu_buffer_rsrc_t rd = matrix_rsrc(a.sh8_d_w, (uint32_t)H * I);
  const __amdgpu_buffer_rsrc_t rs = matrix_rsrc(a.sh8_d_s, (uint32_t)((H >> 5) * sb));
  uint4 wd[kF8DnU];
  uint32_t sd[kF8DnU];
#pragma unroll
  for (int u = 0; u < kF8DnU; ++u) {
    const int cc = q + 8 * u;
    wd[u] = bload16(rd, nr * I + cc * 16);
    sd[u] = bload8(rs, (nr >> 5) * sb + (cc >> 1));
  }
  shared_down_waits(a, n_sh, L);
  f32x4_t* s_h = L.h;
  const uint64_t* hrow = reinterpret_cast<const uint64_t*>(a.h + (size_t)a.R * I);
  for (int f = threadIdx.x; f < (I >> 2); f += kThreads) {
    const uint64_t lo = cld(hrow + 2 * f), hi = cld(hrow + 2 * f + 1);
    s_h[f] = f32x4_t{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                     __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
  }
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kF8DnU; ++u) {
    const int cc = q + 8 * u;
    if (cc < nch) {
      const float f = e8m0_to_f32(sd[u]);
      const uint32_t ww[4] = {wd[u].x, wd[u].y, wd[u].z, wd[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4_t h4 = s_h[4 * cc + i];
        const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ww[i], f, false);
        const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ww[i], f, true);
        acc = fmaf(p0.x, h4.x, acc);
        acc = fmaf(p0.y, h4.y, acc);
        acc = fmaf(p1.x, h4.z, acc);
        acc = fmaf(p1.y, h4.w, acc);
      }
    }
  }
  acc = group_sum<8>(acc);
  if (ok && q == 0) cst(a.yw + (size_t)a.R * H + n, value_word(a, acc));
}

// NVFP4 shared expert, one token: gate/up item (h write-through) and down
// item (after the gate/up flags), as the MXFP4 ones.
__device__ void nv_shared_gu_item(const DecodeArgs& a, int item, uint4* s_x) {
  GuRegs r;
  gu_issue_nv(a, a.shared.gu_codes, a.shared.gu_scales, item, r, true);
  stage_rows<uint4>(
      a.H >> 3, [&](int idx) { return reinterpret_cast<const uint4*>(a.x)[idx]; },
      [&](int idx, uint4 v) { s_x[(idx & 3) * (kGuLanes * kGuU) + (idx >> 2)] = v; });
  __syncthreads();
  gu_compute_nv<false>(a, item, min(a.R, a.rows - 1), nv_matrix_scale(a.shared, 0, 0),
                      nv_matrix_scale(a.shared, 0, 1), r, s_x);
}

// Down items c0 and c0 + 1 (live1: the second exists) of one slot, or of
// the shared expert (slot < 0), in one workgroup of the one-token launch:
// both items' weights are in flight before the wait for the slot's h row
// (its value words, or the shared gate/up flags and then the shared row),
// which is read once. A routed pair takes the routing copy first (it names
// the expert); a shared pair requests its weights at once.
template <bool NV>
__device__ void down_pair(const DecodeArgs& a, int slot, int c0, bool live1, int n_sh,
                          const DownLds& L) {
  const int r = blockIdx.x % kReplicas;
  const int nr = a.max_slots * a.dn_items;
  const int wave = threadIdx.x >> 6;
  const int it = slot < 0 ? nr + c0 : slot * a.dn_items + c0;
  DnRegs A, B;
  auto issue = [&](int i, DnRegs& R, bool live) {
    if constexpr (NV)
      dn_issue_nv(a, L.tab, nr, i, R, live, false);
    else
      dn_issue(a, L.tab, nr, i, R, live, false);
  };
  if (slot < 0) {
    issue(it, A, true);
    issue(live1 ? it + 1 : it, B, live1);
    if (wave == 0) {
      uint32_t v[6];
      poll_tagged<6, 1>(a, a.tag, kSpinLimit, kWaitShared, shared_flags(a), n_sh, v);
    } else if (wave == 1) {
      routing_copy(a, r, L.tab, L.inv);
    } else if (wave == 2) {
      routing_weights(a, r, L.w);
    }
    __syncthreads();
  } else {
    if (wave == 0)
      routing_copy(a, r, L.tab, L.inv);
    else if (wave == 1)
      routing_weights(a, r, L.w);
    __syncthreads();
    issue(it, A, true);
    issue(live1 ? it + 1 : it, B, live1);
  }
  if (slot < 0)
    dn_issue_h<true>(a, min(a.R, a.rows - 1), A);
  else
    poll_h_words(a, min(max(L.tab[1 + a.max_slots + slot], 0), a.rows - 1), A);
#pragma unroll
  for (int i = 0; i < 3; ++i) B.h[i] = A.h[i];
  auto compute = [&](int i, const DnRegs& R) {
    if constexpr (NV)
      dn_compute_nv(a, L.tab, nr, i, R, L.h);
    else
      dn_compute(a, L.tab, nr, i, R, L.h);
  };
  compute(it, A);
  if (live1) compute(it + 1, B);
}

// After a workgroup's down items (column groups c0, and c0 + 1 if live1):
// once their y words have landed, combine whichever of the groups has all
// its parts. Every wait whose data reach a group comes before that group's
// last part is written, so its combine sees any of them that gave up in
// the status word and writes NaN.
__device__ void finish_parts(const DecodeArgs& a, int c0, bool live1, const DownLds& L) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < kWave) try_combine(a, c0, live1, L.inv, L.w, call_wait_code(a) != 0);
}

// The whole one-token layer in one launch, workgroups in dispatch order:
// [router rows | the routing workgroup | shared gate/up items | G routed
// gate/up workgroups | shared down items | routed down items].
// * The routed gate/up workgroups stage the token, poll a replica of the
//   routing table and then stream the items b, b + G, ... of the selected
//   experts (slot-major, 8 rows each) with two register buffers, so the
//   weights of the next item are in flight while the current one is
//   computed. Each item counts itself for its slot once its h rows have
//   landed.
// * The down items (32 output rows each) come last, so they are dispatched
//   as gate/up workgroups retire: each requests its weights at once and then
//   waits for its h row (the slot's count, or the shared flags), and the
//   last of a column group's items combines it.
// A workgroup waits only on workgroups before it in dispatch order, which
// were dispatched before it and never wait on it.
// NV: NVFP4 banks (routed and shared); otherwise MXFP4 (shared possibly FP8).
template <bool NV>
__global__ __launch_bounds__(kThreads, 3) void gateup_fused_kernel(DecodeArgs a, int n_shared,
                                                                int n_sd, int G, int per,
                                                                int dpw, int ns_pair) {
  extern __shared__ __align__(16) char lds[];
  const int b0 = blockIdx.x;
  if (b0 < a.nb_router) {
    router_rows_one(a, b0, reinterpret_cast<uint4*>(lds));
    return;
  }
  if (b0 == a.nb_router) {
    if (threadIdx.x < kWave) {
      if (a.E <= 6 * kWave)
        route_token_tagged<6>(a);
      else
        route_token_tagged<16>(a);
    }
    return;
  }
  if (b0 <= a.nb_router + n_shared) {
    // a shared gate/up item, then its flag once its h stores have landed
    const int item = b0 - a.nb_router - 1;
    if constexpr (NV)
      nv_shared_gu_item(a, item, reinterpret_cast<uint4*>(lds));
    else if (a.shared_fp8)
      fp8_shared_gu_item(a, item, reinterpret_cast<uint4*>(lds));
    else
      gateup_item<1, true>(a, shared_slot(a), item, reinterpret_cast<uint4*>(lds), nullptr);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) cst(shared_flags(a) + item, tag_word(a.tag, 1));
    return;
  }
  if (b0 >= a.nb_router + 1 + n_shared + G) {
    // down workgroups: dpw (1 or 2) column groups each (one for the FP8
    // shared expert), the shared expert's first, then slot by slot; slots
    // from ns_pair on take one column group per workgroup
    const int d = b0 - (a.nb_router + 1 + n_shared + G);
    const DownLds L(a, lds);
    const int per_slot = (a.dn_items + dpw - 1) / dpw;
    if (d < n_sd && !NV && a.shared_fp8) {
      fp8_shared_down_item(a, d, n_shared, L);
      finish_parts(a, d, false, L);
      return;
    }
    const int dr = d - n_sd, n_pair = ns_pair * per_slot;
    int slot = -1, c0 = dpw * d;
    bool live1 = dpw == 2 && c0 + 1 < a.dn_items;
    if (d >= n_sd && dr < n_pair) {
      slot = dr / per_slot;
      c0 = dpw * (dr - slot * per_slot);
      live1 = dpw == 2 && c0 + 1 < a.dn_items;
    } else if (d >= n_sd) {
      slot = ns_pair + (dr - n_pair) / a.dn_items;
      c0 = (dr - n_pair) % a.dn_items;
      live1 = false;
    }
    down_pair<NV>(a, slot, c0, live1, n_shared, L);
    finish_parts(a, c0, live1, L);
    return;
  }
  const int b = b0 - a.nb_router - 1 - n_shared;
  uint4* s_x = reinterpret_cast<uint4*>(lds);
  int* tab = reinterpret_cast<int*>(lds + a.H * 2);
  stage_rows<uint4>(
      a.H >> 3, [&](int idx) { return reinterpret_cast<const uint4*>(a.x)[idx]; },
      [&](int idx, uint4 v) { s_x[(idx & 3) * (kGuLanes * kGuU) + (idx >> 2)] = v; });
  load_routing_tagged(a, b % kReplicas, tab);
  const int n = tab[0] * a.gu_items;
  // Items first .. first + mine - 1, contiguous, so the slots complete in
  // the order their workgroups are dispatched. Fixed trip over pairs of
  // items with no early exit (an exit between the halves would let the
  // compiler merge them and move the buffers to scratch). Issues past this
  // workgroup's last item are padding: their weight loads read nothing
  // (empty resources) and are not used.
  const int first = b * per;
  const int mine = max(0, min(per, n - first));
  GuRegs A, B;
  auto issue = [&](int it, GuRegs& r, bool live) {
    if constexpr (NV)
      gu_issue_nv_routed(a, tab, it, r, live);
    else
      gu_issue(a, tab, it, r, live);
  };
  auto compute = [&](int it, const GuRegs& r) {
    if constexpr (NV)
      gu_compute_nv_routed(a, tab, it, r, s_x);
    else
      gu_compute(a, tab, it, r, s_x);
  };
  issue(mine > 0 ? first : 0, A, mine > 0);
  for (int kk = 0; kk < mine; kk += 2) {
    const int i0 = first + kk;
    const bool l1 = kk + 1 < mine, l2 = kk + 2 < mine;
    issue(l1 ? i0 + 1 : i0, B, l1);
    compute(i0, A);
    issue(l2 ? i0 + 2 : i0, A, l2);
    if (l1) compute(i0 + 1, B);
  }
}

// ---------------------------------------------------------------------------
// A block of a few tokens (2 <= T <= kBlockT, a verification block): the
// one-token streaming design over the union of the block's experts. A
// verification step pays for the union of its tokens' experts (ai.rs
// article, "The draft head that works and does not pay"), so each selected
// expert's rows are read once per call and used for every token routed to
// it. Launch 1 is the router and the routing (route_kernel without shared
// items); launch 2 streams the gate/up items of the shared expert and of
// every routed slot, each item's weights in registers while the slot's
// tokens are taken from the block staged in LDS; launch 3 streams the down
// items the same way, and the workgroup that completes a column group
// combines it for every token.
// ---------------------------------------------------------------------------
// The block kernels are instantiated for at most TB = 5 and TB = 8 tokens
// (the smaller keeps the gate/up workgroups at three a CU).
constexpr int kBlockT = 8;
constexpr int kXRow = 4 * kGuLanes * kGuU;  // uint4 per staged token row (H <= 5120)
constexpr int kBlockXLoads = 20;            // router: T * H / 8 <= 20 * kThreads

// Gate/up item `it` of the block: items [0, n_sh) are the shared expert's
// 8-row groups (all T tokens), then (routed slot, 8-row group) pairs,
// slot-major. Every field is clamped to the bank and rows that exist.
struct BlkItem {
  const uint8_t* codes;
  const uint8_t* scales;
  int rb;     // row group
  int row0;   // first h / y row of the slot
  int m;      // the slot's rows (tokens)
  bool shared;
  int e;      // routed expert (NVFP4 matrix scales); -1: the shared expert
};

// A small table held across the lanes of a wave: entry i sits in lane
// i % 64 of word i / 64, and is read with readlane (the index is uniform).
// It keeps the slot table off LDS and off the path of memory latency.
struct LaneTable {
  static constexpr int kMax = 256;  // entries
  int v[4];
  __device__ __forceinline__ void load(const int* src, int n) {
    const int l = lane_id();
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = src[min(64 * q + l, n - 1)];
  }
  __device__ __forceinline__ int operator[](int i) const {
    i = min(max(__builtin_amdgcn_readfirstlane(i), 0), kMax - 1);
    const int w = i < 64 ? v[0] : i < 128 ? v[1] : i < 192 ? v[2] : v[3];
    return __builtin_amdgcn_readlane(w, i & 63);
  }
};

template <int TB, bool NV, class Tab>
__device__ __forceinline__ BlkItem blk_item(const DecodeArgs& a, const Tab& tab, int n_sh, int it,
                                            int per, bool gu) {
  const uint32_t crow = (uint32_t)(gu ? a.H : a.I) >> 1;
  const uint32_t srow = (uint32_t)(gu ? a.H : a.I) >> (NV ? 4 : 5);
  const size_t mat = gu ? 2 * (size_t)a.I : (size_t)a.H;
  const uint8_t* c0 = gu ? a.routed.gu_codes : a.routed.d_codes;
  const uint8_t* s0 = gu ? a.routed.gu_scales : a.routed.d_scales;
  if (it < n_sh)
    return BlkItem{gu ? a.shared.gu_codes : a.shared.d_codes,
                   gu ? a.shared.gu_scales : a.shared.d_scales, it, a.R, min(a.T, TB), true, -1};
  const int q = it - n_sh, sl = q / per, rb = q - sl * per;
  const int e = __builtin_amdgcn_readfirstlane(min(max(tab[1 + sl], 0), a.routed.E - 1));
  const int row0 = min(max(tab[1 + a.max_slots + sl], 0), a.R);
  const int m = min(max(tab[1 + 2 * a.max_slots + sl], 0), min(a.R - row0, TB));
  return BlkItem{c0 + (size_t)e * mat * crow, s0 + (size_t)e * mat * srow, rb, row0, m, false, e};
}

// NV: an NVFP4 bank, whose 32-code chunk j + 32 u has its two scale bytes
// in half j % 2 of the word at 4 (j / 2) + 64 u of the row's H / 16.
template <bool NV>
__device__ __forceinline__ void gu_issue_blk(const DecodeArgs& a, const BlkItem& d, GuRegs& r,
                                             bool live) {
  live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & (kGuLanes - 1);
  const int nr = min(d.rb * kGuRows + wave * (kWave / kGuLanes) + lane / kGuLanes, a.I - 1);
  const uint32_t crow = (uint32_t)a.H >> 1, srow = (uint32_t)a.H >> (NV ? 4 : 5);
  const uint8_t* gbase = uniform_ptr(d.codes);
  const uint8_t* sbase = uniform_ptr(d.scales);
  const uint32_t cb = live ? a.I * crow : 0u, sb = live ? a.I * srow : 0u;
  const __amdgpu_buffer_rsrc_t rg = matrix_rsrc(gbase, cb);
  const __amdgpu_buffer_rsrc_t ru = matrix_rsrc(gbase + (size_t)a.I * crow, cb);
  const __amdgpu_buffer_rsrc_t rgs = matrix_rsrc(sbase, sb);
  const __amdgpu_buffer_rsrc_t rus = matrix_rsrc(sbase + (size_t)a.I * srow, sb);
  const int co = nr * crow + j * 16, so = nr * srow + (NV ? 4 * (j >> 1) : (j & ~3));
  constexpr int su_step = NV ? 2 * kGuLanes : kGuLanes;
#pragma unroll
  for (int u = 0; u < kGuU; ++u) {
    r.g[u] = bload16(rg, co + u * kGuLanes * 16);
    r.u[u] = bload16(ru, co + u * kGuLanes * 16);
    r.sg[u] = bload32(rgs, so + u * su_step);
    r.su[u] = bload32(rus, so + u * su_step);
  }
}

// One item's rows for each of the slot's tokens: each 16-byte chunk of
// weights is converted to bf16 once and used for every token, whose row
// comes from the staged block at s_x + t * kXRow. Unrolled over the block
// (no loop-carried store, so the waits for this item's weights do not also
// wait for the next item's).
template <int TB, bool NV, class Tab>
__device__ __forceinline__ void gu_compute_blk(const DecodeArgs& a, const BlkItem& d,
                                               const Tab& s_rt, const GuRegs& r,
                                               const uint4* s_x) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & (kGuLanes - 1);
  const int n = d.rb * kGuRows + wave * (kWave / kGuLanes) + lane / kGuLanes;
  const int kc = a.H >> 5;
  const uint32_t sh = 8u * (j & 3);
  constexpr int P = kGuLanes * kGuU;
  const uint4* xt[TB];
  float ag[TB], au[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int t = i >= d.m ? 0 : d.shared ? i : min(max(s_rt[d.row0 + i], 0), a.T - 1);
    xt[i] = s_x + t * kXRow;
    ag[i] = au[i] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < kGuU; ++u) {
    const int c = kGuLanes * u + j;
    if (c < kc) {
      // MXFP4: one scale per chunk; NVFP4: one per 16-code half (.x, .y)
      f32x2_t fg, fu;
      if constexpr (NV) {
        fg = nv_scale_pair(r.sg[u], 16u * (j & 1));
        fu = nv_scale_pair(r.su[u], 16u * (j & 1));
      } else {
        fg.x = fg.y = e8m0_to_f32(__builtin_amdgcn_ubfe(r.sg[u], sh, 8));
        fu.x = fu.y = e8m0_to_f32(__builtin_amdgcn_ubfe(r.su[u], sh, 8));
      }
      const uint32_t gw[4] = {r.g[u].x, r.g[u].y, r.g[u].z, r.g[u].w};
      const uint32_t uw[4] = {r.u[u].x, r.u[u].y, r.u[u].z, r.u[u].w};
      bf16x2_t wg[16], wu[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wg[4 * q + 0] = fp4x2_to_bf16<0>(gw[q]);
        wg[4 * q + 1] = fp4x2_to_bf16<1>(gw[q]);
        wg[4 * q + 2] = fp4x2_to_bf16<2>(gw[q]);
        wg[4 * q + 3] = fp4x2_to_bf16<3>(gw[q]);
        wu[4 * q + 0] = fp4x2_to_bf16<0>(uw[q]);
        wu[4 * q + 1] = fp4x2_to_bf16<1>(uw[q]);
        wu[4 * q + 2] = fp4x2_to_bf16<2>(uw[q]);
        wu[4 * q + 3] = fp4x2_to_bf16<3>(uw[q]);
      }
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        if (i < d.m) {
          const uint4* xv = xt[i] + c;
          float pg[2] = {0.0f, 0.0f}, pu[2] = {0.0f, 0.0f};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 xq = xv[q * P];
            const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w};
            const int hf = NV ? q >> 1 : 0;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              pg[hf] = __builtin_amdgcn_fdot2_f32_bf16(wg[4 * q + p], as_bf16x2(xw[p]), pg[hf], false);
              pu[hf] = __builtin_amdgcn_fdot2_f32_bf16(wu[4 * q + p], as_bf16x2(xw[p]), pu[hf], false);
            }
          }
          if constexpr (NV) {
            ag[i] = fmaf(pg[1], fg.y, fmaf(pg[0], fg.x, ag[i]));
            au[i] = fmaf(pu[1], fu.y, fmaf(pu[0], fu.x, au[i]));
          } else {
            ag[i] = fmaf(pg[0], fg.x, ag[i]);
            au[i] = fmaf(pu[0], fu.x, au[i]);
          }
        }
      }
    }
  }
  float mg = 1.0f, mu = 1.0f;  // NVFP4 matrix scales, applied to the row sums
  if constexpr (NV) {
    const BankView& bv = d.e < 0 ? a.shared : a.routed;
    mg = nv_matrix_scale(bv, max(d.e, 0), 0);
    mu = nv_matrix_scale(bv, max(d.e, 0), 1);
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    if (i < d.m) {
      float g = group_sum<kGuLanes>(ag[i]), u = group_sum<kGuLanes>(au[i]);
      if constexpr (NV) {
        g *= mg;
        u *= mu;
      }
      if (j == 0 && n < a.I) a.h[(size_t)(d.row0 + i) * a.I + n] = silu_mul(g, u);
    }
  }
}

// Block router rows: a wave per expert row, the row's loads issued before
// the block's T token rows are staged in LDS, then T dot products. Each
// logit goes out as one tagged word, which the routing wave's poll returns
// with its value: no flag, and no second read once the flags are seen.
__device__ void router_rows_blk(const DecodeArgs& a, int b, uint4* s_x) {
  const int lane = lane_id();
  const int e0 = b * 4 + (int)(threadIdx.x >> 6);
  const int e = min(e0, a.E - 1);
  const int nv = a.H >> 3;
  const uint4* wrow = reinterpret_cast<const uint4*>(a.wr + (size_t)e * a.H);
  // the block's rows first (L2, all loads in flight together: T * H / 8 <=
  // 16 * 256), then the weight row (HBM), so staging waits for the rows only
  const int total = a.T * nv;
  const uint4* xs = reinterpret_cast<const uint4*>(a.x);
  uint4 v[kBlockXLoads];
#pragma unroll
  for (int i = 0; i < kBlockXLoads; ++i) v[i] = xs[min((int)threadIdx.x + i * kThreads, total - 1)];
  uint4 wv[kRouterV];
#pragma unroll
  for (int i = 0; i < kRouterV; ++i) wv[i] = wrow[min(lane + kWave * i, nv - 1)];
#pragma unroll
  for (int i = 0; i < kBlockXLoads; ++i)
    if ((int)threadIdx.x + i * kThreads < total) s_x[threadIdx.x + i * kThreads] = v[i];
  __syncthreads();
  const float bb = a.bias ? a.bias[e] : 0.0f;
  // token by token, each logit published as soon as it is summed (all the
  // block's dot products first, then every logit, measured slower: the
  // routing waves start on the early tokens while the later ones are summed)
  for (int t = 0; t < a.T; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kRouterV; ++i)
      if (lane + kWave * i < nv) acc = dot8_bf16(wv[i], s_x[t * nv + lane + kWave * i], acc);
    acc = wave_sum(acc);
    if (lane == 0 && e0 < a.E) {
      const uint32_t v = __float_as_uint(acc + bb);
      cst(a.tagged + (size_t)t * 2 * a.E + e, tag_word(a.tag, v));
      cst(a.tagged + (size_t)t * 2 * a.E + a.E + e, tag_word(a.tag, v >> 16));
    }
  }
}

// The block's T token rows into LDS (row t at s_x + t * kXRow, chunk-
// transposed like the one-token row).
__device__ __forceinline__ void stage_block_rows(const DecodeArgs& a, uint4* s_x) {
  const int T = min(a.T, kBlockT);  // the host keeps T within the instantiation's TB
  const int nv = a.H >> 3;
  stage_rows<uint4>(
      T * nv, [&](int idx) { return reinterpret_cast<const uint4*>(a.x)[idx]; },
      [&](int idx, uint4 v) {
        const int t = idx / nv, q = idx - t * nv;
        s_x[t * kXRow + (q & 3) * (kGuLanes * kGuU) + (q >> 2)] = v;
      });
}

// Streams gate/up items b, b + G, ... < n (item numbering of blk_item with
// n_sh shared items first) with two register buffers.
template <int TB, bool NV, class Tab>
__device__ __forceinline__ void gateup_block_items(const DecodeArgs& a, const Tab& s_tab,
                                                   const Tab& s_rt, const uint4* s_x, int n_sh,
                                                   int n, int b, int G) {
  // fixed trip over pairs of items; padding issues read nothing
  const int mine = b < n ? (n - b + G - 1) / G : 0;
  GuRegs A, B;
  auto item = [&](int it) { return blk_item<TB, NV>(a, s_tab, n_sh, it, a.gu_items, true); };
  gu_issue_blk<NV>(a, item(b < n ? b : 0), A, b < n);
  for (int kk = 0; kk < mine; kk += 2) {
    const int i0 = b + kk * G, i1 = i0 + G, i2 = i1 + G;
    gu_issue_blk<NV>(a, item(i1 < n ? i1 : i0), B, i1 < n);
    gu_compute_blk<TB, NV>(a, item(i0), s_rt, A, s_x);
    gu_issue_blk<NV>(a, item(i2 < n ? i2 : i0), A, i2 < n);
    if (i1 < n) gu_compute_blk<TB, NV>(a, item(i1), s_rt, B, s_x);
  }
}

// FP8 shared expert in the block launches: the columns and rows of the
// one-token FP8 items, each 16-byte weight chunk converted once and used for
// every token of the block. Gate/up item `item` (the route launch): 8
// columns of the block's shared h rows R .. R + T - 1, 32 lanes per column;
// the weights are requested before the token rows are staged (row t at
// s_x + t * H / 8, when `stage`).
template <int TB>
__device__ void fp8_shared_gu_blk(const DecodeArgs& a, int item, uint4* s_x, bool stage) {
  const int H = a.H, I = a.I, T = min(a.T, TB);
  const int lane = lane_id(), wave = threadIdx.x >> 6, j = lane & 31;
  const int n = item * kGuRows + wave * 2 + (lane >> 5);
  const bool ok = n < I;
  const int nr = ok ? n : I - 1;
  const int nch = H >> 4, sb = H >> 5, nv = H >> 3;
  const __amdgpu_buffer_rsrc_t rg = matrix_rsrc(a.sh8_gu_w, (uint32_t)I * H);
  const __amdgpu_buffer_rsrc_t ru = matrix_rsrc(a.sh8_gu_w + (size_t)I * H, (uint32_t)I * H);
  const __amdgpu_buffer_rsrc_t rs = matrix_rsrc(a.sh8_gu_s, (uint32_t)(2 * (I >> 5) * sb));
  uint4 wg[kF8GuU], wu[kF8GuU];
  uint32_t sg[kF8GuU], su[kF8GuU];
#pragma unroll
  for (int u = 0; u < kF8GuU; ++u) {
    const int c = j + 32 * u;
    wg[u] = bload16(rg, nr * H + c * 16);
    wu[u] = bload16(ru, nr * H + c * 16);
    sg[u] = bload8(rs, (nr >> 5) * sb + (c >> 1));
    su[u] = bload8(rs, ((I + nr) >> 5) * sb + (c >> 1));
  }
  if (stage) {
    stage_rows<uint4>(
        T * nv, [&](int idx) { return reinterpret_cast<const uint4*>(a.x)[idx]; },
        [&](int idx, uint4 v) { s_x[idx] = v; });
    __syncthreads();
  }
  float ag[TB], au[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) ag[t] = au[t] = 0.0f;
#pragma unroll
  for (int u = 0; u < kF8GuU; ++u) {
    const int c = j + 32 * u;
    if (c < nch) {
      const float fg = e8m0_to_f32(sg[u]), fu = e8m0_to_f32(su[u]);
      const uint32_t gw[4] = {wg[u].x, wg[u].y, wg[u].z, wg[u].w};
      const uint32_t uw[4] = {wu[u].x, wu[u].y, wu[u].z, wu[u].w};
      bf16x2_t g2[8], u2[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g2[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw[i], fg, false);
        g2[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw[i], fg, true);
        u2[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(uw[i], fu, false);
        u2[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(uw[i], fu, true);
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t < T) {
          const uint4 x0 = s_x[t * nv + 2 * c], x1 = s_x[t * nv + 2 * c + 1];
          const uint32_t xx[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            ag[t] = __builtin_amdgcn_fdot2_f32_bf16(g2[p], as_bf16x2(xx[p]), ag[t], false);
            au[t] = __builtin_amdgcn_fdot2_f32_bf16(u2[p], as_bf16x2(xx[p]), au[t], false);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    if (t < T) {
      const float g = group_sum<32>(ag[t]), u = group_sum<32>(au[t]);
      if (ok && j == 0) a.h[(size_t)(a.R + t) * I + n] = silu_mul(g, u);
    }
  }
}

// Down item c (the gate/up launch's tail): 32 rows of the block's shared y
// rows, 8 lanes per row, from the h rows the route launch wrote (staged in
// LDS, row t at s_h + t * I / 4, after the weights are requested).
template <int TB>
__device__ void fp8_shared_down_blk(const DecodeArgs& a, int c, f32x4_t* s_h) {
  const int H = a.H, I = a.I, T = min(a.T, TB);
  const int q = threadIdx.x & 7;
  const int n = c * kDnRows + (threadIdx.x >> 3);
  const bool ok = n < H;
  const int nr = ok ? n : H - 1;
  const int nch = I >> 4, sb = I >> 5, nv = I >> 2;
  const __amdgpu_buffer_rsrc_t rd = matrix_rsrc(a.sh8_d_w, (uint32_t)H * I);
  const __amdgpu_buffer_rsrc_t rs = matrix_rsrc(a.sh8_d_s, (uint32_t)((H >> 5) * sb));
  uint4 wd[kF8DnU];
  uint32_t sd[kF8DnU];
#pragma unroll
  for (int u = 0; u < kF8DnU; ++u) {
    const int cc = q + 8 * u;
    wd[u] = bload16(rd, nr * I + cc * 16);
    sd[u] = bload8(rs, (nr >> 5) * sb + (cc >> 1));
  }
  const f32x4_t* hrows = reinterpret_cast<const f32x4_t*>(a.h + (size_t)a.R * I);
  for (int f = threadIdx.x; f < T * nv; f += kThreads) s_h[f] = hrows[f];
  __syncthreads();
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int u = 0; u < kF8DnU; ++u) {
    const int cc = q + 8 * u;
    if (cc < nch) {
      const float f = e8m0_to_f32(sd[u]);
      const uint32_t ww[4] = {wd[u].x, wd[u].y, wd[u].z, wd[u].w};
      f32x2_t p[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ww[i], f, false);
        p[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ww[i], f, true);
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t < T) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4_t h4 = s_h[t * nv + 4 * cc + i];
            acc[t] = fmaf(p[2 * i].x, h4.x, acc[t]);
            acc[t] = fmaf(p[2 * i].y, h4.y, acc[t]);
            acc[t] = fmaf(p[2 * i + 1].x, h4.z, acc[t]);
            acc[t] = fmaf(p[2 * i + 1].y, h4.w, acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    if (t < T) {
      const float v = group_sum<8>(acc[t]);
      if (ok && q == 0) cst(a.y + (size_t)(a.R + t) * H + n, v);
    }
  }
}

// Block launch 1: [router rows | the routing workgroup | n_sw workgroups
// streaming the shared expert's gate/up items (MXFP4 or FP8), which need no
// routing and use the bandwidth the router and the routing leave idle].
template <int TB, bool NV>
__global__ __launch_bounds__(kThreads) void route_block_kernel(DecodeArgs a, int n_sw) {
  extern __shared__ __align__(16) char lds[];
  const int b = blockIdx.x;
  if (b < a.nb_router) {
    router_rows_blk(a, b, reinterpret_cast<uint4*>(lds));
  } else if (b == a.nb_router) {
    routing<true>(a, lds);
  } else if (a.shared_fp8) {
    bool stage = true;
    for (int it = b - a.nb_router - 1; it < a.gu_items; it += n_sw, stage = false)
      fp8_shared_gu_blk<TB>(a, it, reinterpret_cast<uint4*>(lds), stage);
  } else {
    uint4* s_x = reinterpret_cast<uint4*>(lds);
    stage_block_rows(a, s_x);
    __syncthreads();
    const int* none = nullptr;
    gateup_block_items<TB, NV>(a, none, none, s_x, a.gu_items, a.gu_items, b - a.nb_router - 1,
                               n_sw);
  }
}

struct DnW {
  uint4 w[kDnU];
  uint32_t sc[kDnU];
};

// NV: chunk j + 8 u's two scale bytes are half j % 2 of the word at
// 4 (j / 2) + 16 u of the row's I / 16.
template <bool NV>
__device__ __forceinline__ void dn_issue_blk(const DecodeArgs& a, const BlkItem& d, DnW& r,
                                             bool live) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int nr = min(d.rb * kDnRows + wave * 8 + (lane >> 3), a.H - 1);
  const uint32_t crow = (uint32_t)a.I >> 1, srow = (uint32_t)a.I >> (NV ? 4 : 5);
  live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  const __amdgpu_buffer_rsrc_t rd = matrix_rsrc(uniform_ptr(d.codes), live ? a.H * crow : 0u);
  const __amdgpu_buffer_rsrc_t rds = matrix_rsrc(uniform_ptr(d.scales), live ? a.H * srow : 0u);
  const int co = nr * crow + j * 16, so = nr * srow + (NV ? 4 * (j >> 1) : 4 * (j >> 2));
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    r.w[u] = bload16(rd, co + u * 8 * 16);
    r.sc[u] = bload32(rds, so + u * (NV ? 16 : 8));
  }
}

// Direct global -> LDS copy: lane l's 16 bytes at base + voff land at LDS
// byte address lds + 16 l (lds wave-uniform). Invisible to the compiler's
// wait counting: the caller waits for it explicitly.
// m0 is named as clobbered so the compiler keeps nothing there and puts
// the needed wait state between a copy and the next write of m0 (clang's
// warning that m0 is reserved is silenced here only).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
               :
               : "v"(voff), "s"(lds), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr int kHRow = 8 * kDnU * 8;    // f32x4_t per staged h row (I <= 2304)
constexpr int kDnIssueLoads = 2 * kDnU;  // vector loads of one dn_issue_blk

// Copy the h rows of down item d's slot (written by the previous launch)
// into LDS: slot q of row i holds float4 f = (q % 72) * 8 + q / 72 of the
// row, the transposed order the compute reads without bank conflicts.
__device__ __forceinline__ void dn_copy_h(const DecodeArgs& a, const BlkItem& d, uint32_t s_h_lds) {
  const int nv = a.I >> 2;
  const int total = d.m * kHRow;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  for (int q0 = 0; q0 < total; q0 += kThreads) {
    const int q = q0 + (int)threadIdx.x;
    const int i = min(q / kHRow, max(d.m - 1, 0)), qq = q - (q / kHRow) * kHRow;
    const int f = min((qq % (8 * kDnU)) * 8 + qq / (8 * kDnU), nv - 1);
    if (q < total)
      lds_copy16(a.h, (uint32_t)(((size_t)(d.row0 + i) * a.I + 4 * f) * 4),
                 s_h_lds + (uint32_t)((q0 + 64 * wave) * 16));
  }
}

// One down item for each of the slot's rows, y rows stored write-through
// for the combine in this launch. `fresh`: the slot's h rows were just
// copied (before the kDnIssueLoads loads of the next item's weights), so
// wait for the copies and make them visible to every wave first.
template <int TB, bool NV>
__device__ __forceinline__ void dn_compute_blk(const DecodeArgs& a, const BlkItem& d, bool fresh,
                                               const DnW& r, const f32x4_t* s_h) {
  if (fresh) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDnIssueLoads) : "memory");
    __syncthreads();
  }
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int n = d.rb * kDnRows + wave * 8 + (lane >> 3);
  const int kc = a.I >> 5;
  const uint32_t sh = 8u * (j & 3);
  constexpr int P = 8 * kDnU;
  float acc[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) acc[i] = 0.0f;
  // each 16-byte chunk of weights converted to fp32 once, used by every row
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    const int ch = 8 * u + j;
    if (ch < kc) {
      f32x2_t fd;  // MXFP4: one scale per chunk; NVFP4: one per 16-code half
      if constexpr (NV)
        fd = nv_scale_pair(r.sc[u], 16u * (j & 1));
      else
        fd.x = fd.y = e8m0_to_f32(__builtin_amdgcn_ubfe(r.sc[u], sh, 8));
      const uint32_t ww[4] = {r.w[u].x, r.w[u].y, r.w[u].z, r.w[u].w};
      f32x2_t wf[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wf[4 * q + 0] = fp4x2_to_f32<0>(ww[q]);
        wf[4 * q + 1] = fp4x2_to_f32<1>(ww[q]);
        wf[4 * q + 2] = fp4x2_to_f32<2>(ww[q]);
        wf[4 * q + 3] = fp4x2_to_f32<3>(ww[q]);
      }
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        if (i < d.m) {
          const f32x4_t* hv = s_h + i * kHRow + ch;
          float pd[2] = {0.0f, 0.0f};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t ha = hv[2 * q * P], hb = hv[(2 * q + 1) * P];
            const int hf = NV ? q >> 1 : 0;
            pd[hf] = fmaf(wf[4 * q + 0].x, ha.x, pd[hf]);
            pd[hf] = fmaf(wf[4 * q + 0].y, ha.y, pd[hf]);
            pd[hf] = fmaf(wf[4 * q + 1].x, ha.z, pd[hf]);
            pd[hf] = fmaf(wf[4 * q + 1].y, ha.w, pd[hf]);
            pd[hf] = fmaf(wf[4 * q + 2].x, hb.x, pd[hf]);
            pd[hf] = fmaf(wf[4 * q + 2].y, hb.y, pd[hf]);
            pd[hf] = fmaf(wf[4 * q + 3].x, hb.z, pd[hf]);
            pd[hf] = fmaf(wf[4 * q + 3].y, hb.w, pd[hf]);
          }
          if constexpr (NV)
            acc[i] = fmaf(pd[1], fd.y, fmaf(pd[0], fd.x, acc[i]));
          else
            acc[i] = fmaf(pd[0], fd.x, acc[i]);
        }
      }
    }
  }
  float md = 1.0f;
  if constexpr (NV) md = nv_matrix_scale(d.e < 0 ? a.shared : a.routed, max(d.e, 0), 2);
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    if (i < d.m) {
      float v = group_sum<8>(acc[i]);
      if constexpr (NV) v *= md;
      if (j == 0 && n < a.H) cst(a.y + (size_t)(d.row0 + i) * a.H + n, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Block down on the matrix cores (blocks of at most 5 tokens). For one slot,
// y[t][n] = sum_k W[n][k] h_t[k] over the slot's m <= 5 tokens is a dense
// contraction of 64 weight rows (an item, 16 per wave) with m token rows.
// Each fp32 h value is split exactly into three bf16 parts, h = hi + mid +
// lo (each part holds the next 8 significant bits; bf16 has fp32's
// exponent range), and the 16 rows of the MFMA's A operand are the (token,
// part) pairs 3 t + p, read from LDS; the B operand is the weight rows'
// codes converted exactly to bf16 with their E8M0 scales. One
// v_mfma_f32_16x16x32_bf16 per 32 K values then serves every token and
// part, each product of bf16 parts is exact and every sum is fp32, so the
// result matches the fp32 GEMV to within fp32 rounding. The three parts of
// a token are added at the end of the item. Compared with the fp32 GEMV,
// where every 8 weight rows of a wave read the same h values from LDS, the
// LDS reads per weight row drop by about 4x at the block's average of two
// tokens per slot.
// K order: lane group g (lanes 16 g .. 16 g + 15) of a wave takes K range
// [128 S + 32 g, + 32) of super-step S, one E8M0 block: 16 bytes of codes
// of its weight row, used by MFMA steps s = 0..3 for K values 8 s .. 8 s + 7
// of that range, and A is read in the same order.
// ---------------------------------------------------------------------------
constexpr int kMfRows = 64;   // weight rows per item (16 per wave)
constexpr int kMfSup = 18;    // super-steps of 128 K (I <= 2304)
// bytes per staged row of bf16 h parts, padded so that the 16 rows a
// fragment read touches fall in distinct LDS banks
constexpr int kMfRowBytes = kMfSup * 256 + 16;
// rows, a 16 x 16 tile per wave, the choice of each bucket row (R <= 256)
constexpr int kMfLds = 16 * kMfRowBytes + 4 * 256 * 4 + 256 * 4;

// One item's weights for a lane: 23 vector loads (NVFP4: 27), so that two
// buffers stay under the 63 loads a wave can have in flight.
constexpr int kMfScl = (kMfSup * 4 + 15) / 16;  // 16-byte loads of a row's scales
template <bool NV>
struct MfW {
  uint4 c[kMfSup];  // codes of super-step S
  uint4 sc[kMfScl];  // the row's scale bytes: block b at byte b % 16 of sc[b / 16]
};
template <>
struct MfW<true> {
  uint4 c[kMfSup];
  uint32_t sc[kMfSup / 2];  // the lane group's scale bytes of super-steps 2 S', 2 S' + 1
};

// Item `it` of the routed slots: slot it / per, 64-row group it % per.
struct MfItem {
  const uint8_t* codes;
  const uint8_t* scales;
  int rg, row0, m, e;
};
template <bool NV>
__device__ __forceinline__ MfItem mf_item(const DecodeArgs& a, const LaneTable& tab, int it,
                                          int per) {
  const int sl = it / per, rg = it - sl * per;
  const int e = __builtin_amdgcn_readfirstlane(min(max(tab[1 + sl], 0), a.routed.E - 1));
  const int row0 = min(max(tab[1 + a.max_slots + sl], 0), a.R);
  const int m = min(max(tab[1 + 2 * a.max_slots + sl], 0), min(a.R - row0, 8));
  const uint32_t crow = (uint32_t)a.I >> 1, srow = (uint32_t)a.I >> (NV ? 4 : 5);
  return MfItem{a.routed.d_codes + (size_t)e * a.H * crow,
                a.routed.d_scales + (size_t)e * a.H * srow, rg, row0, m, e};
}

// NVFP4 banks (one E4M3 scale per 16 codes, 36 words a row at I = 2304)
// take another K order, so that a lane's scales of two super-steps are one
// word: lane group g's 32 K values of super-step S = 2 S' + p are block
// 8 S' + 2 g + p of 32, whose four scale bytes (p = 0, 1; MFMA steps 0-1 and
// 2-3) are word 4 S' + g of the row. The code loads of S and S + 1 then
// read one 128-byte span of each row. Needs an even number of super-steps
// (I % 256 == 0).

template <bool NV>
__device__ __forceinline__ void mf_issue(const DecodeArgs& a, const MfItem& d, MfW<NV>& r,
                                         bool live) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4;
  const int row = min(d.rg * kMfRows + wave * 16 + (lane & 15), a.H - 1);
  const uint32_t crow = (uint32_t)a.I >> 1, srow = (uint32_t)a.I >> (NV ? 4 : 5);
  live = __builtin_amdgcn_readfirstlane((int)live) != 0;
  const __amdgpu_buffer_rsrc_t rc = matrix_rsrc(uniform_ptr(d.codes), live ? a.H * crow : 0u);
  const __amdgpu_buffer_rsrc_t rs = matrix_rsrc(uniform_ptr(d.scales), live ? a.H * srow : 0u);
  const int nsup = a.I >> 7;
  if constexpr (NV) {
    const int cg = row * crow + g * 32, sg = row * srow + g * 4;
#pragma unroll
    for (int S = 0; S < kMfSup; ++S)
      r.c[S] = bload16(rc, S < nsup ? cg + (S >> 1) * 128 + (S & 1) * 16 : 0x7ffffff0);
#pragma unroll
    for (int j = 0; j < kMfSup / 2; ++j)
      r.sc[j] = bload32(rs, 2 * j < nsup ? sg + 16 * j : 0x7ffffff0);
  } else {
#pragma unroll
    for (int S = 0; S < kMfSup; ++S) {
      // super-steps past the row's K read nothing (an offset past the
      // resource returns zeros)
      r.c[S] = bload16(rc, S < nsup ? row * crow + S * 64 + g * 16 : 0x7ffffff0);
    }
    // the row's I / 32 scale bytes (the last load may run into the next
    // row, or past the resource, which returns zeros; those bytes are not
    // used)
#pragma unroll
    for (int j = 0; j < kMfScl; ++j)
      r.sc[j] = bload16(rs, 16 * j < (int)srow ? row * srow + 16 * j : 0x7ffffff0);
  }
}

// Parts of each h value a slot of m tokens carries: three bf16 (exact) up
// to 5 tokens, so that the (token, part) rows fit one 16-row tile; two (16
// significant bits, relative error at most 2^-17) for 6 to 8 tokens.
__device__ __forceinline__ int mf_parts(int m) { return m <= 5 ? 3 : 2; }

// The slot's m h rows (fp32, written by the previous launch) into LDS as
// bf16 parts: row P t + p of s_a holds part p of token t (P = mf_parts(m)).
__device__ __forceinline__ void mf_stage_h(const DecodeArgs& a, int row0, int m, char* s_a,
                                           int rs) {
  const int n8 = a.I >> 3;  // 8 values per thread and round
  const int P = mf_parts(m);
  for (int q = threadIdx.x; q < m * n8; q += kThreads) {
    const int t = q / n8, k = (q - t * n8) * 8;
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.h + (size_t)(row0 + t) * a.I + k);
    const f32x4_t v0 = src[0], v1 = src[1];
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t part[3][4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float x0 = v[i], x1 = v[i + 1];
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        // round to bf16 (nearest even); the remainder is exact in fp32
        const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
        const uint32_t r0 = (b0 + 0x7fffu + ((b0 >> 16) & 1u)) & 0xffff0000u;
        const uint32_t r1 = (b1 + 0x7fffu + ((b1 >> 16) & 1u)) & 0xffff0000u;
        part[p][i >> 1] = (r0 >> 16) | (r1 & 0xffff0000u);
        x0 -= __uint_as_float(r0);
        x1 -= __uint_as_float(r1);
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
      if (p < P)
        *reinterpret_cast<uint4*>(s_a + (P * t + p) * rs + k * 2) =
            make_uint4(part[p][0], part[p][1], part[p][2], part[p][3]);
  }
}

// One item: 16 weight rows per wave against the staged (token, part) rows,
// then y[row0 + t] for the item's rows, t < m.
// y rows go out in choice order (row t k + j: token t's j-th expert), as
// value words, so the combine workgroups of the launch read them without the
// row map and without a count: a word carrying the call's tag has landed.
template <bool NV>
__device__ __forceinline__ void mf_compute(const DecodeArgs& a, const MfItem& d,
                                           const MfW<NV>& r, const char* s_a, int rs,
                                           float* s_c, const int* s_rp) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, ar = lane & 15;
  const int nsup = a.I >> 7;
  const int P = mf_parts(d.m);
  const bool arow = ar < P * d.m;
  // A: K of super-step S for lane group g at 128 S + 32 g (NVFP4, S = 2 S' + p:
  // 256 S' + 64 g + 32 p)
  const char* arow_p = s_a + ar * rs + (NV ? g * 128 : g * 64);
  // two accumulators (steps 0, 2 and 1, 3 of each super-step), and the
  // super-step's four A fragments read together: the MFMAs do not wait on
  // one another, nor each on its own LDS read
  f32x4_t c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
#pragma unroll
  for (int S = 0; S < kMfSup; ++S) {
    if (S < nsup) {
      uint4 av[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        av[q] = arow ? *reinterpret_cast<const uint4*>(
                           arow_p + (NV ? (S >> 1) * 512 + (S & 1) * 64 : S * 256) + q * 16)
                     : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w[4] = {r.c[S].x, r.c[S].y, r.c[S].z, r.c[S].w};
      float sc = 0.0f;
      f32x2_t sn = {0.0f, 0.0f};
      if constexpr (NV) {
        sn = nv_scale_pair(r.sc[S >> 1], 16u * (S & 1));
      } else {
        const uint4 sv = r.sc[S >> 2];
        const uint32_t sw = (S & 3) == 0 ? sv.x : (S & 3) == 1 ? sv.y : (S & 3) == 2 ? sv.z : sv.w;
        sc = e8m0_to_f32(__builtin_amdgcn_ubfe(sw, 8u * g, 8));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x8_t b;
        if constexpr (NV) {
          // the scaled conversion applies only a power of two: convert, then
          // multiply by the E4M3 scale in fp32 (E2M1 x E4M3 is exact in bf16)
          const float s2 = q < 2 ? sn.x : sn.y;
          const f32x2_t f0 = fp4x2_to_f32<0>(w[q]), f1 = fp4x2_to_f32<1>(w[q]);
          const f32x2_t f2 = fp4x2_to_f32<2>(w[q]), f3 = fp4x2_to_f32<3>(w[q]);
          b = bf16x8_t{(__bf16)(f0.x * s2), (__bf16)(f0.y * s2), (__bf16)(f1.x * s2),
                       (__bf16)(f1.y * s2), (__bf16)(f2.x * s2), (__bf16)(f2.y * s2),
                       (__bf16)(f3.x * s2), (__bf16)(f3.y * s2)};
        } else {
          const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 0);
          const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 1);
          const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 2);
          const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 3);
          b = bf16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
        }
        if (q & 1)
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[q]), b, c1,
                                                        0, 0, 0);
        else
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[q]), b, c0,
                                                        0, 0, 0);
      }
    }
  }
  const f32x4_t c = c0 + c1;
  // lane holds C[(t, p) = 4 g + i][weight row ar]; add the three parts of
  // each token (hi, then mid, then lo) through this wave's 16 x 16 LDS tile
  float* cw = s_c + wave * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i) cw[(4 * g + i) * 16 + ar] = c[i];
  __builtin_amdgcn_wave_barrier();
  const int n = d.rg * kMfRows + wave * 16 + ar;
  const float md = NV ? nv_matrix_scale(a.routed, d.e, 2) : 1.0f;
  for (int t = g; t < d.m; t += 4) {
    float v = cw[(P * t) * 16 + ar] + cw[(P * t + 1) * 16 + ar];
    if (P == 3) v += cw[(P * t + 2) * 16 + ar];
    if (NV) v *= md;
    const int yr = min(max(s_rp[min(d.row0 + t, a.R - 1)], 0), a.R - 1);
    if (n < a.H) cst(a.yw + (size_t)yr * a.H + n, value_word(a, v));
  }
}

// Block combine, in the down launch after its matrix-core workgroups:
// workgroup c sums output columns [32 c, 32 c + 32) of every token in fixed
// order (shared row, then j = 0..k-1). Each wave polls its tokens' k routed
// y words (choice order, so every load is independent) until all carry the
// call's tag; dispatched after every down workgroup, it waits only for
// their last stores to land. On a wait that gave up in an earlier launch
// (or this one) its columns are NaN; workgroup 0 also writes -1 ids and NaN
// weights then, and the call's result word.
__device__ void combine_block_words(const DecodeArgs& a, int c) {
  const uint32_t code = call_wait_code(a);
  bool failed = code != 0;
  const int n = min(c * kDnRows + (int)(threadIdx.x & 31), a.H - 1);
  const bool col = c * kDnRows + (int)(threadIdx.x & 31) < a.H;
  for (int t = threadIdx.x >> 5; t < a.T; t += kThreads / 32) {  // wave-uniform trip
    const float base = a.y_shared_ext ? a.y_shared_ext[(size_t)t * a.H + n]
                       : a.has_shared ? a.y[(size_t)(a.R + t) * a.H + n] : 0.0f;
    float v = base;
    for (long it = 0; !failed; ++it) {
      bool ok = true;
      v = base;
      for (int j0 = 0; j0 < a.k; j0 += 8) {  // 8 rows' loads in flight at a time
        uint64_t yv[8];
        float wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int p = t * a.k + min(j0 + u, a.k - 1);
          yv[u] = cld(a.yw + (size_t)p * a.H + n);
          wv[u] = a.route_w[p];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j0 + u < a.k) {
            ok &= is_mine(a, yv[u]);
            v = fmaf(wv[u], __uint_as_float((uint32_t)yv[u]), v);
          }
      }
      if (__all(ok)) break;
      if (it >= kSpinLimit) {
        if ((threadIdx.x & (kWave - 1)) == 0) report_timeout(a, kWaitDown);
        failed = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (col) a.out[(size_t)t * a.H + n] = failed ? __builtin_nanf("") : v;
  }
  if (c == 0) {
    if (code)
      for (int i = threadIdx.x; i < a.R; i += kThreads) {
        if (a.ids_out) a.ids_out[i] = -1;
        if (a.w_out) a.w_out[i] = __builtin_nanf("");
      }
    if (threadIdx.x == 0) a.wstat[1] = result_word(a);
  }
}

// Block down for blocks of at most 5 tokens: routed (slot, 64-row group)
// items slot-major, workgroup b taking the contiguous stretch
// [n b / G, n (b + 1) / G) with two register buffers for the weights; the
// slot's h parts are staged when an item's slot differs from the staged one.
template <bool NV>
__global__ __launch_bounds__(kThreads, 2) void down_block_mfma_kernel(DecodeArgs a, int G) {
  __shared__ __align__(16) char lds[kMfLds];
  if ((int)blockIdx.x >= G) {  // the combine workgroups, last in the grid
    combine_block_words(a, (int)blockIdx.x - G);
    return;
  }
  constexpr int rs = kMfRowBytes;
  char* s_a = lds;
  float* s_c = reinterpret_cast<float*>(lds + 16 * rs);
  int* s_rp = reinterpret_cast<int*>(lds + 16 * rs + 4 * 256 * 4);
  for (int i = threadIdx.x; i < a.R; i += kThreads) s_rp[i] = a.row_pair[i];  // seen after restage
  LaneTable tab;
  tab.load(a.tab, 1 + 3 * a.max_slots);
  const int ns = min(max(tab[0], 0), a.max_slots);
  const int per = (a.H + kMfRows - 1) / kMfRows;
  const int n = ns * per;
  const int b = blockIdx.x;
  const int lo = (int)((long)n * b / G), hi = (int)((long)n * (b + 1) / G);
  if (lo >= hi) return;
  int staged = -1;
  auto restage = [&](int it) {
    const MfItem d = mf_item<NV>(a, tab, it, per);
    __syncthreads();  // every wave is done with the staged rows
    mf_stage_h(a, d.row0, d.m, s_a, rs);
    __syncthreads();
    staged = it / per;
  };
  MfW<NV> A, B;
  auto item = [&](int it) { return mf_item<NV>(a, tab, it, per); };
  mf_issue<NV>(a, item(lo), A, true);
  restage(lo);
  for (int i0 = lo; i0 < hi; i0 += 2) {
    const int i1 = i0 + 1, i2 = i0 + 2;
    mf_issue<NV>(a, item(i1 < hi ? i1 : i0), B, i1 < hi);
    mf_compute<NV>(a, item(i0), A, s_a, rs, s_c, s_rp);
    if (i1 < hi && i1 / per != staged) restage(i1);
    mf_issue<NV>(a, item(i2 < hi ? i2 : i0), A, i2 < hi);
    if (i1 < hi) {
      mf_compute<NV>(a, item(i1), B, s_a, rs, s_c, s_rp);
      if (i2 < hi && i2 / per != staged) restage(i2);
    }
  }
}

// Block gate/up: G persistent workgroups stage the T token rows and the
// slot table, then stream the routed items with two register buffers. The
// last n_sd workgroups of the grid each take one 32-row group of the shared
// expert's down rows (MXFP4 or FP8; its h rows came from the previous
// launch); dispatched last, they run in the tail of the routed stream.
template <int TB, bool NV>
__global__ __launch_bounds__(kThreads, 3) void gateup_block_kernel(DecodeArgs a, int G) {
  extern __shared__ __align__(16) char lds[];
  if ((int)blockIdx.x >= G) {
    if (a.shared_fp8) {
      fp8_shared_down_blk<TB>(a, (int)blockIdx.x - G, reinterpret_cast<f32x4_t*>(lds));
      return;
    }
    const int* none = nullptr;
    const BlkItem d =
        blk_item<TB, NV>(a, none, a.dn_items, (int)blockIdx.x - G, a.dn_items, false);
    DnW A;
    dn_issue_blk<NV>(a, d, A, true);
    dn_copy_h(a, d, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the weights and the copies
    __syncthreads();
    dn_compute_blk<TB, NV>(a, d, false, A, reinterpret_cast<const f32x4_t*>(lds));
    return;
  }
  uint4* s_x = reinterpret_cast<uint4*>(lds);
  stage_block_rows(a, s_x);
  if constexpr (TB <= 5) {
    // the slot table and row map in LDS too: their reads sit on the path of
    // every item's weight addresses
    const int T = min(a.T, TB);
    int* s_tab = reinterpret_cast<int*>(lds + (size_t)T * kXRow * 16);
    int* s_rt = s_tab + 1 + 3 * a.max_slots;
    for (int i = threadIdx.x; i < 1 + 3 * a.max_slots; i += kThreads) s_tab[i] = a.tab[i];
    for (int i = threadIdx.x; i < a.R; i += kThreads) s_rt[i] = a.row_token[i];
    __syncthreads();
    const int ns = min(max(s_tab[0], 0), a.max_slots);
    gateup_block_items<TB, NV>(a, s_tab, s_rt, s_x, 0, ns * a.gu_items, blockIdx.x, G);
  } else {
    // LDS holds only the T token rows (at most 80 KB: two workgroups a CU);
    // the slot table and row map ride in registers across each wave's lanes
    LaneTable tab, rt;
    tab.load(a.tab, 1 + 3 * a.max_slots);
    rt.load(a.row_token, a.R);
    __syncthreads();
    const int ns = min(max(tab[0], 0), a.max_slots);
    gateup_block_items<TB, NV>(a, tab, rt, s_x, 0, ns * a.gu_items, blockIdx.x, G);
  }
}


// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(kThreads) void route_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int b = blockIdx.x;
  if (b < a.nb_router) {
    router_rows(a, b);
  } else if (b == a.nb_router) {
    routing<false>(a, lds);
  } else {
    gateup_item<MT>(a, shared_slot(a), b - a.nb_router - 1, reinterpret_cast<uint4*>(lds), nullptr);
  }
}

// Items are slot-minor (item = rb * max_slots + s), so workgroups of slots
// that turn out empty are spread over the grid instead of trailing it.
template <int MT>
__global__ __launch_bounds__(kThreads) void gateup_kernel(DecodeArgs a, int routed_items,
                                                          const int32_t* rtok) {
  extern __shared__ __align__(16) char lds[];
  const int b = blockIdx.x;
  if (b < routed_items) {
    const int s = b % a.max_slots, rb = b / a.max_slots;
    if (s >= load_nslots(a)) return;
    gateup_item<MT>(a, load_slot(a, s), rb, reinterpret_cast<uint4*>(lds), rtok);
  } else {
    down_item<MT>(a, shared_slot(a), b - routed_items, reinterpret_cast<f32x4_t*>(lds), a.y, false);
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void down_kernel(DecodeArgs a, int combine) {
  extern __shared__ __align__(16) char lds[];
  __shared__ int s_last;
  const int b = blockIdx.x;
  const int s = b % a.max_slots, c = b / a.max_slots;
  // the last launch of the call: every wait ran in the route launch (the
  // FFN mode has none)
  const uint32_t code = combine ? call_wait_code(a) : 0u;
  finish_call(a, code, b, gridDim.x);
  const int ns = load_nslots(a);
  if (s >= ns) return;
  down_item<MT>(a, load_slot(a, s), c, reinterpret_cast<f32x4_t*>(lds), a.y, combine != 0);
  if (!combine) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.cnt_dn + c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             ns - 1;
  __syncthreads();
  if (s_last) combine_column(a, c, code != 0);
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {
constexpr uint64_t kTagMask = (1ull << 48) - 1;

// 48-bit tags unique per call: a counter on a base drawn from the process's
// start time and id, so words left in a reused workspace by earlier calls
// (of this or another process) never carry the tag of a new call.
uint64_t next_tag() {
  static std::atomic<uint64_t> counter{0};
  static const uint64_t base = [] {
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return (t << 16) ^ ((uint64_t)getpid() << 28) ^ (t >> 20);
  }();
  const uint64_t v = (base + (++counter)) & kTagMask;
  return v == 0 ? 1 : v;
}

// Test hook (moe_set_wait_test): the routing's first wait of each call
// expects a tag no word carries and gives up after a few polls; every other
// wait keeps its usual limit and completes.
thread_local int g_force_timeout = 0;
constexpr long kForcedSpinLimit = 256;

struct DecodeLayout {
  int max_slots, rows, gu_items, dn_items, nb_router;
  size_t off_wstat, off_flags, off_cnt, off_tab, off_rt, off_inv, off_rp, off_logits, off_w, off_h,
      off_y, off_tagged, off_hw, off_yw, bytes;
};

size_t al(size_t v) { return (v + 255) & ~(size_t)255; }

DecodeLayout layout(int T, int H, int I, int E, int k, int R, bool ffn, bool shared) {
  DecodeLayout L{};
  L.max_slots = E < R ? E : R;
  L.rows = R + (shared && !ffn ? T : 0);
  L.gu_items = (I + kGuRows - 1) / kGuRows;
  L.dn_items = (H + kDnRows - 1) / kDnRows;
  L.nb_router = ffn ? 0 : (E + 3) / 4;
  size_t o = 0;
  L.off_wstat = o;  // first, at a fixed place: moe_workspace_status reads it
  o += al(2 * sizeof(uint64_t));
  L.off_flags = o;
  o += al(sizeof(uint64_t) * (L.nb_router + 1));
  L.off_cnt = o;
  o += al(sizeof(int32_t) * (size_t)L.dn_items);
  L.off_tab = o;
  o += al(sizeof(int32_t) * (1 + 3 * (size_t)L.max_slots));
  L.off_rt = o;
  o += al(sizeof(int32_t) * (size_t)L.rows);
  L.off_inv = o;
  o += al(sizeof(int32_t) * (size_t)R);
  L.off_rp = o;
  o += al(sizeof(int32_t) * (size_t)R);
  L.off_tagged = o;
  // one token: [2][E] tagged logit halves, kReplicas routing copies, the
  // shared items' flags; more tokens: [T][2][E] (the block path's)
  o += al(sizeof(uint64_t) *
          (ffn ? 0 : T == 1 ? 2 * (size_t)E + kReplicas * kReplicaWords + L.gu_items
                            : 2 * (size_t)T * E));
  L.off_logits = o;
  o += al(sizeof(float) * (size_t)T * E);
  L.off_w = o;
  o += al(sizeof(float) * (size_t)R);
  L.off_h = o;
  o += al(sizeof(float) * (size_t)L.rows * I);
  L.off_y = o;
  o += al(ffn ? 0 : sizeof(float) * (size_t)L.rows * H);
  // one token: h and y as value words; a block: y as value words
  const bool one = T == 1 && !ffn;
  const bool blk = T >= 2 && T <= kBlockT && !ffn;
  L.off_hw = o;
  o += al(one ? sizeof(uint64_t) * (size_t)L.rows * I : 0);
  L.off_yw = o;
  o += al(one || blk ? sizeof(uint64_t) * (size_t)L.rows * H : 0);
  L.bytes = o;
  return L;
}
}  // namespace

size_t decode_ws_bytes(int T, int H, int I, int E, int k, int R, bool ffn, bool shared) {
  return layout(T, H, I, E, k, R, ffn, shared).bytes;
}

void set_force_wait_timeout(int on) { g_force_timeout = on; }

int read_decode_status(const void* ws) {
  uint64_t v[2] = {0, 0};
  if (hipMemcpy(v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  if ((v[1] >> 48) != kResultMagic) return 0;  // no few-token call recorded
  const uint64_t tag = v[1] & 0xffffffffffffull;
  return (v[0] >> kTagShift) == tag ? (int)(v[0] & 0xffffu) : 0;
}

template <int MT>
void launch_chain(const DecodeArgs& a, const DecodeLayout& L, bool ffn, bool shared, int routed_gu,
                  int shared_dn, const int32_t* rtok, hipStream_t s) {
  if (!ffn) {
    const int grid = L.nb_router + 1 + (shared ? L.gu_items : 0);
    launch("route_kernel", route_kernel<MT>, dim3(grid), dim3(kThreads), kLdsBytes, s, a);
  }
  launch("gateup_kernel", gateup_kernel<MT>, dim3(routed_gu + shared_dn), dim3(kThreads), kLdsBytes, s,
                     a, routed_gu, rtok);
  launch("down_kernel", down_kernel<MT>, dim3(L.max_slots * L.dn_items), dim3(kThreads), kLdsBytes, s,
                     a, ffn ? 0 : 1);
}

// Compute units of the current device (cached per device; 256 if the query
// fails).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Persistent grids no larger than the workgroups the CUs hold at once:
// three a CU by registers, fewer where the LDS a workgroup needs allows less.
int resident_grid(uint32_t lds_bytes) {
  const int by_lds = lds_bytes ? (int)(163840u / lds_bytes) : 3;
  return cu_count() * (by_lds < 3 ? (by_lds < 1 ? 1 : by_lds) : 3);
}

template <int TB, bool NV>
void launch_block(const DecodeArgs& a, const DecodeLayout& L, const DecodeLaunch& d, bool shared,
                  hipStream_t s) {
  const uint32_t lds_x = (uint32_t)(d.T * kXRow * 16);
  const uint32_t lds_rt = lds_x > (uint32_t)kLdsBytes ? lds_x : (uint32_t)kLdsBytes;
  const int n_sw = shared ? L.gu_items : 0;  // one item each (at most 288 at I <= 2304)
  launch("route_block_kernel", route_block_kernel<TB, NV>, dim3(L.nb_router + 1 + n_sw),
         dim3(kThreads), lds_rt, s, a, n_sw);
  const uint32_t lds_gu =
      lds_x + (TB <= 5 ? (uint32_t)(sizeof(int) * (1 + 3 * L.max_slots + d.R)) : 0u);
  const int ng = L.max_slots * L.gu_items, rg = resident_grid(lds_gu);
  const int gg = ng < rg ? ng : rg;
  const int n_sd = shared ? L.dn_items : 0;
  launch("gateup_block_kernel", gateup_block_kernel<TB, NV>, dim3(gg + n_sd), dim3(kThreads), lds_gu,
         s, a, gg);
  {
    // on the matrix cores: 16 staged rows of bf16 h parts and a 16 x 16
    // fp32 tile per wave (76 KB of LDS); two workgroups a CU
    const int nd = L.max_slots * ((d.H + kMfRows - 1) / kMfRows), rd = 2 * cu_count();
    const int gd = nd < rd ? nd : rd;
    launch("down_block_mfma_kernel", down_block_mfma_kernel<NV>, dim3(gd + L.dn_items),
           dim3(kThreads), 0, s, a, gd);
  }
}

// The one-token fused launches take this call.
static bool stream_path(const DecodeLaunch& d, const DecodeLayout& L) {
  const bool ffn = d.ffn_mode != 0;
  return d.T == 1 && !ffn && (d.H >> 5) <= kGuLanes * kGuU && d.H % 128 == 0 &&
         d.I % 128 == 0 && (d.I >> 5) <= 8 * kDnU && d.I <= 3 * 4 * kThreads &&
         d.H * 2 + 4 * (1 + 3 * L.max_slots) <= kLdsBytes &&
         1 + 3 * L.max_slots + 2 * d.k <= 1024 && d.k <= kWave && d.E <= 16 * kWave;
}

// A block of 2..8 tokens takes this call.
static bool block_path(const DecodeLaunch& d, const DecodeLayout& L) {
  return d.T >= 2 && d.T <= kBlockT && d.ffn_mode == 0 && (d.H >> 5) <= kGuLanes * kGuU &&
         d.H % 128 == 0 && d.I % 128 == 0 && (d.I >> 5) <= 8 * kDnU && d.E <= 16 * kWave &&
         1 + 3 * L.max_slots <= LaneTable::kMax && d.R <= LaneTable::kMax &&
         d.T * (d.H >> 3) <= kBlockXLoads * kThreads &&
         (d.routed.codec != kCodecNvfp4 || d.I % 256 == 0);  // NVFP4 down: word-aligned scales
}

bool decode_fuses_nvfp4(const DecodeLaunch& d) {
  if (d.ffn_mode != 0) return false;
  const DecodeLayout L = layout(d.T, d.H, d.I, d.E, d.k, d.R, false, d.has_shared);
  return d.T == 1 ? stream_path(d, L) : block_path(d, L);
}

bool decode_fuses_fp8_shared(const DecodeLaunch& d) {
  if (d.ffn_mode != 0) return false;
  const DecodeLayout L = layout(d.T, d.H, d.I, d.E, d.k, d.R, false, true);
  // the FP8 items hold K = H in 32 x kF8GuU chunks and K = I in 8 x kF8DnU
  if ((d.H >> 4) > 32 * kF8GuU || (d.I >> 4) > 8 * kF8DnU) return false;
  return d.T == 1 ? stream_path(d, L) : block_path(d, L);
}

void launch_decode(const DecodeLaunch& d, void* ws, hipStream_t s) {
  const bool ffn = d.ffn_mode != 0;
  const bool shared = d.has_shared && !ffn;
  const DecodeLayout L = layout(d.T, d.H, d.I, d.E, d.k, d.R, ffn, shared);
  char* w = static_cast<char*>(ws);
  DecodeArgs a{};
  a.x = d.x;
  a.wr = d.wr;
  a.bias = d.bias;
  a.routed = d.routed;
  a.shared = d.shared;
  a.has_shared = shared;
  a.y_shared_ext = ffn ? nullptr : d.y_shared_ext;
  a.shared_fp8 = shared && d.shared_fp8;
  a.sh8_gu_w = d.sh8_gu_w;
  a.sh8_gu_s = d.sh8_gu_s;
  a.sh8_d_w = d.sh8_d_w;
  a.sh8_d_s = d.sh8_d_s;
  a.T = d.T;
  a.H = d.H;
  a.I = d.I;
  a.E = d.E;
  a.k = d.k;
  a.R = d.R;
  a.offsets_in = d.offsets;
  a.row_token_in = d.row_token;
  a.out = d.out;
  a.ids_out = d.ids_out;
  a.w_out = d.w_out;
  a.flags = reinterpret_cast<uint64_t*>(w + L.off_flags);
  a.tagged = reinterpret_cast<uint64_t*>(w + L.off_tagged);
  a.cnt_dn = reinterpret_cast<int32_t*>(w + L.off_cnt);
  a.hw = reinterpret_cast<uint64_t*>(w + L.off_hw);
  a.yw = reinterpret_cast<uint64_t*>(w + L.off_yw);
  a.wstat = reinterpret_cast<uint64_t*>(w + L.off_wstat);
  a.tab = reinterpret_cast<int32_t*>(w + L.off_tab);
  a.row_token = reinterpret_cast<int32_t*>(w + L.off_rt);
  a.inv_row = reinterpret_cast<int32_t*>(w + L.off_inv);
  a.row_pair = reinterpret_cast<int32_t*>(w + L.off_rp);
  a.logits = reinterpret_cast<float*>(w + L.off_logits);
  a.route_w = reinterpret_cast<float*>(w + L.off_w);
  a.h = reinterpret_cast<float*>(w + L.off_h);
  a.y = ffn ? d.y_rows : reinterpret_cast<float*>(w + L.off_y);
  a.tag = next_tag();
  a.wait_tag = g_force_timeout ? (a.tag ^ 1) : a.tag;
  a.wait_limit = g_force_timeout ? kForcedSpinLimit : kSpinLimit;
  a.max_slots = L.max_slots;
  a.rows = L.rows;
  a.nb_router = L.nb_router;
  a.gu_items = L.gu_items;
  a.dn_items = L.dn_items;

  const int routed_gu = L.max_slots * L.gu_items;
  const int shared_dn = shared ? L.dn_items : 0;
  if (ffn) {
    launch("ffn_table_kernel", ffn_table_kernel, dim3(1), dim3(kThreads), 0, s, a);
  }
  // One token (or one row per expert): every slot holds a single row, and a
  // kernel built for one staged row needs far fewer registers.
  const bool one = d.T == 1 || (ffn && d.R <= 1);
  const bool stream = stream_path(d, L);
  if (stream) {
    const int n_sh = shared ? L.gu_items : 0;
    int n_sd = shared ? L.dn_items : 0;
    const int per = max(2, (routed_gu + kGuStreamMax - 1) / kGuStreamMax);
    const int gg = (routed_gu + per - 1) / per;
    const bool nv = d.routed.codec == kCodecNvfp4;
    // down workgroups: kDnPerWg 32-row groups each (FP8 shared expert: one),
    // one each for the last kDnSingleSlots slots
    const int per_slot = (L.dn_items + kDnPerWg - 1) / kDnPerWg;
    const int ns_pair = max(L.max_slots - kDnSingleSlots, 0);
    const int nd = ns_pair * per_slot + (L.max_slots - ns_pair) * L.dn_items;
    if (shared && !d.shared_fp8) n_sd = per_slot;
    launch("gateup_fused_kernel", nv ? gateup_fused_kernel<true> : gateup_fused_kernel<false>,
           dim3(L.nb_router + 1 + n_sh + gg + n_sd + nd), dim3(kThreads), kLdsBytes, s, a, n_sh,
           n_sd, gg, per, kDnPerWg, ns_pair);
    return;
  }
  // A block of 2..8 tokens: router + routing, then the streaming gate/up
  // and down launches over the union of the block's experts.
  if (block_path(d, L)) {
    const bool nv = d.routed.codec == kCodecNvfp4;
    if (d.T <= 5)
      (nv ? launch_block<5, true> : launch_block<5, false>)(a, L, d, shared, s);
    else
      (nv ? launch_block<8, true> : launch_block<8, false>)(a, L, d, shared, s);
    return;
  }
  if (one)
    launch_chain<1>(a, L, ffn, shared, routed_gu, shared_dn, ffn ? d.row_token : a.row_token, s);
  else
    launch_chain<kMT>(a, L, ffn, shared, routed_gu, shared_dn, ffn ? d.row_token : a.row_token, s);
}

}  // namespace moe
