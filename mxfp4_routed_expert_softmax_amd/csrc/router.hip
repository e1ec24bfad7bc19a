// Router: logits = x W_r^T (+ bias) and the softmax top-k selection.
//
// The gate chooses k of E experts per token (ai.rs article on
// DeepSeek-V4.1-Flash, "How 502 GB runs on a 32 GB card") and acts as a
// switch whose choice amplifies rounding (same article, "What remains is the
// reference rounding itself"), so the selection here is exact on the fp32
// logits with a fixed tie rule: larger logit first, equal logits -> lower id.
#include "moe_device.h"
#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {

// ---------------------------------------------------------------------------
// Small T: one wave per expert row, 16-byte loads of W_r, fp32 dot products.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_gemv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int H, int E, float* __restrict__ logits) {
  const int lane = lane_id();
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int nv = H >> 3;  // 16-byte vectors per row
  const uint4* wrow = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
  const float b = bias ? bias[e] : 0.0f;
  for (int t0 = 0; t0 < T; t0 += 4) {
    const int nt = min(4, T - t0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 5
    for (int c = lane; c < nv; c += kWave) {
      const uint4 w = wrow[c];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < nt) {
          const uint4 xv = reinterpret_cast<const uint4*>(x + (size_t)(t0 + t) * H)[c];
          acc[t] = dot8_bf16(w, xv, acc[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && t < nt) logits[(size_t)(t0 + t) * E + e] = s + b;
    }
  }
}

// ---------------------------------------------------------------------------
// Large T: bf16 MFMA GEMM, C[T][E] = X[T][H] W[E][H]^T. A workgroup of four
// waves owns a 128 x 128 tile; each wave a 64 x 64 sub-tile made of 4 x 4
// v_mfma_f32_16x16x32_bf16 blocks. Both operands are K-contiguous, so every
// lane loads 8 consecutive bf16 (16 bytes) of one row per operand and K step.
// A and B use the same (lane group -> K offset) assignment, which is all a
// dot product needs; the output layout is lane l, element v ->
// (row 4*(l/16) + v, column l%16) of each 16 x 16 block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int H, int E, float* __restrict__ logits) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 128 + (wave >> 1) * 64;
  const int n0 = blockIdx.y * 128 + (wave & 1) * 64;
  const int r16 = lane & 15, kg = (lane >> 4) * 8;

  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = min(m0 + 16 * i + r16, T - 1);
    const int n = min(n0 + 16 * i + r16, E - 1);
    arow[i] = x + (size_t)m * H + kg;
    brow[i] = wr + (size_t)n * H + kg;
  }
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < H; k0 += 32) {
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const bf16x8_t*>(arow[i] + k0);
      b[i] = *reinterpret_cast<const bf16x8_t*>(brow[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + r16;
    if (n >= E) continue;
    const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * i + 4 * (lane >> 4) + v;
        if (m < T) logits[(size_t)m * E + n] = acc[i][j][v] + bn;
      }
  }
}

// ---------------------------------------------------------------------------
// Router GEMM staged through LDS (H a multiple of 64): the same 128 x 128
// tile and 64 x 64 wave blocks, but each K step of 64 is copied into LDS by
// direct global -> LDS loads in which 8 lanes cover a row's 128 contiguous
// bytes (whole cache lines), double buffered, so the fragment reads hit LDS
// instead of scattering 64-byte pieces of 16 rows over the cache. Piece p of
// row r sits at slot p ^ (r % 8). ST stages: with 2, two workgroups share a
// CU; with 4 (one a CU), the copies run three steps ahead, for grids of at
// most one tile per CU (a 2k-token call has 48 tiles), whose workgroups
// cannot hide a step's load latency behind each other. Measured: 2k tokens
// 66 against 85 us; at 16k tokens (384 tiles) four stages took 142 against
// 103 us.
// ---------------------------------------------------------------------------
constexpr int kRtBK = 64;
constexpr int kRtStage = 2 * 128 * kRtBK * 2;  // A and B tiles, bf16: 32 KB

// m0 is named as clobbered: each copy rewrites it, so the compiler must keep
// no value of its own there (clang warns that m0 is a reserved register; the
// warning is silenced for this function only).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void rt_lds_load16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
               :
               : "v"(voff), "s"(lds), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// blockIdx.z: the range of H (steps K steps of 64 from z * steps) whose
// partial sums go to logits + z T E; the bias goes into the first.
template <int ST>
__global__ __launch_bounds__(256) void router_mfma_lds_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int H, int E, float* __restrict__ logits,
    int steps) {
  __shared__ __align__(16) char lds[ST * kRtStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, c = lane & 15, g = lane >> 4;
  const int mt = blockIdx.x * 128, nt = blockIdx.y * 128;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  // thread tid copies slots (row 32 u + tid / 8, slot tid % 8) of A and of B
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 32 * u + (tid >> 3);
    const int piece = (tid & 7) ^ (r & 7);
    const uint32_t kz = (uint32_t)(blockIdx.z * steps * kRtBK);
    a_off[u] = ((uint32_t)min(mt + r, T - 1) * (uint32_t)H + kz + (uint32_t)(piece * 8)) * 2u;
    b_off[u] = ((uint32_t)min(nt + r, E - 1) * (uint32_t)H + kz + (uint32_t)(piece * 8)) * 2u;
  }
  auto issue = [&](int st, int k0) {
    const uint32_t base = lds_base + (uint32_t)(st * kRtStage);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      rt_lds_load16(x, a_off[u] + 2u * k0, base + (uint32_t)((u * 256 + 64 * wave) * 16));
      rt_lds_load16(wr, b_off[u] + 2u * k0, base + 16384u + (uint32_t)((u * 256 + 64 * wave) * 16));
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Stage ks lands while earlier steps compute: at the top of step ks the
  // copies of up to ST - 2 later stages (8 per thread each) may still be in
  // flight (loads complete in order), then one barrier makes stage ks
  // visible and frees the buffer of step ks - 1 for ks + ST - 1.
  static_assert(ST >= 2 && ST <= 4, "2..4 stages");
  for (int p = 0; p < ST - 1 && p < steps; ++p) issue(p, p * kRtBK);
  for (int ks = 0; ks < steps; ++ks) {
    const int ahead = min(steps - 1 - ks, ST - 2);
    if (ahead >= 2)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (ahead == 1)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ks + ST - 1 < steps) issue((ks + ST - 1) % ST, (ks + ST - 1) * kRtBK);
    const uint4* sa = reinterpret_cast<const uint4*>(lds + (ks % ST) * kRtStage);
    const uint4* sb = sa + 1024;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = 64 * wm + 16 * i + c, rb = 64 * wn + 16 * i + c;
        a[i] = __builtin_bit_cast(bf16x8_t, sa[ra * 8 + ((4 * sub + g) ^ (ra & 7))]);
        b[i] = __builtin_bit_cast(bf16x8_t, sb[rb * 8 + ((4 * sub + g) ^ (rb & 7))]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = nt + 64 * wn + 16 * j + c;
    if (n >= E) continue;
    const float bn = bias && blockIdx.z == 0 ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = mt + 64 * wm + 16 * i + 4 * g + v;
        if (m < T) logits[(size_t)blockIdx.z * T * E + (size_t)m * E + n] = acc[i][j][v] + bn;
      }
  }
}

// Grids of at most 64 tiles (2k tokens at E = 384: 48) split H in four, so
// four times as many workgroups each take a quarter of the K steps.
int router_split(int T, int H, int E) {
  const long tiles = (long)((T + 127) / 128) * ((E + 127) / 128);
  const bool lds_path = T > kRouterGemvMaxT && H % kRtBK == 0 &&
                        (size_t)T * H * 2 < (1ull << 32) && (size_t)E * H * 2 < (1ull << 32);
  return lds_path && (H / kRtBK) % 4 == 0 && tiles <= 64 ? 4 : 1;
}

// split: 1, or router_split(T, H, E) (which takes this LDS path)
void launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias,
                          int T, int H, int E, float* logits, hipStream_t s, int split) {
  if (T > kRouterGemvMaxT && H % kRtBK == 0 && (size_t)T * H * 2 < (1ull << 32) &&
      (size_t)E * H * 2 < (1ull << 32)) {
    const dim3 grid((T + 127) / 128, (E + 127) / 128, split);
    launch("router_mfma_lds_kernel",
           grid.x * grid.y * grid.z <= 256 ? router_mfma_lds_kernel<4> : router_mfma_lds_kernel<2>,
           grid, dim3(256), 0, s, x, wr, bias, T, H, E, logits, H / kRtBK / split);
    return;
  }
  if (T <= kRouterGemvMaxT) {
    launch("router_gemv_kernel", router_gemv_kernel, dim3((E + 3) / 4), dim3(256), 0, s,
                       x, wr, bias, T, H, E, logits);
  } else {
    launch("router_mfma_kernel", router_mfma_kernel, dim3((T + 127) / 128, (E + 127) / 128),
                       dim3(256), 0, s, x, wr, bias, T, H, E, logits);
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token, lane l holding the logits of experts l, l + 64,
// ... (NK per lane: 6 where E <= 384, else 16 for E <= 1024), summed over
// the router's partial arrays in order. The selection is the wave-wide one
// of the few-token routing (topk_wave.h): k rounds of a lane-local maximum
// and a wave maximum over keys ordered by (larger logit, then lower id);
// NaN logits rank as -inf. Weights are exp(l_j - l_1) normalised over the
// chosen k (the full-softmax normaliser cancels).
// ---------------------------------------------------------------------------
template <int NK>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w, int split) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* L = logits + (size_t)t * E;
  float lv[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + kWave * i;
    float val = 0.0f;
    if (e < E) {
      val = L[e];
      for (int z = 1; z < split; ++z) val += L[(size_t)z * T * E + e];  // partials in order
    }
    lv[i] = val;
  }
  topk_row_f64<NK>(lv, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

void launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                 hipStream_t s, int split) {
  launch("topk_kernel", E <= 6 * kWave ? topk_kernel<6> : topk_kernel<16>, dim3((T + 3) / 4),
         dim3(256), 0, s, logits, T, E, k, ids, w, split);
}

}  // namespace moe
