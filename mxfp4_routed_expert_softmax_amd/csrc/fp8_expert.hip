// One FP8 expert (E4M3 elements, one E8M0 scale per 32 x 32 block) over a
// few tokens: the checkpoint's dense format, used here for the shared
// expert (FreeToken issue #444, "Is the quantization already supported": fp8
// dense weights with 32 x 32 blocks and ue8m0 scales; the shared expert takes the
// same input as the routed ones: ai.rs article on DeepSeek-V4.1-Flash, "What
// remains is the reference rounding itself").
//
// HBM-bound GEMVs: every weight byte is read once per call, for all T
// tokens. The weights are twice the bytes of an MXFP4 expert, so the work
// is spread wider: gate/up gives one wave to each output column n (gate row
// n and up row n, 64 lanes x 16-byte chunks along K), down gives 32 lanes
// to each output row. A 16-byte chunk is 16 E4M3 elements inside one 32 x 32
// scale block; the gfx950 scaled conversion turns them into bf16 (gate/up,
// against bf16 x) or fp32 (down, against fp32 h) with the block's power of
// two applied exactly (E4M3 x 2^s is representable in both). Activations
// are read through the cache (all waves read the same few rows). h is fp32.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kF8Threads = 256;
constexpr int kF8GuU = 5;   // gate/up: chunks per lane per batch (K = 5120 in one)
constexpr int kF8DnLanes = 32;  // down: lanes per output row
constexpr int kF8DnU = 5;       // down: chunks per lane per batch (K = 2304 in one)

template <int SEL>
__device__ __forceinline__ bf16x2_t fp8x2_bf16(uint32_t w, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, SEL != 0);
}
template <int SEL>
__device__ __forceinline__ f32x2_t fp8x2_f32(uint32_t w, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, sc, SEL != 0);
}

// 16 E4M3 elements (scaled) dotted with 16 bf16 of x (two 16-byte pieces).
__device__ __forceinline__ float dot16_fp8_bf16(uint4 w, float sc, uint4 x0, uint4 x1, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<0>(w.x, sc), as_bf16x2(x0.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<1>(w.x, sc), as_bf16x2(x0.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<0>(w.y, sc), as_bf16x2(x0.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<1>(w.y, sc), as_bf16x2(x0.w), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<0>(w.z, sc), as_bf16x2(x1.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<1>(w.z, sc), as_bf16x2(x1.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<0>(w.w, sc), as_bf16x2(x1.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_bf16<1>(w.w, sc), as_bf16x2(x1.w), acc, false);
  return acc;
}

// gate/up: h[t][n] = silu(W_g[n] . x_t) * (W_u[n] . x_t), one wave per n;
// instantiated for at most MT tokens (at one token the instantiation for
// 16 measured 8.2 us against 7.0 us at the real shape).
template <int MT>
__global__ __launch_bounds__(kF8Threads) void fp8_gateup_gemv_kernel(Fp8Ffn p) {
  const int lane = lane_id();
  const int n = blockIdx.x * (kF8Threads / kWave) + (threadIdx.x >> 6);
  if (n >= p.I) return;  // uniform per wave
  const int H = p.H, nch = H >> 4, sb = H >> 5;
  const uint8_t* gw = p.gu_w + (size_t)n * H;
  const uint8_t* uw = p.gu_w + ((size_t)p.I + n) * H;
  const uint8_t* gs = p.gu_s + (size_t)(n >> 5) * sb;
  const uint8_t* us = p.gu_s + (size_t)((p.I + n) >> 5) * sb;
  float ag[MT], au[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) ag[t] = au[t] = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += kWave * kF8GuU) {
    uint4 wg[kF8GuU], wu[kF8GuU];
    uint32_t sg[kF8GuU], su[kF8GuU];
#pragma unroll
    for (int u = 0; u < kF8GuU; ++u) {
      const int c = min(c0 + kWave * u + lane, nch - 1);
      wg[u] = *reinterpret_cast<const uint4*>(gw + (size_t)c * 16);
      wu[u] = *reinterpret_cast<const uint4*>(uw + (size_t)c * 16);
      sg[u] = gs[c >> 1];
      su[u] = us[c >> 1];
    }
#pragma unroll
    for (int u = 0; u < kF8GuU; ++u) {
      const int c = c0 + kWave * u + lane;
      if (c < nch) {
        const float fg = e8m0_to_f32(sg[u]), fu = e8m0_to_f32(su[u]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < p.T) {
            const uint4* xv = reinterpret_cast<const uint4*>(p.x + (size_t)t * H) + 2 * c;
            const uint4 x0 = xv[0], x1 = xv[1];
            ag[t] = dot16_fp8_bf16(wg[u], fg, x0, x1, ag[t]);
            au[t] = dot16_fp8_bf16(wu[u], fu, x0, x1, au[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t < p.T) {
      const float g = wave_sum(ag[t]), u = wave_sum(au[t]);
      if (lane == 0) p.h[(size_t)t * p.I + n] = silu_mul(g, u);
    }
  }
}

// down: y[t][n] = W_d[n] . h_t, kF8DnLanes lanes per output row n (each
// load instruction reads kF8DnLanes x 16 contiguous bytes of a row).
template <int MT>
__global__ __launch_bounds__(kF8Threads) void fp8_down_gemv_kernel(Fp8Ffn p) {
  const int lane = lane_id(), q = lane & (kF8DnLanes - 1);
  const int n = blockIdx.x * (kF8Threads / kF8DnLanes) + (threadIdx.x / kF8DnLanes);
  const bool row_ok = n < p.H;
  const int nr = row_ok ? n : p.H - 1;
  const int I = p.I, nch = I >> 4, sb = I >> 5;
  const uint8_t* dw = p.d_w + (size_t)nr * I;
  const uint8_t* ds = p.d_s + (size_t)(nr >> 5) * sb;
  float acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += kF8DnLanes * kF8DnU) {
    uint4 wd[kF8DnU];
    uint32_t sd[kF8DnU];
#pragma unroll
    for (int u = 0; u < kF8DnU; ++u) {
      const int c = min(c0 + kF8DnLanes * u + q, nch - 1);
      wd[u] = *reinterpret_cast<const uint4*>(dw + (size_t)c * 16);
      sd[u] = ds[c >> 1];
    }
#pragma unroll
    for (int u = 0; u < kF8DnU; ++u) {
      const int c = c0 + kF8DnLanes * u + q;
      if (c < nch) {
        const float f = e8m0_to_f32(sd[u]);
        f32x2_t w[8];
        w[0] = fp8x2_f32<0>(wd[u].x, f); w[1] = fp8x2_f32<1>(wd[u].x, f);
        w[2] = fp8x2_f32<0>(wd[u].y, f); w[3] = fp8x2_f32<1>(wd[u].y, f);
        w[4] = fp8x2_f32<0>(wd[u].z, f); w[5] = fp8x2_f32<1>(wd[u].z, f);
        w[6] = fp8x2_f32<0>(wd[u].w, f); w[7] = fp8x2_f32<1>(wd[u].w, f);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < p.T) {
            const f32x4_t* hv = reinterpret_cast<const f32x4_t*>(p.h + (size_t)t * I) + 4 * c;
            float a = acc[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4_t h4 = hv[i];
              a = fmaf(w[2 * i].x, h4.x, a);
              a = fmaf(w[2 * i].y, h4.y, a);
              a = fmaf(w[2 * i + 1].x, h4.z, a);
              a = fmaf(w[2 * i + 1].y, h4.w, a);
            }
            acc[t] = a;
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t < p.T) {
      const float v = group_sum<kF8DnLanes>(acc[t]);
      if (row_ok && q == 0) p.y[(size_t)t * p.H + n] = v;
    }
  }
}

}  // namespace

size_t fp8_gemv_ws_bytes(int T, int I) { return ((size_t)T * I * sizeof(float) + 255) & ~(size_t)255; }

template <int MT>
void launch_fp8_gemv_mt(const Fp8Ffn& p, hipStream_t s) {
  const int wpb = kF8Threads / kWave;
  launch("fp8_gateup_gemv_kernel", fp8_gateup_gemv_kernel<MT>, dim3((p.I + wpb - 1) / wpb),
         dim3(kF8Threads), 0, s, p);
  const int rpb = kF8Threads / kF8DnLanes;
  launch("fp8_down_gemv_kernel", fp8_down_gemv_kernel<MT>, dim3((p.H + rpb - 1) / rpb),
         dim3(kF8Threads), 0, s, p);
}

void launch_fp8_ffn_gemv(const Fp8Ffn& p, hipStream_t s) {
  if (p.T <= 1)
    launch_fp8_gemv_mt<1>(p, s);
  else if (p.T <= 4)
    launch_fp8_gemv_mt<4>(p, s);
  else if (p.T <= 8)
    launch_fp8_gemv_mt<8>(p, s);
  else
    launch_fp8_gemv_mt<kDecodeMaxT>(p, s);
}

}  // namespace moe
