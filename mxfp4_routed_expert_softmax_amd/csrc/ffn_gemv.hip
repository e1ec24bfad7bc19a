// Expert FFN for few rows per expert (decode, verification blocks): an
// HBM-bound MXFP4 dequant-GEMV over only the experts that own rows.
//
// Bytes are the cost: decode speed is roughly bandwidth over routed expert
// bytes per token (FreeToken issue #444, janit's comment, section 1), and a
// verification block pays for the union of its tokens' experts (ai.rs
// article on DeepSeek-V4.1-Flash, "The draft head that works and does not
// pay"). So each selected expert's weights are streamed exactly once per
// group of up to kGemvMT rows, and unselected experts are never touched.
//
// Work decomposition (wave64): a wave owns 8 output rows; lane l = 8*r + j
// works on row r of those 8 and on the 32-element chunks j, j+8, j+16, ...
// of K. Each chunk is one 16-byte load of 32 packed E2M1 codes plus its one
// E8M0 scale byte, and 8 lanes of a row read 128 contiguous bytes, so every
// wave-wide load touches 8 whole 128-byte lines. Codes become bf16 (gate/up)
// or fp32 (down) in registers with the gfx950 scaled conversions; the chunk's
// partial dot product is multiplied by its power-of-two scale (exact) and
// added to an fp32 accumulator. The activations of the rows being processed
// sit in LDS; rows of a wave share the chunk index, so LDS reads broadcast.
// Gate and up rows n are processed by the same lane, so SwiGLU happens in
// registers and only h = silu(g) * u (fp32) is written.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvRowsPerBlock = 32;  // 4 waves x 8 rows
constexpr int kGemvMT = 4;             // rows (tokens) per pass over the weights

struct SlotInfo {
  int e;      // expert slot in its bank, -1 when the slot is empty
  int row0;   // first bucketed row
  int m;      // number of rows
  bool shared;
};

// Block slot s -> expert. Slots [0, routed_slots) are the routed experts
// with rows, in ascending id order; slot routed_slots is the shared expert.
__device__ __forceinline__ SlotInfo resolve_slot(const FfnProblem& p, int s) {
  SlotInfo si{-1, 0, 0, false};
  if (s >= p.routed_slots) {
    if (p.has_shared && s == p.routed_slots) si = SlotInfo{0, 0, p.T, true};
    return si;
  }
  if (p.offsets == nullptr) {
    if (s == 0) si = SlotInfo{0, 0, p.R, false};
    return si;
  }
  int e = -1;
  if (p.active != nullptr) {
    e = p.active[s];
  } else {
    // s-th expert with a non-empty bucket, by ballots over 64 experts at a time
    const int lane = lane_id();
    int rem = s;
    for (int base = 0; base < p.routed.E; base += kWave) {
      const int ee = base + lane;
      const bool act = ee < p.routed.E && p.offsets[ee + 1] > p.offsets[ee];
      uint64_t mask = __ballot(act);
      const int n = __popcll(mask);
      if (rem < n) {
        for (int i = 0; i < rem; ++i) mask &= mask - 1;
        e = base + __ffsll((long long)mask) - 1;
        break;
      }
      rem -= n;
    }
  }
  if (e >= 0 && e < p.routed.E) {
    // clamp to [0, R]: offsets from a caller never move a row out of bounds
    const int lo = min(max(p.offsets[e], 0), p.R);
    const int hi = min(max(p.offsets[e + 1], lo), p.R);
    si.e = e;
    si.row0 = lo;
    si.m = hi - lo;
  }
  return si;
}

// Matrix scale of an NVFP4 bank (1 when absent or MXFP4).
__device__ __forceinline__ float matrix_scale(const BankView& b, int e, int m) {
  return (b.codec == kCodecNvfp4 && b.gscale) ? b.gscale[e * 3 + m] : 1.0f;
}
// The two E4M3 scales of a 32-code chunk (NVFP4), from their two bytes.
__device__ __forceinline__ f32x2_t e4m3x2_to_f32(uint32_t two_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(two_bytes, 1.0f, false);
}

// gate/up + SwiGLU: h[row][n] = silu(W_g[n] . x) * (W_u[n] . x), K = H.
// NV: NVFP4 bank (two E4M3 scales per 32-code chunk, one per 16 codes).
template <int U, bool NV>
__global__ __launch_bounds__(kGemvThreads) void gateup_gemv_kernel(FfnProblem p) {
  extern __shared__ __align__(16) uint4 s_x[];  // [kGemvMT][H/8] bf16
  const SlotInfo si = resolve_slot(p, blockIdx.y);
  if (si.e < 0 || si.m <= 0) return;
  const BankView bk = si.shared ? p.shared : p.routed;
  const int H = p.H, I = p.I;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int n = blockIdx.x * kGemvRowsPerBlock + wave * 8 + (lane >> 3);
  const bool row_ok = n < I;
  const int nr = row_ok ? n : I - 1;
  const int kc = H >> 5;
  const size_t crow = (size_t)H >> 1, srow = (size_t)H >> (NV ? 4 : 5);
  const uint8_t* gc = bk.gu_codes + ((size_t)si.e * 2 * I + nr) * crow;
  const uint8_t* uc = gc + (size_t)I * crow;
  const uint8_t* gs = bk.gu_scales + ((size_t)si.e * 2 * I + nr) * srow;
  const uint8_t* us = gs + (size_t)I * srow;
  const int vpr = H >> 3;
  float* hout = si.shared ? p.h_sh : p.h;

  for (int t0 = 0; t0 < si.m; t0 += kGemvMT) {
    const int nt = min(kGemvMT, si.m - t0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nt * vpr; idx += kGemvThreads) {
      const int t = idx / vpr, c = idx - t * vpr;
      const int r = si.row0 + t0 + t;
      int tok = (si.shared || p.row_token == nullptr) ? r : p.row_token[r];
      tok = min(max(tok, 0), p.T - 1);  // a caller's bad row_token cannot read out of bounds
      s_x[idx] = reinterpret_cast<const uint4*>(p.x + (size_t)tok * H)[c];
    }
    __syncthreads();
    float ag[kGemvMT], au[kGemvMT];
#pragma unroll
    for (int t = 0; t < kGemvMT; ++t) ag[t] = au[t] = 0.0f;
    for (int c0 = 0; c0 < kc; c0 += 8 * U) {
      uint4 wg[U], wu[U];
      uint32_t sg[U], su[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 8 * u + j;
        if (c < kc) {
          wg[u] = *reinterpret_cast<const uint4*>(gc + (size_t)c * 16);
          wu[u] = *reinterpret_cast<const uint4*>(uc + (size_t)c * 16);
          if constexpr (NV) {
            sg[u] = *reinterpret_cast<const uint16_t*>(gs + 2 * (size_t)c);
            su[u] = *reinterpret_cast<const uint16_t*>(us + 2 * (size_t)c);
          } else {
            sg[u] = gs[c];
            su[u] = us[c];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 8 * u + j;
        if (c < kc) {
          f32x2_t fg, fu;
          if constexpr (NV) {
            fg = e4m3x2_to_f32(sg[u]);
            fu = e4m3x2_to_f32(su[u]);
          } else {
            fg.x = fg.y = e8m0_to_f32(sg[u]);
            fu.x = fu.y = e8m0_to_f32(su[u]);
          }
#pragma unroll
          for (int t = 0; t < kGemvMT; ++t) {
            if (t < nt) {
              const uint4* xv = s_x + t * vpr + c * 4;
              const uint4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
              float pg = dot8_fp4_bf16(wg[u].x, x0, 0.0f);
              pg = dot8_fp4_bf16(wg[u].y, x1, pg);
              float pg1 = NV ? 0.0f : pg;
              pg1 = dot8_fp4_bf16(wg[u].z, x2, pg1);
              pg1 = dot8_fp4_bf16(wg[u].w, x3, pg1);
              float pu = dot8_fp4_bf16(wu[u].x, x0, 0.0f);
              pu = dot8_fp4_bf16(wu[u].y, x1, pu);
              float pu1 = NV ? 0.0f : pu;
              pu1 = dot8_fp4_bf16(wu[u].z, x2, pu1);
              pu1 = dot8_fp4_bf16(wu[u].w, x3, pu1);
              if constexpr (NV) {
                ag[t] = fmaf(pg1, fg.y, fmaf(pg, fg.x, ag[t]));
                au[t] = fmaf(pu1, fu.y, fmaf(pu, fu.x, au[t]));
              } else {
                ag[t] = fmaf(pg1, fg.x, ag[t]);
                au[t] = fmaf(pu1, fu.x, au[t]);
              }
            }
          }
        }
      }
    }
    const float mg = matrix_scale(bk, si.e, 0), mu = matrix_scale(bk, si.e, 1);
#pragma unroll
    for (int t = 0; t < kGemvMT; ++t) {
      const float g = group_sum<8>(ag[t]) * mg;
      const float u = group_sum<8>(au[t]) * mu;
      if (row_ok && j == 0 && t < nt) hout[(size_t)(si.row0 + t0 + t) * I + n] = silu_mul(g, u);
    }
  }
}

// down: y[row][n] = W_d[n] . h[row], K = I, h in fp32.
template <int U, bool NV>
__global__ __launch_bounds__(kGemvThreads) void down_gemv_kernel(FfnProblem p) {
  extern __shared__ __align__(16) f32x4_t s_h[];  // [kGemvMT][I/4] fp32
  const SlotInfo si = resolve_slot(p, blockIdx.y);
  if (si.e < 0 || si.m <= 0) return;
  const BankView bk = si.shared ? p.shared : p.routed;
  const int H = p.H, I = p.I;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = lane & 7;
  const int n = blockIdx.x * kGemvRowsPerBlock + wave * 8 + (lane >> 3);
  const bool row_ok = n < H;
  const int nr = row_ok ? n : H - 1;
  const int kc = I >> 5;
  const size_t crow = (size_t)I >> 1, srow = (size_t)I >> (NV ? 4 : 5);
  const uint8_t* dc = bk.d_codes + ((size_t)si.e * H + nr) * crow;
  const uint8_t* ds = bk.d_scales + ((size_t)si.e * H + nr) * srow;
  const int vpr = I >> 2;
  const float* hin = si.shared ? p.h_sh : p.h;
  float* yout = si.shared ? p.y_sh : p.y;

  for (int t0 = 0; t0 < si.m; t0 += kGemvMT) {
    const int nt = min(kGemvMT, si.m - t0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nt * vpr; idx += kGemvThreads) {
      const int t = idx / vpr, c = idx - t * vpr;
      s_h[idx] = reinterpret_cast<const f32x4_t*>(hin + (size_t)(si.row0 + t0 + t) * I)[c];
    }
    __syncthreads();
    float acc[kGemvMT];
#pragma unroll
    for (int t = 0; t < kGemvMT; ++t) acc[t] = 0.0f;
    for (int c0 = 0; c0 < kc; c0 += 8 * U) {
      uint4 wd[U];
      uint32_t sd[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 8 * u + j;
        if (c < kc) {
          wd[u] = *reinterpret_cast<const uint4*>(dc + (size_t)c * 16);
          if constexpr (NV)
            sd[u] = *reinterpret_cast<const uint16_t*>(ds + 2 * (size_t)c);
          else
            sd[u] = ds[c];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 8 * u + j;
        if (c < kc) {
          f32x2_t fd;
          if constexpr (NV)
            fd = e4m3x2_to_f32(sd[u]);
          else
            fd.x = fd.y = e8m0_to_f32(sd[u]);
#pragma unroll
          for (int t = 0; t < kGemvMT; ++t) {
            if (t < nt) {
              const f32x4_t* hv = s_h + t * vpr + c * 8;
              float pd = dot8_fp4_f32(wd[u].x, hv[0], hv[1], 0.0f);
              pd = dot8_fp4_f32(wd[u].y, hv[2], hv[3], pd);
              float pd1 = NV ? 0.0f : pd;
              pd1 = dot8_fp4_f32(wd[u].z, hv[4], hv[5], pd1);
              pd1 = dot8_fp4_f32(wd[u].w, hv[6], hv[7], pd1);
              if constexpr (NV)
                acc[t] = fmaf(pd1, fd.y, fmaf(pd, fd.x, acc[t]));
              else
                acc[t] = fmaf(pd1, fd.x, acc[t]);
            }
          }
        }
      }
    }
    const float md = matrix_scale(bk, si.e, 2);
#pragma unroll
    for (int t = 0; t < kGemvMT; ++t) {
      const float v = group_sum<8>(acc[t]) * md;
      if (row_ok && j == 0 && t < nt) yout[(size_t)(si.row0 + t0 + t) * H + n] = v;
    }
  }
}

size_t ffn_ws_bytes(int T, int H, int I, int R, bool shared) {
  (void)H;
  size_t b = (size_t)R * I * sizeof(float);
  if (shared) b += (size_t)T * I * sizeof(float) + 256;
  return b;
}

void launch_expert_ffn(const FfnProblem& p, hipStream_t s) {
  const int slots = p.routed_slots + (p.has_shared ? 1 : 0);
  if (slots == 0) return;
  const size_t lds_gu = (size_t)kGemvMT * p.H * sizeof(uint16_t);
  const size_t lds_d = (size_t)kGemvMT * p.I * sizeof(float);
  const bool nv = p.routed.codec == kCodecNvfp4;
  launch("gateup_gemv_kernel", nv ? gateup_gemv_kernel<5, true> : gateup_gemv_kernel<5, false>,
                     dim3((p.I + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock, slots),
                     dim3(kGemvThreads), lds_gu, s, p);
  launch("down_gemv_kernel", nv ? down_gemv_kernel<9, true> : down_gemv_kernel<9, false>,
                     dim3((p.H + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock, slots),
                     dim3(kGemvThreads), lds_d, s, p);
}

}  // namespace moe
