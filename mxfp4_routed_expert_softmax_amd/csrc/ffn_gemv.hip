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

// gate/up + SwiGLU: h[row][n] = silu(W_g[n] . x) * (W_u[n] . x), K = H.
template <int U>
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
  const size_t crow = (size_t)H >> 1, srow = (size_t)H >> 5;
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
          sg[u] = gs[c];
          su[u] = us[c];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 8 * u + j;
        if (c < kc) {
          const float fg = e8m0_to_f32(sg[u]), fu = e8m0_to_f32(su[u]);
#pragma unroll
          for (int t = 0; t < kGemvMT; ++t) {
            if (t < nt) {
              const uint4* xv = s_x + t * vpr + c * 4;
              const uint4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
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
    for (int t = 0; t < kGemvMT; ++t) {
      const float g = group_sum<8>(ag[t]);
      const float u = group_sum<8>(au[t]);
      if (row_ok && j == 0 && t < nt) hout[(size_t)(si.row0 + t0 + t) * I + n] = silu_mul(g, u);
    }
  }
}

// down: y[row][n] = W_d[n] . h[row], K = I, h in fp32.
template <int U>
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
  const size_t crow = (size_t)I >> 1, srow = (size_t)I >> 5;
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
          sd[u] = ds[c];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 8 * u + j;
        if (c < kc) {
          const float fd = e8m0_to_f32(sd[u]);
#pragma unroll
          for (int t = 0; t < kGemvMT; ++t) {
            if (t < nt) {
              const f32x4_t* hv = s_h + t * vpr + c * 8;
              float pd = dot8_fp4_f32(wd[u].x, hv[0], hv[1], 0.0f);
              pd = dot8_fp4_f32(wd[u].y, hv[2], hv[3], pd);
              pd = dot8_fp4_f32(wd[u].z, hv[4], hv[5], pd);
              pd = dot8_fp4_f32(wd[u].w, hv[6], hv[7], pd);
              acc[t] = fmaf(pd, fd, acc[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kGemvMT; ++t) {
      const float v = group_sum<8>(acc[t]);
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
  launch("gateup_gemv_kernel", gateup_gemv_kernel<5>,
                     dim3((p.I + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock, slots),
                     dim3(kGemvThreads), lds_gu, s, p);
  launch("down_gemv_kernel", down_gemv_kernel<9>,
                     dim3((p.H + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock, slots),
                     dim3(kGemvThreads), lds_d, s, p);
}

}  // namespace moe
