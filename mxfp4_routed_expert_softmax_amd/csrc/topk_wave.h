// Wave-wide top-k of one row of logits on gfx950, shared by the few-token
// routing and the top-k launch: fp64 max over order-preserving 64-bit keys
// of (logit, expert), exchanged with DPP inside rows of 16 lanes and lane
// swaps across rows, so a round never leaves the vector unit.
#pragma once

#include "moe_device.h"

namespace moe {

// Key of (logit, expert) that orders like (logit descending, id ascending)
// and whose bits, read as an fp64, are a positive normal number (or +0 for
// an empty slot), so fp64 max picks the larger key: the order-preserving
// 32-bit image of the logit in bits 62..31, 2^31 - 1 - e below. NaN logits
// rank as -inf, so no key is an fp64 NaN, infinity or subnormal.
__device__ __forceinline__ uint64_t topk_key_f64(float v, int e) {
  v = (v != v) ? -INFINITY : v;
  uint32_t b = __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 31) | (uint32_t)(0x7fffffffu - (uint32_t)e);
}

template <int CTRL>
__device__ __forceinline__ double dpp_max_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)u, (int)(uint32_t)u, CTRL,
                                                            0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(u >> 32),
                                                            (int)(uint32_t)(u >> 32), CTRL, 0xf,
                                                            0xf, false);
  return fmax(v, __longlong_as_double((long long)(((uint64_t)hi << 32) | lo)));
}

// Wave-wide maximum of such keys, in every lane, without leaving the vector
// unit: DPP within each row of 16 lanes (xor 1, xor 2, half-row mirror, row
// mirror), then lane swaps across rows (16, then 32 apart).
__device__ __forceinline__ uint64_t wave_max_key_f64(uint64_t k) {
  double v = __longlong_as_double((long long)k);
  v = dpp_max_f64<0xB1>(v);
  v = dpp_max_f64<0x4E>(v);
  v = dpp_max_f64<0x141>(v);
  v = dpp_max_f64<0x140>(v);
  uint64_t u = (uint64_t)__double_as_longlong(v);
  {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false,
                                                     false);
    v = fmax(__longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0])),
             __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1])));
  }
  u = (uint64_t)__double_as_longlong(v);
  {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false,
                                                     false);
    v = fmax(__longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0])),
             __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1])));
  }
  return (uint64_t)__double_as_longlong(v);
}

// Wave-wide top-k of one logit row; lanes < k write ids / weights, in
// selection order (logit descending, ties to the lower id), with fp64-max
// keys (one v_max_f64 per exchange); lane l holds experts l, l + 64, ...
// (E <= 64 NK). Weights: softmax over the k chosen logits, summed over
// j = 0..k-1 in order.
template <int NK>
__device__ void topk_row_f64(const float (&lv)[NK], int E, int k, int* ids, float* w) {
  const int lane = lane_id();
  double key[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + kWave * i;
    key[i] = __longlong_as_double(e < E ? (long long)topk_key_f64(lv[i], e) : 0);
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
      my_id = (int)min(id, (uint32_t)(E - 1));
    }
    if (j == 0) top = val;
  }
  const float z = lane < k ? expf(my_val - top) : 0.0f;
  float zsum = 0.0f;
  for (int q = 0; q < k; ++q)
    zsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), q));
  if (lane < k) {
    ids[lane] = my_id;
    w[lane] = z / zsum;
  }
}

}  // namespace moe
