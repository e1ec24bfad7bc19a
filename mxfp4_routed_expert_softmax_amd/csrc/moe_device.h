// Device-side helpers for the gfx950 kernels: bf16 / E2M1 / E8M0 decoding,
// wave64 reductions and scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// E8M0 scale byte -> fp32 2^(s-127). s == 0 is the subnormal 2^-127 and
// s == 255 encodes NaN (OCP Microscaling v1.0).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t b = s << 23;
  b = (s == 0u) ? 0x00400000u : b;
  b = (s == 255u) ? 0x7fc00000u : b;
  return __uint_as_float(b);
}

// Two E2M1 codes (byte SEL of `w`: low nibble -> .x, high nibble -> .y) to
// bf16 / fp32 / fp16 with the gfx950 scaled conversion at scale 1.0. Every
// E2M1 value is exact in all three formats.
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f16x2_t fp4x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) {
  return __builtin_bit_cast(bf16x2_t, v);
}

// 8 E2M1 codes of a 32-bit word dotted with 8 bf16 (4 words) of x, fp32
// accumulation: sum_i code_i * x_i + acc.
__device__ __forceinline__ float dot8_fp4_bf16(uint32_t w, uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16<0>(w), as_bf16x2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16<1>(w), as_bf16x2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16<2>(w), as_bf16x2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16<3>(w), as_bf16x2(x.w), acc, false);
  return acc;
}

// 8 E2M1 codes of a word times 8 fp32 values, fp32 fused multiply-adds.
__device__ __forceinline__ float dot8_fp4_f32(uint32_t w, f32x4_t a, f32x4_t b, float acc) {
  f32x2_t p0 = fp4x2_to_f32<0>(w), p1 = fp4x2_to_f32<1>(w);
  f32x2_t p2 = fp4x2_to_f32<2>(w), p3 = fp4x2_to_f32<3>(w);
  acc = fmaf(p0.x, a.x, acc); acc = fmaf(p0.y, a.y, acc);
  acc = fmaf(p1.x, a.z, acc); acc = fmaf(p1.y, a.w, acc);
  acc = fmaf(p2.x, b.x, acc); acc = fmaf(p2.y, b.y, acc);
  acc = fmaf(p3.x, b.z, acc); acc = fmaf(p3.y, b.w, acc);
  return acc;
}

// bf16 pair dot product with fp32 accumulation.
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
  return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                        0xf, 0xf, false));
}

// Sum over groups of G consecutive lanes (G a power of two <= 64), in every
// lane of the group, without the LDS pipe: DPP within each row of 16 lanes
// (xor 1, xor 2, half-row mirror, row mirror; each step pairs lanes that
// already hold equal partial sums), then the gfx950 lane swaps across rows
// (16 apart, then 32), each of which hands every lane its own value and its
// partner's. Both operands of every add are the same pair in the two lanes,
// so all lanes of a group end with the same bits.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G: a power of two up to 64");
  if constexpr (G >= 2) v = dpp_add<0xB1>(v);
  if constexpr (G >= 4) v = dpp_add<0x4E>(v);
  if constexpr (G >= 8) v = dpp_add<0x141>(v);
  if constexpr (G >= 16) v = dpp_add<0x140>(v);
  if constexpr (G >= 32) {
    const uint32_t u = __float_as_uint(v);
    const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  }
  if constexpr (G >= 64) {
    const uint32_t u = __float_as_uint(v);
    const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum over a block of up to 1024 threads (blockDim.x a
// multiple of 64). `tmp` holds >= 16 ints of shared memory. Also returns the
// block total. Contains __syncthreads: call from uniform control flow.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  int inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == kWave - 1) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int t = (lane < nwaves) ? tmp[lane] : 0;
    int ti = wave_inclusive_scan(t);
    if (lane < nwaves) tmp[lane] = ti - t;   // exclusive wave offsets
    if (lane == nwaves - 1) tmp[16] = ti;    // block total
  }
  __syncthreads();
  int r = tmp[wave] + inc - v;
  *total = tmp[16];
  return r;
}

}  // namespace moe
