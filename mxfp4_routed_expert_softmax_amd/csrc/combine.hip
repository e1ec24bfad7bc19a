// Weighted combine in a fixed order: out[t] = y_shared[t] + sum_j w[t][j] *
// y_rows[inv_row[t][j]], j ascending, one fp32 fused multiply-add per term.
// A gather, not a scatter: no atomics, so the summation order never depends
// on scheduling (the pages tie irreproducible runs to a varying accumulation
// order: ai.rs article on DeepSeek-V4.1-Flash, "What remains is the
// reference rounding itself").
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_rows,
                                                      const int32_t* __restrict__ inv_row,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ y_sh, int T,
                                                      int k, int H, int R,
                                                      float* __restrict__ out) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;  // float4 column
  const int nv = H >> 2;
  if (c >= nv) return;
  float4 acc = y_sh ? reinterpret_cast<const float4*>(y_sh + (size_t)t * H)[c]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int r = inv_row[(size_t)t * k + j];
    if (r < 0) continue;
    const float wj = w[(size_t)t * k + j];
    float4 y;
    if (r < R) {
      y = reinterpret_cast<const float4*>(y_rows + (size_t)r * H)[c];
    } else {
      const float nan = __builtin_nanf("");
      y = make_float4(nan, nan, nan, nan);
    }
    acc.x = fmaf(wj, y.x, acc.x);
    acc.y = fmaf(wj, y.y, acc.y);
    acc.z = fmaf(wj, y.z, acc.z);
    acc.w = fmaf(wj, y.w, acc.w);
  }
  reinterpret_cast<float4*>(out + (size_t)t * H)[c] = acc;
}

void launch_combine(const float* y_rows, const int32_t* inv_row, const float* w,
                    const float* y_shared, int T, int k, int H, int R, float* out,
                    hipStream_t s) {
  const int nv = H >> 2;
  launch("combine_kernel", combine_kernel, dim3(T, (nv + 255) / 256), dim3(256), 0, s, y_rows,
                     inv_row, w, y_shared, T, k, H, R, out);
}

}  // namespace moe
