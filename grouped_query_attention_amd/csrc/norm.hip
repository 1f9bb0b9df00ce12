// Root-mean-square normalisation of token rows ahead of the QKV projection.
//
// "Llama 3.1 8B · Merge and project", section "Contextual evidence from
// Output projection": the attention half of the block reads attention_norm(x)
// (RMSNorm with norm_eps = 1e-5 in the catalogue entry) and adds its update to
// x. The formula is not on the pages; the one implemented is root-mean-square
// layer normalisation with a per-feature gain and eps under the root:
//   y[t][i] = w[i] · x[t][i] / sqrt(mean over j of x[t][j]^2 + eps).
//
// HBM-bound: 8 KiB read and 8 KiB written per token (the gain, 8 KiB in all,
// stays in L2). One wave per row; lane l holds features 512 i + 8 l .. + 7 for
// i = 0..7, so each of the eight 16-byte loads of a wave covers 1 KiB of
// consecutive bytes. The sum of squares is taken in fp32 (lane partials, then a
// butterfly across the wave), the products in fp32 and one bf16 rounding
// (nearest even) at the end.

#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr int NORM_ROWS = 4;  // rows (waves) per workgroup

__global__ __launch_bounds__(64 * NORM_ROWS) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ w,
                                                                 float eps, int M,
                                                                 uint16_t* __restrict__ y) {
  const int row = blockIdx.x * NORM_ROWS + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const uint16_t* xr = x + (size_t)row * D_MODEL + 8 * lane;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = ld16(xr + 512 * i);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = bf16lo(v[i][c]), hi = bf16hi(v[i][c]);
      ss = __builtin_fmaf(lo, lo, ss);
      ss = __builtin_fmaf(hi, hi, ss);
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float r = 1.0f / __builtin_sqrtf(ss * (1.0f / D_MODEL) + eps);
  uint16_t* yr = y + (size_t)row * D_MODEL + 8 * lane;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 g = ld16(w + 512 * i + 8 * lane);
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c] = pack_bf16x2(bf16lo(v[i][c]) * r * bf16lo(g[c]), bf16hi(v[i][c]) * r * bf16hi(g[c]));
    st16(yr + 512 * i, o);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, int M, uint16_t* y,
                          hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((M + NORM_ROWS - 1) / NORM_ROWS), dim3(64 * NORM_ROWS),
                     0, s, x, w, eps, M, y);
  return hipGetLastError();
}

}  // namespace gqa
