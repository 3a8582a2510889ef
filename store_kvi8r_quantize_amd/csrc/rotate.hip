// rotate_q / unrotate_o: the query rotation and the single output un-rotation
// of the kvi8r store ("H3 Streamed Blocks" node page, Inputs table, kv_store
// row; "Low VRAM, low RAM", "The K/V store options", rotation paragraph:
// scores are invariant under the rotation and P.V is brought back through the
// transpose once).  The basis is symmetric, so both directions are y = x H.
//
// Same lane layout as kvi8r_quantize: 4 lanes per 128-value row, 16 rows per
// wave.  rotate_q multiplies each value by post before its one rounding to
// fp16: 1, or softmax_scale * log2 e for the kvi8r32 store, whose attention
// then needs no per-score factor.  Both kernels are HBM-bound streams: rotate reads 256 B and writes 256 B
// per row; unrotate reads 512 B and writes 256 B per row (fp16 or bf16).
#include "h3a_device.h"
#include "launch.h"

namespace h3a {

namespace {

__global__ __launch_bounds__(256) void rotate_q_kernel(const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ y, int64_t n_rows, float post) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 3;
  const int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 2);
  if (row >= n_rows) return;  // whole quads leave together: DPP partners stay active
  const float cs = kInvSqrt128f * post;  // post = 1 leaves 1/sqrt(128) unchanged
  const uint16_t* src = x + row * kHeadDim;
  float v[32];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + 32 * k + 8 * sub);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * k + 2 * i] = bf16lo_to_f32(w[i]);
      v[8 * k + 2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  }
  fwht32_in_lane(v);
  fwht32_cross_lane(v, sub);
  uint16_t* dst = y + row * kHeadDim;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_f16x2(v[8 * k + 2 * i] * cs, v[8 * k + 2 * i + 1] * cs);
    *reinterpret_cast<u32x4*>(dst + 32 * k + 8 * sub) = w;
  }
}

// F16: the output is fp16 (the precision kvi8r attention runs in), else bf16.
template <bool F16>
__global__ __launch_bounds__(256) void unrotate_o_kernel(const float* __restrict__ x,
                                                         uint16_t* __restrict__ y, int64_t n_rows) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 3;
  const int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 2);
  if (row >= n_rows) return;
  const float* src = x + row * kHeadDim;
  float v[32];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(src + 32 * k + 8 * sub);
    const u32x4 b = *reinterpret_cast<const u32x4*>(src + 32 * k + 8 * sub + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * k + i] = __uint_as_float(a[i]);
      v[8 * k + 4 + i] = __uint_as_float(b[i]);
    }
  }
  fwht32_in_lane(v);
  fwht32_cross_lane(v, sub);
  uint16_t* dst = y + row * kHeadDim;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = v[8 * k + 2 * i] * kInvSqrt128f, b = v[8 * k + 2 * i + 1] * kInvSqrt128f;
      w[i] = F16 ? pack_f16x2(a, b) : pack_bf16x2(a, b);
    }
    *reinterpret_cast<u32x4*>(dst + 32 * k + 8 * sub) = w;
  }
}

}  // namespace

hipError_t launch_rotate_q(const uint16_t* x, uint16_t* y, int64_t n_rows, float post, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rotate_q_kernel, dim3((unsigned)((n_rows + 63) / 64)), dim3(256), 0, stream, x, y,
                     n_rows, post);
  return hipGetLastError();
}

hipError_t launch_unrotate_o(const float* x, uint16_t* y, int64_t n_rows, bool f16, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_rows + 63) / 64));
  if (f16)
    hipLaunchKernelGGL(unrotate_o_kernel<true>, grid, dim3(256), 0, stream, x, y, n_rows);
  else
    hipLaunchKernelGGL(unrotate_o_kernel<false>, grid, dim3(256), 0, stream, x, y, n_rows);
  return hipGetLastError();
}

}  // namespace h3a
