// kvi8r_quantize: bf16 K/V rows -> rotated int8 codes + one fp16 scale per row.
//
// Computes what the kv_store row of the "H3 Streamed Blocks" node page's Inputs
// table describes for the kvi8r store (see also "Low VRAM, low RAM", "The K/V
// store options"): rotate each (token, head) row of 128 values into the fixed
// orthonormal Hadamard basis, take its absmax, store fp16(absmax/127) and the
// int8 codes of the row against that stored scale.
//
// GROUPED: the per-32-value variant ("Low VRAM, low RAM", "What is next": a
// scale per 32 values, finer than per row).  Each group of 32 consecutive
// rotated values gets its own fp16 scale and its codes are taken against it;
// scales are stored [n_heads, s_total, 4].
//
// Layout on MI355X: one workgroup = 4 waves = 64 rows = 8 tokens x 8 heads; a
// row is handled by 4 lanes holding 32 values each, so 5 of the 7 butterfly
// stages stay in registers and 2 use quad DPP moves.  The 8 heads of a token
// are adjacent in the input, so a workgroup reads 8 runs of 2 KB, and writes
// per head a run of 8 x 128 B codes in the head-major store.  Consecutive
// workgroups take consecutive head blocks of the same tokens, so the blocks
// in flight read whole token rows.  The kernel is HBM-bound: 256 B read +
// 130 B written per row.
#include "h3a_device.h"
#include "launch.h"

namespace h3a {

namespace {

constexpr int kHeadsPerBlock = 8;
constexpr int kTokensPerBlock = 64 / kHeadsPerBlock;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: adding it rounds |x| < 2^22 to an integer, ties to even

// One tensor of a launch: input rows and the store they go to.
struct QuantTensor {
  const uint16_t* x;
  int8_t* codes;
  uint16_t* scales;
};

// blockIdx.y selects the tensor: a launch quantises K and V of one kv_chunk together.
template <bool GROUPED>
__global__ __launch_bounds__(256) void kvi8r_quantize_kernel(QuantTensor t0, QuantTensor t1,
                                                             int64_t x_token_stride, int64_t n_tokens,
                                                             int64_t token_offset, int64_t s_total, int32_t n_heads,
                                                             uint32_t n_head_blocks) {
  const QuantTensor tt = blockIdx.y == 0 ? t0 : t1;
  const uint16_t* __restrict__ x = tt.x;
  int8_t* __restrict__ codes = tt.codes;
  uint16_t* __restrict__ scales = tt.scales;
  const int lane = threadIdx.x & 63;
  const int sub = lane & 3;
  const int row_in_block = (threadIdx.x >> 6) * 16 + (lane >> 2);
  const uint32_t hb = blockIdx.x % n_head_blocks, tb = blockIdx.x / n_head_blocks;
  const int head = (int)hb * kHeadsPerBlock + row_in_block % kHeadsPerBlock;
  const int64_t t = (int64_t)tb * kTokensPerBlock + row_in_block / kHeadsPerBlock;
  const bool valid = t < n_tokens && head < n_heads;

  // Element j = 32k + 8*sub + e  <->  v[8k + e].
  float v[32];
  const uint16_t* src = x + (valid ? t : 0) * x_token_stride + (int64_t)(valid ? head : 0) * kHeadDim;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (valid) w = *reinterpret_cast<const u32x4*>(src + 32 * k + 8 * sub);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * k + 2 * i] = bf16lo_to_f32(w[i]);
      v[8 * k + 2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  }

  fwht32_in_lane(v);
  fwht32_cross_lane(v, sub);  // v now holds y * sqrt(128)

  // Absmax of the row (one group) or of each 32-value group k = elements
  // 32k..32k+31, held as v[8k..8k+7] on the quad's four lanes.
  constexpr int NG = GROUPED ? 4 : 1;
  float a[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) a[gi] = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a[GROUPED ? i >> 3 : 0] = fmaxf(a[GROUPED ? i >> 3 : 0], fabsf(v[i]));
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    a[gi] = fmaxf(a[gi], dpp_f32<kDppXor1>(a[gi]));
    a[gi] = fmaxf(a[gi], dpp_f32<kDppXor2>(a[gi]));
  }

  // scale = fp16(max|y| / 127) from the (exact) fp32 absmax, in fp64; then the
  // reciprocal that maps unnormalised values onto the code grid.
  uint32_t sbits[NG];
  float r[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    sbits[gi] = f64_to_f16_rne_sat((double)a[gi] * kInv127Sqrt128);
    r[gi] = sbits[gi] ? (float)(1.0 / (f16_bits_to_f64(sbits[gi]) * kSqrt128)) : 0.0f;
  }

  // code = clamp(round-half-even(y / s)): one fused multiply-add with the magic
  // constant rounds the exact product once; med3 clamps to [-127, 127].
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float f = __builtin_fmaf(v[4 * i + j], r[GROUPED ? i >> 1 : 0], kMagic);
      f = __builtin_amdgcn_fmed3f(f, kMagic - 127.0f, kMagic + 127.0f);
      b[j] = __float_as_uint(f);
    }
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
    packed[i] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }

  if (valid) {
    const int64_t row = (int64_t)head * s_total + token_offset + t;
    int8_t* dst = codes + row * kHeadDim;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x2 w = {packed[2 * k], packed[2 * k + 1]};
      *reinterpret_cast<u32x2*>(dst + 32 * k + 8 * sub) = w;
    }
    if constexpr (GROUPED) {
      if (sub == 0)
        *reinterpret_cast<u32x2*>(scales + row * 4) = u32x2{sbits[0] | (sbits[1] << 16), sbits[2] | (sbits[3] << 16)};
    } else {
      if (sub == 0) scales[row] = (uint16_t)sbits[0];
    }
  }
}

}  // namespace

hipError_t launch_kvi8r_quantize(const uint16_t* x, const uint16_t* x2, int64_t x_token_stride, int64_t n_tokens,
                                 int32_t n_heads, int64_t token_offset, int64_t s_total, int8_t* codes,
                                 int8_t* codes2, uint16_t* scales, uint16_t* scales2, bool grouped,
                                 hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  // head blocks fastest: workgroup b covers head block b % n_head_blocks of token block b / n_head_blocks
  const uint32_t n_head_blocks = (uint32_t)((n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
  const int64_t n_wg = (n_tokens + kTokensPerBlock - 1) / kTokensPerBlock * n_head_blocks;
  if (n_wg > 0xFFFFFFFFll) return hipErrorInvalidValue;
  const QuantTensor t0{x, codes, scales}, t1{x2, codes2, scales2};
  const dim3 grid((unsigned)n_wg, x2 != nullptr ? 2u : 1u);
  if (grouped)
    hipLaunchKernelGGL(kvi8r_quantize_kernel<true>, grid, dim3(256), 0, stream, t0, t1, x_token_stride, n_tokens,
                       token_offset, s_total, n_heads, n_head_blocks);
  else
    hipLaunchKernelGGL(kvi8r_quantize_kernel<false>, grid, dim3(256), 0, stream, t0, t1, x_token_stride, n_tokens,
                       token_offset, s_total, n_heads, n_head_blocks);
  return hipGetLastError();
}

}  // namespace h3a
