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
// row is handled by 4 lanes holding 32 values each.  5 of the 7 butterfly
// stages run in registers on the loaded layout, the other 2 in registers after
// an exchange through LDS, so no stage needs a cross-lane move per value.  The
// 8 heads of a token are adjacent in the input, so a workgroup reads 8 runs of
// 2 KB, and writes per head a run of 8 x 128 B codes in the head-major store.
// Consecutive workgroups take consecutive head blocks of the same tokens, so
// the blocks in flight read whole token rows.  256 B are read and 130 B
// written per row; at about 460 vector instructions per wave of 16 rows the
// kernel keeps up with HBM.
#include "h3a_device.h"
#include "launch.h"

#include <type_traits>

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
//
// Rotation: the 4 lanes of a row load 8 bf16 values from each 32-value quarter
// (lane sub holds elements 32k + 8sub + e in v[8k + e]) and run the 5
// butterfly stages on index bits 0-2 and 5-6 in registers.  The remaining two
// stages (bits 3-4) run in registers too after an exchange through LDS that
// leaves lane sub with the 32 consecutive elements 32sub .. 32sub+31.  The
// exchange goes in two halves (e < 4, then e >= 4) so that a wave needs 4 KB
// of LDS: 16 rows of 64 floats, in 16-byte chunks whose index c is XOR-swizzled
// with the row and the high bits of c, which keeps the 16 lanes of each quarter
// wave on distinct banks for both the writes and the reads.  Each wave only
// touches its own 16 rows, and the LDS requests of one wave complete in issue
// order, so the wavefront-scope fences are enough: they stop the compiler from
// moving a read above the writes it depends on, or a write above a read.
template <bool GROUPED>
__global__ __launch_bounds__(256) void kvi8r_quantize_kernel(QuantTensor t0, QuantTensor t1,
                                                             int64_t x_token_stride, int64_t n_tokens,
                                                             int64_t token_offset, int64_t s_total, int32_t n_heads,
                                                             uint32_t n_head_blocks) {
  __shared__ __align__(16) float lds[4 * 16 * 64];
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

  float v[32];
  const uint16_t* src = x + (valid ? t : 0) * x_token_stride + (int64_t)(valid ? head : 0) * kHeadDim;
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

  // Chunk c of a row's half holds 4 values; writer lane sub puts quarter k at
  // c = 4k + sub, reader lane sub takes c = 4sub + s.  Stored at c ^ (c >> 2) ^ 4(row & 3).
  float* rowbuf = lds + row_in_block * 64;
  const int m = lane & 15;                      // 4 (row & 3) + sub
  const int rbase = (5 * sub) ^ (4 * ((lane >> 2) & 3));
  float y[32];                                   // y[i] = element 32sub + i
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 q = {v[8 * k + 4 * h], v[8 * k + 4 * h + 1], v[8 * k + 4 * h + 2], v[8 * k + 4 * h + 3]};
      *reinterpret_cast<float4*>(rowbuf + 4 * (m ^ (5 * k))) = q;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const float4 q = *reinterpret_cast<const float4*>(rowbuf + 4 * (rbase ^ s2));
      y[8 * s2 + 4 * h] = q.x;
      y[8 * s2 + 4 * h + 1] = q.y;
      y[8 * s2 + 4 * h + 2] = q.z;
      y[8 * s2 + 4 * h + 3] = q.w;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int mm = 8; mm < 32; mm <<= 1)           // bits 3..4
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (!(i & mm)) {
        const float u = y[i], w = y[i + mm];
        y[i] = u + w;
        y[i + mm] = u - w;
      }
  // y now holds the rotated row times sqrt(128), elements 32sub .. 32sub+31.

  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(y[i]));
  if constexpr (!GROUPED) {
    a = fmaxf(a, dpp_f32<kDppXor1>(a));
    a = fmaxf(a, dpp_f32<kDppXor2>(a));
  }
  // scale = fp16(max|y| / 127) from the (exact) fp32 absmax, in fp64; then the
  // reciprocal that maps unnormalised values onto the code grid.
  const uint32_t sbits = f64_to_f16_rne_sat((double)a * kInv127Sqrt128);
  const float r = sbits ? (float)(1.0 / (f16_bits_to_f64(sbits) * kSqrt128)) : 0.0f;

  // code = round-half-even(y / s): one fused multiply-add with the magic
  // constant rounds the exact product once, and the integer sits in the low
  // bits of the result.  |y / s| stays below 127.07 when s is a normal fp16
  // short of the largest (s is within 2^-11 of max|y| / 127); a wave holding
  // a subnormal or saturated scale clamps with med3 to [-127, 127].
  const bool wide = sbits != 0u && (sbits < 0x0400u || sbits >= 0x7BFFu);
  uint32_t packed[8];
  auto quantise = [&](auto clamp) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f = __builtin_fmaf(y[4 * i + j], r, kMagic);
        if constexpr (decltype(clamp)::value) f = __builtin_amdgcn_fmed3f(f, kMagic - 127.0f, kMagic + 127.0f);
        b[j] = __float_as_uint(f);
      }
      const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
      packed[i] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  };
  if (__any(wide)) quantise(std::true_type{});
  else quantise(std::false_type{});

  if (valid) {
    const int64_t row = (int64_t)head * s_total + token_offset + t;
    u32x4* dst = reinterpret_cast<u32x4*>(codes + row * kHeadDim + 32 * sub);
    dst[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
    dst[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
    if constexpr (GROUPED) {
      scales[row * 4 + sub] = (uint16_t)sbits;
    } else {
      if (sub == 0) scales[row] = (uint16_t)sbits;
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
