// Internal launchers (host side); the C ABI in h3a_api.hip validates arguments
// and then calls these.  Every launcher queues work on `stream` and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3a {

// grouped: one scale per 32 rotated values, scales [n_heads, s_total, 4]; else one per row [n_heads, s_total].
// x2 / codes2 / scales2: a second tensor quantised in the same launch (K and V of one chunk), or null.
hipError_t launch_kvi8r_quantize(const uint16_t* x, const uint16_t* x2, int64_t x_token_stride, int64_t n_tokens,
                                 int32_t n_heads, int64_t token_offset, int64_t s_total, int8_t* codes,
                                 int8_t* codes2, uint16_t* scales, uint16_t* scales2, bool grouped,
                                 hipStream_t stream);

// post: a factor applied before the rounding to fp16 (1, or softmax_scale * log2 e
// for the kvi8r32 store's attention).
hipError_t launch_rotate_q(const uint16_t* x, uint16_t* y, int64_t n_rows, float post, hipStream_t stream);
// f16: write fp16 rows, else bf16.
hipError_t launch_unrotate_o(const float* x, uint16_t* y, int64_t n_rows, bool f16, hipStream_t stream);

// One query chunk of attention.
struct AttnChunk {
  const uint16_t* q;       // exact: bf16 Q rows [rows, H, 128]; kvi8r: rotated fp16 Q' [rows, H, 128]
  const void* k;           // exact: bf16 [s_kv, H, 128]; kvi8r, kvi8r32: int8 codes [H, s_kv, 128]
  const void* v;
  const uint16_t* k_scale; // kvi8r: fp16 [H, s_kv]; kvi8r32: fp16 [H, s_kv, 4]
  const uint16_t* v_scale;
  void* out;               // exact: bf16 [rows, H, 128]; kvi8r: fp32 O' (normalised, rotated) [rows, H, 128]
  union {
    const int32_t* counts;  // sparse: kept-tile count per (head, 64-row q-tile) of the chunk
    const float* state_in;  // dense, K/V streamed block by block: (m, l, O) to resume from; null on the first block
  };
  union {
    const int32_t* lists;   // sparse: kept KV-tile indices [H, n_qtiles, n_kt], increasing
    float* state_out;       // dense, block by block: where to leave (m, l, O); null on the last block
  };
  int64_t rows;
  int64_t s_kv;
  int32_t n_heads;
  float scale_log2;        // softmax_scale * log2(e)
};

// Sol residual of the sparse kernel: dropped tiles as pseudo-keys.
struct SolArgs {
  const int32_t* drops;    // dropped KV-tile indices [H, n_qtiles, n_kt], increasing; count = n_kt - kept
  const uint16_t* kmean;   // per (head, KV tile): tile-mean key / kmscale, fp16 (kvi8r) or bf16 [H, n_kt, 128]
  const uint16_t* vmean;   // per (head, KV tile): tile-mean value, same type [H, n_kt, 128]
  const float* kmscale;    // per (head, KV tile): power-of-two scale of kmean [H, n_kt]
};
// Longest store with the Sol residual: the kernel addresses one head's mean
// tables (n_kt rows of 256 bytes) with 32-bit offsets, one row past the end
// included, so n_kt * 256 must stay below 2^32.
constexpr int64_t kSolMaxKv = ((int64_t)1 << 30) - 64;

constexpr int kSparseBlockRows = 64;  // q-tile of the sparse kernel = the routing granularity

// sol: null, or the Sol residual (sparse only).
hipError_t launch_attn_fwd(int mode, bool sparse, const AttnChunk& a, const SolArgs* sol, hipStream_t stream);

// Dense attention of one query chunk against one K/V block, carrying the
// online-softmax state through a.state_in / a.state_out.  The state takes
// kStateFloats floats per thread of the launch: dense_state_floats(rows, H).
constexpr int kStateFloats = 66;  // 64 O accumulators, m, l
int64_t dense_state_floats(int64_t rows, int32_t n_heads);
hipError_t launch_attn_fwd_block(int mode, const AttnChunk& a, hipStream_t stream);

// Kept-tile lists (and, when drops is not null, dropped-tile lists) for the
// q-tiles [qt0, qt0 + n_qt) of every head.
hipError_t launch_route_build(const uint8_t* mask, int64_t n_qt_total, int64_t qt0, int32_t n_qt,
                              int32_t n_kt, int32_t n_heads, int32_t* counts, int32_t* lists,
                              int32_t* drops, hipStream_t stream);

// Tile means of the whole store (Sol residual): kmean, vmean [H, n_kt, 128]
// and kmscale [H, n_kt], as described in SolArgs.  k, v, k_scale, v_scale as
// in AttnChunk for `mode`.
hipError_t launch_tile_means(int mode, const void* k, const void* v, const uint16_t* k_scale,
                             const uint16_t* v_scale, int64_t s_kv, int32_t n_heads, uint16_t* kmean,
                             uint16_t* vmean, float* kmscale, hipStream_t stream);

}  // namespace h3a
