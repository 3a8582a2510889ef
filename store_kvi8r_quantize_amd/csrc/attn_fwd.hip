// attn_fwd: one query chunk of full attention against the whole K/V store, with
// the online-softmax state carried in registers across every K/V block.
//
// What it computes: the attention step of the "H3 Streamed Blocks" node page
// ("How it works"; Inputs table rows q_chunk, kv_block, kv_store) for the
// "bf16 (exact)" store and the "kvi8r" store ("Low VRAM, low RAM", "The K/V
// store options": a K/V block dequant is one int8 -> fp16 cast times the row
// scale, attention in fp16 with an online-softmax combine), optionally
// restricted to the kept 64Q x 64KV tiles of a mask ("H3-Optimizations" page,
// Nodes: routed 64Q x 64KV geometry, hard arm drops rejected tiles), with the
// dropped tiles optionally entering as block-mean pseudo-keys (the Sol arm of
// that paragraph).  Also here: the kept/dropped tile lists, the tile means of
// the Sol arm, and a dense variant that takes the K/V store one block at a
// time and carries the softmax state through memory between blocks (a store
// held in host memory; node page, kv_block row).
//
// MI355X design
//   * Dense: workgroup = 8 waves x 32 query rows = 256 rows of one head, two
//     waves per SIMD in a ping-pong (see attn_fwd_dense_kernel).  Sparse:
//     2 waves x 32 rows = one 64-row routing tile; for the exact store, 8 waves
//     for two routing tiles, half of them only staging (attn_fwd_sparse_pair_kernel).
//     Key/value tiles of 64 tokens.
//   * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_{f16,bf16}: the
//     query index runs across lanes, keys across the 16 accumulator registers,
//     so the softmax row sums are in-lane (plus one exchange between lanes l
//     and l^32).  P^T then feeds O^T += V^T P^T directly from registers as the
//     B operand; the key order inside each 16-key step is chosen to match the
//     accumulator layout.  V stays key-major in LDS and its V^T fragments are
//     gathered in that same key order by transposing LDS reads
//     (ds_read_b64_tr_b16).  K and V fragments are read from LDS four MFMAs
//     ahead of their use, with the independent accumulator chains interleaved.
//   * K/V tiles are fetched with buffer loads whose range check zero-fills rows
//     past the end of the store (no per-row compares), held in registers one
//     tile ahead, and written to LDS once per workgroup: kvi8r codes become
//     fp16 by one SDWA conversion of the sign-extended byte each; V rows then
//     get one packed multiply by their scale.  K stays as exact
//     integer codes and each key's scale (times softmax_scale * log2 e) is
//     applied to that key's fp32 score, which keeps the fp16 rounding of
//     code * scale out of the scores.  The kvi8r32 store (one scale per 32
//     values, "Low VRAM, low RAM", "What is next") has four scales per key, so
//     its K is dequantised to fp16 in LDS like V.  Its score factor is then the
//     same for every key, so the rotation folds softmax_scale * log2 e into Q'
//     (one fp16 rounding, as before) and each QK chain starts its accumulators
//     at -m (the MFMA C operand): the scores come out as exponents, and the
//     softmax takes no fma.
//   * LDS: K and V both [key][dim], rows padded so fragment reads and staging
//     writes are bank-conflict free; triple-buffered in the dense kernel
//     (112 KB), one buffer in the sparse one (38 KB, four workgroups per CU).
//   * Softmax: exponents are taken against the running max already held,
//     p = exp2(score * c - m), in one fma.  Only when a row's tile sum of p
//     exceeds 2^8 (always on the first tile) does that row recompute its max,
//     rescale O and l, and redo the tile, so P never exceeds 2^8.  Row sums use
//     plain and packed-fp16 adds, not v_dot2, which shares the matrix pipeline
//     and stalls while the other wave of the SIMD issues MFMA.
//   * Every per-row decision depends only on that row's scores, so a row's
//     result is independent of q_chunk, kv_block and of which kernel variant
//     (dense, or sparse with all tiles kept) computed it.
//   * blockIdx -> (head, q-tile) is remapped so that consecutive workgroups on
//     one XCD (dispatch is round-robin over the 8 XCDs) share a head and
//     reuse its K/V tiles from that XCD's L2.
#include <type_traits>

#include "h3a_device.h"
#include "launch.h"
#include "tile_span.h"

namespace h3a {

namespace {

constexpr float kLazyBound = 256.0f;  // 2^8: largest p allowed before the max is raised
constexpr int kBufWord3 = 0x00020000;  // raw buffer resource, gfx9 data format word

template <int MODE>
struct Operand;
template <>
struct Operand<0> {  // exact store: bf16 operands
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};
template <>
struct Operand<1> {  // kvi8r store: fp16 operands
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c,
                                                 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
};
template <>
struct Operand<2> : Operand<1> {};  // kvi8r32 store (one scale per 32 values): fp16 operands

// int8 codes -> fp16.  code_pair<K> converts bytes (2K, 2K+1) of a dword, as
// signed codes, into an fp16 pair with two SDWA conversions: v_cvt_f16_i16 on
// the sign-extended byte (exact, |code| <= 128), the first writing the whole
// dword (low half), the second the high half while keeping the low.  That is
// two instructions a pair; the byte-under-exponent form (a byte permute under
// 0x64, one packed subtract of 1152, and one xor per four codes to make them
// unsigned) took 2.25, and the compiler does not form this sequence from C (it
// shifts each byte down and converts through fp32).  The first conversion
// writes a whole dword so that the second, which reads it to keep the low
// half, does not read a partial (dst_sel) write of the instruction before it.
// The asm reads and writes only the registers it names; after it the compiler
// puts one wait state before a vector instruction that reads the result (it
// cannot see that the last write was a partial one, which needs it).
template <int K>
__device__ __forceinline__ uint32_t code_pair(uint32_t w) {
  static_assert(K == 0 || K == 1, "a dword holds two byte pairs");
  uint32_t r;
  if constexpr (K == 0)
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1"
        : "=&v"(r) : "v"(w));
  else
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
        : "=&v"(r) : "v"(w));
  return r;
}

// A pair of codes times a packed scale: fp16(code * scale), rounded once.
template <int K>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t w, half2v s2) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, code_pair<K>(w)) * s2);
}

// Buffer resource over `bytes` bytes from base; loads past them read 0.  Every
// caller passes wave-uniform values; readfirstlane states that to the compiler,
// which otherwise may keep the resource in vector registers and wrap each load
// in a readfirstlane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kBufWord3);
}

// Size of the buffer resource of KV tile kt: from the tile's first row to the
// end of the store, `rows` rows of row_bytes whose last one ends after
// last_bytes, saturated at 2^32 - 1.  The row count stays in 32 bits (s_kv <
// 2^31, checked on the host) and the saturation tests the high word, held
// opaque to the optimizer (an empty asm on a scalar register) so that it stays
// a 32-bit scalar compare: folded back into a 64-bit bound, the test would take
// vector compares on every tile.  (A resource of just
// the tile's 64 rows also bounds every access, but with it the exact store's
// tiles, 64 rows spread over n_heads * 256-byte token strides, fetch about 4x
// the bytes from memory at 217088 tokens, by the FETCH_SIZE counter.)  A
// negative kt is read as tile 0, so no buffer base can precede the store.
__device__ __forceinline__ uint32_t store_span(const AttnChunk& a, int kt, uint32_t row_bytes, uint32_t last_bytes) {
  const int32_t rows = rows_to_end(a.s_kv, kt);
  if (rows <= 0) return 0u;  // an empty store: every load reads 0
  const uint64_t b = span_bytes(rows, row_bytes, last_bytes);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  asm("" : "+s"(hi));
  return hi ? 0xFFFFFFFFu : (uint32_t)b;
}

// Staging unit j of thread tid among NT threads: per key row, PER_ROW units
// (K: 8 units of 16 dims, V: 16 units of 8 dims).  Unit tid + NT*j lies in key
// row (tid + NT*j) / PER_ROW at column (tid + NT*j) % PER_ROW.  The sparse
// kernels (128 staging threads) write that as tid / PER_ROW + (NT / PER_ROW)*j
// and tid % PER_ROW, so every unit's addresses are one base plus immediate
// offsets (6 fewer vector instructions per tile, no spill); the dense kernel
// keeps the first form, which measured faster there.
template <int NT, int PER_ROW>
__device__ __forceinline__ int unit_row(int tid, int j) {
  static_assert(NT % PER_ROW == 0 && (PER_ROW & (PER_ROW - 1)) == 0, "units of a thread share a column");
  constexpr int SH = PER_ROW == 8 ? 3 : 4;
  static_assert(PER_ROW == (1 << SH), "8 or 16 units per row");
  if constexpr (NT < 256) return (tid >> SH) + (NT >> SH) * j;
  else return (tid + NT * j) >> SH;
}
template <int NT, int PER_ROW>
__device__ __forceinline__ int unit_col(int tid, int j) {
  if constexpr (NT < 256) return tid & (PER_ROW - 1);
  else return (tid + NT * j) & (PER_ROW - 1);
}

// Per-thread staging registers for one K/V tile.  K unit = one key row x 16
// dims; V unit = one key row x 8 dims.
template <int MODE, int NT>
struct Stage {
  static constexpr int KU = 512 / NT;
  static constexpr int VU = 1024 / NT;
  u32x4 k[KU][MODE == 0 ? 2 : 1];
  uint32_t ks[MODE == 2 ? KU : 1];  // kvi8r32: each unit's group scale; kvi8r: key tid's scale (threads 0-63)
  std::conditional_t<MODE == 0, u32x4, u32x2> v[VU];  // 8 bf16 values, or 8 int8 codes
  uint32_t vs[MODE == 0 ? 1 : VU];  // kvi8r: the unit's key scale; kvi8r32: the scale of its 32-value group
};

// Tile kt of one head: rows kt*64 .. kt*64+63 of the store; rows past s_kv read
// as 0 through the buffer range check.  K and V parts can be fetched separately.
template <int MODE, int NT>
__device__ __forceinline__ void load_tile_k(Stage<MODE, NT>& st, const AttnChunk& a, int head, int kt, int tid) {
  const int64_t row0 = (int64_t)tile_index_clamped(kt) * kTile;  // never a base before the store
  if constexpr (MODE == 0) {
    const int rstride = a.n_heads * kHeadDim * 2;  // bytes between tokens
    const int64_t off0 = (row0 * a.n_heads + head) * kHeadDim * 2;
    const auto rk = make_rsrc(static_cast<const char*>(a.k) + off0, store_span(a, kt, rstride, kHeadDim * 2));
#pragma unroll
    for (int j = 0; j < Stage<MODE, NT>::KU; ++j) {
      const int o = unit_row<NT, 8>(tid, j) * rstride + 32 * unit_col<NT, 8>(tid, j);
      st.k[j][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
      st.k[j][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o + 16, 0, 0));
    }
  } else {
    constexpr int G = MODE == 2 ? 4 : 1;  // scales per row
    const int64_t hrow = (int64_t)head * a.s_kv + row0;
    const auto rk = make_rsrc(static_cast<const int8_t*>(a.k) + hrow * kHeadDim, store_span(a, kt, kHeadDim, kHeadDim));
    const auto rks = make_rsrc(a.k_scale + hrow * G, store_span(a, kt, 2 * G, 2 * G));
#pragma unroll
    for (int j = 0; j < Stage<MODE, NT>::KU; ++j) {
      const int kr = unit_row<NT, 8>(tid, j), kc = unit_col<NT, 8>(tid, j);
      st.k[j][0] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, kr * kHeadDim + 16 * kc, 0, 0));
      // kvi8r32: the scale of the unit's 32-value group (dims 16*(u&7)..)
      if constexpr (MODE == 2) st.ks[j] = __builtin_amdgcn_raw_buffer_load_b16(rks, (kr * G + (kc >> 1)) * 2, 0, 0);
    }
    // One scale per key: the first wave (threads 0-63) fetches them.  The test
    // is made on a wave-uniform value so the branch is a scalar one: under an
    // exec-mask branch the compiler merges this descriptor's size with the V
    // scales' and then moves both into vector registers, and every V-scale
    // load becomes a readfirstlane loop.
    if constexpr (MODE == 1)
      if (__builtin_amdgcn_readfirstlane(tid) < kTile)
        st.ks[0] = __builtin_amdgcn_raw_buffer_load_b16(rks, tid * 2, 0, 0);
  }
}

template <int MODE, int NT>
__device__ __forceinline__ void load_tile_v(Stage<MODE, NT>& st, const AttnChunk& a, int head, int kt, int tid) {
  const int64_t row0 = (int64_t)tile_index_clamped(kt) * kTile;  // never a base before the store
  if constexpr (MODE == 0) {
    const int rstride = a.n_heads * kHeadDim * 2;
    const int64_t off0 = (row0 * a.n_heads + head) * kHeadDim * 2;
    const auto rv = make_rsrc(static_cast<const char*>(a.v) + off0, store_span(a, kt, rstride, kHeadDim * 2));
#pragma unroll
    for (int j = 0; j < Stage<MODE, NT>::VU; ++j) {
      st.v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rv, unit_row<NT, 16>(tid, j) * rstride + 16 * unit_col<NT, 16>(tid, j), 0, 0));
    }
  } else {
    constexpr int G = MODE == 2 ? 4 : 1;  // scales per row
    const int64_t hrow = (int64_t)head * a.s_kv + row0;
    const auto rv = make_rsrc(static_cast<const int8_t*>(a.v) + hrow * kHeadDim, store_span(a, kt, kHeadDim, kHeadDim));
    const auto rvs = make_rsrc(a.v_scale + hrow * G, store_span(a, kt, 2 * G, 2 * G));
    // kvi8r, 128 staging threads (the sparse kernels): each thread takes 8
    // consecutive keys at one 8-dim column, so on a whole tile one 16-byte load
    // brings its 8 V scales (8 loads before; sparse64k 0.7-1.3 % faster).  The
    // partial last tile loads them key by key, each range-checked.  The dense
    // kernel keeps one key per 16 threads and unit: there the change measured
    // no faster.
    if constexpr (MODE == 1 && NT == 128) {
      constexpr int VU = Stage<MODE, NT>::VU;
      const int r0 = VU * (tid >> 4), d8 = tid & 15;
#pragma unroll
      for (int j = 0; j < VU; ++j)
        st.v[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, (r0 + j) * kHeadDim + 8 * d8, 0, 0));
      if (rows_to_end(a.s_kv, kt) >= kTile) {  // whole tile: the 8 keys' scales in one load
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, r0 * 2, 0, 0));
        st.vs[0] = w[0]; st.vs[1] = w[1]; st.vs[2] = w[2]; st.vs[3] = w[3];
      } else {  // the partial last tile: key by key, each range-checked
#pragma unroll
        for (int j = 0; j < VU; j += 2)
          st.vs[j >> 1] = __builtin_amdgcn_raw_buffer_load_b16(rvs, (r0 + j) * 2, 0, 0) |
                          (__builtin_amdgcn_raw_buffer_load_b16(rvs, (r0 + j + 1) * 2, 0, 0) << 16);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < Stage<MODE, NT>::VU; ++j) {
      const int r = unit_row<NT, 16>(tid, j), d8 = unit_col<NT, 16>(tid, j);
      st.v[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, r * kHeadDim + 8 * d8, 0, 0));
      // kvi8r32: dims 8*d8.. lie in 32-value group d8 / 4
      st.vs[j] = __builtin_amdgcn_raw_buffer_load_b16(rvs, (r * G + (MODE == 2 ? d8 >> 2 : 0)) * 2, 0, 0);
    }
  }
}

template <int MODE, int NT>
__device__ __forceinline__ void load_tile(Stage<MODE, NT>& st, const AttnChunk& a, int head, int kt, int tid) {
  load_tile_k<MODE, NT>(st, a, head, kt, tid);
  load_tile_v<MODE, NT>(st, a, head, kt, tid);
}

// LDS layouts (16-bit elements), rows padded so that every fragment read and
// every staging write of a wave is bank-conflict free and every lane's
// addresses are one base register plus compile-time offsets:
//   K [64 keys][128 dims], row stride 136 elements (272 B): the 16 lanes of a
//     ds_read_b128 pass hit rows r..r+15 at banks 4r mod 64, disjoint;
//   V [64 keys][128 dims], row stride 160 elements (320 B): a staging write
//     of 16 lanes covers one row, all 64 banks; a transposed read
//     (ds_read_b64_tr_b16, below) of 32 lanes takes rows r..r+3 at dims
//     d0 + 16h + 4q (h = 0, 1; q = 0..3), banks 16r + 8h + 2q mod 64, disjoint.
//   kvi8r score factors: lc[key] = key scale * softmax_scale * log2(e).
constexpr int kKStride = kHeadDim + 8;   // elements
constexpr int kVStride = kHeadDim + 32;  // elements
constexpr int kKTileElems = kTile * kKStride;
constexpr int kVTileElems = kTile * kVStride;

// One staging unit of the tile held in registers, written to LDS: K unit j
// (one key x 16 dims), V unit j (one key x 8 dims), and the key factors.
template <int MODE, int NT>
__device__ __forceinline__ void store_k_unit(const Stage<MODE, NT>& st, int j, uint16_t* lk, int tid) {
  const int r = unit_row<NT, 8>(tid, j), d16 = unit_col<NT, 8>(tid, j);
  u32x4 c0, c1;
  if constexpr (MODE == 0) {
    c0 = st.k[j][0];
    c1 = st.k[j][1];
  } else if constexpr (MODE == 1) {
    const u32x4 w = st.k[j][0];
    c0 = u32x4{code_pair<0>(w[0]), code_pair<1>(w[0]), code_pair<0>(w[1]), code_pair<1>(w[1])};
    c1 = u32x4{code_pair<0>(w[2]), code_pair<1>(w[2]), code_pair<0>(w[3]), code_pair<1>(w[3])};
  } else {  // kvi8r32: a key has four scales, so K is dequantised to fp16 here like V
    const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)st.ks[j]);
    const half2v s2 = {sc, sc};
    const u32x4 w = st.k[j][0];
    c0 = u32x4{dequant_pair<0>(w[0], s2), dequant_pair<1>(w[0], s2), dequant_pair<0>(w[1], s2),
               dequant_pair<1>(w[1], s2)};
    c1 = u32x4{dequant_pair<0>(w[2], s2), dequant_pair<1>(w[2], s2), dequant_pair<0>(w[3], s2),
               dequant_pair<1>(w[3], s2)};
  }
  *reinterpret_cast<u32x4*>(lk + r * kKStride + 16 * d16) = c0;
  *reinterpret_cast<u32x4*>(lk + r * kKStride + 16 * d16 + 8) = c1;
}

template <int MODE, int NT>
__device__ __forceinline__ void store_k_factors(const Stage<MODE, NT>& st, float* lc, float sl2, int tid) {
  if constexpr (MODE == 1)  // the first wave, tested wave-uniformly as in load_tile_k
    if (__builtin_amdgcn_readfirstlane(tid) < kTile)
      lc[tid] = (float)__builtin_bit_cast(_Float16, (uint16_t)st.ks[0]) * sl2;
}

template <int MODE, int NT>
__device__ __forceinline__ void store_v_unit(const Stage<MODE, NT>& st, int j, uint16_t* lv, int tid) {
  constexpr bool kRun = MODE == 1 && NT == 128;  // 8 consecutive keys per thread, scales packed in pairs
  const int r = kRun ? Stage<MODE, NT>::VU * (tid >> 4) + j : unit_row<NT, 16>(tid, j);
  const int d8 = kRun ? (tid & 15) : unit_col<NT, 16>(tid, j);
  u32x4 c;
  if constexpr (MODE == 0) {
    c = st.v[j];
  } else {
    const uint32_t sw = kRun ? ((j & 1) ? st.vs[j >> 1] >> 16 : st.vs[j >> 1]) : st.vs[j];
    const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)sw);
    const half2v s2 = {sc, sc};
    const uint32_t w0 = st.v[j][0], w1 = st.v[j][1];
    c = u32x4{dequant_pair<0>(w0, s2), dequant_pair<1>(w0, s2), dequant_pair<0>(w1, s2), dequant_pair<1>(w1, s2)};
  }
  *reinterpret_cast<u32x4*>(lv + r * kVStride + 8 * d8) = c;
}

template <int MODE, int NT>
__device__ __forceinline__ void store_tile_k(const Stage<MODE, NT>& st, uint16_t* lk, float* lc, float sl2, int tid) {
#pragma unroll
  for (int j = 0; j < Stage<MODE, NT>::KU; ++j) store_k_unit<MODE, NT>(st, j, lk, tid);
  store_k_factors<MODE, NT>(st, lc, sl2, tid);
}

template <int MODE, int NT>
__device__ __forceinline__ void store_tile_v(const Stage<MODE, NT>& st, uint16_t* lv, int tid) {
#pragma unroll
  for (int j = 0; j < Stage<MODE, NT>::VU; ++j) store_v_unit<MODE, NT>(st, j, lv, tid);
}

template <int MODE, int NT>
__device__ __forceinline__ void store_tile(const Stage<MODE, NT>& st, uint16_t* lk, uint16_t* lv, float* lc,
                                           float sl2, int tid) {
  store_tile_k<MODE, NT>(st, lk, lc, sl2, tid);
  store_tile_v<MODE, NT>(st, lv, tid);
}

// Pseudo-key tile of the Sol residual ("H3-Optimizations" page, Nodes, routed
// geometry: a rejected tile is stood in for by its block-mean K and block-sum
// V).  Slot s < n_valid holds dropped KV tile dl[s] as one key, its tile-mean
// key divided by kmscale, with its tile-mean value; the other slots hold
// zeros.  lc[s] = kmscale * softmax_scale * log2 e and lc[kTile + s] = log2 of
// the tile's key count, so the key's weight is count * exp(scale * q . mean).
// First the slots' tile indices go to lt (-1 = empty), then every thread
// fetches its K and V pieces with buffer loads at 32-bit offsets from the
// head's tables (an empty slot's offset is past the table end and reads 0).
template <int NT>
__device__ __forceinline__ void stage_pseudo_tile(const AttnChunk& a, const SolArgs& sa, const int32_t* dl,
                                                  int n_valid, int head, int n_kt, uint16_t* lk, uint16_t* lv,
                                                  float* lc, int32_t* lt, float sl2, int tid) {
  const int64_t hbase = (int64_t)head * n_kt;
  if (tid < kTile) {
    float f = 0.0f, b = 0.0f;
    int t = -1;
    if (tid < n_valid) {
      t = dl[tid];
      const int64_t cnt = a.s_kv - (int64_t)t * kTile;
      f = sa.kmscale[hbase + t] * sl2;
      b = log2f((float)(cnt < kTile ? cnt : kTile));
    }
    lc[tid] = f;
    lc[kTile + tid] = b;
    lt[tid] = t;
  }
  __syncthreads();
  const uint32_t table = (uint32_t)n_kt * (kHeadDim * 2);  // bytes per head (< 2^32)
  const auto rk = make_rsrc(sa.kmean + hbase * kHeadDim, table);
  const auto rv = make_rsrc(sa.vmean + hbase * kHeadDim, table);
#pragma unroll
  for (int j = 0; j < 512 / NT; ++j) {  // K: unit = one slot x 16 dims
    const int r = unit_row<NT, 8>(tid, j), d16 = unit_col<NT, 8>(tid, j);
    const int t = lt[r];
    const uint32_t o = t >= 0 ? (uint32_t)t * (kHeadDim * 2) + 32 * d16 : table;
    const u32x4 c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
    const u32x4 c1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o + 16, 0, 0));
    *reinterpret_cast<u32x4*>(lk + r * kKStride + 16 * d16) = c0;
    *reinterpret_cast<u32x4*>(lk + r * kKStride + 16 * d16 + 8) = c1;
  }
#pragma unroll
  for (int j = 0; j < 1024 / NT; ++j) {  // V: unit = one slot x 8 dims
    const int r = unit_row<NT, 16>(tid, j), d8 = unit_col<NT, 16>(tid, j);
    const int t = lt[r];
    const uint32_t o = t >= 0 ? (uint32_t)t * (kHeadDim * 2) + 16 * d8 : table;
    *reinterpret_cast<u32x4*>(lv + r * kVStride + 8 * d8) =
        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
  }
}

// State of one 32-query block of a wave: its rows are lanes c = 0..31 (both
// halves g = 0, 1 of the wave hold the same query, different keys / dims).
struct RowBlock {
  u32x4 q[8];      // B operand of S^T = K Q^T: Q[row][16t + 8g .. 16t + 8g + 7]
  f32x16 acc[4];   // O^T accumulator: dims 32*db + 8*(j/4) + 4g + j%4, this lane's row
  f32x16 s[2];     // S^T of the current tile: key 32*kb + 8*(j/4) + 4g + j%4
  u32x4 pf[2][2];  // packed P of the current tile, B operand of O^T += V^T P^T
  f32x16 cneg;     // kvi8r32: -m (0 while m is -inf) in every register, where QK starts
  float m, l;      // running max (log2 units) and row sum of this lane's keys
  int64_t row;
  bool valid;
};

// Scores that start from -m: kvi8r32, except on pseudo-key tiles.
template <int MODE, bool PSEUDO = false>
constexpr bool kBiasedScores = MODE == 2 && !PSEUDO;

// lk points at this lane's K row c, dims 8g.. of the current buffer.  The two
// 32-key chains are interleaved.  CN: the chains start at rb.cneg.
template <int MODE, bool CN = kBiasedScores<MODE>>
__device__ __forceinline__ void qk_issue(RowBlock& rb, const uint16_t* lk) {
  using Op = Operand<MODE>;
  u32x4 ka[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) ka[i] = *reinterpret_cast<const u32x4*>(lk + 32 * (i & 1) * kKStride + 16 * (i >> 1));
  f32x16 s0 = CN ? rb.cneg : f32x16{}, s1 = CN ? rb.cneg : f32x16{};
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    s0 = Op::mfma(ka[i], rb.q[i >> 1], s0);
    s1 = Op::mfma(ka[i + 1], rb.q[i >> 1], s1);
  }
  rb.s[0] = s0;
  rb.s[1] = s1;
}

// Issue order of 16 MFMAs and the LDS fragment reads feeding them: each read
// runs kAhead MFMAs ahead of its use (RD reads per MFMA).
template <int RD>
__device__ __forceinline__ void mfma_read_pattern() {
  constexpr int kAhead = 4;
  __builtin_amdgcn_sched_group_barrier(0x100, RD * kAhead, 0);
#pragma unroll
  for (int i = 0; i < 16 - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
}

template <int MODE, bool CN = kBiasedScores<MODE>>
__device__ __forceinline__ void qk_block(RowBlock& rb, const uint16_t* lk) {
  qk_issue<MODE, CN>(rb, lk);
  mfma_read_pattern<1>();
}

// QK(i) of one wave with the staging of the next tile written among its MFMAs
// (one scheduling region; in the source one staging unit follows every second
// MFMA, so the LDS writes are not held behind all of the fragment reads).  The
// kvi8r dense kernel uses it: 1.3 % faster than QK then staging as two
// regions; the exact store measured 1 % slower with it and keeps two regions.
template <int MODE, int NT>
__device__ __forceinline__ void qk_stage(RowBlock& rb, const uint16_t* lk, const Stage<MODE, NT>& st, uint16_t* wk,
                                         uint16_t* wv, float* wc, float sl2, int tid) {
  using Op = Operand<MODE>;
  constexpr int KU = Stage<MODE, NT>::KU, NU = KU + Stage<MODE, NT>::VU;
  auto kfrag = [&](int i) { return *reinterpret_cast<const u32x4*>(lk + 32 * (i & 1) * kKStride + 16 * (i >> 1)); };
  u32x4 ka[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) ka[i] = kfrag(i);
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + 4 < 16) ka[i + 4] = kfrag(i + 4);
    if (i & 1)
      s1 = Op::mfma(ka[i], rb.q[i >> 1], s1);
    else
      s0 = Op::mfma(ka[i], rb.q[i >> 1], s0);
    if (i & 1) {
      const int u = i >> 1;
      if (u < KU)
        store_k_unit<MODE, NT>(st, u, wk, tid);
      else if (u < NU)
        store_v_unit<MODE, NT>(st, u - KU, wv, tid);
      else if (u == NU)
        store_k_factors<MODE, NT>(st, wc, sl2, tid);
    }
  }
  rb.s[0] = s0;
  rb.s[1] = s1;
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j receives element j % 4 of the 8-byte blocks addressed by lanes
// 4k + j / 4, k = 0..3.  When lane i of the group addresses V row r0 + i / 4
// at dims d0 + 4 (i % 4), lane j receives V[r0 + k][d0 + j], k = 0..3: four
// keys of one dim, a column of V, as the A operand of O^T += V^T P^T needs.
__device__ __forceinline__ u32x2 read_v_column(const uint16_t* p) {
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v lds_short4v;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p)));
}

// This lane's address for read_v_column in a V buffer: row 4g + i / 4 and dims
// 16h + 4 (i % 4), i = lane % 16, h = (lane / 16) % 2, so that the lane receives
// dim 32 db + c (c = lane % 32) of keys 4g .. 4g + 3 past the row offset.
__device__ __forceinline__ int v_lane_offset(int lane) {
  const int i = lane & 15, h = (lane >> 4) & 1, g = lane >> 5;
  return (4 * g + (i >> 2)) * kVStride + 16 * h + 4 * (i & 3);
}

// O^T += V^T P^T.  k-step j covers keys 32*(j/2) + 16*(j%2) + 4g + {0..3} and
// the same + 8, matching the order of the S^T accumulator registers in pf.
// lv points at this lane's v_lane_offset in the current V buffer.
template <int MODE>
__device__ __forceinline__ void pv_issue(RowBlock& rb, const uint16_t* lv) {
  using Op = Operand<MODE>;
  u32x4 va[16];  // k-step major, so the four accumulator chains interleave
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = i >> 2, db = i & 3;
    const uint16_t* p = lv + (32 * (j >> 1) + 16 * (j & 1)) * kVStride + 32 * db;
    const u32x2 lo = read_v_column(p);
    const u32x2 hi = read_v_column(p + 8 * kVStride);
    va[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = i >> 2, db = i & 3;
    rb.acc[db] = Op::mfma(va[i], rb.pf[j >> 1][j & 1], rb.acc[db]);
  }
}

template <int MODE>
__device__ __forceinline__ void pv_block(RowBlock& rb, const uint16_t* lv) {
  pv_issue<MODE>(rb, lv);
  mfma_read_pattern<2>();
}

// Score factors of this lane's keys 32*kb + 8*jg + 4g + {0..3}: key scale *
// softmax_scale * log2 e (kvi8r, from LDS) or softmax_scale * log2 e (exact;
// kvi8r32, whose K is dequantised in LDS and whose Q' already carries the
// factor, takes 1).
// Pseudo-key tiles (Sol residual) take theirs from LDS in both modes, and also
// a per-key additive term, log2 of the key's multiplicity, from lc + kTile.
template <int MODE, bool PSEUDO = false>
__device__ __forceinline__ u32x4 score_factors(const float* lc, float sl2, int kb, int jg, int g) {
  if constexpr (MODE == 1 || PSEUDO) return *reinterpret_cast<const u32x4*>(lc + 32 * kb + 8 * jg + 4 * g);
  const uint32_t f = __float_as_uint(sl2);
  return u32x4{f, f, f, f};
}
__device__ __forceinline__ u32x4 score_bias(const float* lc, int kb, int jg, int g) {
  return *reinterpret_cast<const u32x4*>(lc + kTile + 32 * kb + 8 * jg + 4 * g);
}

// p = exp2(s * factor - m) for this lane's 32 keys, packed into pf; returns the
// sum of this lane's p in a fixed order.  kvi8r sums the fp16-rounded P with
// packed fp16 adds (pairs, then a tree); exact sums the fp32 p in a tree.  Row
// sums avoid v_dot2: it runs on the matrix pipeline and stalls next to MFMA.
// PSEUDO adds each key's log2 multiplicity to its exponent.
// The exponents, the exponentials and the packing are written as three passes.
// For the exact store they are also three scheduling regions (all 32 fma, then
// all 32 exp, then packs and sums), which measured ~1 % faster; in the kvi8r
// modes the compiler interleaves them, which measured faster there.
// Biased scores (kvi8r32) already are s * factor - m for the m the QK started
// from: p = exp2(s), or exp2(s + nm) with nm the change of m when ADD.
template <int MODE, bool PARTIAL, bool PSEUDO = false, bool ADD = false>
__device__ __forceinline__ float tile_exps(RowBlock& rb, const float* lc, float sl2, float nm, int n_valid, int g) {
  using Op = Operand<MODE>;
  constexpr bool kBiased = kBiasedScores<MODE, PSEUDO>;
  constexpr bool kPhased = MODE == 0;
  float x[32];  // x[16 kb + 4 jg + e]: key 32 kb + 8 jg + 4 g + e
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const u32x4 cc = score_factors<MODE, PSEUDO>(lc, sl2, kb, jg, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t;
        if constexpr (kBiased) t = ADD ? rb.s[kb][4 * jg + e] + nm : rb.s[kb][4 * jg + e];
        else t = __builtin_fmaf(rb.s[kb][4 * jg + e], __uint_as_float(cc[e]), nm);
        if constexpr (PSEUDO) t += __uint_as_float(score_bias(lc, kb, jg, g)[e]);
        if constexpr (PARTIAL) t = 32 * kb + 8 * jg + 4 * g + e < n_valid ? t : -__builtin_inff();
        x[16 * kb + 4 * jg + e] = t;
      }
    }
  if constexpr (kPhased) __builtin_amdgcn_sched_barrier(0);
  float p[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) p[i] = __builtin_amdgcn_exp2f(x[i]);
  if constexpr (kPhased) __builtin_amdgcn_sched_barrier(0);
  float gs[8];     // exact: sum of each group of 4
  half2v hs[8];    // kvi8r: packed sum of each group of 4
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const float* q = p + 16 * kb + 4 * jg;
      const uint32_t q01 = Op::pack(q[0], q[1]), q23 = Op::pack(q[2], q[3]);
      if constexpr (MODE != 0)
        hs[4 * kb + jg] = __builtin_bit_cast(half2v, q01) + __builtin_bit_cast(half2v, q23);
      else
        gs[4 * kb + jg] = (q[0] + q[1]) + (q[2] + q[3]);
      rb.pf[kb][jg >> 1][2 * (jg & 1)] = q01;
      rb.pf[kb][jg >> 1][2 * (jg & 1) + 1] = q23;
    }
  if constexpr (MODE != 0) {
    const half2v h = ((hs[0] + hs[1]) + (hs[2] + hs[3])) + ((hs[4] + hs[5]) + (hs[6] + hs[7]));
    return (float)h[0] + (float)h[1];
  } else {
    return ((gs[0] + gs[1]) + (gs[2] + gs[3])) + ((gs[4] + gs[5]) + (gs[6] + gs[7]));
  }
}

template <int MODE, bool PARTIAL, bool PSEUDO = false>
__device__ __forceinline__ float softmax_fast(RowBlock& rb, const float* lc, float sl2, int n_valid, int g) {
  return tile_exps<MODE, PARTIAL, PSEUDO>(rb, lc, sl2, -rb.m, n_valid, g);
}

template <int MODE, bool PARTIAL, bool PSEUDO = false>
__device__ __forceinline__ void softmax_finish(RowBlock& rb, float lsum, const float* lc, float sl2, int n_valid,
                                               int g) {
  constexpr bool kBiased = kBiasedScores<MODE, PSEUDO>;
  bool redo = !(pair_max(lsum) <= kLazyBound);
  // Biased scores start from 0 while m is -inf, so the first tile is redone
  // by this test rather than by an infinite sum.
  if constexpr (kBiased) redo = redo || rb.m == -__builtin_inff();
  if (redo) {
    const float mb = rb.m == -__builtin_inff() ? 0.0f : rb.m;  // the m the biased scores hold
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const u32x4 cc = score_factors<MODE, PSEUDO>(lc, sl2, kb, jg, g);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!PARTIAL || 32 * kb + 8 * jg + 4 * g + e < n_valid) {
            float x = kBiased ? rb.s[kb][4 * jg + e] : rb.s[kb][4 * jg + e] * __uint_as_float(cc[e]);
            if constexpr (PSEUDO) x += __uint_as_float(score_bias(lc, kb, jg, g)[e]);
            mx = fmaxf(mx, x);
          }
      }
    mx = pair_max(mx);
    if constexpr (kBiased) mx += mb;
    const float alpha = __builtin_amdgcn_exp2f(rb.m - mx);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb.acc[i] *= alpha;
    rb.l *= alpha;
    rb.m = mx;
    if constexpr (MODE == 2)
#pragma unroll
      for (int i = 0; i < 16; ++i) rb.cneg[i] = -mx;
    if constexpr (kBiased) lsum = tile_exps<MODE, PARTIAL, PSEUDO, true>(rb, lc, sl2, mb - mx, n_valid, g);
    else lsum = tile_exps<MODE, PARTIAL, PSEUDO>(rb, lc, sl2, -rb.m, n_valid, g);
  }
  rb.l += lsum;
}

// Online softmax of one tile.  Exponentials are taken against the running max
// already held (one fma each).  Only when the row's tile sum of p exceeds 2^8
// (so that no p can exceed 2^8 otherwise; always true on the first tile, where
// the running max is -inf) does the row take the tile max as its new running
// max, rescale O and l, and redo the tile.  A sum above 2^8 implies some p
// above 2^3, so the new max is always above the old one.
template <int MODE, bool PARTIAL, bool PSEUDO = false>
__device__ __forceinline__ void softmax_block(RowBlock& rb, const float* lc, float sl2, int n_valid, int g) {
  softmax_finish<MODE, PARTIAL, PSEUDO>(rb, softmax_fast<MODE, PARTIAL, PSEUDO>(rb, lc, sl2, n_valid, g), lc, sl2,
                                        n_valid, g);
}

// Normalise and store this lane's 64 dims of its query row.
template <int MODE>
__device__ __forceinline__ void store_rows(const RowBlock& rb, const AttnChunk& a, int head, int g) {
  const float lt = pair_sum(rb.l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (!rb.valid) return;
  const int64_t base = (rb.row * a.n_heads + head) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * db + 8 * rg + 4 * g;  // accumulator registers 4rg..4rg+3 = dims d0..d0+3
      const float o0 = rb.acc[db][4 * rg] * inv, o1 = rb.acc[db][4 * rg + 1] * inv;
      const float o2 = rb.acc[db][4 * rg + 2] * inv, o3 = rb.acc[db][4 * rg + 3] * inv;
      if constexpr (MODE == 0) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + base + d0) =
            u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      } else {
        *reinterpret_cast<u32x4*>(static_cast<float*>(a.out) + base + d0) =
            u32x4{__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2), __float_as_uint(o3)};
      }
    }
}

// Block-sparse kernel: one workgroup = 2 waves x 32 rows = one 64-row routing
// q-tile of one head, iterating only the KV tiles its mask row keeps, in
// increasing order.  A single LDS buffer (38 KB) and at most 256 registers per
// wave let four workgroups share a CU, two waves per SIMD, so one workgroup's
// staging and softmax run under another's matrix-core work.  Per kept tile:
//     stage(i) [barrier] fetch(i+1), QK(i), softmax(i), PV(i) [barrier]
// Each row's arithmetic is that of the dense kernel.  With SOL, the dropped
// tiles then follow as pseudo-keys, 64 per pass (stage_pseudo_tile).
// lds_k, lds_v: one K and one V tile; lds_c: score factors, with SOL followed
// by the pseudo slots' biases and tile indices.
template <int MODE, bool SOL>
__device__ __forceinline__ void attn_fwd_sparse_body(const AttnChunk& a, int32_t n_qt, int32_t n_kt,
                                                     const SolArgs& sa, uint16_t* lds_k, uint16_t* lds_v,
                                                     float* lds_c) {
  constexpr int NT = 128;
  constexpr int BM = 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, g = lane >> 5;

  // XCD-aware remap: physical block b runs on XCD b % 8; give each XCD a
  // contiguous range of (head-major) logical tiles.
  int b = blockIdx.x;
  const int per = (int)gridDim.x >> 3;
  if (b < per * 8) b = (b & 7) * per + (b >> 3);
  const int head = b / n_qt;
  const int qt = b - head * n_qt;

  RowBlock rb;
  rb.row = (int64_t)qt * BM + wave * 32 + c;
  rb.valid = rb.row < a.rows;
  {
    const uint16_t* qp = a.q + ((rb.valid ? rb.row : 0) * a.n_heads + head) * kHeadDim + 8 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      rb.q[t] = rb.valid ? *reinterpret_cast<const u32x4*>(qp + 16 * t) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) rb.acc[i] = f32x16{};
  rb.m = -__builtin_inff();
  rb.cneg = f32x16{};
  rb.l = 0.0f;

  const int n_tiles = a.counts[head * n_qt + qt];
  const int32_t* list = a.lists + ((int64_t)head * n_qt + qt) * n_kt;
  const float sl2 = MODE == 2 ? 1.0f : a.scale_log2;  // kvi8r32: Q' carries it
  const int last_full = (int)(a.s_kv / kTile);  // tiles with index >= this one are partial
  const uint16_t* lk = lds_k + c * kKStride + 8 * g;
  const uint16_t* lv = lds_v + v_lane_offset(lane);

  // Kept-tile indices are the same in every lane: readfirstlane keeps the
  // buffer descriptors built from them in scalar registers.
  Stage<MODE, NT> st;
  if (n_tiles > 0) load_tile<MODE, NT>(st, a, head, __builtin_amdgcn_readfirstlane(list[0]), tid);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the first tile are in registers on every path

  // Only the last kept tile can be partial (lists are increasing): full tiles
  // run the loop without key masking, a partial one runs after it.
  const bool tail = n_tiles > 0 && __builtin_amdgcn_readfirstlane(list[n_tiles - 1]) >= last_full;
  const int n_main = n_tiles - (tail ? 1 : 0);
  // Iteration i fetches tile i+1 (past the end: tile i again, never staged).
  // kvi8r modes read that index one iteration earlier, so the read has long
  // completed when it is used (its wait falls where the previous tile's data
  // is needed anyway).  The exact mode reads it in place: its staging
  // registers leave no room to carry the index across the iteration.
  int nxt_idx = MODE != 0 && n_tiles > 0 ? list[n_tiles > 1 ? 1 : 0] : 0;
  for (int i = 0; i < n_main; ++i) {
    store_tile<MODE, NT>(st, lds_k, lds_v, lds_c, sl2, tid);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    int nxt;
    if constexpr (MODE == 0) {
      nxt = list[i + 1 < n_tiles ? i + 1 : i];
    } else {
      nxt = __builtin_amdgcn_readfirstlane(nxt_idx);
      nxt_idx = list[i + 2 < n_tiles ? i + 2 : n_tiles - 1];
    }
    load_tile_v<MODE, NT>(st, a, head, nxt, tid);
    __builtin_amdgcn_sched_barrier(0);
    qk_block<MODE>(rb, lk);
    __builtin_amdgcn_sched_barrier(0);
    softmax_block<MODE, false>(rb, lds_c, sl2, kTile, g);
    __builtin_amdgcn_sched_barrier(0);
    load_tile_k<MODE, NT>(st, a, head, nxt, tid);  // K registers stay free through QK and softmax
    __builtin_amdgcn_sched_barrier(0);
    pv_block<MODE>(rb, lv);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }
  if (tail) {
    store_tile<MODE, NT>(st, lds_k, lds_v, lds_c, sl2, tid);
    __syncthreads();
    const int n_valid = (int)(a.s_kv - (int64_t)__builtin_amdgcn_readfirstlane(list[n_main]) * kTile);
    qk_block<MODE>(rb, lk);
    softmax_block<MODE, true>(rb, lds_c, sl2, n_valid, g);
    pv_block<MODE>(rb, lv);
  }
  if constexpr (SOL) {
    const int n_drop = n_kt - n_tiles;
    const int32_t* dl = sa.drops + ((int64_t)head * n_qt + qt) * n_kt;
    for (int p0 = 0; p0 < n_drop; p0 += kTile) {
      __syncthreads();  // both waves are done with the tile in LDS
      const int nv = n_drop - p0 < kTile ? n_drop - p0 : kTile;
      stage_pseudo_tile<NT>(a, sa, dl + p0, nv, head, n_kt, lds_k, lds_v, lds_c,
                            reinterpret_cast<int32_t*>(lds_c + 2 * kTile), sl2, tid);
      __syncthreads();
      qk_block<MODE, false>(rb, lk);
      softmax_block<MODE, true, true>(rb, lds_c, sl2, nv, g);
      pv_block<MODE>(rb, lv);
    }
  }
  store_rows<MODE>(rb, a, head, g);
}

template <int MODE>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_sparse_kernel(AttnChunk a, int32_t n_qt, int32_t n_kt) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kKTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kVTileElems];
  __shared__ __attribute__((aligned(16))) float lds_c[kTile];
  attn_fwd_sparse_body<MODE, false>(a, n_qt, n_kt, SolArgs{}, lds_k, lds_v, lds_c);
}

// Block-sparse kernel, paired form: one workgroup = 8 waves = two 64-row routing
// q-tiles (2j and 2j+1) of one head.  Waves 0-1 attend q-tile 2j's rows and
// waves 2-3 q-tile 2j+1's; waves 4-5 stage q-tile 2j's kept tiles and 6-7 those
// of 2j+1.  Wave w runs on SIMD w % 4, so each SIMD holds one attending and one
// staging wave, and the staging runs beside the attending wave's matrix-core
// work instead of in its chain.  Each q-tile has two LDS slots: in period p its
// attending waves take tile p of its list from slot p % 2 while its staging
// waves write tile p+1 into the other slot and fetch tile p+2.  One barrier per
// period; a q-tile whose list is shorter idles for the remaining periods.
// Each row's arithmetic is that of attn_fwd_sparse_kernel.  Launched for the
// exact store, where it is ~20 % faster than the one-q-tile kernel; for the
// kvi8r stores, whose staging is dominated by code conversions, it is ~4 %
// slower (the vector work per SIMD is the same, and there it sets the pace).
template <int MODE>
__global__ __launch_bounds__(512) void attn_fwd_sparse_pair_kernel(AttnChunk a, int32_t n_qt, int32_t n_kt) {
  constexpr int NT = 128;
  constexpr int BM = 64;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][2][kKTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][2][kVTileElems];
  __shared__ __attribute__((aligned(16))) float lds_c[2][2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int x = (wave >> 1) & 1;  // which q-tile of the pair
  const bool stager = wave >= 4;

  const int n_pairs = (n_qt + 1) >> 1;
  int b = blockIdx.x;
  const int per = (int)gridDim.x >> 3;
  if (b < per * 8) b = (b & 7) * per + (b >> 3);
  const int head = b / n_pairs;
  const int qt0 = 2 * (b - head * n_pairs);
  const int qt = qt0 + x;
  const int32_t* cnt = a.counts + (int64_t)head * n_qt;
  const int n0 = cnt[qt0];
  const int n1 = qt0 + 1 < n_qt ? cnt[qt0 + 1] : 0;
  const int n_tiles = x == 0 ? n0 : n1;
  const int n_per = n0 > n1 ? n0 : n1;
  const int32_t* list = a.lists + ((int64_t)head * n_qt + (qt < n_qt ? qt : qt0)) * n_kt;
  const float sl2 = MODE == 2 ? 1.0f : a.scale_log2;  // kvi8r32: Q' carries it

  if (stager) {
    const int stid = tid - 256 - 128 * x;
    Stage<MODE, NT> st;
    if (n_tiles > 0) {
      load_tile<MODE, NT>(st, a, head, __builtin_amdgcn_readfirstlane(list[0]), stid);
      store_tile<MODE, NT>(st, lds_k[x][0], lds_v[x][0], lds_c[x][0], sl2, stid);
    }
    if (n_tiles > 1) load_tile<MODE, NT>(st, a, head, __builtin_amdgcn_readfirstlane(list[1]), stid);
    int nxt = n_tiles > 2 ? list[2] : 0;  // read one period ahead of its use
    __syncthreads();
    for (int p = 0; p < n_per; ++p) {
      const int sl = (p + 1) & 1;
      if (p + 1 < n_tiles) store_tile<MODE, NT>(st, lds_k[x][sl], lds_v[x][sl], lds_c[x][sl], sl2, stid);
      if (p + 2 < n_tiles) {
        const int kt = __builtin_amdgcn_readfirstlane(nxt);
        if (p + 3 < n_tiles) nxt = list[p + 3];
        load_tile<MODE, NT>(st, a, head, kt, stid);
      }
      __syncthreads();
    }
  } else {
    RowBlock rb;
    rb.row = (int64_t)qt * BM + (wave & 1) * 32 + c;
    rb.valid = qt < n_qt && rb.row < a.rows;
    {
      const uint16_t* qp = a.q + ((rb.valid ? rb.row : 0) * a.n_heads + head) * kHeadDim + 8 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        rb.q[t] = rb.valid ? *reinterpret_cast<const u32x4*>(qp + 16 * t) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) rb.acc[i] = f32x16{};
    rb.m = -__builtin_inff();
    rb.cneg = f32x16{};
    rb.l = 0.0f;
    // Only the last kept tile can be partial (lists are increasing): full
    // tiles run in the loop, a partial one after it, then idle periods up to
    // the longer list of the pair.
    const int last_full = (int)(a.s_kv / kTile);  // tiles with index >= this one are partial
    const bool tail = n_tiles > 0 && __builtin_amdgcn_readfirstlane(list[n_tiles - 1]) >= last_full;
    const int n_full = n_tiles - (tail ? 1 : 0);
    __syncthreads();
    int p = 0;
    for (; p < n_full; ++p) {
      const int sl = p & 1;
      const uint16_t* lk = lds_k[x][sl] + c * kKStride + 8 * g;
      const uint16_t* lv = lds_v[x][sl] + v_lane_offset(lane);
      qk_block<MODE>(rb, lk);
      __builtin_amdgcn_sched_barrier(0);
      softmax_block<MODE, false>(rb, lds_c[x][sl], sl2, kTile, g);
      __builtin_amdgcn_sched_barrier(0);
      pv_block<MODE>(rb, lv);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
    if (tail) {
      const int sl = p & 1;
      const int kt = __builtin_amdgcn_readfirstlane(list[p]);
      qk_block<MODE>(rb, lds_k[x][sl] + c * kKStride + 8 * g);
      softmax_block<MODE, true>(rb, lds_c[x][sl], sl2, (int)(a.s_kv - (int64_t)kt * kTile), g);
      pv_block<MODE>(rb, lds_v[x][sl] + v_lane_offset(lane));
      __syncthreads();
      ++p;
    }
    for (; p < n_per; ++p) __syncthreads();
    store_rows<MODE>(rb, a, head, g);
  }
}

// The same with the Sol residual: dropped tiles enter as pseudo-keys.
template <int MODE>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_sparse_sol_kernel(AttnChunk a, int32_t n_qt, int32_t n_kt, SolArgs sa) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kKTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kVTileElems];
  __shared__ __attribute__((aligned(16))) float lds_c[3 * kTile];
  attn_fwd_sparse_body<MODE, true>(a, n_qt, n_kt, sa, lds_k, lds_v, lds_c);
}

// Dense kernel: 8 waves x 32 query rows = 256 rows of one head, two waves per
// SIMD, software-pipelined across the two waves of each SIMD ("ping-pong").
// Group 0 (waves 0-3) and group 1 (waves 4-7) hold one wave on every SIMD
// each.  Between two barriers (one period) group 0 runs
//     QK(i), stage(i+1), softmax(i), PV(i) + fetch(i+2), [barrier]
// and group 1 runs
//     softmax(i-1), PV(i-1), QK(i), [barrier]
// so each matrix-core phase of one wave meets a vector phase of the other wave
// on the same SIMD.  Group 0 alone fetches and stages the K/V tiles (it has
// the shorter chain of dependent work), so group 1 starts its softmax right
// after the barrier.  The fetch of tile i+2 is issued among the PV MFMAs: a
// wave issuing a burst of buffer loads stalls while the CU's address unit
// works through them, and between MFMAs that wait costs nothing.  Tiles are
// triple-buffered in LDS: during period i tiles i-1 and i are read while tile
// i+1 is written.
// STATE: the K/V is one block of a longer store ("H3 Streamed Blocks" node
// page, kv_block row: K/V attended block by block with a log-sum-exp combine).
// Each thread resumes its rows' running max, row sum and O accumulators from
// a.state_in (unless null) and leaves them in a.state_out (unless null, in
// which case it writes the normalised output).  The layout is one array per
// register, indexed by the thread's position in the grid, so the state moves
// in coalesced 256-byte runs.  Carrying it through memory is exact, so a store
// attended block by block gives the bits of one pass over the whole store.
template <int MODE, bool STATE = false>
__global__ __launch_bounds__(512) void attn_fwd_dense_kernel(AttnChunk a, int32_t n_qt, int32_t n_kt) {
  constexpr int NS = 256;  // staging threads (group 0)
  constexpr int BM = 256;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[3][kKTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[3][kVTileElems];
  __shared__ __attribute__((aligned(16))) float lds_c[3][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const bool late = wave >= 4;  // group 1: runs each tile half a period behind

  int b = blockIdx.x;
  const int per = (int)gridDim.x >> 3;
  if (b < per * 8) b = (b & 7) * per + (b >> 3);
  const int head = b / n_qt;
  const int qt = b - head * n_qt;

  RowBlock rb;
  rb.row = (int64_t)qt * BM + wave * 32 + c;
  rb.valid = rb.row < a.rows;
  {
    const uint16_t* qp = a.q + ((rb.valid ? rb.row : 0) * a.n_heads + head) * kHeadDim + 8 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      rb.q[t] = rb.valid ? *reinterpret_cast<const u32x4*>(qp + 16 * t) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) rb.acc[i] = f32x16{};
  rb.m = -__builtin_inff();
  rb.cneg = f32x16{};
  rb.l = 0.0f;
  const int64_t state_stride = (int64_t)gridDim.x * 512;      // one array per state register
  const int64_t state_at = (int64_t)b * 512 + tid;             // this thread's slot (logical block b)
  if constexpr (STATE) {
    if (a.state_in != nullptr) {
      const float* sp = a.state_in + state_at;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) rb.acc[i][j] = sp[(16 * i + j) * state_stride];
      rb.m = sp[64 * state_stride];
      rb.l = sp[65 * state_stride];
      if (MODE == 2 && rb.m != -__builtin_inff())
#pragma unroll
        for (int i = 0; i < 16; ++i) rb.cneg[i] = -rb.m;
    }
  }

  const int n = n_kt;
  const float sl2 = MODE == 2 ? 1.0f : a.scale_log2;  // kvi8r32: Q' carries it
  const bool tail = n > 0 && (int64_t)n * kTile > a.s_kv;  // the last tile is partial
  const int n_valid_last = n > 0 ? (int)(a.s_kv - (int64_t)(n - 1) * kTile) : 0;
  // Buffer b of tile t is t % 3; callers pass b, kept in scalar registers.
  auto lk = [&](int b) { return lds_k[b] + c * kKStride + 8 * g; };
  auto lv = [&](int b) { return lds_v[b] + v_lane_offset(lane); };
  auto lc = [&](int b) -> const float* { return lds_c[b]; };
  auto next3 = [](int b) { return __builtin_amdgcn_readfirstlane(b == 2 ? 0 : b + 1); };
  auto sm_full = [&](int b) { softmax_block<MODE, false>(rb, lc(b), sl2, kTile, g); };
  auto sm_last = [&](int b) {
    if (tail)
      softmax_block<MODE, true>(rb, lc(b), sl2, n_valid_last, g);
    else
      softmax_block<MODE, false>(rb, lc(b), sl2, kTile, g);
  };

  if (!late) {
    Stage<MODE, NS> st;
    auto stage = [&](int b) {  // write the tile held in registers to buffer b
      store_tile<MODE, NS>(st, lds_k[b], lds_v[b], lds_c[b], sl2, tid);
    };
    if (n > 0) {
      load_tile<MODE, NS>(st, a, head, 0, tid);
      stage(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and tile 0 are in registers on every path
    if (n > 1) load_tile<MODE, NS>(st, a, head, 1, tid);
    __syncthreads();
    int bi = 0;  // buffer of tile i
    for (int i = 0; i + 1 < n; ++i) {  // periods 0 .. n-2
      const int bn = next3(bi);
      const int nx = i + 2 < n ? i + 2 : n - 1;  // tile i+2; past the end, the last tile again (never staged)
      if constexpr (MODE == 1) {
        qk_stage<MODE, NS>(rb, lk(bi), st, lds_k[bn], lds_v[bn], lds_c[bn], sl2, tid);
      } else {
        qk_block<MODE>(rb, lk(bi));
        __builtin_amdgcn_sched_barrier(0);
        stage(bn);
      }
      __builtin_amdgcn_sched_barrier(0);
      sm_full(bi);
      __builtin_amdgcn_sched_barrier(0);
      load_tile<MODE, NS>(st, a, head, nx, tid);
      pv_block<MODE>(rb, lv(bi));
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      bi = bn;
    }
    if (n > 0) {  // period n-1
      qk_block<MODE>(rb, lk(bi));
      __builtin_amdgcn_sched_barrier(0);
      sm_last(bi);
      __builtin_amdgcn_sched_barrier(0);
      pv_block<MODE>(rb, lv(bi));
      __syncthreads();
    }
    __syncthreads();  // period n: group 1 finishes tile n-1
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q is in registers
    __syncthreads();
    if (n > 0) {  // period 0
      qk_block<MODE>(rb, lk(0));
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
    int bp = 0;  // buffer of tile i-1
    for (int i = 1; i < n; ++i) {  // periods 1 .. n-1
      const int bi = next3(bp);
      sm_full(bp);
      __builtin_amdgcn_sched_barrier(0);
      pv_block<MODE>(rb, lv(bp));
      __builtin_amdgcn_sched_barrier(0);
      qk_block<MODE>(rb, lk(bi));
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      bp = bi;
    }
    if (n > 0) {  // period n
      sm_last(bp);
      __builtin_amdgcn_sched_barrier(0);
      pv_block<MODE>(rb, lv(bp));
    }
    __syncthreads();
  }
  if constexpr (STATE) {
    if (a.state_out != nullptr) {
      float* sp = a.state_out + state_at;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) sp[(16 * i + j) * state_stride] = rb.acc[i][j];
      sp[64 * state_stride] = rb.m;
      sp[65 * state_stride] = rb.l;
      return;
    }
  }
  store_rows<MODE>(rb, a, head, g);
}

// Kept-tile list of one (head, q-tile) row of the mask, in increasing key
// order; with drops, also the list of the dropped tiles, in increasing order.
__global__ __launch_bounds__(256) void route_build_kernel(const uint8_t* __restrict__ mask, int64_t n_qt_total,
                                                          int64_t qt0, int32_t n_qt, int32_t n_kt,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ lists,
                                                          int32_t* __restrict__ drops) {
  __shared__ int part[256];
  const int qt = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const uint8_t* row = mask + ((int64_t)head * n_qt_total + qt0 + qt) * n_kt;
  const int seg = (n_kt + 255) / 256;
  const int b0 = min(tid * seg, n_kt), b1 = min(b0 + seg, n_kt);
  int cnt = 0;
  for (int j = b0; j < b1; ++j) cnt += row[j] != 0;
  part[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive scan
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int pos = part[tid] - cnt;
  int32_t* out = lists + ((int64_t)head * n_qt + qt) * n_kt;
  for (int j = b0; j < b1; ++j)
    if (row[j]) out[pos++] = j;
  if (drops != nullptr) {
    int dpos = b0 - (part[tid] - cnt);  // tiles before b0 that are dropped
    int32_t* dout = drops + ((int64_t)head * n_qt + qt) * n_kt;
    for (int j = b0; j < b1; ++j)
      if (!row[j]) dout[dpos++] = j;
  }
  if (tid == 255) counts[head * n_qt + qt] = part[255];
}

// Tile means for the Sol residual: one workgroup per (KV tile, head).  Threads
// 0-127 sum the tile's keys and 128-255 its values, in fp32 over the
// dequantised store (a kvi8r code times its fp16 scale is exact in fp32): each
// thread takes 4 consecutive dimensions of every 4th row (4 row groups), and
// the 4 partial sums of a dimension are added in a fixed order through LDS.
// The mean value is rounded to the matrix-core type.  The mean key is first
// divided by a power of two 2^e chosen so that its largest magnitude lies in
// [64, 128) -- an exact step -- then rounded, which keeps fp16 from
// overflowing on large keys; 2^e goes to kmscale.
template <int MODE>
__global__ __launch_bounds__(256) void tile_means_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                         const uint16_t* __restrict__ k_scale,
                                                         const uint16_t* __restrict__ v_scale, int64_t s_kv,
                                                         int32_t n_heads, uint16_t* __restrict__ kmean,
                                                         uint16_t* __restrict__ vmean, float* __restrict__ kmscale) {
  __shared__ float part[2][4][kHeadDim];  // [K|V][row group][dim]
  __shared__ float wmax[2];
  const int t = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const int n_kt = (int)gridDim.x;
  const int side = tid >> 7;              // 0 = K, 1 = V
  const int rg = (tid >> 5) & 3, d4 = 4 * (tid & 31);
  const int64_t r0 = (int64_t)t * kTile;
  const int n = (int)(s_kv - r0 < kTile ? s_kv - r0 : kTile);  // >= 1
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (MODE == 0) {
    const uint16_t* src = static_cast<const uint16_t*>(side ? v : k) + (r0 * n_heads + head) * kHeadDim + d4;
    for (int r = rg; r < n; r += 4) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(src + (int64_t)r * n_heads * kHeadDim);
      acc[0] += bf16lo_to_f32(w[0]);
      acc[1] += bf16hi_to_f32(w[0]);
      acc[2] += bf16lo_to_f32(w[1]);
      acc[3] += bf16hi_to_f32(w[1]);
    }
  } else {
    constexpr int G = MODE == 2 ? 4 : 1;  // scales per row; dims d4..d4+3 lie in group d4 / 32 of kvi8r32
    const int64_t hr = (int64_t)head * s_kv + r0;
    const int8_t* src = static_cast<const int8_t*>(side ? v : k) + hr * kHeadDim + d4;
    const uint16_t* sc = (side ? v_scale : k_scale) + hr * G + (G == 4 ? d4 >> 5 : 0);
    for (int r = rg; r < n; r += 4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + (int64_t)r * kHeadDim);
      const float f = (float)__builtin_bit_cast(_Float16, sc[r * G]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += (float)(int8_t)(w >> (8 * e)) * f;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) part[side][rg][d4 + e] = acc[e];
  __syncthreads();
  const int d = tid & (kHeadDim - 1);
  const float sum = (part[side][0][d] + part[side][1][d]) + (part[side][2][d] + part[side][3][d]);
  const float mean = sum / (float)n;
  const int64_t o = ((int64_t)head * n_kt + t) * kHeadDim + d;
  if (side) vmean[o] = (uint16_t)(Operand<MODE>::pack(mean, 0.0f) & 0xFFFFu);
  float amax = fabsf(mean);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (!side && (tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  if (!side) {
    const float mx = fmaxf(wmax[0], wmax[1]);
    int e = 0;
    if (mx > 0.0f) (void)frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
    kmean[o] = (uint16_t)(Operand<MODE>::pack(ldexpf(mean, 7 - e), 0.0f) & 0xFFFFu);
    if (tid == 0) kmscale[(int64_t)head * n_kt + t] = ldexpf(1.0f, e - 7);
  }
}

template <int MODE, bool SOL>
hipError_t launch_sparse(const AttnChunk& a, const SolArgs& sa, hipStream_t stream) {
  const int32_t n_qt = (int32_t)((a.rows + kSparseBlockRows - 1) / kSparseBlockRows);
  const int32_t n_kt = (int32_t)((a.s_kv + kTile - 1) / kTile);
  const int64_t n_wg = (int64_t)n_qt * a.n_heads;
  if (n_wg == 0) return hipSuccess;
  if constexpr (SOL)
    hipLaunchKernelGGL((attn_fwd_sparse_sol_kernel<MODE>), dim3((unsigned)n_wg), dim3(128), 0, stream, a, n_qt,
                       n_kt, sa);
  else if constexpr (MODE == 0)
    hipLaunchKernelGGL((attn_fwd_sparse_pair_kernel<MODE>), dim3((unsigned)(((int64_t)n_qt + 1) / 2 * a.n_heads)),
                       dim3(512), 0, stream, a, n_qt, n_kt);
  else
    hipLaunchKernelGGL((attn_fwd_sparse_kernel<MODE>), dim3((unsigned)n_wg), dim3(128), 0, stream, a, n_qt, n_kt);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_sparse(const AttnChunk& a, const SolArgs* sol, hipStream_t stream) {
  return sol != nullptr ? launch_sparse<MODE, true>(a, *sol, stream) : launch_sparse<MODE, false>(a, SolArgs{}, stream);
}

}  // namespace

template <int MODE>
hipError_t launch_dense(const AttnChunk& a, hipStream_t stream) {
  const int32_t n_qt = (int32_t)((a.rows + 255) / 256);
  const int32_t n_kt = (int32_t)((a.s_kv + kTile - 1) / kTile);
  const int64_t n_wg = (int64_t)n_qt * a.n_heads;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_dense_kernel<MODE>), dim3((unsigned)n_wg), dim3(512), 0, stream, a, n_qt, n_kt);
  return hipGetLastError();
}

int64_t dense_state_floats(int64_t rows, int32_t n_heads) {
  return (rows + 255) / 256 * n_heads * 512 * (int64_t)kStateFloats;
}

template <int MODE>
hipError_t launch_dense_block(const AttnChunk& a, hipStream_t stream) {
  const int32_t n_qt = (int32_t)((a.rows + 255) / 256);
  const int32_t n_kt = (int32_t)((a.s_kv + kTile - 1) / kTile);
  const int64_t n_wg = (int64_t)n_qt * a.n_heads;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_dense_kernel<MODE, true>), dim3((unsigned)n_wg), dim3(512), 0, stream, a, n_qt, n_kt);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_block(int mode, const AttnChunk& a, hipStream_t stream) {
  if (mode == 0) return launch_dense_block<0>(a, stream);
  if (mode == 1) return launch_dense_block<1>(a, stream);
  return launch_dense_block<2>(a, stream);
}

hipError_t launch_attn_fwd(int mode, bool sparse, const AttnChunk& a, const SolArgs* sol, hipStream_t stream) {
  static_assert(kSparseBlockRows == 2 * 32, "sparse kernel covers one routing tile");
  if (sol != nullptr && (!sparse || a.s_kv > kSolMaxKv)) return hipErrorInvalidValue;
  if (mode == 0) return sparse ? launch_sparse<0>(a, sol, stream) : launch_dense<0>(a, stream);
  if (mode == 1) return sparse ? launch_sparse<1>(a, sol, stream) : launch_dense<1>(a, stream);
  return sparse ? launch_sparse<2>(a, sol, stream) : launch_dense<2>(a, stream);
}

hipError_t launch_route_build(const uint8_t* mask, int64_t n_qt_total, int64_t qt0, int32_t n_qt, int32_t n_kt,
                              int32_t n_heads, int32_t* counts, int32_t* lists, int32_t* drops,
                              hipStream_t stream) {
  if (n_qt == 0) return hipSuccess;
  hipLaunchKernelGGL(route_build_kernel, dim3((unsigned)n_qt, (unsigned)n_heads), dim3(256), 0, stream, mask,
                     n_qt_total, qt0, n_qt, n_kt, counts, lists, drops);
  return hipGetLastError();
}

hipError_t launch_tile_means(int mode, const void* k, const void* v, const uint16_t* k_scale,
                             const uint16_t* v_scale, int64_t s_kv, int32_t n_heads, uint16_t* kmean,
                             uint16_t* vmean, float* kmscale, hipStream_t stream) {
  const int64_t n_kt = (s_kv + kTile - 1) / kTile;
  if (n_kt == 0) return hipSuccess;
  const dim3 grid((unsigned)n_kt, (unsigned)n_heads);
  if (mode == 0)
    hipLaunchKernelGGL(tile_means_kernel<0>, grid, dim3(256), 0, stream, k, v, k_scale, v_scale, s_kv, n_heads,
                       kmean, vmean, kmscale);
  else if (mode == 1)
    hipLaunchKernelGGL(tile_means_kernel<1>, grid, dim3(256), 0, stream, k, v, k_scale, v_scale, s_kv, n_heads,
                       kmean, vmean, kmscale);
  else
    hipLaunchKernelGGL(tile_means_kernel<2>, grid, dim3(256), 0, stream, k, v, k_scale, v_scale, s_kv, n_heads,
                       kmean, vmean, kmscale);
  return hipGetLastError();
}

}  // namespace h3a
