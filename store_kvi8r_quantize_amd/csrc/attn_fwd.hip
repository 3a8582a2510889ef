// attn_fwd: one query chunk of full attention against the whole K/V store, with
// the online-softmax state carried in registers across every K/V block.
//
// What it computes: the attention step of the "H3 Streamed Blocks" node page
// ("How it works"; Inputs table rows q_chunk, kv_block, kv_store) for the
// "bf16 (exact)" store and the "kvi8r" store ("Low VRAM, low RAM", "The K/V
// store options": a K/V block dequant is one int8 -> fp16 cast times the row
// scale, attention in fp16 with an online-softmax combine), optionally
// restricted to the kept 64Q x 64KV tiles of a mask ("H3-Optimizations" page,
// Nodes: routed 64Q x 64KV geometry, hard arm drops rejected tiles).
//
// MI355X design
//   * Workgroup = NW waves x 32 query rows of one head (dense: NW = 8, 256 rows;
//     sparse: NW = 2, one 64-row routing tile).  Key/value tiles of 64 tokens.
//   * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_{f16,bf16}: the
//     query index runs across lanes, keys across the 16 accumulator registers,
//     so the softmax row max / row sum are in-lane (plus one exchange between
//     lanes l and l^32).  P^T then feeds O^T += V^T P^T directly from registers
//     as the B operand; the key order inside each 16-key step is chosen to match
//     the accumulator layout, and V^T is read from LDS in that same order.
//   * K/V tiles go HBM/L2 -> registers -> (kvi8r: int8 -> fp16 by byte permute
//     into the 0x64xx exponent, one packed subtract and one packed multiply by
//     the row scale) -> LDS, once per workgroup, double-buffered, one barrier
//     per tile.  K is stored row-major [key][dim], V transposed [dim][key], both
//     XOR-swizzled against bank conflicts.
//   * Lazy rescale: the running max used for exp2 is only raised when a tile's
//     max exceeds it by more than 2^8, so the O accumulator is rescaled a few
//     times per row instead of every tile (P stays <= 256: safe in fp16/bf16).
//   * Every per-row decision depends only on that row's scores, so a row's
//     result is independent of q_chunk, kv_block and of which kernel variant
//     (dense or sparse with all tiles kept) computed it.
//   * blockIdx -> (head, q-tile) is remapped so that consecutive workgroups on
//     one XCD (dispatch is round-robin over the 8 XCDs) share a head and
//     reuse its K/V tiles from that XCD's L2.
#include "h3a_device.h"
#include "launch.h"

namespace h3a {

namespace {

constexpr float kLazyThreshold = 8.0f;  // log2 units
constexpr uint32_t kExp64 = 0x64646464u;

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

// Four int8 codes (one dword) times a row scale -> two fp16 pairs.
__device__ __forceinline__ u32x2 dequant4(uint32_t w, half2v s2) {
  const uint32_t u = w ^ 0x80808080u;  // code + 128 as an unsigned byte
  const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  half2v a = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kExp64, u, 0x04010400u));  // 1024 + byte
  half2v b = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kExp64, u, 0x04030402u));
  return u32x2{__builtin_bit_cast(uint32_t, (a - bias) * s2), __builtin_bit_cast(uint32_t, (b - bias) * s2)};
}

// Per-thread staging registers for one K/V tile.
template <int MODE, int NT>
struct Stage {
  static constexpr int KU = 512 / NT;  // K units (one key row x 16 dims) per thread
  static constexpr int VU = 512 / NT;  // V units (4 keys x 4 dims) per thread
  u32x4 k[KU][MODE == 0 ? 2 : 1];
  uint32_t ks[KU];
  uint32_t v[VU][4][MODE == 0 ? 2 : 1];
  uint32_t vs[VU][4];
};

// Tile rows are keys kt*64 .. kt*64+63; rows >= s_kv load as zeros.
template <int MODE, int NT>
__device__ __forceinline__ void load_tile(Stage<MODE, NT>& st, const AttnChunk& a, int head, int kt, int tid) {
  const int64_t kv0 = (int64_t)kt * kTile;
#pragma unroll
  for (int j = 0; j < Stage<MODE, NT>::KU; ++j) {
    const int u = tid + NT * j;
    const int64_t kv_raw = kv0 + (u >> 3);
    const int d16 = u & 7;
    const bool ok = kv_raw < a.s_kv;
    const int64_t kv = ok ? kv_raw : 0;  // masked rows address row 0: every pointer stays in bounds
    if constexpr (MODE == 0) {
      const uint16_t* p = static_cast<const uint16_t*>(a.k) + (kv * a.n_heads + head) * kHeadDim + 16 * d16;
      st.k[j][0] = ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
      st.k[j][1] = ok ? *reinterpret_cast<const u32x4*>(p + 8) : u32x4{0, 0, 0, 0};
    } else {
      const int64_t row = (int64_t)head * a.s_kv + kv;
      const int8_t* p = static_cast<const int8_t*>(a.k) + row * kHeadDim + 16 * d16;
      st.k[j][0] = ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
      st.ks[j] = ok ? a.k_scale[row] : 0u;
    }
  }
#pragma unroll
  for (int j = 0; j < Stage<MODE, NT>::VU; ++j) {
    const int u = tid + NT * j;
    const int kvg = u >> 5, dg = u & 31;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t kv_raw = kv0 + 4 * kvg + r;
      const bool ok = kv_raw < a.s_kv;
      const int64_t kv = ok ? kv_raw : 0;
      if constexpr (MODE == 0) {
        const uint16_t* p = static_cast<const uint16_t*>(a.v) + (kv * a.n_heads + head) * kHeadDim + 4 * dg;
        const u32x2 w = ok ? *reinterpret_cast<const u32x2*>(p) : u32x2{0, 0};
        st.v[j][r][0] = w[0];
        st.v[j][r][1] = w[1];
      } else {
        const int64_t row = (int64_t)head * a.s_kv + kv;
        const int8_t* p = static_cast<const int8_t*>(a.v) + row * kHeadDim + 4 * dg;
        st.v[j][r][0] = ok ? *reinterpret_cast<const uint32_t*>(p) : 0u;
        st.vs[j][r] = ok ? a.v_scale[row] : 0u;
      }
    }
  }
}

// LDS layouts (16-bit elements):
//   K  [64 keys][128 dims]: 16-byte chunk c of key row r lives at chunk c ^ (r & 15).
//   V^T[128 dims][64 keys]: 8-byte unit u (4 keys) of dim row d lives at unit u ^ vswz(d).
__device__ __forceinline__ int vswz(int d) { return (d ^ (d >> 4)) & 15; }

template <int MODE, int NT>
__device__ __forceinline__ void store_tile(const Stage<MODE, NT>& st, uint16_t* lk, uint16_t* lv, int tid) {
#pragma unroll
  for (int j = 0; j < Stage<MODE, NT>::KU; ++j) {
    const int u = tid + NT * j;
    const int r = u >> 3, d16 = u & 7;
    u32x4 c0, c1;
    if constexpr (MODE == 0) {
      c0 = st.k[j][0];
      c1 = st.k[j][1];
    } else {
      const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)st.ks[j]);
      const half2v s2 = {s, s};
      const u32x2 e0 = dequant4(st.k[j][0][0], s2), e1 = dequant4(st.k[j][0][1], s2);
      const u32x2 e2 = dequant4(st.k[j][0][2], s2), e3 = dequant4(st.k[j][0][3], s2);
      c0 = u32x4{e0[0], e0[1], e1[0], e1[1]};
      c1 = u32x4{e2[0], e2[1], e3[0], e3[1]};
    }
    *reinterpret_cast<u32x4*>(lk + r * kHeadDim + (((2 * d16) ^ (r & 15)) << 3)) = c0;
    *reinterpret_cast<u32x4*>(lk + r * kHeadDim + (((2 * d16 + 1) ^ (r & 15)) << 3)) = c1;
  }
#pragma unroll
  for (int j = 0; j < Stage<MODE, NT>::VU; ++j) {
    const int u = tid + NT * j;
    const int kvg = u >> 5, dg = u & 31;
    uint32_t p01[4], p23[4];  // per key row r: packed (dim0, dim1) and (dim2, dim3)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (MODE == 0) {
        p01[r] = st.v[j][r][0];
        p23[r] = st.v[j][r][1];
      } else {
        const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)st.vs[j][r]);
        const half2v s2 = {s, s};
        const u32x2 e = dequant4(st.v[j][r][0], s2);
        p01[r] = e[0];
        p23[r] = e[1];
      }
    }
    // transpose 4 keys x 4 dims: dim i gets (key0, key1 | key2, key3)
    u32x2 t[4];
    t[0] = u32x2{__builtin_amdgcn_perm(p01[1], p01[0], 0x05040100u), __builtin_amdgcn_perm(p01[3], p01[2], 0x05040100u)};
    t[1] = u32x2{__builtin_amdgcn_perm(p01[1], p01[0], 0x07060302u), __builtin_amdgcn_perm(p01[3], p01[2], 0x07060302u)};
    t[2] = u32x2{__builtin_amdgcn_perm(p23[1], p23[0], 0x05040100u), __builtin_amdgcn_perm(p23[3], p23[2], 0x05040100u)};
    t[3] = u32x2{__builtin_amdgcn_perm(p23[1], p23[0], 0x07060302u), __builtin_amdgcn_perm(p23[3], p23[2], 0x07060302u)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 4 * dg + i;
      *reinterpret_cast<u32x2*>(lv + d * kTile + ((kvg ^ vswz(d)) << 2)) = t[i];
    }
  }
}

template <int MODE, int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(AttnChunk a, int32_t n_qt, int32_t n_kt) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  using Op = Operand<MODE>;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kTile * kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kHeadDim * kTile];

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
  const int64_t qrow = (int64_t)qt * BM + wave * 32 + c;
  const bool qvalid = qrow < a.rows;

  // B operand of S^T = K Q^T: lane holds Q[qrow][16t + 8g .. 16t + 8g + 7].
  u32x4 qf[8];
  {
    const uint16_t* qp = a.q + ((qvalid ? qrow : 0) * a.n_heads + head) * kHeadDim + 8 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qf[t] = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * t) : u32x4{0, 0, 0, 0};
  }

  int n_tiles = n_kt;
  const int32_t* list = nullptr;
  if (SPARSE) {
    n_tiles = a.counts[head * n_qt + qt];
    list = a.lists + ((int64_t)head * n_qt + qt) * n_kt;
  }
  auto tile_at = [&](int i) -> int { return SPARSE ? list[i] : i; };

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  const float sl2 = a.scale_log2;
  const int last_full = (int)(a.s_kv / kTile);  // tiles with index >= this one are partial

  Stage<MODE, NT> st;
  if (n_tiles > 0) {
    load_tile<MODE, NT>(st, a, head, tile_at(0), tid);
    store_tile<MODE, NT>(st, lds_k[0], lds_v[0], tid);
  }
  __syncthreads();
  if (n_tiles > 1) load_tile<MODE, NT>(st, a, head, tile_at(1), tid);

  for (int i = 0; i < n_tiles; ++i) {
    const int kt = tile_at(i);
    const uint16_t* lk = lds_k[i & 1];
    const uint16_t* lv = lds_v[i & 1];

    // ---- S^T (64 keys x 32 queries) = K Q^T -------------------------------------
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int r = 32 * kb + c;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(lk + r * kHeadDim + (((2 * t + g) ^ (r & 15)) << 3));
        s[kb] = Op::mfma(ka, qf[t], s[kb]);
      }
    }
    // Accumulator register j of block kb holds key 32*kb + 8*(j/4) + 4*g + j%4.
    if (kt >= last_full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if ((int64_t)kt * kTile + 32 * kb + 8 * (j >> 2) + 4 * g + (j & 3) >= a.s_kv) s[kb][j] = -__builtin_inff();
    }

    // ---- online softmax (base 2) ----------------------------------------------
    float mx = s[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[1][j]);
    mx = fmaxf(mx, xor32_f32(mx));
    const float mt = mx * sl2;
    if (mt > m_run + kLazyThreshold) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) acc[i2] *= alpha;
      l_run *= alpha;
      m_run = mt;
    }
    const float nm = -m_run;
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][j], sl2, nm));
        s[kb][j] = p;
        ls += p;
      }
    l_run += ls;
    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[kb][hf][e] = Op::pack(s[kb][8 * hf + 2 * e], s[kb][8 * hf + 2 * e + 1]);

    // ---- O^T (128 dims x 32 queries) += V^T P^T ---------------------------------
    // k-step j covers keys 32*(j/2) + 16*(j%2) + 4g + {0..3} and the same + 8.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + c;
      const uint16_t* row = lv + d * kTile;
      const int sw = vswz(d);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u0 = 8 * (j >> 1) + 4 * (j & 1) + g;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(row + ((u0 ^ sw) << 2));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(row + (((u0 + 2) ^ sw) << 2));
        acc[db] = Op::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[j >> 1][j & 1], acc[db]);
      }
    }

    if (i + 1 < n_tiles) store_tile<MODE, NT>(st, lds_k[(i + 1) & 1], lds_v[(i + 1) & 1], tid);
    __syncthreads();
    if (i + 2 < n_tiles) load_tile<MODE, NT>(st, a, head, tile_at(i + 2), tid);
  }

  // ---- epilogue: normalise and store this lane's 64 dims of its query row ------
  const float lt = l_run + xor32_f32(l_run);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (qvalid) {
    const int64_t base = (qrow * a.n_heads + head) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * db + 8 * rg + 4 * g;  // accumulator registers 4rg..4rg+3 = dims d0..d0+3
        const float o0 = acc[db][4 * rg] * inv, o1 = acc[db][4 * rg + 1] * inv;
        const float o2 = acc[db][4 * rg + 2] * inv, o3 = acc[db][4 * rg + 3] * inv;
        if constexpr (MODE == 0) {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + base + d0) =
              u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        } else {
          *reinterpret_cast<u32x4*>(static_cast<float*>(a.out) + base + d0) =
              u32x4{__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2), __float_as_uint(o3)};
        }
      }
  }
}

// Kept-tile list of one (head, q-tile) row of the mask, in increasing key order.
__global__ __launch_bounds__(256) void route_build_kernel(const uint8_t* __restrict__ mask, int64_t n_qt_total,
                                                          int64_t qt0, int32_t n_qt, int32_t n_kt,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ lists) {
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
  if (tid == 255) counts[head * n_qt + qt] = part[255];
}

template <int MODE, int NW, bool SPARSE>
hipError_t launch_variant(const AttnChunk& a, hipStream_t stream) {
  constexpr int BM = NW * 32;
  const int32_t n_qt = (int32_t)((a.rows + BM - 1) / BM);
  const int32_t n_kt = (int32_t)((a.s_kv + kTile - 1) / kTile);
  const int64_t n_wg = (int64_t)n_qt * a.n_heads;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_kernel<MODE, NW, SPARSE>), dim3((unsigned)n_wg), dim3(NW * 64), 0, stream, a, n_qt,
                     n_kt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(int mode, bool sparse, const AttnChunk& a, hipStream_t stream) {
  static_assert(kSparseBlockRows == 2 * 32, "sparse kernel covers one routing tile");
  if (mode == 0) return sparse ? launch_variant<0, 2, true>(a, stream) : launch_variant<0, 8, false>(a, stream);
  return sparse ? launch_variant<1, 2, true>(a, stream) : launch_variant<1, 8, false>(a, stream);
}

hipError_t launch_route_build(const uint8_t* mask, int64_t n_qt_total, int64_t qt0, int32_t n_qt, int32_t n_kt,
                              int32_t n_heads, int32_t* counts, int32_t* lists, hipStream_t stream) {
  if (n_qt == 0) return hipSuccess;
  hipLaunchKernelGGL(route_build_kernel, dim3((unsigned)n_qt, (unsigned)n_heads), dim3(256), 0, stream, mask,
                     n_qt_total, qt0, n_qt, n_kt, counts, lists);
  return hipGetLastError();
}

}  // namespace h3a
