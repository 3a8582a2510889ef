// C ABI entry points: argument checks, the query-chunk loop and kernel timing.
//
// The query-chunk loop is the one of the "H3 Streamed Blocks" node page ("How it
// works", Inputs table q_chunk row): every chunk of q_chunk query tokens attends
// the whole K/V store; for the kvi8r store the chunk is rotated first and its
// output rotated back once ("Low VRAM, low RAM", "The K/V store options").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "h3a.h"
#include "launch.h"

// Scratch of h3a_attention_noalloc: one file-scope device array; every GPU the
// library runs on holds its own copy for the life of the process.  In host code
// `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current
// (scratch_address below), and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[H3A_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(H3A_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// `p` must be device-accessible memory with `bytes` bytes inside one allocation.
int check_buffer(const void* p, uint64_t bytes, unsigned align, const char* name) {
  if (bytes == 0) return H3A_OK;
  if (p == nullptr) return fail(H3A_EINVAL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align != 0) return fail(H3A_EINVAL, "%s is not %u-byte aligned", name, align);
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(H3A_EINVAL, "%s is not device memory (%s)", name, hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(H3A_EINVAL, "%s is not device memory", name);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(H3A_EINVAL, "%s: cannot query its allocation (%s)", name, hipGetErrorString(e));
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
  if (q < b || (q - b) + bytes > size)
    return fail(H3A_EINVAL, "%s: needs %llu bytes but its allocation holds %llu from this pointer", name,
                (unsigned long long)bytes, (unsigned long long)(q >= b ? size - (q - b) : 0));
  return H3A_OK;
}

// Factor the query rotation applies before rounding: the kvi8r32 attention
// kernels take softmax_scale * log2 e from Q' (their K is dequantised, so every
// key has the same score factor); the kvi8r kernels apply it per key.
float q_post(int32_t mode, float scale_log2) { return mode == H3A_MODE_KVI8R32 ? scale_log2 : 1.0f; }

// kvi8r32 multiplies the fp16 query by softmax_scale * log2 e: at most 1, so
// that the product cannot leave the fp16 range of the rotated query itself.
int check_mode_scale(int32_t mode, float softmax_scale) {
  if (mode == H3A_MODE_KVI8R32 && softmax_scale * 1.4426950408889634f > 1.0f)
    return fail(H3A_EINVAL, "H3A_MODE_KVI8R32 takes softmax_scale <= ln 2 (softmax_scale * log2 e <= 1; got %g)",
                (double)softmax_scale);
  return H3A_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct WorkspaceLayout {
  uint64_t kmean = 0, vmean = 0, kmscale = 0;  // whole call (Sol)
  uint64_t qrot = 0, orot = 0, counts = 0, lists = 0, drops = 0, total = 0;  // one query chunk
};

// Workspace: Sol tile means of the store (once per call), then per query chunk
// rotated Q (fp16), rotated output (fp32), sparse kept (and Sol dropped) lists.
// mode is the base mode; sol needs sparse.
bool workspace_layout(int64_t s_q, int64_t s_kv, int32_t n_heads, int64_t q_chunk, int32_t mode, bool sparse,
                      bool sol, WorkspaceLayout* w) {
  *w = WorkspaceLayout{};
  if (s_q <= 0 || q_chunk <= 0) return true;
  const int64_t rows = q_chunk < s_q ? q_chunk : s_q;
  int64_t elems;
  if (!mul_ok(rows, (int64_t)n_heads * H3A_HEAD_DIM, &elems)) return false;
  uint64_t off = 0;
  if (sol) {
    const int64_t n_kt = (s_kv + H3A_TILE - 1) / H3A_TILE;
    int64_t nm;
    if (!mul_ok(n_kt * n_heads, H3A_HEAD_DIM, &nm)) return false;
    w->kmean = off;
    off = align256(off + (uint64_t)nm * 2);
    w->vmean = off;
    off = align256(off + (uint64_t)nm * 2);
    w->kmscale = off;
    off = align256(off + (uint64_t)(n_kt * n_heads) * 4);
  }
  if (mode != H3A_MODE_EXACT_BF16) {
    w->qrot = off;
    off = align256(off + (uint64_t)elems * 2);
    w->orot = off;
    off = align256(off + (uint64_t)elems * 4);
  }
  if (sparse) {
    const int64_t n_qt = (rows + H3A_TILE - 1) / H3A_TILE;
    const int64_t n_kt = (s_kv + H3A_TILE - 1) / H3A_TILE;
    int64_t nl, nc;
    if (!mul_ok(n_qt * n_heads, n_kt, &nl) || !mul_ok(n_qt, n_heads, &nc)) return false;
    w->counts = off;
    off = align256(off + (uint64_t)nc * 4);
    w->lists = off;
    off = align256(off + (uint64_t)nl * 4);
    if (sol) {
      w->drops = off;
      off = align256(off + (uint64_t)nl * 4);
    }
  }
  w->total = off;
  return true;
}

// ---- kernel timing --------------------------------------------------------------
std::mutex g_timing_mu;
bool g_timing_on = false;
// Recorded event pairs per timed kernel kind (H3A_TIMING_ATTENTION, _ROTATE_Q, _UNROTATE_O, _KV_QUANTIZE).
constexpr int kTimingKinds = 4;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_events[kTimingKinds];

// A pair of timing events around one kernel launch on `st`: begin() records the
// start, end() the stop and hands both to the list of its kind; a pair that
// never reached end() is destroyed with the guard.
struct LaunchTimer {
  int kind = H3A_TIMING_ATTENTION;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  explicit LaunchTimer(int k = H3A_TIMING_ATTENTION) : kind(k) {}
  hipError_t begin(hipStream_t st) {
    hipError_t e;
    if ((e = hipEventCreate(&ev0)) != hipSuccess || (e = hipEventCreate(&ev1)) != hipSuccess) return e;
    return hipEventRecord(ev0, st);
  }
  hipError_t end(hipStream_t st) {
    hipError_t e = hipEventRecord(ev1, st);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_events[kind].emplace_back(ev0, ev1);
    ev0 = ev1 = nullptr;
    return hipSuccess;
  }
  ~LaunchTimer() {
    if (ev0) (void)hipEventDestroy(ev0);
    if (ev1) (void)hipEventDestroy(ev1);
  }
};

// ---- argument checks shared by the attention entry points ----------------------
int check_shapes(int64_t s_q, int64_t s_kv, int32_t n_heads, int64_t q_chunk, int64_t kv_block,
                 float softmax_scale) {
  // The kernels count a tile's rows in 32 bits and address 64 token rows of the
  // exact store ([s_kv, n_heads, 128] bf16) with 32-bit offsets.
  if (n_heads < 1 || n_heads > 65536) return fail(H3A_EINVAL, "n_heads must be in [1, 65536] (got %d)", n_heads);
  if (s_q < 0 || s_kv < 0) return fail(H3A_EINVAL, "s_q and s_kv must be >= 0");
  if (s_q > ((int64_t)1 << 31) || s_kv >= ((int64_t)1 << 31)) return fail(H3A_EINVAL, "sequence too long");
  if (q_chunk < 1) return fail(H3A_EINVAL, "q_chunk must be >= 1 (got %lld)", (long long)q_chunk);
  if (kv_block < 0 || kv_block % H3A_TILE != 0)
    return fail(H3A_EINVAL, "kv_block must be 0 or a positive multiple of 64 (got %lld)", (long long)kv_block);
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(H3A_EINVAL, "softmax_scale must be finite and > 0");
  return H3A_OK;
}

// q and out: bf16 [s_q, n_heads, 128].
int check_rows(const void* q, const void* out, int64_t s_q, int32_t n_heads) {
  int64_t n;
  if (!mul_ok(s_q, (int64_t)n_heads * H3A_HEAD_DIM, &n)) return fail(H3A_EINVAL, "size overflow");
  int rc;
  if ((rc = check_buffer(q, (uint64_t)n * 2, 16, "q")) != H3A_OK) return rc;
  return check_buffer(out, (uint64_t)n * 2, 16, "out");
}

// One K/V store of `mode` over s_kv tokens.
int check_store(int32_t mode, const void* k, const void* v, const void* scales, int64_t s_kv, int32_t n_heads,
                const char* k_name, const char* v_name) {
  int64_t n;
  if (!mul_ok(s_kv, (int64_t)n_heads * H3A_HEAD_DIM, &n)) return fail(H3A_EINVAL, "size overflow");
  const bool q8 = mode != H3A_MODE_EXACT_BF16;
  const uint64_t bytes = (uint64_t)n * (q8 ? 1 : 2);
  int rc;
  if ((rc = check_buffer(k, bytes, 16, k_name)) != H3A_OK) return rc;
  if ((rc = check_buffer(v, bytes, 16, v_name)) != H3A_OK) return rc;
  if (mode == H3A_MODE_KVI8R) return check_buffer(scales, (uint64_t)s_kv * n_heads * 4, 2, "scales");
  if (mode == H3A_MODE_KVI8R32) return check_buffer(scales, (uint64_t)s_kv * n_heads * 16, 8, "scales");
  return H3A_OK;
}

int check_workspace(const void* workspace, size_t workspace_bytes, const WorkspaceLayout& wl) {
  if (wl.total == 0) return H3A_OK;
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(H3A_EWORKSPACE, "workspace needs %llu bytes (got %llu)", (unsigned long long)wl.total,
                (unsigned long long)(workspace == nullptr ? 0 : workspace_bytes));
  return check_buffer(workspace, wl.total, 256, "workspace");
}

// `p` must be pinned host memory (hipHostMalloc) with `bytes` bytes inside one allocation.
int check_host_buffer(const void* p, uint64_t bytes, const char* name) {
  if (bytes == 0) return H3A_OK;
  if (p == nullptr) return fail(H3A_EINVAL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(H3A_EINVAL, "%s is not 16-byte aligned", name);
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(H3A_EINVAL, "%s is not pinned host memory (allocate it with hipHostMalloc)", name);
  }
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(H3A_EINVAL, "%s: cannot query its allocation (%s)", name, hipGetErrorString(e));
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
  if (q < b || (q - b) + bytes > size)
    return fail(H3A_EINVAL, "%s: needs %llu bytes but its allocation holds %llu from this pointer", name,
                (unsigned long long)bytes, (unsigned long long)(q >= b ? size - (q - b) : 0));
  return H3A_OK;
}

// Device workspace of h3a_attention_host_kv: the per-chunk buffers of a dense
// call, the (m, l, O) state of one query chunk, and two K/V block buffers.
struct StagedLayout {
  WorkspaceLayout base;
  uint64_t state = 0;
  uint64_t blk[2] = {0, 0};  // each: K, V, K scales, V scales
  uint64_t k_bytes = 0, s_bytes = 0;  // per block buffer: K (= V) bytes, K (= V) scale bytes
  int64_t blk_rows = 0;
  uint64_t total = 0;
};

int64_t default_kv_block(int64_t kv_block) { return kv_block > 0 ? kv_block : 16384; }

bool staged_layout(int64_t s_q, int64_t s_kv, int32_t n_heads, int64_t q_chunk, int64_t kv_block, int32_t mode,
                   StagedLayout* w) {
  *w = StagedLayout{};
  if (!workspace_layout(s_q, s_kv, n_heads, q_chunk, mode, false, false, &w->base)) return false;
  if (s_q <= 0 || s_kv <= 0) {
    w->total = w->base.total;
    return true;
  }
  const int64_t rows = q_chunk < s_q ? q_chunk : s_q;
  const int64_t blk = default_kv_block(kv_block) < s_kv ? default_kv_block(kv_block) : s_kv;
  const int64_t g = mode == H3A_MODE_KVI8R32 ? 4 : 1;
  int64_t kb;
  if (!mul_ok(blk * n_heads, (int64_t)H3A_HEAD_DIM * (mode == H3A_MODE_EXACT_BF16 ? 2 : 1), &kb)) return false;
  const int64_t st = h3a::dense_state_floats(rows, n_heads) * 4;
  uint64_t off = w->base.total;
  w->state = off;
  off = align256(off + (uint64_t)st);
  w->k_bytes = align256((uint64_t)kb);
  w->s_bytes = mode == H3A_MODE_EXACT_BF16 ? 0 : align256((uint64_t)(blk * n_heads * g * 2));
  for (int i = 0; i < 2; ++i) {
    w->blk[i] = off;
    off += 2 * w->k_bytes + 2 * w->s_bytes;
  }
  w->blk_rows = blk;
  w->total = off;
  return true;
}

// One copy stream per device for host-staged K/V (default priority, does not
// synchronise with the null stream).  Kept until the process ends.
std::mutex g_copy_mu;
std::vector<std::pair<int, hipStream_t>> g_copy_streams;

hipError_t copy_stream(hipStream_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_copy_mu);
  for (auto& p : g_copy_streams)
    if (p.first == dev) {
      *out = p.second;
      return hipSuccess;
    }
  hipStream_t s = nullptr;
  if ((e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking)) != hipSuccess) return e;
  g_copy_streams.emplace_back(dev, s);
  *out = s;
  return hipSuccess;
}

// ---- the query-chunk loop -----------------------------------------------------------
// One validated call over one store.
struct Pass {
  int32_t mode = 0;
  bool sol = false;
  bool out_f16 = false;  // kvi8r modes: fp16 output rows (H3A_OUT_F16), else bf16
  const uint16_t* q = nullptr;
  uint16_t* out = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const uint16_t* k_scale = nullptr;
  const uint16_t* v_scale = nullptr;
  int64_t s_q = 0, s_kv = 0;
  int32_t n_heads = 0;
  float scale_log2 = 0.0f;
  int64_t q_chunk = 0;
  const uint8_t* tile_mask = nullptr;  // sparse when set; passes then start at multiples of 64 rows
  char* ws = nullptr;
  WorkspaceLayout wl;
  hipStream_t st = nullptr;
  bool timing = false;
};

Pass make_pass(int32_t mode, const void* q, void* out, const void* k, const void* v, const void* scales,
               int64_t s_q, int64_t s_kv, int32_t n_heads, float softmax_scale, int64_t q_chunk, char* ws,
               const WorkspaceLayout& wl, void* stream) {
  Pass p;
  p.mode = mode;
  p.q = static_cast<const uint16_t*>(q);
  p.out = static_cast<uint16_t*>(out);
  p.k = k;
  p.v = v;
  if (mode != H3A_MODE_EXACT_BF16 && scales != nullptr) {
    p.k_scale = static_cast<const uint16_t*>(scales);
    p.v_scale = p.k_scale + s_kv * n_heads * (mode == H3A_MODE_KVI8R32 ? 4 : 1);
  }
  p.s_q = s_q;
  p.s_kv = s_kv;
  p.n_heads = n_heads;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.q_chunk = q_chunk;
  p.ws = ws;
  p.wl = wl;
  p.st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lk(g_timing_mu);
  p.timing = g_timing_on;
  return p;
}

// Query rows [r0, r1), in passes of at most q_chunk rows ("H3 Streamed Blocks"
// node page, "How it works": each query chunk attends the whole K/V store).
int attend_rows(const Pass& p, int64_t r0, int64_t r1) {
  const int64_t n_qt_total = (p.s_q + H3A_TILE - 1) / H3A_TILE, n_kt = (p.s_kv + H3A_TILE - 1) / H3A_TILE;
  const bool sparse = p.tile_mask != nullptr;
  for (int64_t c0 = r0; c0 < r1; c0 += p.q_chunk) {
    const int64_t rows = (r1 - c0) < p.q_chunk ? (r1 - c0) : p.q_chunk;
    const int64_t off = c0 * p.n_heads * H3A_HEAD_DIM;
    h3a::AttnChunk a{};
    h3a::SolArgs sa{};
    a.rows = rows;
    a.s_kv = p.s_kv;
    a.n_heads = p.n_heads;
    a.scale_log2 = p.scale_log2;
    a.k = p.k;
    a.v = p.v;
    hipError_t e;
    if (p.mode != H3A_MODE_EXACT_BF16) {
      uint16_t* qrot = reinterpret_cast<uint16_t*>(p.ws + p.wl.qrot);
      LaunchTimer rt(H3A_TIMING_ROTATE_Q);
      if (p.timing && (e = rt.begin(p.st)) != hipSuccess) return hip_fail(e, "timing event");
      if ((e = h3a::launch_rotate_q(p.q + off, qrot, rows * p.n_heads, q_post(p.mode, p.scale_log2), p.st)) !=
          hipSuccess)
        return hip_fail(e, "rotate_q launch");
      if (p.timing && (e = rt.end(p.st)) != hipSuccess) return hip_fail(e, "timing event");
      a.q = qrot;
      a.k_scale = p.k_scale;
      a.v_scale = p.v_scale;
      a.out = p.ws + p.wl.orot;
    } else {
      a.q = p.q + off;
      a.out = p.out + off;
    }
    if (sparse) {
      a.counts = reinterpret_cast<const int32_t*>(p.ws + p.wl.counts);
      a.lists = reinterpret_cast<const int32_t*>(p.ws + p.wl.lists);
      int32_t* drops = nullptr;
      if (p.sol) {
        drops = reinterpret_cast<int32_t*>(p.ws + p.wl.drops);
        sa.drops = drops;
        sa.kmean = reinterpret_cast<const uint16_t*>(p.ws + p.wl.kmean);
        sa.vmean = reinterpret_cast<const uint16_t*>(p.ws + p.wl.vmean);
        sa.kmscale = reinterpret_cast<const float*>(p.ws + p.wl.kmscale);
      }
      const int32_t n_qt = (int32_t)((rows + H3A_TILE - 1) / H3A_TILE);
      if ((e = h3a::launch_route_build(p.tile_mask, n_qt_total, c0 / H3A_TILE, n_qt, (int32_t)n_kt, p.n_heads,
                                       reinterpret_cast<int32_t*>(p.ws + p.wl.counts),
                                       reinterpret_cast<int32_t*>(p.ws + p.wl.lists), drops, p.st)) != hipSuccess)
        return hip_fail(e, "route_build launch");
    }
    LaunchTimer timer;
    if (p.timing && (e = timer.begin(p.st)) != hipSuccess) return hip_fail(e, "timing event");
    if ((e = h3a::launch_attn_fwd(p.mode, sparse, a, p.sol ? &sa : nullptr, p.st)) != hipSuccess)
      return hip_fail(e, "attn_fwd launch");
    if (p.timing && (e = timer.end(p.st)) != hipSuccess) return hip_fail(e, "timing event");
    if (p.mode != H3A_MODE_EXACT_BF16) {
      LaunchTimer ut(H3A_TIMING_UNROTATE_O);
      if (p.timing && (e = ut.begin(p.st)) != hipSuccess) return hip_fail(e, "timing event");
      if ((e = h3a::launch_unrotate_o(reinterpret_cast<const float*>(p.ws + p.wl.orot), p.out + off,
                                      rows * p.n_heads, p.out_f16, p.st)) != hipSuccess)
        return hip_fail(e, "unrotate_o launch");
      if (p.timing && (e = ut.end(p.st)) != hipSuccess) return hip_fail(e, "timing event");
    }
  }
  return H3A_OK;
}

// One quantize call; grouped: one scale per 32 values.  x2 / codes2 / scales2: a
// second tensor of the same shape quantised in the same launch, or null.
int kv_quantize(const void* x, const void* x2, int64_t x_token_stride, int64_t n_tokens, int32_t n_heads,
                int32_t head_dim, int64_t token_offset, int64_t s_total, int8_t* codes, int8_t* codes2,
                void* scales_f16, void* scales2_f16, bool grouped, void* stream) {
  g_err.clear();
  if (head_dim != H3A_HEAD_DIM) return fail(H3A_EUNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  if (n_heads < 1) return fail(H3A_EINVAL, "n_heads must be >= 1 (got %d)", n_heads);
  if (n_tokens < 0 || token_offset < 0 || s_total < 0)
    return fail(H3A_EINVAL, "n_tokens, token_offset and s_total must be >= 0");
  if (token_offset > s_total || n_tokens > s_total - token_offset)
    return fail(H3A_EINVAL, "token_offset + n_tokens (%lld + %lld) exceeds s_total %lld", (long long)token_offset,
                (long long)n_tokens, (long long)s_total);
  if (x_token_stride < (int64_t)n_heads * H3A_HEAD_DIM || x_token_stride % 8 != 0)
    return fail(H3A_EINVAL, "x_token_stride must be >= n_heads*128 and a multiple of 8 (got %lld)",
                (long long)x_token_stride);
  if (n_tokens == 0) return H3A_OK;
  if (n_tokens > INT32_MAX / 2 || s_total > (int64_t)1 << 40) return fail(H3A_EINVAL, "sizes too large");
  const int64_t g = grouped ? 4 : 1;
  int64_t xb, cb, sb;
  if (!mul_ok(n_tokens - 1, x_token_stride, &xb) || !mul_ok(s_total * n_heads, H3A_HEAD_DIM, &cb) ||
      !mul_ok(s_total, (int64_t)n_heads * 2 * g, &sb))
    return fail(H3A_EINVAL, "size overflow");
  xb = (xb + (int64_t)n_heads * H3A_HEAD_DIM) * 2;
  int rc;
  const bool pair = x2 != nullptr;
  if ((rc = check_buffer(x, (uint64_t)xb, 16, pair ? "k" : "x")) != H3A_OK) return rc;
  if ((rc = check_buffer(codes, (uint64_t)cb, 16, pair ? "k_codes" : "codes")) != H3A_OK) return rc;
  if ((rc = check_buffer(scales_f16, (uint64_t)sb * (pair ? 2 : 1), grouped ? 8 : 2, "scales")) != H3A_OK) return rc;
  if (pair) {
    if ((rc = check_buffer(x2, (uint64_t)xb, 16, "v")) != H3A_OK) return rc;
    if ((rc = check_buffer(codes2, (uint64_t)cb, 16, "v_codes")) != H3A_OK) return rc;
    if (codes2 == codes) return fail(H3A_EINVAL, "k_codes and v_codes must be different buffers");
  }
  bool timing;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    timing = g_timing_on;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  LaunchTimer timer(H3A_TIMING_KV_QUANTIZE);
  hipError_t e = timing ? timer.begin(st) : hipSuccess;
  if (e == hipSuccess)
    e = h3a::launch_kvi8r_quantize(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(x2), x_token_stride,
                                   n_tokens, n_heads, token_offset, s_total, codes, codes2,
                                   static_cast<uint16_t*>(scales_f16), static_cast<uint16_t*>(scales2_f16), grouped,
                                   st);
  if (e == hipSuccess && timing) e = timer.end(st);
  return e == hipSuccess ? H3A_OK : hip_fail(e, "kvi8r_quantize launch");
}

// ---- scratch of h3a_attention_noalloc --------------------------------------------------
std::mutex g_scratch_mu;
std::vector<std::pair<int, char*>> g_scratch;  // (device, address of that device's copy of `scratch`)

int scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  for (auto& p : g_scratch)
    if (p.first == dev) {
      *out = p.second;
      return H3A_OK;
    }
  void* ptr = nullptr;
  if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
    return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0)
    return fail(H3A_EHIP, "scratch: device address %p is not 256-byte aligned", ptr);
  g_scratch.emplace_back(dev, static_cast<char*>(ptr));
  *out = static_cast<char*>(ptr);
  return H3A_OK;
}

// h3a_attention and h3a_attention_noalloc: the same checks and the same query-chunk
// loop; the second takes its workspace from `scratch` instead of the caller.
int attention_call(const void* q, const void* k_store, const void* v_store, const void* scales, int64_t s_q,
                   int64_t s_kv, int32_t n_heads, int32_t head_dim, float softmax_scale, int64_t q_chunk,
                   int64_t kv_block, int32_t mode, const uint8_t* tile_mask, void* out, void* workspace,
                   size_t workspace_bytes, bool use_scratch, void* stream) {
  g_err.clear();
  if (head_dim != H3A_HEAD_DIM) return fail(H3A_EUNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  const bool sol = (mode & H3A_SOL) != 0, out_f16 = (mode & H3A_OUT_F16) != 0;
  const int32_t mode_arg = mode;
  mode &= ~(H3A_SOL | H3A_OUT_F16);
  if (mode != H3A_MODE_EXACT_BF16 && mode != H3A_MODE_KVI8R && mode != H3A_MODE_KVI8R32)
    return fail(H3A_EINVAL, "unknown mode %d", mode_arg);
  if (out_f16 && mode == H3A_MODE_EXACT_BF16)
    return fail(H3A_EINVAL, "H3A_OUT_F16 applies to the kvi8r stores; the exact store's output is bf16");
  if (sol && tile_mask == nullptr) return fail(H3A_EINVAL, "H3A_SOL needs a tile_mask");
  if (sol && s_kv > h3a::kSolMaxKv) return fail(H3A_EINVAL, "H3A_SOL supports s_kv up to 2^30 - 64");
  int rc;
  if ((rc = check_shapes(s_q, s_kv, n_heads, q_chunk, kv_block, softmax_scale)) != H3A_OK) return rc;
  if ((rc = check_mode_scale(mode, softmax_scale)) != H3A_OK) return rc;
  const bool sparse = tile_mask != nullptr;
  if (sparse && q_chunk % H3A_TILE != 0)
    return fail(H3A_EINVAL, "q_chunk must be a multiple of 64 with a tile_mask (got %lld)", (long long)q_chunk);
  if (mode != H3A_MODE_EXACT_BF16 && scales == nullptr && s_kv > 0)
    return fail(H3A_EINVAL, "kvi8r modes need scales");
  if (mode == H3A_MODE_EXACT_BF16 && scales != nullptr) return fail(H3A_EINVAL, "exact mode takes no scales");
  WorkspaceLayout wl;
  if (!workspace_layout(s_q, s_kv, n_heads, q_chunk, mode, sparse, sol, &wl))
    return fail(H3A_EINVAL, "size overflow");
  if (use_scratch && wl.total > (uint64_t)H3A_NOALLOC_SCRATCH_BYTES)
    return fail(H3A_EWORKSPACE,
                "h3a_attention_noalloc: this call needs %llu bytes of scratch, more than its %llu; a smaller "
                "q_chunk needs less and gives the same output",
                (unsigned long long)wl.total, (unsigned long long)H3A_NOALLOC_SCRATCH_BYTES);
  if (s_q == 0) return H3A_OK;

  if ((rc = check_rows(q, out, s_q, n_heads)) != H3A_OK) return rc;
  if ((rc = check_store(mode, k_store, v_store, scales, s_kv, n_heads, "k_store", "v_store")) != H3A_OK) return rc;
  const int64_t n_qt_total = (s_q + H3A_TILE - 1) / H3A_TILE, n_kt = (s_kv + H3A_TILE - 1) / H3A_TILE;
  if (sparse) {
    int64_t mb;
    if (!mul_ok(n_qt_total * n_heads, n_kt, &mb)) return fail(H3A_EINVAL, "tile_mask size overflow");
    if ((rc = check_buffer(tile_mask, (uint64_t)mb, 1, "tile_mask")) != H3A_OK) return rc;
  }
  char* ws = static_cast<char*>(workspace);
  if (use_scratch) {
    if (wl.total > 0 && (rc = scratch_address(&ws)) != H3A_OK) return rc;
  } else if ((rc = check_workspace(workspace, workspace_bytes, wl)) != H3A_OK) {
    return rc;
  }

  Pass p = make_pass(mode, q, out, k_store, v_store, scales, s_q, s_kv, n_heads, softmax_scale, q_chunk, ws, wl,
                     stream);
  p.tile_mask = tile_mask;
  p.sol = sol;
  p.out_f16 = out_f16;
  if (sol) {
    hipError_t e = h3a::launch_tile_means(mode, k_store, v_store, p.k_scale, p.v_scale, s_kv, n_heads,
                                          reinterpret_cast<uint16_t*>(p.ws + wl.kmean),
                                          reinterpret_cast<uint16_t*>(p.ws + wl.vmean),
                                          reinterpret_cast<float*>(p.ws + wl.kmscale), p.st);
    if (e != hipSuccess) return hip_fail(e, "tile_means launch");
  }
  return attend_rows(p, 0, s_q);
}
}  // namespace

extern "C" {

int32_t h3a_abi_version(void) { return H3A_ABI_VERSION; }

const char* h3a_last_error(void) { return g_err.c_str(); }

int32_t h3a_kv_quantize(const void* x, int64_t x_token_stride, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                        int64_t token_offset, int64_t s_total, int8_t* codes, void* scales_f16, void* stream) {
  return kv_quantize(x, nullptr, x_token_stride, n_tokens, n_heads, head_dim, token_offset, s_total, codes, nullptr,
                     scales_f16, nullptr, false, stream);
}

int32_t h3a_kv_quantize_g32(const void* x, int64_t x_token_stride, int64_t n_tokens, int32_t n_heads,
                            int32_t head_dim, int64_t token_offset, int64_t s_total, int8_t* codes, void* scales_f16,
                            void* stream) {
  return kv_quantize(x, nullptr, x_token_stride, n_tokens, n_heads, head_dim, token_offset, s_total, codes, nullptr,
                     scales_f16, nullptr, true, stream);
}

int32_t h3a_kv_quantize_pair(const void* k, const void* v, int64_t x_token_stride, int64_t n_tokens, int32_t n_heads,
                             int32_t head_dim, int64_t token_offset, int64_t s_total, int8_t* k_codes,
                             int8_t* v_codes, void* scales_f16, void* stream) {
  g_err.clear();
  if (head_dim != H3A_HEAD_DIM) return fail(H3A_EUNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  if (n_tokens > 0 && (k == nullptr || v == nullptr)) return fail(H3A_EINVAL, "k and v must both be given");
  void* v_scales = scales_f16 == nullptr ? nullptr
                                         : static_cast<char*>(scales_f16) + (size_t)s_total * (size_t)n_heads * 2;
  return kv_quantize(k, v, x_token_stride, n_tokens, n_heads, head_dim, token_offset, s_total, k_codes, v_codes,
                     scales_f16, v_scales, false, stream);
}

size_t h3a_attention_workspace_bytes(int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim, int64_t q_chunk,
                                     int32_t mode, int32_t sparse) {
  if (head_dim != H3A_HEAD_DIM || n_heads < 1 || s_kv < 0) return 0;
  const bool sol = (mode & H3A_SOL) != 0;
  mode &= ~(H3A_SOL | H3A_OUT_F16);
  if ((mode != H3A_MODE_EXACT_BF16 && mode != H3A_MODE_KVI8R && mode != H3A_MODE_KVI8R32) || (sol && !sparse))
    return 0;
  WorkspaceLayout w;
  if (!workspace_layout(s_q, s_kv, n_heads, q_chunk, mode, sparse != 0, sol, &w)) return 0;
  return (size_t)w.total;
}

int32_t h3a_attention(const void* q, const void* k_store, const void* v_store, const void* scales, int64_t s_q,
                      int64_t s_kv, int32_t n_heads, int32_t head_dim, float softmax_scale, int64_t q_chunk,
                      int64_t kv_block, int32_t mode, const uint8_t* tile_mask, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return attention_call(q, k_store, v_store, scales, s_q, s_kv, n_heads, head_dim, softmax_scale, q_chunk, kv_block,
                        mode, tile_mask, out, workspace, workspace_bytes, false, stream);
}

int32_t h3a_attention_noalloc(const void* q, const void* k_store, const void* v_store, const void* scales,
                              int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim, float softmax_scale,
                              int64_t q_chunk, int64_t kv_block, int32_t mode, const uint8_t* tile_mask, void* out,
                              void* stream) {
  return attention_call(q, k_store, v_store, scales, s_q, s_kv, n_heads, head_dim, softmax_scale, q_chunk, kv_block,
                        mode, tile_mask, out, nullptr, 0, true, stream);
}

int32_t h3a_attention_routed(const void* q, const void* k_bf16, const void* v_bf16, const void* k_codes,
                             const void* v_codes, const void* scales, int64_t s_q, int64_t s_kv, int32_t n_heads,
                             int32_t head_dim, float softmax_scale, int64_t q_chunk, int64_t kv_block,
                             const int64_t* exact_spans, int32_t n_spans, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (head_dim != H3A_HEAD_DIM) return fail(H3A_EUNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  int rc;
  if ((rc = check_shapes(s_q, s_kv, n_heads, q_chunk, kv_block, softmax_scale)) != H3A_OK) return rc;
  if (n_spans < 0 || (n_spans > 0 && exact_spans == nullptr))
    return fail(H3A_EINVAL, "exact_spans must hold n_spans >= 0 [begin, end) pairs");
  int64_t prev_end = 0;
  for (int32_t i = 0; i < n_spans; ++i) {
    const int64_t b = exact_spans[2 * i], e = exact_spans[2 * i + 1];
    if (!(prev_end <= b && b <= e && e <= s_q))
      return fail(H3A_EINVAL, "exact span %d [%lld, %lld) is out of order or outside [0, s_q = %lld]", i,
                  (long long)b, (long long)e, (long long)s_q);
    prev_end = e;
  }
  if (scales == nullptr && s_kv > 0) return fail(H3A_EINVAL, "the kvi8r store needs scales");
  if (s_q == 0) return H3A_OK;
  if ((rc = check_rows(q, out, s_q, n_heads)) != H3A_OK) return rc;
  if ((rc = check_store(H3A_MODE_EXACT_BF16, k_bf16, v_bf16, nullptr, s_kv, n_heads, "k_bf16", "v_bf16")) != H3A_OK)
    return rc;
  if ((rc = check_store(H3A_MODE_KVI8R, k_codes, v_codes, scales, s_kv, n_heads, "k_codes", "v_codes")) != H3A_OK)
    return rc;
  WorkspaceLayout wl;
  if (!workspace_layout(s_q, s_kv, n_heads, q_chunk, H3A_MODE_KVI8R, false, false, &wl))
    return fail(H3A_EINVAL, "size overflow");
  if ((rc = check_workspace(workspace, workspace_bytes, wl)) != H3A_OK) return rc;

  char* ws = static_cast<char*>(workspace);
  const Pass exact = make_pass(H3A_MODE_EXACT_BF16, q, out, k_bf16, v_bf16, nullptr, s_q, s_kv, n_heads,
                               softmax_scale, q_chunk, ws, wl, stream);
  const Pass quant = make_pass(H3A_MODE_KVI8R, q, out, k_codes, v_codes, scales, s_q, s_kv, n_heads,
                               softmax_scale, q_chunk, ws, wl, stream);
  // Rows in increasing order: the kvi8r stretch before each span, then the span.
  int64_t r = 0;
  for (int32_t i = 0; i <= n_spans; ++i) {
    const int64_t b = i < n_spans ? exact_spans[2 * i] : s_q, e = i < n_spans ? exact_spans[2 * i + 1] : s_q;
    if ((rc = attend_rows(quant, r, b)) != H3A_OK) return rc;
    if ((rc = attend_rows(exact, b, e)) != H3A_OK) return rc;
    r = e;
  }
  return H3A_OK;
}

size_t h3a_attention_host_kv_workspace_bytes(int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim,
                                             int64_t q_chunk, int64_t kv_block, int32_t mode) {
  if (head_dim != H3A_HEAD_DIM || n_heads < 1 || s_kv < 0 || kv_block < 0 || kv_block % H3A_TILE != 0) return 0;
  mode &= ~H3A_OUT_F16;
  if (mode != H3A_MODE_EXACT_BF16 && mode != H3A_MODE_KVI8R && mode != H3A_MODE_KVI8R32) return 0;
  StagedLayout w;
  if (!staged_layout(s_q, s_kv, n_heads, q_chunk, kv_block, mode, &w)) return 0;
  return (size_t)w.total;
}

int32_t h3a_attention_host_kv(const void* q, const void* k_host, const void* v_host, const void* scales_host,
                              int64_t s_q, int64_t s_kv, int32_t n_heads, int32_t head_dim, float softmax_scale,
                              int64_t q_chunk, int64_t kv_block, int32_t mode, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (head_dim != H3A_HEAD_DIM) return fail(H3A_EUNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  const bool out_f16 = (mode & H3A_OUT_F16) != 0;
  const int32_t mode_arg = mode;
  mode &= ~H3A_OUT_F16;
  if (mode != H3A_MODE_EXACT_BF16 && mode != H3A_MODE_KVI8R && mode != H3A_MODE_KVI8R32)
    return fail(H3A_EINVAL, "unknown mode %d", mode_arg);
  if (out_f16 && mode == H3A_MODE_EXACT_BF16)
    return fail(H3A_EINVAL, "H3A_OUT_F16 applies to the kvi8r stores; the exact store's output is bf16");
  int rc;
  if ((rc = check_shapes(s_q, s_kv, n_heads, q_chunk, kv_block, softmax_scale)) != H3A_OK) return rc;
  if ((rc = check_mode_scale(mode, softmax_scale)) != H3A_OK) return rc;
  if (mode != H3A_MODE_EXACT_BF16 && scales_host == nullptr && s_kv > 0)
    return fail(H3A_EINVAL, "kvi8r modes need scales");
  if (mode == H3A_MODE_EXACT_BF16 && scales_host != nullptr) return fail(H3A_EINVAL, "exact mode takes no scales");
  if (s_q == 0) return H3A_OK;
  if ((rc = check_rows(q, out, s_q, n_heads)) != H3A_OK) return rc;
  const int64_t g = mode == H3A_MODE_KVI8R32 ? 4 : 1;
  int64_t n_kv;
  if (!mul_ok(s_kv, (int64_t)n_heads * H3A_HEAD_DIM, &n_kv)) return fail(H3A_EINVAL, "size overflow");
  const uint64_t kv_bytes = (uint64_t)n_kv * (mode == H3A_MODE_EXACT_BF16 ? 2 : 1);
  if ((rc = check_host_buffer(k_host, kv_bytes, "k_host")) != H3A_OK) return rc;
  if ((rc = check_host_buffer(v_host, kv_bytes, "v_host")) != H3A_OK) return rc;
  if (mode != H3A_MODE_EXACT_BF16 &&
      (rc = check_host_buffer(scales_host, (uint64_t)s_kv * n_heads * g * 4, "scales_host")) != H3A_OK)
    return rc;
  StagedLayout wl;
  if (!staged_layout(s_q, s_kv, n_heads, q_chunk, kv_block, mode, &wl)) return fail(H3A_EINVAL, "size overflow");
  if (wl.total > 0) {
    if (workspace == nullptr || workspace_bytes < wl.total)
      return fail(H3A_EWORKSPACE, "workspace needs %llu bytes (got %llu)", (unsigned long long)wl.total,
                  (unsigned long long)(workspace == nullptr ? 0 : workspace_bytes));
    if ((rc = check_buffer(workspace, wl.total, 256, "workspace")) != H3A_OK) return rc;
  }

  char* ws = static_cast<char*>(workspace);
  Pass p = make_pass(mode, q, out, nullptr, nullptr, nullptr, s_q, s_kv, n_heads, softmax_scale, q_chunk, ws,
                     wl.base, stream);
  p.out_f16 = out_f16;
  if (s_kv == 0) return attend_rows(p, 0, s_q);  // no K/V: every row is zero

  hipStream_t cs;
  hipError_t e;
  if ((e = copy_stream(&cs)) != hipSuccess) return hip_fail(e, "copy stream");
  // ready: the caller's earlier work on `stream` (which may still use the workspace);
  // copied[i] / freed[i]: block buffer i filled / released by its kernel.
  hipEvent_t ready = nullptr, copied[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr};
  auto destroy = [&]() {
    for (hipEvent_t ev : {ready, copied[0], copied[1], freed[0], freed[1]})
      if (ev) (void)hipEventDestroy(ev);
  };
  for (hipEvent_t* ev : {&ready, &copied[0], &copied[1], &freed[0], &freed[1]})
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) {
      destroy();
      return hip_fail(e, "hipEventCreate");
    }
  int status = H3A_OK;
  auto check = [&](hipError_t err, const char* what) {
    if (err != hipSuccess && status == H3A_OK) status = hip_fail(err, what);
    return status == H3A_OK;
  };
  if (check(hipEventRecord(ready, p.st), "hipEventRecord")) check(hipStreamWaitEvent(cs, ready, 0), "wait");

  const char* kh = static_cast<const char*>(k_host);
  const char* vh = static_cast<const char*>(v_host);
  const char* sh = static_cast<const char*>(scales_host);
  float* state = reinterpret_cast<float*>(ws + wl.state);
  const int64_t blk = wl.blk_rows, n_blk = (s_kv + blk - 1) / blk;
  int64_t k = 0;  // blocks streamed so far in this call
  for (int64_t c0 = 0; c0 < s_q && status == H3A_OK; c0 += q_chunk) {
    const int64_t rows = (s_q - c0) < q_chunk ? (s_q - c0) : q_chunk;
    const int64_t off = c0 * n_heads * H3A_HEAD_DIM;
    h3a::AttnChunk a{};
    a.rows = rows;
    a.n_heads = n_heads;
    a.scale_log2 = p.scale_log2;
    if (mode != H3A_MODE_EXACT_BF16) {
      uint16_t* qrot = reinterpret_cast<uint16_t*>(ws + wl.base.qrot);
      if (!check(h3a::launch_rotate_q(p.q + off, qrot, rows * n_heads, q_post(mode, p.scale_log2), p.st),
                 "rotate_q launch"))
        break;
      a.q = qrot;
      a.out = ws + wl.base.orot;
    } else {
      a.q = p.q + off;
      a.out = p.out + off;
    }
    for (int64_t j = 0; j < n_blk && status == H3A_OK; ++j, ++k) {
      const int slot = (int)(k & 1);
      const int64_t t0 = j * blk, bl = (s_kv - t0) < blk ? (s_kv - t0) : blk;
      char* bk = ws + wl.blk[slot];
      char* bv = bk + wl.k_bytes;
      char* bks = bv + wl.k_bytes;
      char* bvs = bks + wl.s_bytes;
      if (k >= 2 && !check(hipStreamWaitEvent(cs, freed[slot], 0), "wait")) break;
      if (mode == H3A_MODE_EXACT_BF16) {  // token-major: a block is one contiguous range
        const size_t nb = (size_t)bl * n_heads * H3A_HEAD_DIM * 2, o = (size_t)t0 * n_heads * H3A_HEAD_DIM * 2;
        check(hipMemcpyAsync(bk, kh + o, nb, hipMemcpyHostToDevice, cs), "K block copy");
        check(hipMemcpyAsync(bv, vh + o, nb, hipMemcpyHostToDevice, cs), "V block copy");
      } else {  // head-major: one strided row of bl tokens per head
        const size_t w = (size_t)bl * H3A_HEAD_DIM, sp = (size_t)s_kv * H3A_HEAD_DIM, o = (size_t)t0 * H3A_HEAD_DIM;
        check(hipMemcpy2DAsync(bk, w, kh + o, sp, w, n_heads, hipMemcpyHostToDevice, cs), "K block copy");
        check(hipMemcpy2DAsync(bv, w, vh + o, sp, w, n_heads, hipMemcpyHostToDevice, cs), "V block copy");
        const size_t ws2 = (size_t)bl * g * 2, ss = (size_t)s_kv * g * 2, so = (size_t)t0 * g * 2;
        const size_t vso = (size_t)s_kv * n_heads * g * 2;  // V scales follow the K scales
        check(hipMemcpy2DAsync(bks, ws2, sh + so, ss, ws2, n_heads, hipMemcpyHostToDevice, cs), "K scale copy");
        check(hipMemcpy2DAsync(bvs, ws2, sh + vso + so, ss, ws2, n_heads, hipMemcpyHostToDevice, cs),
              "V scale copy");
      }
      if (!check(hipEventRecord(copied[slot], cs), "hipEventRecord")) break;
      if (!check(hipStreamWaitEvent(p.st, copied[slot], 0), "wait")) break;
      a.k = bk;
      a.v = bv;
      a.k_scale = reinterpret_cast<const uint16_t*>(bks);
      a.v_scale = reinterpret_cast<const uint16_t*>(bvs);
      a.s_kv = bl;
      a.state_in = j == 0 ? nullptr : state;
      a.state_out = j + 1 == n_blk ? nullptr : state;
      LaunchTimer timer;
      if (p.timing && !check(timer.begin(p.st), "timing event")) break;
      if (!check(h3a::launch_attn_fwd_block(mode, a, p.st), "attn_fwd launch")) break;
      if (p.timing && !check(timer.end(p.st), "timing event")) break;
      if (!check(hipEventRecord(freed[slot], p.st), "hipEventRecord")) break;
    }
    if (status == H3A_OK && mode != H3A_MODE_EXACT_BF16)
      check(h3a::launch_unrotate_o(reinterpret_cast<const float*>(ws + wl.base.orot), p.out + off, rows * n_heads,
                                   p.out_f16, p.st),
            "unrotate_o launch");
  }
  destroy();
  return status;
}

int32_t h3a_rotate_rows(const void* x_bf16, void* y_f16, int64_t n_rows, void* stream) {
  g_err.clear();
  if (n_rows < 0 || n_rows > ((int64_t)1 << 40)) return fail(H3A_EINVAL, "n_rows out of range");
  if (n_rows == 0) return H3A_OK;
  int rc;
  if ((rc = check_buffer(x_bf16, (uint64_t)n_rows * 256, 16, "x")) != H3A_OK) return rc;
  if ((rc = check_buffer(y_f16, (uint64_t)n_rows * 256, 16, "y")) != H3A_OK) return rc;
  hipError_t e = h3a::launch_rotate_q(static_cast<const uint16_t*>(x_bf16), static_cast<uint16_t*>(y_f16), n_rows, 1.0f,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3A_OK : hip_fail(e, "rotate_q launch");
}

int32_t h3a_unrotate_rows(const float* x_f32, void* y_bf16, int64_t n_rows, void* stream) {
  g_err.clear();
  if (n_rows < 0 || n_rows > ((int64_t)1 << 40)) return fail(H3A_EINVAL, "n_rows out of range");
  if (n_rows == 0) return H3A_OK;
  int rc;
  if ((rc = check_buffer(x_f32, (uint64_t)n_rows * 512, 16, "x")) != H3A_OK) return rc;
  if ((rc = check_buffer(y_bf16, (uint64_t)n_rows * 256, 16, "y")) != H3A_OK) return rc;
  hipError_t e =
      h3a::launch_unrotate_o(x_f32, static_cast<uint16_t*>(y_bf16), n_rows, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H3A_OK : hip_fail(e, "unrotate_o launch");
}

int32_t h3a_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = on != 0;
  return H3A_OK;
}

int32_t h3a_timing_collect_kernel(int32_t kind, double* ms, int64_t* launches) {
  g_err.clear();
  if (kind < 0 || kind >= kTimingKinds) return fail(H3A_EINVAL, "unknown timing kind %d", kind);
  std::vector<std::pair<hipEvent_t, hipEvent_t>> evs;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    evs.swap(g_events[kind]);
  }
  double total = 0.0;
  int rc = H3A_OK;
  for (auto& p : evs) {
    float t = 0.0f;
    hipError_t e = hipEventSynchronize(p.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, p.first, p.second);
    if (e != hipSuccess && rc == H3A_OK) rc = hip_fail(e, "kernel timing");
    total += t;
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  if (ms) *ms = total;
  if (launches) *launches = (int64_t)evs.size();
  return rc;
}

int32_t h3a_timing_collect(double* attn_ms, int64_t* attn_launches) {
  return h3a_timing_collect_kernel(H3A_TIMING_ATTENTION, attn_ms, attn_launches);
}

}  // extern "C"
