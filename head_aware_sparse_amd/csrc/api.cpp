// C ABI of libhas.so: host-side validation, workspace carving and launch
// sequencing.  Every check runs before the first HIP call, so an invalid
// argument returns without touching the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "has.h"
#include "internal.h"
#include "label.h"

// Scratch of sparse_decode_step_noalloc: one fixed device array per GPU the
// library runs on, allocated with the code object and held until the
// process ends.  Host code never passes this name to a kernel (on the host
// it is only a stand-in for the device symbol); it uses the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[HAS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

has_status fail(has_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

has_status ok() {
  g_err[0] = '\0';
  return HAS_OK;
}

has_status hip_fail(hipError_t e, const char* what) {
  return fail(HAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int pow2_floor(long long v) {
  int p = 1;
  while ((long long)p * 2 <= v && p < (1 << 30)) p *= 2;
  return p;
}

int clampi(long long v, int lo, int hi) { return (int)(v < lo ? lo : (v > hi ? hi : v)); }

int esize(int dt) { return dt == HAS_BF16 ? 2 : 4; }

int kdom_elems(int n_dom, int dt) {
  const int bytes = 2 * n_dom * esize(dt);
  int vecs = 1;
  while (vecs * 16 < bytes) vecs *= 2;
  return vecs * 16 / esize(dt);
}

// Validates a decode shape.  clsa selects the shared-index limits; a call
// that ignores the streaming (n_sink, window) or dominant-chunk (n_dom,
// rope_layout) fields says so and they are not checked.
has_status check_dims(const has_decode_dims* d, bool clsa, bool uses_stream = true, bool uses_dom = true) {
  if (!d) return fail(HAS_ERR_INVALID_ARG, "dims is NULL");
  if (d->n_layers < 1 || d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(HAS_ERR_INVALID_ARG, "n_layers, batch, n_q_heads and n_kv_heads must be >= 1");
  if (d->n_q_heads % d->n_kv_heads)
    return fail(HAS_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(HAS_ERR_UNSUPPORTED, "group size %d not in {1,2,4,8}", G);
  if (d->d_head < 2 || (d->d_head & 1)) return fail(HAS_ERR_INVALID_ARG, "d_head must be even and >= 2");
  if (d->d_head != 64 && d->d_head != 128) return fail(HAS_ERR_UNSUPPORTED, "d_head %d not in {64,128}", d->d_head);
  if (d->ctx_len < 1) return fail(HAS_ERR_INVALID_ARG, "ctx_len must be >= 1");
  if (d->ctx_len > has::kMaxTipChunks * 4096)
    return fail(HAS_ERR_UNSUPPORTED, "ctx_len %d above %d", d->ctx_len, has::kMaxTipChunks * 4096);
  if (d->n_fac < 1 || d->n_fac > d->ctx_len)
    return fail(HAS_ERR_INVALID_ARG, "n_fac %d outside [1, ctx_len=%d]", d->n_fac, d->ctx_len);
  if (uses_stream) {
    if (d->n_sink < 0 || d->window < 0) return fail(HAS_ERR_INVALID_ARG, "n_sink and window must be >= 0");
    if ((long long)d->n_sink + d->window < 1) return fail(HAS_ERR_INVALID_ARG, "n_sink + window must be >= 1");
  }
  if (uses_dom) {
    if (d->n_dom < 1 || d->n_dom > d->d_head / 2)
      return fail(HAS_ERR_INVALID_ARG, "n_dom %d outside [1, d_head/2]", d->n_dom);
    if (d->rope_layout != HAS_ROPE_ROTATE_HALF && d->rope_layout != HAS_ROPE_INTERLEAVED)
      return fail(HAS_ERR_INVALID_ARG, "bad rope_layout");
  }
  if (d->kv_dtype != HAS_F32 && d->kv_dtype != HAS_BF16) return fail(HAS_ERR_INVALID_ARG, "bad kv_dtype");
  // the scoring kernels hold a dominant-key row in at most 16 lanes of 16
  // bytes: 2 n_dom channels of at most 256 bytes (always so for bf16)
  if (uses_dom && 2 * d->n_dom * esize(d->kv_dtype) > 256)
    return fail(HAS_ERR_UNSUPPORTED, "n_dom %d: 2 n_dom fp32 channels exceed the 256-byte dominant-key row (n_dom <= 32)",
                d->n_dom);
  if ((long long)d->n_layers * d->n_kv_heads > has::kMaxPairs)
    return fail(HAS_ERR_UNSUPPORTED, "n_layers * n_kv_heads above %d", has::kMaxPairs);
  (void)clsa;
  return HAS_OK;
}

struct Layout {
  has::Geo g;
  size_t off_plan, off_hist, off_info, off_cand, off_ngt, off_off, off_thr, off_scores, off_idx, off_part, off_skeys, off_tau,
      off_qbar;
  size_t bytes;
};

Layout make_layout(const has_decode_dims* d, bool clsa) {
  Layout L{};
  has::Geo& g = L.g;
  g.Lq = d->n_layers;
  g.Lkv = clsa ? 1 : d->n_layers;
  g.B = d->batch;
  g.Hq = d->n_q_heads;
  g.Hkv = d->n_kv_heads;
  g.G = g.Hq / g.Hkv;
  g.d = d->d_head;
  g.T = d->ctx_len;
  g.n_fac = d->n_fac;
  g.n_sink = d->n_sink;
  g.window = d->window;
  g.n_dom = d->n_dom;
  g.R = kdom_elems(d->n_dom, d->kv_dtype);
  g.bf16 = d->kv_dtype == HAS_BF16;
  g.clsa = clsa ? 1 : 0;
  g.interleaved = d->rope_layout == HAS_ROPE_INTERLEAVED;
  g.tstride = d->ctx_len;
  g.kv_shift = 0;
  g.hkv_kv = g.Hkv;
  g.sgrp = 1;
  const long long n_idx = (long long)(clsa ? g.Hkv : g.Lq * g.Hkv) * g.B;
  const long long n_att = (long long)g.Lq * g.Hkv * g.B;
  // Score chunks: aim for ~1024 units over the worst-case item count.
  g.ct = clampi(pow2_floor((long long)g.T * n_idx / 1024), 256, 4096);
  while ((g.T + g.ct - 1) / g.ct > has::kMaxTipChunks && g.ct < 4096) g.ct *= 2;
  g.nch_t = (g.T + g.ct - 1) / g.ct;
  g.Ts = (g.T + 63) / 64 * 64;
  // the matrix cores pay off once several layers' queries share each
  // gathered row; a single layer's G heads go faster on the vector ALUs
  g.clsa_mfma = clsa && g.bf16 && g.d == 128 && g.Lq >= 2 && g.Lq * g.G <= 32;
  g.s_end = g.n_sink < g.T ? g.n_sink : g.T;
  g.w_start = (g.T - g.window) > g.s_end ? (g.T - g.window) : g.s_end;
  g.n_srows = g.s_end + (g.T - g.w_start);
  g.cs = clampi(pow2_floor((long long)g.n_srows * n_att / 2048), 128, has::kMaxChunkRows);
  g.nch_s = (g.n_srows + g.cs - 1) / g.cs;
  g.cs = (g.n_srows + g.nch_s - 1) / g.nch_s;  // equal chunks (no short tail)
  // Prefiltered selection: a sample of kSampleTokens scores places a key
  // threshold expected to pass about 1.25 n_fac tokens plus 4 standard
  // deviations of the sampled count; used when that fits the kCandFast
  // candidate slots comfortably: the expected count within 80% of them, and
  // beyond kShortMaxT tokens n_fac within the kSelMaxLong words that the
  // final kernel keeps for the selected tokens beside its token bitmap.
  {
    const double S = has::kSampleTokens, p = (double)g.n_fac / g.T;
    const double r = 1.25 * S * p + 4.0 * std::sqrt(S * p) + 16.0;
    g.samp_rank = (int)std::ceil(r);
    const bool fits = std::ceil(r) / S * g.T <= 0.8 * has::kCandFast &&
                      (g.T <= has::kShortMaxT || g.n_fac <= has::kSelMaxLong);
    g.prefilter = (g.T >= 2 * has::kSampleTokens && g.T <= has::kPrefilterMaxT && fits &&
                   g.samp_rank < has::kSampleTokens / 2) ? 1 : 0;
  }
  g.cand_cap = g.prefilter ? has::kCandFast : (g.T < has::kCandLds ? g.T : has::kCandLds);
  // The shared-index attention units find their item's cut themselves when
  // the token bitmap fits their LDS beside the expected candidates (at most
  // 70% of the slots they hold; more are read from global memory).
  {
    const double expect = (double)g.samp_rank / has::kSampleTokens * g.T;
    g.fuse_sel = (g.clsa_mfma && g.prefilter && g.T <= has::kShortMaxT && g.n_fac < 65536 &&
                  expect <= 0.7 * has::kFusedSelCand) ? 1 : 0;
  }
  // retrieval chunks: the shared-index units' LDS tiles (kFusedRows when they
  // also select), else about 2048 units over the worst-case item count
  g.cf = g.fuse_sel ? has::kFusedRows
       : g.clsa_mfma ? has::kClsaRows
                     : clampi(pow2_floor((long long)g.n_fac * n_att / 2048), 128, has::kMaxChunkRows);
  g.nch_f = (g.n_fac + g.cf - 1) / g.cf;
  g.nparts = g.nch_f > g.nch_s ? g.nch_f : g.nch_s;
  // prefiltered scoring units: about 2048 over the worst-case item count,
  // between 1024 and 16384 tokens (a shared-index step without labels sizes
  // them to whole rounds of the resident scoring workgroups at launch)
  g.ct_tip = clampi(pow2_floor((long long)g.T * n_idx / 2048), 1024, 16384);
  g.nch_tip = (g.T + g.ct_tip - 1) / g.ct_tip;
  g.bm_words = (g.T + 31) / 32;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.off_plan = take(sizeof(int) * (4 + 3 * has::kMaxPairs));
  L.off_hist = take((size_t)n_idx * has::kHistBins * 4);
  L.off_info = take((size_t)n_idx * 16);
  L.off_cand = take((size_t)n_idx * g.cand_cap * 8);
  L.off_ngt = take((size_t)n_idx * g.nch_t * 4);
  L.off_off = take((size_t)n_idx * g.nch_t * 4);
  L.off_thr = take((size_t)n_idx * 8);
  L.off_scores = take((size_t)n_idx * g.Ts * 4);
  L.off_idx = take((size_t)n_idx * g.n_fac * 4);
  L.off_part = take((size_t)n_att * g.nparts * g.G * (g.d + 4) * 4);
  L.off_skeys = take((size_t)n_idx * has::kSampleTokens * 4);
  L.off_tau = take((size_t)n_idx * 8);
  L.off_qbar = take((size_t)n_idx * g.R * 4);
  L.bytes = o;
  return L;
}

void carve(Layout& L, void* ws) {
  char* b = (char*)ws;
  has::Geo& g = L.g;
  g.plan = (int*)(b + L.off_plan);
  g.hist = (uint32_t*)(b + L.off_hist);
  g.info = (uint32_t*)(b + L.off_info);
  g.cand = (uint2*)(b + L.off_cand);
  g.ngt = (uint32_t*)(b + L.off_ngt);
  g.off = (uint32_t*)(b + L.off_off);
  g.thr = (uint2*)(b + L.off_thr);
  g.scores = (float*)(b + L.off_scores);
  g.idx = (int32_t*)(b + L.off_idx);
  g.part = (float*)(b + L.off_part);
  g.skeys = (uint32_t*)(b + L.off_skeys);
  g.tau = (uint2*)(b + L.off_tau);
  g.qbar = (float*)(b + L.off_qbar);
}

// Per-device side stream and fork/join events.  The enqueue sequence that
// uses them is serialised by g_side_mu so concurrent callers cannot
// interleave their event records.
struct SideState {
  int device = -1;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::vector<SideState> g_side;

has_status side_streams(int dev, SideState*& out) {
  for (SideState& st : g_side)
    if (st.device == dev) {
      out = &st;
      return HAS_OK;
    }
  SideState st;
  st.device = dev;
  hipError_t e = hipStreamCreateWithFlags(&st.side, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
  if ((e = hipEventCreateWithFlags(&st.fork, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  if ((e = hipEventCreateWithFlags(&st.join, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  g_side.push_back(st);
  out = &g_side.back();
  return HAS_OK;
}

has_status persistent_grid(int& grid) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  grid = cus * 8;
  return HAS_OK;
}

#define REQUIRE_PTR(p, name)                                                              \
  do {                                                                                    \
    if (!(p)) return fail(HAS_ERR_INVALID_ARG, "%s is NULL", name);                       \
    if (!aligned16(p)) return fail(HAS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

#define OPTIONAL_PTR(p, name)                                                             \
  do {                                                                                    \
    if ((p) && !aligned16(p)) return fail(HAS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

// HAS_DEBUG=1: the array contents the kernels rely on are copied to the
// host (synchronising the stream) and checked before anything is launched.
bool debug_checks() {
  const char* e = std::getenv("HAS_DEBUG");
  return e && e[0] == '1' && e[1] == 0;
}

has_status debug_check_arrays(const has_decode_dims* d, int pairs, const int32_t* i_dom, const uint8_t* labels,
                              int label_pairs, void* stream) {
  std::vector<int32_t> dom((size_t)pairs * d->n_dom);
  std::vector<uint8_t> lab(labels ? (size_t)label_pairs : 0);
  hipError_t e = hipMemcpyAsync(dom.data(), i_dom, dom.size() * 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess && labels)
    e = hipMemcpyAsync(lab.data(), labels, lab.size(), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "HAS_DEBUG copy");
  const int hd = d->d_head / 2;
  std::vector<uint8_t> seen(hd);
  for (int p = 0; p < pairs; ++p) {
    std::fill(seen.begin(), seen.end(), 0);
    for (int i = 0; i < d->n_dom; ++i) {
      const int f = dom[(size_t)p * d->n_dom + i];
      if (f < 0 || f >= hd) return fail(HAS_ERR_INVALID_ARG, "i_dom[%d][%d] = %d outside [0, %d)", p, i, f, hd);
      if (seen[f]++) return fail(HAS_ERR_INVALID_ARG, "i_dom[%d] repeats chunk %d", p, f);
    }
  }
  for (size_t i = 0; i < lab.size(); ++i)
    if (lab[i] > 1) return fail(HAS_ERR_INVALID_ARG, "labels[%zu] = %d is neither 0 nor 1", i, (int)lab[i]);
  return HAS_OK;
}

// One-layer shapes for sparse_select / fac_attend: fields the call does not
// use are replaced by valid placeholders before the layout is built.
has_status one_layer_dims(const has_decode_dims* dims, bool uses_dom, has_decode_dims& out) {
  has_status s = check_dims(dims, true, false, uses_dom);
  if (s != HAS_OK) return s;
  if (dims->n_layers != 1) return fail(HAS_ERR_INVALID_ARG, "n_layers must be 1 (got %d)", dims->n_layers);
  out = *dims;
  out.n_sink = 1;
  out.window = 0;
  if (!uses_dom) {
    out.n_dom = 1;
    out.rope_layout = HAS_ROPE_ROTATE_HALF;
  }
  return HAS_OK;
}

// Workspace of fac_attend: the chunk partials only.
size_t fac_attend_bytes(const Layout& L) {
  const has::Geo& g = L.g;
  return align_up((size_t)g.Lq * g.Hkv * g.B * g.nparts * g.G * (g.d + 4) * 4, 256);
}

has_status debug_check_idx(const has_decode_dims* d, const int32_t* idx, void* stream) {
  std::vector<int32_t> h((size_t)d->batch * d->n_kv_heads * d->n_fac);
  hipError_t e = hipMemcpyAsync(h.data(), idx, h.size() * 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "HAS_DEBUG copy");
  for (size_t i = 0; i < h.size(); ++i)
    if (h[i] < 0 || h[i] >= d->ctx_len)
      return fail(HAS_ERR_INVALID_ARG, "idx[%zu] = %d outside [0, %d)", i, h[i], d->ctx_len);
  return HAS_OK;
}

// The retrieval rows of a split cache (k_ret, v_ret) may live in pinned host
// memory (FASA §2.C, FASA-M: only the dominant-key copy stays in HBM); the
// kernels then reach them over the host link through their device-visible
// address.  Anything but device or pinned host memory is refused: a kernel
// touching pageable or unresident memory would fault.
has_status row_store(const void* p, const char* name, const void*& dev) {
  hipPointerAttribute_t a{};
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // an unregistered pointer: clear the error it leaves
    return fail(HAS_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", name);
  }
  if (a.type == hipMemoryTypeDevice) {
    dev = p;
    return HAS_OK;
  }
  if (a.type == hipMemoryTypeHost) {
    void* d = nullptr;
    const hipError_t e2 = hipHostGetDevicePointer(&d, const_cast<void*>(p), 0);
    if (e2 != hipSuccess) return hip_fail(e2, "hipHostGetDevicePointer");
    dev = d;
    return HAS_OK;
  }
  return fail(HAS_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", name);
}

// Device address of `scratch` on each device, looked up once per device
// with that device current.
struct ScratchAddr {
  int device;
  void* ptr;
};
std::mutex g_scratch_mu;
std::vector<ScratchAddr> g_scratch;

has_status scratch_address(void*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  for (const ScratchAddr& a : g_scratch)
    if (a.device == dev) {
      out = a.ptr;
      return HAS_OK;
    }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (!p || !aligned16(p)) return fail(HAS_ERR_HIP, "scratch has no usable device address on device %d", dev);
  g_scratch.push_back(ScratchAddr{dev, p});
  out = p;
  return HAS_OK;
}

// The split cache of sparse_decode_step_split: slabs of `capacity` rows for
// retrieval groups, rings of n_sink + window rows for streaming groups.
struct SplitCache {
  int capacity;
  const void* k_str;
  const void* v_str;
};

has_status run_decode(const has_decode_dims* dims, bool clsa, const void* q, const void* q_index,
                      const void* k_cache, const void* v_cache, const void* k_dom, const int32_t* i_dom,
                      const uint8_t* labels, float* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                      void* stream, const SplitCache* sc = nullptr, int kv_div = 1, bool static_scratch = false) {
  has_status s = check_dims(dims, clsa);
  if (s != HAS_OK) return s;
  if (sc) {
    if (sc->capacity < dims->ctx_len || sc->capacity > has::kMaxTipChunks * 4096)
      return fail(HAS_ERR_INVALID_ARG, "capacity %d outside [ctx_len=%d, %d]", sc->capacity, dims->ctx_len,
                  has::kMaxTipChunks * 4096);
    REQUIRE_PTR(sc->k_str, "k_str");
    REQUIRE_PTR(sc->v_str, "v_str");
  }
  REQUIRE_PTR(q, "q");
  OPTIONAL_PTR(q_index, "q_index");
  REQUIRE_PTR(k_cache, "k_cache");
  REQUIRE_PTR(v_cache, "v_cache");
  REQUIRE_PTR(k_dom, "k_dom");
  REQUIRE_PTR(i_dom, "i_dom");
  if (!clsa) REQUIRE_PTR(labels, "labels");
  OPTIONAL_PTR(labels, "labels");
  REQUIRE_PTR(out, "out");
  OPTIONAL_PTR(idx_out, "idx_out");
  Layout L = make_layout(dims, clsa);
  if (static_scratch) {
    // sparse_decode_step_noalloc: the fixed per-device array stands in for ws
    if (L.bytes > (size_t)HAS_NOALLOC_SCRATCH_BYTES)
      return fail(HAS_ERR_WORKSPACE,
                  "sparse_decode_step_noalloc: these dims need %zu bytes of scratch, above the fixed %zu; "
                  "call sparse_decode_step with a workspace instead",
                  L.bytes, (size_t)HAS_NOALLOC_SCRATCH_BYTES);
    if ((s = scratch_address(ws)) != HAS_OK) return s;
    ws_bytes = (size_t)HAS_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws) return fail(HAS_ERR_WORKSPACE, "ws is NULL");
  if (!aligned16(ws)) return fail(HAS_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  if (ws_bytes < L.bytes) return fail(HAS_ERR_WORKSPACE, "ws_bytes %zu < required %zu", ws_bytes, L.bytes);
  carve(L, ws);
  has::Geo& g = L.g;
  g.q = q;
  g.q_index = q_index;
  g.k = k_cache;
  g.v = v_cache;
  g.kdom = k_dom;
  g.i_dom = i_dom;
  g.labels = labels;
  g.host_plan = (clsa && labels == nullptr && g.prefilter) ? 1 : 0;
  g.out = out;
  g.idx_out = idx_out;
  if (sc) {
    g.split = 1;
    g.tstride = sc->capacity;
    g.scap = dims->n_sink + dims->window;
    g.k_str = sc->k_str;
    g.v_str = sc->v_str;
  }
  // kv_div is the group size G, a power of two
  g.kv_shift = kv_div == 8 ? 3 : kv_div == 4 ? 2 : kv_div == 2 ? 1 : 0;
  g.hkv_kv = g.Hkv >> g.kv_shift;
  if (debug_checks()) {
    const int kv_heads = dims->n_kv_heads / kv_div;
    s = debug_check_arrays(dims, clsa ? kv_heads : dims->n_layers * kv_heads, i_dom, labels,
                           dims->n_layers * kv_heads, stream);
    if (s != HAS_OK) return s;
  }
  if (sc) {
    if ((s = row_store(k_cache, "k_ret", g.k)) != HAS_OK) return s;
    if ((s = row_store(v_cache, "v_ret", g.v)) != HAS_OK) return s;
  }
  s = persistent_grid(g.grid);
  if (s != HAS_OK) return s;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideState* st = nullptr;
  s = side_streams(dev, st);
  if (s != HAS_OK) return s;
  e = has::launch_decode(g, has::StreamSet{(hipStream_t)stream, st->side, st->fork, st->join});
  if (e != hipSuccess) return hip_fail(e, clsa ? "shared_index_decode launch" : "sparse_decode_step launch");
  return ok();
}

// Per-kernel event timing (diagnostics).
struct TimerRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimerRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace has {

KTimer::KTimer(const char* name, hipStream_t s) : slot(-1), stream(s) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing) return;
  TimerRec r{name, take_event(), take_event()};
  if (!r.a || !r.b) return;
  if (hipEventRecord(r.a, s) != hipSuccess) return;
  slot = (int)g_recs.size();
  g_recs.push_back(r);
}

KTimer::~KTimer() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (slot < (int)g_recs.size()) (void)hipEventRecord(g_recs[slot].b, stream);
}

}  // namespace has

extern "C" {

has_status has_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
  return ok();
}

int has_timing_collect(const char** names, double* total_ms, int* launches, int max) {
  std::lock_guard<std::mutex> lk(g_tmu);
  int n = 0;
  int rc = 0;
  for (const TimerRec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = -1;
    int k = 0;
    while (k < n && strcmp(names[k], r.name) != 0) ++k;
    if (k == n && n < max) {
      names[n] = r.name;
      total_ms[n] = 0.0;
      launches[n] = 0;
      ++n;
    }
    if (k < n) {
      total_ms[k] += ms;
      launches[k] += 1;
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  if (rc < 0) {
    fail(HAS_ERR_HIP, "timing events failed");
    return -1;
  }
  return n;
}

const char* has_status_string(has_status s) {
  switch (s) {
    case HAS_OK: return "HAS_OK";
    case HAS_ERR_INVALID_ARG: return "HAS_ERR_INVALID_ARG";
    case HAS_ERR_UNSUPPORTED: return "HAS_ERR_UNSUPPORTED";
    case HAS_ERR_WORKSPACE: return "HAS_ERR_WORKSPACE";
    case HAS_ERR_HIP: return "HAS_ERR_HIP";
    default: return "HAS_ERR_UNKNOWN";
  }
}

const char* has_last_error(void) { return g_err; }

int kdom_row_elems(const has_decode_dims* dims) {
  if (check_dims(dims, false) != HAS_OK) return -1;
  return kdom_elems(dims->n_dom, dims->kv_dtype);
}

has_status kdom_pack(const has_decode_dims* dims, const void* k_cache, const int32_t* i_dom, void* k_dom,
                     void* stream) {
  has_status s = check_dims(dims, false);
  if (s != HAS_OK) return s;
  REQUIRE_PTR(k_cache, "k_cache");
  REQUIRE_PTR(i_dom, "i_dom");
  REQUIRE_PTR(k_dom, "k_dom");
  Layout L = make_layout(dims, false);
  L.g.k = k_cache;
  L.g.i_dom = i_dom;
  if (debug_checks()) {
    s = debug_check_arrays(dims, dims->n_layers * dims->n_kv_heads, i_dom, nullptr, 0, stream);
    if (s != HAS_OK) return s;
  }
  s = persistent_grid(L.g.grid);
  if (s != HAS_OK) return s;
  hipError_t e = has::launch_kdom_pack(L.g, k_dom, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kdom_pack launch");
  return ok();
}

size_t sparse_decode_workspace(const has_decode_dims* dims) {
  if (check_dims(dims, false) != HAS_OK) return 0;
  return make_layout(dims, false).bytes;
}

int sparse_selection_path(const has_decode_dims* dims) {
  if (check_dims(dims, false) != HAS_OK) return -1;
  return make_layout(dims, false).g.prefilter;
}

has_status sparse_decode_step(const has_decode_dims* dims, const void* q, const void* k_cache,
                              const void* v_cache, const void* k_dom, const int32_t* i_dom,
                              const uint8_t* labels, float* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                              void* stream) {
  return run_decode(dims, false, q, nullptr, k_cache, v_cache, k_dom, i_dom, labels, out, idx_out, ws,
                    ws_bytes, stream);
}

has_status sparse_decode_step_noalloc(const has_decode_dims* dims, const void* q, const void* k_cache,
                                      const void* v_cache, const void* k_dom, const int32_t* i_dom,
                                      const uint8_t* labels, float* out, int32_t* idx_out, void* stream) {
  return run_decode(dims, false, q, nullptr, k_cache, v_cache, k_dom, i_dom, labels, out, idx_out, nullptr, 0,
                    stream, nullptr, 1, true);
}

size_t sparse_decode_per_head_workspace(const has_decode_dims* dims) {
  if (check_dims(dims, false) != HAS_OK) return 0;
  has_decode_dims v = *dims;
  v.n_kv_heads = dims->n_q_heads;  // one index group per query head
  return make_layout(&v, false).bytes;
}

has_status sparse_decode_step_per_head(const has_decode_dims* dims, const void* q, const void* k_cache,
                                       const void* v_cache, const void* k_dom, const int32_t* i_dom,
                                       const uint8_t* labels, float* out, int32_t* idx_out, void* ws,
                                       size_t ws_bytes, void* stream) {
  has_status s = check_dims(dims, false);
  if (s != HAS_OK) return s;
  has_decode_dims v = *dims;
  v.n_kv_heads = dims->n_q_heads;
  return run_decode(&v, false, q, nullptr, k_cache, v_cache, k_dom, i_dom, labels, out, idx_out, ws, ws_bytes,
                    stream, nullptr, dims->n_q_heads / dims->n_kv_heads);
}

has_status sparse_decode_step_split(const has_decode_dims* dims, int capacity, const void* q, const void* k_ret,
                                    const void* v_ret, const void* k_dom_ret, const void* k_str, const void* v_str,
                                    const int32_t* i_dom, const uint8_t* labels, float* out, int32_t* idx_out,
                                    void* ws, size_t ws_bytes, void* stream) {
  const SplitCache sc{capacity, k_str, v_str};
  return run_decode(dims, false, q, nullptr, k_ret, v_ret, k_dom_ret, i_dom, labels, out, idx_out, ws, ws_bytes,
                    stream, &sc);
}

has_status kv_append(const has_decode_dims* dims, int capacity, int pos, int n_new, const void* k_new,
                     const void* v_new, const int32_t* i_dom, const uint8_t* labels, void* k_ret, void* v_ret,
                     void* k_dom_ret, void* k_str, void* v_str, void* stream) {
  if (!dims) return fail(HAS_ERR_INVALID_ARG, "dims is NULL");
  // ctx_len and n_fac are not used: the capacity stands in for the length
  has_decode_dims d = *dims;
  d.ctx_len = capacity;
  d.n_fac = 1;
  has_status s = check_dims(&d, false);
  if (s != HAS_OK) return s;
  if (pos < 0 || n_new < 1 || (long long)pos + n_new > capacity)
    return fail(HAS_ERR_INVALID_ARG, "positions [%d, %d + %d) outside [0, capacity=%d)", pos, pos, n_new, capacity);
  REQUIRE_PTR(k_new, "k_new");
  REQUIRE_PTR(v_new, "v_new");
  REQUIRE_PTR(i_dom, "i_dom");
  REQUIRE_PTR(labels, "labels");
  REQUIRE_PTR(k_ret, "k_ret");
  REQUIRE_PTR(v_ret, "v_ret");
  REQUIRE_PTR(k_dom_ret, "k_dom_ret");
  REQUIRE_PTR(k_str, "k_str");
  REQUIRE_PTR(v_str, "v_str");
  Layout L = make_layout(&d, false);
  has::Geo& g = L.g;
  g.i_dom = i_dom;
  g.labels = labels;
  g.tstride = capacity;
  g.scap = d.n_sink + d.window;
  if (debug_checks()) {
    s = debug_check_arrays(&d, d.n_layers * d.n_kv_heads, i_dom, labels, d.n_layers * d.n_kv_heads, stream);
    if (s != HAS_OK) return s;
  }
  const void *k_dev = nullptr, *v_dev = nullptr;
  if ((s = row_store(k_ret, "k_ret", k_dev)) != HAS_OK) return s;
  if ((s = row_store(v_ret, "v_ret", v_dev)) != HAS_OK) return s;
  s = persistent_grid(g.grid);
  if (s != HAS_OK) return s;
  const hipError_t e = has::launch_kv_append(g, pos, n_new, k_new, v_new, const_cast<void*>(k_dev),
                                             const_cast<void*>(v_dev), k_dom_ret, k_str, v_str, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return ok();
}

size_t shared_index_workspace(const has_decode_dims* dims) {
  if (check_dims(dims, true) != HAS_OK) return 0;
  return make_layout(dims, true).bytes;
}

has_status shared_index_decode(const has_decode_dims* dims, const void* q, const void* q_index,
                               const void* k_cache, const void* v_cache, const void* k_dom, const int32_t* i_dom,
                               const uint8_t* labels, float* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                               void* stream) {
  return run_decode(dims, true, q, q_index, k_cache, v_cache, k_dom, i_dom, labels, out, idx_out, ws, ws_bytes,
                    stream);
}

size_t sparse_select_workspace(const has_decode_dims* dims) {
  has_decode_dims d1;
  if (one_layer_dims(dims, true, d1) != HAS_OK) return 0;
  return make_layout(&d1, true).bytes;
}

has_status sparse_select(const has_decode_dims* dims, const void* q_index, const void* k_dom,
                         const int32_t* i_dom, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  has_decode_dims d1;
  has_status s = one_layer_dims(dims, true, d1);
  if (s != HAS_OK) return s;
  REQUIRE_PTR(q_index, "q_index");
  REQUIRE_PTR(k_dom, "k_dom");
  REQUIRE_PTR(i_dom, "i_dom");
  REQUIRE_PTR(idx_out, "idx_out");
  Layout L = make_layout(&d1, true);
  if (!ws) return fail(HAS_ERR_WORKSPACE, "ws is NULL");
  if (!aligned16(ws)) return fail(HAS_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  if (ws_bytes < L.bytes) return fail(HAS_ERR_WORKSPACE, "ws_bytes %zu < required %zu", ws_bytes, L.bytes);
  carve(L, ws);
  has::Geo& g = L.g;
  g.q = q_index;
  g.q_index = q_index;
  g.kdom = k_dom;
  g.i_dom = i_dom;
  g.host_plan = g.prefilter;
  g.idx_out = idx_out;
  g.select_only = 1;
  if (debug_checks()) {
    s = debug_check_arrays(&d1, d1.n_kv_heads, i_dom, nullptr, 0, stream);
    if (s != HAS_OK) return s;
  }
  s = persistent_grid(g.grid);
  if (s != HAS_OK) return s;
  // no streaming groups: the side stream is never used
  const hipError_t e = has::launch_decode(g, has::StreamSet{(hipStream_t)stream, nullptr, nullptr, nullptr});
  if (e != hipSuccess) return hip_fail(e, "sparse_select launch");
  return ok();
}

size_t fac_attend_workspace(const has_decode_dims* dims) {
  has_decode_dims d1;
  if (one_layer_dims(dims, false, d1) != HAS_OK) return 0;
  return fac_attend_bytes(make_layout(&d1, true));
}

has_status fac_attend(const has_decode_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* idx, float* out, void* ws, size_t ws_bytes, void* stream) {
  has_decode_dims d1;
  has_status s = one_layer_dims(dims, false, d1);
  if (s != HAS_OK) return s;
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k_cache, "k_cache");
  REQUIRE_PTR(v_cache, "v_cache");
  REQUIRE_PTR(idx, "idx");
  REQUIRE_PTR(out, "out");
  Layout L = make_layout(&d1, true);
  const size_t need = fac_attend_bytes(L);
  if (!ws) return fail(HAS_ERR_WORKSPACE, "ws is NULL");
  if (!aligned16(ws)) return fail(HAS_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  if (ws_bytes < need) return fail(HAS_ERR_WORKSPACE, "ws_bytes %zu < required %zu", ws_bytes, need);
  has::Geo& g = L.g;
  g.part = (float*)ws;
  g.q = q;
  g.k = k_cache;
  g.v = v_cache;
  g.idx = const_cast<int32_t*>(idx);  // read only: the attention kernels never write it
  g.idx_bmajor = 1;
  g.host_plan = 1;  // one layer, all groups retrieval
  g.out = out;
  if (debug_checks()) {
    s = debug_check_idx(&d1, idx, stream);
    if (s != HAS_OK) return s;
  }
  s = persistent_grid(g.grid);
  if (s != HAS_OK) return s;
  const hipError_t e = has::launch_fac_attend(g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fac_attend launch");
  return ok();
}

size_t aoh_label_workspace(int n_layers, int n_q_heads, int n_kv_heads, int d_model, int d_head) {
  return has::label_workspace_bytes(n_layers, n_q_heads, n_kv_heads, d_model, d_head);
}

has_status aoh_label(int n_layers, int n_q_heads, int n_kv_heads, int d_model, int d_head, has_dtype wdt,
                     const void* w_q, const void* w_k, int n_retrieval, float er_threshold, float* er_head,
                     float* er_group, uint8_t* labels, void* ws, size_t ws_bytes, void* stream) {
  if (n_layers < 1 || n_q_heads < 1 || n_kv_heads < 1 || d_model < 1 || d_head < 1)
    return fail(HAS_ERR_INVALID_ARG, "sizes must be >= 1");
  if (n_q_heads % n_kv_heads)
    return fail(HAS_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", n_q_heads, n_kv_heads);
  if (wdt != HAS_F32 && wdt != HAS_BF16) return fail(HAS_ERR_INVALID_ARG, "bad wdt");
  if (d_head != 64 && d_head != 128) return fail(HAS_ERR_UNSUPPORTED, "d_head %d not in {64,128}", d_head);
  if (d_model < d_head || d_model % 64)
    return fail(HAS_ERR_UNSUPPORTED, "d_model %d must be a multiple of 64 and >= d_head", d_model);
  if ((long long)n_layers * n_kv_heads > has::kMaxPairs || (long long)n_layers * n_q_heads > 65535)
    return fail(HAS_ERR_UNSUPPORTED, "too many heads");
  if (n_retrieval > n_layers * n_kv_heads)
    return fail(HAS_ERR_INVALID_ARG, "n_retrieval %d above n_layers*n_kv_heads", n_retrieval);
  if (n_retrieval < 0 && !(er_threshold == er_threshold))
    return fail(HAS_ERR_INVALID_ARG, "er_threshold is NaN");
  REQUIRE_PTR(w_q, "w_q");
  REQUIRE_PTR(w_k, "w_k");
  OPTIONAL_PTR(er_head, "er_head");
  OPTIONAL_PTR(er_group, "er_group");
  REQUIRE_PTR(labels, "labels");
  const size_t need = has::label_workspace_bytes(n_layers, n_q_heads, n_kv_heads, d_model, d_head);
  if (!ws) return fail(HAS_ERR_WORKSPACE, "ws is NULL");
  if (!aligned16(ws)) return fail(HAS_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  if (ws_bytes < need) return fail(HAS_ERR_WORKSPACE, "ws_bytes %zu < required %zu", ws_bytes, need);
  has::LabelArgs a{n_layers, n_q_heads, n_kv_heads, d_model, d_head, wdt == HAS_BF16, w_q, w_k,
                   n_retrieval, er_threshold, er_head, er_group, labels, ws};
  hipError_t e = has::launch_label(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "aoh_label launch");
  return ok();
}

}  // extern "C"
