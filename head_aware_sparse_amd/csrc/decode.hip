// Decode-step kernels for gfx950: TIP scoring over the dominant-chunk key
// copy, exact radix top-N_fac selection, and split-K attention over gathered
// (retrieval) or contiguous sink+window (streaming) rows.
//
// Method: "FASA: Frequency-aware Sparse Attention" §2.B (TIP, then FAC over
// the selected tokens at their original positions), §2.C (FASA-C: the cache
// stays in device memory and only a sparse subset of it is read);
// "Resumen Técnico: Autonomía de Cabezales (AoH)" §4 (streaming heads: sink
// + recent window); the CLSA article, "Cómo funciona CLSA" (one index reused
// by every layer sharing the cache).
//
// Launch sequences (all on the caller's stream, no host synchronisation;
// launch_decode picks one per call):
//   prefiltered (8192 <= T <= 524288 and the expected candidates fit):
//     plan      labels -> work lists, counters (inside the sampling launch
//               when no side stream is used)
//     [side stream: attn over streaming groups, when they attend to >= 2^20 rows]
//     sample    TIP keys of 4096 evenly spread tokens per item
//     tau       per item: the candidate threshold (inside TIP on smaller steps)
//     tip       scores; only tokens at or above tau are written as candidates
//     final     per item: the exact top-n_fac cut among the candidates,
//               ascending indices (inside the FAC units on small steps, and
//               inside the shared-index attention units)
//     attn      per (item, chunk of rows): logits, softmax partial, P.V
//     merge     log-sum-exp merge of the chunk partials -> out
//   general (other lengths, or too many expected candidates): plan, tip
//     (every score + a first-digit histogram), select_bin, select_a,
//     select_b, select_c (exact radix threshold, ordered compaction), attn,
//     merge.
// Work is split into units (item x chunk) processed by a persistent grid;
// unit counts depend on the labels and are read from device memory.
#include "internal.h"

namespace has {
namespace {

constexpr int NT = 256;  // threads per workgroup for every kernel here
constexpr int NWAVE = NT / 64;

// ------------------------------------------------------------------ helpers
// Order-preserving map of an fp32 score to uint32 (larger key = larger
// score); -0 is folded onto +0 so equal scores have equal keys.
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Lane exchanges across 16-lane rows (gfx950): with both operands equal,
// v_permlane16_swap / v_permlane32_swap return x and the value of lane ^ 16
// (lane ^ 32) as the pair, in some order; their sum or max is the same in
// both lanes of each pair.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned groups of N consecutive lanes; every lane of the group
// receives the total.  quad_perm swaps, half-row and row mirrors, then the
// row exchanges.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x = xor16_sum(x);
  if constexpr (N >= 64) x = xor32_sum(x);
  return x;
}

// Max over aligned groups of N consecutive lanes, as group_sum.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = xor16_max(x);
  if constexpr (N >= 64) x = xor32_max(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) { return group_max<64>(x); }
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix over the workgroup (BT threads; s_w holds BT / 64) and the
// total.
template <int BT = NT>
__device__ int block_excl_scan(int v, int* s_w, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < BT / 64; ++w) {
    const int t = s_w[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  total = tot;
  return base + x - v;
}

// 16-byte vectors of the cache element type.
template <typename E>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void cvt(const uint4& r, float* o) {
    o[0] = __uint_as_float(r.x); o[1] = __uint_as_float(r.y);
    o[2] = __uint_as_float(r.z); o[3] = __uint_as_float(r.w);
  }
  __device__ __forceinline__ static float one(const float* p, size_t i) { return p[i]; }
};
template <>
struct Vec<uint16_t> {  // bf16 bits
  static constexpr int N = 8;
  __device__ __forceinline__ static void cvt(const uint4& r, float* o) {
    o[0] = __uint_as_float(r.x << 16); o[1] = __uint_as_float(r.x & 0xFFFF0000u);
    o[2] = __uint_as_float(r.y << 16); o[3] = __uint_as_float(r.y & 0xFFFF0000u);
    o[4] = __uint_as_float(r.z << 16); o[5] = __uint_as_float(r.z & 0xFFFF0000u);
    o[6] = __uint_as_float(r.w << 16); o[7] = __uint_as_float(r.w & 0xFFFF0000u);
  }
  __device__ __forceinline__ static float one(const uint16_t* p, size_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
  }
};

// s_waitcnt immediate (gfx9 encoding) that waits for every vector memory
// operation: vmcnt 0, expcnt and lgkmcnt at their maxima.
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Streaming (read-once) 16-byte load: nontemporal, so the cache rows and the
// dominant-key copy, each read once per step, do not evict reused data.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer resource word 3 (data format) for raw 32-bit buffer accesses on
// gfx9-family parts, and a streaming 16-byte buffer load (nontemporal).
constexpr int kBufRsrcWord3 = 0x00020000;
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ uint4 buf_load16_stream(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, kCachePolicyNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Index groups are the KV groups, or with kv_shift > 0 the query heads (each
// selecting its own tokens): (layer, index group) pairs and cache slabs map
// to the KV group that holds the rows, i_dom and the label.
__device__ __forceinline__ int kv_pair(const Geo& g, int pair) {
  if (g.kv_shift == 0) return pair;
  const int l = pair / g.Hkv, gi = pair - l * g.Hkv;
  return l * g.hkv_kv + (gi >> g.kv_shift);
}
__device__ __forceinline__ size_t kv_slice(const Geo& g, int l, int b, int gi) {
  return ((size_t)l * g.B + b) * g.hkv_kv + (gi >> g.kv_shift);
}

__device__ __forceinline__ int label_at(const Geo& g, int pair) {
  return g.labels ? (g.labels[kv_pair(g, pair)] != 0) : 1;
}

// Plan accessors: index pairs (one selection each), retrieval and streaming
// (layer, group) pairs for attention.  With a host-known plan (shared-index
// mode without labels) every KV group is an index pair, every (layer, group)
// is retrieval and nothing streams, so no plan launch is needed.
__device__ __forceinline__ int n_idx_pairs(const Geo& g) { return g.host_plan ? g.Hkv : g.plan[0]; }
__device__ __forceinline__ int idx_pair(const Geo& g, int i) { return g.host_plan ? i : g.plan[4 + i]; }
__device__ __forceinline__ int n_ret_pairs(const Geo& g) { return g.host_plan ? g.Lq * g.Hkv : g.plan[1]; }
__device__ __forceinline__ int ret_pair(const Geo& g, int i) { return g.host_plan ? i : g.plan[4 + kMaxPairs + i]; }
__device__ __forceinline__ int n_str_pairs(const Geo& g) { return g.host_plan ? 0 : g.plan[2]; }
__device__ __forceinline__ int str_pair(const Geo& g, int i) { return g.plan[4 + 2 * kMaxPairs + i]; }

// Finds, over s_hist[0..nbins) read from the top bin down, the bin where the
// running count first reaches `need` (1 <= need <= total).  Returns the bin
// and the count strictly above it, identical in every thread.
template <int BT = NT>
__device__ void find_bin_top(const uint32_t* s_hist, int nbins, uint32_t need, int* s_w,
                             uint32_t* s_res, int& bin, uint32_t& above) {
  const int per = nbins / BT;  // nbins is a multiple of BT
  const int tid = threadIdx.x;
  const int hi = nbins - tid * per;  // this thread owns bins [hi - per, hi)
  uint32_t seg = 0;
  for (int i = 1; i <= per; ++i) seg += s_hist[hi - i];
  int total;
  const uint32_t before = (uint32_t)block_excl_scan<BT>((int)seg, s_w, total);
  if (before < need && need <= before + seg) {
    uint32_t run = before;
    for (int i = 1; i <= per; ++i) {
      const uint32_t c = s_hist[hi - i];
      if (run + c >= need) {
        s_res[0] = (uint32_t)(hi - i);
        s_res[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  bin = (int)s_res[0];
  above = s_res[1];
  __syncthreads();
}

// ------------------------------------------------------------------ plan
__global__ __launch_bounds__(NT) void plan_kernel(Geo g) {
  __shared__ int s_w[NWAVE];
  const int P = g.Lq * g.Hkv;
  const int tid = threadIdx.x;
  const int per = (P + NT - 1) / NT;
  const int p0 = min(P, tid * per), p1 = min(P, p0 + per);
  int cnt = 0;
  for (int p = p0; p < p1; ++p) cnt += label_at(g, p);
  int n_ret;
  const int excl = block_excl_scan(cnt, s_w, n_ret);
  const int n_idx_pairs = g.clsa ? g.Hkv : n_ret;
  if (blockIdx.x == 0) {
    int* lists = g.plan + 4;
    int r = excl, s = p0 - excl;
    for (int p = p0; p < p1; ++p) {
      if (label_at(g, p)) {
        if (!g.clsa) lists[r] = p;
        lists[kMaxPairs + r++] = p;
      } else {
        lists[2 * kMaxPairs + s++] = p;
      }
    }
    if (g.clsa)
      for (int gi = tid; gi < g.Hkv; gi += NT) lists[gi] = gi;
    if (tid == 0) {
      g.plan[0] = n_idx_pairs;
      g.plan[1] = n_ret;
      g.plan[2] = P - n_ret;
      g.plan[3] = 0;
    }
  }
  // Clear the histograms and counters of every index item.
  const size_t n_items = (size_t)n_idx_pairs * g.B;
  const size_t gtid = (size_t)blockIdx.x * NT + tid, gstride = (size_t)gridDim.x * NT;
  uint4* h4 = reinterpret_cast<uint4*>(g.hist);
  const size_t nh4 = n_items * kHistBins / 4;
  if (!g.prefilter)
    for (size_t i = gtid; i < nh4; i += gstride) h4[i] = make_uint4(0, 0, 0, 0);
  uint4* i4 = reinterpret_cast<uint4*>(g.info);
  for (size_t i = gtid; i < n_items; i += gstride) i4[i] = make_uint4(0, 0, 0, 0);
  // Streaming groups report -1 indices.
  if (g.idx_out && !g.clsa) {
    const size_t tot = (size_t)g.Lq * g.B * g.Hkv * g.n_fac;
    for (size_t i = gtid; i < tot; i += gstride) {
      const size_t item = i / (size_t)g.n_fac;
      const int gi = (int)(item % g.Hkv);
      const int l = (int)(item / ((size_t)g.Hkv * g.B));
      if (!label_at(g, l * g.Hkv + gi)) g.idx_out[i] = -1;
    }
  }
}

// Group query of an index item in k_dom channel order (zero padded) into
// s_q[R]; returns the item's cache slice.  Callers synchronise around it.
template <typename E>
__device__ size_t group_query_dom_at(const Geo& g, int pidx, int pair, int b, float* s_q) {
  const int l = pair / g.Hkv, gi = pair - l * g.Hkv;
  const E* qg;
  if (g.clsa)
    qg = (const E*)(g.q_index ? g.q_index : g.q) + ((size_t)b * g.Hq + gi * g.G) * g.d;
  else
    qg = (const E*)g.q + (((size_t)l * g.B + b) * g.Hq + gi * g.G) * g.d;
  const int32_t* dom = g.i_dom + (size_t)kv_pair(g, pair) * g.n_dom;
  const int hd = g.d / 2;
  for (int c = threadIdx.x; c < g.R; c += NT) {
    float v = 0.f;
    if (c < 2 * g.n_dom) {
      // i_dom entries lie in [0, d/2) by contract; the clamp keeps an invalid
      // one from reading outside the query row
      const int f = min(max(dom[c >> 1], 0), hd - 1), cc = c & 1;
      const int chn = g.interleaved ? 2 * f + cc : f + cc * hd;
      float sum = 0.f;
      for (int h = 0; h < g.G; ++h) sum += Vec<E>::one(qg, (size_t)h * g.d + chn);
      v = sum / (float)g.G;
    }
    s_q[c] = v;
  }
  return g.split ? (size_t)pidx * g.B + b : kv_slice(g, l, b, gi);
}
template <typename E>
__device__ size_t group_query_dom(const Geo& g, int item, float* s_q) {
  const int pidx = item / g.B, b = item - pidx * g.B;
  return group_query_dom_at<E>(g, pidx, idx_pair(g, pidx), b, s_q);
}

// One token's TIP score by a single thread (row of R elements).
template <typename E>
__device__ __forceinline__ float score_one(const E* row, const float* s_q, int R) {
  constexpr int EPV = Vec<E>::N;
  float s = 0.f;
  for (int v = 0; v < R / EPV; ++v) {
    float kv[EPV];
    Vec<E>::cvt(ld16(row + v * EPV), kv);
#pragma unroll
    for (int e = 0; e < EPV; ++e) s += s_q[v * EPV + e] * kv[e];
  }
  return s;
}

constexpr int kMaxR = 128;  // k_dom row elements: 2 * (d/2) at most

// Wave-wide reduction of a uint32 with the same lane exchanges as group_sum.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u(uint32_t x, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r32[0], r32[1]);
}
// Inclusive prefix sum over the 64 lanes with DPP only: shifts by 1, 2, 4
// and 8 within each 16-lane row (lanes shifted in from outside the row add
// 0), then lane 15 of each row is added to the next row and lane 31 to rows
// 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan_u(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t x) {
  return wave_reduce_u(x, [](uint32_t a, uint32_t b) { return min(a, b); });
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t x) {
  return wave_reduce_u(x, [](uint32_t a, uint32_t b) { return max(a, b); });
}

__device__ uint2 item_tau(const Geo& g, int item, uint32_t* s_hist, int* s_w, uint32_t* s_res) {
  constexpr int KPT = kSampleTokens / NT;
  const uint32_t* sk = g.skeys + (size_t)item * kSampleTokens;
  uint32_t k[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) k[i] = sk[i * NT + threadIdx.x];
  uint32_t lo = k[0], hi = k[0];
#pragma unroll
  for (int i = 1; i < KPT; ++i) {
    lo = min(lo, k[i]);
    hi = max(hi, k[i]);
  }
  lo = wave_min_u(lo);
  hi = wave_max_u(hi);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kHistBins; i += NT) s_hist[i] = 0;
  if (lane == 0) {
    s_w[wave] = (int)lo;
    s_w[NWAVE + wave] = (int)hi;
  }
  __syncthreads();
  for (int w = 0; w < NWAVE; ++w) {
    lo = min(lo, (uint32_t)s_w[w]);
    hi = max(hi, (uint32_t)s_w[NWAVE + w]);
  }
  const uint32_t span = hi - lo;
  const int bits = span ? 32 - __clz(span) : 0;
  const int sh = bits > 11 ? bits - 11 : 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) atomicAdd(&s_hist[(k[i] - lo) >> sh], 1u);
  __syncthreads();
  int bin;
  uint32_t above;
  find_bin_top(s_hist, kHistBins, (uint32_t)g.samp_rank, s_w, s_res, bin, above);
  uint32_t tau = lo + ((uint32_t)bin << sh);
  if (sh > 0) {
    // second digit inside that bin
    // (the bits of the offset inside that bin: sh - sh2 <= 11 of them, so a
    // narrow span never folds bits of the first digit into the second)
    const int sh2 = sh > 11 ? sh - 11 : 0;
    const uint32_t b1 = (uint32_t)bin, mask2 = (1u << (sh - sh2)) - 1u;
    for (int i = threadIdx.x; i < kHistBins; i += NT) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (((k[i] - lo) >> sh) == b1) atomicAdd(&s_hist[((k[i] - lo) >> sh2) & mask2], 1u);
    __syncthreads();
    find_bin_top(s_hist, kHistBins, (uint32_t)g.samp_rank - above, s_w, s_res, bin, above);
    tau += (uint32_t)bin << sh2;
  }
  return make_uint2(tau, hi);
}

// tau: per index item, the candidate threshold from its sampled keys -- the
// lower edge of the bin, of two range-relative 11-bit digits, that holds the
// samp_rank-th largest sampled key (so at least samp_rank sampled keys are
// >= tau; the final selection is exact whatever tau is) -- and the largest
// sampled key.
__global__ __launch_bounds__(NT) void tau_kernel(Geo g) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ int s_w[2 * NWAVE];
  __shared__ uint32_t s_res[2];
  const int n_items = n_idx_pairs(g) * g.B;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    __syncthreads();
    const uint2 t = item_tau(g, item, s_hist, s_w, s_res);
    if (threadIdx.x == 0) g.tau[item] = t;
  }
}


// ------------------------------------------------------------------ TIP
// One unit = (index item, chunk of ct tokens).  A wave scores 64 tokens per
// step: lane L loads 16 bytes of row (L / V) of each of V consecutive
// 64/V-token slabs, the V lanes of a row reduce their partial dot products,
// and lane L keeps the score of token (L % V) * 64/V + L / V, so each wave
// writes 64 consecutive scores.
// MODE 0: every score and a histogram (general path); 1: prefiltered, tau
// from tau_kernel; 2: prefiltered, each unit derives tau from the sampled
// keys itself (steps with few scoring units, where a separate launch costs
// more than the redundant work), unit 0 of the item storing it; 3: as 2,
// with the unit's first ring loads issued before tau is derived, so they
// are in flight meanwhile (steps with more units, up to kTauInlineUnitsMax).
// HG > 1 (prefiltered with a tau launch, per-query-head selection): the HG
// index items of one KV group's heads share a unit, so the group's dominant
// key rows are read once and scored against HG queries, each head with its
// own threshold and candidate list.
template <typename E, int V, int MODE, int HG = 1>
__global__ __launch_bounds__(NT) void tip_kernel(Geo g) {
  constexpr bool PF = MODE != 0;
  static_assert(HG == 1 || MODE == 1, "heads share units only with a tau launch");
  static_assert(MODE >= 0 && MODE <= 3, "scoring modes 0-3");
  constexpr int EPV = Vec<E>::N;
  constexpr int U = V >= 8 ? 2 : 16 / V;  // 64-token steps in flight per wave (16 loads per lane)
  __shared__ uint32_t s_hist[PF ? 1 : kHistBins];
  // candidates staged in LDS per unit and head; the rest go straight out
  constexpr int kCandUnit = HG == 1 ? 2048 : 1536;
  __shared__ uint2 s_cand[PF ? HG : 1][PF ? kCandUnit : 1];
  __shared__ float s_q[V * EPV];
  __shared__ int s_n[HG];
  __shared__ uint32_t s_base[HG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = PF ? g.nch_tip : g.nch_t;
  const int ct = PF ? g.ct_tip : g.ct;
  const int n_units = n_idx_pairs(g) / HG * g.B * nch;
  if constexpr (!PF)
    for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0;
  const int R = V * EPV;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int unit_item = u / nch, ch = u - unit_item * nch;
    __syncthreads();
    uint4 ring0[U][V];  // the prefiltered ring (MODE 3 fills it before tau)
    float qr[HG][EPV];
    int item[HG];  // index items of the unit (the heads' items when HG > 1)
    size_t slice;
    uint32_t tau[HG];
    if constexpr (PF) {
      // the sample pass stored each item's group query; each lane reads its slice
      const int pg = unit_item / g.B, b = unit_item - pg * g.B;
      const int pidx0 = pg * HG;  // the heads of a KV group are consecutive index pairs
      const int pair = idx_pair(g, pidx0);
      const int l = pair / g.Hkv, gi = pair - l * g.Hkv;
      slice = g.split ? (size_t)pidx0 * g.B + b : kv_slice(g, l, b, gi);
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        item[h] = (pidx0 + h) * g.B + b;
        const float* qb = g.qbar + (size_t)item[h] * R + (lane % V) * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) qr[h][e] = qb[e];
      }
      if constexpr (MODE == 3) {
        const E* kd0 = (const E*)g.kdom + slice * (size_t)g.tstride * R;
        const int tt0 = ch * ct, tt1 = min(g.T, tt0 + ct);
#pragma unroll
        for (int j = 0; j < U; ++j) {
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const int tok = min(tt0 + wave * 64 + j * NT + i * (64 / V) + lane / V, tt1 - 1);
            ring0[j][i] = ld16_stream(kd0 + (size_t)tok * R + (lane % V) * EPV);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (MODE >= 2) {
        __shared__ int s_w2[2 * NWAVE];
        __shared__ uint32_t s_res2[2];
        static_assert(kCandUnit * sizeof(uint2) >= kHistBins * sizeof(uint32_t), "tau histogram in s_cand");
        const uint2 t2 = item_tau(g, item[0], reinterpret_cast<uint32_t*>(&s_cand[0][0]), s_w2, s_res2);
        tau[0] = t2.x;
        if (ch == 0 && tid == 0) g.tau[item[0]] = t2;  // for the final kernel
      } else {
#pragma unroll
        for (int h = 0; h < HG; ++h) tau[h] = g.tau[item[h]].x;
      }
      if (tid < HG) s_n[tid] = 0;
      __syncthreads();
    } else {
      item[0] = unit_item;
      tau[0] = 0u;
      slice = group_query_dom<E>(g, unit_item, s_q);
      __syncthreads();
#pragma unroll
      for (int e = 0; e < EPV; ++e) qr[0][e] = s_q[(lane % V) * EPV + e];
    }
    const E* kd = (const E*)g.kdom + slice * (size_t)g.tstride * R;
    float* sc = g.scores + (size_t)item[0] * g.Ts;
    const int t0 = ch * ct, t1 = min(g.T, t0 + ct);
    // the scores (one per head) of the token this lane keeps, from the V
    // 16-byte pieces of a 64-token step
    auto score = [&](const float (&kv)[V][EPV], float (&mine)[HG]) {
#pragma unroll
      for (int h = 0; h < HG; ++h) mine[h] = 0.f;
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int h = 0; h < HG; ++h) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPV; ++e) s += qr[h][e] * kv[i][e];
          s = group_sum<V>(s);
          if ((lane % V) == i) mine[h] = s;
        }
    };
    auto cvt_step = [&](const uint4 (&raw)[V], float (&kv)[V][EPV]) {
#pragma unroll
      for (int i = 0; i < V; ++i) Vec<E>::cvt(raw[i], kv[i]);
    };
    if constexpr (PF) {
      // A ring of UR steps per wave: a step's pieces are reloaded with the step
      // UR ahead as soon as they are converted, so (UR - 1) V loads stay in
      // flight while a step is scored and its candidates are staged.  Steps
      // past the end load the unit's last row (in bounds) and select nothing.
      // The rare direct appends wait for their store, so no store is pending
      // beside the ring's loads.
      constexpr int UR = U;
      const int wbase0 = t0 + wave * 64;
      auto ld_step = [&](uint4 (&raw)[V], int base) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int tok = min(base + i * (64 / V) + lane / V, t1 - 1);
          raw[i] = ld16_stream(kd + (size_t)tok * R + (lane % V) * EPV);
        }
      };
      uint4 (&ring)[UR][V] = ring0;
      // issued in ring order (the scheduler may not reorder them), so each
      // step's wait leaves the later steps' loads in flight
      if constexpr (MODE != 3) {
#pragma unroll
        for (int j = 0; j < UR; ++j) {
          ld_step(ring[j], wbase0 + j * NT);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      for (int base = wbase0; base < t1; base += NT * UR) {
#pragma unroll
        for (int j = 0; j < UR; ++j) {
          const int sb = base + j * NT;
          float kv[V][EPV];
          cvt_step(ring[j], kv);
          ld_step(ring[j], sb + NT * UR);
          float mine[HG];
          score(kv, mine);
          const int tok = sb + (lane % V) * (64 / V) + lane / V;
#pragma unroll
          for (int h = 0; h < HG; ++h) {
            const uint32_t key = f2key(mine[h]);
            const bool cand = tok < t1 && key >= tau[h];
            const uint64_t m = __ballot(cand);
            if (m) {
              int wb = 0;
              if (lane == 0) wb = atomicAdd(&s_n[h], __popcll(m));
              wb = __builtin_amdgcn_readfirstlane(wb);
              if (cand) {
                const int at = wb + mbcnt(m);
                if (at < kCandUnit) {
                  s_cand[h][at] = make_uint2(key, (uint32_t)tok);
                } else {  // dense unit: append directly (rare)
                  const uint32_t gpos = atomicAdd(&g.info[(size_t)item[h] * 4 + 2], 1u);
                  if (gpos < (uint32_t)g.cand_cap)
                    g.cand[(size_t)item[h] * g.cand_cap + gpos] = make_uint2(key, (uint32_t)tok);
                  __builtin_amdgcn_s_waitcnt(kWaitVm0);
                }
              }
            }
          }
        }
      }
    } else {
      for (int base = t0 + wave * 64; base < t1; base += NT * U) {
        uint4 raw[U][V];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const int tok = base + j * NT + i * (64 / V) + lane / V;
            raw[j][i] = tok < t1 ? ld16_stream(kd + (size_t)tok * R + (lane % V) * EPV) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
        for (int j = 0; j < U; ++j) {
          float kv[V][EPV];
          cvt_step(raw[j], kv);
          float mine[HG];
          score(kv, mine);
          const int tok = base + j * NT + (lane % V) * (64 / V) + lane / V;
          if (tok < t1) {
            sc[tok] = mine[0];
            atomicAdd(&s_hist[f2key(mine[0]) >> 21], 1u);
          }
        }
      }
    }
    __syncthreads();
    if constexpr (PF) {
      if (tid < HG) s_base[tid] = atomicAdd(&g.info[(size_t)item[tid] * 4 + 2], (uint32_t)min(s_n[tid], kCandUnit));
      __syncthreads();
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const int n = min(s_n[h], kCandUnit);
        const uint32_t cbase = s_base[h];
        uint2* cd = g.cand + (size_t)item[h] * g.cand_cap;
        for (int i = tid; i < n; i += NT)
          if (cbase + (uint32_t)i < (uint32_t)g.cand_cap) cd[cbase + i] = s_cand[h][i];
      }
      // no store pending when the next unit's ring starts
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    } else {
      uint32_t* gh = g.hist + (size_t)item[0] * kHistBins;
      for (int i = tid; i < kHistBins; i += NT) {
        const uint32_t c = s_hist[i];
        if (c) {
          atomicAdd(&gh[i], c);
          s_hist[i] = 0;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ select
// select_bin: per index item, the bin b1 of the first key digit that holds
// the n_fac-th largest score, and the count of tokens above it.
__global__ __launch_bounds__(NT) void select_bin_kernel(Geo g) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ int s_w[NWAVE];
  __shared__ uint32_t s_res[2];
  const int n_items = n_idx_pairs(g) * g.B;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    __syncthreads();
    const uint4* gh = reinterpret_cast<const uint4*>(g.hist + (size_t)item * kHistBins);
    for (int i = threadIdx.x; i < kHistBins / 4; i += NT) reinterpret_cast<uint4*>(s_hist)[i] = gh[i];
    __syncthreads();
    int b1;
    uint32_t above1;
    find_bin_top(s_hist, kHistBins, (uint32_t)g.n_fac, s_w, s_res, b1, above1);
    if (threadIdx.x == 0) {
      g.info[(size_t)item * 4 + 0] = (uint32_t)b1;
      g.info[(size_t)item * 4 + 1] = above1;
    }
  }
}

// select_a: per chunk, tokens above bin b1 are counted and tokens inside it
// appended to the item's candidate list.  Each thread reads 4 consecutive
// scores per 1024-token tile.
__global__ __launch_bounds__(NT) void select_a_kernel(Geo g) {
  __shared__ uint2 s_cand[4096];
  __shared__ int s_w[NWAVE];
  __shared__ int s_n;
  __shared__ uint32_t s_base;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n_units = n_idx_pairs(g) * g.B * g.nch_t;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int item = u / g.nch_t, ch = u - item * g.nch_t;
    __syncthreads();
    if (tid == 0) s_n = 0;
    __syncthreads();
    const int b1 = (int)g.info[(size_t)item * 4 + 0];
    const float* sc = g.scores + (size_t)item * g.Ts;
    const int t0 = ch * g.ct, t1 = min(g.T, t0 + g.ct);
    int ngt = 0;
    for (int base = t0; base < t1; base += 4 * NT) {
      const int tok0 = base + 4 * tid;
      const float4 v4 = tok0 < t1 ? *reinterpret_cast<const float4*>(sc + tok0) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float vs[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = tok0 + e;
        const bool valid = tok < t1;
        const uint32_t key = f2key(vs[e]);
        const int bin = (int)(key >> 21);
        ngt += (valid && bin > b1) ? 1 : 0;
        const bool eq = valid && bin == b1;
        const uint64_t m = __ballot(eq);
        if (m) {
          int wbase = 0;
          if (lane == 0) wbase = atomicAdd(&s_n, __popcll(m));
          wbase = __builtin_amdgcn_readfirstlane(wbase);
          if (eq) s_cand[wbase + mbcnt(m)] = make_uint2(key, (uint32_t)tok);
        }
      }
    }
    int tot;
    block_excl_scan(ngt, s_w, tot);
    __syncthreads();
    const int n = s_n;
    if (tid == 0) {
      s_base = atomicAdd(&g.info[(size_t)item * 4 + 2], (uint32_t)n);
      g.ngt[(size_t)item * g.nch_t + ch] = (uint32_t)tot;
    }
    __syncthreads();
    const uint32_t cbase = s_base;
    uint2* cd = g.cand + (size_t)item * g.cand_cap;
    for (int i = tid; i < n; i += NT)
      if (cbase + (uint32_t)i < (uint32_t)g.cand_cap) cd[cbase + i] = s_cand[i];
  }
}

// Candidates of one item: from LDS when they fit, else re-derived from the
// item's scores (every token whose first digit is b1).
struct CandSource {
  const uint2* lds;
  int n;
  const float* sc;
  int T;
  uint32_t b1;
  template <class F>
  __device__ __forceinline__ void for_each(F f) const {
    if (lds) {
      for (int i = threadIdx.x; i < n; i += NT) f(lds[i].x, lds[i].y);
    } else {
      // every score of the item (rows are 64-float aligned): eight 16-byte
      // loads in flight per thread, then the scalar tail
      auto visit = [&](float v, int t) {
        const uint32_t key = f2key(v);
        if ((key >> 21) == b1) f(key, (uint32_t)t);
      };
      const float4* s4 = reinterpret_cast<const float4*>(sc);
      const int n4 = T / 4;
      for (int i0 = threadIdx.x; i0 < n4; i0 += 8 * NT) {
        float4 r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = i0 + j * NT < n4 ? s4[i0 + j * NT] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = i0 + j * NT;
          if (i < n4) {
            visit(r[j].x, 4 * i);
            visit(r[j].y, 4 * i + 1);
            visit(r[j].z, 4 * i + 2);
            visit(r[j].w, 4 * i + 3);
          }
        }
      }
      for (int t = n4 * 4 + (int)threadIdx.x; t < T; t += NT) visit(sc[t], t);
    }
  }
};

template <int BT = NT, class Src, class Pred, class Dig>
__device__ void histogram(const Src& src, uint32_t* s_hist, int nbins, Pred pred, Dig dig) {
  for (int i = threadIdx.x; i < nbins; i += BT) s_hist[i] = 0;
  __syncthreads();
  src.for_each([&](uint32_t key, uint32_t tok) {
    if (pred(key, tok)) atomicAdd(&s_hist[dig(key, tok)], 1u);
  });
  __syncthreads();
}

// Sources of (key, token) elements for the selection helpers.  for_each
// visits each element once, in the calling thread's strided share; reads are
// issued four at a time so their latencies overlap.

// (key, token) pairs held in LDS (BT threads).
template <int BT = NT>
struct LdsPairsT {
  const uint2* p;
  int n;
  template <class F>
  __device__ __forceinline__ void for_each(F f) const {
    int i = threadIdx.x;
    for (; i + 3 * BT < n; i += 4 * BT) {
      const uint2 a = p[i], b = p[i + BT], c = p[i + 2 * BT], d = p[i + 3 * BT];
      f(a.x, a.y);
      f(b.x, b.y);
      f(c.x, c.y);
      f(d.x, d.y);
    }
    for (; i < n; i += BT) f(p[i].x, p[i].y);
  }
};
using LdsPairs = LdsPairsT<>;

// Every token of an item's score row (BT threads).
template <int BT = NT>
struct ScoreScanT {
  const float* sc;
  int T;
  template <class F>
  __device__ __forceinline__ void for_each(F f) const {
    int t = threadIdx.x;
    for (; t + 3 * BT < T; t += 4 * BT) {
      const float a = sc[t], b = sc[t + BT], c = sc[t + 2 * BT], d = sc[t + 3 * BT];
      f(f2key(a), (uint32_t)t);
      f(f2key(b), (uint32_t)(t + BT));
      f(f2key(c), (uint32_t)(t + 2 * BT));
      f(f2key(d), (uint32_t)(t + 3 * BT));
    }
    for (; t < T; t += BT) f(f2key(sc[t]), (uint32_t)t);
  }
};
using ScoreScan = ScoreScanT<>;

// Workgroup min and max of the keys of src (every thread gets both).
template <int BT = NT, class Src>
__device__ void key_range(const Src& src, uint32_t* s_res, uint32_t& lo, uint32_t& hi) {
  __shared__ uint32_t s_lo[BT / 64], s_hi[BT / 64];
  uint32_t a = 0xFFFFFFFFu, b = 0u;
  src.for_each([&](uint32_t k, uint32_t) {
    a = min(a, k);
    b = max(b, k);
  });
  a = wave_min_u(a);
  b = wave_max_u(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    s_lo[wave] = a;
    s_hi[wave] = b;
  }
  __syncthreads();
  lo = s_lo[0];
  hi = s_hi[0];
  for (int w = 1; w < BT / 64; ++w) {
    lo = min(lo, s_lo[w]);
    hi = max(hi, s_hi[w]);
  }
  (void)s_res;
}

constexpr int kRankMax = 256;  // bin size resolved by direct ranking

// 1 when the (key, token) pair a comes before b in the order (key desc, token
// asc), else 0.  Bitwise, so both halves load as one LDS read and the
// comparisons of a ranking loop stay free of branches and their waits.
__device__ __forceinline__ uint32_t before(uint2 a, uint2 b) {
  return (uint32_t)(a.x > b.x) | ((uint32_t)(a.x == b.x) & (uint32_t)(a.y < b.y));
}

// The element of rank need-1 (0-based) in the order (key desc, token asc)
// among the elements whose key satisfies ((key - lo) >> sh) == pre; there
// are at most kRankMax of them.  Each counts the members ordered before it.
template <int BT = NT, class Src>
__device__ void rank_in_bin(const Src& src, uint32_t lo, int sh, uint32_t pre, uint32_t need, uint32_t* s_res,
                            uint32_t& kstar, uint32_t& tstar) {
  __shared__ uint2 s_list[kRankMax];
  __shared__ int s_m;
  if (threadIdx.x == 0) s_m = 0;
  __syncthreads();
  src.for_each([&](uint32_t k, uint32_t t) {
    if (((k - lo) >> sh) == pre) s_list[atomicAdd(&s_m, 1)] = make_uint2(k, t);
  });
  __syncthreads();
  const int m = s_m;
  for (int i = threadIdx.x; i < m; i += BT) {
    const uint2 me = s_list[i];
    uint32_t r = 0;
#pragma unroll 8
    for (int j = 0; j < m; ++j) {
      const uint2 o = s_list[j];
      r += before(o, me);
    }
    if (r == need - 1) {
      s_res[0] = me.x;
      s_res[1] = me.y;
    }
  }
  __syncthreads();
  kstar = s_res[0];
  tstar = s_res[1];
  __syncthreads();
}

// The need-th element of src in the order (key desc, token asc), as (key*,
// token*).  Keys are resolved by radix digits of at most 11 bits taken over
// the span [lo, hi] of the keys present (so the first digit spreads them over
// its 2048 bins).  As soon as the bin holding the element has at most
// kRankMax members it is resolved by ranking them directly; otherwise the
// digits run out at key*, and the need-th smallest token among the elements
// equal to key* follows: directly when all of them are selected, else by
// three more 10-bit digits.
template <int BT = NT, class Src>
__device__ void exact_threshold(const Src& src, uint32_t need, uint32_t* s_hist, int* s_w, uint32_t* s_res,
                                uint32_t& kstar, uint32_t& tstar) {
  uint32_t lo, hi;
  key_range<BT>(src, s_res, lo, hi);
  const uint32_t span = hi - lo;
  int rem = span ? 32 - __clz(span) : 0;  // bits of (key - lo) still open
  uint32_t pre = 0;
  while (rem > 0) {
    const int w = rem < 11 ? rem : 11;
    rem -= w;
    const int sh = rem;
    const int nbins = (1 << w) < BT ? BT : (1 << w);
    const uint32_t p = pre;
    const int up = sh + w;
    histogram<BT>(src, s_hist, nbins,
              [=](uint32_t k, uint32_t) { return up >= 32 ? true : (((k - lo) >> up) == p); },
              [=](uint32_t k, uint32_t) { return ((k - lo) >> sh) & ((1u << w) - 1u); });
    int bin;
    uint32_t above;
    find_bin_top<BT>(s_hist, nbins, need, s_w, s_res, bin, above);
    const uint32_t members = s_hist[bin];
    __syncthreads();
    need -= above;
    pre = (pre << w) | (uint32_t)bin;
    if (rem > 0 && members <= (uint32_t)kRankMax) {
      rank_in_bin<BT>(src, lo, sh, pre, need, s_res, kstar, tstar);
      return;
    }
  }
  kstar = lo + pre;
  tstar = 0;
  const uint32_t ks = kstar;
  // how many elements carry kstar, and the largest such token
  constexpr int BW = BT / 64;
  __shared__ uint32_t s_eq[2 * BW];
  uint32_t n_eq = 0, t_max = 0;
  src.for_each([&](uint32_t k, uint32_t t) {
    if (k == ks) {
      ++n_eq;
      t_max = max(t_max, t);
    }
  });
  n_eq = wave_reduce_u(n_eq, [](uint32_t a, uint32_t b) { return a + b; });
  t_max = wave_max_u(t_max);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    s_eq[wave] = n_eq;
    s_eq[BW + wave] = t_max;
  }
  __syncthreads();
  n_eq = 0;
  t_max = 0;
  for (int w = 0; w < BW; ++w) {
    n_eq += s_eq[w];
    t_max = max(t_max, s_eq[BW + w]);
  }
  if (need == n_eq) {
    tstar = t_max;
  } else {
    uint32_t tpre = 0;
    for (int shift = 20; shift >= 0; shift -= 10) {
      const uint32_t hmask = (shift == 20) ? 0u : (0xFFFFFFFFu << (shift + 10));
      histogram<BT>(src, s_hist, 1024, [=](uint32_t k, uint32_t t) { return k == ks && (t & hmask) == tpre; },
                [=](uint32_t, uint32_t t) { return 1023u - ((t >> shift) & 0x3FFu); });
      int bin;
      uint32_t above;
      find_bin_top<BT>(s_hist, 1024, need, s_w, s_res, bin, above);
      need -= above;
      tpre |= (1023u - (uint32_t)bin) << shift;
    }
    tstar = tpre;
  }
}

// Elements for the selection fused into the attention: (key, token) pairs
// through a generic pointer (LDS, or global memory when an item's
// candidates do not fit there), or an item's whole score row.  One type for
// the three cases, so the threshold helpers (and their LDS) are instantiated
// once; four reads in flight per thread.
template <int BT = NT>
struct SelSrcT {
  const uint2* pairs;  // null: the score row sc
  const float* sc;
  int n;
  template <class F>
  __device__ __forceinline__ void for_each(F f) const {
    int i = threadIdx.x;
    if (pairs) {
      for (; i + 3 * BT < n; i += 4 * BT) {
        const uint2 a = pairs[i], b = pairs[i + BT], c = pairs[i + 2 * BT], d = pairs[i + 3 * BT];
        f(a.x, a.y);
        f(b.x, b.y);
        f(c.x, c.y);
        f(d.x, d.y);
      }
      for (; i < n; i += BT) f(pairs[i].x, pairs[i].y);
    } else {
      for (; i + 3 * BT < n; i += 4 * BT) {
        const float a = sc[i], b = sc[i + BT], c = sc[i + 2 * BT], d = sc[i + 3 * BT];
        f(f2key(a), (uint32_t)i);
        f(f2key(b), (uint32_t)(i + BT));
        f(f2key(c), (uint32_t)(i + 2 * BT));
        f(f2key(d), (uint32_t)(i + 3 * BT));
      }
      for (; i < n; i += BT) f(f2key(sc[i]), (uint32_t)i);
    }
  }
};

// The bit position of the k-th set bit (0-based, k < popcount) of x.
__device__ __forceinline__ int nth_set_bit(uint32_t x, int k) {
  int pos = 0;
#pragma unroll
  for (int half = 16; half >= 1; half >>= 1) {
    const uint32_t low = x & ((1u << half) - 1u);
    const int c = __popc(low);
    if (k >= c) {
      k -= c;
      x >>= half;
      pos += half;
    } else {
      x = low;
    }
  }
  return pos;
}

// sample: TIP keys of kSampleTokens tokens per index item, in 64 V evenly
// spread blocks of 64 / V tokens (V 16-byte pieces per key row: 256 blocks of
// 16 for bf16 d 128); one unit = (item, 256 of the tokens), each wave scoring
// 64 of them (one block per load) with tip_kernel's reduction.  Unit 0 of the
// item also stores its group query for the scoring pass.
// PLAN (steps without the side stream): no plan launch precedes; every
// workgroup lists the retrieval pairs from the labels in LDS, workgroup 0
// writes the plan for the later launches, and the grid fills the -1 index
// rows of streaming groups.
// HG > 1 (per-query-head selection with a tau launch): a unit serves the HG
// head items of one KV group, reading the group's sampled rows once.
template <typename E, int V, bool PLAN, int HG = 1>
__global__ __launch_bounds__(NT) void sample_kernel(Geo g) {
  static_assert(HG == 1 || !PLAN, "heads share units only without the fused plan");
  constexpr int EPV = Vec<E>::N;
  constexpr int kBlocks = kSampleTokens / 256;
  __shared__ float s_q[HG][kMaxR];
  __shared__ uint16_t s_ret[PLAN ? kMaxPairs : 1];
  __shared__ int s_w[NWAVE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = V * EPV;
  int n_idx;
  if constexpr (PLAN) {
    const int P = g.Lq * g.Hkv;
    const int per = (P + NT - 1) / NT;
    const int p0 = min(P, tid * per), p1 = min(P, p0 + per);
    int cnt = 0;
    for (int p = p0; p < p1; ++p) cnt += label_at(g, p);
    int n_ret;
    const int excl = block_excl_scan(cnt, s_w, n_ret);
    int* lists = g.plan + 4;
    int r = excl, st = p0 - excl;
    for (int p = p0; p < p1; ++p) {
      if (label_at(g, p)) {
        s_ret[r] = (uint16_t)p;
        if (blockIdx.x == 0) lists[r] = lists[kMaxPairs + r] = p;
        ++r;
      } else {
        if (blockIdx.x == 0) lists[2 * kMaxPairs + st] = p;
        ++st;
      }
    }
    if (blockIdx.x == 0 && tid == 0) {
      g.plan[0] = n_ret;
      g.plan[1] = n_ret;
      g.plan[2] = P - n_ret;
      g.plan[3] = 0;
    }
    n_idx = n_ret;
    if (g.idx_out) {
      const size_t tot = (size_t)g.Lq * g.B * g.Hkv * g.n_fac;
      for (size_t i = (size_t)blockIdx.x * NT + tid; i < tot; i += (size_t)gridDim.x * NT) {
        const size_t it = i / (size_t)g.n_fac;
        const int gi = (int)(it % g.Hkv), l = (int)(it / ((size_t)g.Hkv * g.B));
        if (!label_at(g, l * g.Hkv + gi)) g.idx_out[i] = -1;
      }
    }
    __syncthreads();
  } else {
    n_idx = n_idx_pairs(g);
  }
  const int n_units = n_idx / HG * g.B * kBlocks;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int unit_item = u / kBlocks, blk = u - unit_item * kBlocks;
    const int pg = unit_item / g.B, b = unit_item - pg * g.B;
    const int pidx0 = pg * HG;  // the heads of a KV group are consecutive index pairs
    __syncthreads();
    size_t slice = 0;
#pragma unroll
    for (int h = 0; h < HG; ++h)
      slice = group_query_dom_at<E>(g, pidx0 + h, PLAN ? (int)s_ret[pidx0 + h] : idx_pair(g, pidx0 + h), b, s_q[h]);
    __syncthreads();
    if (blk == 0) {
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const size_t item = (size_t)(pidx0 + h) * g.B + b;
        for (int c = tid; c < R; c += NT) g.qbar[item * R + c] = s_q[h][c];
        if ((PLAN || g.host_plan) && tid < 4) g.info[item * 4 + tid] = 0u;  // else the plan clears them
      }
    }
    float qr[HG][EPV];
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < EPV; ++e) qr[h][e] = s_q[h][(lane % V) * EPV + e];
    const E* kd = (const E*)g.kdom + slice * (size_t)g.tstride * R;
    // The sampled tokens: 64 V blocks of 64 / V consecutive tokens, evenly
    // spread over the context, one block per load of a wave (the unit holds
    // blocks blk * 4V .. blk * 4V + 4V - 1).  Many short blocks: nearby TIP
    // scores are correlated, so the blocks, not the tokens, set how well the
    // sample places tau.
    constexpr int kBlen = 64 / V, kNsb = 64 * V;
    uint4 raw[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int sb = blk * (NWAVE * V) + wave * V + i;
      const int tok = (int)((long long)sb * (g.T - kBlen) / (kNsb - 1)) + lane / V;
      raw[i] = ld16_stream(kd + (size_t)tok * R + (lane % V) * EPV);
    }
    float mine[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) mine[h] = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float kv[EPV];
      Vec<E>::cvt(raw[i], kv);
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) sum += qr[h][e] * kv[e];
        sum = group_sum<V>(sum);
        if ((lane % V) == i) mine[h] = sum;
      }
    }
#pragma unroll
    for (int h = 0; h < HG; ++h)
      g.skeys[((size_t)(pidx0 + h) * g.B + b) * kSampleTokens + blk * 256 + wave * 64 + lane] = f2key(mine[h]);
  }
}

// final: per index item, the exact top-n_fac among the candidates (key >=
// tau) held in LDS.  While the candidates load, they are counted in 2048
// bins of (key - tau) >> sh, sh sized so the largest sampled key falls in the
// top bin (larger keys are clamped into it).  The cut (key*, token*) -- the
// n_fac-th candidate in the order (key desc, token asc) -- comes from ranking
// the members of the bin that holds it when that bin is not the clamped top
// bin and has at most kRankMax members, else from the general radix
// threshold.  The selected tokens are then compacted to the front of the
// candidate buffer, marked in a token bitmap built in the rest of it, and
// each is written to the slot given by the number of marked tokens before
// it (per-word prefix counts), which emits the selection in ascending order.
// If the candidates are fewer than n_fac or overflowed, the item is rescored
// in full here and selected from its score row (exact either way).
// LONG = false (T <= kShortMaxT): the bitmap has an LDS array of its own, so
// it always fits beside the candidates and the compacting path is compiled
// out; LONG = true: the bitmap goes in the candidate buffer.
// One item per workgroup of kFinalThreads: the kernel's LDS admits one
// workgroup per CU, so it brings sixteen waves.
constexpr int kFinalThreads = 1024;

template <typename E, bool LONG>
__global__ __launch_bounds__(kFinalThreads) void final_kernel(Geo g) {
  constexpr int BT = kFinalThreads, BW = BT / 64;
  // candidates; for LONG, later the selected tokens, the bitmap and the prefix counts
  __shared__ __attribute__((aligned(16))) uint2 s_c[kCandFast];
  __shared__ __attribute__((aligned(16))) uint32_t s_bm[LONG ? 4 : kShortMaxT / 32];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
  __shared__ float s_q[kMaxR];
  __shared__ int s_w[BW];
  __shared__ uint32_t s_res[2];
  __shared__ uint2 s_list[kRankMax];
  __shared__ int s_m;
  // !LONG: the prefix counts (u16) reuse the histogram, free by then
  static_assert(kHistBins * sizeof(uint32_t) >= kShortMaxT / 32 * sizeof(uint16_t), "u16 prefixes in s_hist");
  // bitmap words per thread for the prefix counts, so the bitmap spans BT *
  // per words; for LONG a multiple of 4, which keeps the prefix counts
  // placed behind it 16-byte aligned
  const int per = LONG ? ((g.bm_words + BT - 1) / BT + 3) & ~3 : (g.bm_words + BT - 1) / BT;
  constexpr int kSelWords = kSelMaxLong;  // n_fac on this path, a multiple of 4 words
  constexpr int kPerMax = (kPrefilterMaxT / 32 / BT + 3) & ~3;
  static_assert(kCandFast * sizeof(uint2) >= (kSelWords + BT * kPerMax) * sizeof(uint32_t) +
                                                 BT * kPerMax * sizeof(uint16_t),
                "selected tokens, bitmap and u16 prefixes fit the candidate buffer");
  static_assert(kSelMaxLong % 4 == 0 && kSelMaxLong < 65536, "16-byte aligned bitmap; n_fac fits u16 prefixes");
  const int tid = threadIdx.x;
  const int n_items = n_idx_pairs(g) * g.B;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    __syncthreads();
    const uint32_t count = g.info[(size_t)item * 4 + 2];
    const uint2 th = g.tau[item];
    for (int i = tid; i < kHistBins; i += BT) s_hist[i] = 0u;
    if (tid == 0) s_m = 0;
    const int pidx = item / g.B, b = item - pidx * g.B;
    const int pair = idx_pair(g, pidx);
    const int l = pair / g.Hkv, gi = pair - l * g.Hkv;
    int32_t* ix = g.idx + (size_t)item * g.n_fac;
    int32_t* ox = g.idx_out ? g.idx_out + (((size_t)l * g.B + b) * g.Hkv + gi) * g.n_fac : nullptr;
    // bitmap of BT * per words at bm, u16 prefix counts after it
    auto clear_bitmap = [&](uint32_t* bm) {
      for (int w = tid; w < BT * per; w += BT) bm[w] = 0u;
    };
    // exclusive prefix counts of the set bits, one u16 per bitmap word
    // (< n_fac < 2^16).  Each wave scans a contiguous quarter of the bitmap,
    // lane i on word i of each 64-word tile, so LDS accesses are
    // conflict-free; a first pass sums the quarters for the wave offsets.
    auto prefix = [&](const uint32_t* bm, uint16_t* pre) {
      const int lane = tid & 63, wave = tid >> 6;
      const int qw = BT * per / BW;  // a multiple of 64 (BT / BW = 64)
      const uint32_t* wb = bm + wave * qw;
      uint16_t* wp = pre + wave * qw;
      uint32_t tot = 0;
      for (int k = lane; k < qw; k += 64) tot += __popc(wb[k]);
      tot = wave_reduce_u(tot, [](uint32_t x, uint32_t y) { return x + y; });
      if (lane == 0) s_w[wave] = (int)tot;
      __syncthreads();
      uint32_t carry = 0;
      for (int w = 0; w < wave; ++w) carry += (uint32_t)s_w[w];
      for (int k0 = 0; k0 < qw; k0 += 64) {
        const uint32_t x = __popc(wb[k0 + lane]);
        const uint32_t inc = wave_incl_scan_u(x);
        wp[k0 + lane] = (uint16_t)(carry + inc - x);
        carry += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      }
    };
    auto put = [&](const uint32_t* bm, const uint16_t* pre, uint32_t t) {
      const uint32_t word = bm[t >> 5], bit = 1u << (t & 31);
      const uint32_t pos = pre[t >> 5] + __popc(word & (bit - 1u));
      if (pos < (uint32_t)g.n_fac) {  // always, with exactly n_fac marked
        ix[pos] = (int32_t)t;
        if (ox) ox[pos] = (int32_t)t;
      }
    };
    if (count >= (uint32_t)g.n_fac && count <= (uint32_t)g.cand_cap) {
      const uint32_t tau = th.x;
      const uint32_t span = th.y > tau ? th.y - tau : 0u;
      const int bits = span ? 32 - __clz(span) : 0;
      const int sh = bits > 11 ? bits - 11 : 0;
      // direct: the bitmap and its prefix counts fit after the candidates,
      // and tokens are marked while the threshold is found; else the
      // selected tokens are compacted first and the bitmap built behind them
      const int cand_words = ((int)count * 2 + 3) & ~3;
      const bool direct =
          !LONG || (size_t)(cand_words + BT * per) * 4 + (size_t)BT * per * 2 <= sizeof(s_c);
      uint32_t* bm = !LONG ? s_bm : reinterpret_cast<uint32_t*>(s_c) + (direct ? cand_words : kSelWords);
      uint16_t* pre = !LONG ? reinterpret_cast<uint16_t*>(s_hist) : reinterpret_cast<uint16_t*>(bm + BT * per);
      if (direct) clear_bitmap(bm);
      __syncthreads();
      // candidates -> LDS, two per 16-byte load, eight loads in flight,
      // counted by their first digit on the way
      const uint4* c4 = reinterpret_cast<const uint4*>(g.cand + (size_t)item * g.cand_cap);
      const int n4 = (int)(count + 1) / 2;
      for (int i0 = tid; i0 < n4; i0 += 8 * BT) {
        uint4 r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = i0 + j * BT < n4 ? c4[i0 + j * BT] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = i0 + j * BT;
          if (i < n4) {
            s_c[2 * i] = make_uint2(r[j].x, r[j].y);
            atomicAdd(&s_hist[min((r[j].x - tau) >> sh, (uint32_t)kHistBins - 1u)], 1u);
            if (2 * i + 1 < (int)count) {
              s_c[2 * i + 1] = make_uint2(r[j].z, r[j].w);
              atomicAdd(&s_hist[min((r[j].z - tau) >> sh, (uint32_t)kHistBins - 1u)], 1u);
            }
          }
        }
      }
      __syncthreads();
      const LdsPairsT<BT> src{s_c, (int)count};
      auto mark = [&](uint32_t t) { atomicOr(&bm[t >> 5], 1u << (t & 31)); };
      int bin;
      uint32_t above;
      find_bin_top<BT>(s_hist, kHistBins, (uint32_t)g.n_fac, s_w, s_res, bin, above);
      const uint32_t members = s_hist[bin];
      __syncthreads();
      uint32_t kstar = 0, tstar = 0;
      if (bin < kHistBins - 1 && members <= (uint32_t)kRankMax) {
        // every candidate in a higher bin has a larger key; within the bin a
        // member is selected when fewer than need members precede it in
        // (key desc, token asc), and the cut is the one preceded by need - 1
        const uint32_t ub = (uint32_t)bin;
        src.for_each([&](uint32_t k, uint32_t t) {
          const uint32_t d = min((k - tau) >> sh, (uint32_t)kHistBins - 1u);
          if (d > ub) {
            if (direct) mark(t);
          } else if (d == ub) {
            s_list[atomicAdd(&s_m, 1)] = make_uint2(k, t);
          }
        });
        __syncthreads();
        const uint32_t need = (uint32_t)g.n_fac - above;
        const int m = s_m;
        for (int i = tid; i < m; i += BT) {
          const uint2 me = s_list[i];
          uint32_t r = 0;
#pragma unroll 8
          for (int j = 0; j < m; ++j) {
            const uint2 o = s_list[j];
            r += before(o, me);
          }
          if (direct && r < need) mark(me.y);
          if (r == need - 1) {
            s_res[0] = me.x;
            s_res[1] = me.y;
          }
        }
        __syncthreads();
        kstar = s_res[0];
        tstar = s_res[1];
      } else {
        exact_threshold<BT>(src, (uint32_t)g.n_fac, s_hist, s_w, s_res, kstar, tstar);
        if (direct)
          src.for_each([&](uint32_t k, uint32_t t) {
            if (k > kstar || (k == kstar && t <= tstar)) mark(t);
          });
      }
      uint32_t* s_sel = reinterpret_cast<uint32_t*>(s_c);
      int n_sel = 0;
      if (!direct) {
        // compact the selected tokens (n_fac of them) to the front of the
        // buffer as u32.  Per chunk, every read precedes every write; a
        // write lands below 4 bytes x (candidates read so far), under the
        // next chunk's first read at 8 bytes x that.
        __syncthreads();
        if (tid == 0) s_m = 0;
        __syncthreads();
        for (int c0 = 0; c0 < (int)count; c0 += 8 * BT) {
          uint2 r[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = c0 + j * BT + tid;
            r[j] = i < (int)count ? s_c[i] : make_uint2(0u, 0xFFFFFFFFu);
          }
          __syncthreads();
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c0 + j * BT + tid < (int)count && (r[j].x > kstar || (r[j].x == kstar && r[j].y <= tstar)))
              s_sel[atomicAdd(&s_m, 1)] = r[j].y;
          __syncthreads();
        }
        n_sel = min(s_m, g.n_fac);  // == n_fac
        clear_bitmap(bm);
        __syncthreads();
        for (int i = tid; i < n_sel; i += BT) mark(s_sel[i]);
      }
      __syncthreads();
      prefix(bm, pre);
      __syncthreads();
      if (direct) {
        src.for_each([&](uint32_t, uint32_t t) {
          if (bm[t >> 5] & (1u << (t & 31))) put(bm, pre, t);
        });
      } else {
        for (int i = tid; i < n_sel; i += BT) put(bm, pre, s_sel[i]);
      }
    } else {
      const size_t slice = group_query_dom<E>(g, item, s_q);
      __syncthreads();
      const E* kd = (const E*)g.kdom + slice * (size_t)g.tstride * g.R;
      float* sc = g.scores + (size_t)item * g.Ts;
      for (int t = tid; t < g.T; t += BT) sc[t] = score_one<E>(kd + (size_t)t * g.R, s_q, g.R);
      __threadfence();
      __syncthreads();
      const ScoreScanT<BT> src{sc, g.T};
      uint32_t kstar, tstar;
      exact_threshold<BT>(src, (uint32_t)g.n_fac, s_hist, s_w, s_res, kstar, tstar);
      uint32_t* bm = !LONG ? s_bm : reinterpret_cast<uint32_t*>(s_c);
      uint16_t* pre = !LONG ? reinterpret_cast<uint16_t*>(s_hist) : reinterpret_cast<uint16_t*>(bm + BT * per);
      clear_bitmap(bm);
      __syncthreads();
      src.for_each([&](uint32_t k, uint32_t t) {
        if (k > kstar || (k == kstar && t <= tstar)) atomicOr(&bm[t >> 5], 1u << (t & 31));
      });
      __syncthreads();
      prefix(bm, pre);
      __syncthreads();
      src.for_each([&](uint32_t k, uint32_t t) {
        if (k > kstar || (k == kstar && t <= tstar)) put(bm, pre, t);
      });
    }
  }
}

// select_b: exact threshold.  Ordering is (score desc, token asc); the
// n_fac-th element (key*, token*) is found digit by digit: key bits 20..10
// and 9..0 among the candidates, then token bits 29..20, 19..10, 9..0 among
// candidates equal to key* (ascending).  Then per-chunk output offsets.
__global__ __launch_bounds__(NT) void select_b_kernel(Geo g) {
  __shared__ uint2 s_c[kCandLds];
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_chunk[kMaxTipChunks];
  __shared__ int s_w[NWAVE];
  __shared__ uint32_t s_res[2];
  __shared__ uint32_t s_n;
  const int tid = threadIdx.x;
  const int ct = g.ct;
  const int n_items = n_idx_pairs(g) * g.B;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    __syncthreads();
    const uint32_t b1 = g.info[(size_t)item * 4 + 0];
    const uint32_t above1 = g.info[(size_t)item * 4 + 1];
    const uint32_t count = g.info[(size_t)item * 4 + 2];
    const bool in_lds = count <= (uint32_t)min(g.cand_cap, kCandLds);
    CandSource src{nullptr, 0, g.scores + (size_t)item * g.Ts, g.T, b1};
    if (in_lds) {
      const uint2* cd = g.cand + (size_t)item * g.cand_cap;
      for (int i = tid; i < (int)count; i += NT) s_c[i] = cd[i];
      src.lds = s_c;
      src.n = (int)count;
    }
    __syncthreads();
    uint32_t need = (uint32_t)g.n_fac - above1;
    int bin;
    uint32_t above;
    // key bits 20..10
    histogram(src, s_hist, 2048, [](uint32_t, uint32_t) { return true; },
              [](uint32_t k, uint32_t) { return (k >> 10) & 0x7FFu; });
    find_bin_top(s_hist, 2048, need, s_w, s_res, bin, above);
    need -= above;
    const uint32_t pre22 = (b1 << 11) | (uint32_t)bin;
    // scores rescanned: when the members of the threshold's 22-bit key prefix
    // fit the LDS, one more scan moves them there and counts per chunk the
    // tokens above that prefix (all selected); the later passes read the LDS
    const uint32_t members = s_hist[bin];
    const bool compact = !in_lds && members <= (uint32_t)kCandLds;
    for (int c = tid; c < g.nch_t; c += NT) s_chunk[c] = 0;
    if (tid == 0) s_n = 0;
    __syncthreads();
    if (compact) {
      src.for_each([&](uint32_t k, uint32_t t) {
        const uint32_t p = k >> 10;
        if (p == pre22)
          s_c[atomicAdd(&s_n, 1u)] = make_uint2(k, t);
        else if (p > pre22)
          atomicAdd(&s_chunk[t / ct], 1u);
      });
      __syncthreads();
      src.lds = s_c;
      src.n = (int)members;
    }
    // key bits 9..0
    histogram(src, s_hist, 1024, [=](uint32_t k, uint32_t) { return (k >> 10) == pre22; },
              [](uint32_t k, uint32_t) { return k & 0x3FFu; });
    find_bin_top(s_hist, 1024, need, s_w, s_res, bin, above);
    need -= above;
    const uint32_t kstar = (pre22 << 10) | (uint32_t)bin;
    // the need-th smallest token among key == kstar, 10 bits at a time
    uint32_t tpre = 0;
    for (int shift = 20; shift >= 0; shift -= 10) {
      const uint32_t hmask = (shift == 20) ? 0u : (0xFFFFFFFFu << (shift + 10));
      histogram(src, s_hist, 1024,
                [=](uint32_t k, uint32_t t) { return k == kstar && (t & hmask) == tpre; },
                [=](uint32_t, uint32_t t) { return 1023u - ((t >> shift) & 0x3FFu); });
      find_bin_top(s_hist, 1024, need, s_w, s_res, bin, above);
      need -= above;
      tpre |= (1023u - (uint32_t)bin) << shift;
    }
    const uint32_t tstar = tpre;
    // per-chunk counts of selected candidates (after a compaction, those of
    // the prefix's members, the rest being counted already)
    src.for_each([&](uint32_t k, uint32_t t) {
      if (k > kstar || (k == kstar && t <= tstar)) atomicAdd(&s_chunk[t / ct], 1u);
    });
    __syncthreads();
    // exclusive prefix over chunks of (tokens above b1 + selected candidates)
    const uint32_t* ngt = g.ngt + (size_t)item * g.nch_t;
    uint32_t* off = g.off + (size_t)item * g.nch_t;
    const int per = (g.nch_t + NT - 1) / NT;
    const int c0 = min(g.nch_t, tid * per), c1 = min(g.nch_t, c0 + per);
    int seg = 0;
    for (int c = c0; c < c1; ++c) seg += (int)(ngt[c] + s_chunk[c]);
    int tot;
    int run = block_excl_scan(seg, s_w, tot);
    for (int c = c0; c < c1; ++c) {
      off[c] = (uint32_t)run;
      run += (int)(ngt[c] + s_chunk[c]);
    }
    if (tid == 0) g.thr[item] = make_uint2(kstar, tstar);
  }
}

// select_c: ordered compaction of the selected tokens of one chunk (each
// thread owns 4 consecutive tokens of a 1024-token tile).
__global__ __launch_bounds__(NT) void select_c_kernel(Geo g) {
  __shared__ int s_w[NWAVE];
  const int tid = threadIdx.x;
  const int n_units = n_idx_pairs(g) * g.B * g.nch_t;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int item = u / g.nch_t, ch = u - item * g.nch_t;
    const int pidx = item / g.B, b = item - pidx * g.B;
    const int pair = idx_pair(g, pidx);
    const int l = pair / g.Hkv, gi = pair - l * g.Hkv;
    const uint2 th = g.thr[item];
    const float* sc = g.scores + (size_t)item * g.Ts;
    int32_t* ix = g.idx + (size_t)item * g.n_fac;
    int32_t* ox = g.idx_out ? g.idx_out + (((size_t)l * g.B + b) * g.Hkv + gi) * g.n_fac : nullptr;
    const int t0 = ch * g.ct, t1 = min(g.T, t0 + g.ct);
    uint32_t run = g.off[(size_t)item * g.nch_t + ch];
    for (int base = t0; base < t1; base += 4 * NT) {
      const int tok0 = base + 4 * tid;
      const float4 v4 = tok0 < t1 ? *reinterpret_cast<const float4*>(sc + tok0) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float vs[4] = {v4.x, v4.y, v4.z, v4.w};
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = f2key(vs[e]);
        const bool sel = (tok0 + e < t1) && (k > th.x || (k == th.x && (uint32_t)(tok0 + e) <= th.y));
        m |= sel ? (1u << e) : 0u;
      }
      int tot;
      uint32_t pos = run + (uint32_t)block_excl_scan(__popc(m), s_w, tot);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((m >> e) & 1u) {
          if (pos < (uint32_t)g.n_fac) {
            ix[pos] = tok0 + e;
            if (ox) ox[pos] = tok0 + e;
          }
          ++pos;
        }
      }
      run += (uint32_t)tot;
    }
  }
}

// ------------------------------------------------------------------ attention
// LDS of the selection inside an attention unit: the histogram (later the u16
// prefix counts), the member list, a token bitmap of kShortMaxT bits and up
// to kUnitSelCand candidates (more are read from global memory again).
constexpr int kUnitSelCand = 4096;
constexpr int kUnitSelCandOfs = kHistBins * 4 + kRankMax * 8 + kShortMaxT / 32 * 4;
constexpr int kUnitSelBytes = kUnitSelCandOfs + kUnitSelCand * 8;

// The exact top-n_fac cut of index item `item` from its candidates, by one
// attention unit (NT threads) for itself -- FASA §2.B.1, the same selection
// as final_kernel, repeated by every unit of the item side by side instead
// of one workgroup per item in a launch of its own -- and the cache
// positions of the selected tokens of ascending rank r0 .. r0 + nrows - 1
// into rows (LDS), with those idx_out entries (ox, or null).  The item's
// units read its candidates through the L2, each staging up to kUnitSelCand
// in LDS (more are read from global memory again for the cut) while counting
// them in 2048 bins of (key - tau) >> sh; the members of the bin
// holding the n_fac-th are ranked directly (at most kRankMax, below the
// clamped top bin), else the general radix threshold; selected tokens are
// marked in a token bitmap, whose words' exclusive prefix counts give each
// rank's word and bit.  Fewer than n_fac candidates or an overflow: the unit
// rescores the item in full (every unit writes the same score row).
// lds: kUnitSelBytes, 16-byte aligned; s_qd: R floats of LDS (rescoring).
template <typename E>
__device__ void unit_select_rows(const Geo& g, int item, int r0, int nrows, int* rows, int32_t* ox,
                                 unsigned char* lds, float* s_qd) {
  __shared__ int s_w[NWAVE];
  __shared__ uint32_t s_res[2];
  __shared__ int s_m;
  uint32_t* s_hist = reinterpret_cast<uint32_t*>(lds);
  uint16_t* s_pre = reinterpret_cast<uint16_t*>(lds);
  uint2* s_list = reinterpret_cast<uint2*>(lds + kHistBins * 4);
  uint32_t* s_bm = reinterpret_cast<uint32_t*>(lds + kHistBins * 4 + kRankMax * 8);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // bitmap words per wave: whole 64-word rows covering bm_words (<= kShortMaxT / 32)
  const int qw = (g.bm_words + NT - 1) / NT * 64;
  const int nwords = NWAVE * qw;
  const uint32_t count = g.info[(size_t)item * 4 + 2];
  const uint2 th = g.tau[item];
  for (int w = tid; w < nwords; w += NT) s_bm[w] = 0u;
  for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
  if (tid == 0) s_m = 0;
  auto mark = [&](uint32_t t) { atomicOr(&s_bm[t >> 5], 1u << (t & 31)); };
  auto cut_general = [&](const SelSrcT<NT>& src) {
    uint32_t kstar, tstar;
    exact_threshold<NT>(src, (uint32_t)g.n_fac, s_hist, s_w, s_res, kstar, tstar);
    src.for_each([&](uint32_t k, uint32_t t) {
      if (k > kstar || (k == kstar && t <= tstar)) mark(t);
    });
  };
  const uint2* gc = g.cand + (size_t)item * g.cand_cap;
  if (count >= (uint32_t)g.n_fac && count <= (uint32_t)g.cand_cap) {
    const uint32_t tau = th.x;
    const uint32_t span = th.y > tau ? th.y - tau : 0u;
    const int bits = span ? 32 - __clz(span) : 0;
    const int sh = bits > 11 ? bits - 11 : 0;
    __syncthreads();
    // candidates -> LDS when they fit, counted by their first digit
    uint2* s_c = reinterpret_cast<uint2*>(lds + kUnitSelCandOfs);
    const bool in_lds = count <= (uint32_t)kUnitSelCand;
    const uint4* c4 = reinterpret_cast<const uint4*>(gc);
    const int n4 = (int)(count + 1) / 2;
    constexpr int kLd = 4;  // 16-byte loads in flight per thread
    for (int i0 = tid; i0 < n4; i0 += kLd * NT) {
      uint4 r[kLd];
#pragma unroll
      for (int q = 0; q < kLd; ++q) r[q] = i0 + q * NT < n4 ? c4[i0 + q * NT] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < kLd; ++q) {
        const int i = i0 + q * NT;
        if (i < n4) {
          if (in_lds) s_c[2 * i] = make_uint2(r[q].x, r[q].y);
          atomicAdd(&s_hist[min((r[q].x - tau) >> sh, (uint32_t)kHistBins - 1u)], 1u);
          if (2 * i + 1 < (int)count) {
            if (in_lds) s_c[2 * i + 1] = make_uint2(r[q].z, r[q].w);
            atomicAdd(&s_hist[min((r[q].z - tau) >> sh, (uint32_t)kHistBins - 1u)], 1u);
          }
        }
      }
    }
    __syncthreads();
    int bin;
    uint32_t above;
    find_bin_top<NT>(s_hist, kHistBins, (uint32_t)g.n_fac, s_w, s_res, bin, above);
    const uint32_t members = s_hist[bin];
    __syncthreads();
    const SelSrcT<NT> gsrc{gc, nullptr, (int)count};
    // everything above bin ub is selected; its members are ranked
    auto cut_binned = [&](const auto& src, uint32_t ub) {
      src.for_each([&](uint32_t k, uint32_t t) {
        const uint32_t d = min((k - tau) >> sh, (uint32_t)kHistBins - 1u);
        if (d > ub) mark(t);
        const bool mem = d == ub;
        const uint64_t bal = __ballot(mem);
        if (bal) {  // one reservation per wave, by its first active lane
          const int leader = __builtin_amdgcn_readfirstlane(lane);
          int base = 0;
          if (lane == leader) base = atomicAdd(&s_m, __popcll(bal));
          base = __builtin_amdgcn_readfirstlane(base);
          if (mem) s_list[base + mbcnt(bal)] = make_uint2(k, t);
        }
      });
      __syncthreads();
      const uint32_t need = (uint32_t)g.n_fac - above;
      const int m = s_m;
      for (int i = tid; i < m; i += NT) {
        const uint2 me = s_list[i];
        uint32_t rk = 0;
#pragma unroll 8
        for (int q = 0; q < m; ++q) rk += before(s_list[q], me);
        if (rk < need) mark(me.y);
      }
    };
    if (bin < kHistBins - 1 && members <= (uint32_t)kRankMax) {
      if (in_lds)
        cut_binned(LdsPairsT<NT>{s_c, (int)count}, (uint32_t)bin);
      else
        cut_binned(gsrc, (uint32_t)bin);
    } else {
      cut_general(gsrc);
    }
  } else {
    // rescoring: the item's full score row (the same values from every unit)
    __syncthreads();
    const size_t slice = group_query_dom<E>(g, item, s_qd);
    __syncthreads();
    const E* kd = (const E*)g.kdom + slice * (size_t)g.tstride * g.R;
    float* sc = g.scores + (size_t)item * g.Ts;
    for (int t = tid; t < g.T; t += NT) sc[t] = score_one<E>(kd + (size_t)t * g.R, s_qd, g.R);
    __threadfence();
    __syncthreads();
    cut_general(SelSrcT<NT>{nullptr, sc, g.T});
  }
  __syncthreads();
  // exclusive prefix counts of the bitmap words (u16: < n_fac < 2^16): wave w
  // scans words [w qw, (w + 1) qw), lane L on word L of each 64-word row
  {
    const uint32_t* wb = s_bm + wave * qw;
    uint32_t tot = 0;
    for (int k = lane; k < qw; k += 64) tot += (uint32_t)__popc(wb[k]);
    tot = wave_reduce_u(tot, [](uint32_t x, uint32_t y) { return x + y; });
    if (lane == 0) s_w[wave] = (int)tot;
    __syncthreads();  // the histogram (aliased by the prefixes) is free since the cut
    uint32_t carry = 0;
    for (int w = 0; w < wave; ++w) carry += (uint32_t)s_w[w];
    uint16_t* wp = s_pre + wave * qw;
    for (int k0 = 0; k0 < qw; k0 += 64) {
      const uint32_t x = (uint32_t)__popc(wb[k0 + lane]);
      const uint32_t inc = wave_incl_scan_u(x);
      wp[k0 + lane] = (uint16_t)(carry + inc - x);
      carry += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    }
  }
  __syncthreads();
  // rank r0 + r: the last word whose prefix count is at most it, then the
  // set bit of that order inside the word
  for (int r = tid; r < nrows; r += NT) {
    const uint32_t rank = (uint32_t)(r0 + r);
    int lo = 0, hi = nwords - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((uint32_t)s_pre[mid] <= rank) lo = mid;
      else hi = mid - 1;
    }
    const int t = lo * 32 + nth_set_bit(s_bm[lo], (int)(rank - s_pre[lo]));
    rows[r] = min(max(t, 0), g.T - 1);
    if (ox) ox[rank] = t;
  }
}

// One unit = (attention item, chunk of <= kMaxChunkRows rows).  The group's G
// query heads share every loaded row: lanes of a row (LPR of them, 16 bytes
// each) form the dot products, then p = exp2(z - m) per head, then P.V.
// Output: per head acc[d] = sum p v, m (log2 domain), l = sum p.
// SEL: the prefiltered path's selection runs in the FAC units themselves
// (unit_select_rows), with no final-selection launch before; its LDS shares
// the space of the logits and row sums, which are used only after it.
template <typename E, int D, int G, bool SEL = false>
__global__ __launch_bounds__(NT) void attn_kernel(Geo g) {
  constexpr int CPL = Vec<E>::N;
  constexpr int LPR = D / CPL;
  constexpr int RPW = 64 / LPR;
  constexpr int RPB = RPW * NWAVE;
  constexpr float kScale = (D == 128 ? 0.08838834764831845f : 0.125f) * 1.4426950408889634f;
  constexpr int AU = 4;  // row groups (16 B per lane each) in flight per wave
  constexpr int kZBytes = G * kMaxChunkRows * 4;
  constexpr int kUBytes = kZBytes + NWAVE * G * D * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_u[SEL && kUnitSelBytes > kUBytes ? kUnitSelBytes : kUBytes];
  float (*s_z)[kMaxChunkRows] = reinterpret_cast<float (*)[kMaxChunkRows]>(s_u);
  float (*s_red)[G][D] = reinterpret_cast<float (*)[G][D]>(s_u + kZBytes);
  __shared__ int s_rows[kMaxChunkRows];
  __shared__ float s_ml[G][2];
  __shared__ float s_qd[SEL ? kMaxR : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane % LPR, rsub = lane / LPR;
  // sgrp > 1 (per-head selection): a streaming unit serves the sgrp = G
  // consecutive head pairs of one KV group (G here is that group size, the
  // index groups hold one head each), so the group's rows are read once
  const int n_ret = g.attn_mode == 2 ? 0 : n_ret_pairs(g);
  const int n_str = g.attn_mode == 1 ? 0 : n_str_pairs(g) / g.sgrp;
  const int n_fac_units = n_ret * g.B * g.nch_f;
  const int n_units = n_fac_units + n_str * g.B * g.nch_s;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const bool fac = u < n_fac_units;
    const int uu = fac ? u : u - n_fac_units;
    const int nchunk = fac ? g.nch_f : g.nch_s;
    const int item = uu / nchunk, chunk = uu - item * nchunk;
    const int pa = item / g.B, b = item - pa * g.B;
    const int pair = fac ? ret_pair(g, pa) : str_pair(g, pa * g.sgrp);
    const int lq = pair / g.Hkv, gi = pair - lq * g.Hkv;
    const int lkv = g.clsa ? 0 : lq;
    // split cache: slab = list position x B + b, a streaming group's rows in its ring
    const bool ring = g.split && !fac;
    const size_t kvs = g.split ? (size_t)(pa * (fac ? 1 : g.sgrp)) * g.B + b : kv_slice(g, lkv, b, gi);
    const size_t rows_per = ring ? (size_t)g.scap : (size_t)g.tstride;
    const E* kb = (const E*)(ring ? g.k_str : g.k) + kvs * rows_per * D;
    const E* vb = (const E*)(ring ? g.v_str : g.v) + kvs * rows_per * D;
    __syncthreads();
    int nrows;
    if (fac) {
      const int iitem = g.idx_bmajor ? b * g.Hkv + gi : (g.clsa ? gi * g.B + b : pa * g.B + b);
      nrows = min(g.cf, g.n_fac - chunk * g.cf);
      if constexpr (SEL) {
        int32_t* ox = g.idx_out ? g.idx_out + (((size_t)lq * g.B + b) * g.Hkv + gi) * g.n_fac : nullptr;
        unit_select_rows<E>(g, iitem, chunk * g.cf, nrows, s_rows, ox, s_u, s_qd);
      } else {
        const int32_t* ix = g.idx + (size_t)iitem * g.n_fac + (size_t)chunk * g.cf;
        // indices come from select_c and are always in [0, T); the clamp only
        // keeps a corrupted workspace from turning into out-of-range reads
        for (int r = tid; r < nrows; r += NT) s_rows[r] = min(max(ix[r], 0), g.T - 1);
      }
    } else {
      nrows = min(g.cs, g.n_srows - chunk * g.cs);
      for (int r = tid; r < nrows; r += NT) {
        const int v = chunk * g.cs + r;
        const int pos = v < g.s_end ? v : g.w_start + (v - g.s_end);
        // ring slot of a position: the sink as is, the window modulo its size
        s_rows[r] = !ring || pos < g.n_sink ? pos : g.n_sink + (pos - g.n_sink) % g.window;
      }
    }
    float qr[G][CPL];
    // the unit's first query head: index groups of G heads, or of one head each (sgrp > 1)
    const int qh0 = g.sgrp > 1 ? gi : gi * G;
    const E* qp = (const E*)g.q + (((size_t)lq * g.B + b) * g.Hq + (size_t)qh0) * D + slot * CPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      Vec<E>::cvt(ld16(qp + (size_t)h * D), qr[h]);
#pragma unroll
      for (int c = 0; c < CPL; ++c) qr[h][c] *= kScale;
    }
    // nothing of the unit's set-up (the query, the row indices, the last
    // unit's partial stores) stays pending: the ring's waits then count only
    // row loads, and registers freed by the query need no wait later
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // pass 1: logits (log2 domain) into s_z.  A ring of AU row groups per
    // wave: each is reloaded with the group AU steps ahead as soon as it has
    // been used, so AU - 1 loads stay in flight.  Rows past the end load the
    // last row again (in bounds) and are ignored.
    constexpr int kStep = AU * RPB;
    auto row_ptr = [&](const E* base, int r) {
      return base + (size_t)s_rows[min(r, nrows - 1)] * D + slot * CPL;
    };
    uint4 raw[AU];
    if (nrows > 0) {
      const int r0 = wave * RPW + rsub;
#pragma unroll
      for (int j = 0; j < AU; ++j) raw[j] = ld16_stream(row_ptr(kb, r0 + j * RPB));
    }
    for (int r0 = wave * RPW; r0 < nrows; r0 += kStep) {
#pragma unroll
      for (int j = 0; j < AU; ++j) {
        const int r = r0 + j * RPB + rsub;
        float kf[CPL];
        Vec<E>::cvt(raw[j], kf);
        // the last step loads the first V row groups of pass 2 instead
        const bool more = r0 + kStep < nrows;
        raw[j] = ld16_stream(row_ptr(more ? kb : vb, more ? r + kStep : r - r0 + wave * RPW));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float s = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) s += qr[h][c] * kf[c];
          s = group_sum<LPR>(s);
          if (slot == h && r < nrows) s_z[h][r] = s;
        }
      }
    }
    __syncthreads();
    for (int h = wave; h < G; h += NWAVE) {
      float m = -INFINITY;
      for (int r = lane; r < nrows; r += 64) m = fmaxf(m, s_z[h][r]);
      m = wave_max(m);
      float l = 0.f;
      for (int r = lane; r < nrows; r += 64) {
        const float p = exp2f(s_z[h][r] - m);
        s_z[h][r] = p;
        l += p;
      }
      l = wave_sum(l);
      if (lane == 0) {
        s_ml[h][0] = m;
        s_ml[h][1] = l;
      }
    }
    __syncthreads();
    // pass 2: acc += p v (the ring already holds the first V row groups)
    float acc[G][CPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[h][c] = 0.f;
    for (int r0 = wave * RPW; r0 < nrows; r0 += kStep) {
#pragma unroll
      for (int j = 0; j < AU; ++j) {
        const int r = r0 + j * RPB + rsub;
        float vf[CPL];
        Vec<E>::cvt(raw[j], vf);
        raw[j] = ld16_stream(row_ptr(vb, r + kStep));
        // rows past the end weigh 0 (no branch, so the conversion stays
        // ahead of the reload and the ring's registers are not copied)
        const bool live = r < nrows;
        const int rr = live ? r : 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float z = s_z[h][rr];
          const float p = live ? z : 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[h][c] += p * vf[c];
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the ring order: each step waits for its own loads only
      }
    }
    // sum over the row groups of the wave (lanes LPR, 2 LPR, ... apart)
    static_assert(LPR >= 8 && LPR <= 32, "row groups of 8 to 32 lanes");
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float x = acc[h][c];
        if constexpr (LPR <= 8) x += dpp<0x128>(x);  // row_ror:8 = lane ^ 8 within a row
        if constexpr (LPR <= 16) x = xor16_sum(x);
        x = xor32_sum(x);
        acc[h][c] = x;
      }
    if (rsub == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < CPL; ++c) s_red[wave][h][slot * CPL + c] = acc[h][c];
    }
    __syncthreads();
    // head h's partial: item a + h / g.G (heads past an index group's g.G
    // belong to the next item when sgrp > 1), slot h % g.G
    const size_t a = ((size_t)lq * g.B + b) * g.Hkv + gi;
    auto part_of = [&](int h) {
      return g.part + (((a + (size_t)(h / g.G)) * g.nparts + chunk) * g.G + (size_t)(h % g.G)) * (size_t)(D + 4);
    };
    for (int e = tid; e < G * D; e += NT) {
      const int h = e / D, c = e - h * D;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) s += s_red[w][h][c];
      part_of(h)[c] = s;
    }
    if (tid < G) {
      part_of(tid)[D] = s_ml[tid][0];
      part_of(tid)[D + 1] = s_ml[tid][1];
    }
  }
}

// ------------------------------------------------------------------ merge
// Merge of the chunk partials, one thread per output element (small steps:
// more threads in flight than the vector form).
__global__ __launch_bounds__(NT) void merge_scalar_kernel(Geo g) {
  const size_t total = (size_t)g.Lq * g.B * g.Hkv * g.G * g.d;
  const int dd = g.d + 4;
  for (size_t e = (size_t)blockIdx.x * NT + threadIdx.x; e < total; e += (size_t)gridDim.x * NT) {
    const int c = (int)(e % g.d);
    const size_t r = e / g.d;
    const int h = (int)(r % g.G);
    const size_t a = r / g.G;
    const int gi = (int)(a % g.Hkv);
    const size_t lb = a / g.Hkv;
    const int b = (int)(lb % g.B);
    const int lq = (int)(lb / g.B);
    const int np = label_at(g, lq * g.Hkv + gi) ? g.nch_f : g.nch_s;
    const float* pp = g.part + (a * g.nparts * g.G + h) * (size_t)dd;
    const size_t stride = (size_t)g.G * dd;
    float M = -INFINITY, L = 0.f, O = 0.f;
#pragma unroll 8
    for (int s = 0; s < np; ++s) {
      const float* q = pp + s * stride;
      const float ms = q[g.d], ls = q[g.d + 1], as = q[c];
      const float Mn = fmaxf(M, ms);
      const float f_old = exp2f(M - Mn), f_new = exp2f(ms - Mn);
      L = L * f_old + ls * f_new;
      O = O * f_old + as * f_new;
      M = Mn;
    }
    g.out[(((size_t)lq * g.B + b) * g.Hq + (size_t)gi * g.G + h) * g.d + c] = O / L;
  }
}

__global__ __launch_bounds__(NT) void merge_kernel(Geo g) {
  // (large steps) one thread per 4 channels of one head of one attention item: d/4 and G
  // are powers of two, so the thread's (item, head, channel block) come from
  // shifts; the partials and the output move as 16-byte vectors
  const int sh_c = g.d == 128 ? 5 : 4;                   // log2(d / 4)
  const int sh_h = g.G == 8 ? 3 : g.G == 4 ? 2 : g.G == 2 ? 1 : 0;
  const int sh_i = sh_c + sh_h;                          // log2(G * d / 4)
  const long long total = ((long long)g.Lq * g.B * g.Hkv) << sh_i;
  const int dd = g.d + 4;
  for (long long e = (long long)blockIdx.x * NT + threadIdx.x; e < total; e += (long long)gridDim.x * NT) {
    const int a = (int)(e >> sh_i);
    const int rem = (int)(e & ((1 << sh_i) - 1));
    const int h = rem >> sh_c, c = (rem & ((1 << sh_c) - 1)) * 4;
    const int gi = a % g.Hkv, lb = a / g.Hkv;
    const int b = lb % g.B, lq = lb / g.B;
    const int np = label_at(g, lq * g.Hkv + gi) ? g.nch_f : g.nch_s;
    const float* pp = g.part + ((size_t)a * g.nparts * g.G + h) * (size_t)dd;
    const size_t stride = (size_t)g.G * dd;
    // single pass, online log-sum-exp; partial loads are independent of the
    // running state, so unrolling keeps several in flight
    float M = -INFINITY, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int s = 0; s < np; ++s) {
      const float* q = pp + s * stride;
      const float ms = q[g.d], ls = q[g.d + 1];
      const float4 as = *reinterpret_cast<const float4*>(q + c);
      const float Mn = fmaxf(M, ms);
      const float f_old = exp2f(M - Mn), f_new = exp2f(ms - Mn);
      L = L * f_old + ls * f_new;
      O.x = O.x * f_old + as.x * f_new;
      O.y = O.y * f_old + as.y * f_new;
      O.z = O.z * f_old + as.z * f_new;
      O.w = O.w * f_old + as.w * f_new;
      M = Mn;
    }
    *reinterpret_cast<float4*>(g.out + (((size_t)lq * g.B + b) * g.Hq + (size_t)gi * g.G + h) * g.d + c) =
        make_float4(O.x / L, O.y / L, O.z / L, O.w / L);
  }
}

// ------------------------------------------------------------------ CLSA attention
// Shared-index retrieval attention on the matrix cores.  With one index per
// (sequence, group) the N >= 2 layers' G query heads -- QV = N*G <= 32 query
// vectors -- all attend to the same gathered rows, a dense contraction:
//   S[qv][row] = Q[qv][:] . K[row][:]       (bf16 MFMA 32x32x16, fp32 sums)
//   P = softmax over the unit's rows per qv (fp32, in LDS)
//   O[qv][d]   = sum_row P[qv][row] V[row][d]
// P V also runs on bf16 MFMA: P = P_hi + P_lo, P_hi the upper 16 bits of P
// and P_lo those of the exact remainder P - P_hi, so the product keeps P to a
// relative error below 2^-14 (V is bf16 already) and accumulates in fp32.
// One unit = (group, sequence, chunk of ROWS selected rows) run by ROWS * 2
// threads: 128 rows and four waves, or 256 rows and eight waves (the units
// that also select); its K and V rows are gathered into LDS once, and P
// reuses the K tile's LDS once S is computed.  Wave w owns row block w for S
// and, for O, channel block w % 4 over row part w / 4 (with eight waves the
// two parts are summed through LDS).  MFMA 32x32: A element (lane%32,
// k-slice lane/32), B element (k-slice lane/32, lane%32), result (8*(r/4) +
// 4*(lane/32) + r%4, lane%32) in register r.  Layers labelled streaming for
// the group are computed and discarded.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kClsaPad = 136;  // bf16 elements per K/V/Q LDS row (128 + 16 B of padding)
// LDS of a unit of ROWS rows: the K and V tiles, then the query tile
template <int ROWS>
constexpr int clsa_lds_bytes() { return 2 * ROWS * kClsaPad * 2 + 32 * kClsaPad * 2; }
constexpr int kClsaLdsBytes = clsa_lds_bytes<kClsaRows>();
constexpr int kFusedLdsBytes = clsa_lds_bytes<kFusedRows>();

// The attention of one unit over its nrows gathered rows, whose cache
// positions rows(r) gives (r < nrows; values in [0, T)), into the chunk
// partials.  qreg holds this thread's 16-byte pieces of the query tile (see
// clsa_load_q), already loaded.  lds: clsa_lds_bytes<ROWS>(), 16-byte
// aligned; s_ml/s_lab small LDS arrays.  The caller synchronises before the
// call when lds was in other use.
template <int BT>
__device__ __forceinline__ void clsa_load_q(const Geo& g, int b, int gi, uint4 (&qreg)[32 * 16 / BT]) {
  constexpr int D = 128;
  const int QV = g.Lq * g.G;
  static_assert((32 * 16) % BT == 0, "whole query elements per thread");
#pragma unroll
  for (int i = 0; i < 32 * 16 / BT; ++i) {
    const int e = threadIdx.x + i * BT, qv = min(e >> 4, QV - 1), part = e & 15;
    const int n = qv / g.G, h = qv - n * g.G;
    qreg[i] = ld16((const uint16_t*)g.q + (((size_t)n * g.B + b) * g.Hq + (size_t)gi * g.G + h) * D + part * 8);
  }
}

// Q_FIRST: the query tile goes to LDS before the row loads are issued (its
// registers are then free during the gather; the query loads completed
// earlier); otherwise after them, so its loads overlap theirs.
template <int ROWS, int BT, bool Q_FIRST, class Rows>
__device__ __forceinline__ void clsa_attend_unit(const Geo& g, int b, int gi, int chunk, int nrows, Rows rows,
                                                 const uint4 (&qreg)[32 * 16 / BT], unsigned char* lds,
                                                 float (*s_ml)[2], uint8_t* s_lab) {
  constexpr int D = 128;
  constexpr int NWV = BT / 64;         // waves
  constexpr int QPT = 32 * 16 / BT;    // query tile elements per thread
  constexpr int PP = ROWS + 4;         // floats per P row (16-byte aligned rows)
  constexpr int TILE = ROWS * kClsaPad * 2;  // one K or V tile in LDS
  constexpr int NPART = NWV / 4;       // row parts of P V (four channel blocks)
  constexpr int LPQ = BT / 32;         // softmax lanes per query vector
  constexpr float kScale = 0.08838834764831845f * 1.4426950408889634f;
  static_assert(ROWS == 32 * NWV && (NPART == 1 || NPART == 2), "a 32-row block of S per wave");
  static_assert(ROWS == 16 * LPQ, "16 softmax rows per lane");
  static_assert(32 * PP * sizeof(float) + (NPART - 1) * 4 * 16 * 64 * sizeof(float) <= TILE,
                "P (and the second row part of O) fit the K tile");
  uint16_t (*s_k)[kClsaPad] = reinterpret_cast<uint16_t (*)[kClsaPad]>(lds);
  float (*s_p)[PP] = reinterpret_cast<float (*)[PP]>(lds);
  uint16_t (*s_v)[kClsaPad] = reinterpret_cast<uint16_t (*)[kClsaPad]>(lds + TILE);
  uint16_t (*s_q)[kClsaPad] = reinterpret_cast<uint16_t (*)[kClsaPad]>(lds + 2 * TILE);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int QV = g.Lq * g.G;
  const size_t kvs = (size_t)b * g.Hkv + gi;
  const uint16_t* kb = (const uint16_t*)g.k + kvs * (size_t)g.T * D;
  const uint16_t* vb = (const uint16_t*)g.v + kvs * (size_t)g.T * D;
  // every K and V element of the tile (16 bytes per element e = row * 16 +
  // part) is loaded unconditionally (rows past the end read the last valid
  // one, then store zeros), so the loads issue as one group
  static_assert(ROWS * 16 == 8 * BT, "eight tile elements per thread");
  auto store_q = [&]() {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = tid + i * BT;
      *reinterpret_cast<uint4*>(&s_q[e >> 4][(e & 15) * 8]) = (e >> 4) < QV ? qreg[i] : make_uint4(0, 0, 0, 0);
    }
  };
  if constexpr (Q_FIRST) store_q();
  // K and V rows through buffer loads: one 32-bit byte offset per element
  // serves both slices (their bases sit in scalar resource descriptors), and
  // the hardware returns zeros past the slice instead of reading outside it
  const __amdgpu_buffer_rsrc_t k_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), 0,
                                                                        g.T * D * 2, kBufRsrcWord3);
  const __amdgpu_buffer_rsrc_t v_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), 0,
                                                                        g.T * D * 2, kBufRsrcWord3);
  int off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    // positions come from the selection and lie in [0, T); the clamp only
    // keeps a corrupted index from reading another row of the slice
    const int r = min((tid + u * BT) >> 4, nrows - 1);
    off[u] = min(max(rows(r), 0), g.T - 1) * (D * 2) + ((tid + u * BT) & 15) * 16;
  }
  uint4 rk[8], rv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    rk[u] = buf_load16_stream(k_rs, off[u]);
    rv[u] = buf_load16_stream(v_rs, off[u]);
  }
  if (tid < 32) s_lab[tid] = tid < QV ? (uint8_t)label_at(g, (tid / g.G) * g.Hkv + gi) : (uint8_t)0;
  if constexpr (!Q_FIRST) store_q();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = tid + u * BT, r = e >> 4;
    const bool live = r < nrows;
    *reinterpret_cast<uint4*>(&s_k[r][(e & 15) * 8]) = live ? rk[u] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&s_v[r][(e & 15) * 8]) = live ? rv[u] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  // S = Q K^T for row block `wave`, then (the K tile being free) into s_p
  {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int kofs = (lane >> 5) * 8;
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 16) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&s_q[lane & 31][k0 + kofs]);
      const bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&s_k[wave * 32 + (lane & 31)][k0 + kofs]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
    }
    __syncthreads();
    const int row = wave * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qv = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      s_p[qv][row] = row < nrows ? acc[r] * kScale : -INFINITY;
    }
  }
  __syncthreads();
  // softmax: LPQ consecutive lanes per query vector, 16 rows each
  {
    const int qv = tid / LPQ, seg = tid % LPQ;
    float4* pr = reinterpret_cast<float4*>(&s_p[qv][seg * 16]);
    float z[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v4 = pr[i];
      z[4 * i] = v4.x;
      z[4 * i + 1] = v4.y;
      z[4 * i + 2] = v4.z;
      z[4 * i + 3] = v4.w;
    }
    float m = z[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, z[i]);
    m = group_max<LPQ>(m);
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      z[i] = exp2f(z[i] - m);
      l += z[i];
    }
    l = group_sum<LPQ>(l);
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = make_float4(z[4 * i], z[4 * i + 1], z[4 * i + 2], z[4 * i + 3]);
    if (seg == 0) {
      s_ml[qv][0] = m;
      s_ml[qv][1] = l;
    }
  }
  __syncthreads();
  // O = P V for channel block cb over row part rp, P split into bf16 hi +
  // lo: a pair of values packs the upper halves of two words in one byte
  // permute
  const int cb = wave & 3, rp = wave >> 2;
  const int dcol = cb * 32 + (lane & 31);
  f32x16_t o;
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = 0.f;
  {
    constexpr int RW = ROWS / NPART;
    const int ks = (lane >> 5) * 8;
#pragma unroll 2
    for (int k0 = rp * RW; k0 < rp * RW + RW; k0 += 16) {
      const float4 p0 = *reinterpret_cast<const float4*>(&s_p[lane & 31][k0 + ks]);
      const float4 p1 = *reinterpret_cast<const float4*>(&s_p[lane & 31][k0 + ks + 4]);
      const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      constexpr uint32_t kUpperHalves = 0x07060302u;  // bytes 2-3 of the second operand, then of the first
      uint32_t hw[4], lw[4];
      u16x8_t vv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = __float_as_uint(pv[2 * i]), c = __float_as_uint(pv[2 * i + 1]);
        hw[i] = __builtin_amdgcn_perm(c, a, kUpperHalves);
        const float la = pv[2 * i] - __uint_as_float(a & 0xFFFF0000u);
        const float lc = pv[2 * i + 1] - __uint_as_float(c & 0xFFFF0000u);
        lw[i] = __builtin_amdgcn_perm(__float_as_uint(lc), __float_as_uint(la), kUpperHalves);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) vv[i] = s_v[k0 + ks + i][dcol];
      const bf16x8_t vb8 = __builtin_bit_cast(bf16x8_t, vv);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, hw), vb8, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, lw), vb8, o, 0, 0, 0);
    }
  }
  if constexpr (NPART == 2) {
    // the second row part's sums through the K tile's LDS behind P
    float* s_o = reinterpret_cast<float*>(lds + 32 * PP * sizeof(float));
    if (rp == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_o[(cb * 16 + r) * 64 + lane] = o[r];
    }
    __syncthreads();
    if (rp == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] += s_o[(cb * 16 + r) * 64 + lane];
    }
  }
  // partials: acc for (layer, head) = qv, channel block cb
  if (rp == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qv = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (s_lab[qv]) {  // 0 past QV
        const int n = qv / g.G, h = qv - n * g.G;
        const size_t a = ((size_t)n * g.B + b) * g.Hkv + gi;
        g.part[(((a * g.nparts + chunk) * g.G) + h) * (size_t)(D + 4) + dcol] = o[r];
      }
    }
  }
  if (tid < QV && s_lab[tid]) {
    const int n = tid / g.G, h = tid - n * g.G;
    const size_t a = ((size_t)n * g.B + b) * g.Hkv + gi;
    float* pp = g.part + (((a * g.nparts + chunk) * g.G) + h) * (size_t)(D + 4);
    pp[D] = s_ml[tid][0];
    pp[D + 1] = s_ml[tid][1];
  }
}

// The shared-index attention over an index already in g.idx (the final
// kernel's, or a caller's for fac_attend).
__global__ __launch_bounds__(NT) void attn_clsa_mfma_kernel(Geo g) {
  __shared__ __attribute__((aligned(16))) unsigned char s_lds[kClsaLdsBytes];
  __shared__ float s_ml[32][2];
  __shared__ uint8_t s_lab[32];  // per query vector: its layer attends (retrieval label)
  const int J = g.Hkv * g.B * g.nch_f;
  for (int j = blockIdx.x; j < J; j += gridDim.x) {
    const int chunk = j % g.nch_f;
    const int r2 = j / g.nch_f;
    const int b = r2 % g.B, gi = r2 / g.B;
    const size_t iitem = g.idx_bmajor ? (size_t)b * g.Hkv + gi : (size_t)gi * g.B + b;
    const int32_t* ix = g.idx + iitem * g.n_fac + (size_t)chunk * g.cf;
    const int nrows = min(g.cf, g.n_fac - chunk * g.cf);
    __syncthreads();
    uint4 qreg[32 * 16 / NT];
    clsa_load_q<NT>(g, b, gi, qreg);
    clsa_attend_unit<kClsaRows, NT, false>(g, b, gi, chunk, nrows, [&](int r) { return ix[r]; }, qreg, s_lds, s_ml,
                                           s_lab);
  }
}

// Selection fused into the shared-index attention (prefiltered path, T <=
// kShortMaxT): every unit (sequence, group, chunk of kFusedRows rows; eight
// waves and almost all of a CU's LDS, so a CU runs one copy of the
// selection) finds its item's exact top-n_fac cut from the candidates
// itself -- the item's units repeat the same deterministic work side by
// side instead of waiting for one final workgroup -- then takes the
// selected tokens whose ascending rank falls in its chunk, writes those
// idx_out entries, and attends over them.
//   1. candidates -> LDS (from global memory when more than fit), counted
//      in 2048 bins of (key - tau) >> sh as in the final kernel;
//   2. the bin holding the n_fac-th candidate; its members (<= kRankMax)
//      ranked directly, else the general radix threshold: the cut (k*, t*);
//      every selected token is marked in a token bitmap;
//   3. exclusive prefix counts of the bitmap words (u16);
//   4. thread r finds rank r0 + r: the last word whose prefix count is at
//      most that rank, then the set bit of that order inside the word.
// With fewer than n_fac candidates or an overflow, the unit rescores the
// item in full (every unit of the item writes the same score row) and
// selects from it: exact either way.
constexpr int kSelBitmapWords = kShortMaxT / 32;                      // 4096
constexpr int kSelHistBytes = kHistBins * 4;                          // 8 KB: histogram, later u16 prefixes
constexpr int kSelListBytes = kRankMax * 8;                           // 2 KB
constexpr int kSelCandOfs = kSelHistBytes + kSelListBytes + kSelBitmapWords * 4;
constexpr int kSelCandLds = (kFusedLdsBytes - kSelCandOfs) / 8;       // candidates held in LDS
static_assert(kSelBitmapWords * 2 <= kSelHistBytes, "u16 prefixes fit the histogram");
static_assert(kSelCandLds == kFusedSelCand, "the host sizes the fused selection with this capacity");
static_assert(kFusedRows <= kFusedThreads && kFusedRows * 2 == kFusedThreads, "one thread per row of a unit");

__global__ __launch_bounds__(kFusedThreads, 1) void select_attn_clsa_kernel(Geo g) {
  constexpr int BT = kFusedThreads;
  constexpr int NWV = BT / 64;
  __shared__ __attribute__((aligned(16))) unsigned char s_lds[kFusedLdsBytes];
  __shared__ float s_ml[32][2];
  __shared__ uint8_t s_lab[32];
  __shared__ int s_rows[kFusedRows];
  __shared__ int s_w[NWV];
  __shared__ uint32_t s_res[2];
  __shared__ int s_m;
  uint32_t* s_hist = reinterpret_cast<uint32_t*>(s_lds);
  uint16_t* s_pre = reinterpret_cast<uint16_t*>(s_lds);
  uint2* s_list = reinterpret_cast<uint2*>(s_lds + kSelHistBytes);
  uint32_t* s_bm = reinterpret_cast<uint32_t*>(s_lds + kSelHistBytes + kSelListBytes);
  uint2* s_c = reinterpret_cast<uint2*>(s_lds + kSelCandOfs);
  float* s_qd = reinterpret_cast<float*>(s_lds + kSelCandOfs);  // rescoring only: the group query
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the bitmap always spans kShortMaxT tokens (the words past T stay 0), so
  // the prefix scan below has a fixed shape
  constexpr int nrow64 = kSelBitmapWords / (64 * NWV);  // 64-word rows per wave
  constexpr int nwords = kSelBitmapWords;
  const int J = g.Hkv * g.B * g.nch_f;
  for (int j = blockIdx.x; j < J; j += gridDim.x) {
    const int chunk = j % g.nch_f;
    const int r2 = j / g.nch_f;
    const int b = r2 % g.B, gi = r2 / g.B;
    const int item = gi * g.B + b;  // index item (pidx = gi in the shared-index mode)
    const int r0 = chunk * g.cf;
    const int nrows = min(g.cf, g.n_fac - r0);
    int32_t* ox = g.idx_out ? g.idx_out + ((size_t)b * g.Hkv + gi) * g.n_fac : nullptr;
    __syncthreads();
    uint4 qreg[32 * 16 / BT];
    clsa_load_q<BT>(g, b, gi, qreg);  // in flight during the selection
    const uint32_t count = g.info[(size_t)item * 4 + 2];
    const uint2 th = g.tau[item];
    for (int w = tid; w < nwords; w += BT) s_bm[w] = 0u;
    for (int i = tid; i < kHistBins; i += BT) s_hist[i] = 0u;
    if (tid == 0) s_m = 0;
    auto mark = [&](uint32_t t) { atomicOr(&s_bm[t >> 5], 1u << (t & 31)); };
    // the general cut (key desc, token asc) over any source, every selected
    // token marked
    auto cut_general = [&](const SelSrcT<BT>& src) {
      uint32_t kstar, tstar;
      exact_threshold<BT>(src, (uint32_t)g.n_fac, s_hist, s_w, s_res, kstar, tstar);
      src.for_each([&](uint32_t k, uint32_t t) {
        if (k > kstar || (k == kstar && t <= tstar)) mark(t);
      });
    };
    // the cut inside the first-digit bin `ub` that holds the n_fac-th
    // candidate: everything above it is selected, its members (m <=
    // kRankMax) are ranked against each other
    auto cut_binned = [&](const auto& src, uint32_t tau, int sh, uint32_t ub, uint32_t above) {
      src.for_each([&](uint32_t k, uint32_t t) {
        const uint32_t d = min((k - tau) >> sh, (uint32_t)kHistBins - 1u);
        if (d > ub) mark(t);
        const bool mem = d == ub;
        const uint64_t bal = __ballot(mem);
        if (bal) {  // one reservation per wave, by its first active lane (the
                    // strided loop's tail runs with part of the wave)
          const int leader = __builtin_amdgcn_readfirstlane(lane);
          int base = 0;
          if (lane == leader) base = atomicAdd(&s_m, __popcll(bal));
          base = __builtin_amdgcn_readfirstlane(base);
          if (mem) s_list[base + mbcnt(bal)] = make_uint2(k, t);
        }
      });
      __syncthreads();
      const uint32_t need = (uint32_t)g.n_fac - above;
      const int m = s_m;
      for (int i = tid; i < m; i += BT) {
        const uint2 me = s_list[i];
        uint32_t r = 0;
#pragma unroll 8
        for (int q = 0; q < m; ++q) {
          const uint2 o = s_list[q];
          r += before(o, me);
        }
        if (r < need) mark(me.y);
      }
    };
    if (count >= (uint32_t)g.n_fac && count <= (uint32_t)g.cand_cap) {
      const uint32_t tau = th.x;
      const uint32_t span = th.y > tau ? th.y - tau : 0u;
      const int bits = span ? 32 - __clz(span) : 0;
      const int sh = bits > 11 ? bits - 11 : 0;
      const bool in_lds = count <= (uint32_t)kSelCandLds;
      const uint2* gc = g.cand + (size_t)item * g.cand_cap;
      __syncthreads();
      // candidates -> LDS when they fit, counted by their first digit
      const uint4* c4 = reinterpret_cast<const uint4*>(gc);
      const int n4 = (int)(count + 1) / 2;
      constexpr int kLd = 8;  // 16-byte loads in flight per thread: up to 4096 candidates in one round
      for (int i0 = tid; i0 < n4; i0 += kLd * BT) {
        uint4 r[kLd];
#pragma unroll
        for (int q = 0; q < kLd; ++q) r[q] = i0 + q * BT < n4 ? c4[i0 + q * BT] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < kLd; ++q) {
          const int i = i0 + q * BT;
          if (i < n4) {
            if (in_lds) s_c[2 * i] = make_uint2(r[q].x, r[q].y);
            atomicAdd(&s_hist[min((r[q].x - tau) >> sh, (uint32_t)kHistBins - 1u)], 1u);
            if (2 * i + 1 < (int)count) {
              if (in_lds) s_c[2 * i + 1] = make_uint2(r[q].z, r[q].w);
              atomicAdd(&s_hist[min((r[q].z - tau) >> sh, (uint32_t)kHistBins - 1u)], 1u);
            }
          }
        }
      }
      __syncthreads();
      int bin;
      uint32_t above;
      find_bin_top<BT>(s_hist, kHistBins, (uint32_t)g.n_fac, s_w, s_res, bin, above);
      const uint32_t members = s_hist[bin];
      __syncthreads();
      const SelSrcT<BT> gsrc{in_lds ? s_c : gc, nullptr, (int)count};
      if (bin < kHistBins - 1 && members <= (uint32_t)kRankMax) {
        if (in_lds)
          cut_binned(LdsPairsT<BT>{s_c, (int)count}, tau, sh, (uint32_t)bin, above);
        else
          cut_binned(gsrc, tau, sh, (uint32_t)bin, above);
      } else {
        cut_general(gsrc);
      }
    } else {
      // rescoring: the item's full score row (the same values from every unit)
      __syncthreads();
      const size_t slice = group_query_dom<uint16_t>(g, item, s_qd);
      __syncthreads();
      const uint16_t* kd = (const uint16_t*)g.kdom + slice * (size_t)g.tstride * g.R;
      float* sc = g.scores + (size_t)item * g.Ts;
      for (int t = tid; t < g.T; t += BT) sc[t] = score_one<uint16_t>(kd + (size_t)t * g.R, s_qd, g.R);
      __threadfence();
      __syncthreads();
      cut_general(SelSrcT<BT>{nullptr, sc, g.T});
    }
    __syncthreads();
    // exclusive prefix counts of the bitmap words: each wave a contiguous
    // share, lane L on word L of each 64-word row; the rows' scans are
    // independent, then carried through
    {
      const uint32_t* wb = s_bm + wave * nrow64 * 64;
      uint32_t x[nrow64], inc[nrow64];
      uint32_t tot = 0;
#pragma unroll
      for (int k = 0; k < nrow64; ++k) {
        x[k] = (uint32_t)__popc(wb[k * 64 + lane]);
        inc[k] = wave_incl_scan_u(x[k]);
        tot += (uint32_t)__builtin_amdgcn_readlane((int)inc[k], 63);
      }
      if (lane == 0) s_w[wave] = (int)tot;
      __syncthreads();  // the histogram (aliased by the prefixes) is free since the cut
      uint32_t carry = 0;
      for (int w = 0; w < wave; ++w) carry += (uint32_t)s_w[w];
      uint16_t* wp = s_pre + wave * nrow64 * 64;
#pragma unroll
      for (int k = 0; k < nrow64; ++k) {
        wp[k * 64 + lane] = (uint16_t)(carry + inc[k] - x[k]);
        carry += (uint32_t)__builtin_amdgcn_readlane((int)inc[k], 63);
      }
    }
    __syncthreads();
    // rank r0 + tid: the last word whose prefix count is at most it, then
    // the set bit of that order inside the word
    if (tid < nrows) {
      const uint32_t rank = (uint32_t)(r0 + tid);
      int lo = 0, hi = nwords - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((uint32_t)s_pre[mid] <= rank) lo = mid;
        else hi = mid - 1;
      }
      const int t = lo * 32 + nth_set_bit(s_bm[lo], (int)(rank - s_pre[lo]));
      s_rows[tid] = t;
      if (ox) ox[rank] = t;
    }
    __syncthreads();
    clsa_attend_unit<kFusedRows, BT, true>(g, b, gi, chunk, nrows, [&](int r) { return s_rows[r]; }, qreg, s_lds,
                                           s_ml, s_lab);
  }
}

// ------------------------------------------------------------------ kdom_pack
template <typename E>
__global__ __launch_bounds__(NT) void kdom_pack_kernel(Geo g, E* __restrict__ kd) {
  // One work item = (slice, tile of 32 KB of cache rows): the tile is read
  // whole (16-byte nontemporal loads, all issued before any is used) into
  // LDS, then each thread gathers 16-byte output vectors of dominant-chunk
  // channels.
  constexpr int EPV = 16 / (int)sizeof(E);
  constexpr int kTileVec = 8 * NT;  // 16-byte vectors per tile (32 KB)
  __shared__ uint4 s_rows[kTileVec];
  __shared__ int s_chn[kMaxR];  // the slice's source channel of each output element (-1: zero padding)
  const int vpr = g.d * (int)sizeof(E) / 16;  // 16-byte vectors per cache row (8, 16 or 32)
  const int tt = kTileVec / vpr;              // tokens per tile
  const int ovt = g.R / EPV;                  // 16-byte output vectors per token
  const int n_slices = g.Lkv * g.B * g.Hkv;
  const int n_tiles = (g.T + tt - 1) / tt;
  const long long n_work = (long long)n_slices * n_tiles;
  const int hd = g.d / 2;
  // the next tile's rows are loaded into registers while this one is gathered
  auto load_tile = [&](long long w, uint4* r) {
    const int s = (int)(w / n_tiles), tile = (int)(w - (long long)s * n_tiles);
    const int t0 = tile * tt, nv = min(tt, g.T - t0) * vpr;
    const uint4* src = reinterpret_cast<const uint4*>((const E*)g.k + ((size_t)s * g.T + t0) * g.d);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = threadIdx.x + j * NT;
      r[j] = v < nv ? ld16_stream(src + v) : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 r[8];
  if (blockIdx.x < n_work) load_tile(blockIdx.x, r);
  int cur = -1;  // slice whose channel list s_chn holds (uniform in the workgroup)
  for (long long w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int s = (int)(w / n_tiles), tile = (int)(w - (long long)s * n_tiles);
    const int t0 = tile * tt, nt = min(tt, g.T - t0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) s_rows[threadIdx.x + j * NT] = r[j];
    if (s != cur) {
      const int gi = s % g.Hkv, l = s / (g.Hkv * g.B);
      const int32_t* dom = g.i_dom + ((size_t)l * g.Hkv + gi) * g.n_dom;
      for (int e = threadIdx.x; e < g.R; e += NT) {
        int c = -1;
        if (e < 2 * g.n_dom) {
          const int f = min(max(dom[e >> 1], 0), hd - 1), cc = e & 1;  // as in group_query_dom
          c = g.interleaved ? 2 * f + cc : f + cc * hd;
        }
        s_chn[e] = c;
      }
      cur = s;
    }
    __syncthreads();
    if (w + gridDim.x < n_work) load_tile(w + gridDim.x, r);
    for (int o = threadIdx.x; o < nt * ovt; o += NT) {
      const int tok = o / ovt, part = o - tok * ovt;
      const E* row = reinterpret_cast<const E*>(s_rows + tok * vpr);
      E vals[EPV];
#pragma unroll
      for (int q = 0; q < EPV; ++q) {
        const int c = s_chn[part * EPV + q];
        vals[q] = c >= 0 ? row[c] : E(0);
      }
      uint4 packed;
      __builtin_memcpy(&packed, vals, sizeof(packed));
      // streaming store: the copy is read by later decode steps, not by this kernel
      const u32x4 pv = {packed.x, packed.y, packed.z, packed.w};
      __builtin_nontemporal_store(pv, reinterpret_cast<u32x4*>(kd + ((size_t)s * g.T + t0 + tok) * g.R + part * EPV));
    }
  }
}

template <typename E, int D, bool SEL>
hipError_t launch_attn_g(const Geo& g, int grid, hipStream_t s) {
  switch (g.G * g.sgrp) {
    case 1: attn_kernel<E, D, 1, SEL><<<grid, NT, 0, s>>>(g); break;
    case 2: attn_kernel<E, D, 2, SEL><<<grid, NT, 0, s>>>(g); break;
    case 4: attn_kernel<E, D, 4, SEL><<<grid, NT, 0, s>>>(g); break;
    case 8: attn_kernel<E, D, 8, SEL><<<grid, NT, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool SEL = false>
hipError_t launch_attn(const Geo& g, int grid, hipStream_t s) {
  if (g.bf16)
    return g.d == 128 ? launch_attn_g<uint16_t, 128, SEL>(g, grid, s) : launch_attn_g<uint16_t, 64, SEL>(g, grid, s);
  return g.d == 128 ? launch_attn_g<float, 128, SEL>(g, grid, s) : launch_attn_g<float, 64, SEL>(g, grid, s);
}

template <typename E, int MODE>
hipError_t launch_tip_v(const Geo& g, int grid, hipStream_t s) {
  const int V = g.R * (int)sizeof(E) / 16;
  switch (V) {
    case 1: tip_kernel<E, 1, MODE><<<grid, NT, 0, s>>>(g); break;
    case 2: tip_kernel<E, 2, MODE><<<grid, NT, 0, s>>>(g); break;
    case 4: tip_kernel<E, 4, MODE><<<grid, NT, 0, s>>>(g); break;
    case 8: tip_kernel<E, 8, MODE><<<grid, NT, 0, s>>>(g); break;
    case 16: tip_kernel<E, 16, MODE><<<grid, NT, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Scoring workgroups of the in-unit tau mode resident per CU (the occupancy
// query, once per element type and row width).
template <typename E, int V>
int tip_resident_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, tip_kernel<E, V, 3>, NT, 0) != hipSuccess) b = 0;
    return b;
  }();
  return n;
}
template <typename E>
int tip_resident_per_cu(const Geo& g) {
  switch (g.R * (int)sizeof(E) / 16) {
    case 1: return tip_resident_per_cu<E, 1>();
    case 2: return tip_resident_per_cu<E, 2>();
    case 4: return tip_resident_per_cu<E, 4>();
    case 8: return tip_resident_per_cu<E, 8>();
    case 16: return tip_resident_per_cu<E, 16>();
    default: return 0;
  }
}

// Prefiltered scoring with a tau launch when every query head selects its
// own tokens: the hg heads of a KV group share each unit (bf16 caches).
template <int V>
hipError_t launch_tip_heads(const Geo& g, int hg, int grid, hipStream_t s) {
  switch (hg) {
    case 2: tip_kernel<uint16_t, V, 1, 2><<<grid, NT, 0, s>>>(g); break;
    case 4: tip_kernel<uint16_t, V, 1, 4><<<grid, NT, 0, s>>>(g); break;
    case 8: tip_kernel<uint16_t, V, 1, 8><<<grid, NT, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename E, bool PLAN>
hipError_t launch_sample_p(const Geo& g, int grid, hipStream_t s) {
  const int V = g.R * (int)sizeof(E) / 16;
  switch (V) {
    case 1: sample_kernel<E, 1, PLAN><<<grid, NT, 0, s>>>(g); break;
    case 2: sample_kernel<E, 2, PLAN><<<grid, NT, 0, s>>>(g); break;
    case 4: sample_kernel<E, 4, PLAN><<<grid, NT, 0, s>>>(g); break;
    case 8: sample_kernel<E, 8, PLAN><<<grid, NT, 0, s>>>(g); break;
    case 16: sample_kernel<E, 16, PLAN><<<grid, NT, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
// Sampling when every query head selects its own tokens: the hg heads of a
// KV group share each unit (bf16 caches).
template <int V>
hipError_t launch_sample_heads(const Geo& g, int hg, int grid, hipStream_t s) {
  switch (hg) {
    case 2: sample_kernel<uint16_t, V, false, 2><<<grid, NT, 0, s>>>(g); break;
    case 4: sample_kernel<uint16_t, V, false, 4><<<grid, NT, 0, s>>>(g); break;
    case 8: sample_kernel<uint16_t, V, false, 8><<<grid, NT, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <typename E>
hipError_t launch_sample_v(const Geo& g, int grid, hipStream_t s, bool plan) {
  return plan ? launch_sample_p<E, true>(g, grid, s) : launch_sample_p<E, false>(g, grid, s);
}

int clampi(long long v, int lo, int hi) { return (int)(v < lo ? lo : (v > hi ? hi : v)); }

}  // namespace

hipError_t launch_kdom_pack(const Geo& g, void* k_dom, hipStream_t s) {
  const int tt = 8 * NT * 16 / (g.d * (g.bf16 ? 2 : 4));  // tokens per 32 KB tile
  const long long n_work = (long long)g.Lkv * g.B * g.Hkv * ((g.T + tt - 1) / tt);
  const int grid = clampi(n_work, 1, 8 * g.grid);
  KTimer t("kdom_pack", s);
  if (g.bf16)
    kdom_pack_kernel<uint16_t><<<grid, NT, 0, s>>>(g, (uint16_t*)k_dom);
  else
    kdom_pack_kernel<float><<<grid, NT, 0, s>>>(g, (float*)k_dom);
  return hipGetLastError();
}

// kv_append ([AoH] §4: a streaming head keeps only the sink and the recent
// window).  One unit = (layer, KV group, sequence, block of up to 256 new
// rows).  A retrieval group's rows go to its slab at their positions, with
// their dominant-chunk copy; a streaming group keeps the sink positions and
// the last `window` positions of this call, the window in a ring (so no two
// writes of one call share a slot).  A pair's slab is its rank among the
// pairs of its label, counted from the labels before it.
constexpr int kAppendRows = 256;

template <typename E>
__global__ __launch_bounds__(NT) void kv_append_kernel(Geo g, int pos0, int n_new, const E* k_new, const E* v_new,
                                                       E* k_ret, E* v_ret, E* k_dom_ret, E* k_str, E* v_str) {
  constexpr int EPV = Vec<E>::N;
  __shared__ int s_w[NWAVE];
  const int tid = threadIdx.x;
  const int P = g.Lq * g.Hkv;
  const int nb = (n_new + kAppendRows - 1) / kAppendRows;
  const long long n_units = (long long)P * g.B * nb;
  const int nvec = g.d / EPV, hd = g.d / 2;
  for (long long u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int blk = (int)(u % nb);
    const long long pb = u / nb;
    const int b = (int)(pb % g.B), pair = (int)(pb / g.B);
    const int l = pair / g.Hkv, gi = pair - l * g.Hkv;
    int cnt = 0;
    for (int p = tid; p < pair; p += NT) cnt += label_at(g, p);
    int before;
    block_excl_scan(cnt, s_w, before);  // retrieval pairs before this one
    const bool ret = label_at(g, pair);
    const size_t slab = (size_t)(ret ? before : pair - before) * g.B + b;
    const E* ks = k_new + ((((size_t)l * g.B + b) * g.Hkv + gi) * n_new) * g.d;
    const E* vs = v_new + ((((size_t)l * g.B + b) * g.Hkv + gi) * n_new) * g.d;
    const int r0 = blk * kAppendRows, r1 = min(n_new, r0 + kAppendRows);
    if (ret) {
      E* kd = k_ret + slab * g.tstride * g.d;
      E* vd = v_ret + slab * g.tstride * g.d;
      for (int e = tid; e < (r1 - r0) * nvec; e += NT) {
        const int r = r0 + e / nvec, c = e - (e / nvec) * nvec;
        const size_t src = (size_t)r * g.d + (size_t)c * EPV, dst = (size_t)(pos0 + r) * g.d + (size_t)c * EPV;
        *reinterpret_cast<uint4*>(kd + dst) = ld16(ks + src);
        *reinterpret_cast<uint4*>(vd + dst) = ld16(vs + src);
      }
      // dominant-chunk copy, element 2i+c = channel c of chunk i_dom[i] (zero padded)
      const int32_t* dom = g.i_dom + (size_t)pair * g.n_dom;
      E* dd = k_dom_ret + slab * g.tstride * g.R;
      for (int e = tid; e < (r1 - r0) * g.R; e += NT) {
        const int r = r0 + e / g.R, j = e - (e / g.R) * g.R;
        E v = E(0);
        if (j < 2 * g.n_dom) {
          const int f = min(max(dom[j >> 1], 0), hd - 1), cc = j & 1;
          v = ks[(size_t)r * g.d + (g.interleaved ? 2 * f + cc : f + cc * hd)];
        }
        dd[(size_t)(pos0 + r) * g.R + j] = v;
      }
    } else {
      E* kd = k_str + slab * g.scap * g.d;
      E* vd = v_str + slab * g.scap * g.d;
      const int keep_from = pos0 + n_new - g.window;  // the last `window` positions of this call
      for (int e = tid; e < (r1 - r0) * nvec; e += NT) {
        const int r = r0 + e / nvec, c = e - (e / nvec) * nvec;
        const int pos = pos0 + r;
        if (pos >= g.n_sink && pos < keep_from) continue;
        const int slot = pos < g.n_sink ? pos : g.n_sink + (pos - g.n_sink) % g.window;
        const size_t src = (size_t)r * g.d + (size_t)c * EPV, dst = (size_t)slot * g.d + (size_t)c * EPV;
        *reinterpret_cast<uint4*>(kd + dst) = ld16(ks + src);
        *reinterpret_cast<uint4*>(vd + dst) = ld16(vs + src);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_kv_append(const Geo& g, int pos0, int n_new, const void* k_new, const void* v_new, void* k_ret,
                            void* v_ret, void* k_dom_ret, void* k_str, void* v_str, hipStream_t s) {
  const long long units = (long long)g.Lq * g.Hkv * g.B * ((n_new + kAppendRows - 1) / kAppendRows);
  const int grid = clampi(units, 1, g.grid);
  KTimer t("kv_append", s);
  if (g.bf16)
    kv_append_kernel<uint16_t><<<grid, NT, 0, s>>>(g, pos0, n_new, (const uint16_t*)k_new, (const uint16_t*)v_new,
                                                   (uint16_t*)k_ret, (uint16_t*)v_ret, (uint16_t*)k_dom_ret,
                                                   (uint16_t*)k_str, (uint16_t*)v_str);
  else
    kv_append_kernel<float><<<grid, NT, 0, s>>>(g, pos0, n_new, (const float*)k_new, (const float*)v_new,
                                                (float*)k_ret, (float*)v_ret, (float*)k_dom_ret, (float*)k_str,
                                                (float*)v_str);
  return hipGetLastError();
}

// Attention units per call up to which the FAC units select for themselves
// (no final-selection launch): about one round of the selecting kernel's
// resident workgroups, two per CU; larger steps repeat the selection in too
// many units.
constexpr long long kSelAttnMaxUnits = 512;
// Streaming rows per call (over all (layer, sequence, group) items) from which
// the streaming attention runs on the side stream.
constexpr long long kSideStreamRows = 1LL << 20;
// Prefiltered scoring units per call (index items x units per item) up to
// which each unit derives tau itself instead of a separate launch.
constexpr long long kTauInlineUnits = 512;
constexpr long long kTauInlineUnitsMax = 4096;
// Tokens per prefiltered scoring unit: the bounds of the sizes chosen.
constexpr long long kTipUnitMinTokens = 1024;
constexpr long long kTipUnitMaxTokens = 16384;
// Output elements per call from which the merge moves 4 per thread in
// 16-byte vectors; below, one per thread keeps more threads in flight.
constexpr long long kMergeVecOutputs = 1LL << 18;

hipError_t launch_decode(const Geo& g0, const StreamSet& ss) {
  hipError_t e;
  const hipStream_t s = ss.main;
  Geo g = g0;
  const long long n_idx_items = (long long)(g.clsa ? g.Hkv : g.Lq * g.Hkv) * g.B;
  const long long n_att_items = (long long)g.Lq * g.Hkv * g.B;
  // the plan launch clears per-item histograms (general path) or counters
  // (prefiltered) and fills the -1 index rows of streaming groups; its grid
  // covers that work, no more
  const long long plan_work =
      g.prefilter ? std::max(n_idx_items, g.idx_out && !g.clsa ? (long long)g.Lq * g.B * g.Hkv * g.n_fac : 0LL)
                  : n_idx_items * kHistBins / 4;
  const int grid_plan = clampi((plan_work + NT - 1) / NT, 1, g.grid);
  const bool any_stream = !(g.clsa && g.labels == nullptr);
  const bool side = any_stream && (long long)n_att_items * g.n_srows >= kSideStreamRows;
  // Without the side stream (which forks right after the plan), the sampling
  // launch builds the plan itself and the plan launch is saved.
  const bool fuse_plan = g.prefilter && !side && !g.host_plan && !g.clsa;
  if (!g.host_plan && !fuse_plan) {
    KTimer t("plan", s);
    plan_kernel<<<grid_plan, NT, 0, s>>>(g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // Streaming groups need nothing but the plan.  When their rows are worth
  // overlapping with scoring, their attention runs on the side stream beside
  // the scoring and selection of retrieval groups; small (latency-bound)
  // steps attend to them in the retrieval attention's launch instead and
  // skip the event waits.  (The shared-index mode without labels has none.)
  if (side) {
    if ((e = hipEventRecord(ss.fork, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss.side, ss.fork, 0)) != hipSuccess) return e;
    {
      Geo gs = g;
      gs.attn_mode = 2;
      gs.sgrp = 1 << g.kv_shift;  // per-head selection: the group's heads share its rows
      const int grid_s = clampi(n_att_items / gs.sgrp * (long long)g.nch_s, 1, g.grid);
      KTimer t("attention_stream", ss.side);
      e = launch_attn(gs, grid_s, ss.side);
    }
    if (e != hipSuccess) return e;
    if ((e = hipEventRecord(ss.join, ss.side)) != hipSuccess) return e;
  }
  // Small prefiltered steps (no side stream, T <= kShortMaxT, one index per
  // KV group, device cache): the FAC units select for themselves, so the
  // final-selection launch is saved.
  const bool sel_attn = g.prefilter && !side && !g.clsa && g.kv_shift == 0 && !g.split && !g.select_only &&
                        g.T <= kShortMaxT &&
                        n_att_items * (long long)(g.nch_f + g.nch_s) <= kSelAttnMaxUnits;
  const int grid_tip = clampi(n_idx_items * g.nch_t, 1, g.grid);
  const int grid_item = clampi(n_idx_items, 1, g.grid);
  // per-query-head selection: a KV group's hg heads share the sampling and
  // scoring units (bf16 caches, steps with a tau launch)
  const int hg = 1 << g.kv_shift;
  // A shared-index step without labels scores every index item, so its
  // scoring units can fill whole rounds of the resident scoring workgroups:
  // the fewest rounds that keep a unit within 16384 tokens (one round for 32
  // items of 131072 tokens), which also derives tau in the fewest units.
  if (g.prefilter && g.clsa && g.labels == nullptr) {
    const int per_cu = g.bf16 ? tip_resident_per_cu<uint16_t>(g) : tip_resident_per_cu<float>(g);
    const long long slots = (long long)(g.grid / 8) * per_cu;  // g.grid: 8 workgroups per CU
    if (slots > 0) {
      const long long cap = kTipUnitMaxTokens;
      const long long rounds = std::max(1LL, (n_idx_items * g.T + slots * cap - 1) / (slots * cap));
      const long long per_item = std::max(1LL, (rounds * slots + n_idx_items - 1) / n_idx_items);
      const long long ct = ((g.T + per_item - 1) / per_item + 63) / 64 * 64;
      g.ct_tip = (int)std::min(std::max(ct, (long long)kTipUnitMinTokens), cap);
      g.nch_tip = (g.T + g.ct_tip - 1) / g.ct_tip;
    }
  }
  // tau inside the scoring units: always up to kTauInlineUnits units; up to
  // kTauInlineUnitsMax (with the ring issued first) when no heads share units
  const long long units_tip = n_idx_items * g.nch_tip;
  const bool tau_early = hg == 1 && units_tip > kTauInlineUnits && units_tip <= kTauInlineUnitsMax;
  const bool tau_inline = units_tip <= kTauInlineUnits || tau_early;
  const int tip_v = g.R * (g.bf16 ? 2 : 4) / 16;
  const bool share = !tau_inline && hg > 1 && g.bf16 && (tip_v == 2 || tip_v == 4 || tip_v == 8);
  const bool share_sample = share && !fuse_plan;  // the plan-building sampler serves one item per unit
  if (g.prefilter) {
    {
      KTimer t("sample", s);
      const int grid_sample = clampi(n_idx_items / (share_sample ? hg : 1) * (kSampleTokens / 256), 1, g.grid);
      if (share_sample)
        e = tip_v == 2 ? launch_sample_heads<2>(g, hg, grid_sample, s)
            : tip_v == 4 ? launch_sample_heads<4>(g, hg, grid_sample, s) : launch_sample_heads<8>(g, hg, grid_sample, s);
      else
        e = g.bf16 ? launch_sample_v<uint16_t>(g, grid_sample, s, fuse_plan)
                   : launch_sample_v<float>(g, grid_sample, s, fuse_plan);
    }
    if (e != hipSuccess) return e;
    if (!tau_inline) {
      KTimer t("tau", s);
      tau_kernel<<<grid_item, NT, 0, s>>>(g);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
      const int grid_tip_pf = clampi(n_idx_items / (share ? hg : 1) * g.nch_tip, 1, g.grid);
      KTimer t("tip_score", s);
      if (share)
        e = tip_v == 2 ? launch_tip_heads<2>(g, hg, grid_tip_pf, s)
            : tip_v == 4 ? launch_tip_heads<4>(g, hg, grid_tip_pf, s) : launch_tip_heads<8>(g, hg, grid_tip_pf, s);
      else if (tau_inline && tau_early)
        e = g.bf16 ? launch_tip_v<uint16_t, 3>(g, grid_tip_pf, s) : launch_tip_v<float, 3>(g, grid_tip_pf, s);
      else if (tau_inline)
        e = g.bf16 ? launch_tip_v<uint16_t, 2>(g, grid_tip_pf, s) : launch_tip_v<float, 2>(g, grid_tip_pf, s);
      else
        e = g.bf16 ? launch_tip_v<uint16_t, 1>(g, grid_tip_pf, s) : launch_tip_v<float, 1>(g, grid_tip_pf, s);
    }
    if (e != hipSuccess) return e;
    if (!g.fuse_sel && !sel_attn) {
      KTimer t("select_final", s);
      if (g.T <= kShortMaxT) {
        if (g.bf16) final_kernel<uint16_t, false><<<grid_item, kFinalThreads, 0, s>>>(g);
        else final_kernel<float, false><<<grid_item, kFinalThreads, 0, s>>>(g);
      } else {
        if (g.bf16) final_kernel<uint16_t, true><<<grid_item, kFinalThreads, 0, s>>>(g);
        else final_kernel<float, true><<<grid_item, kFinalThreads, 0, s>>>(g);
      }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    {
      KTimer t("tip_score", s);
      e = g.bf16 ? launch_tip_v<uint16_t, 0>(g, grid_tip, s) : launch_tip_v<float, 0>(g, grid_tip, s);
    }
    if (e != hipSuccess) return e;
    {
      KTimer t("select_bin", s);
      select_bin_kernel<<<grid_item, NT, 0, s>>>(g);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
      KTimer t("select_a", s);
      select_a_kernel<<<grid_tip, NT, 0, s>>>(g);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
      KTimer t("select_b", s);
      select_b_kernel<<<grid_item, NT, 0, s>>>(g);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
      KTimer t("select_c", s);
      select_c_kernel<<<grid_tip, NT, 0, s>>>(g);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (g.select_only) return hipSuccess;
  {
    // mode 1: retrieval units only; mode 0: retrieval and streaming units
    const bool with_stream = any_stream && !side;
    g.attn_mode = with_stream && !g.clsa_mfma ? 0 : 1;
    KTimer t("attention_fac", s);
    if (g.clsa_mfma) {
      const int grid_c = clampi((long long)g.Hkv * g.B * g.nch_f, 1, g.grid);
      if (g.fuse_sel) {
        KTimer ts("select_attend", s);
        select_attn_clsa_kernel<<<grid_c, kFusedThreads, 0, s>>>(g);
      } else {
        attn_clsa_mfma_kernel<<<grid_c, NT, 0, s>>>(g);
      }
      e = hipGetLastError();
      if (e == hipSuccess && with_stream) {
        Geo gs = g;
        gs.attn_mode = 2;
        e = launch_attn(gs, clampi(n_att_items * (long long)g.nch_s, 1, g.grid), s);
      }
    } else {
      const long long units = n_att_items * (long long)(g.nch_f + (with_stream ? g.nch_s : 0));
      e = sel_attn ? launch_attn<true>(g, clampi(units, 1, g.grid), s) : launch_attn(g, clampi(units, 1, g.grid), s);
    }
  }
  if (e != hipSuccess) return e;
  if (side && (e = hipStreamWaitEvent(s, ss.join, 0)) != hipSuccess) return e;
  const long long n_out = n_att_items * g.G * g.d;
  {
    KTimer t("merge", s);
    if (n_out >= kMergeVecOutputs)  // 4 outputs per thread
      merge_kernel<<<clampi((n_out / 4 + NT - 1) / NT, 1, g.grid), NT, 0, s>>>(g);
    else
      merge_scalar_kernel<<<clampi((n_out + NT - 1) / NT, 1, g.grid), NT, 0, s>>>(g);
  }
  return hipGetLastError();
}

// FAC attention of one layer over a caller's index (batch-major), then the
// merge of the chunk partials.
hipError_t launch_fac_attend(const Geo& g0, hipStream_t s) {
  Geo g = g0;
  g.attn_mode = 1;
  const long long n_att_items = (long long)g.Hkv * g.B;
  {
    KTimer t("attention_fac", s);
    if (g.clsa_mfma) {
      attn_clsa_mfma_kernel<<<clampi(n_att_items * g.nch_f, 1, g.grid), NT, 0, s>>>(g);
    } else {
      const hipError_t e = launch_attn(g, clampi(n_att_items * g.nch_f, 1, g.grid), s);
      if (e != hipSuccess) return e;
    }
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const long long n_out = n_att_items * g.G * g.d;
  {
    KTimer t("merge", s);
    if (n_out >= kMergeVecOutputs)  // 4 outputs per thread
      merge_kernel<<<clampi((n_out / 4 + NT - 1) / NT, 1, g.grid), NT, 0, s>>>(g);
    else
      merge_scalar_kernel<<<clampi((n_out + NT - 1) / NT, 1, g.grid), NT, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace has
