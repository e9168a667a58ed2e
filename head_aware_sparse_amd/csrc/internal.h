// Internal geometry shared by the host launch code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace has {

constexpr int kHistBins = 2048;      // first radix digit: key bits 31..21
constexpr int kCandLds = 8192;       // candidates held in LDS by the threshold pass
constexpr int kMaxChunkRows = 1024;  // attention rows per work unit
constexpr int kClsaRows = 128;       // rows per layer-fused shared-index unit (staged in LDS)
constexpr int kMaxTipChunks = 1024;  // score chunks per item
constexpr int kMaxPairs = 8192;      // (layer, KV group) pairs per call
constexpr int kCandFast = 16384;     // candidates per item on the prefiltered path (LDS)
constexpr int kSampleTokens = 4096;  // tokens scored per item to place the prefilter
constexpr int kPrefilterMaxT = 524288;  // token bitmap of the prefiltered path fits the final kernel's LDS
constexpr int kShortMaxT = 131072;      // up to here the final kernel's token bitmap has an LDS array of its own
constexpr int kSelMaxLong = 8192;       // beyond kShortMaxT: n_fac the final kernel compacts beside its bitmap
constexpr int kFusedSelCand = 15168;    // candidates the selection fused into the shared-index attention holds in LDS
constexpr int kFusedRows = 256;         // rows per unit of that fused kernel (eight waves, one unit per CU)
constexpr int kFusedThreads = 512;

// One decode call, with the workspace carved.  Passed by value to kernels.
struct Geo {
  // shape
  int Lq, Lkv, B, Hq, Hkv, G, d, T, n_fac, n_sink, window, n_dom;
  int R;            // k_dom row elements
  int bf16;         // kv dtype
  int clsa;         // 1: one index per (b, g) shared by Lq layers over one cache
  int clsa_mfma;    // shared-index retrieval attention on the matrix cores (bf16, d 128, 2 <= Lq, Lq*G <= 32)
  int fuse_sel;     // prefiltered shared-index step: the exact selection runs inside the attention units
  int interleaved;  // rope pairing
  int host_plan;    // shared-index mode, no labels, prefiltered: the plan is implicit (no plan launch)
  // chunking
  int ct, nch_t;    // score/select chunk tokens and count per item
  int Ts;           // score row stride (T rounded up to 64)
  int cf, nch_f;    // FAC chunk rows and count per item
  int cs, nch_s;    // stream chunk rows and count per item
  int n_srows, s_end, w_start;  // streaming rows: [0, s_end) U [w_start, T)
  int nparts;       // partial slots per attention item
  int cand_cap;     // candidate slots per index item
  int prefilter;    // 1: sample -> candidates above a threshold -> exact select
  int samp_rank;    // the threshold is the samp_rank-th largest sampled score
  int bm_words;     // words of the per-item token bitmap (T / 32 rounded up)
  int grid;         // persistent grid size
  int attn_mode;    // attention launch: 1 = retrieval (FAC) units, 2 = streaming units
  int select_only;  // stop after the selection (sparse_select)
  int idx_bmajor;   // FAC reads a caller's index laid out [B][Hkv][n_fac] (fac_attend)
  int split;        // split cache: retrieval groups' slabs [n_ret][B][tstride], streaming groups' rings
  int tstride;      // rows per cache (and k_dom) slab: T, or the split cache's capacity
  int scap;         // split cache: rows per streaming ring slab (n_sink + window)
  int kv_shift;     // log2(index groups per KV group): 0, or log2 G when every query head selects its own tokens
  int sgrp;         // query heads per streaming attention unit beyond G: with kv_shift > 0, the KV group's heads (1 otherwise)
  int hkv_kv;       // KV groups per layer (Hkv >> kv_shift)
  // workspace
  int* plan;         // [4 + 3*kMaxPairs]: n_idx_pairs, n_att_ret, n_att_str, -, lists
  uint32_t* hist;    // [idx items][kHistBins]
  uint32_t* info;    // [idx items][4]: b1, count above b1, candidate count, -
  uint2* cand;       // [idx items][cand_cap] (key, token)
  uint32_t* ngt;     // [idx items][nch_t] tokens above the first digit bin per chunk
  uint32_t* off;     // [idx items][nch_t] output offset of each chunk
  uint2* thr;        // [idx items] (key*, token*) selection threshold
  float* scores;     // [idx items][Ts]
  int32_t* idx;      // [idx items][n_fac]
  uint32_t* skeys;   // [idx items][kSampleTokens] sampled TIP keys (prefiltered path)
  uint2* tau;        // [idx items] candidate key threshold and largest sampled key (prefiltered path)
  float* qbar;       // [idx items][R] group query in k_dom channel order (prefiltered path)
  int ct_tip;        // tokens per scoring unit on the prefiltered path
  int nch_tip;       // scoring units per item on the prefiltered path
  float* part;       // [att items][nparts][G][d + 4]: acc[d], m, l
  // inputs / outputs
  const void* q;
  const void* q_index;
  const void* k;
  const void* v;
  const void* kdom;
  const void* k_str;  // split cache: streaming groups' rings [n_str][B][scap][d]
  const void* v_str;
  const int32_t* i_dom;
  const uint8_t* labels;
  float* out;
  int32_t* idx_out;
};


// Brackets one kernel launch with HIP events on its stream while per-kernel
// timing is enabled (has_timing_enable); a no-op otherwise.
struct KTimer {
  KTimer(const char* name, hipStream_t s);
  ~KTimer();
  int slot;
  hipStream_t stream;
};

// The caller's stream plus a library-owned side stream and two events used
// to run the streaming-group attention concurrently with the retrieval chain.
struct StreamSet {
  hipStream_t main;
  hipStream_t side;
  hipEvent_t fork;  // main -> side: the plan is ready
  hipEvent_t join;  // side -> main: streaming attention is done
};

hipError_t launch_kdom_pack(const Geo& g, void* k_dom, hipStream_t s);
hipError_t launch_decode(const Geo& g, const StreamSet& ss);
hipError_t launch_fac_attend(const Geo& g, hipStream_t s);
// Writes positions [pos0, pos0 + n_new) of new K/V rows ([L][B][Hkv][n_new][d])
// into a split cache, with the dominant-chunk copy of retrieval groups' keys.
hipError_t launch_kv_append(const Geo& g, int pos0, int n_new, const void* k_new, const void* v_new, void* k_ret,
                            void* v_ret, void* k_dom_ret, void* k_str, void* v_str, hipStream_t s);

}  // namespace has
