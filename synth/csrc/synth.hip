// Seeded synthetic-input generator shared by the oracle side (host functions)
// and the GPU side (device fill kernels).  It holds none of the attention
// method's arithmetic: only counter-based random numbers, the rotary position
// rotation that turns raw keys/queries into post-RoPE cache contents, and
// fp32 -> bf16 rounding.
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11).  One counter = (e_lo, e_hi, slice,
// tensor id), key = (seed, 0x5EED0001).  A unit-variance deviate is the
// centred Irwin-Hall sum of the four 22-bit words of one Philox output,
// scaled by sqrt(3)/2^22.  Every step is an exact integer operation or one
// correctly rounded fp32 operation, so host and device produce identical bits
// (the library is built with -ffp-contract=off).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <string.h>

#define HD __host__ __device__ static inline

namespace {

constexpr uint32_t kKey1 = 0x5EED0001u;
// fp32 nearest to sqrt(3) / 2^22.
constexpr float kIhScale = 0x1.bb67aep-22f;
constexpr int32_t kIhMean = (1 << 23) - 2;

struct W4 { uint32_t x, y, z, w; };

HD W4 philox4x32_10(W4 c, uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c = W4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

HD W4 draw(uint32_t seed, uint32_t tid, uint32_t slice, uint64_t e) {
  return philox4x32_10(W4{(uint32_t)e, (uint32_t)(e >> 32), slice, tid}, seed, kKey1);
}

HD float ih_unit(uint32_t seed, uint32_t tid, uint32_t slice, uint64_t e) {
  const W4 r = draw(seed, tid, slice, e);
  const uint32_t s = (r.x >> 10) + (r.y >> 10) + (r.z >> 10) + (r.w >> 10);
  const int32_t n = (int32_t)s - kIhMean;  // |n| < 2^23: exact in fp32
  return (float)n * kIhScale;
}

HD uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Raw (pre-rotation) key or value channel.  kind 0 = key: outlier channels
// are scaled by `outlier_mul` and position 0 (the sink) by `sink_mul`.
HD float kv_raw(uint32_t seed, uint32_t tid, uint32_t slice, int t, int c, int d,
                int kind, const uint8_t* outlier_mask, float outlier_mul, float sink_mul) {
  float x = ih_unit(seed, tid, slice, (uint64_t)t * (uint64_t)d + (uint64_t)c);
  if (kind == 0) {
    if (outlier_mask && outlier_mask[c]) x = x * outlier_mul;
    if (t == 0) x = x * sink_mul;
  }
  return x;
}

// Rotate-half rotary rotation of channel c of a d-vector at table row `cs`,
// `sn` (cos/sin of position * theta_f for f < d/2).
HD float rope_rotate(float xc, float xpair, int c, int d, const float* cs, const float* sn) {
  const int h = d / 2;
  if (c < h) {
    const float a = xc * cs[c];
    const float b = xpair * sn[c];
    return a - b;
  }
  const float a = xc * cs[c - h];
  const float b = xpair * sn[c - h];
  return a + b;
}

HD float kv_value(uint32_t seed, uint32_t tid, uint32_t slice, int t, int c, int d, int kind,
                  const uint8_t* outlier_mask, float outlier_mul, float sink_mul,
                  const float* cos_tab, const float* sin_tab) {
  const float x = kv_raw(seed, tid, slice, t, c, d, kind, outlier_mask, outlier_mul, sink_mul);
  if (kind != 0 || cos_tab == nullptr) return x;
  const int h = d / 2;
  const int cp = c < h ? c + h : c - h;
  const float xp = kv_raw(seed, tid, slice, t, cp, d, kind, outlier_mask, outlier_mul, sink_mul);
  return rope_rotate(x, xp, c, d, cos_tab + (size_t)t * h, sin_tab + (size_t)t * h);
}

// Grid (x, slice): one thread per (t, channel-pair) of one slice; writes
// channels c and c + d/2 of row t.
template <typename OutT>
__global__ void kv_fill_kernel(uint32_t seed, uint32_t tid, int kind, int T, int d,
                               const int32_t* __restrict__ slice_ids,
                               const uint8_t* __restrict__ outlier_masks,  // [n_slices, d] or null
                               float outlier_mul, float sink_mul,
                               const float* __restrict__ cos_tab, const float* __restrict__ sin_tab,
                               OutT* __restrict__ out) {
  const int h = d / 2;
  const int s = blockIdx.y;
  const uint32_t per_slice = (uint32_t)T * (uint32_t)h;
  const uint32_t slice = (uint32_t)slice_ids[s];
  const uint8_t* om = outlier_masks ? outlier_masks + (size_t)s * d : nullptr;
  OutT* base = out + (size_t)s * T * d;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < per_slice;
       i += gridDim.x * blockDim.x) {
    const int t = (int)(i / (uint32_t)h);
    const int c = (int)(i - (uint32_t)t * (uint32_t)h);
    const float x0 = kv_raw(seed, tid, slice, t, c, d, kind, om, outlier_mul, sink_mul);
    const float x1 = kv_raw(seed, tid, slice, t, c + h, d, kind, om, outlier_mul, sink_mul);
    float y0 = x0, y1 = x1;
    if (kind == 0 && cos_tab) {
      const float* cs = cos_tab + (size_t)t * h;
      const float* sn = sin_tab + (size_t)t * h;
      y0 = rope_rotate(x0, x1, c, d, cs, sn);
      y1 = rope_rotate(x1, x0, c + h, d, cs, sn);
    }
    OutT* row = base + (size_t)t * d;
    if constexpr (sizeof(OutT) == 2) {
      row[c] = bf16_rne(y0);
      row[c + h] = bf16_rne(y1);
    } else {
      row[c] = y0;
      row[c + h] = y1;
    }
  }
}

}  // namespace

extern "C" {

// Known-answer access to the raw generator (for tests).
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const W4 r = philox4x32_10(W4{ctr[0], ctr[1], ctr[2], ctr[3]}, key[0], key[1]);
  out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
}

// out[i] = unit-variance deviate of element e0 + i of stream (seed, tid, slice).
void synth_ih(uint32_t seed, uint32_t tid, uint32_t slice, uint64_t e0, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ih_unit(seed, tid, slice, e0 + (uint64_t)i);
}

// out[i] = first Philox word of element e0 + i.
void synth_u32(uint32_t seed, uint32_t tid, uint32_t slice, uint64_t e0, int64_t n, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = draw(seed, tid, slice, e0 + (uint64_t)i).x;
}

// Elementwise fp32 -> bf16 round-to-nearest-even (bits).
void synth_bf16_rne(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(in[i]);
}

// cos/sin of pos * base^(-2f/d) for pos < T, f < d/2, evaluated in fp64 and
// rounded to fp32.  Row-major [T, d/2].
void synth_rope_table(int T, int d, double base, float* cos_out, float* sin_out) {
  const int h = d / 2;
  for (int f = 0; f < h; ++f) {
    const double theta = pow(base, -2.0 * (double)f / (double)d);
    for (int t = 0; t < T; ++t) {
      const double a = (double)t * theta;
      cos_out[(size_t)t * h + f] = (float)cos(a);
      sin_out[(size_t)t * h + f] = (float)sin(a);
    }
  }
}

// Rotate-half rotation of n_vec fp32 d-vectors, all at table row `pos`.
void synth_rope_apply(const float* x, int64_t n_vec, int d, int pos, const float* cos_tab,
                      const float* sin_tab, float* y) {
  const int h = d / 2;
  const float* cs = cos_tab + (size_t)pos * h;
  const float* sn = sin_tab + (size_t)pos * h;
  for (int64_t v = 0; v < n_vec; ++v) {
    const float* xv = x + v * d;
    for (int c = 0; c < d; ++c) {
      const int cp = c < h ? c + h : c - h;
      y[v * d + c] = rope_rotate(xv[c], xv[cp], c, d, cs, sn);
    }
  }
}

// Host generation of rows [t0, t1) of one key/value slice, fp32 values
// (post-rotation for keys when cos_tab != NULL).  kind 0 = key, 1 = value.
void synth_kv_rows(uint32_t seed, uint32_t tid, uint32_t slice, int kind, int d, int t0, int t1,
                   const uint8_t* outlier_mask, float outlier_mul, float sink_mul,
                   const float* cos_tab, const float* sin_tab, float* out) {
  for (int t = t0; t < t1; ++t)
    for (int c = 0; c < d; ++c)
      out[(size_t)(t - t0) * d + c] = kv_value(seed, tid, slice, t, c, d, kind, outlier_mask,
                                               outlier_mul, sink_mul, cos_tab, sin_tab);
}

// Device fill of a whole cache tensor [n_slices, T, d] (bf16 bits when
// out_bf16 != 0, else fp32).  All pointers are device pointers.  Returns the
// hipError_t of the launch.
int synth_kv_fill_device(uint32_t seed, uint32_t tid, int kind, int n_slices, int T, int d,
                         const int32_t* slice_ids, const uint8_t* outlier_masks, float outlier_mul,
                         float sink_mul, const float* cos_tab, const float* sin_tab, void* out,
                         int out_bf16, hipStream_t stream) {
  if (n_slices <= 0 || n_slices > 65535 || T <= 0 || d <= 0 || (d & 1)) return (int)hipErrorInvalidValue;
  const uint32_t per_slice = (uint32_t)T * (uint32_t)(d / 2);
  const int block = 256;
  uint32_t gx = (per_slice + block - 1) / block;
  if (gx > 4096) gx = 4096;
  const dim3 grid(gx, (unsigned)n_slices);
  if (out_bf16)
    kv_fill_kernel<uint16_t><<<grid, dim3(block), 0, stream>>>(
        seed, tid, kind, T, d, slice_ids, outlier_masks, outlier_mul, sink_mul, cos_tab, sin_tab,
        (uint16_t*)out);
  else
    kv_fill_kernel<float><<<grid, dim3(block), 0, stream>>>(
        seed, tid, kind, T, d, slice_ids, outlier_masks, outlier_mul, sink_mul, cos_tab, sin_tab,
        (float*)out);
  return (int)hipGetLastError();
}

}  // extern "C"
