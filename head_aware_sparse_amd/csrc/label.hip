// AoH labeller kernels for gfx950.
//
// Method: "Resumen Técnico: Autonomía de Cabezales (AoH)", Metodología:
//   §1 M_h = W_K^T W_Q; §2 ER = exp of the entropy of the normalised singular
//   values of M_h; §3 those singular values (squared) are the eigenvalues of
//   the d_head x d_head proxy C_h = (W_Q W_Q^T)(W_K W_K^T); §4 rank by ER, the
//   k lowest are retrieval heads, GQA groups aggregate by the mean.
//
// Pipeline (one stream, no host synchronisation):
//   gram      G = W W^T for every query and key head (matrix cores, bf16 or
//             fp32 in, fp32 accumulate).  Reads every weight once: the
//             HBM-bound step.
//   cholesky  per key head, in fp64 LDS: G_K = L L^T.
//   spectrum  per query head: the symmetric S = L^T G_Q L (fp64 matrix
//             cores), which is similar to C_h = G_Q G_K; Householder
//             tridiagonalisation of S in fp64, the matrix in registers.
//   bisect    eigenvalues of the tridiagonal by Sturm-count bisection (one
//             thread per eigenvalue), sigma = sqrt(max(lambda, 0)) and ER.
//   finalize  group mean of ER, global rank with ties to the lower index,
//             labels.
#include "internal.h"
#include "label.h"

namespace has {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int NWAVE = NT / 64;

struct LGeo {
  int L, Hq, Hkv, dm, d, G;
  int n_ret;
  float thr;
  const void* wq;
  const void* wk;
  float* gram;     // [L*Hq + L*Hkv][d][d]: query heads, then key heads
  double* lscr;    // [L*Hkv][d][d] Cholesky factor of each key head's Gram matrix
  double* tscr;    // [L*Hq][d][d] scratch for G_Q L
  float* tri;      // [L*Hq][2][d]: diagonal, off-diagonal (fp32)
  float* er_head;  // [L*Hq]
  float* er_group; // [L*Hkv]
  uint8_t* labels;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct LabelLayout {
  size_t gram, lscr, tscr, tri, erh, erg, bytes;
};

LabelLayout label_layout(int L, int Hq, int Hkv, int d) {
  LabelLayout o{};
  size_t at = 0;
  o.gram = at;
  at = align256(at + (size_t)(L * Hq + L * Hkv) * d * d * 4);
  o.lscr = at;
  at = align256(at + (size_t)L * Hkv * d * d * 8);
  o.tscr = at;
  at = align256(at + (size_t)L * Hq * d * d * 8);
  o.tri = at;
  at = align256(at + (size_t)L * Hq * 2 * d * 4);
  o.erh = at;
  at = align256(at + (size_t)L * Hq * 4);
  o.erg = at;
  at = align256(at + (size_t)L * Hkv * 4);
  o.bytes = at;
  return o;
}

// ------------------------------------------------------------------ gram
// One workgroup per head: G = W W^T over d_model.  The head's rows are
// staged through LDS in 128-byte-wide k tiles (double buffered); wave w owns
// a row band of 32 x 32 output tiles.  MFMA 32x32: output element
// (8*(r/4) + 4*(lane/32) + r%4, lane%32) sits in register r of lane.
template <typename E, int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void gram_kernel(LGeo g) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int KT = 128 / sizeof(E);           // elements per k tile
  constexpr int LDW = BF ? KT + 8 : KT + 1;     // padded LDS row
  constexpr int CPR = KT * sizeof(E) / 16;       // 16-byte chunks per row
  constexpr int CH = D * CPR / NT;               // chunks per thread
  constexpr int NB = D / 32;
  constexpr int TPW = NB * NB / NWAVE;
  __shared__ __attribute__((aligned(16))) E s_w[2][D][LDW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.x;
  const int nq = g.L * g.Hq;
  const E* W = m < nq ? (const E*)g.wq + (size_t)m * D * g.dm
                      : (const E*)g.wk + (size_t)(m - nq) * D * g.dm;
  // two k tiles in flight: a ring of two register sets, the loop unrolled by
  // two so that each set is named statically
  uint4 ra[CH], rb2[CH];
  auto gload = [&](int k0, uint4* reg) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int id = tid + c * NT;
      const int row = id / CPR, col = (id % CPR) * (16 / (int)sizeof(E));
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + (size_t)row * g.dm + k0 + col));
      reg[c] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  auto sstore = [&](int buf, const uint4* reg) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int id = tid + c * NT;
      const int row = id / CPR, col = (id % CPR) * (16 / (int)sizeof(E));
      if constexpr (BF) {
        *reinterpret_cast<uint4*>(&s_w[buf][row][col]) = reg[c];
      } else {
        s_w[buf][row][col + 0] = __uint_as_float(reg[c].x);
        s_w[buf][row][col + 1] = __uint_as_float(reg[c].y);
        s_w[buf][row][col + 2] = __uint_as_float(reg[c].z);
        s_w[buf][row][col + 3] = __uint_as_float(reg[c].w);
      }
    }
  };
  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  const int nk = g.dm / KT;
  // one k tile: tile kt is in LDS buffer kt & 1, tile kt + 1 in `next`; the
  // loads of tile kt + 2 go to `free` (which held tile kt)
  auto step = [&](int kt, uint4* next, uint4* free) {
    const int buf = kt & 1;
    if (kt + 2 < nk) gload((kt + 2) * KT, free);
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < KT; ks += 16) {
        const int kk = ks + (lane >> 5) * 8;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const int t = wave * TPW + i, rb = t / NB, cb = t % NB;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s_w[buf][rb * 32 + (lane & 31)][kk]);
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(&s_w[buf][cb * 32 + (lane & 31)][kk]);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
        }
      }
    } else {
#pragma unroll 4
      for (int ks = 0; ks < KT; ks += 2) {
        const int kk = ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const int t = wave * TPW + i, rb = t / NB, cb = t % NB;
          const float a = s_w[buf][rb * 32 + (lane & 31)][kk];
          const float b = s_w[buf][cb * 32 + (lane & 31)][kk];
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1, next);
    __syncthreads();
  };
  gload(0, ra);
  if (nk > 1) gload(KT, rb2);
  sstore(0, ra);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, rb2, ra);
    if (kt + 1 < nk) step(kt + 1, ra, rb2);
  }
  float* out = g.gram + (size_t)m * D * D;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave * TPW + i, rb = t / NB, cb = t % NB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      out[(size_t)row * D + cb * 32 + (lane & 31)] = acc[i][r];
    }
  }
}

// ------------------------------------------------------------------ spectrum
// fp64 lane moves: DPP on the two 32-bit halves, readlane into a uniform value
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const unsigned long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(u & 0xFFFFFFFFull), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const unsigned long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xFFFFFFFFull), l);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
  return __longlong_as_double(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
// Sum over the wave, identical in every lane: DPP within each 16-lane row
// (quad swaps, half-row and row mirrors), then the four row sums.
__device__ __forceinline__ double wave_sum_d(double x) {
  x += dpp_d<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_d<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_d<0x141>(x);  // row_half_mirror
  x += dpp_d<0x140>(x);  // row_mirror
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}

// Cholesky G_K = L L^T of each key head's Gram matrix (fp64, in LDS), once
// per (layer, KV group): right-looking, the trailing update tiled 16 x 16
// over the threads.  Columns whose pivot is not positive (rank-deficient key
// projections) are zeroed.  L (lower, zeros above) goes to lscr.
template <int D>
__global__ __launch_bounds__(NT) void chol_kernel(LGeo g) {
  constexpr int LD = D + 1;
  __shared__ double s_m[D * LD];
  __shared__ double s_ld[D];  // the diagonal of L, written back at the end
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int grp = blockIdx.x;  // l*Hkv + gk
  const float* GK = g.gram + (size_t)(g.L * g.Hq + grp) * D * D;
  double* A = s_m;
  for (int e = tid; e < D * D; e += NT) A[(e / D) * LD + (e % D)] = (double)GK[e];
  __syncthreads();
  double dmax = 0.0;
  for (int i = 0; i < D; ++i) dmax = fmax(dmax, A[i * LD + i]);
  const double tol = 1e-12 * dmax;
  for (int j = 0; j < D; ++j) {
    // the diagonal entry is only read here (its square root is kept apart),
    // so the column can be scaled without waiting for every thread to read it
    const double piv = A[j * LD + j];
    const bool zero = !(piv > tol);
    const double ljj = zero ? 0.0 : sqrt(piv);
    const double inv = zero ? 0.0 : 1.0 / ljj;
    if (tid == 0) s_ld[j] = ljj;
    for (int i = j + 1 + tid; i < D; i += NT) A[i * LD + j] *= inv;
    __syncthreads();
    for (int r = j + 1 + ty; r < D; r += 16) {
      const double arj = A[r * LD + j];
      for (int c = j + 1 + tx; c <= r; c += 16) A[r * LD + c] -= arj * A[c * LD + j];
    }
    __syncthreads();
  }
  double* Lo = g.lscr + (size_t)grp * D * D;
  for (int e = tid; e < D * D; e += NT) {
    const int i = e / D, j = e % D;
    Lo[e] = j < i ? A[i * LD + j] : (j == i ? s_ld[i] : 0.0);
  }
}

// MFMA f64 16x16x4: A element (lane%16, lane/16), B element (lane/16,
// lane%16); output (4*r + lane/16, lane%16) in register r (checked on the
// device: unlike the fp32 16x16 forms, rows interleave across lane groups).
// Per query head: S = L^T G_Q L (similar to C_h = G_Q G_K) on the fp64 matrix
// cores, symmetrised into a packed lower triangle in LDS, then Householder
// tridiagonalisation of S with the matrix spread over the threads' registers.
template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void spectrum_kernel(LGeo g) {
  constexpr int RB = D / 64;  // 16-row bands per wave
  constexpr int CB = D / 16;  // 16-col bands
  constexpr int CH = CB / 2;  // column bands per pass
  __shared__ double s_m[D * (D + 1) / 2];
  __shared__ float s_d[D], s_e[D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.x;                 // l*Hq + h
  const int l = head / g.Hq, h = head - l * g.Hq;
  const int grp = l * g.Hkv + h / g.G;
  const float* GQ = g.gram + (size_t)head * D * D;
  const double* Lg = g.lscr + (size_t)grp * D * D;
  double* A = s_m;
  auto pk = [](int i, int j) { return i * (i + 1) / 2 + j; };  // (i, j <= i)

  // 1. T = G_Q L (A operand G_Q fp32 -> fp64, B operand L, both from global),
  //    in two halves of the columns to bound the accumulator registers.
  double* T = g.tscr + (size_t)head * D * D;
  f64x4 acc[RB][CH];
  for (int c0 = 0; c0 < CB; c0 += CH) {
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[a][c] = f64x4{0.0, 0.0, 0.0, 0.0};
    // unrolled so that several k steps' operand loads are in flight together
#pragma unroll 8
    for (int k = 0; k < D; k += 4) {
      const int kk = k + (lane >> 4);
      double av[RB];
#pragma unroll
      // G_Q is symmetric: element (row, kk) is read at (kk, row), so the 16 lanes of a row band read consecutive words
      for (int a = 0; a < RB; ++a) av[a] = (double)GQ[(size_t)kk * D + (wave * RB + a) * 16 + (lane & 15)];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const double bv = Lg[(size_t)kk * D + (c0 + c) * 16 + (lane & 15)];
#pragma unroll
        for (int a = 0; a < RB; ++a) acc[a][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv, acc[a][c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          T[(size_t)((wave * RB + a) * 16 + 4 * r + (lane >> 4)) * D + (c0 + c) * 16 + (lane & 15)] = acc[a][c][r];
  }
  __threadfence();
  __syncthreads();

  // 2. S = L^T T (A operand L^T, B operand T, from global) in two column
  //    halves, symmetrised into the packed lower triangle straight from the
  //    registers: each pass first writes its elements on or below the
  //    diagonal (halved off it), then, after a barrier, adds half of each of
  //    its elements above the diagonal to the mirror element -- which an
  //    earlier write of this pass or of the first pass placed.
  for (int c0 = 0; c0 < CB; c0 += CH) {
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[a][c] = f64x4{0.0, 0.0, 0.0, 0.0};
    // unrolled so that several k steps' operand loads are in flight together
#pragma unroll 8
    for (int k = 0; k < D; k += 4) {
      const int kk = k + (lane >> 4);
      double av[RB];
#pragma unroll
      for (int a = 0; a < RB; ++a) av[a] = Lg[(size_t)kk * D + (wave * RB + a) * 16 + (lane & 15)];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const double bv = T[(size_t)kk * D + (c0 + c) * 16 + (lane & 15)];
#pragma unroll
        for (int a = 0; a < RB; ++a) acc[a][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv, acc[a][c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = (wave * RB + a) * 16 + 4 * r + (lane >> 4), j = (c0 + c) * 16 + (lane & 15);
          if (j <= i) A[pk(i, j)] = j == i ? acc[a][c][r] : 0.5 * acc[a][c][r];
        }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = (wave * RB + a) * 16 + 4 * r + (lane >> 4), j = (c0 + c) * 16 + (lane & 15);
          if (j > i) A[pk(j, i)] += 0.5 * acc[a][c][r];
        }
    __syncthreads();
  }

  // 3. Householder tridiagonalisation (similarity, eigenvalues kept), the
  //    symmetric matrix held in registers: thread (ty, tx) of a 16 x 16 grid
  //    holds rows ty + 16 r and columns tx + 16 c (r, c < BS), so the lanes of
  //    a row band read consecutive LDS words.  Step k
  //    reflects rows/columns k+1.. with v = x - alpha e1 (x: column k below
  //    the diagonal), p = beta A v, w = p - (beta/2)(v.p) v, A -= v w^T + w v^T;
  //    v and w vanish on rows and columns <= k, which stay as they are.
  //    Column k and p pass through LDS in two buffers taken in turn, so a step
  //    needs two barriers; every wave forms the norms and dot products itself.
  constexpr int BS = D / 16;
  __shared__ double s_x[2][D], s_pp[2][D];
  const int ty = tid >> 4, tx = tid & 15;
  double a[BS][BS];
#pragma unroll
  for (int r = 0; r < BS; ++r)
#pragma unroll
    for (int c = 0; c < BS; ++c) {
      const int i = ty + 16 * r, j = tx + 16 * c;
      a[r][c] = j <= i ? A[pk(i, j)] : A[pk(j, i)];
    }
  for (int k = 0; k < D - 2; ++k) {
    const int r0 = k + 1;
    double* sx = s_x[k & 1];
    double* sp = s_pp[k & 1];
    if (tx == k % 16) {  // column k: below the diagonal into LDS, the diagonal to d
      // k / 16 is the same in every thread, so only one register column is read
#pragma unroll
      for (int c = 0; c < BS; ++c) {
        if (c != k / 16) continue;
#pragma unroll
        for (int r = 0; r < BS; ++r) {
          const int i = ty + 16 * r;
          sx[i] = i > k ? a[r][c] : 0.0;
          if (i == k) s_d[k] = (float)a[r][c];
        }
      }
    }
    __syncthreads();
    double xx = 0.0;
    for (int i = lane; i < D; i += 64) xx += sx[i] * sx[i];
    const double nrm2 = wave_sum_d(xx);
    const double x0 = sx[r0];
    const double alpha = x0 >= 0.0 ? -sqrt(nrm2) : sqrt(nrm2);
    const double vn2 = nrm2 - x0 * x0 + (x0 - alpha) * (x0 - alpha);
    if (tid == 0) s_e[k] = (float)(vn2 > 0.0 ? alpha : x0);
    if (!(vn2 > 0.0)) continue;  // uniform: the column is already reduced
    const double beta = 2.0 / vn2;
    auto vof = [&](int i) { return i == r0 ? x0 - alpha : sx[i]; };  // 0 on rows <= k
    double vc[BS];
#pragma unroll
    for (int c = 0; c < BS; ++c) vc[c] = vof(tx + 16 * c);
    // p for this thread's rows: its block's share, summed over the row band's
    // 16 lanes (one 16-lane row of the wave)
#pragma unroll
    for (int r = 0; r < BS; ++r) {
      double pr = 0.0;
#pragma unroll
      for (int c = 0; c < BS; ++c) pr += a[r][c] * vc[c];
      pr += dpp_d<0xB1>(pr);   // quad_perm [1,0,3,2]
      pr += dpp_d<0x4E>(pr);   // quad_perm [2,3,0,1]
      pr += dpp_d<0x141>(pr);  // row_half_mirror
      pr += dpp_d<0x140>(pr);  // row_mirror
      const int i = ty + 16 * r;
      if (tx == r) sp[i] = i >= r0 ? beta * pr : 0.0;
    }
    __syncthreads();
    double vpp = 0.0;
    for (int i = lane; i < D; i += 64) vpp += vof(i) * sp[i];
    const double kk = 0.5 * beta * wave_sum_d(vpp);
    double wc[BS];
#pragma unroll
    for (int c = 0; c < BS; ++c) wc[c] = sp[tx + 16 * c] - kk * vc[c];
#pragma unroll
    for (int r = 0; r < BS; ++r) {
      const double vr = vof(ty + 16 * r), wr = sp[ty + 16 * r] - kk * vr;
#pragma unroll
      for (int c = 0; c < BS; ++c) a[r][c] -= vr * wc[c] + wr * vc[c];
    }
  }
  // the last 2 x 2 block
#pragma unroll
  for (int r = 0; r < BS; ++r)
#pragma unroll
    for (int c = 0; c < BS; ++c) {
      const int i = ty + 16 * r, j = tx + 16 * c;
      if (i == j && i >= D - 2) s_d[i] = (float)a[r][c];
      if (i == D - 1 && j == D - 2) s_e[D - 2] = (float)a[r][c];
    }
  if (tid == 0) s_e[D - 1] = 0.f;
  __syncthreads();
  float* tri = g.tri + (size_t)head * 2 * D;
  for (int i = tid; i < D; i += NT) {
    tri[i] = s_d[i];
    tri[D + i] = s_e[i];
  }
}

// ------------------------------------------------------------------ bisect
// Number of eigenvalues of the tridiagonal below x (Sturm sequence of the
// LDL^T pivots; an exact zero pivot is nudged negative).
template <int D>
__device__ __forceinline__ int sturm_count(const float* d, const float* e2, float x) {
  int cnt = 0;
  float q = d[0] - x;
  cnt += q < 0.f;
  for (int i = 1; i < D; ++i) {
    if (fabsf(q) < 1e-30f) q = -1e-30f;
    q = (d[i] - x) - e2[i - 1] * __builtin_amdgcn_rcpf(q);
    cnt += q < 0.f;
  }
  return cnt;
}

template <int D>
__global__ __launch_bounds__(D) void bisect_kernel(LGeo g) {
  __shared__ float s_d[D], s_e2[D];
  __shared__ float s_lo[D / 64], s_hi[D / 64];
  __shared__ double s_sum[D / 64];
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6;
  const int head = blockIdx.x;
  const float* tri = g.tri + (size_t)head * 2 * D;
  const float dj = tri[j], ej = tri[D + j];
  s_d[j] = dj;
  s_e2[j] = ej * ej;
  const float ejm = j > 0 ? tri[D + j - 1] : 0.f;
  float lo = dj - fabsf(ej) - fabsf(ejm), hi = dj + fabsf(ej) + fabsf(ejm);
  for (int o = 32; o >= 1; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
  }
  __syncthreads();
  for (int w = 0; w < D / 64; ++w) {
    lo = fminf(lo, s_lo[w]);
    hi = fmaxf(hi, s_hi[w]);
  }
  const float pad = 1e-6f * fmaxf(fabsf(lo), fabsf(hi)) + 1e-30f;
  float a = lo - pad, b = hi + pad;
  for (int it = 0; it < 64; ++it) {
    const float mid = 0.5f * (a + b);
    if (!(mid > a && mid < b)) break;
    if (sturm_count<D>(s_d, s_e2, mid) > j) b = mid;
    else a = mid;
  }
  const double lam = fmax(0.5 * ((double)a + (double)b), 0.0);
  const double sigma = sqrt(lam);
  double tot = wave_sum_d(sigma);
  if (lane == 0) s_sum[wave] = tot;
  __syncthreads();
  tot = 0.0;
  for (int w = 0; w < D / 64; ++w) tot += s_sum[w];
  __syncthreads();
  const double p = tot > 0.0 ? sigma / tot : 0.0;
  double hterm = p > 0.0 ? -p * log(p) : 0.0;
  hterm = wave_sum_d(hterm);
  if (lane == 0) s_sum[wave] = hterm;
  __syncthreads();
  if (j == 0) {
    double H = 0.0;
    for (int w = 0; w < D / 64; ++w) H += s_sum[w];
    g.er_head[head] = (float)exp(H);
  }
}

// ------------------------------------------------------------------ finalize
__global__ __launch_bounds__(NT) void finalize_kernel(LGeo g) {
  __shared__ float s_eg[kMaxPairs];
  const int P = g.L * g.Hkv;
  for (int p = threadIdx.x; p < P; p += NT) {
    const int l = p / g.Hkv, gi = p - l * g.Hkv;
    const float* eh = g.er_head + (size_t)l * g.Hq + gi * g.G;
    float s = 0.f;
    for (int h = 0; h < g.G; ++h) s += eh[h];
    s_eg[p] = s / (float)g.G;
  }
  __syncthreads();
  const int p = blockIdx.x * NT + threadIdx.x;
  if (p >= P) return;
  const float e = s_eg[p];
  g.er_group[p] = e;
  uint8_t lab;
  if (g.n_ret >= 0) {
    int rank = 0;
    for (int q = 0; q < P; ++q) {
      const float f = s_eg[q];
      rank += (f < e || (f == e && q < p)) ? 1 : 0;
    }
    lab = rank < g.n_ret ? 1 : 0;
  } else {
    lab = e < g.thr ? 1 : 0;
  }
  g.labels[p] = lab;
}

}  // namespace

size_t label_workspace_bytes(int L, int Hq, int Hkv, int dm, int d) {
  (void)dm;
  if (L < 1 || Hq < 1 || Hkv < 1 || d < 1) return 0;
  return label_layout(L, Hq, Hkv, d).bytes;
}

hipError_t launch_label(const LabelArgs& a, hipStream_t s) {
  const LabelLayout lo = label_layout(a.L, a.Hq, a.Hkv, a.d);
  char* ws = (char*)a.ws;
  LGeo g{};
  g.L = a.L;
  g.Hq = a.Hq;
  g.Hkv = a.Hkv;
  g.dm = a.dm;
  g.d = a.d;
  g.G = a.Hq / a.Hkv;
  g.n_ret = a.n_retrieval;
  g.thr = a.threshold;
  g.wq = a.w_q;
  g.wk = a.w_k;
  g.gram = (float*)(ws + lo.gram);
  g.lscr = (double*)(ws + lo.lscr);
  g.tscr = (double*)(ws + lo.tscr);
  g.tri = (float*)(ws + lo.tri);
  g.er_head = a.er_head ? a.er_head : (float*)(ws + lo.erh);
  g.er_group = a.er_group ? a.er_group : (float*)(ws + lo.erg);
  g.labels = a.labels;
  const int n_mats = a.L * a.Hq + a.L * a.Hkv;
  const int n_heads = a.L * a.Hq;
  {
    KTimer t("gram", s);
    if (a.d == 128) {
      if (a.bf16) gram_kernel<uint16_t, 128><<<n_mats, NT, 0, s>>>(g);
      else gram_kernel<float, 128><<<n_mats, NT, 0, s>>>(g);
    } else {
      if (a.bf16) gram_kernel<uint16_t, 64><<<n_mats, NT, 0, s>>>(g);
      else gram_kernel<float, 64><<<n_mats, NT, 0, s>>>(g);
    }
  }
  {
    KTimer t("cholesky", s);
    if (a.d == 128) chol_kernel<128><<<a.L * a.Hkv, NT, 0, s>>>(g);
    else chol_kernel<64><<<a.L * a.Hkv, NT, 0, s>>>(g);
  }
  {
    KTimer t("spectrum", s);
    if (a.d == 128) spectrum_kernel<128><<<n_heads, NT, 0, s>>>(g);
    else spectrum_kernel<64><<<n_heads, NT, 0, s>>>(g);
  }
  {
    KTimer t("bisect", s);
    if (a.d == 128) bisect_kernel<128><<<n_heads, 128, 0, s>>>(g);
    else bisect_kernel<64><<<n_heads, 64, 0, s>>>(g);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int P = a.L * a.Hkv;
  {
    KTimer t("finalize", s);
    finalize_kernel<<<(P + NT - 1) / NT, NT, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace has
