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
//   cholesky  per key head, in fp64 with the matrix in registers:
//             G_K = L L^T.
//   spectrum  per query head: the symmetric S = L^T G_Q L (fp64 matrix
//             cores, L's zero blocks skipped, the lower triangle only),
//             which is similar to C_h = G_Q G_K; Householder
//             tridiagonalisation of S in fp64, the matrix in registers.
//   bisect    eigenvalues of the tridiagonal by Sturm counts (a shared
//             first round, then trisection by a pair of threads per
//             eigenvalue), sigma = sqrt(max(lambda, 0)) and ER.
//   finalize  group mean of ER, global rank with ties to the lower index,
//             labels.
#include <type_traits>
#include <utility>

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
  float* tri;      // [L*Hq][2][d]: diagonal, off-diagonal (fp32)
  float* er_head;  // [L*Hq]
  float* er_group; // [L*Hkv]
  uint8_t* labels;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct LabelLayout {
  size_t gram, lscr, tri, erh, erg, bytes;
};

LabelLayout label_layout(int L, int Hq, int Hkv, int d) {
  LabelLayout o{};
  size_t at = 0;
  o.gram = at;
  at = align256(at + (size_t)(L * Hq + L * Hkv) * d * d * 4);
  o.lscr = at;
  at = align256(at + (size_t)L * Hkv * d * d * 8);
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

// Sum over the 16 lanes of a DPP row, identical in every lane of the row.
// In the 16 x 16 thread grids below a row is the 16 tx of one ty.
__device__ __forceinline__ double row16_sum(double x) {
  x += dpp_d<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_d<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_d<0x141>(x);  // row_half_mirror
  x += dpp_d<0x140>(x);  // row_mirror
  return x;
}

// f(std::integral_constant<int, B>{}) for B = 0 .. N-1 in turn: code
// specialised on a 16-wide band B indexes the register blocks statically and
// skips the blocks that no longer change.
template <class F, int... B>
__device__ __forceinline__ void each_band(F&& f, std::integer_sequence<int, B...>) {
  (f(std::integral_constant<int, B>{}), ...);
}

// Cholesky G_K = L L^T of each key head's Gram matrix (fp64), once per
// (layer, KV group), right-looking with the matrix in registers: thread
// (ty, tx) of a 16 x 16 grid holds rows ty + 16 r and columns tx + 16 c.
// Step j: the threads holding column j put it in LDS; after one barrier
// every thread scales its rows' and columns' entries of it by 1/sqrt(pivot)
// and updates its trailing entries (blocks left of or above column j's band
// are final and skipped).  Columns whose pivot is not above 1e-12 of the
// largest diagonal entry (rank-deficient key projections) are zeroed.  L
// (lower, zeros above) goes to lscr.
template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void chol_kernel(LGeo g) {
  constexpr int BS = D / 16;
  __shared__ double s_x[2][D];
  __shared__ double s_max[NWAVE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ty = tid >> 4, tx = tid & 15;
  const int grp = blockIdx.x;  // l*Hkv + gk
  const float* GK = g.gram + (size_t)(g.L * g.Hq + grp) * D * D;
  double a[BS][BS];
#pragma unroll
  for (int r = 0; r < BS; ++r)
#pragma unroll
    for (int c = 0; c < BS; ++c) a[r][c] = (double)GK[(size_t)(ty + 16 * r) * D + tx + 16 * c];
  double dm = 0.0;
#pragma unroll
  for (int r = 0; r < BS; ++r) dm = fmax(dm, tx == ty ? a[r][r] : 0.0);
  for (int o = 32; o >= 1; o >>= 1) dm = fmax(dm, __shfl_xor(dm, o));
  if (lane == 0) s_max[wave] = dm;
  __syncthreads();
  for (int w = 0; w < NWAVE; ++w) dm = fmax(dm, s_max[w]);
  const double tol = 1e-12 * dm;
  each_band([&](auto band) {
    constexpr int JB = decltype(band)::value;
#pragma unroll 1
    for (int jl = 0; jl < 16; ++jl) {
      const int j = 16 * JB + jl;
      double* sx = s_x[j & 1];
      if (tx == jl) {
#pragma unroll
        for (int r = JB; r < BS; ++r) sx[ty + 16 * r] = a[r][JB];
      }
      __syncthreads();
      const double piv = sx[j];
      const bool zero = !(piv > tol);
      const double ljj = zero ? 0.0 : sqrt(piv);
      const double inv = zero ? 0.0 : 1.0 / ljj;
      double lr[BS], lc[BS];
#pragma unroll
      for (int r = JB; r < BS; ++r) lr[r] = ty + 16 * r > j ? sx[ty + 16 * r] * inv : 0.0;
#pragma unroll
      for (int c = JB; c < BS; ++c) lc[c] = tx + 16 * c > j ? sx[tx + 16 * c] * inv : 0.0;
#pragma unroll
      for (int r = JB; r < BS; ++r)
#pragma unroll
        for (int c = JB; c < BS; ++c) a[r][c] = fma(-lr[r], lc[c], a[r][c]);
      if (tx == jl) {  // column j of L in place (the update left that column as it was)
#pragma unroll
        for (int r = JB; r < BS; ++r) {
          const int i = ty + 16 * r;
          if (i >= j) a[r][JB] = i == j ? ljj : lr[r];
        }
      }
    }
  }, std::make_integer_sequence<int, BS>{});
  double* Lo = g.lscr + (size_t)grp * D * D;
#pragma unroll
  for (int r = 0; r < BS; ++r)
#pragma unroll
    for (int c = 0; c < BS; ++c) {
      const int i = ty + 16 * r, j = tx + 16 * c;
      Lo[(size_t)i * D + j] = j <= i ? a[r][c] : 0.0;
    }
}

// MFMA f64 16x16x4: A element (lane%16, lane/16), B element (lane/16,
// lane%16); output (4*r + lane/16, lane%16) in register r (checked on the
// device: unlike the fp32 16x16 forms, rows interleave across lane groups).
// Per query head: S = L^T G_Q L (similar to C_h = G_Q G_K) on the fp64 matrix
// cores, its lower triangle packed into LDS, then Householder
// tridiagonalisation of S with the matrix spread over the threads' registers.
template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void spectrum_kernel(LGeo g) {
  constexpr int NB = D / 16;       // 16-wide bands
  __shared__ double s_m[D * (D + 1) / 2];
  __shared__ float s_d[D], s_e[D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lk = lane >> 4;
  const int head = blockIdx.x;  // l*Hq + h
  const int l = head / g.Hq, h = head - l * g.Hq;
  const int grp = l * g.Hkv + h / g.G;
  const float* GQ = g.gram + (size_t)head * D * D;
  const double* Lg = g.lscr + (size_t)grp * D * D;
  double* A = s_m;
  auto pk = [](int i, int j) { return i * (i + 1) / 2 + j; };  // (i, j <= i)

  // 1. S = L^T (G_Q L), lower triangle, by column bands: wave w takes bands
  //    w and NB-1-w (about equal shares of the triangular work), each with
  //    its band index a compile-time constant, so that the operand loads of a
  //    band form one straight run that the scheduler can issue ahead.  For
  //    band CB, T = G_Q L[:, CB] (L[k][16 CB ..] = 0 for k < 16 CB, so k starts
  //    there) is only needed on row bands >= CB and stays in registers: in the
  //    matrix cores' output layout, register r of T's tile kb holds row
  //    16 kb + 4 r + lane/16 -- the B operand of k step 16 kb + 4 r of the next
  //    product.  Then S[a][CB] = sum over k >= 16 a of L[k][16 a + n] T[k][..]
  //    for the row bands a >= CB.
  each_band([&](auto band) {
    constexpr int CB = decltype(band)::value;
    if (CB != wave && CB != NB - 1 - wave) return;
    f64x4 t[NB];
#pragma unroll
    for (int a = CB; a < NB; ++a) t[a] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int k = 16 * CB; k < D; k += 4) {
      const int kk = k + lk;
      const double bv = Lg[(size_t)kk * D + CB * 16 + ln];
#pragma unroll
      for (int a = CB; a < NB; ++a) {
        // G_Q is symmetric: element (row, kk) is read at (kk, row), so the 16 lanes of a row band read consecutive words
        const double av = (double)GQ[(size_t)kk * D + a * 16 + ln];
        t[a] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, t[a], 0, 0, 0);
      }
    }
    f64x4 s[NB];
#pragma unroll
    for (int a = CB; a < NB; ++a) s[a] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = CB; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * kb + 4 * r + lk;
#pragma unroll
        for (int a = CB; a <= kb; ++a) {
          const double av = Lg[(size_t)kk * D + a * 16 + ln];
          s[a] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, t[kb][r], s[a], 0, 0, 0);
        }
      }
#pragma unroll
    for (int a = CB; a < NB; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * a + 4 * r + lk, j = 16 * CB + ln;
        if (j <= i) A[pk(i, j)] = s[a][r];
      }
  }, std::make_integer_sequence<int, NB>{});
  __syncthreads();

  // 2. Householder tridiagonalisation (similarity, eigenvalues kept) with the
  //    symmetric matrix in registers: thread (ty, tx) of a 16 x 16 grid holds
  //    rows ty + 16 r and columns tx + 16 c (r, c < BS), so the lanes of a row
  //    band read consecutive LDS words.  Step k reflects rows/columns k+1..
  //    with v = x - alpha e1 (x: column k below the diagonal), p = beta A v,
  //    w = p - (beta/2)(v.p) v, A -= v w^T + w v^T.  v and w vanish on rows
  //    and columns <= k, which stay as they are: the blocks left of or above
  //    column k's band are skipped.  Column k and p pass through LDS (two
  //    buffers taken in turn: two barriers a step); norms and dot products
  //    are summed over the 16 lanes of a row, whose columns cover every index
  //    from the band on.  A v is formed from x while alpha's square root is
  //    in flight (v differs from x in entry k+1 only) and corrected after.
  constexpr int BS = NB;
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
  each_band([&](auto band) {
    constexpr int KB = decltype(band)::value;
    constexpr int KB1 = KB + 1 < BS ? KB + 1 : KB;
#pragma unroll 1
    for (int kl = 0; kl < 16; ++kl) {
      const int k = 16 * KB + kl;
      if (k >= D - 2) break;
      const int r0 = k + 1;
      double* sx = s_x[k & 1];
      double* sp = s_pp[k & 1];
      if (tx == kl) {  // column k below the diagonal (zero on rows <= k), the diagonal to d
        sx[ty + 16 * KB] = ty > kl ? a[KB][KB] : 0.0;
#pragma unroll
        for (int r = KB + 1; r < BS; ++r) sx[ty + 16 * r] = a[r][KB];
        if (ty == kl) s_d[k] = (float)a[KB][KB];
      }
      __syncthreads();
      double xc[BS], xr[BS], pr[BS];
#pragma unroll
      for (int c = KB; c < BS; ++c) xc[c] = sx[tx + 16 * c];
#pragma unroll
      for (int r = KB; r < BS; ++r) xr[r] = sx[ty + 16 * r];
      const double x0 = sx[r0];
      double nn = 0.0;
#pragma unroll
      for (int c = KB; c < BS; ++c) nn = fma(xc[c], xc[c], nn);
      nn = row16_sum(nn);
#pragma unroll
      for (int r = KB; r < BS; ++r) {
        pr[r] = 0.0;
#pragma unroll
        for (int c = KB; c < BS; ++c) pr[r] = fma(a[r][c], xc[c], pr[r]);
      }
      const double sq = sqrt(nn);
      const double alpha = x0 >= 0.0 ? -sq : sq;
      // beta = 2 / |v|^2 with |v|^2 = 2 (|x|^2 + |x0| |x|); 0 when x = 0 (then v = 0)
      const double beta = nn > 0.0 ? 1.0 / fma(fabs(x0), sq, nn) : 0.0;
      if (tid == 0) s_e[k] = (float)alpha;
      // v = x - alpha e_{k+1}: A v = A x - alpha (column k+1), corrected in
      // the lanes holding column k+1; entry k+1 of v in the lanes holding it
      if (tx == (r0 & 15)) {
        if (kl == 15) {
#pragma unroll
          for (int r = KB; r < BS; ++r) pr[r] = fma(-alpha, a[r][KB1], pr[r]);
          xc[KB1] -= alpha;
        } else {
#pragma unroll
          for (int r = KB; r < BS; ++r) pr[r] = fma(-alpha, a[r][KB], pr[r]);
          xc[KB] -= alpha;
        }
      }
      if (ty == (r0 & 15)) {
        if (kl == 15) xr[KB1] -= alpha;
        else xr[KB] -= alpha;
      }
#pragma unroll
      for (int r = KB; r < BS; ++r) pr[r] = row16_sum(pr[r]);
      if (tx == 0) {  // p of this thread's rows (zero on rows <= k)
        sp[ty + 16 * KB] = ty > kl ? beta * pr[KB] : 0.0;
#pragma unroll
        for (int r = KB + 1; r < BS; ++r) sp[ty + 16 * r] = beta * pr[r];
      }
      __syncthreads();
      double pc[BS];
      const double* vc = xc;
#pragma unroll
      for (int c = KB; c < BS; ++c) pc[c] = sp[tx + 16 * c];
      double vp = 0.0;
#pragma unroll
      for (int c = KB; c < BS; ++c) vp = fma(vc[c], pc[c], vp);
      const double kk = 0.5 * beta * row16_sum(vp);
      double wc[BS];
#pragma unroll
      for (int c = KB; c < BS; ++c) wc[c] = fma(-kk, vc[c], pc[c]);
#pragma unroll
      for (int r = KB; r < BS; ++r) {
        const double vr = xr[r];
        const double wr = fma(-kk, vr, sp[ty + 16 * r]);
#pragma unroll
        for (int c = KB; c < BS; ++c) a[r][c] = fma(-vr, wc[c], fma(-wr, vc[c], a[r][c]));
      }
    }
  }, std::make_integer_sequence<int, BS>{});
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
// Number of eigenvalues of the tridiagonal below x: the negative LDL^T
// pivots of T - x I (Sturm sequence), an exact zero pivot nudged negative.
// d4 holds the diagonal, e4 the squared off-diagonal entry left of each row
// (0 for the first), four entries a read (broadcast to every lane).
template <int D>
__device__ __forceinline__ int sturm_count(const float4* d4, const float4* e4, float x) {
  int cnt = 0;
  float q = 1.f;
  auto step = [&](float d, float e2) {
    if (fabsf(q) < 1e-30f) q = -1e-30f;
    q = (d - x) - e2 * __builtin_amdgcn_rcpf(q);
    cnt += q < 0.f;
  };
#pragma unroll 8
  for (int i = 0; i < D / 4; ++i) {
    const float4 dv = d4[i], ev = e4[i];
    step(dv.x, ev.x);
    step(dv.y, ev.y);
    step(dv.z, ev.z);
    step(dv.w, ev.w);
  }
  return cnt;
}

// Two threads per eigenvalue j (ascending), in Gershgorin's interval,
// padded.  A first round is shared: thread t counts at the t-th of 2D equally
// spaced interior points, and eigenvalue j starts between the last point whose
// count is <= j and the first whose count is above it.  Then trisection: each
// thread of the pair counts at one of the bracket's two interior thirds, the
// pair swaps counts and both keep the third that holds eigenvalue j (the
// same floating-point steps in both, so their brackets stay equal), until the
// bracket's image under sqrt(max(., 0)) -- the singular value it brackets --
// is 2^-19 of sqrt(the interval's magnitude) wide, what the ER needs.  A
// bracket that still reaches 0 or below (an exact zero eigenvalue: a
// rank-deficient projection) goes on until its upper end is 2^-48 of the
// magnitude, so that each zero's singular value stays below 2^-24 of its
// square root: even 127 zeros beside one nonzero singular value move the ER
// by about 1e-4.  lambda is the bracket's midpoint; sigma = sqrt(max(lambda,
// 0)) and the head's ER follow.
template <int D>
__global__ __launch_bounds__(2 * D) void bisect_kernel(LGeo g) {
  constexpr int NTB = 2 * D, NWB = NTB / 64;
  __shared__ float4 s_d4[D / 4], s_e4[D / 4];
  __shared__ float s_lo[NWB], s_hi[NWB], s_x[NTB];
  __shared__ int s_cnt[NTB];
  __shared__ double s_sum[NWB];
  float* s_d = reinterpret_cast<float*>(s_d4);
  float* s_e2 = reinterpret_cast<float*>(s_e4);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = tid >> 1, part = tid & 1;
  const int head = blockIdx.x;
  const float* tri = g.tri + (size_t)head * 2 * D;
  float lo = INFINITY, hi = -INFINITY;
  if (tid < D) {
    const float dj = tri[tid], ej = tri[D + tid];
    const float ejm = tid > 0 ? tri[D + tid - 1] : 0.f;
    s_d[tid] = dj;
    s_e2[tid] = ejm * ejm;
    lo = dj - fabsf(ej) - fabsf(ejm);
    hi = dj + fabsf(ej) + fabsf(ejm);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
  }
  __syncthreads();
  for (int w = 0; w < NWB; ++w) {
    lo = fminf(lo, s_lo[w]);
    hi = fmaxf(hi, s_hi[w]);
  }
  const float pad = 1e-6f * fmaxf(fabsf(lo), fabsf(hi)) + 1e-30f;
  float a = lo - pad, b = hi + pad;
  const float tol_s = 0x1p-19f * sqrtf(fmaxf(fabsf(a), fabsf(b)));
  const float tol_z = 0x1p-48f * fmaxf(fabsf(a), fabsf(b));
  const float xt = a + (b - a) * ((float)(tid + 1) / (float)(NTB + 1));
  s_x[tid] = xt;
  s_cnt[tid] = sturm_count<D>(s_d4, s_e4, xt);
  __syncthreads();
  int t0 = 0, t1 = NTB;  // the first point whose count is above j
  while (t0 < t1) {
    const int m = (t0 + t1) >> 1;
    if (s_cnt[m] > j) t1 = m;
    else t0 = m + 1;
  }
  if (t0 < NTB) b = s_x[t0];
  if (t0 > 0) a = s_x[t0 - 1];
  for (int it = 0; it < 64; ++it) {
    if (a > 0.f ? !(sqrtf(b) - sqrtf(a) > tol_s) : !(b > tol_z)) break;
    const float w3 = (b - a) * (1.f / 3.f);
    const float x1 = a + w3, x2 = b - w3;
    if (!(x1 > a && x2 > x1 && b > x2)) break;
    const int mine = sturm_count<D>(s_d4, s_e4, part ? x2 : x1);
    const int other = __shfl_xor(mine, 1);
    const int c1 = part ? other : mine, c2 = part ? mine : other;
    if (c1 > j) b = x1;
    else if (c2 > j) {
      a = x1;
      b = x2;
    } else {
      a = x2;
    }
  }
  const double lam = fmax(0.5 * ((double)a + (double)b), 0.0);
  const double sigma = part ? 0.0 : sqrt(lam);  // one thread of the pair counts
  double tot = wave_sum_d(sigma);
  if (lane == 0) s_sum[wave] = tot;
  __syncthreads();
  tot = 0.0;
  for (int w = 0; w < NWB; ++w) tot += s_sum[w];
  __syncthreads();
  const double p = tot > 0.0 ? sigma / tot : 0.0;
  double hterm = p > 0.0 ? -p * log(p) : 0.0;
  hterm = wave_sum_d(hterm);
  if (lane == 0) s_sum[wave] = hterm;
  __syncthreads();
  if (tid == 0) {
    double H = 0.0;
    for (int w = 0; w < NWB; ++w) H += s_sum[w];
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
    if (a.d == 128) bisect_kernel<128><<<n_heads, 256, 0, s>>>(g);
    else bisect_kernel<64><<<n_heads, 128, 0, s>>>(g);
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
