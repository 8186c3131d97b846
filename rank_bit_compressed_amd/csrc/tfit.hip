// tfit.hip -- fit of a layer group's partial Tucker factors on the GPU (prefill side, gfx950).
//
// One sequence's keys (or values) of a layer group form X[t, l, h, i] (token, layer, head, feature); its
// token-mode unfolding is the matrix A = X_(1) [T, D], D = L Hkv d, columns in (l, h, i) order.  The partial
// Tucker form keeps heads and layers whole and truncates the token and feature modes ("JoLT: Near-Lossless KV
// Cache Compression" thesis page, "How JoLT works"); FlashJoLT replaces the exact token-mode SVD by a
// randomized one ("A JoLT for the KV cache", abstract).  Computed here, per sequence:
//   * token factor: randomized subspace iteration (Halko, Martinsson and Tropp, 2011) from a Gaussian test
//     matrix Omega [D, r_t] the caller draws: Q = orth(A Omega); q times: Z = orth(A^T Q), Q = orth(A Z).
//     orth is the Q factor of the QR decomposition with a positive diagonal R, formed by CholeskyQR2: the Gram
//     matrix Y^T Y in fp64, its Cholesky factor L (fp64, one workgroup), R^-1 = L^-T (fp64, one wave per
//     column), Q = Y R^-1 on the matrix cores; the second pass repeats it on Q, restoring orthogonality to
//     fp32 rounding.  Both passes multiply by upper-triangular factors with positive diagonals, so the result
//     is that unique QR factor up to rounding;
//   * feature factor: the r_f leading left singular vectors of the feature-mode unfolding, i.e. the basis fit
//     of every (t, l, h) row of the sequence (the per-head fit run with the rows viewed as one head);
//   * core: P = U_t^T A [r_t, D] on the matrix cores, then core[l][h] = P[:, (l, h) block] U_f.
// The large products run on v_mfma_f32_32x32x2_f32 (fp32 operands and accumulation): 128 x 128 output tiles
// per workgroup, four waves of 64 x 64, 16-deep k steps double-buffered through LDS, a workgroup-to-tile map
// that keeps neighbouring tiles (which share their A rows) on one XCD, and a split of the token sum into fixed
// chunks whose partial products are added in a fixed order, so the results are deterministic.
// Rows t >= seq_len[b] of x are never read: they count as zero rows, and the token factor is zero there.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "kvc_common.hpp"

namespace kvc {

size_t fit_part_floats(const kvc_fit_in& in);
hipError_t fit_gram_launch(const kvc_fit_in& in, float* part, float* gram, hipStream_t st);
hipError_t fit_eig_launch(const float* gram, int n, int rank, int r_cap, uint16_t* basis_bf16, float* basis_f32,
                          float* sigma2, hipStream_t st);

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace tf {
constexpr int BM = 128, BN = 128, BK = 16;
constexpr int LS = BM + 4;        // LDS row stride of the operand tiles (floats)
constexpr int RMAX = 256;         // largest token rank
constexpr int CP = 64;            // Cholesky panel width
constexpr int CT = 1024;          // Cholesky threads
constexpr int STG_LOADS = (RMAX - CP) * CP / CT;      // staging loads per thread for one finished panel
constexpr int GT = 64;            // Gram tile
constexpr int GR = 32;            // Gram rows per LDS stage
constexpr int D = 128;            // head dimension

struct GemmArgs {
  const float* a;
  const float* b;
  float* c;
  int M, N, K, lda, ldb, ldc;
  int64_t sa_o, sa_i, sb_o, sb_i, sc_o, sc_i, sc_split;
  int n_inner, tiles_m, tiles_n, kchunk;
  const int32_t* mlim;  // rows m >= mlim[outer] * lim_mul of A are zero (NULL: none)
  const int32_t* klim;  // k >= klim[outer] * lim_mul are zero (NULL: none)
  int lim_mul;
};

__device__ inline f32x16 mfma32(float a, float b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }

// C[outer, inner] (+ split) = op(A) op(B); op(A) is M x K (TA: A stored K x M), op(B) is K x N (TB: B stored
// N x K).  The contiguous dimension of each stored operand is a multiple of 4 and its rows 16-byte aligned.
template <bool TA, bool TB>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  __shared__ float as[2][BK][LS];
  __shared__ float bs[2][BK][LS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lo = lane & 31, hi = lane >> 5;
  const int wm = wv >> 1, wn = wv & 1;
  const int nt = g.tiles_m * g.tiles_n;
  int tile = blockIdx.x;
  // consecutive workgroups go to different XCDs: give each XCD a contiguous run of tiles, so the tiles of one
  // A row block meet in one L2
  if ((nt & 7) == 0) tile = (tile & 7) * (nt >> 3) + (tile >> 3);
  const int tm = tile / g.tiles_n, tn = tile - tm * g.tiles_n;
  const int bo = blockIdx.y / g.n_inner, bi = blockIdx.y - bo * g.n_inner;
  const float* A = g.a + bo * g.sa_o + bi * g.sa_i;
  const float* Bm = g.b + bo * g.sb_o + bi * g.sb_i;
  float* Cm = g.c + bo * g.sc_o + bi * g.sc_i + (int64_t)blockIdx.z * g.sc_split;
  const int m0 = tm * BM, n0 = tn * BN;
  const int mmax = g.mlim ? min(g.M, g.mlim[bo] * g.lim_mul) : g.M;
  const int kend = g.klim ? min(g.K, g.klim[bo] * g.lim_mul) : g.K;
  const int kb = blockIdx.z * g.kchunk;
  const int ke = min(kend, kb + g.kchunk);
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;
  if (m0 < mmax && kb < ke) {
    const int ns = (ke - kb + BK - 1) / BK;
    float4 ra[2], rb[2];
    auto load = [&](int s) {
      const int k0 = kb + s * BK;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (!TA) {
          const int m = m0 + (tid >> 2) + 64 * i, k = k0 + (tid & 3) * 4;
          ra[i] = (m < mmax && k < ke) ? *(const float4*)(A + (int64_t)m * g.lda + k) : make_float4(0, 0, 0, 0);
        } else {
          const int k = k0 + (tid >> 5) + 8 * i, m = m0 + (tid & 31) * 4;
          ra[i] = (k < ke && m < mmax) ? *(const float4*)(A + (int64_t)k * g.lda + m) : make_float4(0, 0, 0, 0);
        }
        if (!TB) {
          const int k = k0 + (tid >> 5) + 8 * i, n = n0 + (tid & 31) * 4;
          rb[i] = (k < ke && n < g.N) ? *(const float4*)(Bm + (int64_t)k * g.ldb + n) : make_float4(0, 0, 0, 0);
        } else {
          const int n = n0 + (tid >> 2) + 64 * i, k = k0 + (tid & 3) * 4;
          rb[i] = (n < g.N && k < ke) ? *(const float4*)(Bm + (int64_t)n * g.ldb + k) : make_float4(0, 0, 0, 0);
        }
      }
    };
    auto store = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (!TA) {
          const int row = (tid >> 2) + 64 * i, kq = (tid & 3) * 4;
          as[buf][kq + 0][row] = ra[i].x;
          as[buf][kq + 1][row] = ra[i].y;
          as[buf][kq + 2][row] = ra[i].z;
          as[buf][kq + 3][row] = ra[i].w;
        } else {
          *(float4*)&as[buf][(tid >> 5) + 8 * i][(tid & 31) * 4] = ra[i];
        }
        if (!TB) {
          *(float4*)&bs[buf][(tid >> 5) + 8 * i][(tid & 31) * 4] = rb[i];
        } else {
          const int col = (tid >> 2) + 64 * i, kq = (tid & 3) * 4;
          bs[buf][kq + 0][col] = rb[i].x;
          bs[buf][kq + 1][col] = rb[i].y;
          bs[buf][kq + 2][col] = rb[i].z;
          bs[buf][kq + 3][col] = rb[i].w;
        }
      }
    };
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < ns; ++s) {
      if (s + 1 < ns) load(s + 1);
      const int buf = s & 1;
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        const float a0 = as[buf][2 * kk + hi][wm * 64 + lo], a1 = as[buf][2 * kk + hi][wm * 64 + 32 + lo];
        const float b0 = bs[buf][2 * kk + hi][wn * 64 + lo], b1 = bs[buf][2 * kk + hi][wn * 64 + 32 + lo];
        acc[0][0] = mfma32(a0, b0, acc[0][0]);
        acc[0][1] = mfma32(a0, b1, acc[0][1]);
        acc[1][0] = mfma32(a1, b0, acc[1][0]);
        acc[1][1] = mfma32(a1, b1, acc[1][1]);
      }
      if (s + 1 < ns) store(buf ^ 1);
      __syncthreads();
    }
  }
  // output element r of block (x, y): row 8 (r / 4) + 4 hi + r % 4, column lo
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int col = n0 + wn * 64 + y * 32 + lo;
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + x * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row < g.M) Cm[(int64_t)row * g.ldc + col] = acc[x][y][r];
      }
    }
}

// out[e] = sum over s = 0, 1, ... of part[s * stride + e], e < n (n a multiple of 4)
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int64_t stride, int splits,
                                                         float* __restrict__ out, int64_t n) {
  const int64_t e = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (e >= n) return;
  float4 s = *(const float4*)(part + e);
  for (int k = 1; k < splits; ++k) {
    const float4 v = *(const float4*)(part + k * stride + e);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  *(float4*)(out + e) = s;
}

// Partial Gram matrices in fp64: part[split][b][i][j] = sum over the split's rows t of y[b][t][i] y[b][t][j],
// for the 64 x 64 tiles (ti, tj), ti >= tj, of the lower triangle.  Rows t >= mlim[b] * lim_mul are skipped.
__global__ __launch_bounds__(256) void gram64_kernel(const float* __restrict__ y, int64_t sy, int rows, int r,
                                                     const int32_t* __restrict__ mlim, int lim_mul, int chunk,
                                                     double* __restrict__ part) {
  __shared__ double ysi[GR][GT + 4];
  __shared__ double ysj[GR][GT + 4];
  int p = blockIdx.x, ti = 0;
  while (p > ti) p -= ++ti;  // tile p of the lower triangle: (ti, tj = p)
  const int tj = p;
  const int split = blockIdx.y, b = blockIdx.z, B = gridDim.z;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float* Y = y + b * sy;
  const int rend = mlim ? min(rows, mlim[b] * lim_mul) : rows;
  const int t_lo = split * chunk, t_hi = min(rend, t_lo + chunk);
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  for (int t0 = t_lo; t0 < t_hi; t0 += GR) {
    // 32 rows x 64 columns of each tile's column block: 512 quads each, two per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, tt = q >> 4, cq = (q & 15) * 4;
      const int t = t0 + tt;
      const int ci = ti * GT + cq, cj = tj * GT + cq;
      float4 vi = make_float4(0, 0, 0, 0), vj = make_float4(0, 0, 0, 0);
      if (t < t_hi && ci < r) vi = *(const float4*)(Y + (int64_t)t * r + ci);
      if (t < t_hi && cj < r) vj = *(const float4*)(Y + (int64_t)t * r + cj);
      ysi[tt][cq + 0] = vi.x;
      ysi[tt][cq + 1] = vi.y;
      ysi[tt][cq + 2] = vi.z;
      ysi[tt][cq + 3] = vi.w;
      ysj[tt][cq + 0] = vj.x;
      ysj[tt][cq + 1] = vj.y;
      ysj[tt][cq + 2] = vj.z;
      ysj[tt][cq + 3] = vj.w;
    }
    __syncthreads();
#pragma unroll 4
    for (int tt = 0; tt < GR; ++tt) {
      double a[4], c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = ysi[tt][4 * ty + u];
        c[u] = ysj[tt][4 * tx + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fma(a[u], c[v], acc[u][v]);
    }
    __syncthreads();
  }
  double* P = part + ((int64_t)split * B + b) * r * r;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = ti * GT + 4 * ty + u;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = tj * GT + 4 * tx + v;
      if (i < r && j < r) P[(int64_t)i * r + j] = acc[u][v];
    }
  }
}

// G[b] = sum over splits of the partials (lower triangle), in split order, mirrored into the upper one
__global__ __launch_bounds__(256) void gram_sum_kernel(const double* __restrict__ part, int splits, int B, int r,
                                                       double* __restrict__ G) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)B * r * r;
  if (e >= n) return;
  const int64_t ij = e % ((int64_t)r * r);
  const int i = (int)(ij / r), j = (int)(ij % r);
  if (j > i) return;
  double s = part[e];
  for (int k = 1; k < splits; ++k) s += part[k * n + e];
  G[e] = s;
  G[e - ij + (int64_t)j * r + i] = s;  // the mirror entry: G is stored whole
}

__device__ inline double readlane_f64(double v, int ln) {
  const int2 w = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(w.x, ln), __builtin_amdgcn_readlane(w.y, ln)));
}

// Cholesky factor of G[b] (fp64, full symmetric), G = L L^T, one workgroup of 16 waves per sequence; writes
// Lt[b][m][i] = L[i][m] (i >= m).  Left-looking by panels of 64 columns: the panel's entries are updated with
// the finished panels (each staged through LDS whole), then factored right-looking in registers.  Wave w holds
// the panel's columns w, w + 16, w + 32, w + 48 and lane l its rows l, l + 64, ... ; at step j the wave that
// holds column j broadcasts it (and the reciprocal of its pivot) through LDS, and entry (i, m), m > j, loses
// a[i][j] a[m][j] / a[j][j]; at the end L[i][m] = a[i][m] / sqrt(a[m][m]).  Every branch is uniform over a
// wave.  A pivot a[j][j] is the squared distance of column j of Y from the span of the columns before it; one
// at or below 2^-40 G[j][j] (an angle under about 8 fp32 roundoffs: numerically dependent at the precision of
// Y), or not finite, sets info[b] = 1 and the factor is replaced by the identity.
__global__ __launch_bounds__(CT) void chol_kernel(const double* __restrict__ Gm, double* __restrict__ Ltm, int r,
                                                  int32_t* __restrict__ info) {
  constexpr int NW = CT / 64;           // waves
  constexpr int KC = CP / NW;           // panel columns per wave
  constexpr int SR = RMAX / 64;         // row slots per lane
  constexpr int SR1 = (RMAX - CP) / 64; // row slots that exist past the first panel
  __shared__ double colb[2][RMAX];
  __shared__ double rcpb[2];
  __shared__ double stg[RMAX - CP][CP + 1];
  __shared__ int bad;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const double* G = Gm + (int64_t)b * r * r;
  double* Lt = Ltm + (int64_t)b * r * r;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int c0 = 0; c0 < r; c0 += CP) {
    const int w = min(CP, r - c0), rows = r - c0;
    double a[KC][SR], gdiag[KC], piv[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int m = wv + NW * k;
      gdiag[k] = m < w ? G[(int64_t)(c0 + m) * r + c0 + m] : 1.0;
      piv[k] = 1.0;
#pragma unroll
      for (int s = 0; s < SR; ++s) {
        const int i = lane + 64 * s;
        a[k][s] = (m < w && i < rows) ? G[(int64_t)(c0 + m) * r + c0 + i] : 0.0;  // G symmetric: row m
      }
    }
    // left-looking update by the finished panels; past the first panel at most RMAX - CP rows remain
    for (int m0 = 0; m0 < c0; m0 += CP) {
#pragma unroll 4
      for (int q = 0; q < STG_LOADS; ++q) {
        const int e = tid + CT * q, mm = e / (RMAX - CP), ii = e - mm * (RMAX - CP);
        if (ii < rows) stg[ii][mm] = Lt[(int64_t)(m0 + mm) * r + c0 + ii];
      }
      __syncthreads();
#pragma unroll 2
      for (int mm = 0; mm < CP; ++mm) {
        double li[SR1];
#pragma unroll
        for (int s = 0; s < SR1; ++s) li[s] = stg[lane + 64 * s][mm];  // rows past `rows`: stale, never stored
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const double lm = stg[wv + NW * k][mm];
#pragma unroll
          for (int s = 0; s < SR1; ++s) a[k][s] = __builtin_fma(-li[s], lm, a[k][s]);
        }
      }
      __syncthreads();
    }
    for (int j = 0; j < w; ++j) {
      double* cb = colb[j & 1];
      const int kj = j / NW;
      if (wv == j % NW) {
        // entries above the diagonal or past `rows` are written too: they only meet entries never stored
#pragma unroll
        for (int k = 0; k < KC; ++k)
          if (k == kj) {
#pragma unroll
            for (int s = 0; s < SR; ++s) cb[lane + 64 * s] = a[k][s];
            if (lane == j) {
              rcpb[j & 1] = 1.0 / a[k][0];
              if (!(a[k][0] > 0x1p-40 * gdiag[k])) bad = 1;
            }
          }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int m = wv + NW * k;
        if (m == j) piv[k] = cb[j];
        if (m > j && m < w) {
          const double f = cb[m] * rcpb[j & 1];
#pragma unroll
          for (int s = 0; s < SR; ++s) a[k][s] = __builtin_fma(-cb[lane + 64 * s], f, a[k][s]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int m = wv + NW * k;
      if (m < w) {
        const double sq = sqrt(piv[k]), rs = 1.0 / sq;
#pragma unroll
        for (int s = 0; s < SR; ++s) {
          const int i = lane + 64 * s;
          if (i >= m && i < rows) Lt[(int64_t)(c0 + m) * r + c0 + i] = i == m ? sq : a[k][s] * rs;
        }
      }
    }
    __syncthreads();
  }
  if (bad) {
    for (int e = tid; e < r * r; e += CT) {
      const int m = e / r, i = e - m * r;
      if (i >= m) Lt[e] = i == m ? 1.0 : 0.0;
    }
    if (tid == 0) info[b] = 1;
  }
}

// R^-1 = L^-T from Lt (fp64), stored fp32 as rinv[b][c][m] = (L^-1)[m][c] (zero for m < c): column c of L^-1
// by forward substitution, one wave per column, the pending sums s_m = sum_{i<m} L[m][i] x_i held by lane
// (m - c) % 64; step i takes x_i = (delta_ic - s_i) / L[i][i] and adds L[m][i] x_i (row i of Lt) to every s_m.
__global__ __launch_bounds__(256) void trinv_kernel(const double* __restrict__ Ltm, float* __restrict__ rinv, int r) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (c >= r) return;
  const double* Lt = Ltm + (int64_t)b * r * r;
  float* R = rinv + (int64_t)b * r * r + (int64_t)c * r;
  double s[4] = {0.0, 0.0, 0.0, 0.0}, x[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = c; i < r; ++i) {
    const int k = (i - c) >> 6, ln = (i - c) & 63;
    double lrow[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int m = c + lane + 64 * kk;
      lrow[kk] = (m > i && m < r) ? Lt[(int64_t)i * r + m] : 0.0;
    }
    const double sk = k == 0 ? s[0] : k == 1 ? s[1] : k == 2 ? s[2] : s[3];
    const double si = readlane_f64(sk, ln);
    const double xi = ((i == c ? 1.0 : 0.0) - si) / Lt[(int64_t)i * r + i];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk == k && lane == ln) x[kk] = xi;
      s[kk] = __builtin_fma(lrow[kk], xi, s[kk]);
    }
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int m = c + lane + 64 * kk;
    if (m < r) R[m] = (float)x[kk];
  }
  for (int m = lane; m < c; m += 64) R[m] = 0.0f;
}

__global__ void tfit_setup_kernel(const int32_t* __restrict__ seq_len, int B, int max_T, int rows_per_token,
                                  int32_t* __restrict__ lens4, int32_t* __restrict__ info) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int t = min(max(seq_len[b], 0), max_T);
  lens4[4 * b] = t * rows_per_token;
  if (info) info[b] = 0;
}

inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int64_t D;          // columns of the token-mode unfolding
  int ksplit, kchunk; // split of the token sum in A^T Q and Q^T A
  int gsplit_t, gchunk_t, gsplit_d, gchunk_d;
  size_t o_y, o_q1, o_q, o_z, o_z1, o_kp, o_gp, o_g, o_lt, o_ri, o_len, o_fit, o_fg, total;
  size_t fit_bytes;
};

inline int gram_tiles(int r) { const int n = (r + GT - 1) / GT; return n * (n + 1) / 2; }

inline void gram_split(int rows, int r, int B, int* splits, int* chunk) {
  const int want = std::max(1, 1024 / std::max(1, gram_tiles(r) * B));
  int s = std::min(want, std::max(1, (rows + GR - 1) / GR));
  int c = (rows + s - 1) / s;
  c = (c + GR - 1) / GR * GR;
  *chunk = c;
  *splits = std::max(1, (rows + c - 1) / c);
}

}  // namespace tf

namespace {
// The feature factor does not depend on the token factor, so it runs on a stream of the library's own (one per
// device, default priority), forked from and joined back to the caller's stream with events; its eigensolver
// (one workgroup per sequence) then overlaps the token factor's products.  The lock is held while a call
// enqueues its fork and join, so calls from several host threads keep their event pairs apart.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

SideStream* side_stream() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& s = g_side[dev];
  if (!s.st) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      if (f) (void)hipEventDestroy(f);
      (void)hipStreamDestroy(st);
      return nullptr;
    }
    s.st = st;
    s.fork = f;
    s.join = j;
  }
  return &s;
}
}  // namespace

static kvc_fit_in feature_fit_in(const kvc_tucker_fit_in& in, int64_t rows_per_token, const int32_t* lens4, int b) {
  kvc_fit_in f{};
  f.B = 1;
  f.max_T = (int32_t)(in.max_T * rows_per_token);
  f.n_kv_heads = 1;
  f.head_dim = in.head_dim;
  f.rank = in.r_f;
  f.r_cap = in.r_f;
  f.seq_len = lens4 ? lens4 + 4 * b : nullptr;
  f.x = in.x ? in.x + (int64_t)b * in.max_T * rows_per_token * in.head_dim : nullptr;
  return f;
}

static kvc_status tfit_plan(const kvc_tucker_fit_in& in, tf::Plan* p) {
  using namespace tf;
  if (in.B < 1 || in.max_T < 1 || in.n_layers < 1 || in.n_kv_heads < 1 || in.head_dim < 1 || in.power_iters < 0 ||
      in.power_iters > 8)
    return KVC_ERR_INVALID_ARG;
  if (in.head_dim != D) return KVC_ERR_UNSUPPORTED;
  if (in.r_t < 4 || in.r_t > RMAX || in.r_t % 4 || in.r_f < 4 || in.r_f > D || in.r_f % 4) return KVC_ERR_UNSUPPORTED;
  const int ld = in.ut_ld ? in.ut_ld : in.r_t;
  if (ld < in.r_t || ld % 4) return KVC_ERR_INVALID_ARG;
  const int64_t rpt = (int64_t)in.n_layers * in.n_kv_heads;
  p->D = rpt * D;
  if (p->D > (1 << 20) || (int64_t)in.max_T * rpt >= (1 << 30) || (int64_t)in.B * in.max_T * p->D >= ((int64_t)1 << 40) ||
      (int64_t)in.B * in.n_layers * in.n_kv_heads > 65535 || in.B > 65535)
    return KVC_ERR_INVALID_ARG;
  const int64_t r = in.r_t, B = in.B, T = in.max_T;
  // split of the token sum: about 2048 workgroups over the (D / 128) x (r / 128) tiles, chunks of 256 tokens or more
  const int64_t tiles = ((p->D + BM - 1) / BM) * ((r + BN - 1) / BN) * B;
  int ks = (int)std::max<int64_t>(1, std::min<int64_t>((2048 + tiles - 1) / tiles, (T + 255) / 256));
  ks = std::min(ks, 16);
  int kc = (int)((T + ks - 1) / ks);
  kc = (kc + BK - 1) / BK * BK;
  p->kchunk = kc;
  p->ksplit = (int)((T + kc - 1) / kc);
  gram_split((int)T, (int)r, (int)B, &p->gsplit_t, &p->gchunk_t);
  gram_split((int)p->D, (int)r, (int)B, &p->gsplit_d, &p->gchunk_d);
  const size_t fb = fit_part_floats(feature_fit_in(in, rpt, nullptr, 0)) * 4;  // one sequence's partial Grams
  p->fit_bytes = fb;
  const size_t ybytes = al((size_t)B * T * r * 4), zbytes = al((size_t)B * p->D * r * 4);
  const int gs = std::max(p->gsplit_t, p->gsplit_d);
  size_t o = 0;
  p->o_y = o;   o += ybytes;
  p->o_q1 = o;  o += ybytes;
  p->o_q = o;   o += in.power_iters ? ybytes : 0;
  p->o_z = o;   o += zbytes;
  p->o_z1 = o;  o += zbytes;
  p->o_kp = o;  o += al((size_t)p->ksplit * B * p->D * r * 4);
  p->o_gp = o;  o += al((size_t)gs * B * r * r * 8);
  p->o_g = o;   o += al((size_t)B * r * r * 8);
  p->o_lt = o;  o += al((size_t)B * r * r * 8);
  p->o_ri = o;  o += al((size_t)B * r * r * 4);
  p->o_len = o; o += al((size_t)B * 20);
  p->o_fit = o; o += al(fb);
  p->o_fg = o;  o += al((size_t)B * D * D * 4);
  p->total = o;
  return KVC_OK;
}

template <bool TA, bool TB>
static hipError_t gemm(const tf::GemmArgs& g0, int batches, int splits, hipStream_t st) {
  tf::GemmArgs g = g0;
  g.tiles_m = (g.M + tf::BM - 1) / tf::BM;
  g.tiles_n = (g.N + tf::BN - 1) / tf::BN;
  if (g.kchunk <= 0) g.kchunk = (g.K + tf::BK - 1) / tf::BK * tf::BK;
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n), (unsigned)batches, (unsigned)splits);
  hipLaunchKernelGGL((tf::gemm_kernel<TA, TB>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

// orth of the B matrices y[b] [rows x r] (row stride r, batch stride sy): two CholeskyQR passes, the result in
// out (row stride ldo, batch stride so); tmp holds the first pass.
static hipError_t orth(const tf::Plan& p, char* ws, int B, int rows, int r, const float* y, int64_t sy, float* tmp,
                       float* out, int ldo, int64_t so, const int32_t* mlim, int gsplit, int gchunk, int32_t* info,
                       hipStream_t st) {
  using namespace tf;
  double* gp = (double*)(ws + p.o_gp);
  double* G = (double*)(ws + p.o_g);
  double* Lt = (double*)(ws + p.o_lt);
  float* ri = (float*)(ws + p.o_ri);
  for (int pass = 0; pass < 2; ++pass) {
    const float* src = pass == 0 ? y : tmp;
    const int64_t ss = pass == 0 ? sy : (int64_t)rows * r;
    hipLaunchKernelGGL(gram64_kernel, dim3(gram_tiles(r), gsplit, B), dim3(256), 0, st, src, ss, rows, r, mlim, 1,
                       gchunk, gp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)B * r * r;
    hipLaunchKernelGGL(gram_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, gp, gsplit, B, r, G);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(chol_kernel, dim3(B), dim3(CT), 0, st, G, Lt, r, info);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(trinv_kernel, dim3((r + 3) / 4, B), dim3(256), 0, st, Lt, ri, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GemmArgs g{};
    g.a = src;
    g.b = ri;
    g.c = pass == 0 ? tmp : out;
    g.M = rows;
    g.N = r;
    g.K = r;
    g.lda = r;
    g.ldb = r;
    g.ldc = pass == 0 ? r : ldo;
    g.sa_o = ss;
    g.sb_o = (int64_t)r * r;
    g.sc_o = pass == 0 ? (int64_t)rows * r : so;
    g.n_inner = 1;
    g.mlim = mlim;
    g.lim_mul = 1;
    if ((e = gemm<false, false>(g, B, 1, st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

kvc_status tfit_impl(const kvc_tucker_fit_in& in, float* u_t, float* u_f, float* core, int32_t* info, void* ws,
                     size_t ws_bytes, hipStream_t st, size_t* bytes_out) {
  using namespace tf;
  Plan p{};
  kvc_status s = tfit_plan(in, &p);
  if (s != KVC_OK) return s;
  if (bytes_out) {
    *bytes_out = p.total;
    return KVC_OK;
  }
  if (!in.seq_len || !in.x || !in.omega || !u_t || !u_f || !core || !ws) return KVC_ERR_INVALID_ARG;
  for (const void* q : {(const void*)in.x, (const void*)in.omega, (const void*)u_t, (const void*)u_f,
                        (const void*)core, (const void*)ws})
    if ((uintptr_t)q & 15u) return KVC_ERR_MISALIGNED;
  if (((uintptr_t)in.seq_len & 3u) || ((uintptr_t)info & 3u)) return KVC_ERR_MISALIGNED;
  if (ws_bytes < p.total) return KVC_ERR_WORKSPACE;
  char* w = (char*)ws;
  const int B = in.B, T = in.max_T, r = in.r_t;
  const int64_t DX = p.D, rpt = (int64_t)in.n_layers * in.n_kv_heads;
  const int ldo = in.ut_ld ? in.ut_ld : r;
  float* y = (float*)(w + p.o_y);
  float* q1 = (float*)(w + p.o_q1);
  float* qc = in.power_iters ? (float*)(w + p.o_q) : u_t;
  float* z = (float*)(w + p.o_z);
  float* z1 = (float*)(w + p.o_z1);
  float* kp = (float*)(w + p.o_kp);
  int32_t* lens4 = (int32_t*)(w + p.o_len);
  int32_t* inf = info ? info : lens4 + 4 * B;  // words of the length block when info is NULL
  hipLaunchKernelGGL(tfit_setup_kernel, dim3((B + 63) / 64), dim3(64), 0, st, in.seq_len, B, T, (int)rpt, lens4,
                     info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  // U_f on the side stream (when one is available; otherwise in order on the caller's stream): the basis fit of
  // each sequence's (t, l, h) rows, its Gram matrix, then one eigensolver launch for all sequences
  std::lock_guard<std::mutex> side_lock(g_side_mu);
  SideStream* side = side_stream();
  hipStream_t fst = st;
  if (side && hipEventRecord(side->fork, st) == hipSuccess && hipStreamWaitEvent(side->st, side->fork, 0) == hipSuccess)
    fst = side->st;
  float* fg = (float*)(w + p.o_fg);
  for (int b = 0; b < B; ++b) {
    const kvc_fit_in f = feature_fit_in(in, rpt, lens4, b);
    if ((e = fit_gram_launch(f, (float*)(w + p.o_fit), fg + (int64_t)b * tf::D * tf::D, fst)) != hipSuccess)
      return hip_fail(e);
  }
  if ((e = fit_eig_launch(fg, B, in.r_f, in.r_f, nullptr, u_f, nullptr, fst)) != hipSuccess) return hip_fail(e);
  if (fst != st && (e = hipEventRecord(side->join, fst)) != hipSuccess) return hip_fail(e);
  const int64_t sx = (int64_t)T * DX;  // batch stride of x
  // Y = A Omega
  GemmArgs g{};
  g.a = in.x;
  g.b = in.omega;
  g.c = y;
  g.M = T;
  g.N = r;
  g.K = (int)DX;
  g.lda = (int)DX;
  g.ldb = r;
  g.ldc = r;
  g.sa_o = sx;
  g.sc_o = (int64_t)T * r;
  g.n_inner = 1;
  g.mlim = in.seq_len;
  g.lim_mul = 1;
  if ((e = gemm<false, false>(g, B, 1, st)) != hipSuccess) return hip_fail(e);
  for (int it = 0; it <= in.power_iters; ++it) {
    const bool last = it == in.power_iters;
    float* qdst = last ? u_t : qc;
    const int ld = last ? ldo : r;
    if ((e = orth(p, w, B, T, r, y, (int64_t)T * r, q1, qdst, ld, (int64_t)T * ld, in.seq_len, p.gsplit_t, p.gchunk_t,
                  inf, st)) != hipSuccess)
      return hip_fail(e);
    if (last) break;
    // Z = A^T Q over token chunks, then the chunks summed in order
    GemmArgs gz{};
    gz.a = in.x;
    gz.b = qc;
    gz.c = kp;
    gz.M = (int)DX;
    gz.N = r;
    gz.K = T;
    gz.lda = (int)DX;
    gz.ldb = r;
    gz.ldc = r;
    gz.sa_o = sx;
    gz.sb_o = (int64_t)T * r;
    gz.sc_o = DX * r;
    gz.sc_split = (int64_t)B * DX * r;
    gz.n_inner = 1;
    gz.kchunk = p.kchunk;
    gz.klim = in.seq_len;
    gz.lim_mul = 1;
    if ((e = gemm<true, false>(gz, B, p.ksplit, st)) != hipSuccess) return hip_fail(e);
    const int64_t nz = (int64_t)B * DX * r;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((nz / 4 + 255) / 256)), dim3(256), 0, st, kp, nz, p.ksplit, z,
                       nz);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e);
    if ((e = orth(p, w, B, (int)DX, r, z, DX * r, z1, z, r, DX * r, nullptr, p.gsplit_d, p.gchunk_d, inf, st)) !=
        hipSuccess)
      return hip_fail(e);
    // Y = A Z
    GemmArgs gy = g;
    gy.b = z;
    gy.sb_o = DX * r;
    if ((e = gemm<false, false>(gy, B, 1, st)) != hipSuccess) return hip_fail(e);
  }
  // P = U_t^T A [r x D], token chunks summed in order
  GemmArgs gp{};
  gp.a = u_t;
  gp.b = in.x;
  gp.c = kp;
  gp.M = r;
  gp.N = (int)DX;
  gp.K = T;
  gp.lda = ldo;
  gp.ldb = (int)DX;
  gp.ldc = (int)DX;
  gp.sa_o = (int64_t)T * ldo;
  gp.sb_o = sx;
  gp.sc_o = (int64_t)r * DX;
  gp.sc_split = (int64_t)B * r * DX;
  gp.n_inner = 1;
  gp.kchunk = p.kchunk;
  gp.klim = in.seq_len;
  gp.lim_mul = 1;
  if ((e = gemm<true, false>(gp, B, p.ksplit, st)) != hipSuccess) return hip_fail(e);
  const int64_t np_ = (int64_t)B * r * DX;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((np_ / 4 + 255) / 256)), dim3(256), 0, st, kp, np_, p.ksplit, z,
                     np_);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e);
  // the core needs U_f: join the side stream
  if (fst != st && (e = hipStreamWaitEvent(st, side->join, 0)) != hipSuccess) return hip_fail(e);
  // core[b][l][h] = P[b][:, (l, h) block] U_f[b]
  GemmArgs gc{};
  gc.a = z;
  gc.b = u_f;
  gc.c = core;
  gc.M = r;
  gc.N = in.r_f;
  gc.K = tf::D;
  gc.lda = (int)DX;
  gc.ldb = in.r_f;
  gc.ldc = in.r_f;
  gc.sa_o = (int64_t)r * DX;
  gc.sa_i = tf::D;
  gc.sb_o = (int64_t)tf::D * in.r_f;
  gc.sc_o = rpt * r * in.r_f;
  gc.sc_i = (int64_t)r * in.r_f;
  gc.n_inner = (int)rpt;
  if ((e = gemm<false, false>(gc, (int)(B * rpt), 1, st)) != hipSuccess) return hip_fail(e);
  return KVC_OK;
}

}  // namespace kvc
