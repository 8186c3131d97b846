// fit.hip -- per-KV-head basis fitting for the prefill side (gfx950): the r leading right singular vectors of
// each head's pre-RoPE rows ("JoLT: Near-Lossless KV Cache Compression", "Key findings": per-head SVD, keys
// decomposed before RoPE; "A JoLT for the KV cache", abstract: the feature mode is the one truncated).
//
// At head dimension 128 the decomposition is exact through the 128 x 128 Gram matrix G = X^T X: its
// eigenvectors are the right singular vectors of X and its eigenvalues the squared singular values.
//   1. fit_gram_kernel: G on v_mfma_f32_32x32x2_f32 (fp32 operands and accumulation).  Features are tiled
//      as four 32-row tiles with row i of tile I <-> feature 4i + I, so one 16-byte load per lane (features
//      4i..4i+3 of one token) supplies the operands of all ten upper tiles (I <= J) of a two-token step.
//      A workgroup (h, slice) walks the 1024-token chunks slice, slice + n_slices, ... of all sequences, its
//      four waves each take a quarter of every chunk, and their sums are added in a fixed order in LDS into
//      one partial per workgroup.
//   2. fit_reduce_kernel: the partials of a head summed in slice order into the symmetric G.
//   3. fit_eig_kernel: one workgroup of 1024 threads per head runs cyclic Jacobi (Golub & Van Loan's
//      symmetric Schur rotations) on G in LDS, 64 disjoint rotations per round in round-robin order (127
//      rounds a sweep, every pair once), until a sweep rotates nothing; eigenvalues sorted in decreasing
//      order, each column's entry of largest magnitude made positive.
// Every summation order is fixed, so the same inputs give bit-identical outputs.
#include <math.h>

#include <algorithm>

#include "kvc_common.hpp"

namespace kvc {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace fit {
constexpr int D = 128;
constexpr int NT = 10;          // upper tiles I <= J of the 4 x 4 tiling
constexpr int TF = 1024;        // floats per 32 x 32 tile
constexpr int CHUNK = 1024;     // tokens of one sequence per work item
constexpr int WTOK = CHUNK / 4;  // tokens per wave per work item
constexpr int U = 8;            // two-token steps per load batch
constexpr int MAX_SWEEPS = 30;
constexpr int EIG_THREADS = 1024;
constexpr int EIG_WAVES = EIG_THREADS / 64;
constexpr int BPW = 64 / EIG_WAVES;            // row pairs per wave in the block update
constexpr int VPT = D * 64 / EIG_THREADS;      // entries of V^T rows p and q per thread

__host__ __device__ constexpr int tile_i(int k) { return k < 4 ? 0 : k < 7 ? 1 : k < 9 ? 2 : 3; }
__host__ __device__ constexpr int tile_j(int k) { return k < 4 ? k : k < 7 ? k - 3 : k < 9 ? k - 5 : 3; }

inline int slices(int Hkv, int B, int max_T) {
  const int items = B * ceil_div(max_T, CHUNK);
  const int target = std::max(1, 512 / std::max(Hkv, 1));  // about 512 workgroups: two per compute unit
  return std::max(1, std::min(items, target));
}
inline size_t part_floats(int Hkv, int n_slices) { return (size_t)Hkv * n_slices * NT * TF; }
}  // namespace fit

__device__ inline f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256, 2) void fit_gram_kernel(const float* __restrict__ x, const int32_t* __restrict__ seq_len,
                                                          int B, int max_T, int Hkv, int n_slices, float* __restrict__ part) {
  using namespace fit;
  __shared__ float red[NT * TF];
  const int h = blockIdx.x % Hkv, slice = blockIdx.x / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 31, hh = lane >> 5;
  const int n_chunks = ceil_div(max_T, CHUNK);
  const size_t tstride = (size_t)Hkv * D;
  f32x16 acc[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) acc[k] = f32x16{};

  for (int item = slice; item < B * n_chunks; item += n_slices) {
    const int b = item / n_chunks, c = item % n_chunks;
    const int T = min(max(seq_len[b], 0), max_T);
    const int t0 = c * CHUNK + wv * WTOK;
    const int t1 = min(t0 + WTOK, T);
    if (t0 >= t1) continue;  // wave-uniform
    const float* base = x + ((size_t)b * max_T * Hkv + h) * D + 4 * m;
    // step s covers tokens t0 + 2s (lanes 0-31) and t0 + 2s + 1 (lanes 32-63); rows past t1 read as zero
    const int nsteps = (t1 - t0 + 1) / 2;
    auto load = [&](int s) -> f4 {
      const int t = t0 + 2 * s + hh;
      return t < t1 ? *(const f4*)(base + (size_t)t * tstride) : f4{0, 0, 0, 0};
    };
    f4 cur[U], nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load(u);
    for (int s0 = 0; s0 < nsteps; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) nxt[u] = load(s0 + U + u);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const f4 v = cur[u];
#pragma unroll
        for (int k = 0; k < NT; ++k) acc[k] = mfma_f32(v[tile_i(k)], v[tile_j(k)], acc[k]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
  }
  // the four waves' sums, added in wave order; entry (k, e = 64 v + lane) of the tile layout
  for (int w = 0; w < 4; ++w) {
    if (wv == w)
#pragma unroll
      for (int k = 0; k < NT; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int e = k * TF + 64 * v + lane;
          red[e] = (w == 0 ? 0.0f : red[e]) + acc[k][v];
        }
    __syncthreads();
  }
  float* dst = part + ((size_t)h * n_slices + slice) * NT * TF;
  for (int e = tid; e < NT * TF; e += 256) dst[e] = red[e];
}

// G[h] (row-major 128 x 128, symmetric) = sum over slices of the partials, in slice order.  Entry e = 64 v +
// lane of tile k holds G[4 i + I][4 j + J] with i = 8 (v / 4) + 4 (lane / 32) + v % 4, j = lane % 32.
__global__ __launch_bounds__(256) void fit_reduce_kernel(const float* __restrict__ part, int n_slices, float* __restrict__ gram) {
  using namespace fit;
  const int h = blockIdx.x / (NT * 4), k = (blockIdx.x / 4) % NT;
  const int e = (blockIdx.x % 4) * 256 + threadIdx.x;
  const float* src = part + (size_t)h * n_slices * NT * TF + (size_t)k * TF + e;
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int sl = 0;
  for (; sl + 4 <= n_slices; sl += 4) {
    s0 += src[(size_t)(sl + 0) * NT * TF];
    s1 += src[(size_t)(sl + 1) * NT * TF];
    s2 += src[(size_t)(sl + 2) * NT * TF];
    s3 += src[(size_t)(sl + 3) * NT * TF];
  }
  for (; sl < n_slices; ++sl) s0 += src[(size_t)sl * NT * TF];
  const float s = (s0 + s1) + (s2 + s3);
  const int v = e / 64, lane = e % 64;
  const int i = 8 * (v / 4) + 4 * (lane / 32) + v % 4, j = lane % 32;
  const int I = tile_i(k), J = tile_j(k);
  const int fi = 4 * i + I, fj = 4 * j + J;
  float* G = gram + (size_t)h * D * D;
  if (I < J) {
    G[fi * D + fj] = s;
    G[fj * D + fi] = s;
  } else if (i <= j) {  // diagonal tile: one of the two mirrored entries defines both
    G[fi * D + fj] = s;
    G[fj * D + fi] = s;
  }
}

// Pair P of round k (0..126) of the round-robin schedule over 128 indices: (k, 127) for P = 0, else
// ((k + P) mod 127, (k - P) mod 127); over the 127 rounds every pair meets once (127 is prime).  The pair is
// left unordered: across the lanes of a wave (consecutive P) both members then run through consecutive
// indices, so the block updates' LDS accesses fall on distinct banks.
__device__ inline void rr_pair(int k, int P, int& p, int& q) {
  if (P == 0) {
    p = k;
    q = 127;
  } else {
    p = k + P;
    q = k - P;
    p -= p >= 127 ? 127 : 0;
    q += q < 0 ? 127 : 0;
  }
}

namespace fit {
constexpr int VS = D + 4;  // row stride of V^T (floats): 16-byte rows, and column walks spread over the banks
constexpr int AS = D + 1;  // row stride of A (floats): rows and columns both walk across the banks
}

// Storage: A (the matrix being diagonalized) keeps its upper triangle only, entry (i, j), i <= j, at
// A[i * AS + j]; V^T keeps eigenvector c in row c.  Per round, the 64 disjoint pairs (p_P, q_P) split A into
// 2 x 2 blocks (P, Q); block (P, Q) with P <= Q owns every stored entry it touches, so the blocks update in
// place without conflicts.
__global__ __launch_bounds__(fit::EIG_THREADS) void fit_eig_kernel(const float* __restrict__ gram, int rank, int r_cap,
                                                        uint16_t* __restrict__ basis_bf16, float* __restrict__ basis_f32,
                                                        float* __restrict__ sigma2) {
  using namespace fit;
  extern __shared__ __attribute__((aligned(16))) float eig_smem[];
  float* A = eig_smem;                  // [128][AS], upper triangle
  float* Vt = A + D * AS;               // [128][VS] (16-byte aligned: D * AS is a multiple of 4)
  float* cs = Vt + D * VS;              // [2 rounds][64][4]: c, s, t = s / c
  int* pq = (int*)(cs + 2 * 256);       // [2 rounds][64][2]: the pair
  float* lam = (float*)(pq + 2 * 128);  // [128]
  int* order = (int*)(lam + D);         // [128] eigenvector index of output column c
  int* flag = order + D;                // [0..1] rotated in round parity; [2..3] rotated in sweep parity
  float* sgn = (float*)(flag + 4);      // [128]
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* G = gram + (size_t)h * D * D;
  for (int e = tid; e < D * D; e += EIG_THREADS) A[(e / D) * AS + e % D] = G[e];
  for (int e = tid; e < D * VS; e += EIG_THREADS) Vt[e] = (e / VS == e % VS) ? 1.0f : 0.0f;
  if (tid < 4) flag[tid] = 0;
  __syncthreads();
  // trace (the sum of the eigenvalues of a positive semidefinite G, at least its largest) sets the absolute
  // floor of the off-diagonal entries worth rotating away: u tr(G).  Entries below it bound the angle error of
  // eigenvector c by about sqrt(128) u tr / gap_c, far below what the fp32 Gram matrix itself carries; rotating
  // them away would only chase rounding noise for another sweep or two.
  float tr = 0.0f;
  for (int i = 0; i < D; ++i) tr += fabsf(A[i * AS + i]);
  const float floor_abs = tr * 0x1p-24f;
  auto sym = [](int i, int j) -> int { return i <= j ? i * AS + j : j * AS + i; };  // stored entry (i, j)

  for (int sweep = 0; sweep < MAX_SWEEPS; ++sweep) {
    for (int k = 0; k < 127; ++k) {
      const int rb = (sweep * 127 + k) & 1;  // parity of the global round count: consecutive rounds alternate
      float* csr = cs + rb * 256;
      int* pqr = pq + rb * 128;
      if (tid < 64) {
        // this wave alone writes the round's tables and flags; the slots of parity rb were last read before the
        // previous round's first barrier (tables) or right after it (the round flag, then known to be 0 if the
        // round was skipped); the other parity's round flag is cleared here for the next round
        if (tid == 0) flag[rb ^ 1] = 0;
        int p, q;
        rr_pair(k, tid, p, q);
        const float app = A[p * AS + p], aqq = A[q * AS + q], apq = A[sym(p, q)];
        // the rotation of the symmetric 2 x 2 problem (Golub & Van Loan's symmetric Schur step), with the
        // hardware square root, reciprocal and reciprocal square root (about 1 ulp): any c, s with c^2 + s^2 = 1
        // to a few ulps serve, and the correctly rounded sequences would lengthen the round's serial part
        float c = 1.0f, s = 0.0f, ts = 0.0f;
        if (fabsf(apq) > floor_abs &&
            fabsf(apq) > 0x1p-24f * __builtin_amdgcn_sqrtf(fabsf(app)) * __builtin_amdgcn_sqrtf(fabsf(aqq))) {
          const float tau = (aqq - app) * (0.5f * __builtin_amdgcn_rcpf(apq));
          const float atau = fabsf(tau);
          const float t = atau > 1e18f ? 0.5f * __builtin_amdgcn_rcpf(atau)
                                       : __builtin_amdgcn_rcpf(atau + __builtin_amdgcn_sqrtf(1.0f + tau * tau));
          ts = tau >= 0.0f ? t : -t;
          c = __builtin_amdgcn_rsqf(1.0f + ts * ts);
          s = ts * c;
          flag[rb] = 1;
          flag[2 + (sweep & 1)] = 1;
        }
        *(f4*)(csr + 4 * tid) = f4{c, s, ts, 0.0f};
        pqr[2 * tid] = p;
        pqr[2 * tid + 1] = q;
      }
      __syncthreads();
      if (!flag[rb]) continue;  // uniform: nothing rotates this round
      // A <- J^T A J on the blocks P <= Q (wave w takes the row pairs P = BPW w .., lane = Q) and V <- V J on
      // rows p, q of V^T (VPT entries per thread: pair tid / (D / VPT), entries VPT (tid % (D / VPT)) ..).  The blocks of
      // a round are disjoint, so every read is issued first, then the arithmetic, then the writes: one LDS
      // round trip per round instead of one per block.
      {
        const int Q = tid & 63;
        const f4 cq = *(const f4*)(csr + 4 * Q);
        const int p2 = pqr[2 * Q], q2 = pqr[2 * Q + 1];
        int ad[BPW][4];
        float m[BPW][4];
        f4 cpj[BPW];
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
          const int P = BPW * (tid >> 6) + j;
          cpj[j] = *(const f4*)(csr + 4 * P);
          const int p1 = pqr[2 * P], q1 = pqr[2 * P + 1];
          ad[j][0] = sym(p1, p2);
          ad[j][1] = sym(p1, q2);
          ad[j][2] = sym(q1, p2);
          ad[j][3] = sym(q1, q2);
#pragma unroll
          for (int e = 0; e < 4; ++e) m[j][e] = A[ad[j][e]];
        }
        constexpr int NV = VPT / 4;
        const int PV = tid / (D / VPT), seg = VPT * (tid % (D / VPT));
        const f4 cv = *(const f4*)(csr + 4 * PV);
        f4* vp = (f4*)(Vt + pqr[2 * PV] * VS + seg);
        f4* vq = (f4*)(Vt + pqr[2 * PV + 1] * VS + seg);
        f4 va[NV], vb[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          va[i] = vp[i];
          vb[i] = vq[i];
        }
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
          const int P = BPW * (tid >> 6) + j;
          const float c1 = cpj[j][0], s1 = cpj[j][1], c2 = cq[0], s2 = cq[1];
          const float m00 = m[j][0], m01 = m[j][1], m10 = m[j][2], m11 = m[j][3];
          const float n00 = c1 * m00 - s1 * m10, n01 = c1 * m01 - s1 * m11;
          const float n10 = s1 * m00 + c1 * m10, n11 = s1 * m01 + c1 * m11;
          float r00 = c2 * n00 - s2 * n01, r01 = s2 * n00 + c2 * n01;
          float r10 = c2 * n10 - s2 * n11, r11 = s2 * n10 + c2 * n11;
          if (P == Q) {
            // the rotated pair's own block (entries (p,p), (p,q) twice, (q,q)): a_pq becomes zero and the
            // diagonal moves by t a_pq (the direct form keeps the rounding of the many small updates off the
            // eigenvalues); a pair left unrotated keeps its entries
            r00 = m00 - cpj[j][2] * m01;
            r11 = m11 + cpj[j][2] * m01;
            r01 = s1 != 0.0f ? 0.0f : m01;
            r10 = r01;
          }
          if (P <= Q && (s1 != 0.0f || s2 != 0.0f)) {
            A[ad[j][0]] = r00;
            A[ad[j][1]] = r01;
            A[ad[j][2]] = r10;
            A[ad[j][3]] = r11;
          }
        }
        if (cv[1] != 0.0f)
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            vp[i] = cv[0] * va[i] - cv[1] * vb[i];
            vq[i] = cv[1] * va[i] + cv[0] * vb[i];
          }
      }
      __syncthreads();
    }
    // the sweep flags: set only by the first wave; the one for the next sweep is cleared by that wave here,
    // in program order before it can set it, and every thread read this sweep's after the same barrier
    const int rotated = flag[2 + (sweep & 1)];
    __syncthreads();
    if (tid == 0) flag[2 + ((sweep + 1) & 1)] = 0;
    if (!rotated) break;
  }
  __syncthreads();
  if (tid < D) order[tid] = tid;  // a complete permutation even if non-finite values make positions collide
  __syncthreads();
  // eigenvalues in decreasing order (index order among equal values)
  if (tid < D) {
    const float l = A[tid * AS + tid];
    int pos = 0;
    for (int j = 0; j < D; ++j) {
      const float lj = A[j * AS + j];
      pos += (lj > l) || (lj == l && j < tid);
    }
    order[pos] = tid;
    lam[pos] = l;
  }
  __syncthreads();
  // output column c: unit norm (the rotations' rounding lets the norms drift by a few ulps), its entry of
  // largest magnitude positive (the first one on ties)
  if (tid < D) {
    const float* row = Vt + order[tid] * VS;
    float best = -1.0f, val = 0.0f, nrm = 0.0f;
    for (int i = 0; i < D; ++i) {
      const float v = row[i];
      nrm += v * v;
      if (fabsf(v) > best) {
        best = fabsf(v);
        val = v;
      }
    }
    sgn[tid] = (val < 0.0f ? -1.0f : 1.0f) / sqrtf(nrm);
    if (sigma2) sigma2[(size_t)h * D + tid] = fmaxf(lam[tid], 0.0f);
  }
  __syncthreads();
  if (basis_bf16)
    for (int e = tid; e < D * r_cap; e += EIG_THREADS) {
      const int d = e / r_cap, c = e % r_cap;
      basis_bf16[(size_t)h * D * r_cap + e] = c < rank ? f32_to_bf16_rne(sgn[c] * Vt[order[c] * VS + d]) : (uint16_t)0;
    }
  if (basis_f32)
    for (int e = tid; e < D * rank; e += EIG_THREADS) {
      const int d = e / rank, c = e % rank;
      basis_f32[(size_t)h * D * rank + e] = sgn[c] * Vt[order[c] * VS + d];
    }
}

namespace fit {
constexpr size_t EIG_LDS = ((size_t)D * AS + D * VS + 2 * 256 + 2 * 128 + D + D + 4 + D) * 4;
}

kvc_status hip_fail(hipError_t e);

kvc_status fit_impl(const kvc_fit_in& in, uint16_t* basis_bf16, float* basis_f32, float* sigma2, void* ws,
                    size_t ws_bytes, hipStream_t st, size_t* bytes_out) {
  using namespace fit;
  if (in.B < 1 || in.max_T < 1 || in.n_kv_heads < 1 || in.head_dim < 1) return KVC_ERR_INVALID_ARG;
  if (in.head_dim != D) return KVC_ERR_UNSUPPORTED;
  if (in.rank < 1 || in.rank > D || in.r_cap < in.rank || in.r_cap > D) return KVC_ERR_INVALID_ARG;
  if ((int64_t)in.B * in.max_T * in.n_kv_heads * D >= ((int64_t)1 << 40)) return KVC_ERR_UNSUPPORTED;
  const int n_slices = slices(in.n_kv_heads, in.B, in.max_T);
  const size_t pf = part_floats(in.n_kv_heads, n_slices);
  const size_t need = (pf + (size_t)in.n_kv_heads * D * D) * sizeof(float);
  if (bytes_out) {
    *bytes_out = need;
    return KVC_OK;
  }
  if (!in.seq_len || !in.x || !ws || (!basis_bf16 && !basis_f32 && !sigma2)) return KVC_ERR_INVALID_ARG;
  for (const void* p : {(const void*)in.seq_len, (const void*)in.x, (const void*)basis_bf16, (const void*)basis_f32,
                        (const void*)sigma2, (const void*)ws})
    if ((uintptr_t)p & 15u) return KVC_ERR_MISALIGNED;
  if (ws_bytes < need) return KVC_ERR_WORKSPACE;
  float* part = (float*)ws;
  float* gram = part + pf;
  hipError_t e = mark(g_marks.begin, st);
  if (e != hipSuccess) return hip_fail(e);
  fit_gram_kernel<<<in.n_kv_heads * n_slices, 256, 0, st>>>(in.x, in.seq_len, in.B, in.max_T, in.n_kv_heads, n_slices,
                                                             part);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  e = mark(g_marks.end, st);
  if (e != hipSuccess) return hip_fail(e);
  fit_reduce_kernel<<<in.n_kv_heads * NT * 4, 256, 0, st>>>(part, n_slices, gram);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  e = hipFuncSetAttribute((const void*)fit_eig_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)EIG_LDS);
  if (e != hipSuccess) return hip_fail(e);
  fit_eig_kernel<<<in.n_kv_heads, EIG_THREADS, EIG_LDS, st>>>(gram, in.rank, in.r_cap, basis_bf16, basis_f32, sigma2);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return KVC_OK;
}

// The two passes of fit_impl as separate launches, for callers that fit several independent row sets: the
// Gram matrices of in's heads into gram [Hkv][D][D] (part: fit_part_floats(in) floats), and the eigensolver
// over n such matrices at once (one workgroup each).
size_t fit_part_floats(const kvc_fit_in& in) {
  return fit::part_floats(in.n_kv_heads, fit::slices(in.n_kv_heads, in.B, in.max_T));
}

hipError_t fit_gram_launch(const kvc_fit_in& in, float* part, float* gram, hipStream_t st) {
  using namespace fit;
  const int n_slices = slices(in.n_kv_heads, in.B, in.max_T);
  fit_gram_kernel<<<in.n_kv_heads * n_slices, 256, 0, st>>>(in.x, in.seq_len, in.B, in.max_T, in.n_kv_heads, n_slices,
                                                             part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  fit_reduce_kernel<<<in.n_kv_heads * NT * 4, 256, 0, st>>>(part, n_slices, gram);
  return hipGetLastError();
}

hipError_t fit_eig_launch(const float* gram, int n, int rank, int r_cap, uint16_t* basis_bf16, float* basis_f32,
                          float* sigma2, hipStream_t st) {
  using namespace fit;
  hipError_t e = hipFuncSetAttribute((const void*)fit_eig_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)EIG_LDS);
  if (e != hipSuccess) return e;
  fit_eig_kernel<<<n, EIG_THREADS, EIG_LDS, st>>>(gram, rank, r_cap, basis_bf16, basis_f32, sigma2);
  return hipGetLastError();
}

}  // namespace kvc
