// alloc.hip -- per-token rank allocation by query salience for the prefill side (gfx950): every token keeps a
// nonzero rank chosen by how much attention the prefill's last queries pay it ("VarRate: Training-Free
// Variable-Rate KV Cache Compression for Long-Context LLMs", "Method" and "Principles").
//
// Salience of token t of sequence b: the attention probability that the last W (<= 32) prefill queries put on
// t, summed over those queries and all query heads; query i of the window sits at position seq_len - W + i,
// attends causally, and RoPE rotates queries and keys at their positions.
//   1. sal_kernel<1>: per (b, KV head h, split of 32-key tiles), wave w takes query head 4h + w with its window
//      queries as the 32 rows of v_mfma_f32_32x32x2_f32 (fp32 operands and accumulation) and each key tile as
//      the 32 columns; every lane keeps an online (max, sum) of exp2 for its 16 rows over its column, reduced
//      across the columns at the end into one (max, sum) per row and split.
//   2. sal_stats_kernel: the splits' (max, sum) combined per row, in split order.
//   3. sal_kernel<2>: the same scores again; p = 2^(s - max) / sum summed over the 32 rows of each query head,
//      then over the 4 heads in LDS: one value per (b, h, t).
//   4. sal_sum_kernel: the KV heads added in order; zero past seq_len.
// Keys are rotated once per tile into LDS, laid out by element parity so that each lane reads its 64 operand
// values as 16-byte runs; angles are t * theta_j in fp64 turns, reduced to [-1/2, 1/2], then v_sin / v_cos.
//
// Rank allocation (one workgroup per sequence): ranks come from a ladder r_0 < ... < r_{m-1}, every token
// starts at r_0; the step r_j -> r_{j+1} of token t costs r_{j+1} - r_j and gains the fp32 product s_t w_j
// (w non-increasing).  Steps are taken in decreasing order of gain, equal gains together, while the total stays
// within floor(mean_rank * seq_len).  The taken set is {gain >= lambda} for the smallest lambda whose set fits;
// the kernel finds lambda by bisection on the fp32 bit pattern (the order of non-negative floats), each probe
// a count over the sequence's steps.
#include <math.h>

#include <algorithm>

#include "kvc_common.hpp"

namespace kvc {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace sal {
constexpr int D = 128, GQ = 4, NP = 64;
constexpr int TILE = 32;          // keys per tile
constexpr int ROWS = 32;          // window queries per query head (rows of the MFMA); W <= ROWS
constexpr int KS = NP + 4;                // key row stride in LDS: 16-byte reads of consecutive tokens spread over the banks
constexpr int KT_FLOATS = 2 * TILE * KS;  // rotated key tile: [parity][token][64 (+4)]
__host__ __device__ inline int n_tiles(int max_T) { return ceil_div(max_T, TILE); }
inline int splits(int B, int Hkv, int max_T) {
  const int items = B * Hkv;
  const int target = std::max(1, ceil_div(512, items));  // about 512 workgroups: two per compute unit
  return std::max(1, std::min(target, n_tiles(max_T)));
}
struct Ws {  // workspace layout (floats)
  size_t part, stats, salh, total;
};
inline Ws ws_layout(int B, int Hkv, int max_T, int n_splits) {
  Ws w;
  size_t o = 0;
  w.part = o; o += (size_t)B * Hkv * n_splits * GQ * ROWS * 2;
  w.stats = o; o += (size_t)B * Hkv * GQ * ROWS * 2;
  w.salh = o; o += (size_t)B * Hkv * max_T;
  w.total = o;
  return w;
}
}  // namespace sal

struct SalArgs {
  const float* q;
  const float* k;
  const int32_t* seq_len;
  float* ws;
  int B, max_T, W, Hq, Hkv, n_splits, tiles_per_split;
  double theta;
  size_t ws_part, ws_stats, ws_salh;
};

__device__ inline f32x16 sal_mfma(float a, float b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }

// (cos, sin) of pos * theta_j, theta_j in turns per position (fp64), reduced to [-1/2, 1/2] turn
__device__ inline void turn_cs(double pos, double tturn, float& c, float& s) {
  double rev = pos * tturn;
  rev -= rint(rev);
  c = __builtin_amdgcn_cosf((float)rev);
  s = __builtin_amdgcn_sinf((float)rev);
}

template <int PASS>
__global__ __launch_bounds__(256, 2) void sal_kernel(SalArgs a) {
  using namespace sal;
  __shared__ __attribute__((aligned(16))) float kt[KT_FLOATS];
  __shared__ double tturn[NP];
  __shared__ float colsum[GQ][TILE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int split = blockIdx.x % a.n_splits;
  const int h = (blockIdx.x / a.n_splits) % a.Hkv;
  const int b = blockIdx.x / (a.n_splits * a.Hkv);
  const int T = min(max(a.seq_len[b], 0), a.max_T);
  const int hq = h * GQ + wv;
  if (tid < NP) tturn[tid] = (a.theta > 0.0 ? pow(a.theta, -2.0 * tid / D) : 0.0) * 0.15915494309189535;
  __syncthreads();
  // this lane's query row (window query i = col, position T - W + i) as A operands: element e = 2 s + hh of
  // the rotated, scaled query for step s; pairs (e, e + 64) sit in one lane
  const int qi = col, qpos = T - a.W + qi;
  const bool qok = qi < a.W && qpos >= 0;
  float qa[64];
  {
    const float sc = 1.4426950408889634f / sqrtf((float)D);  // exp2 domain
    const float* qr = a.q + (((size_t)b * a.W + (qok ? qi : 0)) * a.Hq + hq) * D;
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int e = 2 * s + hh;
      const float x0 = qok ? qr[e] : 0.0f, x1 = qok ? qr[e + NP] : 0.0f;
      float c, sn;
      turn_cs((double)qpos, tturn[e], c, sn);
      qa[s] = (x0 * c - x1 * sn) * sc;
      qa[s + 32] = (x1 * c + x0 * sn) * sc;
    }
  }
  // rows of this lane's accumulator entries: row 8 (v / 4) + 4 hh + v % 4 (window query index)
  float rm[16], rl[16];
  if constexpr (PASS == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      rm[v] = -INFINITY;
      rl[v] = 0.0f;
    }
  } else {
    const float* st = a.ws + a.ws_stats + (((size_t)b * a.Hkv + h) * GQ + wv) * ROWS * 2;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v / 4) + 4 * hh + v % 4;
      rm[v] = st[2 * r];
      rl[v] = st[2 * r + 1] > 0.0f ? 1.0f / st[2 * r + 1] : 0.0f;
    }
  }
  const int nt = n_tiles(a.max_T);
  const int tile0 = split * a.tiles_per_split, tile1 = min(nt, tile0 + a.tiles_per_split);
  const int last_pos = T - 1;  // the window's last query position: no key beyond it is attended
  // raw keys of one tile for this thread (token tid / 8, pairs 8 (tid % 8) .. + 7), loaded one tile ahead so
  // that the loads are in flight while the current tile's products run
  const int tok = tid >> 3, j0 = 8 * (tid & 7);
  f4 rk[4];
  auto load_keys = [&](int t0n) {
    const int t = t0n + tok;
    const bool ok = t < T;
    const float* kr = a.k + (((size_t)b * a.max_T + (ok ? t : 0)) * a.Hkv + h) * D;
    rk[0] = ok ? *(const f4*)(kr + j0) : f4{0, 0, 0, 0};
    rk[1] = ok ? *(const f4*)(kr + j0 + 4) : f4{0, 0, 0, 0};
    rk[2] = ok ? *(const f4*)(kr + j0 + NP) : f4{0, 0, 0, 0};
    rk[3] = ok ? *(const f4*)(kr + j0 + NP + 4) : f4{0, 0, 0, 0};
  };
  if (tile0 < tile1 && tile0 * TILE <= last_pos) load_keys(tile0 * TILE);
  for (int tile = tile0; tile < tile1; ++tile) {
    const int t0 = tile * TILE;
    if (t0 > last_pos) break;  // uniform
    // rotated key tile into LDS
    __syncthreads();  // the previous tile's reads are done
    {
      const int t = t0 + tok;
      float xl[8] = {rk[0][0], rk[0][1], rk[0][2], rk[0][3], rk[1][0], rk[1][1], rk[1][2], rk[1][3]};
      float xh[8] = {rk[2][0], rk[2][1], rk[2][2], rk[2][3], rk[3][0], rk[3][1], rk[3][2], rk[3][3]};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = j0 + u;
        float c, sn;
        turn_cs((double)t, tturn[e], c, sn);
        // element e (parity e % 2, slot e / 2) and e + 64 (same parity, slot e / 2 + 32)
        kt[(e & 1) * TILE * KS + tok * KS + (e >> 1)] = xl[u] * c - xh[u] * sn;
        kt[(e & 1) * TILE * KS + tok * KS + (e >> 1) + 32] = xh[u] * c + xl[u] * sn;
      }
    }
    __syncthreads();
    if (tile + 1 < tile1 && t0 + TILE <= last_pos) load_keys(t0 + TILE);
    // scores: rows = window queries of head hq, columns = the tile's keys; even and odd steps accumulate
    // apart, so that consecutive matrix instructions do not wait for each other's results
    f32x16 acc0 = {}, acc1 = {};
    const float* kb = kt + hh * TILE * KS + col * KS;
#pragma unroll
    for (int s4 = 0; s4 < 16; ++s4) {
      const f4 kv = *(const f4*)(kb + 4 * s4);
      acc0 = sal_mfma(qa[4 * s4], kv[0], acc0);
      acc1 = sal_mfma(qa[4 * s4 + 1], kv[1], acc1);
      acc0 = sal_mfma(qa[4 * s4 + 2], kv[2], acc0);
      acc1 = sal_mfma(qa[4 * s4 + 3], kv[3], acc1);
    }
    const f32x16 acc = acc0 + acc1;
    const int t = t0 + col;
    // every row present attends every key of the tile: the tile ends at or before the first query's position
    const bool full = t0 + TILE - 1 <= T - a.W && a.W <= ROWS;
    if constexpr (PASS == 1) {
      // online (reference maximum, sum of 2^(s - max)) per row; the reference is raised only when a score
      // exceeds it by more than 2^8 (or the first time), so most updates are one exp2 and one add
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v / 4) + 4 * hh + v % 4;
        const int p = T - a.W + r;
        const bool ok = full ? r < a.W : (r < a.W && t <= p);
        const float s = acc[v];
        if (ok) {
          if (s > rm[v] + 8.0f) {
            rl[v] = rl[v] * __builtin_amdgcn_exp2f(rm[v] - s) + 1.0f;  // 2^-inf = 0 the first time
            rm[v] = s;
          } else {
            rl[v] += __builtin_amdgcn_exp2f(s - rm[v]);
          }
        }
      }
    } else {
      float cs = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v / 4) + 4 * hh + v % 4;
        const int p = T - a.W + r;
        const bool ok = full ? r < a.W : (r < a.W && t <= p);
        if (ok) cs += __builtin_amdgcn_exp2f(acc[v] - rm[v]) * rl[v];
      }
      cs += __shfl_xor(cs, 32);  // the other half's 16 rows
      if (hh == 0) colsum[wv][col] = cs;
      __syncthreads();
      if (tid < TILE && t0 + tid < a.max_T)
        a.ws[a.ws_salh + ((size_t)b * a.Hkv + h) * a.max_T + t0 + tid] =
            ((colsum[0][tid] + colsum[1][tid]) + colsum[2][tid]) + colsum[3][tid];
    }
  }
  if constexpr (PASS == 1) {
    // combine each row's (max, sum) over the 32 columns (the lanes of this half), in butterfly order
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float m = rm[v], l = rl[v];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const float m2 = __shfl_xor(m, o), l2 = __shfl_xor(l, o);
        const float mn = fmaxf(m, m2);
        l = (m == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(m - mn)) +
            (m2 == -INFINITY ? 0.0f : l2 * __builtin_amdgcn_exp2f(m2 - mn));
        m = mn;
      }
      if (col == 0) {
        const int r = 8 * (v / 4) + 4 * hh + v % 4;
        float* pt = a.ws + a.ws_part + ((((size_t)b * a.Hkv + h) * a.n_splits + split) * GQ + wv) * ROWS * 2;
        pt[2 * r] = m;
        pt[2 * r + 1] = l;
      }
    }
  }
}

// final (max, sum) per (b, h, head in group, row): the splits combined in split order
__global__ __launch_bounds__(256) void sal_stats_kernel(SalArgs a) {
  using namespace sal;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int n = a.B * a.Hkv * GQ * ROWS;
  if (idx >= n) return;
  const int bh = idx / (GQ * ROWS), rr = idx % (GQ * ROWS);
  float m = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) m = fmaxf(m, a.ws[a.ws_part + (((size_t)bh * a.n_splits + s) * GQ * ROWS + rr) * 2]);
  float l = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float* pt = a.ws + a.ws_part + (((size_t)bh * a.n_splits + s) * GQ * ROWS + rr) * 2;
    if (pt[0] != -INFINITY) l += pt[1] * __builtin_amdgcn_exp2f(pt[0] - m);
  }
  a.ws[a.ws_stats + (size_t)idx * 2] = m;
  a.ws[a.ws_stats + (size_t)idx * 2 + 1] = l;
}

// sal[b][t] = sum over KV heads in order; zero at t >= seq_len
__global__ __launch_bounds__(256) void sal_sum_kernel(SalArgs a, float* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)a.B * a.max_T) return;
  const int b = (int)(idx / a.max_T), t = (int)(idx % a.max_T);
  const int T = min(max(a.seq_len[b], 0), a.max_T);
  float s = 0.0f;
  if (t < T)
    for (int h = 0; h < a.Hkv; ++h) s += a.ws[a.ws_salh + ((size_t)b * a.Hkv + h) * a.max_T + t];
  out[idx] = s;
}

// ---- rank allocation
struct AllocArgs {
  const float* sal;
  const int32_t* seq_len;
  uint8_t* ranks;
  int max_T, m;
  double mean_rank;
  int ladder[8];
  float w[7];
};

constexpr int ALLOC_THREADS = 1024;
constexpr int ALLOC_LDS_TOKENS = 32768;  // saliences staged in LDS up to this length (128 KiB), else read from memory

__global__ __launch_bounds__(ALLOC_THREADS) void rank_alloc_kernel(AllocArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sal_lds[];
  __shared__ long long part[ALLOC_THREADS / 64];
  __shared__ long long total;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = min(max(a.seq_len[b], 0), a.max_T);
  const float* sg = a.sal + (size_t)b * a.max_T;
  const bool staged = T <= ALLOC_LDS_TOKENS;
  if (staged)
    for (int t = tid; t < T; t += ALLOC_THREADS) sal_lds[t] = sg[t];
  __syncthreads();
  const float* s = staged ? sal_lds : sg;
  const long long extra = (long long)floor(a.mean_rank * (double)T) - (long long)a.ladder[0] * T;
  // cost of the steps of gain >= lam
  int cost[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) cost[j] = j < a.m - 1 ? a.ladder[j + 1] - a.ladder[j] : 0;  // 0 past the ladder
  auto count = [&](float lam) -> long long {
    long long c = 0;
    for (int t0 = 0; t0 < T; t0 += ALLOC_THREADS * 64) {  // int32 per thread over at most 64 tokens x 7 x 255
      int ci = 0;
      for (int t = t0 + tid; t < min(T, t0 + ALLOC_THREADS * 64); t += ALLOC_THREADS) {
        const float st = s[t];
#pragma unroll
        for (int j = 0; j < 7; ++j) ci += (st * a.w[j] >= lam) ? cost[j] : 0;
      }
      c += ci;
    }
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
    if (lane == 0) part[wv] = c;
    __syncthreads();
    if (tid == 0) {
      long long z = 0;
      for (int w = 0; w < ALLOC_THREADS / 64; ++w) z += part[w];
      total = z;
    }
    __syncthreads();
    const long long r = total;
    __syncthreads();  // total and part are reused by the next probe
    return r;
  };
  // smallest bit pattern u in [0, +inf] whose set fits (+inf always fits: no finite gain reaches it)
  uint32_t lo = 0u, hi = 0x7F800000u;
  while (lo < hi) {  // uniform: every thread sees the same totals
    const uint32_t mid = lo + (hi - lo) / 2;
    if (count(__builtin_bit_cast(float, mid)) <= extra)
      hi = mid;
    else
      lo = mid + 1;
  }
  const float lam = __builtin_bit_cast(float, hi);
  for (int t = tid; t < a.max_T; t += ALLOC_THREADS) {
    int r = 0;
    if (t < T) {
      const float st = s[t];
      int n = 0;
      for (int j = 0; j < a.m - 1; ++j) n += (st * a.w[j] >= lam);
      r = a.ladder[n];
    }
    a.ranks[(size_t)b * a.max_T + t] = (uint8_t)r;
  }
}

kvc_status hip_fail(hipError_t e);

kvc_status salience_impl(const kvc_salience_in& in, float* out, void* ws, size_t ws_bytes, hipStream_t st,
                         size_t* bytes_out) {
  using namespace sal;
  if (in.B < 1 || in.max_T < 1 || in.W < 1 || in.n_kv_heads < 1 || in.n_q_heads < 1 || in.head_dim < 1 ||
      !(in.rope_theta >= 0.0) || in.n_q_heads % in.n_kv_heads)
    return KVC_ERR_INVALID_ARG;
  if (in.head_dim != D || in.n_q_heads != GQ * in.n_kv_heads || in.W > ROWS) return KVC_ERR_UNSUPPORTED;
  if ((int64_t)in.B * in.max_T * in.n_kv_heads * D >= ((int64_t)1 << 40)) return KVC_ERR_UNSUPPORTED;
  const int ns = splits(in.B, in.n_kv_heads, in.max_T);
  const Ws L = ws_layout(in.B, in.n_kv_heads, in.max_T, ns);
  const size_t need = L.total * sizeof(float);
  if (bytes_out) {
    *bytes_out = need;
    return KVC_OK;
  }
  if (!in.q || !in.k || !in.seq_len || !out || !ws) return KVC_ERR_INVALID_ARG;
  for (const void* p : {(const void*)in.q, (const void*)in.k, (const void*)in.seq_len, (const void*)out, (const void*)ws})
    if ((uintptr_t)p & 15u) return KVC_ERR_MISALIGNED;
  if (ws_bytes < need) return KVC_ERR_WORKSPACE;
  SalArgs a;
  a.q = in.q; a.k = in.k; a.seq_len = in.seq_len; a.ws = (float*)ws;
  a.B = in.B; a.max_T = in.max_T; a.W = in.W; a.Hq = in.n_q_heads; a.Hkv = in.n_kv_heads;
  a.n_splits = ns; a.tiles_per_split = ceil_div(n_tiles(in.max_T), ns); a.theta = in.rope_theta;
  a.ws_part = L.part; a.ws_stats = L.stats; a.ws_salh = L.salh;
  const int grid = in.B * in.n_kv_heads * ns;
  sal_kernel<1><<<grid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  const int n_rows = in.B * in.n_kv_heads * GQ * ROWS;
  sal_stats_kernel<<<ceil_div(n_rows, 256), 256, 0, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  // pass 2 writes every per-head entry below seq_len (tiles reaching past it write zeros there), which is all
  // the final sum reads: no clearing needed
  sal_kernel<2><<<grid, 256, 0, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  const size_t n_out = (size_t)in.B * in.max_T;
  sal_sum_kernel<<<(unsigned)((n_out + 255) / 256), 256, 0, st>>>(a, out);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return KVC_OK;
}

kvc_status rank_alloc_impl(const kvc_alloc_in& in, uint8_t* ranks, hipStream_t st) {
  if (in.B < 1 || in.max_T < 1 || in.n_ladder < 2 || in.n_ladder > 8) return KVC_ERR_INVALID_ARG;
  for (int j = 0; j < in.n_ladder; ++j) {
    if (in.ladder[j] < 1 || in.ladder[j] > 255) return KVC_ERR_INVALID_ARG;
    if (j && in.ladder[j] <= in.ladder[j - 1]) return KVC_ERR_INVALID_ARG;
  }
  for (int j = 0; j < in.n_ladder - 1; ++j) {
    if (!(in.step_w[j] >= 0.0f) || !(in.step_w[j] < INFINITY)) return KVC_ERR_INVALID_ARG;
    if (j && in.step_w[j] > in.step_w[j - 1]) return KVC_ERR_INVALID_ARG;
  }
  if (!(in.mean_rank >= in.ladder[0]) || !(in.mean_rank <= in.ladder[in.n_ladder - 1])) return KVC_ERR_INVALID_ARG;
  if (!in.sal || !in.seq_len || !ranks) return KVC_ERR_INVALID_ARG;
  for (const void* p : {(const void*)in.sal, (const void*)in.seq_len, (const void*)ranks})
    if ((uintptr_t)p & 15u) return KVC_ERR_MISALIGNED;
  AllocArgs a;
  a.sal = in.sal; a.seq_len = in.seq_len; a.ranks = ranks; a.max_T = in.max_T; a.m = in.n_ladder;
  a.mean_rank = in.mean_rank;
  for (int j = 0; j < 8; ++j) a.ladder[j] = j < in.n_ladder ? in.ladder[j] : 0;
  for (int j = 0; j < 7; ++j) a.w[j] = j < in.n_ladder - 1 ? in.step_w[j] : 0.0f;
  const size_t lds = (size_t)std::min(in.max_T, ALLOC_LDS_TOKENS) * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)rank_alloc_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return hip_fail(e);
  rank_alloc_kernel<<<in.B, ALLOC_THREADS, lds, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return KVC_OK;
}

}  // namespace kvc
