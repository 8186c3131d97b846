// dense.hip -- plain softmax decode attention over a paged bf16 cache (gfx950): the dense comparison.
//
// Same decomposition as the compressed kernel: one workgroup (4 waves) per (sequence, kv head,
// context split), 32-token super-tiles, per-wave online softmax, the four waves combined in LDS at the
// end, and a merge kernel over the splits.  A super-tile's keys (and values) of one head are 32 rows of
// D bf16, contiguous within a page, so each wave reads them with 16-byte nontemporal loads in which the 64
// lanes cover 1 KB of consecutive bytes (one full run of cache lines per instruction: the read pattern
// the stream probe sustains); it stores them to its own LDS tile (rows padded by 16 bytes, so that the
// column-wise reads below hit distinct banks) and reads them back in the matrix instructions' operand
// layout.  The loads run one super-tile ahead of the one computed.  Scores S^T = K Q^T on the bf16 MFMA
// (k-slot 8g + j of chunk c <-> dim 32c + 8g + j); values go through a one-hot bf16 MFMA (a register
// transpose, exact) and the value product runs on the fp16 MFMA with fp16 probabilities; value tile nt
// holds dims 16 nt .. 16 nt + 15.
#include <math.h>

#include <algorithm>

#include "lds_copy.hpp"

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

namespace kvc {

struct DenseArgs {
  const int32_t* block_table;
  const int32_t* seq_len;
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const void* q;
  float* ws;
  int q_bf16, B, Hkv, Hq, max_blocks, P, n_splits, st_per_split, part_stride;
};

static constexpr int DGQ = 4;

__device__ inline f4 mfma_bf16(bf8 a, bf8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

template <int D>
__global__ __launch_bounds__(256, 2) void dense_kernel(DenseArgs a) {
  constexpr int QC = D / 32;  // chunks of the score product
  constexpr int NT = D / 16;  // N-tiles of the value product
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x % a.n_splits;
  const int h = (blockIdx.x / a.n_splits) % a.Hkv;
  const int b = blockIdx.x / (a.n_splits * a.Hkv);
  const int T = a.seq_len[b];
  const int P = a.P;

  // Q^T as the B operand: column hq = n (rows >= DGQ zero), k-slot 8g + j of chunk c <-> dim 32c + 8g + j
  // (eight consecutive dims per lane and chunk: one 16-byte load of a bf16 query, two of an fp32 one)
  bf8 qop[QC];
  {
    const size_t qrow = ((size_t)b * a.Hq + h * DGQ + min(n, DGQ - 1)) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      bf8 x;
      if (a.q_bf16) {
        x = *(const bf8*)((const uint16_t*)a.q + qrow + 32 * c);
      } else {
        const f4 lo = *(const f4*)((const float*)a.q + qrow + 32 * c);
        const f4 hi = *(const f4*)((const float*)a.q + qrow + 32 * c + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = (__bf16)lo[j];
          x[4 + j] = (__bf16)hi[j];
        }
      }
      qop[c] = n < DGQ ? x : bf8{};
    }
  }
  bf8 oh[2];
  for (int e = 0; e < 2; ++e)
    for (int j = 0; j < 8; ++j) oh[e][j] = (__bf16)((8 * g + j == 16 * e + n) ? 1.0f : 0.0f);
  const float qscale = 1.4426950408889634f / sqrtf((float)D);

  f4 acc[NT];
  for (int i = 0; i < NT; ++i) acc[i] = f4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;
  const int n_st = (T + 31) / 32;
  const int st_begin = split * a.st_per_split;
  const int st_end = min(n_st, st_begin + a.st_per_split);
  // Keys and values of super-tile st as whole rows: load instruction i, lane l holds the 16 bytes at
  // 16 (64 i + l) of the tile, i.e. piece l % PC of row LR i + l / PC.  Rows past the sequence end read
  // the last token's row instead (real, finite data; their scores are masked, so they get probability 0).
  constexpr int RB = 2 * D;           // bytes per row
  constexpr int PC = RB / 16;         // 16-byte pieces per row
  constexpr int LR = 64 / PC;         // rows per load instruction
  constexpr int NI = 32 / LR;         // load instructions per super-tile and tensor
  constexpr int RS = RB + 16;         // LDS row stride
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4][2][32 * RS];
  uint8_t* ktile = tiles[wv][0];
  uint8_t* vtile = tiles[wv][1];
  auto load = [&](int st, u4v (&kr)[NI], u4v (&vr)[NI]) {
    const int t0 = st * 32;
    const int page = uniform(a.block_table[(size_t)b * a.max_blocks + t0 / P]);
    const size_t head_base = ((size_t)page * a.Hkv + h) * P + (t0 % P);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = min(LR * i + lane / PC, T - 1 - t0);
      const size_t off = (head_base + r) * D + 8 * (lane % PC);
      kr[i] = __builtin_nontemporal_load((const u4v*)(a.k_pages + off));
      vr[i] = __builtin_nontemporal_load((const u4v*)(a.v_pages + off));
    }
  };
  auto stage = [&](const u4v (&kr)[NI], const u4v (&vr)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int o = (LR * i + lane / PC) * RS + 16 * (lane % PC);
      *(u4v*)(ktile + o) = kr[i];
      *(u4v*)(vtile + o) = vr[i];
    }
  };
  // the operands of super-tile st from the tiles: lane (n, g) takes row 16 blk + n, dims 32 c + 8 g .. + 7
  auto operands = [&](bf8 (&kc)[2][QC], bf8 (&vc)[2][QC]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const int o = (16 * blk + n) * RS + 16 * (4 * c + g);
        kc[blk][c] = *(const bf8*)(ktile + o);
        vc[blk][c] = *(const bf8*)(vtile + o);
      }
  };
  // one super-tile: scores, online softmax, value product
  auto tile = [&](int st, const bf8 (&kcur)[2][QC], const bf8 (&vcur)[2][QC]) {
    const int t0 = st * 32;
    float sc[2][4];
    h4 vtb[NT][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const bf8* kc = kcur[blk];
      const bf8* vc = vcur[blk];
      f4 s4 = {0, 0, 0, 0};
      for (int c = 0; c < QC; ++c) s4 = mfma_bf16(kc[c], qop[c], s4);
      for (int i = 0; i < 4; ++i) sc[blk][i] = s4[i] * qscale;
      // transpose: chunk c, half e -> column n holds dim 32c + 16e + n of tokens 4g..4g+3
      for (int c = 0; c < QC; ++c)
        for (int e = 0; e < 2; ++e) {
          const f4 tr = mfma_bf16(vc[c], oh[e], f4{0, 0, 0, 0});
          vtb[2 * c + e][blk] = h4{(_Float16)tr[0], (_Float16)tr[1], (_Float16)tr[2], (_Float16)tr[3]};
        }
    }
    float mx = -INFINITY;
    for (int blk = 0; blk < 2; ++blk)
      for (int i = 0; i < 4; ++i) {
        const bool ok = (n < DGQ) && (t0 + 16 * blk + 4 * g + i < T);
        sc[blk][i] = ok ? sc[blk][i] : -INFINITY;
        mx = fmaxf(mx, sc[blk][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
    h8 pop;
    float psum = 0.0f;
    for (int blk = 0; blk < 2; ++blk)
      for (int i = 0; i < 4; ++i) {
        const float p = (m_new == -INFINITY) ? 0.0f : exp2f(sc[blk][i] - m_new);
        const _Float16 ph = (_Float16)p;
        pop[4 * blk + i] = ph;
        psum += (float)ph;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
      float al[4];
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
      for (int nt = 0; nt < NT; ++nt)
        for (int i = 0; i < 4; ++i) acc[nt][i] *= al[i];
    }
    for (int nt = 0; nt < NT; ++nt) {
      const h8 vt = {vtb[nt][0][0], vtb[nt][0][1], vtb[nt][0][2], vtb[nt][0][3],
                     vtb[nt][1][0], vtb[nt][1][1], vtb[nt][1][2], vtb[nt][1][3]};
      acc[nt] = mfma16x16x32(pop, vt, acc[nt]);
    }
  };
  u4v kn[NI], vn[NI];
  if (st_begin + wv < st_end) load(st_begin + wv, kn, vn);
  for (int st = st_begin + wv; st < st_end; st += 4) {
    stage(kn, vn);
    if (st + 4 < st_end) load(st + 4, kn, vn);
    wave_lds_sync();
    bf8 kcur[2][QC], vcur[2][QC];
    operands(kcur, vcur);
    tile(st, kcur, vcur);
    wave_lds_sync();  // the tile's reads are done before the next super-tile is staged over it
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // the four waves' (m, l, acc) combined in LDS into the split's partial
  __shared__ float red[4][2 * DGQ + DGQ * D];
  float* mine = red[wv];
  if (lane < DGQ) {
    mine[lane] = m_run;
    mine[DGQ + lane] = l_run;
  }
  for (int nt = 0; nt < NT; ++nt) {
    const int dim = 16 * nt + n;
    for (int i = 0; i < 4; ++i) {
      const int hq = 4 * g + i;
      if (hq < DGQ) mine[2 * DGQ + hq * D + dim] = acc[nt][i];
    }
  }
  __syncthreads();
  float* part = a.ws + (size_t)((b * a.Hkv + h) * a.n_splits + split) * a.part_stride;
  for (int e = tid; e < DGQ * D; e += 256) {
    const int hq = e / D;
    float mx = -INFINITY;
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, red[w][hq]);
    float av = 0.0f, lv = 0.0f;
    for (int w = 0; w < 4; ++w) {
      const float wt = red[w][hq] == -INFINITY ? 0.0f : exp2f(red[w][hq] - mx);
      av += wt * red[w][2 * DGQ + e];
      lv += wt * red[w][DGQ + hq];
    }
    part[2 * DGQ + e] = av;
    if (e % D == 0) {
      part[hq] = mx;
      part[DGQ + hq] = lv;
    }
  }
}

// One workgroup per (sequence, query head); thread d combines output dim d over the splits.
template <int D>
__global__ __launch_bounds__(D) void dense_merge_kernel(const float* ws, float* out, int Hkv, int Hq, int n_parts,
                                                        int part_stride) {
  const int bq = blockIdx.x, hq_all = bq % Hq, b = bq / Hq;
  const int h = hq_all / DGQ, hq = hq_all % DGQ, d = threadIdx.x;
  const float* parts = ws + (size_t)(b * Hkv + h) * n_parts * part_stride;
  float m = -INFINITY;
  for (int p = 0; p < n_parts; ++p) m = fmaxf(m, parts[(size_t)p * part_stride + hq]);
  float lsum = 0.0f, o = 0.0f;
#pragma unroll 8
  for (int p = 0; p < n_parts; ++p) {
    const float* pp = parts + (size_t)p * part_stride;
    const float mp = pp[hq];
    const float wgt = mp == -INFINITY ? 0.0f : exp2f(mp - m);
    lsum += wgt * pp[DGQ + hq];
    o += wgt * pp[2 * DGQ + hq * D + d];
  }
  out[((size_t)b * Hq + hq_all) * D + d] = o / lsum;
}

static void dense_splits(int B, int Hkv, int max_T, int requested, int* ns, int* sps) {
  const int n_st = (max_T + 31) / 32;
  int s = requested;
  if (s <= 0) {
    s = std::max(1, (1024 + B * Hkv - 1) / (B * Hkv));
    s = std::min(s, std::max(1, n_st / 4));
  }
  s = std::max(1, std::min(s, n_st));
  *sps = (n_st + s - 1) / s;
  *ns = (n_st + *sps - 1) / *sps;
}

kvc_status dense_impl(const kvc_dense_in& in, float* out, void* ws, size_t ws_bytes, hipStream_t st, size_t* need) {
  if (in.n_q_heads <= 0 || in.n_kv_heads <= 0 || in.B <= 0 || in.max_T <= 0 || in.max_blocks <= 0 ||
      in.page_size <= 0 || in.num_splits < 0)
    return KVC_ERR_INVALID_ARG;
  if (in.n_q_heads % in.n_kv_heads || (int64_t)in.max_blocks * in.page_size < in.max_T) return KVC_ERR_INVALID_ARG;
  if (in.q_dtype != KVC_F32 && in.q_dtype != KVC_BF16) return KVC_ERR_INVALID_ARG;
  if (in.n_q_heads != DGQ * in.n_kv_heads || (in.head_dim != 64 && in.head_dim != 128) || in.page_size % 32 ||
      in.page_size > 256)
    return KVC_ERR_UNSUPPORTED;
  int ns, sps;
  dense_splits(in.B, in.n_kv_heads, in.max_T, in.num_splits, &ns, &sps);
  const int stride = 2 * DGQ + DGQ * in.head_dim;
  const size_t bytes = (size_t)in.B * in.n_kv_heads * ns * stride * sizeof(float);
  if (need) {
    *need = bytes;
    return KVC_OK;
  }
  if (!in.block_table || !in.seq_len || !in.k_pages || !in.v_pages || !in.q || !out || !ws)
    return KVC_ERR_INVALID_ARG;
  const void* ptrs[] = {in.block_table, in.seq_len, in.k_pages, in.v_pages, in.q, out, ws};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15u) return KVC_ERR_MISALIGNED;
  if (ws_bytes < bytes) return KVC_ERR_WORKSPACE;
  DenseArgs a;
  a.block_table = in.block_table; a.seq_len = in.seq_len; a.k_pages = in.k_pages; a.v_pages = in.v_pages;
  a.q = in.q; a.ws = (float*)ws; a.q_bf16 = in.q_dtype == KVC_BF16; a.B = in.B; a.Hkv = in.n_kv_heads;
  a.Hq = in.n_q_heads; a.max_blocks = in.max_blocks; a.P = in.page_size; a.n_splits = ns; a.st_per_split = sps;
  a.part_stride = stride;
  const int grid = in.B * in.n_kv_heads * ns;
  if (in.head_dim == 128) {
    hipLaunchKernelGGL(dense_kernel<128>, dim3(grid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(dense_kernel<64>, dim3(grid), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  if (in.head_dim == 128) {
    hipLaunchKernelGGL(dense_merge_kernel<128>, dim3(in.B * in.n_q_heads), dim3(128), 0, st, a.ws, out,
                       in.n_kv_heads, in.n_q_heads, ns, stride);
  } else {
    hipLaunchKernelGGL(dense_merge_kernel<64>, dim3(in.B * in.n_q_heads), dim3(64), 0, st, a.ws, out,
                       in.n_kv_heads, in.n_q_heads, ns, stride);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return KVC_OK;
}

}  // namespace kvc
