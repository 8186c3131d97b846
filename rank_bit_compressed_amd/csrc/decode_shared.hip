// decode_shared.hip -- decode attention over a block-shared latent (gfx950).
//
// One INT4 latent c_t (dim 512, groups of 64) per token serves n_layers layers and all KV heads:
// layer l, KV head h rebuilds k = W_k[l][:, h d : (h+1) d]^T c_t (v likewise through W_v), and the
// keys are rotated (RoPE) after that up-projection.
//
// One workgroup (4 waves) per (layer, kv head, sequence, context split).  The layer/head slice of
// W_k (512 x 128) sits in LDS as fp16 MFMA A fragments (128 KB).  The waves walk the same 32-token
// super-tiles together: wave w computes head dims {16w..16w+15} and {64+16w..64+16w+15} (so its RoPE
// pairs are lane-local), its partial scores over those 32 dims go through LDS and are summed by
// every wave, and wave w accumulates the value latent on coordinates 128w..128w+127.  The value
// up-projection W_v is applied once per (layer, sequence, head) in the merge kernel.
#include <math.h>

#include <algorithm>

#include "kvc_common.hpp"

namespace kvc {

static constexpr int SGQ = 4;     // query heads per KV head
static constexpr int SLAT = 512;  // latent dimension handled here
static constexpr int SD = 128;    // head dimension handled here

struct DecodeSharedArgs {
  const uint8_t* pool;
  const int64_t* page_off;
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* q_pos;
  const void* q;
  const uint16_t* wk;
  float* ws;
  int q_bf16, B, Hkv, Hq, L, max_blocks, P, G, n_splits, st_per_split, part_stride;
  double theta;
};

struct SharedLds {
  int wfrag, rope, qbuf, sp, total;
};
__host__ __device__ inline SharedLds shared_lds() {
  SharedLds L;
  int o = 0;
  L.wfrag = o; o += (SD / 16) * (SLAT / 32) * 64 * 16;   // 128 KB
  L.rope = o; o += 32 * (SD / 2) * 4;                    // 8 KB
  L.qbuf = o; o += SGQ * (SD / 2 + 4) * 4;               // query rows (pairs), padded
  L.sp = o; o += 2 * 4 * 2 * 64 * 16;                    // partial scores [buf][wave][block][lane] f4
  L.total = o;
  return L;
}

__global__ __launch_bounds__(256) void decode_shared_kernel(DecodeSharedArgs a) {
  constexpr int NP = SD / 2;
  constexpr int KCH = SLAT / 32;  // 16 chunks of the up-projection
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const SharedLds LY = shared_lds();
  h8* wfrag = (h8*)(smem + LY.wfrag);
  uint32_t* rope_tab = (uint32_t*)(smem + LY.rope);
  uint32_t(*qbuf)[NP + 4] = (uint32_t(*)[NP + 4])(smem + LY.qbuf);
  f4* sp = (f4*)(smem + LY.sp);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int id = blockIdx.x;
  const int split = id % a.n_splits; id /= a.n_splits;
  const int b = id % a.B; id /= a.B;
  const int h = id % a.Hkv;
  const int l = id / a.Hkv;
  const int T = a.seq_len[b];
  const int qpos = a.q_pos ? a.q_pos[b] : T;
  const int P = a.P;

  // W_k[l][:, h*128 + dim] as A fragments [m][c][lane]: row dim = 16m + n, k-slot 8g + j <-> latent
  // coordinate 32c + 8g + perm8(j)
  {
    const uint16_t* W = a.wk + (size_t)l * SLAT * a.Hkv * SD + (size_t)h * SD;
    const int width = a.Hkv * SD;
    for (int e = tid; e < (SD / 16) * KCH * 64; e += 256) {
      const int m = e / (KCH * 64), c = (e / 64) % KCH, ln = e % 64;
      h8 f;
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * c + 8 * (ln >> 4) + perm8(j);
        f[j] = bf16_to_h(W[(size_t)i * width + 16 * m + (ln & 15)]);
      }
      wfrag[e] = f;
    }
  }
  for (int e = tid; e < 32 * NP; e += 256) {  // in-tile RoPE factors, [c][s][g][i] for pair j = 16c + 4g + i
    const int s = e / NP, j = e % NP;
    const double th = a.theta > 0.0 ? pow(a.theta, -2.0 * j / SD) : 0.0;
    float sn, cs;
    sincosf((float)(s * th), &sn, &cs);
    rope_tab[(((j >> 4) * 32 + s) * 4 + ((j >> 2) & 3)) * 4 + (j & 3)] = pack_h2(cs, sn);
  }
  // query pairs of this wave's 16 frequencies (j = 16w + lane, lanes < 16), scaled for exp2
  float qa[SGQ], qb[SGQ];
  double fj = 0.0;
  {
    const int j = 16 * wv + (lane & 15);
    const float sc = 1.4426950408889634f / sqrtf((float)SD);
    for (int hq = 0; hq < SGQ; ++hq) {
      const size_t base = (((size_t)l * a.B + b) * a.Hq + h * SGQ + hq) * SD;
      float x0, x1;
      if (a.q_bf16) {
        const uint16_t* q = (const uint16_t*)a.q + base;
        x0 = __builtin_bit_cast(float, (uint32_t)q[j] << 16);
        x1 = __builtin_bit_cast(float, (uint32_t)q[j + NP] << 16);
      } else {
        const float* q = (const float*)a.q + base;
        x0 = q[j];
        x1 = q[j + NP];
      }
      qa[hq] = x0 * sc;
      qb[hq] = x1 * sc;
    }
    if (a.theta > 0.0) fj = pow(a.theta, -2.0 * j / SD) * 0.15915494309189535;
  }
  h8 oh[2];
  for (int e = 0; e < 2; ++e)
    for (int j = 0; j < 8; ++j) oh[e][j] = (8 * g + perm8(j) == 16 * e + n) ? (_Float16)1.0f : (_Float16)0.0f;
  __syncthreads();

  f4 acc[8];  // value latent coordinates 128w + 16 nt + n, rows = query heads
  for (int i = 0; i < 8; ++i) acc[i] = f4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;
  const int64_t meta_base = pad16((int64_t)P * SLAT / 2);
  const int mpt = 4 * (SLAT / a.G);  // pair bytes per token

  const int n_st = (T + 31) / 32;
  const int st_begin = split * a.st_per_split;
  const int st_end = min(n_st, st_begin + a.st_per_split);
  int buf = 0;
  for (int st = st_begin; st < st_end; ++st, buf ^= 1) {
    const int t0 = st * 32;
    const int page = uniform(a.block_table[(size_t)b * a.max_blocks + t0 / P]);
    const uint8_t* rec = a.pool + uniform64(a.page_off[page]);
    const int slot0 = t0 % P;
    if (lane < 16) {  // this wave's query pairs rotated by the super-tile base
      double rev = (double)(qpos - t0) * fj;
      rev -= rint(rev);
      const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
      const int j = 16 * wv + lane;
      for (int hq = 0; hq < SGQ; ++hq)
        qbuf[hq][j] = pack_h2(qa[hq] * cs - qb[hq] * sn, qb[hq] * cs + qa[hq] * sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

    // ---- key up-projection of this wave's 32 head dims for both blocks, streaming latent chunks
    f4 kp[2][2];  // [m-tile w | w+4][block]
    h8 vkeep[4][2];
    for (int i = 0; i < 2; ++i)
      for (int k = 0; k < 2; ++k) kp[i][k] = f4{0, 0, 0, 0};
    for (int c = 0; c < KCH; ++c) {
      const h8 A0 = wfrag[(wv * KCH + c) * 64 + lane];
      const h8 A1 = wfrag[((wv + 4) * KCH + c) * 64 + lane];
      for (int blk = 0; blk < 2; ++blk) {
        const int slot = slot0 + 16 * blk + n;
        const bool valid = t0 + 16 * blk + n < T;
        const uint32_t x = valid ? *(const uint32_t*)(rec + (int64_t)slot * (SLAT / 2) + 4 * (4 * c + g)) : 0u;
        const uint32_t sz = valid ? *(const uint32_t*)(rec + meta_base + (int64_t)slot * mpt + 4 * ((32 * c) / a.G)) : 0u;
        const h8 kb = dequant_int4x8(x, sz);
        kp[0][blk] = mfma16x16x32(A0, kb, kp[0][blk]);
        kp[1][blk] = mfma16x16x32(A1, kb, kp[1][blk]);
        if ((c >> 2) == wv) vkeep[c & 3][blk] = kb;
      }
    }

    // ---- RoPE, partial scores over the wave's dims, V transposes
    h4 vtb[8][2];
    for (int blk = 0; blk < 2; ++blk) {
      const int tt = 16 * blk + n;
      const u4 f4v = *(const u4*)&rope_tab[((wv * 32 + tt) * 4 + g) * 4];
      h8 kq;
      for (int i = 0; i < 4; ++i) {
        const h2 r = as_h2(rope_pair(pack_h2(kp[0][blk][i], kp[1][blk][i]), f4v[i]));
        kq[2 * i] = r.x;
        kq[2 * i + 1] = r.y;
      }
      const f4 s4 = mfma16x16x32(kq, *(const h8*)&qbuf[n & (SGQ - 1)][16 * wv + 4 * g], f4{0, 0, 0, 0});
      sp[((buf * 4 + wv) * 2 + blk) * 64 + lane] = s4;
      for (int cc = 0; cc < 4; ++cc)
        for (int e = 0; e < 2; ++e) {
          const f4 tr = mfma16x16x32(vkeep[cc][blk], oh[e], f4{0, 0, 0, 0});
          vtb[2 * cc + e][blk] = h4{(_Float16)tr[0], (_Float16)tr[1], (_Float16)tr[2], (_Float16)tr[3]};
        }
    }
    __syncthreads();  // partial scores of all waves visible (the buffer alternates between super-tiles)

    float sc[2][4];
    for (int blk = 0; blk < 2; ++blk) {
      f4 s = sp[((buf * 4 + 0) * 2 + blk) * 64 + lane];
      for (int w2 = 1; w2 < 4; ++w2) s += sp[((buf * 4 + w2) * 2 + blk) * 64 + lane];
      for (int i = 0; i < 4; ++i) sc[blk][i] = s[i];
    }
    if (t0 + 32 > T)
      for (int blk = 0; blk < 2; ++blk)
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * blk + 4 * g + i >= T) sc[blk][i] = -INFINITY;
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    h8 pop;
    float psum = 0.0f;
    for (int blk = 0; blk < 2; ++blk)
      for (int i = 0; i < 4; ++i) {
        const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(sc[blk][i] - m_new);
        pop[4 * blk + i] = ph;
        psum += (float)ph;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
      float al[4];
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
      for (int nt = 0; nt < 8; ++nt)
        for (int i = 0; i < 4; ++i) acc[nt][i] *= al[i];
    }
    for (int nt = 0; nt < 8; ++nt) {
      const h8 vt = {vtb[nt][0][0], vtb[nt][0][1], vtb[nt][0][2], vtb[nt][0][3],
                     vtb[nt][1][0], vtb[nt][1][1], vtb[nt][1][2], vtb[nt][1][3]};
      acc[nt] = mfma16x16x32(pop, vt, acc[nt]);
    }
  }

  // ---- partial: m[4], l[4] (the same in every wave), acc[4][512] (wave w: coordinates 128w..)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* part = a.ws + ((((size_t)l * a.Hkv + h) * a.B + b) * a.n_splits + split) * a.part_stride;
  if (wv == 0 && lane < SGQ) {
    part[lane] = m_run;
    part[SGQ + lane] = l_run;
  }
  for (int nt = 0; nt < 8; ++nt)
    for (int i = 0; i < 4; ++i) {
      const int hq = 4 * g + i;
      const int coord = 128 * wv + 32 * (nt >> 1) + 16 * (nt & 1) + n;
      if (hq < SGQ) part[2 * SGQ + hq * SLAT + coord] = acc[nt][i];
    }
}

// out[l][b][h*4 + hq] = W_v[l][:, h*128 : (h+1)*128]^T c* / l*, over the splits' partials.
__global__ __launch_bounds__(256) void merge_shared_kernel(const float* ws, const uint16_t* wv, float* out, int B,
                                                           int Hkv, int Hq, int n_splits, int part_stride) {
  __shared__ float cst[SGQ][SLAT];
  __shared__ float lst[SGQ];
  int id = blockIdx.x;
  const int b = id % B; id /= B;
  const int h = id % Hkv;
  const int l = id / Hkv;
  const int tid = threadIdx.x, hq = tid / 64, t64 = tid % 64;
  const float* parts = ws + (((size_t)l * Hkv + h) * B + b) * n_splits * part_stride;
  float m = -INFINITY;
  for (int p = 0; p < n_splits; ++p) m = fmaxf(m, parts[(size_t)p * part_stride + hq]);
  float lsum = 0.0f, c[SLAT / 64];
  for (int k = 0; k < SLAT / 64; ++k) c[k] = 0.0f;
  for (int p = 0; p < n_splits; ++p) {
    const float* pp = parts + (size_t)p * part_stride;
    if (pp[hq] == -INFINITY) continue;
    const float w = exp2f(pp[hq] - m);
    lsum += w * pp[SGQ + hq];
    for (int k = 0; k < SLAT / 64; ++k) c[k] += w * pp[2 * SGQ + hq * SLAT + t64 + 64 * k];
  }
  for (int k = 0; k < SLAT / 64; ++k) cst[hq][t64 + 64 * k] = c[k];
  if (t64 == 0) lst[hq] = lsum;
  __syncthreads();
  const uint16_t* W = wv + (size_t)l * SLAT * Hkv * SD + (size_t)h * SD;
  const float inv = 1.0f / lst[hq];
  for (int d = t64; d < SD; d += 64) {
    float o = 0.0f;
    for (int i = 0; i < SLAT; ++i) o += __builtin_bit_cast(float, (uint32_t)W[(size_t)i * Hkv * SD + d] << 16) * cst[hq][i];
    out[(((size_t)l * B + b) * Hq + h * SGQ + hq) * SD + d] = o * inv;
  }
}

bool shared_supported(const kvc_layout& L) {
  return L.shared && L.head_dim == SD && L.r_k_cap == SLAT && L.n_q_heads == SGQ * L.n_kv_heads &&
         L.latent_bits == 4 && L.group % 32 == 0 && L.group <= SLAT && SLAT % L.group == 0;
}

size_t shared_ws_bytes(const kvc_layout& L, int B, int n_splits) {
  return (size_t)L.n_layers * L.n_kv_heads * B * n_splits * (2 * SGQ + SGQ * SLAT) * sizeof(float);
}

hipError_t launch_decode_shared(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out,
                                void* ws, int n_splits, int st_per_split, hipStream_t st) {
  DecodeSharedArgs a;
  a.pool = C.pool; a.page_off = C.page_off; a.block_table = in.block_table; a.seq_len = in.seq_len;
  a.q_pos = in.q_pos; a.q = in.q; a.wk = in.wk; a.ws = (float*)ws; a.q_bf16 = in.q_dtype == KVC_BF16;
  a.B = in.B; a.Hkv = L.n_kv_heads; a.Hq = L.n_q_heads; a.L = L.n_layers; a.max_blocks = in.max_blocks;
  a.P = L.page_size; a.G = L.group; a.n_splits = n_splits; a.st_per_split = st_per_split;
  a.part_stride = 2 * SGQ + SGQ * SLAT; a.theta = L.rope_theta;
  const int lds = shared_lds().total;
  hipError_t e = hipFuncSetAttribute((const void*)decode_shared_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = L.n_layers * L.n_kv_heads * in.B * n_splits;
  e = mark(g_marks.begin, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_shared_kernel, dim3(grid), dim3(256), lds, st, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(g_marks.end, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_shared_kernel, dim3(L.n_layers * L.n_kv_heads * in.B), dim3(256), 0, st, a.ws, in.wv, out,
                     in.B, L.n_kv_heads, L.n_q_heads, n_splits, a.part_stride);
  return hipGetLastError();
}

}  // namespace kvc
