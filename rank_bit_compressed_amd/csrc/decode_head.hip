// decode_head.hip -- one decode step of attention over a per-KV-head compressed cache (gfx950).
//
// Work decomposition: one workgroup (4 waves) per (sequence b, KV head h, context split); a split
// is a run of consecutive pages.  The workgroup streams its pages' head-h blocks (one contiguous
// byte range per page: codes, scale/zero pairs [, residual]) from HBM into LDS with 16-byte loads,
// double-buffered: the loads of page i+1 are in flight while the waves decode page i from LDS.
// Page addresses of the whole split are resolved once, at the start, into LDS.  Inside a page,
// wave w takes the 32-token super-tiles w, w+4, ...; each wave keeps its own online-softmax state
// and writes one partial (max, sum, latent accumulator) per query head; the merge kernel combines
// the partials and applies the value basis.
//
// Per 16-token block (lane l: token l%16, group g = l/16):
//   K latent codes -> fp16 in registers -> MFMA K_pre = B_k c (basis fragments held in registers;
//   rows = head dims, columns = tokens) [+ rotated residual: MFMA with the +-1 Hadamard] ->
//   RoPE in registers (pairs (j, j+d/2) sit in one lane) -> MFMA scores S^T = K~^T Q~^T, whose
//   output layout is already the A operand of the value product.
//   V latent codes -> fp16 -> MFMA with a one-hot matrix (a register transpose: tokens move from
//   lanes into the reduction slots) -> MFMA acc += P V_latent, in the latent space: the value basis
//   is applied once per (b, head) in the merge (sum_t p_t B c_t = B sum_t p_t c_t).
// RoPE is split as R(t0 + s) = R(t0) R(s): R(s), s < 32, comes from an LDS table built once per
// workgroup; R(t0) is applied to the query once per super-tile (q~ = R(q_pos - t0) q).
#include <math.h>

#include "kvc_common.hpp"

namespace kvc {

struct DecodeHeadArgs {
  const uint8_t* pool;
  const int64_t* page_off;
  const uint32_t* tok_off;
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* q_pos;
  const void* q;
  const uint16_t* wk;
  float* ws;
  int q_bf16;
  int B, Hkv, Hq, max_blocks, P, rk, rv, G, n_splits, pages_per_split, part_stride;
  int hb_max;      // bytes of the largest head block (rank cap)
  double theta;
  HeadSections S_uniform;
};

static constexpr int GQ = 4;            // query heads per KV head handled by these kernels
static constexpr int MAX_SPLIT_PAGES = 128;

// LDS layout (bytes) of the decode kernel, given the head-block buffer size.
struct HeadLds {
  int rope, qbuf, theta, meta_addr, meta_hb, meta_page, hfrag, bfrag, stage, stage_bytes, total;
};
__host__ __device__ inline HeadLds head_lds(int D, int KC, int P, bool res, int hb_max) {
  HeadLds L;
  int o = 0;
  L.bfrag = o; o += (D / 16) * KC * 64 * 16;
  L.rope = o; o += 32 * (D / 2) * 4;
  L.qbuf = o; o += 4 * GQ * (D / 2 + 4) * 4;  // rows padded by 4 dwords: distinct banks per row
  L.theta = o; o += (D / 2) * 8;
  L.meta_addr = o; o += MAX_SPLIT_PAGES * 8;
  L.meta_hb = o; o += MAX_SPLIT_PAGES * 4;
  L.meta_page = o; o += MAX_SPLIT_PAGES * 4;
  L.hfrag = o; o += res ? (D / 16) * 4 * 64 * 16 : 0;
  L.stage_bytes = (int)pad16(hb_max) + (int)pad16(4 * (P + 1));  // head block + offset row
  L.stage = o; o += 2 * L.stage_bytes;
  L.total = o;
  return L;
}

template <int D, int KC, int VC, int KB, int VB, bool RES, bool VAR, int STG>
__global__ __launch_bounds__(256) void decode_head_kernel(DecodeHeadArgs a) {
  // KB, VB: latent bits of keys and values (2, 3, 4; 32 = fp32 latents for both)
  constexpr bool LAT32 = KB == 32;
  static_assert(LAT32 == (VB == 32), "fp32 latents for both or neither");
  constexpr int MT = D / 16;   // M-tiles of the up-projection (16 head dims each)
  constexpr int QC = D / 32;   // K-chunks of the score product
  constexpr int NP = D / 2;    // RoPE pairs
  constexpr int NV = 2 * VC;   // N-tiles of the value product (16 latent dims each)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int P = a.P;
  const HeadLds LY = head_lds(D, KC, P, RES, a.hb_max);
  // in-tile RoPE factors, [c][s][g][i] for pair j = 16c + 4g + i: a lane's four factors are 16
  // contiguous bytes and the 64 lanes of a wave read one contiguous kilobyte (no bank conflicts)
  uint32_t* rope_tab = (uint32_t*)(smem + LY.rope);
  uint32_t(*qbuf)[GQ][NP + 4] = (uint32_t(*)[GQ][NP + 4])(smem + LY.qbuf);
  double* thetas = (double*)(smem + LY.theta);
  int64_t* meta_addr = (int64_t*)(smem + LY.meta_addr);
  int32_t* meta_hb = (int32_t*)(smem + LY.meta_hb);
  int32_t* meta_page = (int32_t*)(smem + LY.meta_page);
  h8* hfrag = (h8*)(smem + LY.hfrag);
  h8* bfrag = (h8*)(smem + LY.bfrag);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x % a.n_splits;
  const int h = (blockIdx.x / a.n_splits) % a.Hkv;
  const int b = blockIdx.x / (a.n_splits * a.Hkv);
  const int T = a.seq_len[b];
  const int qpos = a.q_pos ? a.q_pos[b] : T;
  const int lb0 = split * a.pages_per_split;
  const int n_pages = max(0, min((T + P - 1) / P, lb0 + a.pages_per_split) - lb0);

  // ---- set-up: frequencies, in-tile RoPE table, query buffer, page addresses of the split
  if (tid < NP) thetas[tid] = a.theta > 0.0 ? pow(a.theta, -2.0 * tid / D) : 0.0;
  for (int i = tid; i < n_pages; i += 256) {
    const int page = a.block_table[(size_t)b * a.max_blocks + lb0 + i];
    int64_t hb = a.S_uniform.hb;
    if constexpr (VAR) {
      const uint32_t tot = a.tok_off[(size_t)page * (P + 1) + P];
      const int64_t cb = (int64_t)(tot & 0xFFFFu) * KB / 8, mb = 4 * (int64_t)(tot >> 16);  // variable rank: KB == VB
      hb = head_sections(cb, cb, mb, mb, P, D, RES).hb;
    }
    meta_addr[i] = a.page_off[page] + (int64_t)h * hb;
    meta_hb[i] = (int32_t)hb;
    meta_page[i] = page;
  }
  if constexpr (RES) {
    // +-1 Sylvester Hadamard as MFMA A fragments: row d = 16m + n, k-slot 8g + j <-> rotated dim
    // 32c + 8g + permr(j); entry (-1)^popcount(d & dim)
    for (int e = tid; e < MT * 4 * 64; e += 256) {
      const int m = e / 256, c = (e / 64) % 4, l = e % 64;
      const int d = 16 * m + (l & 15);
      h8 f;
      for (int j = 0; j < 8; ++j) {
        const int dim = 32 * c + 8 * (l >> 4) + permr(j);
        f[j] = (__builtin_popcount(d & dim) & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
      }
      hfrag[e] = f;
    }
  }
  __syncthreads();
  for (int e = tid; e < 32 * NP; e += 256) {  // in-tile RoPE factors (cos, sin)(s * theta_j), s < 32
    const int s = e / NP, j = e % NP;
    float sn, cs;
    sincosf((float)(s * thetas[j]), &sn, &cs);
    rope_tab[(((j >> 4) * 32 + s) * 4 + ((j >> 2) & 3)) * 4 + (j & 3)] = pack_h2(cs, sn);
  }

  // ---- page staging: 16-byte chunks straight from HBM into LDS (global_load_lds, no registers);
  // wave w, lane l copies chunks 256k + 64w + l, which land at consecutive 16-byte slots per wave.
  auto issue = [&](int i, int buf) {
    uint8_t* dst = smem + LY.stage + buf * LY.stage_bytes;
    const int bytes = meta_hb[i];
    const uint8_t* src = a.pool + meta_addr[i];
    for (int k = 0; k < STG; ++k) {
      const int base = 16 * (256 * k + 64 * wv);
      if (base >= bytes) break;
      if (base + 16 * lane < bytes)
        __builtin_amdgcn_global_load_lds((const void*)(src + base + 16 * lane),
                                         (__attribute__((address_space(3))) void*)(dst + base), 16, 0, 0);
    }
    if constexpr (VAR) {  // the page's offset row: P + 1 dwords
      const uint32_t* row = a.tok_off + (size_t)meta_page[i] * (P + 1);
      uint8_t* orow = dst + pad16(a.hb_max);
      for (int base = 64 * wv; base <= P; base += 256)
        if (base + lane <= P)
          __builtin_amdgcn_global_load_lds((const void*)(row + base + lane),
                                           (__attribute__((address_space(3))) void*)(orow + 4 * base), 4, 0, 0);
    }
  };
  // all DMA of this thread done (vmcnt 0), then the workgroup barrier publishes the buffer
  auto settle = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };

  // key basis as A fragments in LDS, [m][c][lane]: row d = 16m + n, k-slot 8g + j <-> latent coordinate
  // 8(4c + g) + perm8(j); each lane later reads its own 16 contiguous bytes
  {
    const uint16_t* Bk = a.wk + (size_t)h * D * a.rk;
    for (int e = tid; e < MT * KC * 64; e += 256) {
      const int m = e / (KC * 64), c = (e / 64) % KC, l = e % 64;
      h8 f;
      for (int j = 0; j < 8; ++j) {
        const int col = 8 * (4 * c + (l >> 4)) + (LAT32 ? j : perm8(j));
        f[j] = col < a.rk ? bf16_to_h(Bk[(size_t)(16 * m + (l & 15)) * a.rk + col]) : (_Float16)0.0f;
      }
      bfrag[e] = f;
    }
  }
  // one-hot B operands of the register transpose: column n of half e takes k-slot with coordinate 16e + n
  // (oh for latents, ohr for the residual, whose codes come in a different order)
  h8 oh[2], ohr[RES ? 2 : 1];
  for (int e = 0; e < 2; ++e)
    for (int j = 0; j < 8; ++j) {
      oh[e][j] = (8 * g + (LAT32 ? j : perm8(j)) == 16 * e + n) ? (_Float16)1.0f : (_Float16)0.0f;
      if constexpr (RES) ohr[e][j] = (8 * g + permr(j) == 16 * e + n) ? (_Float16)1.0f : (_Float16)0.0f;
    }

  // query pairs (j, j + d/2) of the GQ heads in lane j, scaled by log2(e) / sqrt(d) for exp2
  float qa[GQ], qb[GQ];
  double fj = 0.0;
  {
    const float sc = 1.4426950408889634f / sqrtf((float)D);
    const int jj = lane < NP ? lane : 0;
    for (int hq = 0; hq < GQ; ++hq) {
      const size_t base = ((size_t)b * a.Hq + h * GQ + hq) * D;
      float x0, x1;
      if (a.q_bf16) {
        const uint16_t* q = (const uint16_t*)a.q + base;
        x0 = __builtin_bit_cast(float, (uint32_t)q[jj] << 16);
        x1 = __builtin_bit_cast(float, (uint32_t)q[jj + NP] << 16);
      } else {
        const float* q = (const float*)a.q + base;
        x0 = q[jj];
        x1 = q[jj + NP];
      }
      qa[hq] = x0 * sc;
      qb[hq] = x1 * sc;
    }
    fj = thetas[jj] * 0.15915494309189535;  // revolutions per position
  }

  f4 acc[NV];
  f4 accr[RES ? 8 : 1];
  for (int i = 0; i < NV; ++i) acc[i] = f4{0, 0, 0, 0};
  for (int i = 0; i < (RES ? 8 : 1); ++i) accr[i] = f4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;

  // Every code / pair read below stays inside the staged buffer, also for slots past the sequence end
  // or beyond a token's rank (their values are discarded through a zero scale and zero).
  const int kcode_b = slot_code_bytes(KB, a.rk), vcode_b = slot_code_bytes(VB, a.rv);
  const int kmeta_b = LAT32 ? 0 : 4 * ceil_div(a.rk, a.G), vmeta_b = LAT32 ? 0 : 4 * ceil_div(a.rv, a.G);

  if (n_pages > 0) issue(0, 0);
  settle();
  for (int ip = 0; ip < n_pages; ++ip) {
    if (ip + 1 < n_pages) issue(ip + 1, (ip + 1) & 1);  // in flight while this page is decoded
    const uint8_t* sb = smem + LY.stage + (ip & 1) * LY.stage_bytes;
    const uint32_t* so = (const uint32_t*)(sb + pad16(a.hb_max));
    HeadSections S;
    if constexpr (VAR) {
      const uint32_t tot = so[P];
      const int64_t cb = (int64_t)(tot & 0xFFFFu) * KB / 8, mb = 4 * (int64_t)(tot >> 16);
      S = head_sections(cb, cb, mb, mb, P, D, RES);
    } else {
      S = a.S_uniform;
    }
    const int page_t0 = (lb0 + ip) * P;
    const int n_st = min(P, T - page_t0 + 31) / 32;  // super-tiles of this page holding tokens
    for (int sti = wv; sti < n_st; sti += 4) {
      const int slot0 = 32 * sti;
      const int t0 = page_t0 + slot0;

      // query rotated by the super-tile base: q~ = R(q_pos - t0) q
      if (lane < NP) {
        double rev = (double)(qpos - t0) * fj;
        rev -= rint(rev);  // |rev| <= 1/2 turn; v_sin/v_cos take their argument in turns
        const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
        for (int hq = 0; hq < GQ; ++hq)
          qbuf[wv][hq][lane] = pack_h2(qa[hq] * cs - qb[hq] * sn, qb[hq] * cs + qa[hq] * sn);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

      float sc[2][4];
      h4 vtb[NV][2];
      h4 vrtb[RES ? 8 : 1][2];
      for (int blk = 0; blk < 2; ++blk) {
        const int tt = 16 * blk + n;
        const bool valid = t0 + tt < T;
        const int slot = slot0 + tt;
        int rk_t, rv_t;
        int kco, vco, kmo, vmo;
        if constexpr (VAR) {
          const uint32_t o0 = so[slot], o1 = so[slot + 1];
          const int r = valid ? (int)((o1 - o0) & 0xFFFFu) : 0;
          rk_t = rv_t = r;
          kco = vco = (int)((o0 & 0xFFFFu) * KB / 8);
          kmo = vmo = 4 * (o0 >> 16);
        } else {
          rk_t = valid ? a.rk : 0;
          rv_t = valid ? a.rv : 0;
          kco = slot * kcode_b; vco = slot * vcode_b;
          kmo = slot * kmeta_b; vmo = slot * vmeta_b;
        }

        // ---- keys: latent -> fp16 B operand, up-projection
        h8 kb[KC];
        for (int c = 0; c < KC; ++c) {
          const int w = 4 * c + g;
          const bool ok = 8 * w < rk_t;
          if constexpr (LAT32) {
            const float* src = (const float*)(sb + S.kc + kco) + 8 * w;
            for (int j = 0; j < 8; ++j) kb[c][j] = ok ? (_Float16)src[j] : (_Float16)0.0f;
          } else {
            const uint32_t x = codes8_as_nibbles<KB>(sb + S.kc, kco + KB * w);
            const uint32_t sz = *(const uint32_t*)(sb + S.km + kmo + 4 * ((8 * w) / a.G));
            kb[c] = dequant_int4x8(x, ok ? sz : 0u);
          }
        }
        f4 kp[MT];
        for (int m = 0; m < MT; ++m) kp[m] = f4{0, 0, 0, 0};
        for (int c = 0; c < KC; ++c) {
          if (c > 0 && __builtin_amdgcn_ballot_w64(rk_t > 32 * c) == 0) break;
          for (int m = 0; m < MT; ++m) kp[m] = mfma16x16x32(bfrag[(m * KC + c) * 64 + lane], kb[c], kp[m]);
        }
        if constexpr (RES) {
          // key residual: 32 code bytes of the slot; k-slot 8g + j of chunk c <-> rotated dim 32c + 8g + permr(j)
          const uint8_t* rc = sb + S.kr + slot * 32;
          const uint16_t s16 = valid ? *(const uint16_t*)(sb + S.ks + 2 * slot) : (uint16_t)0;
          const float s = (float)__builtin_bit_cast(_Float16, s16) * 0.04419417382415922f;  // 1/(2 sqrt(128))
          const h2 rss = {(_Float16)s, (_Float16)s};
          for (int c = 0; c < 4; ++c) {
            const uint32_t u16 = valid ? *(const uint16_t*)(rc + 8 * c + 2 * g) : 0u;
            const h8 e = dequant_res2x8(u16, rss);
            for (int m = 0; m < MT; ++m) kp[m] = mfma16x16x32(hfrag[(m * 4 + c) * 64 + lane], e, kp[m]);
          }
        }

        // ---- RoPE on the reconstructed key (offset tt inside the super-tile), packed as the score A operand
        h8 kq[QC];
        for (int c = 0; c < QC; ++c) {
          const u4 f4v = *(const u4*)&rope_tab[((c * 32 + tt) * 4 + g) * 4];
          for (int i = 0; i < 4; ++i) {
            const h2 r = as_h2(rope_pair(pack_h2(kp[c][i], kp[c + QC][i]), f4v[i]));
            kq[c][2 * i] = r.x;
            kq[c][2 * i + 1] = r.y;
          }
        }
        f4 s4 = {0, 0, 0, 0};
        // query column n of the score product; columns n >= GQ repeat real heads and are never used
        for (int c = 0; c < QC; ++c) s4 = mfma16x16x32(kq[c], *(const h8*)&qbuf[wv][n & (GQ - 1)][16 * c + 4 * g], s4);
        for (int i = 0; i < 4; ++i) sc[blk][i] = s4[i];

        // ---- values: latent -> fp16, register transpose through a one-hot MFMA
        h8 vb[VC];
        for (int c = 0; c < VC; ++c) {
          const int w = 4 * c + g;
          const bool ok = 8 * w < rv_t;
          if constexpr (LAT32) {
            const float* src = (const float*)(sb + S.vc + vco) + 8 * w;
            for (int j = 0; j < 8; ++j) vb[c][j] = ok ? (_Float16)src[j] : (_Float16)0.0f;
          } else {
            const uint32_t x = codes8_as_nibbles<VB>(sb + S.vc, vco + VB * w);
            const uint32_t sz = *(const uint32_t*)(sb + S.vm + vmo + 4 * ((8 * w) / a.G));
            vb[c] = dequant_int4x8(x, ok ? sz : 0u);
          }
        }
        for (int nt = 0; nt < NV; ++nt) {
          f4 tr = {0, 0, 0, 0};
          if (nt == 0 || __builtin_amdgcn_ballot_w64(rv_t > 16 * nt) != 0) tr = mfma16x16x32(vb[nt >> 1], oh[nt & 1], tr);
          vtb[nt][blk] = h4{(_Float16)tr[0], (_Float16)tr[1], (_Float16)tr[2], (_Float16)tr[3]};
        }
        if constexpr (RES) {
          const uint8_t* rc = sb + S.vr + slot * 32;
          const uint16_t s16 = valid ? *(const uint16_t*)(sb + S.vs + 2 * slot) : (uint16_t)0;
          const float s = (float)__builtin_bit_cast(_Float16, s16) * 0.04419417382415922f;
          const h2 rss = {(_Float16)s, (_Float16)s};
          for (int c = 0; c < 4; ++c) {
            const uint32_t u16 = valid ? *(const uint16_t*)(rc + 8 * c + 2 * g) : 0u;
            const h8 e = dequant_res2x8(u16, rss);
            for (int hlf = 0; hlf < 2; ++hlf) {
              const f4 tr = mfma16x16x32(e, ohr[hlf], f4{0, 0, 0, 0});
              vrtb[2 * c + hlf][blk] = h4{(_Float16)tr[0], (_Float16)tr[1], (_Float16)tr[2], (_Float16)tr[3]};
            }
          }
        }
      }

      // ---- online softmax over the 32 scores; lane (head n, group g) holds tokens 4g..4g+3 of each block
      if (t0 + 32 > T)  // tail of the sequence: drop the scores of slots past its end
        for (int blk = 0; blk < 2; ++blk)
          for (int i = 0; i < 4; ++i)
            if (t0 + 16 * blk + 4 * g + i >= T) sc[blk][i] = -INFINITY;
      // lanes n >= GQ carry copies of real query columns: never mixed with the real heads, never written
      float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      h8 pop;
      float psum = 0.0f;
      for (int blk = 0; blk < 2; ++blk)
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sc[blk][i] - m_new);  // exp2(-inf) = 0
          const _Float16 ph = (_Float16)p;
          pop[4 * blk + i] = ph;
          psum += (float)ph;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
        float al[4];
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
        for (int nt = 0; nt < NV; ++nt)
          for (int i = 0; i < 4; ++i) acc[nt][i] *= al[i];
        if constexpr (RES)
          for (int nt = 0; nt < 8; ++nt)
            for (int i = 0; i < 4; ++i) accr[nt][i] *= al[i];
      }
      for (int nt = 0; nt < NV; ++nt) {
        const h8 vt = {vtb[nt][0][0], vtb[nt][0][1], vtb[nt][0][2], vtb[nt][0][3],
                       vtb[nt][1][0], vtb[nt][1][1], vtb[nt][1][2], vtb[nt][1][3]};
        acc[nt] = mfma16x16x32(pop, vt, acc[nt]);
      }
      if constexpr (RES)
        for (int nt = 0; nt < 8; ++nt) {
          const h8 vt = {vrtb[nt][0][0], vrtb[nt][0][1], vrtb[nt][0][2], vrtb[nt][0][3],
                         vrtb[nt][1][0], vrtb[nt][1][1], vrtb[nt][1][2], vrtb[nt][1][3]};
          accr[nt] = mfma16x16x32(pop, vt, accr[nt]);
        }
    }
    settle();
  }

  // ---- partial of this wave: m[GQ], l[GQ], acc[GQ][NV*16] (latent), accr[GQ][128] (rotated residual)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* part = a.ws + ((size_t)((b * a.Hkv + h) * a.n_splits + split) * 4 + wv) * a.part_stride;
  if (lane < GQ) {
    part[lane] = m_run;
    part[GQ + lane] = l_run;
  }
  float* pacc = part + 2 * GQ;
  for (int nt = 0; nt < NV; ++nt)
    for (int i = 0; i < 4; ++i) {
      const int hq = 4 * g + i;
      if (hq < GQ) pacc[hq * (NV * 16) + 16 * nt + n] = acc[nt][i];
    }
  if constexpr (RES) {
    float* pr = pacc + GQ * NV * 16;
    for (int nt = 0; nt < 8; ++nt)
      for (int i = 0; i < 4; ++i) {
        const int hq = 4 * g + i;
        if (hq < GQ) pr[hq * 128 + 16 * nt + n] = accr[nt][i];
      }
  }
}

// Combine the partials of one (b, kv head): m* = max m, w_p = 2^(m_p - m*), l* = sum w_p l_p,
// c* = sum w_p acc_p; out = (B_v c* [+ H r*]) / l*.
template <int D, int NV, bool RES>
__global__ __launch_bounds__(256) void merge_head_kernel(const float* ws, const uint16_t* wv, float* out, int Hkv,
                                                         int Hq, int rv, int n_parts, int part_stride) {
  __shared__ float cst[GQ][NV * 16];
  __shared__ float rst[RES ? GQ : 1][RES ? 128 : 1];
  __shared__ float lst[GQ];
  const int bh = blockIdx.x, h = bh % Hkv, b = bh / Hkv;
  const int tid = threadIdx.x, hq = tid / 64, l = tid % 64;
  const float* parts = ws + (size_t)bh * n_parts * part_stride;
  float m = -INFINITY;
  for (int p = 0; p < n_parts; ++p) m = fmaxf(m, parts[(size_t)p * part_stride + hq]);
  float lsum = 0.0f, c0 = 0.0f, c1 = 0.0f, r0 = 0.0f, r1 = 0.0f;
  for (int p = 0; p < n_parts; ++p) {
    const float* pp = parts + (size_t)p * part_stride;
    const float mp = pp[hq];
    if (mp == -INFINITY) continue;
    const float wgt = exp2f(mp - m);
    lsum += wgt * pp[GQ + hq];
    const float* pa = pp + 2 * GQ + hq * NV * 16;
    if (l < NV * 16) c0 += wgt * pa[l];
    if (NV * 16 > 64 && l + 64 < NV * 16) c1 += wgt * pa[l + 64];
    if constexpr (RES) {
      const float* pr = pp + 2 * GQ + GQ * NV * 16 + hq * 128;
      r0 += wgt * pr[l];
      r1 += wgt * pr[l + 64];
    }
  }
  if (l < NV * 16) cst[hq][l] = c0;
  if (NV * 16 > 64 && l + 64 < NV * 16) cst[hq][l + 64] = c1;
  if constexpr (RES) {
    rst[hq][l] = r0;
    rst[hq][l + 64] = r1;
  }
  if (l == 0) lst[hq] = lsum;
  __syncthreads();
  const float inv = 1.0f / lst[hq];
  const uint16_t* Bv = wv + (size_t)h * D * rv;
  for (int d = l; d < D; d += 64) {
    float o = 0.0f;
    for (int i = 0; i < rv; ++i) o += __builtin_bit_cast(float, (uint32_t)Bv[(size_t)d * rv + i] << 16) * cst[hq][i];
    if constexpr (RES) {
      float rr = 0.0f;
      for (int i = 0; i < 128; ++i) rr += (__builtin_popcount(d & i) & 1) ? -rst[hq][i] : rst[hq][i];
      o += rr;
    }
    out[((size_t)b * Hq + h * GQ + hq) * D + d] = o * inv;
  }
}

// ---------------------------------------------------------------- host side

template <int D, int KC, int VC, int KB, int VB, bool RES, bool VAR, int STG>
static hipError_t launch_variant(const DecodeHeadArgs& a, int grid, const uint16_t* wv, float* out, hipStream_t st) {
  const int lds = head_lds(D, KC, a.P, RES, a.hb_max).total;
  auto kern = decode_head_kernel<D, KC, VC, KB, VB, RES, VAR, STG>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipError_t e = mark(g_marks.begin, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(g_marks.end, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_head_kernel<D, 2 * VC, RES>), dim3(a.B * a.Hkv), dim3(256), 0, st, a.ws, wv, out, a.Hkv,
                     a.Hq, a.rv, a.n_splits * 4, a.part_stride);
  return hipGetLastError();
}

// Merge of per-wave partials for head dimension 128 without residual (also used by the INT4 fast path).
hipError_t launch_merge_head128(int NV, const float* ws, const uint16_t* wv, float* out, int B, int Hkv, int Hq,
                                int rv, int n_parts, int part_stride, hipStream_t st) {
  if (NV == 4)
    hipLaunchKernelGGL((merge_head_kernel<128, 4, false>), dim3(B * Hkv), dim3(256), 0, st, ws, wv, out, Hkv, Hq, rv,
                       n_parts, part_stride);
  else if (NV == 2)
    hipLaunchKernelGGL((merge_head_kernel<128, 2, false>), dim3(B * Hkv), dim3(256), 0, st, ws, wv, out, Hkv, Hq, rv,
                       n_parts, part_stride);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int head_part_stride(int rv_cap, int residual) {
  const int NV = 2 * ceil_div(rv_cap, 32);
  return 2 * GQ + GQ * NV * 16 + (residual ? GQ * 128 : 0);
}

// Largest head block (every slot at the rank cap).
static int64_t head_block_max(const kvc_layout& L) {
  const int P = L.page_size;
  return head_sections((int64_t)P * slot_code_bytes(lat_bits_k(L), L.r_k_cap),
                       (int64_t)P * slot_code_bytes(lat_bits_v(L), L.r_v_cap),
                       (int64_t)P * slot_meta_bytes(lat_bits_k(L), L.r_k_cap, L.group),
                       (int64_t)P * slot_meta_bytes(lat_bits_v(L), L.r_v_cap, L.group), P, L.head_dim,
                       L.residual_bits)
      .hb;
}

int head_max_pages_per_split() { return MAX_SPLIT_PAGES; }

// INT4 fast path (decode_int4.hip)
bool int4_supported(const kvc_layout& L, int64_t hb_max);
hipError_t launch_decode_int4(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out, void* ws,
                              int n_splits, int pages_per_split, int part_stride, const HeadSections& S_uniform,
                              int hb_max, hipStream_t st);
// INT4 latents with the rotated residual (decode_res.hip)
bool res_supported(const kvc_layout& L, int64_t hb);
hipError_t launch_decode_res(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out, void* ws,
                             int n_splits, int pages_per_split, int part_stride, const HeadSections& S,
                             hipStream_t st);

// The compiled variants (head dim, key chunks, value chunks, key bits, value bits, residual, variable rank,
// staging chunks), used both to decide support and to launch, so that a supported layout always has one.
#define KVC_HEAD_VARIANTS(X)                 \
  X(128, 2, 2, 4, 4, false, false, 5)        \
  X(128, 2, 2, 4, 4, false, true, 5)         \
  X(128, 2, 2, 4, 4, true, false, 9)         \
  X(128, 1, 1, 4, 4, false, false, 3)        \
  X(128, 1, 1, 4, 4, false, true, 3)         \
  X(64, 1, 1, 32, 32, false, false, 9)       \
  X(64, 2, 2, 32, 32, false, false, 9)       \
  X(64, 2, 2, 4, 4, false, false, 5)         \
  X(64, 2, 2, 4, 4, false, true, 5)          \
  X(64, 1, 1, 4, 4, false, false, 3)         \
  X(128, 2, 2, 3, 3, false, false, 5)        \
  X(128, 2, 2, 2, 2, false, false, 5)        \
  X(128, 2, 2, 3, 2, false, false, 5)        \
  X(128, 2, 2, 3, 3, false, true, 5)         \
  X(128, 2, 2, 2, 2, false, true, 5)         \
  X(128, 2, 2, 3, 3, true, false, 9)

static bool head_has_variant(int d, int KC, int VC, int kb, int vb, bool res, bool var, int stg) {
#define KVC_HAS(D_, KC_, VC_, KB_, VB_, RES_, VAR_, STG_)                                                   \
  if (d == D_ && KC == KC_ && VC == VC_ && kb == KB_ && vb == VB_ && res == RES_ && var == VAR_ && stg <= STG_) \
    return true;
  KVC_HEAD_VARIANTS(KVC_HAS)
#undef KVC_HAS
  return false;
}

bool head_supported(const kvc_layout& L) {
  if (L.shared) return false;
  if (L.n_q_heads != GQ * L.n_kv_heads) return false;
  if (L.head_dim != 64 && L.head_dim != 128) return false;
  if (L.r_k_cap > 64 || L.r_v_cap > 64) return false;
  if (L.residual_bits && L.head_dim != 128) return false;
  if (L.latent_bits != 32 && L.group % 16) return false;
  const int64_t hb = head_block_max(L);
  if (hb > 16 * 256 * 9) return false;  // staging registers: at most 9 x 16 bytes per thread
  if (!int4_supported(L, hb) && !res_supported(L, hb) &&
      !head_has_variant(L.head_dim, ceil_div(L.r_k_cap, 32), ceil_div(L.r_v_cap, 32), lat_bits_k(L), lat_bits_v(L),
                        L.residual_bits != 0, L.variable_rank != 0, ceil_div((int)hb, 16 * 256)))
    return false;
  if (head_lds(L.head_dim, ceil_div(L.r_k_cap, 32), L.page_size, L.residual_bits != 0, (int)hb).total > 160 * 1024)
    return false;
  return true;
}

int head_decode_path(const kvc_layout& L) {
  const int64_t hb = head_block_max(L);
  return int4_supported(L, hb) ? KVC_PATH_INT4 : res_supported(L, hb) ? KVC_PATH_RES : KVC_PATH_HEAD;
}

hipError_t launch_decode_head(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out, void* ws,
                              int n_splits, int pages_per_split, hipStream_t st, bool* unsupported) {
  DecodeHeadArgs a;
  a.pool = C.pool; a.page_off = C.page_off; a.tok_off = C.tok_off;
  a.block_table = in.block_table; a.seq_len = in.seq_len; a.q_pos = in.q_pos; a.q = in.q; a.wk = in.wk;
  a.ws = (float*)ws; a.q_bf16 = in.q_dtype == KVC_BF16;
  a.B = in.B; a.Hkv = L.n_kv_heads; a.Hq = L.n_q_heads; a.max_blocks = in.max_blocks; a.P = L.page_size;
  a.rk = L.r_k_cap; a.rv = L.r_v_cap; a.G = L.group; a.n_splits = n_splits; a.pages_per_split = pages_per_split;
  a.part_stride = head_part_stride(L.r_v_cap, L.residual_bits);
  a.theta = L.rope_theta;
  const int P = L.page_size;
  a.S_uniform = head_sections((int64_t)P * slot_code_bytes(lat_bits_k(L), L.r_k_cap),
                              (int64_t)P * slot_code_bytes(lat_bits_v(L), L.r_v_cap),
                              (int64_t)P * slot_meta_bytes(lat_bits_k(L), L.r_k_cap, L.group),
                              (int64_t)P * slot_meta_bytes(lat_bits_v(L), L.r_v_cap, L.group), P, L.head_dim,
                              L.residual_bits);
  a.hb_max = (int)head_block_max(L);
  *unsupported = false;
  if (int4_supported(L, a.hb_max))
    return launch_decode_int4(L, C, in, out, ws, n_splits, pages_per_split, a.part_stride, a.S_uniform, a.hb_max, st);
  if (res_supported(L, a.hb_max))
    return launch_decode_res(L, C, in, out, ws, n_splits, pages_per_split, a.part_stride, a.S_uniform, st);
  const int stg = ceil_div(a.hb_max, 16 * 256);
  const int grid = in.B * L.n_kv_heads * n_splits;
  const int KC = ceil_div(L.r_k_cap, 32), VC = ceil_div(L.r_v_cap, 32);
  const int kb = lat_bits_k(L), vb = lat_bits_v(L);
  const bool res = L.residual_bits != 0, var = L.variable_rank != 0;
#define KVC_TRY(D_, KC_, VC_, KB_, VB_, RES_, VAR_, STG_)                                                       \
  if (L.head_dim == D_ && KC == KC_ && VC == VC_ && kb == KB_ && vb == VB_ && res == RES_ && var == VAR_ && \
      stg <= STG_)                                                                                          \
    return launch_variant<D_, KC_, VC_, KB_, VB_, RES_, VAR_, STG_>(a, grid, in.wv, out, st);
  KVC_HEAD_VARIANTS(KVC_TRY)
#undef KVC_TRY
  *unsupported = true;
  return hipSuccess;
}

}  // namespace kvc
