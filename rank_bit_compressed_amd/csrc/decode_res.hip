// decode_res.hip -- one decode step of attention over a per-KV-head INT4 cache with the 2-bit rotated
// residual, head dimension 128, four query heads per KV head, uniform ranks (gfx950).
//
// A token-head's key is k = B_k c_k + H e_k and its value v = B_v c_v + H e_v, with c the dequantized INT4
// latent (code * scale + zero per group), e = (code - 1.5) * s the dequantized 2-bit residual (one fp16 scale
// per token-head) and H the 128-point Sylvester Hadamard matrix / sqrt(128); RoPE acts on k after it is
// rebuilt.
//
// Work decomposition: one workgroup (4 waves, one workgroup per CU: each wave has the whole register file)
// per (sequence b, KV head h, context split of pages).  The workgroup copies each page's head-h block (codes,
// scale/zero pairs, residual codes and scales) HBM -> LDS with buffer loads that write LDS directly, two
// buffers deep (the next page in flight while this one is decoded).  Wave w decodes the 32-token super-tiles
// w and w + 4 of every page and keeps its own online-softmax state; lane l serves token l % 32, its half l / 32
// supplies eight of the sixteen k-slots of each matrix step.  Per super-tile:
//   keys: latent codes -> fp16 (fp8-conversion trick, one fp16 FMA for scale and zero), K_pre = B_k c on
//     v_mfma_f32_32x32x16_f16.  Residual: the 2-bit codes c are spread one per byte (one shift and one mask
//     per four codes), where each byte is the fp8 e4m3 pattern of c 2^-9; v_mfma_scale_f32_32x32x64_f8f6f4
//     with the +-1 Hadamard H' in fp8 and a B scale of 2^9 gives H' c exactly (two products per head-dim
//     tile over the 128 coordinates).  H' 1 is 128 at head dim 0 and 0 elsewhere, so
//     K_pre += (s / sqrt(128)) (H' c - 192 [d = 0]).  RoPE on the pairs (j, j + 64) (tiles m and m + 2:
//     one lane, one accumulator entry); scores S = Q~ K~^T with the query heads replicated over the 32 rows;
//   values: latent chunks and residual 2c - 3 (exact) into per-wave fp16 tiles in LDS, read back token-major
//     with ds_read_b64_tr_b16 as the B operand of v_mfma_f32_16x16x32_f16.  The A operand is the
//     probabilities for the latent and the probabilities times the token's residual scale S for the residual
//     (both transposed through LDS).  The value latent and the rotated value residual accumulate in registers,
//     and B_v and H are applied once per (b, query head) in the merge (sum_t p_t B c_t = B sum_t p_t c_t).
// RoPE is split as R(t0 + s) = R(t0) R(s): R(s) of the lane's slot s < 32 is held in registers, R(q_pos - t0)
// is applied to the query per super-tile.  Softmax keeps a reference maximum per head that is only raised
// when a score exceeds it by 2^8 in the exp2 domain.
#include <math.h>

#include "lds_copy.hpp"
#include "res_codes.hpp"

namespace kvc {

struct ResArgs {
  const uint8_t* pool;
  const int64_t* page_off;
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* q_pos;
  const void* q;
  const uint16_t* wk;
  float* ws;
  int q_bf16;
  int B, Hkv, Hq, max_blocks, P, rk, rv, G, n_splits, pages_per_split, part_stride;
  double theta;
  HeadSections S;  // sections of a head block (uniform ranks)
};

namespace rsd {
constexpr int D = 128, GQ = 4, NP = 64;
constexpr int MAX_SPLIT_PAGES = 128;
constexpr float TAU = 8.0f;                // lazy-max slack, log2 units
// value tiles: chunk c (8 coordinates) of token t at byte CS c + 16 t; the row of a chunk is padded from 512 to
// 576 bytes so that the transposing reads of a step (two chunks, token groups 256 bytes apart) hit distinct banks
constexpr int CS = 32 * 16 + 64;
constexpr int VLT = 8 * CS;               // a wave's value-latent tile: 8 chunks
constexpr int VRT = 16 * CS;              // a wave's value-residual tile: 16 chunks

struct Lds {
  int meta_addr, theta, qsrc, qbuf, pt, vlat, vres, stage, stage_bytes, total;
};
__host__ __device__ inline Lds lds_layout(int64_t hb) {
  Lds L;
  int o = 0;
  L.meta_addr = o; o += MAX_SPLIT_PAGES * 8;
  L.theta = o; o += NP * 8;                   // RoPE frequencies, turns per position
  L.qsrc = o; o += NP * 2 * GQ * 4;           // scaled query, pair j: x_j of heads 0-3, then x_{j+64}
  L.qbuf = o; o += 4 * 2 * GQ * (NP + 4) * 4;  // per wave: rotated query of its two super-tiles, packed fp16
  L.pt = o; o += 2 * 4 * 32 * GQ * 2;         // per wave: probabilities [token][head] fp16, then times S
  L.vlat = o; o += 4 * VLT;
  L.vres = o; o += 4 * VRT;
  L.stage_bytes = (int)pad16(hb);
  L.stage = o; o += 2 * L.stage_bytes;
  L.total = o;
  return L;
}
}  // namespace rsd

typedef float f16v_r __attribute__((ext_vector_type(16)));
__device__ inline f16v_r mfma32r(h8 a, h8 b, f16v_r c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }

// s_waitcnt vmcnt(k) for a run-time k (this wave's copies still allowed in flight)
__device__ inline void vmcnt_wait_r(int k) {
  switch (k) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
  }
}

// KS, VS: 16-coordinate steps of the key / value ranks (2..4); STG: 4 KiB rounds of a page copy
template <int KS, int VS, int STG>
__global__ __launch_bounds__(256, 1) void decode_res_kernel(ResArgs a) {
  using namespace rsd;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int P = a.P;
  const HeadSections S = a.S;
  const Lds LY = lds_layout(S.hb);
  int64_t* meta_addr = (int64_t*)(smem + LY.meta_addr);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 31, hf = lane >> 5, rho = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x % a.n_splits;
  const int h = (blockIdx.x / a.n_splits) % a.Hkv;
  const int b = blockIdx.x / (a.n_splits * a.Hkv);
  const int T = a.seq_len[b];
  const int qpos = a.q_pos ? a.q_pos[b] : T;
  const int lb0 = split * a.pages_per_split;
  const int n_pages = max(0, min((T + P - 1) / P, lb0 + a.pages_per_split) - lb0);

  // ---- page addresses of the split
  for (int i = tid; i < n_pages; i += 256) {
    const int page = a.block_table[(size_t)b * a.max_blocks + lb0 + i];
    meta_addr[i] = a.page_off[page] + (int64_t)h * S.hb;
  }

  // ---- key basis as A fragments: row = head dim 32m + t, k-slot 8hf + j <-> coordinate 16s + 8hf + perm8(j)
  // (the order in which a code dword dequantizes); zero past the rank
  h8 bf[KS][4];
  {
    const uint16_t* Bk = a.wk + (size_t)h * D * a.rk;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col0 = 16 * s + 8 * hf;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        h8 f = {};
        if (col0 < a.rk) {
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = bf16_to_h(Bk[(size_t)(32 * m + t) * a.rk + col0 + perm8(j)]);
        }
        bf[s][m] = f;
      }
    }
  }
  // ---- +-1 Hadamard fragments of the fp8 key residual product: head-dim tile mt (row r = t <-> dim 32 mt + r),
  // product be; byte b of this lane's 32 <-> coordinate 64 hf + 32 be + res8_coord(0, b) (a lane half reads its
  // token's residual code dwords 4hf..4hf+3 in one 16-byte read, and product be takes dwords 2be, 2be + 1 of them);
  // e4m3 +1 = 0x38, -1 = 0xB8.  The A and B operands share the lane/byte -> k assignment, so the pairing holds
  // whatever it is.
  v8i_t hf8[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int be = 0; be < 2; ++be)
#pragma unroll
      for (int o = 0; o < 8; ++o) {
        uint32_t w = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 64 * hf + 32 * be + res8_coord(0, 4 * o + q);
          w |= ((__builtin_popcount((32 * mt + t) & i) & 1) ? 0xB8u : 0x38u) << (8 * q);
        }
        hf8[mt][be][o] = (int)w;
      }
  // kept in the accumulator registers, which the fp8 products read directly (left to the allocator, they were
  // copied back into vector registers before every product)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int be = 0; be < 2; ++be) asm volatile("" : "=a"(hf8[mt][be]) : "0"(hf8[mt][be]));
  // ---- RoPE frequencies, once per workgroup: theta_j (fp64 pow) in turns per position
  double* tturn = (double*)(smem + LY.theta);
  if (tid < NP) tturn[tid] = (a.theta > 0.0 ? pow(a.theta, -2.0 * tid / D) : 0.0) * 0.15915494309189535;
  // scaled query (log2(e) / sqrt(d), for exp2) into LDS
  float* qsrc = (float*)(smem + LY.qsrc);
  for (int e = tid; e < NP * GQ; e += 256) {
    const int j = e % NP, hq = e / NP;
    const size_t base = ((size_t)b * a.Hq + h * GQ + hq) * D;
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
    const float sc = 1.4426950408889634f / sqrtf((float)D);
    qsrc[j * 8 + hq] = x0 * sc;
    qsrc[j * 8 + 4 + hq] = x1 * sc;
  }
  __syncthreads();
  // RoPE factors (cos, sin)(t theta_j) of this lane's slot t: pair j = 32m + 8(i/4) + 4hf + i%4 for accumulator
  // entry i of tiles m and m + 2; |t theta_j| < 32 turns, where v_sin / v_cos are accurate
  uint32_t rf[2][16];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = 32 * m + 8 * (i / 4) + 4 * hf + i % 4;
      const float rev = (float)(t * tturn[j]);
      rf[m][i] = pack_h2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
    }
  const double fj = tturn[lane];  // turns per position of pair `lane` (query rotation)
  uint32_t* qbuf = (uint32_t*)(smem + LY.qbuf) + wv * 2 * GQ * (NP + 4);
  _Float16* pt = (_Float16*)(smem + LY.pt) + wv * 2 * 32 * GQ;  // then pt2 = pt + 32 GQ
  _Float16* pt2 = pt + 32 * GQ;
  uint8_t* vlat = smem + LY.vlat + wv * VLT;
  uint8_t* vres = smem + LY.vres + wv * VRT;
  const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem + LY.stage));

  // ---- page staging: wave w copies the 16-byte chunks 256k + 64w + l of page i's head block into buffer
  // i % 2 and returns the number of copy instructions it issued
  const int hb = (int)S.hb;
  auto issue = [&](int i) -> int {
    const uint32_t dst = stage_lds + (i & 1) * LY.stage_bytes;
    const i32x4_t rs = buffer_rsrc(a.pool + uniform64(meta_addr[i]), hb);
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < STG; ++k) {
      const int base = 16 * (256 * k + 64 * wv);
      if (base >= hb) break;  // wave-uniform: every issued copy has lane 0 active
      if (base + 16 * lane < hb) copy16_to_lds(rs, dst + base, base + 16 * lane);
      ++cnt;
    }
    return cnt;
  };
  auto settle = [&](int keep) {
    vmcnt_wait_r(keep);
    lds_barrier();
  };

  // running state: value latent (16 coordinates per step) and rotated value residual accumulators, rows =
  // query heads (replicated), sums, reference maxima
  f4 acc[VS], accr[8];
#pragma unroll
  for (int i = 0; i < VS; ++i) acc[i] = f4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) accr[i] = f4{0, 0, 0, 0};
  float psum[GQ], m_ref[GQ];
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    psum[i] = 0.0f;
    m_ref[i] = 0.0f;
  }
  bool fresh = true;

  const int kcb = a.rk / 2, vcb = a.rv / 2;                                  // code bytes per slot
  const int kmb = 4 * ceil_div(a.rk, a.G), vmb = 4 * ceil_div(a.rv, a.G);  // pair bytes per slot
  const float rscale = 0.04419417382415922f;  // 1 / (2 sqrt(128)): e / sqrt(128) = (2c - 3) s / (2 sqrt(128))

  if (n_pages > 0) {
    issue(0);
    settle(0);
  }
  for (int ip = 0; ip < n_pages; ++ip) {
    if (ip + 1 < n_pages) issue(ip + 1);  // into the buffer everyone finished with before the last barrier
    const uint8_t* sb = smem + LY.stage + (ip & 1) * LY.stage_bytes;
    const int page_t0 = (lb0 + ip) * P;
    const int n_st = min(P, T - page_t0 + 31) / 32;    // super-tiles of this page holding tokens
    const int nst_w = (n_st > wv) + (n_st > wv + 4);  // this wave's: super-tiles wv and wv + 4
    // queries rotated by the bases of this wave's super-tiles, q~ = R(q_pos - t0) q; lane j: pair j
    {
      const f4 qa = *(const f4*)&qsrc[lane * 8], qb = *(const f4*)&qsrc[lane * 8 + 4];
      for (int k = 0; k < nst_w; ++k) {
        double rev = (double)(qpos - page_t0 - 32 * (wv + 4 * k)) * fj;
        rev -= rint(rev);  // |rev| <= 1/2 turn; v_sin / v_cos take turns
        const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
#pragma unroll
        for (int hq = 0; hq < GQ; ++hq)
          qbuf[(k * GQ + hq) * (NP + 4) + lane] = pack_h2(qa[hq] * cs - qb[hq] * sn, qb[hq] * cs + qa[hq] * sn);
      }
    }
    wave_lds_sync();

    for (int k = 0; k < nst_w; ++k) {
      const int slot = 32 * (wv + 4 * k) + t;
      const int t0 = page_t0 + 32 * (wv + 4 * k);
      const uint32_t* qrow = qbuf + (k * GQ + (t & 3)) * (NP + 4) + 4 * hf;

      // ---- this lane's key words: key code dwords (2s + hf) with their pairs, its half's residual code dwords
      // 4hf..4hf+3 (32 bytes per token; dword j holds the codes of coordinates 16j ..), residual scales
      uint32_t kw[KS], kp[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kw[s] = *(const uint32_t*)(sb + S.kc + slot * kcb + 8 * s + 4 * hf);
        kp[s] = *(const uint32_t*)(sb + S.km + slot * kmb + 4 * ((16 * s + 8 * hf) / a.G));
      }
      const u4 krw = *(const u4*)(sb + S.kr + 32 * slot + 16 * hf);
      // key residual: K_res = (s / sqrt(128)) (H' c - 1.5 H' 1); value residual: (2c - 3) s / (2 sqrt(128))
      const float ks = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)(sb + S.ks + 2 * slot)) * (2.0f * rscale);
      const float vs = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)(sb + S.vs + 2 * slot)) * rscale;

      // ---- values into this wave's fp16 tiles (chunk c of token t at byte CS c + 16 t): chunk c of the latent is
      // code dword c (pair of coordinate 8c), the residual's chunks 2j, 2j + 1 come from its code dword j
      // (coordinates 16j + res_coord(e, ...), e = 0, 1).  Lane half hf takes the latent's dwords VS hf.. and the
      // residual's dwords 4hf..4hf+3 of its token, each in one wide read: a lane octet's reads, 32 bytes apart, meet
      // two to a bank, where four-byte reads of the 32-byte token rows met eight to a bank.
      {
        uint32_t vq[VS];
        if constexpr (VS == 4) {
          const u4 x = *(const u4*)(sb + S.vc + slot * vcb + 16 * hf);
#pragma unroll
          for (int i = 0; i < 4; ++i) vq[i] = x[i];
        } else {
          static_assert(VS == 2, "value steps");
          const u2 x = *(const u2*)(sb + S.vc + slot * vcb + 8 * hf);
          vq[0] = x[0];
          vq[1] = x[1];
        }
#pragma unroll
        for (int i = 0; i < VS; ++i) {
          const int c = VS * hf + i;  // chunk = code dword of the token
          const uint32_t pr = *(const uint32_t*)(sb + S.vm + slot * vmb + 4 * ((8 * c) / a.G));
          *(h8*)(vlat + CS * c + 16 * t) = dequant_int4x8(vq[i], pr);
        }
        const u4 rq = *(const u4*)(sb + S.vr + 32 * slot + 16 * hf);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *(h8*)(vres + CS * (8 * hf + i) + 16 * t) = res_2c3(rq[i >> 1], i & 1);
      }

      // ---- keys: latent and residual operands, then per half m the tiles m and m + 2 (head dims d, d + 64),
      // RoPE, and the score steps u = 4m + q (pairs 32m + 8q + 4hf + p in k-slots 8hf + 2p, 8hf + 2p + 1)
      h8 kb[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) kb[s] = dequant_int4x8(kw[s], kp[s]);
      // key residual codes one per byte (fp8 B operands of products 0 and 1): byte q of dword o = code m + 4q of
      // the lane's code dword 2be + o / 4, m = o % 4
      v8i_t er[2];
#pragma unroll
      for (int be = 0; be < 2; ++be)
#pragma unroll
        for (int o = 0; o < 8; ++o) er[be][o] = (int)((krw[2 * be + (o >> 2)] >> (2 * (o & 3))) & 0x03030303u);
      f16v_r sc = {};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f16v_r ka = {}, kz = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          ka = mfma32r(bf[s][m], kb[s], ka);
          kz = mfma32r(bf[s][m + 2], kb[s], kz);
        }
        f16v_r ra = {}, rz = {};  // H' c over the 128 residual coordinates (exact integers)
#pragma unroll
        for (int be = 0; be < 2; ++be) {
          ra = mfma_f8_codes(hf8[m][be], er[be], ra);
          rz = mfma_f8_codes(hf8[m + 2][be], er[be], rz);
        }
        // H' 1 is 128 at head dim 0 (entry 0 of tile 0 in the lanes of half 0) and 0 elsewhere
        if (m == 0 && hf == 0) ra[0] -= 192.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          ka[i] += ks * ra[i];
          kz[i] += ks * rz[i];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u4 kr;
#pragma unroll
          for (int p = 0; p < 4; ++p) kr[p] = rope_pair(pack_h2(ka[4 * q + p], kz[4 * q + p]), rf[m][4 * q + p]);
          const h8 qf = *(const h8*)(qrow + 32 * m + 8 * q);
          sc = mfma32r(qf, __builtin_bit_cast(h8, kr), sc);
        }
      }

      // ---- online softmax; lane (token t) holds the scores of heads 0-3 in sc[0..3]
      float s4[GQ] = {sc[0] - m_ref[0], sc[1] - m_ref[1], sc[2] - m_ref[2], sc[3] - m_ref[3]};
      if (t0 + 32 > T && t0 + t >= T)
#pragma unroll
        for (int i = 0; i < GQ; ++i) s4[i] = -INFINITY;
      const float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
      if (fresh || __builtin_amdgcn_ballot_w64(mx > TAU) != 0) {
        // exact per-head maximum over the super-tile, then raise the reference (or set it, first time)
        float alpha[GQ];
#pragma unroll
        for (int i = 0; i < GQ; ++i) {
          float c = s4[i];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) c = fmaxf(c, __shfl_xor(c, o));
          const float d = fresh ? c : fmaxf(c, 0.0f);
          alpha[i] = fresh ? 1.0f : __builtin_amdgcn_exp2f(-d);
          psum[i] *= alpha[i];
          s4[i] -= d;
          m_ref[i] += d;
        }
#pragma unroll
        for (int nt = 0; nt < VS; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[nt][i] *= alpha[i];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) accr[nt][i] *= alpha[i];
        fresh = false;
      }
      float p[GQ];
      _Float16 ph[GQ], pv[GQ];
#pragma unroll
      for (int i = 0; i < GQ; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s4[i]);  // 2^-inf = 0
        psum[i] += p[i];
        ph[i] = (_Float16)p[i];
        pv[i] = (_Float16)(p[i] * vs);
      }
      if (hf == 0) {
        *(h4*)(pt + GQ * t) = h4{ph[0], ph[1], ph[2], ph[3]};
        *(h4*)(pt2 + GQ * t) = h4{pv[0], pv[1], pv[2], pv[3]};
      }
      wave_lds_sync();
      // P as the A operand of the 16x16x32 value products: row l % 16 <-> head l % 4, k-slot 8g + j <-> token
      // 8g + j (g = l / 16); lane rho of its group points at the row of token 8g + 4v + rho / 4
      const h8 pop = lds_tr8s(pt + GQ * (8 * grp + (rho >> 2)), pt + GQ * (8 * grp + 4 + (rho >> 2)));
      const h8 pops = lds_tr8s(pt2 + GQ * (8 * grp + (rho >> 2)), pt2 + GQ * (8 * grp + 4 + (rho >> 2)));
      // value step nt covers chunks 2nt, 2nt + 1; lane rho points at the 4 columns 4(q4 % 2).. of chunk
      // (2nt + q4 / 2, token 8g + 4v + rho / 4)
      const int q4 = rho & 3;
      const int voff = CS * (q4 >> 1) + (8 * grp + (rho >> 2)) * 16 + (q4 & 1) * 8;
#pragma unroll
      for (int nt = 0; nt < VS; ++nt) {
        const uint8_t* vb = vlat + voff + 2 * CS * nt;
        acc[nt] = mfma16x16x32(pop, lds_tr8s(vb, vb + 64), acc[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const uint8_t* vb = vres + voff + 2 * CS * nt;
        accr[nt] = mfma16x16x32(pops, lds_tr8s(vb, vb + 64), accr[nt]);
      }
      wave_lds_sync();  // the tiles and probabilities are rewritten by the next super-tile
    }
    settle(0);  // the next page landed (and everyone is done with this buffer)
  }

  // ---- partial of the workgroup: the four waves' (m, l, acc, accr) combined in LDS (the staging buffers are
  // idle now), then m[GQ], l[GQ], acc[GQ][NC] (value latent), accr[GQ][128] (rotated value residual); m = -inf
  // when the split holds no token
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    float l = hf == 0 ? psum[i] : 0.0f;  // the two halves of the wave hold the same tokens
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
    psum[i] = l;
  }
  constexpr int NC = 32 * ((VS + 1) / 2);  // latent coordinates per head in the partial
  constexpr int WST = 2 * GQ + GQ * NC + GQ * D;
  float* red = (float*)(smem + LY.stage);  // [wave][WST]
  float* mine = red + wv * WST;
  if (lane < GQ) {
    mine[lane] = fresh ? -INFINITY : m_ref[lane];
    mine[GQ + lane] = psum[lane];
  }
  if (grp == 0) {
#pragma unroll
    for (int nt = 0; nt < VS; ++nt) {
      const int coord = 16 * nt + 8 * (rho >> 3) + perm8(rho & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[2 * GQ + i * NC + coord] = acc[nt][i];
    }
    if (VS * 16 < NC)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[2 * GQ + i * NC + VS * 16 + rho] = 0.0f;
    // residual column n of step nt: chunk 2nt + n / 8, element n % 8
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int coord = 16 * nt + res_coord(rho >> 3, rho & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[2 * GQ + GQ * NC + i * D + coord] = accr[nt][i];
    }
  }
  __syncthreads();
  float* part = a.ws + (size_t)((b * a.Hkv + h) * a.n_splits + split) * a.part_stride;
  for (int e = tid; e < GQ * (NC + D); e += 256) {
    const int hq = e / (NC + D), c = e % (NC + D);
    const int src = c < NC ? 2 * GQ + hq * NC + c : 2 * GQ + GQ * NC + hq * D + (c - NC);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, red[w * WST + hq]);
    float av = 0.0f, lv = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* pw = red + w * WST;
      const float wt = pw[hq] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(pw[hq] - mx);
      av += wt * pw[src];
      lv += wt * pw[GQ + hq];
    }
    part[src] = av;
    if (c == 0) {
      part[hq] = mx;
      part[GQ + hq] = lv;
    }
  }
}

// Final combine over the context splits, the value basis and the inverse rotation of the value residual: one
// workgroup per (sequence, query head), thread d computes out[d] = ((B_v c*)[d] + (H' r*)[d]) / l* with
// c* = sum_s 2^(m_s - m*) acc_s, r* likewise, l* = sum_s 2^(m_s - m*) l_s and H' the +-1 Hadamard (the residual
// accumulators already carry 1 / sqrt(128)).
template <int NC>
__global__ __launch_bounds__(128) void merge_res_kernel(const float* ws, const uint16_t* wv, float* out, int Hkv,
                                                         int Hq, int rv, int n_splits, int part_stride) {
  using namespace rsd;
  __shared__ float cst[NC];
  __shared__ float rst[D];
  __shared__ float lst;
  const int bq = blockIdx.x, hq_all = bq % Hq, b = bq / Hq;
  const int h = hq_all / GQ, hq = hq_all % GQ;
  const int tid = threadIdx.x;
  const float* parts = ws + (size_t)(b * Hkv + h) * n_splits * part_stride;
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, parts[(size_t)s * part_stride + hq]);
  float c = 0.0f, r = 0.0f, l = 0.0f;
  for (int s = 0; s < n_splits; ++s) {
    const float* ps = parts + (size_t)s * part_stride;
    const float ms = ps[hq];
    if (ms == -INFINITY) continue;
    const float wt = exp2f(ms - mx);
    if (tid < NC) c += wt * ps[2 * GQ + hq * NC + tid];
    r += wt * ps[2 * GQ + GQ * NC + hq * D + tid];
    l += wt * ps[GQ + hq];
  }
  if (tid < NC) cst[tid] = c;
  rst[tid] = r;
  if (tid == 0) lst = l;
  __syncthreads();
  const uint16_t* row = wv + ((size_t)h * D + tid) * rv;  // B_v row d = tid, rv bf16 values
  float o = 0.0f;
  for (int i = 0; i < rv; ++i) o += __builtin_bit_cast(float, (uint32_t)row[i] << 16) * cst[i];
  float rr = 0.0f;
  for (int i = 0; i < D; ++i) rr += (__builtin_popcount(tid & i) & 1) ? -rst[i] : rst[i];
  out[((size_t)b * Hq + hq_all) * D + tid] = (o + rr) / lst;
}

// ---------------------------------------------------------------- host side

template <int KS, int VS, int STG>
static hipError_t launch_res(const ResArgs& a, int grid, const uint16_t* wv, float* out, hipStream_t st) {
  const int lds = rsd::lds_layout(a.S.hb).total;
  auto kern = decode_res_kernel<KS, VS, STG>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  e = mark(g_marks.begin, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(g_marks.end, st);
  if (e != hipSuccess) return e;
  constexpr int NC = 32 * ((VS + 1) / 2);
  hipLaunchKernelGGL((merge_res_kernel<NC>), dim3(a.B * a.Hq), dim3(128), 0, st, a.ws, wv, out, a.Hkv, a.Hq, a.rv,
                     a.n_splits, a.part_stride);
  return hipGetLastError();
}

int res_max_pages_per_split() { return rsd::MAX_SPLIT_PAGES; }

// The compiled variants (key steps, value steps, staging rounds), used both to decide support and to launch, so that
// a layout this kernel accepts always has a variant.  The value path reads a lane half's code dwords with one 8- or
// 16-byte read, so the value steps are 2 or 4.
#define KVC_RES_VARIANTS(X) \
  X(3, 4, 10)               \
  X(4, 4, 10)               \
  X(2, 2, 10)               \
  X(2, 4, 10)               \
  X(4, 2, 10)

static bool res_has_variant(int ks, int vs, int stg) {
#define KVC_RES_HAS(KS_, VS_, STG_) \
  if (ks == KS_ && vs == VS_ && stg <= STG_) return true;
  KVC_RES_VARIANTS(KVC_RES_HAS)
#undef KVC_RES_HAS
  return false;
}

// The layouts this kernel serves; the rest of the residual layouts go to the general kernel.
bool res_supported(const kvc_layout& L, int64_t hb) {
  if (L.shared || lat_bits_k(L) != 4 || lat_bits_v(L) != 4 || L.residual_bits != 2 || L.head_dim != 128 || L.variable_rank) return false;
  if (L.n_q_heads != rsd::GQ * L.n_kv_heads) return false;
  if (L.r_k_cap > 64 || L.r_v_cap > 64 || L.r_k_cap < 17 || L.r_v_cap < 17 || L.group % 16) return false;
  if (L.r_k_cap % 16 || L.r_v_cap % 16) return false;  // whole steps: no code or pair read past the rank
  if (hb > 16 * 256 * 10) return false;
  if (!res_has_variant(L.r_k_cap / 16, L.r_v_cap / 16, ceil_div((int)hb, 16 * 256))) return false;
  return rsd::lds_layout(hb).total <= 160 * 1024;
}

hipError_t launch_decode_res(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out, void* ws,
                             int n_splits, int pages_per_split, int part_stride, const HeadSections& S,
                             hipStream_t st) {
  ResArgs a;
  a.pool = C.pool; a.page_off = C.page_off;
  a.block_table = in.block_table; a.seq_len = in.seq_len; a.q_pos = in.q_pos; a.q = in.q; a.wk = in.wk;
  a.ws = (float*)ws; a.q_bf16 = in.q_dtype == KVC_BF16;
  a.B = in.B; a.Hkv = L.n_kv_heads; a.Hq = L.n_q_heads; a.max_blocks = in.max_blocks; a.P = L.page_size;
  a.rk = L.r_k_cap; a.rv = L.r_v_cap; a.G = L.group; a.n_splits = n_splits; a.pages_per_split = pages_per_split;
  a.part_stride = part_stride; a.theta = L.rope_theta; a.S = S;
  const int grid = in.B * L.n_kv_heads * n_splits;
  const int KS = ceil_div(L.r_k_cap, 16), VS = ceil_div(L.r_v_cap, 16);
  const int stg = ceil_div((int)S.hb, 16 * 256);
#define KVC_TRYR(KS_, VS_, STG_) \
  if (KS == KS_ && VS == VS_ && stg <= STG_) return launch_res<KS_, VS_, STG_>(a, grid, in.wv, out, st);
  KVC_RES_VARIANTS(KVC_TRYR)
#undef KVC_TRYR
  return hipErrorInvalidValue;
}

}  // namespace kvc
