// decode_shared.hip -- decode attention over a block-shared latent (gfx950).
//
// One INT4 latent c_t (dim 512, groups of G) per token serves n_layers layers and all KV heads:
// layer l, KV head h rebuilds k = W_k[l][:, h d : (h+1) d]^T c_t (v likewise through W_v), and the
// keys are rotated (RoPE) after that up-projection.  The up-projection is the one dense contraction of
// the path (512 -> 128 per token, layer and head), so the kernel is laid out for the matrix cores.
//
// One workgroup (4 waves, one workgroup per CU so that each wave has the full register file) per
// (layer, KV head, sequence, context split).  Wave w
// owns 32 of the head's 128 dims, {16w..16w+15} and {64+16w..64+16w+15}, so that its RoPE pairs
// (j, j + 64) meet in one lane, and holds W_k's 512 x 32 slice for them as v_mfma_f32_32x32x16_f16
// A fragments in registers.  The workgroup walks 32-token super-tiles:
//   - the super-tile's codes and scale/zero pairs (contiguous in the page record) go HBM -> LDS with
//     buffer loads that write LDS directly, four super-tiles deep, gathered into chunk-major order (16-byte
//     chunk c of token t at slot 32c + t), so that lanes reading the same dword of consecutive tokens hit
//     different LDS banks;
//   - the workgroup dequantizes them once into an fp16 tile of 16-byte chunks (8 coordinates of one token),
//     chunk (d, token), d = 2 step + half, at slot 32 d + token: every wave's up-projection operand is one
//     contiguous 1 KiB read per step; the
//     next super-tile is dequantized (into a second tile) while the matrix cores run this one's
//     up-projection;
//   - each wave: K_pre (its 32 dims x 32 tokens, 32 MFMAs), RoPE, partial scores over its dims for the
//     four query heads; the partials are summed through LDS;
//   - every wave repeats the (identical) online softmax and accumulates the value latent on its 128
//     coordinates with v_mfma_f32_16x16x32_f16, whose token-major operands come from the same fp16 tile
//     through transposing LDS reads.
// The value up-projection W_v is applied once per (layer, sequence, head) in the merge kernel.
#include <math.h>

#include <algorithm>

#include "kvc_common.hpp"

namespace kvc {

static constexpr int SGQ = 4;     // query heads per KV head
static constexpr int SLAT = 512;  // latent dimension handled here
static constexpr int SD = 128;    // head dimension handled here
static constexpr int SKS = SLAT / 16;  // 16-coordinate steps of the latent
static constexpr float STAU = 8.0f;    // lazy-max slack, log2 units

typedef float f16v_t __attribute__((ext_vector_type(16)));

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

static constexpr int SMAX_TILES = 1024;  // super-tiles per split (the page record address of each)

struct SharedLds {
  int raw, raw_bytes, pairs_off, tile, qt, theta, sp, pt, addr, total;
};
__host__ __device__ inline SharedLds shared_lds(int G) {
  SharedLds L;
  int o = 0;
  L.pairs_off = 32 * (SLAT / 2);                                       // codes of 32 tokens, then their pairs
  L.raw_bytes = (int)pad16(L.pairs_off + 32 * 4 * (SLAT / G));
  L.raw = o; o += 4 * L.raw_bytes;                                     // staging ring of 4 super-tiles
  L.tile = o; o += 2 * SKS * 2 * 32 * 16;                              // dequantized latents, 2 x 32 KB
  L.qt = o; o += 2 * SGQ * SD * 2;                                     // rotated query [head][dim] fp16, x 2
  L.theta = o; o += (SD / 2) * 8;                                      // RoPE frequencies, turns per position
  L.sp = o; o += 4 * 32 * SGQ * 4;                                     // partial scores [wave][token][head]
  L.pt = o; o += 4 * 32 * SGQ * 2;                                     // probabilities [wave][token][head] fp16
  L.addr = o; o += SMAX_TILES * 8;                                     // page record address of each super-tile
  L.total = o;
  return L;
}

__device__ inline f16v_t mfma32s(h8 a, h8 b, f16v_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }

__device__ inline h8 lds_tr8s(const void* p0, const void* p1) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  const h4 x = __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)p0));
  const h4 y = __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)p1));
  h8 r = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return r;
}

// s_waitcnt vmcnt(k) for a run-time k (copies of this wave still allowed in flight)
__device__ inline void vmcnt_wait_s(int k) {
  switch (k) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F73); break;
  }
}

// workgroup barrier for LDS data: the staging copies write LDS directly and every wave waits for its own
// before this barrier, so the fences only have to keep the compiler from moving LDS accesses across it
// (a workgroup-scope fence would also wait for the copies still in flight)
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__global__ __launch_bounds__(256, 1) void decode_shared_kernel(DecodeSharedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const SharedLds LY = shared_lds(a.G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 31, hf = lane >> 5, rho = lane & 15, grp = lane >> 4;
  int id = blockIdx.x;
  const int split = id % a.n_splits; id /= a.n_splits;
  const int b = id % a.B; id /= a.B;
  const int h = id % a.Hkv;
  const int l = id / a.Hkv;
  const int T = a.seq_len[b];
  const int qpos = a.q_pos ? a.q_pos[b] : T;
  const int P = a.P;
  const int mpt = 4 * (SLAT / a.G);  // pair bytes per token

  // ---- W_k[l] slice of this wave as A fragments: row r = t <-> head dim r < 16 ? 16w + r : 64 + 16w + r - 16,
  // k-slot 8hf + j of step s <-> latent coordinate 16s + 8hf + perm8(j) (the order a code dword dequantizes)
  h8 wf[SKS];
  {
    const int dim = t < 16 ? 16 * wv + t : 64 + 16 * wv + (t - 16);
    const int width = a.Hkv * SD;
    const uint16_t* W = a.wk + (size_t)l * SLAT * width + (size_t)h * SD + dim;
#pragma unroll
    for (int s = 0; s < SKS; ++s) {
      h8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = bf16_to_h(W[(size_t)(16 * s + 8 * hf + perm8(j)) * width]);
      wf[s] = f;
    }
  }
  double* tturn = (double*)(smem + LY.theta);
  if (tid < SD / 2) tturn[tid] = (a.theta > 0.0 ? pow(a.theta, -2.0 * tid / SD) : 0.0) * 0.15915494309189535;
  // this thread's query pair for the per-tile rotation: head tid / 64, pair tid % 64, scaled for exp2
  const int qh = tid >> 6, qj = tid & 63;
  float qx, qy;
  {
    const float sc = 1.4426950408889634f / sqrtf((float)SD);
    const size_t base = (((size_t)l * a.B + b) * a.Hq + h * SGQ + qh) * SD;
    if (a.q_bf16) {
      const uint16_t* q = (const uint16_t*)a.q + base;
      qx = __builtin_bit_cast(float, (uint32_t)q[qj] << 16) * sc;
      qy = __builtin_bit_cast(float, (uint32_t)q[qj + SD / 2] << 16) * sc;
    } else {
      const float* q = (const float*)a.q + base;
      qx = q[qj] * sc;
      qy = q[qj + SD / 2] * sc;
    }
  }
  const int n_st = (T + 31) / 32;
  const int st_begin = split * a.st_per_split;
  const int n_tiles = max(0, min(n_st, st_begin + a.st_per_split) - st_begin);
  int64_t* taddr = (int64_t*)(smem + LY.addr);
  for (int k = tid; k < n_tiles; k += 256) {  // page record of each super-tile, and its first slot
    const int t0 = (st_begin + k) * 32;
    const int page = a.block_table[(size_t)b * a.max_blocks + t0 / P];
    taddr[k] = a.page_off[page] + (int64_t)(t0 % P) * (SLAT / 2);
  }
  __syncthreads();
  const double fq = tturn[qj];
  // RoPE factors of this lane's slot t: up-projection entry i (0..7) is row 8(i/4) + 4hf + i%4 (< 16), paired
  // with entry i + 8 (that row + 16): frequency 16w + row; |t theta| < 32 turns, where v_sin / v_cos are accurate
  uint32_t rf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float rev = (float)(t * tturn[16 * wv + 8 * (i >> 2) + 4 * hf + (i & 3)]);
    rf[i] = pack_h2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
  }

  uint8_t* tiles = smem + LY.tile;            // tile of super-tile k: tiles + (k & 1) * 32 KiB
  _Float16* qts = (_Float16*)(smem + LY.qt);  // query of super-tile k: qts + (k & 1) * SGQ * SD
  float* sp = (float*)(smem + LY.sp);
  _Float16* pt = (_Float16*)(smem + LY.pt) + wv * 32 * SGQ;

  const int64_t meta_base = pad16((int64_t)P * SLAT / 2);

  // ---- staging: super-tile k's codes (32 x 256 bytes) and pairs (32 x mpt bytes) into ring slot k % 3.
  // Returns the number of copy instructions this wave issued.
  auto issue = [&](int k) -> int {
    const int slot0 = ((st_begin + k) * 32) % P;
    // resource based at the super-tile's codes: the codes run 8 KiB from there, its pairs start meta_base - 256 slot0
    // bytes further (within the same page record)
    const int64_t at = uniform64(taddr[k]);
    const int pairs_at = (int)meta_base - slot0 * (SLAT / 2) + slot0 * mpt;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.pool + at), (short)0, pairs_at + 32 * mpt, 0x00020000);
    uint8_t* dst = smem + LY.raw + (k & 3) * LY.raw_bytes;
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {  // codes: 8 KiB, 512 chunks; slot p = 32c + t <- token t's chunk c
      const int p0 = 256 * r + 64 * wv, p = p0 + lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 16 * p0), 16,
                                               (p & 31) * (SLAT / 2) + 16 * (p >> 5), 0, 0, 0);
      ++cnt;
    }
    const int pchunks = 2 * mpt;  // pairs: mpt / 16 chunks per token, slot 32c + t as above
    const int p0 = 64 * wv;
    if (p0 < pchunks) {  // wave-uniform
      const int p = p0 + lane;
      if (p < pchunks)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + LY.pairs_off + 16 * p0),
                                                 16, pairs_at + (p & 31) * mpt + 16 * (p >> 5), 0, 0, 0);
      ++cnt;
    }
    return cnt;
  };

  f4 acc[8];  // value latent on coordinates of steps 8w..8w+7 (16 each), rows = query heads (replicated)
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f4{0, 0, 0, 0};
  float m_ref[SGQ], psum[SGQ];
#pragma unroll
  for (int i = 0; i < SGQ; ++i) {
    m_ref[i] = 0.0f;
    psum[i] = 0.0f;
  }
  bool fresh = true;

  // super-tile k's sources of the dequantization: item i of this thread is chunk d = 2s + hf (coordinates 8d..8d+7)
  // of token tid % 32, s = tid / 64 + 4i, hf = (tid / 32) % 2; code dword d of token t sits in raw slot
  // 32 (d / 4) + t at word d % 4, pair g in pair slot 32 (g / 4) + t at word g % 4.  Then its fp16 tile, and its
  // rotated query q~ = R(q_pos - t0) q.
  const int dq_t = tid & 31, dq_d0 = 2 * (tid >> 6) + ((tid >> 5) & 1);  // d = dq_d0 + 8i
  const int lg = __builtin_ctz(a.G);                                      // G is a power of two (32 .. 512)
  auto dq_load = [&](int k, uint32_t (&xs)[8], uint32_t (&szs)[8]) {
    const uint8_t* raw = smem + LY.raw + (k & 3) * LY.raw_bytes;
    const uint8_t* xb = raw + ((dq_d0 >> 2) * 32 + dq_t) * 16 + (dq_d0 & 3) * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xs[i] = *(const uint32_t*)(xb + 1024 * i);  // d + 8 -> chunk + 2
      const int g = (8 * (dq_d0 + 8 * i)) >> lg;
      szs[i] = *(const uint32_t*)(raw + LY.pairs_off + ((g >> 2) * 32 + dq_t) * 16 + (g & 3) * 4);
    }
  };
  auto dq_store = [&](int k, int i, uint32_t x, uint32_t sz) {
    *(h8*)(tiles + (k & 1) * (SKS * 64 * 16) + ((dq_d0 + 8 * i) * 32 + dq_t) * 16) = dequant_int4x8(x, sz);
  };
  auto rot_q = [&](int k) {
    double rev = (double)(qpos - (st_begin + k) * 32) * fq;
    rev -= rint(rev);
    const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
    _Float16* qt = qts + (k & 1) * SGQ * SD;
    qt[qh * SD + qj] = (_Float16)(qx * cs - qy * sn);
    qt[qh * SD + qj + SD / 2] = (_Float16)(qy * cs + qx * sn);
  };

  // prologue: super-tiles 0-2 in flight, wait for 0 and 1, dequantize 0
  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
  const int c2 = n_tiles > 2 ? issue(2) : 0;
  vmcnt_wait_s(c2);
  lds_barrier();
  if (n_tiles > 0) {
    uint32_t xs[8], szs[8];
    dq_load(0, xs, szs);
#pragma unroll
    for (int i = 0; i < 8; ++i) dq_store(0, i, xs[i], szs[i]);
    rot_q(0);
  }
  lds_barrier();
  for (int k = 0; k < n_tiles; ++k) {
    // ring slot (k + 3) % 4 held super-tile k - 1, dequantized two iterations ago
    const int c_new = (k + 3 < n_tiles) ? issue(k + 3) : 0;
    const int t0 = (st_begin + k) * 32;
    const uint8_t* tile = tiles + (k & 1) * (SKS * 64 * 16);
    const _Float16* qt = qts + (k & 1) * SGQ * SD;

    // ---- key up-projection of this wave's 32 dims for super-tile k, operands read 8 steps ahead, with the
    // dequantization of super-tile k + 1 (landed, and its tile free since the last barrier) in between; past the
    // last super-tile that work reads a stale ring slot into the unused tile
    f16v_t kp = {};
    {
      // step s: chunk (2s + hf, t)
      const uint8_t* bb = tile + (32 * hf + t) * 16;
      auto bsrc = [&](int s) { return *(const h8*)(bb + 1024 * s); };
      constexpr int PF = 8;
      h8 bq[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) bq[i] = bsrc(i);
      uint32_t xs[8], szs[8];
      dq_load(k + 1, xs, szs);
      // scheduling fences keep each read PF steps ahead of its product and the dequantization spread over
      // the matrix instructions (the scheduler would otherwise sink the reads next to their uses)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < SKS; ++s) {
        kp = mfma32s(wf[s], bq[s % PF], kp);
        if (s + PF < SKS) bq[s % PF] = bsrc(s + PF);
        if ((s & 3) == 3) dq_store(k + 1, s >> 2, xs[s >> 2], szs[s >> 2]);
        __builtin_amdgcn_sched_barrier(0);
      }
      rot_q(k + 1);
    }
    h8 kq0, kq1;  // score steps: k-slot 8hf + j <-> pair 8(j/4) + 4hf + j%4 of the wave, x (step 0) and y (step 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const h2 r = as_h2(rope_pair(pack_h2(kp[i], kp[i + 8]), rf[i]));
      kq0[i] = r.x;
      kq1[i] = r.y;
    }
    const _Float16* qrow = qt + (t & 3) * SD + 16 * wv + 4 * hf;
    h8 qf0, qf1;
    {
      const h4 a0 = *(const h4*)qrow, a1 = *(const h4*)(qrow + 8);
      const h4 b0 = *(const h4*)(qrow + SD / 2), b1 = *(const h4*)(qrow + SD / 2 + 8);
      qf0 = h8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      qf1 = h8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
    const f16v_t sc = mfma32s(qf1, kq1, mfma32s(qf0, kq0, f16v_t{}));
    if (hf == 0) *(f4*)(sp + (wv * 32 + t) * SGQ) = f4{sc[0], sc[1], sc[2], sc[3]};
    lds_barrier();

    // ---- scores of the four heads for token t (the same in every wave), lazy online softmax
    float s4[SGQ];
    {
      f4 tot = *(const f4*)(sp + t * SGQ);
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) tot += *(const f4*)(sp + (w2 * 32 + t) * SGQ);
#pragma unroll
      for (int i = 0; i < SGQ; ++i) s4[i] = (t0 + t < T) ? tot[i] - m_ref[i] : -INFINITY;
    }
    const float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
    if (fresh || __builtin_amdgcn_ballot_w64(mx > STAU) != 0) {
      float alpha[SGQ];
#pragma unroll
      for (int i = 0; i < SGQ; ++i) {
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
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] *= alpha[i];
      fresh = false;
    }
    float p[SGQ];
#pragma unroll
    for (int i = 0; i < SGQ; ++i) {
      p[i] = __builtin_amdgcn_exp2f(s4[i]);
      psum[i] += p[i];
    }
    if (hf == 0) *(h4*)(pt + SGQ * t) = h4{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    // P as the A operand of the 16x16x32 value product: row l % 16 <-> head l % 4, k-slot 8g + j <-> token 8g + j
    // (g = l / 16); lane rho of its group points at the row of token 8g + 4v + rho / 4
    const h8 pop = lds_tr8s(pt + SGQ * (8 * grp + (rho >> 2)), pt + SGQ * (8 * grp + 4 + (rho >> 2)));
    // value latent on this wave's coordinates: step s = 8w + nt covers 16 coordinates; column n <-> coordinate
    // 16s + 8(n/8) + perm8(n%8), read token-major from the fp16 tile (4 columns of one token per lane pointer)
    {
      // step s = 8w + nt: lane rho points at the 4 columns 4(q4 % 2).. of chunk (2s + q4 / 2, 8g + 4v + rho / 4)
      const int q4 = rho & 3;
      const uint8_t* vb = tile + ((16 * wv + (q4 >> 1)) * 32 + 8 * grp + (rho >> 2)) * 16 + (q4 & 1) * 8;
      h8 vt[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) vt[nt] = lds_tr8s(vb + 1024 * nt, vb + 1024 * nt + 64);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] = mfma16x16x32(pop, vt[nt], acc[nt]);
    }
    // super-tile k + 2 landed (k + 3 may be in flight), and everyone is done with tile k before it is rewritten
    vmcnt_wait_s(c_new);
    lds_barrier();
  }

  // ---- partial: m[4], l[4] (the same in every wave), acc[4][512] (wave w: coordinates 128w..128w+127)
#pragma unroll
  for (int i = 0; i < SGQ; ++i) {
    float v = hf == 0 ? psum[i] : 0.0f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    psum[i] = v;
  }
  float* part = a.ws + ((((size_t)l * a.Hkv + h) * a.B + b) * a.n_splits + split) * a.part_stride;
  if (wv == 0 && lane < SGQ) {
    part[lane] = fresh ? -INFINITY : m_ref[lane];
    part[SGQ + lane] = psum[lane];
  }
  if (grp == 0) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int coord = 16 * (8 * wv + nt) + 8 * (rho >> 3) + perm8(rho & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) part[2 * SGQ + i * SLAT + coord] = acc[nt][i];
    }
  }
}

// out[l][b][h*4 + hq] = W_v[l][:, h*128 : (h+1)*128]^T c* / l*, over the splits' partials: one workgroup per
// (layer, sequence, query head), thread d computes output dim d (W_v rows read coalesced across the threads,
// eight independent partial sums).
__global__ __launch_bounds__(SD) void merge_shared_kernel(const float* ws, const uint16_t* wv, float* out, int B,
                                                          int Hkv, int Hq, int n_splits, int part_stride) {
  __shared__ float cst[SLAT];
  __shared__ float lst;
  int id = blockIdx.x;
  const int hq_all = id % Hq; id /= Hq;
  const int b = id % B;
  const int l = id / B;
  const int h = hq_all / SGQ, hq = hq_all % SGQ;
  const int d = threadIdx.x;
  const float* parts = ws + (((size_t)l * Hkv + h) * B + b) * n_splits * part_stride;
  float m = -INFINITY;
  for (int p = 0; p < n_splits; ++p) m = fmaxf(m, parts[(size_t)p * part_stride + hq]);
  float lsum = 0.0f, c[SLAT / SD];
#pragma unroll
  for (int k = 0; k < SLAT / SD; ++k) c[k] = 0.0f;
  for (int p = 0; p < n_splits; ++p) {
    const float* pp = parts + (size_t)p * part_stride;
    const float mp = pp[hq];
    const float w = mp == -INFINITY ? 0.0f : exp2f(mp - m);
    lsum += w * pp[SGQ + hq];
#pragma unroll
    for (int k = 0; k < SLAT / SD; ++k) c[k] += w * pp[2 * SGQ + hq * SLAT + d + SD * k];
  }
#pragma unroll
  for (int k = 0; k < SLAT / SD; ++k) cst[d + SD * k] = c[k];
  if (d == 0) lst = lsum;
  __syncthreads();
  const size_t width = (size_t)Hkv * SD;
  const uint16_t* W = wv + (size_t)l * SLAT * width + (size_t)h * SD + d;
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < SLAT; i += 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __builtin_bit_cast(float, (uint32_t)W[(size_t)(i + e) * width] << 16) * cst[i + e];
  }
  const float sum = ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
  out[(((size_t)l * B + b) * Hq + hq_all) * SD + d] = sum / lst;
}

int shared_max_tiles_per_split() { return SMAX_TILES; }

bool shared_supported(const kvc_layout& L) {
  return L.shared && L.head_dim == SD && L.r_k_cap == SLAT && L.n_q_heads == SGQ * L.n_kv_heads &&
         L.latent_bits == 4 && L.group >= 32 && L.group <= SLAT && (L.group & (L.group - 1)) == 0;
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
  const int lds = shared_lds(L.group).total;
  hipError_t e = hipFuncSetAttribute((const void*)decode_shared_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = L.n_layers * L.n_kv_heads * in.B * n_splits;
  e = mark(g_marks.begin, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_shared_kernel, dim3(grid), dim3(256), lds, st, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(g_marks.end, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_shared_kernel, dim3(L.n_layers * in.B * L.n_q_heads), dim3(SD), 0, st, a.ws, in.wv, out,
                     in.B, L.n_kv_heads, L.n_q_heads, n_splits, a.part_stride);
  return hipGetLastError();
}

}  // namespace kvc
