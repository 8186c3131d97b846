// decode_shared.hip -- decode attention over a block-shared latent (gfx950).
//
// One INT4 latent c_t (dim 512, groups of G) per token serves n_layers layers and all KV heads:
// layer l, KV head h rebuilds k = W_k[l][:, h d : (h+1) d]^T c_t (v likewise through W_v), and the
// keys are rotated (RoPE) after that up-projection.  The up-projection is the one dense contraction of
// the path (512 -> 128 per token, layer and head), so the kernel is laid out for the matrix cores.
//
// One workgroup (4 waves, one workgroup per CU so that each wave has the full register file) per
// (layer, KV head, sequence, context split).  The latent is split among the waves, not the head dims:
// wave w owns latent coordinates 128w..128w+127 and holds W_k's 128 x 128 slice for them (all head dims)
// as v_mfma_f32_32x32x16_f16 A fragments in registers.  RoPE and the scores are linear in the key, so
// each wave up-projects, rotates and scores its partial key; the four partial scores are summed through
// LDS, the one exchange (and the one barrier) per 32-token super-tile.  The value latent is accumulated
// on the same 128 coordinates, so everything else a wave touches is its own:
//   - its quarter of each super-tile's codes (64 bytes per token) and its scale/zero pairs go HBM -> LDS
//     through its own four-deep ring of buffer loads that write LDS directly, gathered chunk-major
//     (16-byte chunk c of token t at slot 32c + t, so that lanes of consecutive tokens hit different banks);
//     each wave counts and waits for its own copies only;
//   - it dequantizes its codes once, straight into the up-projection's B fragments (lane = token, k-slots =
//     8 coordinates of one code dword), one super-tile ahead, and stores the same fp16 chunks in a private
//     LDS tile for the value product;
//   - per super-tile: 32 up-projection MFMAs (4 blocks of 32 head dims x 8 steps), RoPE on the pairs
//     (j, j + 64), which sit in one lane, 8 score MFMAs into the partial scores; after the exchange every
//     wave repeats the (identical) online softmax and accumulates its 128 value coordinates with
//     v_mfma_f32_16x16x32_f16, whose token-major operands come from the private tile through transposing
//     LDS reads.
// The value up-projection W_v is applied once per (layer, sequence, head) in the merge kernel.
#include <math.h>

#include <algorithm>

#include "lds_copy.hpp"

namespace kvc {

static constexpr int SGQ = 4;           // query heads per KV head
static constexpr int SLAT = 512;        // latent dimension handled here
static constexpr int SD = 128;          // head dimension handled here
static constexpr int SQC = SLAT / 4;    // latent coordinates per wave
static constexpr int SNJ = SQC / 16;    // 16-coordinate steps per wave
static constexpr int SNB = SD / 32;     // 32-dim blocks of the head
static constexpr float STAU = 8.0f;     // lazy-max slack, log2 units
static constexpr int SRAW = 2048 + 512; // ring slot: a wave's codes of 32 tokens, then its pairs (two copies)
// a wave's fp16 tile: chunk c (8 coordinates) of token t at byte SCS c + 16 t, 16 chunks; the row of a chunk is
// padded from 512 to 576 bytes so that the transposing reads of a step (two chunks, token groups 256 bytes
// apart) hit distinct banks
static constexpr int SCS = 32 * 16 + 64;
static constexpr int SVT = 16 * SCS;

typedef float f16v_t __attribute__((ext_vector_type(16)));

struct DecodeSharedArgs {
  const uint8_t* pool;
  const int64_t* page_off;
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* q_pos;
  const void* q;
  const uint16_t* wk;
  int64_t w_stride;  // elements between sequences' W_k (0: one for all)
  const uint32_t* keep;  // token keep mask [B][keep_words] (bit t % 32 of word t / 32), or null
  int keep_words;
  float* ws;
  int q_bf16, B, Hkv, Hq, L, max_blocks, P, G, n_splits, st_per_split, part_stride;
  double theta;
};

static constexpr int SMAX_TILES = 1024;  // super-tiles per split (the page record address of each)

struct SharedLds {
  int raw, vt, qt, theta, sp, pt, addr, keep, total;
};
__host__ __device__ constexpr SharedLds shared_lds() {
  SharedLds L{};
  int o = 0;
  L.raw = o; o += 4 * 4 * SRAW;                 // per wave: staging ring of 4 super-tiles
  L.vt = o; o += 4 * 2 * SVT;                   // per wave: fp16 value tiles, x 2
  L.qt = o; o += 3 * SGQ * SD * 2;              // rotated query in fragment order, fp16, x 3
  L.theta = o; o += (SD / 2) * 8;               // RoPE frequencies, turns per position
  L.sp = o; o += 2 * 4 * 32 * SGQ * 4;          // partial scores [buffer][wave][token][head], x 2
  L.pt = o; o += 4 * 32 * SGQ * 2;              // probabilities [wave][token][head] fp16
  L.addr = o; o += SMAX_TILES * 8;              // page record address of each super-tile
  L.keep = o; o += SMAX_TILES * 4;              // keep-mask word of each super-tile
  L.total = o;
  return L;
}

__device__ inline f16v_t mfma32s(h8 a, h8 b, f16v_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }

// fragment order of the rotated query: element e of (head, block g, step st, lane half hf) is head dim
// 64 (e % 2) + 16 g + 8 st + 4 hf + e / 2, the k-slot order of the rotated keys of block g (each RoPE pair's
// x and y side by side)
__device__ inline int qfrag_index(int head, int dim) {
  const int xy = dim >> 6, r = dim & 63, g = r >> 4, rem = r & 15;
  const int st = rem >> 3, hf = (rem >> 2) & 1, e = 2 * (rem & 3) + xy;
  return (((head * SNB + g) * 2 + st) * 2 + hf) * 8 + e;
}

// KEEP: a token keep mask is applied (a separate instantiation, so that the unmasked kernel carries none of it).
// SPLIT: latent coordinates below SLAT / 2 feed only the keys and the rest only the values (W_k zero on the upper
// rows, W_v on the lower, as for keys and values with their own token factors): waves 0-1 then do only the key
// work and waves 2-3 only the value product; their skipped products are exact zeros, so the output is the same.
template <bool KEEP, bool SPLIT>
__global__ __launch_bounds__(256, 1) void decode_shared_kernel(DecodeSharedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr SharedLds LY = shared_lds();
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
  const int mpt = 4 * (SLAT / a.G);             // pair bytes per token
  const int lg = __builtin_ctz(a.G);            // G is a power of two (32 .. 512)
  const int npw = max(1, SQC >> lg);            // pairs per token over this wave's coordinates (1, 2 or 4)
  const int g0 = (SQC * wv) >> lg;              // the first of them

  // ---- W_k[l] slice of this wave as A fragments.  Block g: row r = t <-> head dim r < 16 ? 16g + r :
  // 64 + 16g + r - 16; step j: k-slot 8hf + e <-> latent coordinate 128w + 8 (8hf + j) + perm8(e), i.e.
  // element e of code dword 8hf + j of the wave's 64 code bytes (the order a code dword dequantizes).
  h8 wf[SNB][SNJ];
  if (!SPLIT || wv < 2) {
    const int width = a.Hkv * SD;
    const uint16_t* W = a.wk + (size_t)b * a.w_stride + (size_t)l * SLAT * width + (size_t)h * SD;
#pragma unroll
    for (int g = 0; g < SNB; ++g) {
      const int dim = t < 16 ? 16 * g + t : 64 + 16 * g + (t - 16);
#pragma unroll
      for (int j = 0; j < SNJ; ++j) {
        h8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          f[e] = bf16_to_h(W[(size_t)(SQC * wv + 8 * (8 * hf + j) + perm8(e)) * width + dim]);
        // the fragments stay in the accumulator registers (the matrix instructions read their A operand from
        // there directly; the vector registers are needed for the rest)
        asm volatile("" : "=a"(wf[g][j]) : "0"(f));
      }
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
  const int qix = qfrag_index(qh, qj), qiy = qfrag_index(qh, qj + SD / 2);
  const int n_st = (T + 31) / 32;
  const int st_begin = split * a.st_per_split;
  const int n_tiles = max(0, min(n_st, st_begin + a.st_per_split) - st_begin);
  int64_t* taddr = (int64_t*)(smem + LY.addr);
  uint32_t* tkeep = (uint32_t*)(smem + LY.keep);
  for (int k = tid; k < n_tiles; k += 256) {  // page record of each super-tile, its first slot, its keep word
    const int t0 = (st_begin + k) * 32;
    const int page = a.block_table[(size_t)b * a.max_blocks + t0 / P];
    taddr[k] = a.page_off[page] + (int64_t)(t0 % P) * (SLAT / 2);
    const int wd = t0 >> 5;
    if (KEEP) tkeep[k] = wd < a.keep_words ? a.keep[(size_t)b * a.keep_words + wd] : 0u;
  }
  __syncthreads();
  const double fq = tturn[qj];
  // RoPE factors of this lane's slot t: block g's up-projection entry i (0..7) is row 8(i/4) + 4hf + i%4 (< 16),
  // paired with entry i + 8 (that row + 16): frequency 16g + row; |t theta| < 32 turns, where v_sin / v_cos are
  // accurate
  uint32_t rf[SNB][8];
#pragma unroll
  for (int g = 0; g < SNB; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float rev = (float)(t * tturn[16 * g + 8 * (i >> 2) + 4 * hf + (i & 3)]);
      rf[g][i] = pack_h2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
    }

  uint8_t* raw_w = smem + LY.raw + wv * 4 * SRAW;  // this wave's ring; super-tile k in slot k % 4
  const uint32_t raw_lds = __builtin_amdgcn_readfirstlane(lds_addr(raw_w));
  uint8_t* vt_w = smem + LY.vt + wv * 2 * SVT;     // this wave's fp16 tiles; super-tile k in k % 2
  _Float16* qts = (_Float16*)(smem + LY.qt);       // rotated query of super-tile k: qts + (k % 3) * SGQ * SD
  float* sp = (float*)(smem + LY.sp);
  _Float16* pt = (_Float16*)(smem + LY.pt) + wv * 32 * SGQ;

  const int64_t meta_base = pad16((int64_t)P * SLAT / 2);

  // ---- staging: this wave's part of super-tile k into ring slot k % 4; past the last super-tile the slot gets a
  // copy of the last one, which keeps the number of copies in flight constant.  Always four copy instructions:
  //   codes: 32 tokens x 4 chunks (bytes 64w + 16c .. of each token), slot p = 32c + t <- token t's chunk c;
  //   pairs: dword 4 t + i <- pair g0 + (i mod npw) of token t, i < 4 (two instructions, 16 tokens each).
  auto issue = [&](int k) {
    const int kk = min(k, n_tiles - 1);
    const int slot0 = ((st_begin + kk) * 32) % P;
    // resource based at the super-tile's codes: its pairs start meta_base - 256 slot0 bytes further (within the
    // same page record)
    const int64_t at = uniform64(taddr[kk]);
    const int pairs_at = (int)meta_base - slot0 * (SLAT / 2) + slot0 * mpt;
    const i32x4_t rs = buffer_rsrc(a.pool + at, pairs_at + 32 * mpt);
    const uint32_t dst = raw_lds + (k & 3) * SRAW;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int p = 64 * r + lane;
      copy16_to_lds(rs, dst + 1024 * r, (p & 31) * (SLAT / 2) + 64 * wv + 16 * (p >> 5));
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = 64 * r + lane, tok = q >> 2, i = q & 3;
      copy4_to_lds(rs, dst + 2048 + 256 * r, pairs_at + tok * mpt + 4 * (g0 + (i & (npw - 1))));
    }
  };

  f4 acc[SNJ];  // value latent on this wave's coordinates, 16 per step, rows = query heads (replicated)
#pragma unroll
  for (int i = 0; i < SNJ; ++i) acc[i] = f4{0, 0, 0, 0};
  float m_ref[SGQ], psum[SGQ];
#pragma unroll
  for (int i = 0; i < SGQ; ++i) {
    m_ref[i] = 0.0f;
    psum[i] = 0.0f;
  }
  bool fresh = true;
  // ---- super-tile k (ring slot k % 4) dequantized into the B fragments bf (lane = token t, step j: code dword
  // 8hf + j of the wave's part, the k-slot order of wf) and into fp16 tile vb: chunk c (code dword c, 8
  // coordinates) of token t at byte SCS c + 16 t
  const int gr0 = ((SQC * wv + 64 * hf) >> lg) - g0, gr1 = ((SQC * wv + 64 * hf + 32) >> lg) - g0;
  auto dequant = [&](int k, h8 (&bf)[SNJ], int vb) {
    const uint8_t* raw = raw_w + (k & 3) * SRAW;
    // (dword reads: the compiler merges them, and unlike a vector read of this copy target it then adds no wait
    // for every copy in flight)
    const uint32_t* c0 = (const uint32_t*)(raw + (64 * hf + t) * 16);       // chunk 2hf: dwords 8hf + 0..3
    const uint32_t* c1 = (const uint32_t*)(raw + (64 * hf + 32 + t) * 16);  // chunk 2hf + 1: dwords 8hf + 4..7
    const uint32_t z0 = *(const uint32_t*)(raw + 2048 + 4 * (4 * t + gr0));
    const uint32_t z1 = *(const uint32_t*)(raw + 2048 + 4 * (4 * t + gr1));
    uint8_t* dst = vt_w + vb * SVT + SCS * 8 * hf + 16 * t;
    const uint32_t xs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
    for (int j = 0; j < SNJ; ++j) {
      bf[j] = dequant_int4x8(xs[j], j < 4 ? z0 : z1);
      *(h8*)(dst + SCS * j) = bf[j];
    }
  };
  // rotated query q~ = R(q_pos - t0) q of super-tile k into buffer k % 3, in fragment order
  auto rot_q = [&](int k) {
    double rev = (double)(qpos - (st_begin + k) * 32) * fq;
    rev -= rint(rev);
    const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
    _Float16* qt = qts + (k % 3) * SGQ * SD;
    qt[qix] = (_Float16)(qx * cs - qy * sn);
    qt[qiy] = (_Float16)(qy * cs + qx * sn);
  };

  // One super-tile: bc holds its B fragments (its fp16 tile is buffer k % 2); the next super-tile is dequantized
  // into bn on the way.
  auto step = [&](int k, h8 (&bc)[SNJ], h8 (&bn)[SNJ]) {
    issue(k + 4);  // ring slot k % 4 held super-tile k, dequantized in the previous step
    const int t0 = (st_begin + k) * 32;
    // super-tile k + 1 landed: the copies of k + 2 .. k + 4 (four each) may still be in flight
    __builtin_amdgcn_s_waitcnt(0x0F70 | 12);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    // sources of super-tile k + 1's dequantization (dword reads: see dequant)
    const uint8_t* rawn = raw_w + ((k + 1) & 3) * SRAW;
    const uint32_t* c0 = (const uint32_t*)(rawn + (64 * hf + t) * 16);
    const uint32_t* c1 = (const uint32_t*)(rawn + (64 * hf + 32 + t) * 16);
    const uint32_t xs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const uint32_t z0 = *(const uint32_t*)(rawn + 2048 + 4 * (4 * t + gr0));
    const uint32_t z1 = *(const uint32_t*)(rawn + 2048 + 4 * (4 * t + gr1));
    uint8_t* vdst = vt_w + ((k + 1) & 1) * SVT + SCS * 8 * hf + 16 * t;

    // ---- partial keys over this wave's coordinates (block by block), RoPE, partial scores of the four heads.
    // The instruction stream interleaves each block's matrix instructions with vector work that does not wait
    // for them (two chunks of the next super-tile's dequantization, the previous block's RoPE), so that one
    // wave keeps both units busy.
    const h8* qf = (const h8*)(qts + (k % 3) * SGQ * SD) + (t & 3) * (SNB * 4) + hf;
    f16v_t sc = {};
    // a super-tile whose tokens are all evicted contributes nothing: only the next one's dequantization runs
    const bool empty = KEEP && tkeep[k] == 0u;
    if (SPLIT && wv >= 2) {  // value waves: only the next super-tile's value tile
#pragma unroll
      for (int jj = 0; jj < SNJ; ++jj) *(h8*)(vdst + SCS * jj) = dequant_int4x8(xs[jj], jj < 4 ? z0 : z1);
    } else if (empty) {
#pragma unroll
      for (int jj = 0; jj < SNJ; ++jj) {
        bn[jj] = dequant_int4x8(xs[jj], jj < 4 ? z0 : z1);
        if (!SPLIT) *(h8*)(vdst + SCS * jj) = bn[jj];
      }
    } else {
    f16v_t kp[SNB];
#pragma unroll
    for (int g = 0; g <= SNB; ++g) {
      if (g < SNB) {
        kp[g] = f16v_t{};
#pragma unroll
        for (int j = 0; j < SNJ; ++j) kp[g] = mfma32s(wf[g][j], bc[j], kp[g]);
#pragma unroll
        for (int jj = 2 * g; jj < 2 * g + 2; ++jj) {
          bn[jj] = dequant_int4x8(xs[jj], jj < 4 ? z0 : z1);
          if (!SPLIT) *(h8*)(vdst + SCS * jj) = bn[jj];  // key waves of a split latent make no value product
        }
      }
      if (g > 0) {
        // rotated pairs (x, y) of rows 8st + 4hf + m, m < 4, are the k-slots 8hf + 2m, 2m + 1 of score step st
        u32x4_t kr[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) kr[i >> 2][i & 3] = rope_pair(pack_h2(kp[g - 1][i], kp[g - 1][i + 8]), rf[g - 1][i]);
        sc = mfma32s(qf[4 * (g - 1)], __builtin_bit_cast(h8, kr[0]), sc);
        sc = mfma32s(qf[4 * (g - 1) + 2], __builtin_bit_cast(h8, kr[1]), sc);
      }
    }
#pragma unroll
    for (int g = 0; g < SNB; ++g) {
#pragma unroll
      for (int j = 0; j < SNJ; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // then up to five vector instructions
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // the previous block's score products
    }
    }
    float* spb = sp + (k & 1) * (4 * 32 * SGQ);
    if (hf == 0) *(f4*)(spb + (wv * 32 + t) * SGQ) = f4{sc[0], sc[1], sc[2], sc[3]};
    lds_barrier();
    rot_q(k + 2);  // buffer (k + 2) % 3 was last read before the previous barrier

    // ---- scores of the four heads for token t (the same in every wave), lazy online softmax
    float s4[SGQ];
    {
      f4 tot = *(const f4*)(spb + t * SGQ);
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) tot += *(const f4*)(spb + (w2 * 32 + t) * SGQ);
      const bool kept = t0 + t < T && (!KEEP || ((tkeep[k] >> t) & 1u));  // past the end or evicted: no weight
#pragma unroll
      for (int i = 0; i < SGQ; ++i) s4[i] = kept ? tot[i] - m_ref[i] : -INFINITY;
    }
    const float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
    // the first super-tile with a kept token sets the reference maximum; one with none (possible under a keep
    // mask only) leaves it unset
    if (KEEP ? __builtin_amdgcn_ballot_w64(fresh ? mx > -INFINITY : mx > STAU) != 0
             : fresh || __builtin_amdgcn_ballot_w64(mx > STAU) != 0) {
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
      for (int nt = 0; nt < SNJ; ++nt)
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
    wave_lds_sync();
    // P as the A operand of the 16x16x32 value product: row l % 16 <-> head l % 4, k-slot 8g + j <-> token 8g + j
    // (g = l / 16); lane rho of its group points at the row of token 8g + 4v + rho / 4
    // value latent: step nt covers chunks 2nt, 2nt + 1; column n <-> coordinate 128w + 16nt + 8(n/8) + perm8(n%8);
    // lane rho points at the 4 columns 4(q4 % 2).. of chunk (2nt + q4 / 2, token 8g + 4v + rho / 4)
    if ((!SPLIT || wv >= 2) && !empty) {
      const h8 pop = lds_tr8s(pt + SGQ * (8 * grp + (rho >> 2)), pt + SGQ * (8 * grp + 4 + (rho >> 2)));
      const int q4 = rho & 3;
      const uint8_t* vb = vt_w + (k & 1) * SVT + SCS * (q4 >> 1) + (8 * grp + (rho >> 2)) * 16 + (q4 & 1) * 8;
      h8 vt[SNJ];
#pragma unroll
      for (int nt = 0; nt < SNJ; ++nt) vt[nt] = lds_tr8s(vb + 2 * SCS * nt, vb + 2 * SCS * nt + 64);
#pragma unroll
      for (int nt = 0; nt < SNJ; ++nt) acc[nt] = mfma16x16x32(pop, vt[nt], acc[nt]);
    }
  };

  if (n_tiles > 0) {
    // prologue: super-tiles 0-3 in flight, wait for 0, dequantize it; rotated queries of 0 and 1
#pragma unroll
    for (int j = 0; j < 4; ++j) issue(j);
    __builtin_amdgcn_s_waitcnt(0x0F70 | 12);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    h8 ba[SNJ], bb[SNJ];
    dequant(0, ba, 0);
    rot_q(0);
    rot_q(1);
    lds_barrier();
    int k = 0;
    for (; k + 1 < n_tiles; k += 2) {
      step(k, ba, bb);
      step(k + 1, bb, ba);
    }
    if (k < n_tiles) step(k, ba, bb);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the copies past the end land before the workgroup exits
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
    for (int nt = 0; nt < SNJ; ++nt) {
      const int coord = SQC * wv + 16 * nt + 8 * (rho >> 3) + perm8(rho & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) part[2 * SGQ + i * SLAT + coord] = acc[nt][i];
    }
  }
}

// out[l][b][h*4 + hq] = W_v[l][:, h*128 : (h+1)*128]^T c* / l*, over the splits' partials: one workgroup per
// (layer, sequence, query head), thread d computes output dim d (W_v rows read coalesced across the threads,
// eight independent partial sums).
__global__ __launch_bounds__(SD) void merge_shared_kernel(const float* ws, const uint16_t* wv, int64_t w_stride,
                                                          float* out, int B, int Hkv, int Hq, int n_splits,
                                                          int part_stride, int c_begin) {
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
  const uint16_t* W = wv + (size_t)b * w_stride + (size_t)l * SLAT * width + (size_t)h * SD + d;
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = c_begin; i < SLAT; i += 8) {  // (a split latent: W_v is zero below c_begin)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __builtin_bit_cast(float, (uint32_t)W[(size_t)(i + e) * width] << 16) * cst[i + e];
  }
  const float sum = ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
  out[(((size_t)l * B + b) * Hq + hq_all) * SD + d] = lst > 0.0f ? sum / lst : 0.0f;  // zero: no token kept
}

int shared_max_tiles_per_split() { return SMAX_TILES; }

bool shared_supported(const kvc_layout& L) {
  return L.shared && L.head_dim == SD && L.r_k_cap == SLAT && L.n_q_heads == SGQ * L.n_kv_heads &&
         lat_bits_k(L) == 4 && lat_bits_v(L) == 4 && L.group >= 32 && L.group <= SLAT && (L.group & (L.group - 1)) == 0;
}

size_t shared_ws_bytes(const kvc_layout& L, int B, int n_splits) {
  return (size_t)L.n_layers * L.n_kv_heads * B * n_splits * (2 * SGQ + SGQ * SLAT) * sizeof(float);
}

hipError_t launch_decode_shared(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out,
                                void* ws, int n_splits, int st_per_split, hipStream_t st) {
  DecodeSharedArgs a;
  a.pool = C.pool; a.page_off = C.page_off; a.block_table = in.block_table; a.seq_len = in.seq_len;
  a.q_pos = in.q_pos; a.q = in.q; a.wk = in.wk; a.w_stride = in.w_seq_stride; a.ws = (float*)ws;
  a.keep = in.keep_mask; a.keep_words = in.keep_words;
  a.q_bf16 = in.q_dtype == KVC_BF16;
  a.B = in.B; a.Hkv = L.n_kv_heads; a.Hq = L.n_q_heads; a.L = L.n_layers; a.max_blocks = in.max_blocks;
  a.P = L.page_size; a.G = L.group; a.n_splits = n_splits; a.st_per_split = st_per_split;
  a.part_stride = 2 * SGQ + SGQ * SLAT; a.theta = L.rope_theta;
  const int lds = shared_lds().total;
  const bool split = in.kv_split == SLAT / 2;
  const void* kern = in.keep_mask ? (split ? (const void*)decode_shared_kernel<true, true>
                                           : (const void*)decode_shared_kernel<true, false>)
                                  : (split ? (const void*)decode_shared_kernel<false, true>
                                           : (const void*)decode_shared_kernel<false, false>);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = L.n_layers * L.n_kv_heads * in.B * n_splits;
  e = mark(g_marks.begin, st);
  if (e != hipSuccess) return e;
  if (in.keep_mask && split)
    hipLaunchKernelGGL((decode_shared_kernel<true, true>), dim3(grid), dim3(256), lds, st, a);
  else if (in.keep_mask)
    hipLaunchKernelGGL((decode_shared_kernel<true, false>), dim3(grid), dim3(256), lds, st, a);
  else if (split)
    hipLaunchKernelGGL((decode_shared_kernel<false, true>), dim3(grid), dim3(256), lds, st, a);
  else
    hipLaunchKernelGGL((decode_shared_kernel<false, false>), dim3(grid), dim3(256), lds, st, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(g_marks.end, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_shared_kernel, dim3(L.n_layers * in.B * L.n_q_heads), dim3(SD), 0, st, a.ws, in.wv,
                     in.w_seq_stride, out, in.B, L.n_kv_heads, L.n_q_heads, n_splits, a.part_stride,
                     split ? SLAT / 2 : 0);
  return hipGetLastError();
}

}  // namespace kvc
