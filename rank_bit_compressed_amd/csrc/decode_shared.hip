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
//
// Two kernels use this layout: decode_shared_role_kernel (further below: 8 waves, key waves and value waves on
// each SIMD) serves the plain, keep-mask, split-latent and positions modes at every code width;
// decode_shared_res_kernel (one wave per SIMD, as described above) the residual mode, whose residual operands do
// not fit the registers of the role split.  The role split's key waves use 16x16x32 products instead of the
// 32x32x16 ones above (the same sums in another order).
#include <math.h>

#include <algorithm>

#include "lds_copy.hpp"
#include "res_codes.hpp"

namespace kvc {

static constexpr int SGQ = 4;           // query heads per KV head
static constexpr int SLAT = 512;        // latent dimension handled here
static constexpr int SD = 128;          // head dimension handled here
static constexpr int SQC = SLAT / 4;    // latent coordinates per wave
static constexpr int SNJ = SQC / 16;    // 16-coordinate steps per wave
static constexpr int SNB = SD / 32;     // 32-dim blocks of the head
static constexpr float STAU = 8.0f;     // lazy-max slack, log2 units
static constexpr int SRAW = 2048 + 512; // ring slot: a wave's codes of 32 tokens, then its pairs (two copies)
static constexpr int SVAR = 4;          // positions mode: query bases per super-tile (blocks of 32 positions)
static constexpr int RT16 = 20;         // positions mode: dwords per row of the role kernel's RoPE factor table
static constexpr int SRR = 2048 + 128;  // residual mode: a super-tile's K and V residual codes, then their scales
static constexpr int SRRN = 6;          // residual mode: super-tiles in the shared residual ring
static constexpr int SRCS = 32 * 16 + 64;  // residual mode: bytes per chunk row of a value-residual tile (padded)
static constexpr int SQB = SD + 8;      // fp16 per rotated query head (and variant) in LDS: 256 bytes + 16 of padding,
                                        // so that the score operand reads of 16 heads x variants hit distinct banks
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
  const int32_t* tok_pos;  // positions mode: source position of each slot [B][pos_row], -1 for none
  int pos_row;
  int64_t lat_bytes;  // residual mode: bytes of a record's latent sections
  int rec_bytes;      // residual mode: bytes of a record
  float* ws;
  int q_bf16, B, Hkv, Hq, L, max_blocks, P, G, n_splits, st_per_split, part_stride;
  double theta;
};

static constexpr int SMAX_TILES = 1024;  // super-tiles per split (the page record address of each)

struct SharedLds {
  int raw, vt, qt, theta, sp, pt, addr, rres, vres, pt2, total;
};
// the LDS of the one-wave-per-SIMD kernel (the residual mode)
__host__ __device__ constexpr SharedLds shared_lds() {
  SharedLds L{};
  int o = 0;
  L.raw = o; o += 4 * 4 * SRAW;          // per wave: staging ring of 4 super-tiles
  L.vt = o; o += 4 * 2 * SVT;            // per wave: fp16 value tiles, x 2
  L.qt = o; o += 3 * SGQ * SQB * 2;      // rotated query in fragment order, fp16, x 3
  L.theta = o; o += (SD / 2) * 8;        // RoPE frequencies, turns per position
  L.sp = o; o += 2 * 4 * 32 * SGQ * 4;   // partial scores [buffer][wave][token][head], x 2
  L.pt = o; o += 4 * 32 * SGQ * 2;       // probabilities [wave][token][head] fp16
  L.addr = o; o += SMAX_TILES * 8;       // page record address of each super-tile
  L.rres = o; o += SRRN * SRR;           // ring of the super-tiles' residuals
  L.vres = o; o += 16 * SRCS;            // the waves' fp16 value-residual tiles, 16 chunks in all
  L.pt2 = o; o += 4 * 32 * SGQ * 2;      // [wave][token][head] p * value scale
  L.total = o;
  return L;
}

__device__ inline f16v_t mfma32s(h8 a, h8 b, f16v_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }

// fragment order of the rotated query: element e of (head, block g, step st, lane half hf) is head dim
// 64 (e % 2) + 16 g + 8 st + 4 hf + e / 2, the k-slot order of the rotated keys of block g (each RoPE pair's
// x and y side by side); heads SQB elements apart
__device__ inline int qfrag_index(int head, int dim) {
  const int xy = dim >> 6, r = dim & 63, g = r >> 4, rem = r & 15;
  const int st = rem >> 3, hf = (rem >> 2) & 1, e = 2 * (rem & 3) + xy;
  return head * SQB + ((g * 2 + st) * 2 + hf) * 8 + e;
}

// The residual mode: the rotated 2-bit residual of each (layer, head) on top of the INT4 latent (no keep mask, no
// positions; a split latent runs this plain-latent form, whose extra products are then exact zeros).  Waves 0-2
// each stage one more part of every super-tile (the (layer, head)'s K residual codes, V residual codes, both scale
// rows) into a ring every wave reads after the next score barrier.  Keys: wave w adds
// K_res = (s / sqrt(128)) (H' c - 192 [d = 0]) of head-dim block w (the fp8 matrix instruction with the +-1
// Hadamard, as in the per-head residual kernel) to its partial keys before RoPE.  Values: wave w accumulates
// sum_t p_t s_t (2c - 3) / (2 sqrt(128)) on rotated coordinates 32w .. 32w + 31; the merge applies H'.
__global__ __launch_bounds__(256, 1) void decode_shared_res_kernel(DecodeSharedArgs a) {
  constexpr int CB = SLAT / 2;  // code bytes per token (INT4)
  constexpr int QB = CB / 4;    // a wave's quarter of them
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr SharedLds LY = shared_lds();
  constexpr int RST = 2;        // 16-coordinate steps of the wave's 32 rotated value-residual coordinates
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
  {
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
  // +-1 Hadamard rows of this wave's head-dim block (block w) as fp8 A fragments (row t <-> the block's head dim,
  // byte b of lane half hf's 32 of product be <-> coordinate 64 hf + 32 be + res8_coord(0, b): a lane half reads
  // its token's residual code dwords 4hf..4hf+3 with one 16-byte read, and product be takes dwords 2be, 2be + 1 of
  // them; e4m3 +1 = 0x38, -1 = 0xB8), kept in the accumulator registers the fp8 products read directly
  v8i_t hr[2];
  {
    const int dim = t < 16 ? 16 * wv + t : 64 + 16 * wv + (t - 16);
#pragma unroll
    for (int be = 0; be < 2; ++be) {
#pragma unroll
      for (int o = 0; o < 8; ++o) {
        uint32_t w = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 64 * hf + 32 * be + res8_coord(0, 4 * o + q);
          w |= ((__builtin_popcount(dim & i) & 1) ? 0xB8u : 0x38u) << (8 * q);
        }
        hr[be][o] = (int)w;
      }
      asm volatile("" : "=a"(hr[be]) : "0"(hr[be]));
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
  const int qix = qfrag_index(qh, qj);
  const int n_st = (T + 31) / 32;
  const int st_begin = split * a.st_per_split;
  const int n_tiles = max(0, min(n_st, st_begin + a.st_per_split) - st_begin);
  int64_t* taddr = (int64_t*)(smem + LY.addr);
  for (int k = tid; k < n_tiles; k += 256) {  // page record of each super-tile (at its first slot)
    const int t0 = (st_begin + k) * 32;
    const int page = a.block_table[(size_t)b * a.max_blocks + t0 / P];
    taddr[k] = a.page_off[page] + (int64_t)(t0 % P) * CB;
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
  _Float16* qts = (_Float16*)(smem + LY.qt);       // rotated query of super-tile k: buffer k % 3 (see rot_q)
  float* sp = (float*)(smem + LY.sp);
  _Float16* pt = (_Float16*)(smem + LY.pt) + wv * 32 * SGQ;
  const uint8_t* rres = smem + LY.rres;  // super-tile k's residual at rres + (k % SRRN) * SRR
  const uint32_t rres_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem + LY.rres));
  uint8_t* vr_w = smem + LY.vres + wv * 4 * SRCS;  // this wave's value-residual tile (4 chunk rows)
  _Float16* pt2 = (_Float16*)(smem + LY.pt2) + wv * 32 * SGQ;
  constexpr float RSCALE = 0.04419417382415922f;  // 1 / (2 sqrt(128))

  const int64_t meta_base = pad16((int64_t)P * CB);

  // ---- staging: this wave's part of super-tile k into ring slot k % 4; past the last super-tile the slot gets a
  // copy of the last one, which keeps the number of copies in flight constant.  Four copy instructions, and a
  // fifth for waves 0-2 (the residual):
  //   codes: 32 tokens x 4 chunks (bytes 64w + 16c .. of each token), slot p = 32c + t <- token t's chunk c;
  //   pairs: dword 4 t + i <- pair g0 + (i mod npw) of token t, i < 4 (two instructions, 16 tokens each);
  //   residual: wave 0 the K codes, wave 1 the V codes (32 bytes per token), wave 2 both scale rows.
  auto issue = [&](int k) {
    const int kk = min(k, n_tiles - 1);
    const int slot0 = ((st_begin + kk) * 32) % P;
    // resource based at the super-tile's codes: its pairs start meta_base - 256 slot0 bytes further (within the
    // same page record)
    const int64_t at = uniform64(taddr[kk]);
    const int pairs_at = (int)meta_base - slot0 * CB + slot0 * mpt;
    const i32x4_t rs = buffer_rsrc(a.pool + at, pairs_at + 32 * mpt);
    const uint32_t dst = raw_lds + (k & 3) * SRAW;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int p = 64 * r + lane;
      copy16_to_lds(rs, dst + 1024 * r, (p & 31) * CB + QB * wv + 16 * (p >> 5));
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = 64 * r + lane, tok = q >> 2, i = q & 3;
      copy4_to_lds(rs, dst + 2048 + 256 * r, pairs_at + tok * mpt + 4 * (g0 + (i & (npw - 1))));
    }
    if (wv < 3) {  // the super-tile's residual of this (layer, head): K codes, V codes, both scales
      const i32x4_t rr = buffer_rsrc(a.pool + (at - (int64_t)slot0 * CB), a.rec_bytes);
      const uint32_t rdst = rres_lds + (k % SRRN) * SRR;
      const int n = a.L * a.Hkv, idx = l * a.Hkv + h;
      if (wv < 2)
        copy16_to_lds(rr, rdst + 1024 * wv, (int)shared_res_part(a.lat_bytes, P, SD, n, wv, idx) + 32 * slot0 +
                                                16 * lane);
      else if (lane < 32)
        copy4_to_lds(rr, rdst + 2048, (int)shared_res_part(a.lat_bytes, P, SD, n, 2 + (lane >> 4), idx) +
                                          2 * slot0 + 4 * (lane & 15));
    }
  };

  f4 acc[SNJ];  // value latent on this wave's coordinates, 16 per step, rows = query heads (replicated)
#pragma unroll
  for (int i = 0; i < SNJ; ++i) acc[i] = f4{0, 0, 0, 0};
  f4 accr[RST];  // the rotated value residual on this wave's coordinates
#pragma unroll
  for (int i = 0; i < RST; ++i) accr[i] = f4{0, 0, 0, 0};
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
  // the lane's eight code groups of a staged super-tile as INT4 dwords: group j = coordinates 8 (8hf + j)..
  // of the wave's quarter of token t.  (Dword reads: the compiler merges them, and unlike a vector read of this
  // copy target it then adds no wait for every copy in flight.)
  auto code_words = [&](const uint8_t* raw, uint32_t (&xs)[8]) {
    const uint32_t* c0 = (const uint32_t*)(raw + (64 * hf + t) * 16);       // chunk 2hf: dwords 8hf + 0..3
    const uint32_t* c1 = (const uint32_t*)(raw + (64 * hf + 32 + t) * 16);  // chunk 2hf + 1: dwords 8hf + 4..7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[j] = c0[j];
      xs[4 + j] = c1[j];
    }
  };
  auto dequant = [&](int k, h8 (&bf)[SNJ], int vb) {
    const uint8_t* raw = raw_w + (k & 3) * SRAW;
    const uint32_t z0 = *(const uint32_t*)(raw + 2048 + 4 * (4 * t + gr0));
    const uint32_t z1 = *(const uint32_t*)(raw + 2048 + 4 * (4 * t + gr1));
    uint8_t* dst = vt_w + vb * SVT + SCS * 8 * hf + 16 * t;
    uint32_t xs[8];
    code_words(raw, xs);
#pragma unroll
    for (int j = 0; j < SNJ; ++j) {
      bf[j] = dequant_int4x8(xs[j], j < 4 ? z0 : z1);
      *(h8*)(dst + SCS * j) = bf[j];
    }
  };
  // rotated query q~ = R(q_pos - t0) q of super-tile k into buffer k % 3, in fragment order.  A pair's x and y are
  // adjacent elements (qiy = qix + 1).
  auto rot_q = [&](int k) {
    const double t0 = (double)((st_begin + k) * 32);
    double rev = ((double)qpos - t0) * fq;
    rev -= rint(rev);
    const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
    _Float16* qt = qts + (k % 3) * SGQ * SQB;
    const float x0 = qx * cs - qy * sn, y0 = qy * cs + qx * sn;
    *(uint32_t*)(qt + qix) = pack_h2(x0, y0);
  };

  // One super-tile: bc holds its B fragments (its fp16 tile is buffer k % 2); the next super-tile is dequantized
  // into bn on the way.
  auto step = [&](int k, h8 (&bc)[SNJ], h8 (&bn)[SNJ]) {
    issue(k + 4);  // ring slot k % 4 held super-tile k, dequantized in the previous step
    const int t0 = (st_begin + k) * 32;
    // super-tile k + 1 landed: the copies of k + 2 .. k + 4 (four each; five for waves 0-2) may still be in flight
    if (wv < 3)
      __builtin_amdgcn_s_waitcnt(0x0F70 | 15);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70 | 12);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    // sources of super-tile k + 1's dequantization (dword reads: see code_words)
    const uint8_t* rawn = raw_w + ((k + 1) & 3) * SRAW;
    uint32_t xs[8];
    code_words(rawn, xs);
    const uint32_t z0 = *(const uint32_t*)(rawn + 2048 + 4 * (4 * t + gr0));
    const uint32_t z1 = *(const uint32_t*)(rawn + 2048 + 4 * (4 * t + gr1));
    uint8_t* vdst = vt_w + ((k + 1) & 1) * SVT + SCS * 8 * hf + 16 * t;

    // ---- partial keys over this wave's coordinates (block by block), RoPE, partial scores of the four heads.
    // The instruction stream interleaves each block's matrix instructions with vector work that does not wait
    // for them (two chunks of the next super-tile's dequantization, the previous block's RoPE), so that one
    // wave keeps both units busy.
    // score operand row t: query head t % 4
    const h8* qf = (const h8*)(qts + (k % 3) * SGQ * SQB + (t & 3) * SQB) + hf;
    f16v_t sc = {};
    // the key residual codes of this lane's token (one per byte: the fp8 B operands of H' c) and its scale;
    // super-tile k's residual is visible since the previous barrier.  H' c of block w is formed beside that
    // block's up-projection and added, scaled, before its RoPE.
    f16v_t ra = {};
    float ksc = 0.0f;
    const uint8_t* rrk = rres + (k % SRRN) * SRR;
    f16v_t kp[SNB];
#pragma unroll
    for (int g = 0; g <= SNB; ++g) {
      if (g < SNB) {
        kp[g] = f16v_t{};
#pragma unroll
        for (int j = 0; j < SNJ; ++j) kp[g] = mfma32s(wf[g][j], bc[j], kp[g]);
        if (g == wv) {  // H' c of this wave's block (exact integers)
          // (one 16-byte read of the half's code dwords; four-byte reads of the 32-byte token rows met eight lanes
          // to a bank)
          const u4 krw = *(const u4*)(rrk + 32 * t + 16 * hf);
          ksc = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)(rrk + 2048 + 2 * t)) * (2.0f * RSCALE);
          v8i_t er[2];  // the codes one per byte (the fp8 B operands): byte q of dword o = code m + 4q, m = o % 4
#pragma unroll
          for (int be = 0; be < 2; ++be)
#pragma unroll
            for (int o = 0; o < 8; ++o) er[be][o] = (int)((krw[2 * be + (o >> 2)] >> (2 * (o & 3))) & 0x03030303u);
          ra = mfma_f8_codes(hr[1], er[1], mfma_f8_codes(hr[0], er[0], f16v_t{}));
          if (g == 0 && hf == 0) ra[0] -= 192.0f;  // H' 1 is 128 at head dim 0 (row 0): the -1.5 offset
        }
#pragma unroll
        for (int jj = 2 * g; jj < 2 * g + 2; ++jj) {
          bn[jj] = dequant_int4x8(xs[jj], jj < 4 ? z0 : z1);
          *(h8*)(vdst + SCS * jj) = bn[jj];
        }
      }
      if (g > 0) {
        if (g - 1 == wv)  // the key residual of block g - 1, if it is this wave's
#pragma unroll
          for (int i = 0; i < 16; ++i) kp[g - 1][i] += ksc * ra[i];
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
    float* spb = sp + (k & 1) * (4 * 32 * SGQ);
    // row 8 (j / 4) + 4 hf + j % 4 of entry j: lane half 0 holds the four heads in entries 0-3
    if (hf == 0) *(f4*)(spb + (wv * 32 + t) * SGQ) = f4{sc[0], sc[1], sc[2], sc[3]};
    lds_barrier();
    rot_q(k + 2);  // buffer (k + 2) % 3 was last read before the previous barrier

    // ---- scores of the four heads for token t (the same in every wave), lazy online softmax
    float s4[SGQ];
    {
      f4 tot = *(const f4*)(spb + t * SGQ);
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) tot += *(const f4*)(spb + (w2 * 32 + t) * SGQ);
      const bool kept = t0 + t < T;  // past the end: no weight
#pragma unroll
      for (int i = 0; i < SGQ; ++i) s4[i] = kept ? tot[i] - m_ref[i] : -INFINITY;
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
      for (int nt = 0; nt < SNJ; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] *= alpha[i];
#pragma unroll
      for (int nt = 0; nt < RST; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) accr[nt][i] *= alpha[i];
      fresh = false;
    }
    float p[SGQ];
#pragma unroll
    for (int i = 0; i < SGQ; ++i) {
      p[i] = __builtin_amdgcn_exp2f(s4[i]);
      psum[i] += p[i];
    }
    if (hf == 0) *(h4*)(pt + SGQ * t) = h4{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    // the token's 2c - 3 over this wave's coordinates into its tile (chunk 2 jj + hf <-> coordinates
    // 32 w + 16 jj + res_coord(hf, e)), and p times the token's value scale / (2 sqrt(128))
    {
      const uint8_t* rr = rres + (k % SRRN) * SRR;
      static_assert(RST == 2, "the wave's two residual code dwords in one read");
      const u2 rw = *(const u2*)(rr + 1024 + 32 * t + 8 * wv);
#pragma unroll
      for (int jj = 0; jj < RST; ++jj) *(h8*)(vr_w + SRCS * (2 * jj + hf) + 16 * t) = res_2c3(rw[jj], hf);
      const float vsc = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)(rr + 2048 + 64 + 2 * t)) * RSCALE;
      if (hf == 0)
        *(h4*)(pt2 + SGQ * t) = h4{(_Float16)(p[0] * vsc), (_Float16)(p[1] * vsc), (_Float16)(p[2] * vsc),
                                   (_Float16)(p[3] * vsc)};
    }
    wave_lds_sync();
    {  // the rotated value residual: (p s) x (2c - 3), 16 coordinates per step
      const h8 pops = lds_tr8s(pt2 + SGQ * (8 * grp + (rho >> 2)), pt2 + SGQ * (8 * grp + 4 + (rho >> 2)));
      const int q4 = rho & 3;
      const uint8_t* vb = vr_w + SRCS * (q4 >> 1) + (8 * grp + (rho >> 2)) * 16 + (q4 & 1) * 8;
#pragma unroll
      for (int nt = 0; nt < RST; ++nt) accr[nt] = mfma16x16x32(pops, lds_tr8s(vb + 2 * SRCS * nt, vb + 2 * SRCS * nt + 64), accr[nt]);
    }
    // P as the A operand of the 16x16x32 value product: row l % 16 <-> head l % 4, k-slot 8g + j <-> token 8g + j
    // (g = l / 16); lane rho of its group points at the row of token 8g + 4v + rho / 4
    // value latent: step nt covers chunks 2nt, 2nt + 1; column n <-> coordinate 128w + 16nt + 8(n/8) + perm8(n%8);
    // lane rho points at the 4 columns 4(q4 % 2).. of chunk (2nt + q4 / 2, token 8g + 4v + rho / 4)
    {
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
    if (wv < 3)
      __builtin_amdgcn_s_waitcnt(0x0F70 | 15);
    else
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

  // ---- partial: m[4], l[4] (the same in every wave), acc[4][512] (wave w: coordinates 128w..128w+127), then the
  // rotated value residual accr[4][128] (wave w: coordinates 32w..32w+31)
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
#pragma unroll
    for (int nt = 0; nt < RST; ++nt) {  // residual column n of step nt: chunk 2nt + n / 8, element n % 8
      const int coord = 32 * wv + 16 * nt + res_coord(rho >> 3, rho & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) part[2 * SGQ + SGQ * SLAT + i * SD + coord] = accr[nt][i];
    }
  }
}

// ---- The role-split form (all modes but the residual): 8 waves, two per SIMD.  Waves 0-3 are key waves and
// waves 4-7 value waves; key wave w and value wave 4 + w share latent quarter w and, as a workgroup's waves are
// placed round-robin over the SIMDs, one SIMD.  The one-wave-per-SIMD layout above runs a super-tile's vector and
// matrix work largely one after the other; here a SIMD runs a key wave's matrix chain beside a value wave's vector
// work.  Between the barriers of super-tiles k - 1 and k:
//   value wave w: stages its quarter's codes and pairs (a four-deep ring of direct-to-LDS copies), dequantizes
//     super-tile k + 1 into the quarter's fp16 tile, runs the online softmax of super-tile k - 1 from the four
//     partial scores and its value product on the tile of k - 1, and rotates the query of super-tile k + 2;
//   key wave w: reads super-tile k's B fragments back from the quarter's tile, up-projects them (W_k's slice in the
//     accumulator registers) on v_mfma_f32_16x16x32_f16, rotates and scores them, and writes its partial scores.
// RoPE on one fp16 pair v = (x, y) with f = (cos, sin), as rope_pair: the same two packed operations and
// roundings, with f's halves picked by operand selects, so that the compiler keeps one register per factor word
// instead of hoisting its two swizzled copies (cos, cos) and (sin, sin) out of the loop.
__device__ inline uint32_t rope_pair_sel(uint32_t v, uint32_t f) {
  uint32_t t, r;
  asm("v_pk_mul_f16 %0, %1, %2 op_sel:[0,1] op_sel_hi:[1,1]" : "=v"(t) : "v"(v), "v"(f));  // (x sin, y sin)
  asm("v_pk_fma_f16 %0, %1, %2, %3 op_sel:[0,0,1] op_sel_hi:[1,0,0] neg_lo:[0,0,1]"      // (x cos - y sin,
      : "=v"(r) : "v"(v), "v"(f), "v"(t));                                                //  y cos + x sin)
  return r;
}

struct RoleLds {
  int raw, vt, qt, theta, sp, pt, addr, keep, rtab, posr, total;
};
// pos: the positions mode (SVAR query variants per super-tile, the RoPE factors of the 32 in-block offsets, a ring
// of the super-tiles' slot positions)
__host__ __device__ constexpr RoleLds role_lds(bool pos) {
  RoleLds L{};
  int o = 0;
  L.raw = o; o += 4 * 4 * SRAW;                        // per value wave: staging ring of 4 super-tiles
  L.vt = o; o += 4 * 2 * SVT;                          // per quarter: fp16 tiles of two super-tiles
  L.qt = o; o += 3 * (pos ? SVAR : 1) * SGQ * SQB * 2;  // rotated query (variants) in fragment order, fp16, x 3
  L.theta = o; o += (SD / 2) * 8;                      // RoPE frequencies, turns per position
  L.sp = o; o += 2 * 4 * 32 * SGQ * 4;                 // partial scores [buffer][key wave][token][head]
  L.pt = o; o += 4 * 32 * SGQ * 2;                     // probabilities [value wave][token][head] fp16
  L.addr = o; o += SMAX_TILES * 8;                     // page record address of each super-tile
  L.keep = o; o += SMAX_TILES * 4;                     // keep-mask word (positions mode: base block) of each
  L.rtab = o; o += pos ? 4 * 32 * RT16 * 4 : 0;       // positions mode: RoPE factors [group][offset u][16]
  L.posr = o; o += pos ? 8 * 32 * 4 : 0;               // positions mode: slot positions of super-tile k at k % 8
  L.total = o;
  return L;
}

// fragment order of the rotated query for the role-split kernel's 16x16x32 score products: element e of (head, tile
// pair m, lane group g) is head dim 16m + 4g + e/2 + 64 (e % 2), the k-slot order of the rotated keys of tiles m and
// m + 4; heads SQB elements apart
__device__ inline int qfrag16_index(int head, int dim) {
  const int xy = dim >> 6, r = dim & 63, m = r >> 4, g = (r >> 2) & 3, i = r & 3;
  return head * SQB + (m * 4 + g) * 8 + 2 * i + xy;
}
// KEEP: a token keep mask is applied (a separate instantiation, so that the unmasked kernel carries none of it); a
// super-tile whose tokens are all evicted is skipped by the key waves and adds nothing in the value waves.
// SPLIT: latent coordinates below SLAT / 2 feed only the keys and the rest only the values (W_k zero on the upper
// rows, W_v on the lower, as for keys and values with their own token factors): key waves 2-3 and the value
// products of value waves 0-1 are skipped; those products are exact zeros, so the output is the same.
// KB: latent code bits (4; or 3 and 2, whose codes a value wave stages token-major and spreads to the INT4 nibble
// layout).
// POS: a compacted cache whose slots hold tokens at the source positions tok_pos (no keep mask).  A super-tile's
// tokens lie within SVAR blocks of 32 positions from its first slot's block `base` (the layout the compaction
// writes): a token at position 32 (base + v) + u is rotated by R(u), from a table, and scored against the query
// rotated by R(q_pos - 32 (base + v)), one of SVAR variants in the score operand's rows; other slots take no part.
// Value wave 0 also copies each super-tile's 32 slot positions into a ring that both roles read after the barrier
// that follows its wait.
template <bool KEEP, bool SPLIT, int KB, bool POS>
__global__ __launch_bounds__(512, 1) void decode_shared_role_kernel(DecodeSharedArgs a) {
  constexpr int CB = SLAT * KB / 8;  // code bytes per token
  constexpr int QB = CB / 4;         // a quarter of them
  constexpr int NCH = QB / 16;       // its 16-byte chunks per token
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr RoleLds LY = role_lds(POS);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool keyw = wid < 4;
  const int wq = wid & 3;  // latent quarter
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
  const int npw = max(1, SQC >> lg);            // pairs per token over a quarter's coordinates (1, 2 or 4)
  const int g0 = (SQC * wq) >> lg;              // the first of them

  double* tturn = (double*)(smem + LY.theta);
  if (tid < SD / 2) tturn[tid] = (a.theta > 0.0 ? pow(a.theta, -2.0 * tid / SD) : 0.0) * 0.15915494309189535;
  const int n_st = (T + 31) / 32;
  const int st_begin = split * a.st_per_split;
  const int n_tiles = max(0, min(n_st, st_begin + a.st_per_split) - st_begin);
  int64_t* taddr = (int64_t*)(smem + LY.addr);
  uint32_t* tkeep = (uint32_t*)(smem + LY.keep);
  for (int k = tid; k < n_tiles; k += 512) {  // page record of each super-tile, its keep word (or base block)
    const int t0 = (st_begin + k) * 32;
    const int page = a.block_table[(size_t)b * a.max_blocks + t0 / P];
    taddr[k] = a.page_off[page] + (int64_t)(t0 % P) * CB;
    const int wd = t0 >> 5;
    if (KEEP) tkeep[k] = wd < a.keep_words ? a.keep[(size_t)b * a.keep_words + wd] : 0u;
    if (POS) {  // base block of the super-tile: its first slot's (none: no slot of the tile is valid)
      const int p0 = a.tok_pos[(size_t)b * a.pos_row + t0];
      tkeep[k] = (uint32_t)(p0 >= 0 ? p0 >> 5 : 1 << 30);
    }
  }
  const int32_t* posr = (const int32_t*)(smem + LY.posr);
  _Float16* qts = (_Float16*)(smem + LY.qt);  // rotated query of super-tile k: buffer k % 3 (variant v at its v-th quarter)
  float* sp = (float*)(smem + LY.sp);
  const uint8_t* vt_q = smem + LY.vt + wq * 2 * SVT;  // the quarter's fp16 tiles; super-tile k in k % 2
  __syncthreads();

  if (keyw) {
    // ---- W_k[l]'s slice of this quarter as A fragments of v_mfma_f32_16x16x32_f16 in the accumulator registers:
    // row tile m (16 head dims: 16m + r for m < 4, 64 + 16(m - 4) + r above, so that tiles m and m + 4 hold the RoPE
    // pairs (j, j + 64)), row r = lane % 16; k-step s, k-slot 8 grp + e <-> latent coordinate
    // 128w + 8 (4s + grp) + perm8(e), i.e. element e of code dword 4s + grp of the quarter (the order a code dword
    // dequantizes)
    h8 wf[2 * SNB][SNJ / 2];
    if (!SPLIT || wq < 2) {
      const int width = a.Hkv * SD;
      const uint16_t* W = a.wk + (size_t)b * a.w_stride + (size_t)l * SLAT * width + (size_t)h * SD;
#pragma unroll
      for (int m = 0; m < 2 * SNB; ++m) {
        const int dim = m < SNB ? 16 * m + rho : 64 + 16 * (m - SNB) + rho;
#pragma unroll
        for (int s = 0; s < SNJ / 2; ++s) {
          h8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[e] = bf16_to_h(W[(size_t)(SQC * wq + 8 * (4 * s + grp) + perm8(e)) * width + dim]);
          asm volatile("" : "=a"(wf[m][s]) : "0"(f));
        }
      }
    }
    // RoPE factors of this lane's two tokens 16 n + rho: tile pair m's output entry i (0..3) is head dims
    // 16m + 4 grp + i and + 64, frequency 16m + 4 grp + i; |u theta| < 32 turns, where v_sin / v_cos are accurate.
    // Positions mode: a table of the factors of every in-block offset u as a lane of group gg takes them
    // ([gg][u], rows of RT16 dwords), read per super-tile at the tokens' own offsets.
    uint32_t rf[2][SNB * 4];
    uint32_t* rtab = (uint32_t*)(smem + LY.rtab);
    if (POS) {
      for (int e = tid; e < 4 * 32 * 16; e += 256) {
        const int gg = e >> 9, u = (e >> 4) & 31, m = (e >> 2) & 3, i = e & 3;
        const float rev = (float)(u * tturn[16 * m + 4 * gg + i]);
        rtab[(32 * gg + u) * RT16 + 4 * m + i] = pack_h2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
      }
    } else {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int m = 0; m < SNB; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float rev = (float)((16 * n + rho) * tturn[16 * m + 4 * grp + i]);
            rf[n][4 * m + i] = pack_h2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
          }
    }
    lds_barrier();  // the value waves' prologue: the tile of super-tile 0, the rotated queries of 0 and 1; the table
    for (int k = 0; k < n_tiles; ++k) {
      const bool empty = KEEP && __builtin_amdgcn_readfirstlane(tkeep[k]) == 0u;
      // positions mode: a token's block offset v from the super-tile's base picks its query variant, its in-block
      // offset u its RoPE factors (slots of -1 or outside the SVAR blocks take no part)
      int vsel[2] = {0, 0};
      if constexpr (POS) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int pc = posr[(k & 7) * 32 + 16 * n + rho];
          const int v = (pc >> 5) - (int)tkeep[k];
          vsel[n] = pc >= 0 && v >= 0 && v < SVAR ? v : 0;
          const u32x4_t* src = (const u32x4_t*)(rtab + (32 * grp + (pc & 31)) * RT16);
#pragma unroll
          for (int m = 0; m < SNB; ++m) {
            const u32x4_t x = src[m];
#pragma unroll
            for (int i = 0; i < 4; ++i) rf[n][4 * m + i] = x[i];
          }
        }
      }
      f4 sc[2] = {};  // scores of tokens 16 n + rho: rows 4 grp + i <-> head i (positions mode: of variant grp)
      if ((!SPLIT || wq < 2) && !empty) {
        // B fragments: k-step s, token half n: chunk 4s + grp of token 16 n + rho
        const uint8_t* tl = vt_q + (k & 1) * SVT + SCS * grp + 16 * rho;
        h8 bc[SNJ / 2][2];
#pragma unroll
        for (int s = 0; s < SNJ / 2; ++s)
#pragma unroll
          for (int n = 0; n < 2; ++n) bc[s][n] = *(const h8*)(tl + SCS * 4 * s + 256 * n);
        // score A operand: row rho <-> head rho % 4 (positions mode: of variant rho / 4), the k-slots of lane group
        // grp for tile pair m at fragment 4m + grp
        const h8* qf = (const h8*)(qts + ((k % 3) * (POS ? SVAR : 1) + (POS ? rho >> 2 : 0)) * SGQ * SQB +
                                   (rho & 3) * SQB) + grp;
        // tile pair m (head dims of tiles m and m + 4; four independent accumulator chains), then tile pair m - 1's
        // RoPE and score products, so that one pair's vector work goes under the next pair's matrix instructions
        f4 kx[SNB][2], ky[SNB][2];
#pragma unroll
        for (int m = 0; m <= SNB; ++m) {
          if (m < SNB) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              kx[m][n] = f4{0, 0, 0, 0};
              ky[m][n] = f4{0, 0, 0, 0};
            }
#pragma unroll
            for (int s = 0; s < SNJ / 2; ++s)
#pragma unroll
              for (int n = 0; n < 2; ++n) {
                kx[m][n] = mfma16x16x32(wf[m][s], bc[s][n], kx[m][n]);
                ky[m][n] = mfma16x16x32(wf[m + SNB][s], bc[s][n], ky[m][n]);
              }
          }
          if (m > 0) {
            const h8 qa = qf[4 * (m - 1)];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              u32x4_t kr;  // k-slots 8 grp + 2i, + 1 <-> the rotated pair (x, y) of head dims 16(m-1) + 4 grp + i, + 64
#pragma unroll
              for (int i = 0; i < 4; ++i)
                kr[i] = rope_pair_sel(pack_h2(kx[m - 1][n][i], ky[m - 1][n][i]), rf[n][4 * (m - 1) + i]);
              sc[n] = mfma16x16x32(qa, __builtin_bit_cast(h8, kr), sc[n]);
            }
          }
        }
        // a split latent leaves key waves 0-1 beside value waves that make no value product: there one matrix
        // instruction, then up to two vector ones, measured faster (515 against 551 us on the Tucker group); with
        // every wave busy the compiler's own order is (614 against 648 us on the block-shared 32K step)
        if constexpr (SPLIT) {
#pragma unroll
          for (int m = 0; m < SNB; ++m) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
        }
      }
      // lane group 0 holds the four heads of its tokens (positions mode: group vsel, the token's variant)
#pragma unroll
      for (int n = 0; n < 2; ++n)
        if (POS ? grp == vsel[n] : grp == 0)
          *(f4*)(sp + (k & 1) * (4 * 32 * SGQ) + (wq * 32 + 16 * n + rho) * SGQ) = sc[n];
      lds_barrier();
    }
    return;
  }

  // The value waves go first at the SIMD's issue arbiter: they stage and dequantize the tiles the key waves' chains
  // read, and run the softmax and value product between the barriers (measured 648 -> 619 us on the block-shared
  // 32K step, 659 -> 647 on the keep-mask form, the INT3 and positions forms unchanged).  Not for a split latent,
  // whose key waves 0-1 are the critical path (516 -> 613 us on the Tucker group).
  if constexpr (!SPLIT) __builtin_amdgcn_s_setprio(1);
  // ---- value wave of quarter wq
  uint8_t* raw_w = smem + LY.raw + wq * 4 * SRAW;  // its ring; super-tile k in slot k % 4
  const uint32_t raw_lds = __builtin_amdgcn_readfirstlane(lds_addr(raw_w));
  _Float16* pt = (_Float16*)(smem + LY.pt) + wq * 32 * SGQ;
  const int64_t meta_base = pad16((int64_t)P * CB);
  // this thread's query pair for the per-tile rotation: head wq, pair lane, scaled for exp2
  const int qj = lane;
  float qx, qy;
  {
    const float sc = 1.4426950408889634f / sqrtf((float)SD);
    const size_t base = (((size_t)l * a.B + b) * a.Hq + h * SGQ + wq) * SD;
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
  const int qix = qfrag16_index(wq, qj);
  const double fq = tturn[qj];
  // positions mode: this thread's query pair rotated on from variant 0 to variant v by R(-32 v theta), v < SVAR
  float vc[SVAR], vs[SVAR];
  if (POS) {
#pragma unroll
    for (int v = 1; v < SVAR; ++v) {
      double rev = -32.0 * v * fq;
      rev -= rint(rev);
      vc[v] = __builtin_amdgcn_cosf((float)rev);
      vs[v] = __builtin_amdgcn_sinf((float)rev);
    }
  }
  const uint32_t posr_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem + LY.posr));

  // staging of this quarter of super-tile k into ring slot k % 4, as in decode_shared_res_kernel (past the last
  // super-tile the slot gets a copy of the last one; always four copy instructions, and value wave 0 of the
  // positions mode a fifth: the 32 slot positions into ring slot k % 8)
  auto issue = [&](int k) {
    const int kk = min(k, n_tiles - 1);
    const int slot0 = ((st_begin + kk) * 32) % P;
    const int64_t at = uniform64(taddr[kk]);
    const int pairs_at = (int)meta_base - slot0 * CB + slot0 * mpt;
    const i32x4_t rs = buffer_rsrc(a.pool + at, pairs_at + 32 * mpt);
    const uint32_t dst = raw_lds + (k & 3) * SRAW;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int p = 64 * r + lane;
      if (KB == 4) {
        copy16_to_lds(rs, dst + 1024 * r, (p & 31) * CB + QB * wq + 16 * (p >> 5));
      } else {
        const int pc = min(p, 32 * NCH - 1);
        copy16_to_lds(rs, dst + 1024 * r, (pc / NCH) * CB + QB * wq + 16 * (pc % NCH));
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = 64 * r + lane, tok = q >> 2, i = q & 3;
      copy4_to_lds(rs, dst + 2048 + 256 * r, pairs_at + tok * mpt + 4 * (g0 + (i & (npw - 1))));
    }
    if (POS && wq == 0 && lane < 32)
      copy4_to_lds(buffer_rsrc(a.tok_pos + (size_t)b * a.pos_row + (st_begin + kk) * 32, 128), posr_lds + (k & 7) * 128,
                   4 * lane);
  };
  const int gr0 = ((SQC * wq + 64 * hf) >> lg) - g0, gr1 = ((SQC * wq + 64 * hf + 32) >> lg) - g0;
  // the lane's eight code groups of a staged super-tile as INT4 dwords (group j = coordinates 8 (8hf + j).. of
  // the quarter of token t), and its two scale/zero pairs
  auto load_words = [&](int k, uint32_t (&xs)[8], uint32_t& z0, uint32_t& z1) {
    const uint8_t* raw = raw_w + (k & 3) * SRAW;
    if (KB == 4) {
      const uint32_t* c0 = (const uint32_t*)(raw + (64 * hf + t) * 16);
      const uint32_t* c1 = (const uint32_t*)(raw + (64 * hf + 32 + t) * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xs[j] = c0[j];
        xs[4 + j] = c1[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[j] = codes8_as_nibbles<KB>(raw + QB * t, KB * (8 * hf + j));
    }
    z0 = *(const uint32_t*)(raw + 2048 + 4 * (4 * t + gr0));
    z1 = *(const uint32_t*)(raw + 2048 + 4 * (4 * t + gr1));
  };
  // super-tile k's fp16 chunks into tile k % 2: chunk c (code dword c, 8 coordinates) of token t at byte SCS c + 16t
  auto store_tile = [&](int k, const uint32_t (&xs)[8], uint32_t z0, uint32_t z1) {
    uint8_t* dst = (uint8_t*)vt_q + (k & 1) * SVT + SCS * 8 * hf + 16 * t;
#pragma unroll
    for (int j = 0; j < SNJ; ++j) *(h8*)(dst + SCS * j) = dequant_int4x8(xs[j], j < 4 ? z0 : z1);
  };
  // rotated query q~ = R(q_pos - t0) q of super-tile k into buffer k % 3, in fragment order; positions mode: the SVAR
  // variants R(q_pos - 32 (base + v)) q (base: the super-tile's base block)
  auto rot_q = [&](int k, uint32_t base) {
    const double t0 = POS ? 32.0 * (double)base : (double)((st_begin + k) * 32);
    double rev = ((double)qpos - t0) * fq;
    rev -= rint(rev);
    const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
    _Float16* qt = qts + (k % 3) * (POS ? SVAR : 1) * SGQ * SQB;
    const float x0 = qx * cs - qy * sn, y0 = qy * cs + qx * sn;
    *(uint32_t*)(qt + qix) = pack_h2(x0, y0);
    if (POS) {
#pragma unroll
      for (int v = 1; v < SVAR; ++v)
        *(uint32_t*)(qt + v * SGQ * SQB + qix) = pack_h2(x0 * vc[v] - y0 * vs[v], y0 * vc[v] + x0 * vs[v]);
    }
  };

  f4 acc[SNJ];  // value latent on this quarter's coordinates, 16 per step, rows = query heads (replicated)
#pragma unroll
  for (int i = 0; i < SNJ; ++i) acc[i] = f4{0, 0, 0, 0};
  float m_ref[SGQ], psum[SGQ];
#pragma unroll
  for (int i = 0; i < SGQ; ++i) {
    m_ref[i] = 0.0f;
    psum[i] = 0.0f;
  }
  bool fresh = true;
  // the scores of super-tile k (the four key waves' partials), lazy online softmax, value product on tile k % 2
  auto soft_value = [&](int k) {
    const int t0 = (st_begin + k) * 32;
    const bool empty = KEEP && tkeep[k] == 0u;
    const float* spb = sp + (k & 1) * (4 * 32 * SGQ);
    float s4[SGQ];
    {
      f4 tot = *(const f4*)(spb + t * SGQ);
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) tot += *(const f4*)(spb + (w2 * 32 + t) * SGQ);
      bool valid = true;
      if (POS) {  // a slot of -1, or outside the super-tile's SVAR blocks: no token
        const int pc = posr[(k & 7) * 32 + t];
        const int v = (pc >> 5) - (int)tkeep[k];
        valid = pc >= 0 && v >= 0 && v < SVAR;
      }
      const bool kept = t0 + t < T && (!KEEP || ((tkeep[k] >> t) & 1u)) && valid;
#pragma unroll
      for (int i = 0; i < SGQ; ++i) s4[i] = kept ? tot[i] - m_ref[i] : -INFINITY;
    }
    const float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
    // the first super-tile with a kept token sets the reference maximum (one with none leaves it unset)
    if ((KEEP || POS) ? __builtin_amdgcn_ballot_w64(fresh ? mx > -INFINITY : mx > STAU) != 0
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
    // the value product as in decode_shared_res_kernel (P as the A operand of 16x16x32 products, the tile's chunks
    // read transposed as the B operand)
    if ((!SPLIT || wq >= 2) && !empty) {
      const h8 pop = lds_tr8s(pt + SGQ * (8 * grp + (rho >> 2)), pt + SGQ * (8 * grp + 4 + (rho >> 2)));
      const int q4 = rho & 3;
      const uint8_t* vb = vt_q + (k & 1) * SVT + SCS * (q4 >> 1) + (8 * grp + (rho >> 2)) * 16 + (q4 & 1) * 8;
      h8 vt[SNJ];
#pragma unroll
      for (int nt = 0; nt < SNJ; ++nt) vt[nt] = lds_tr8s(vb + 2 * SCS * nt, vb + 2 * SCS * nt + 64);
#pragma unroll
      for (int nt = 0; nt < SNJ; ++nt) acc[nt] = mfma16x16x32(pop, vt[nt], acc[nt]);
    }
  };

  if (n_tiles > 0) {
    // prologue: super-tiles 0-3 in flight, wait for 0, its tile; rotated queries of 0 and 1
#pragma unroll
    for (int j = 0; j < 4; ++j) issue(j);
    if (POS && wq == 0)
      __builtin_amdgcn_s_waitcnt(0x0F70 | 15);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70 | 12);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    uint32_t xs[8], z0, z1;
    load_words(0, xs, z0, z1);
    store_tile(0, xs, z0, z1);
    rot_q(0, POS ? tkeep[0] : 0u);
    rot_q(1, POS ? tkeep[min(1, n_tiles - 1)] : 0u);
  }
  lds_barrier();
  for (int k = 0; k < n_tiles; ++k) {
    issue(k + 4);  // ring slot k % 4 held super-tile k, stored into its tile before the previous barrier
    // super-tile k + 1 landed; the copies of k + 2 .. k + 4 (four each, five for value wave 0 of the positions
    // mode) may be in flight
    if (POS && wq == 0)
      __builtin_amdgcn_s_waitcnt(0x0F70 | 15);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70 | 12);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    uint32_t xs[8], z0, z1;
    load_words(k + 1, xs, z0, z1);
    if (k > 0) soft_value(k - 1);  // reads tile (k - 1) % 2, which super-tile k + 1 then takes
    store_tile(k + 1, xs, z0, z1);
    // buffer (k + 2) % 3 was last read by the key waves before the previous barrier
    rot_q(k + 2, POS ? tkeep[min(k + 2, n_tiles - 1)] : 0u);
    lds_barrier();
  }
  if (n_tiles > 0) soft_value(n_tiles - 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the copies past the end land before the workgroup exits

  // ---- partial: m[4], l[4] (the same in every value wave), acc[4][512] (quarter w: coordinates 128w..128w+127)
#pragma unroll
  for (int i = 0; i < SGQ; ++i) {
    float v = hf == 0 ? psum[i] : 0.0f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    psum[i] = v;
  }
  float* part = a.ws + ((((size_t)l * a.Hkv + h) * a.B + b) * a.n_splits + split) * a.part_stride;
  if (wq == 0 && lane < SGQ) {
    part[lane] = fresh ? -INFINITY : m_ref[lane];
    part[SGQ + lane] = psum[lane];
  }
  if (grp == 0) {
#pragma unroll
    for (int nt = 0; nt < SNJ; ++nt) {
      const int coord = SQC * wq + 16 * nt + 8 * (rho >> 3) + perm8(rho & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) part[2 * SGQ + i * SLAT + coord] = acc[nt][i];
    }
  }
}

// out[l][b][h*4 + hq] = (W_v[l][:, h*128 : (h+1)*128]^T c* + H' r*) / l*, over the splits' partials (r*: the
// rotated value residual of the residual mode, H' the +-1 Hadamard; its accumulators carry 1 / sqrt(128)): one
// workgroup of 256 threads per (layer, sequence, query head).  The splits' (m, l, acc) are combined into c* (two
// latent coordinates per thread); then thread t takes head dims 8 (t % 16) .. + 7 and latent rows 32 (t / 16) .. + 31,
// reading each W_v row segment with one 16-byte load (all of them in flight together; one W_v element per thread and
// row left this kernel waiting on 64 rounds of loads), and the 16 row groups' partial sums are added in LDS in a
// fixed order.
__global__ __launch_bounds__(256) void merge_shared_kernel(const float* ws, const uint16_t* wv, int64_t w_stride,
                                                          float* out, int B, int Hkv, int Hq, int n_splits,
                                                          int part_stride, int c_begin, int res) {
  constexpr int RG = 16, RPG = SLAT / RG;  // row groups, rows per group
  static_assert(SLAT == 2 * 256 && SD == 8 * 16, "thread mapping");
  __shared__ float cst[SLAT];
  __shared__ float rst[SD];
  __shared__ float lst;
  __shared__ float red[RG][SD + 4];
  int id = blockIdx.x;
  const int hq_all = id % Hq; id /= Hq;
  const int b = id % B;
  const int l = id / B;
  const int h = hq_all / SGQ, hq = hq_all % SGQ;
  const int tid = threadIdx.x;
  const float* parts = ws + (((size_t)l * Hkv + h) * B + b) * n_splits * part_stride;
  float m = -INFINITY;
  for (int p = 0; p < n_splits; ++p) m = fmaxf(m, parts[(size_t)p * part_stride + hq]);
  float lsum = 0.0f, c0 = 0.0f, c1 = 0.0f, r = 0.0f;
#pragma unroll 4
  for (int p = 0; p < n_splits; ++p) {
    const float* pp = parts + (size_t)p * part_stride;
    const float mp = pp[hq];
    const float w = mp == -INFINITY ? 0.0f : exp2f(mp - m);
    lsum += w * pp[SGQ + hq];
    c0 += w * pp[2 * SGQ + hq * SLAT + tid];
    c1 += w * pp[2 * SGQ + hq * SLAT + tid + 256];
    if (res && tid < SD) r += w * pp[2 * SGQ + SGQ * SLAT + hq * SD + tid];
  }
  cst[tid] = c0;
  cst[tid + 256] = c1;
  if (tid < SD) rst[tid] = r;
  if (tid == 0) lst = lsum;
  __syncthreads();
  const int cg = tid % 16, rg = tid / 16;
  const size_t width = (size_t)Hkv * SD;
  const uint16_t* W = wv + (size_t)b * w_stride + (size_t)l * SLAT * width + (size_t)h * SD + 8 * cg;
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (RPG * (rg + 1) > c_begin) {  // (a split latent: W_v is zero below c_begin, a multiple of RPG)
    u4 wr[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) wr[i] = *(const u4*)(W + (size_t)(RPG * rg + i) * width);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const float cv = cst[RPG * rg + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w2 = wr[i][e >> 1];
        o[e] += __builtin_bit_cast(float, (e & 1) ? (w2 & 0xFFFF0000u) : (w2 << 16)) * cv;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][8 * cg + e] = o[e];
  __syncthreads();
  if (tid < SD) {
    const int d = tid;
    float sum = 0.0f;
#pragma unroll
    for (int g = 0; g < RG; ++g) sum += red[g][d];
    if (res) {
      float rr = 0.0f;
      for (int i = 0; i < SD; ++i) rr += (__builtin_popcount(d & i) & 1) ? -rst[i] : rst[i];
      sum += rr;
    }
    out[(((size_t)l * B + b) * Hq + hq_all) * SD + d] = lst > 0.0f ? sum / lst : 0.0f;  // zero: no token kept
  }
}

int shared_max_tiles_per_split() { return SMAX_TILES; }

bool shared_supported(const kvc_layout& L) {
  const int kb = lat_bits_k(L);
  return L.shared && L.head_dim == SD && L.r_k_cap == SLAT && L.n_q_heads == SGQ * L.n_kv_heads &&
         (kb == 4 || kb == 3 || kb == 2) && lat_bits_v(L) == kb && L.group >= 32 && L.group <= SLAT &&
         (L.group & (L.group - 1)) == 0 && (!L.residual_bits || kb == 4);
}

static int shared_part_stride(const kvc_layout& L) { return 2 * SGQ + SGQ * SLAT + (L.residual_bits ? SGQ * SD : 0); }

size_t shared_ws_bytes(const kvc_layout& L, int B, int n_splits) {
  return (size_t)L.n_layers * L.n_kv_heads * B * n_splits * shared_part_stride(L) * sizeof(float);
}

static hipError_t launch_shared_res(int grid, hipStream_t st, const DecodeSharedArgs& a) {
  const void* kern = (const void*)decode_shared_res_kernel;
  constexpr int lds = shared_lds().total;
  static_assert(lds <= 160 * 1024, "LDS of the residual-mode kernel");
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_shared_res_kernel, dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <bool KEEP, bool SPLIT, int KB, bool POS>
static hipError_t launch_role_one(int grid, hipStream_t st, const DecodeSharedArgs& a) {
  const void* kern = (const void*)decode_shared_role_kernel<KEEP, SPLIT, KB, POS>;
  constexpr int lds = role_lds(POS).total;
  static_assert(lds <= 160 * 1024, "LDS of the role-split kernel");
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_shared_role_kernel<KEEP, SPLIT, KB, POS>), dim3(grid), dim3(512), lds, st, a);
  return hipGetLastError();
}

template <bool KEEP, bool SPLIT, bool POS>
static hipError_t launch_role_bits(int kb, int grid, hipStream_t st, const DecodeSharedArgs& a) {
  if (kb == 3) return launch_role_one<KEEP, SPLIT, 3, POS>(grid, st, a);
  if (kb == 2) return launch_role_one<KEEP, SPLIT, 2, POS>(grid, st, a);
  return launch_role_one<KEEP, SPLIT, 4, POS>(grid, st, a);
}

// keep mask, positions and the residual are exclusive (the entry point rejects their combinations; the residual
// mode has INT4 latents)
static hipError_t launch_shared_variant(bool keep, bool pos, bool res, bool split, int kb, int grid, hipStream_t st,
                                        const DecodeSharedArgs& a) {
  // the residual mode runs the plain-latent form also for a split latent: the products it then makes are exact
  // zeros, and the output is the full product's
  if (res) return launch_shared_res(grid, st, a);
  if (pos) return split ? launch_role_bits<false, true, true>(kb, grid, st, a) : launch_role_bits<false, false, true>(kb, grid, st, a);
  if (keep) return split ? launch_role_bits<true, true, false>(kb, grid, st, a) : launch_role_bits<true, false, false>(kb, grid, st, a);
  return split ? launch_role_bits<false, true, false>(kb, grid, st, a) : launch_role_bits<false, false, false>(kb, grid, st, a);
}

hipError_t launch_decode_shared(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out,
                                void* ws, int n_splits, int st_per_split, hipStream_t st) {
  DecodeSharedArgs a;
  a.pool = C.pool; a.page_off = C.page_off; a.block_table = in.block_table; a.seq_len = in.seq_len;
  a.q_pos = in.q_pos; a.q = in.q; a.wk = in.wk; a.w_stride = in.w_seq_stride; a.ws = (float*)ws;
  a.keep = in.keep_mask; a.keep_words = in.keep_words;
  a.tok_pos = in.tok_pos; a.pos_row = in.max_blocks * L.page_size;
  a.lat_bytes = shared_latent_bytes(L); a.rec_bytes = (int)uniform_page_bytes(L);
  a.q_bf16 = in.q_dtype == KVC_BF16;
  a.B = in.B; a.Hkv = L.n_kv_heads; a.Hq = L.n_q_heads; a.L = L.n_layers; a.max_blocks = in.max_blocks;
  a.P = L.page_size; a.G = L.group; a.n_splits = n_splits; a.st_per_split = st_per_split;
  a.part_stride = shared_part_stride(L); a.theta = L.rope_theta;
  const bool split = in.kv_split == SLAT / 2;
  const int kb = lat_bits_k(L);
  const int grid = L.n_layers * L.n_kv_heads * in.B * n_splits;
  hipError_t e = mark(g_marks.begin, st);
  if (e != hipSuccess) return e;
  e = launch_shared_variant(in.keep_mask != nullptr, in.tok_pos != nullptr, L.residual_bits != 0, split, kb, grid,
                            st, a);
  if (e == hipSuccess) e = mark(g_marks.end, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_shared_kernel, dim3(L.n_layers * in.B * L.n_q_heads), dim3(256), 0, st, a.ws, in.wv,
                     in.w_seq_stride, out, in.B, L.n_kv_heads, L.n_q_heads, n_splits, a.part_stride,
                     split ? SLAT / 2 : 0, L.residual_bits != 0);
  return hipGetLastError();
}

}  // namespace kvc
