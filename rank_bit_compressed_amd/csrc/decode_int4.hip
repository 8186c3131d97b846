// decode_int4.hip -- one decode step of attention over a per-KV-head INT4 compressed cache, head
// dimension 128, four query heads per KV head (gfx950).  The fast path of the per-head mode.
//
// Work decomposition: one workgroup (4 waves) per (sequence b, KV head h, context split of pages).
// The workgroup copies each page's head-h block (codes, scale/zero pairs) and the page's offset row
// from HBM into LDS with buffer loads that write LDS directly, two buffers deep (the next page in
// flight while one is decoded; a third buffer measured no faster).  Wave w decodes the 64 slots
// 64w..64w+63 of every page as two 32-token super-tiles and keeps its own online-softmax state.
// Under variable rank the wave first orders its 64 slots by their number of 16-coordinate steps (the
// kernel body below), so that a super-tile runs only the steps its largest rank needs.
//
// All products are v_mfma_f32_32x32x16_f16 (on gfx950 it does twice the work of the 16x16x32 form in
// the same issue time).  Lane l serves one token of the super-tile (slot order, or the rank order), and
// its half l / 32 selects the eight k-slots it supplies.  Per super-tile:
//   K codes -> fp16 (code * scale + zero; 8 coordinates per lane per 16-coordinate step)
//   -> K_pre = B_k c (4 tiles of 32 head dims; the basis fragments stay in registers)
//   -> RoPE R(u) in packed fp16 on the pairs (j, j + 64), which sit in one lane (tiles m and m + 2)
//   -> S = Q~ K~^T (rows: the 4 heads of the wave's rotated query, replicated; columns: tokens), each lane
//      keeping the four heads' scores of its token
//   -> p = 2^s; P^T through a one-hot MFMA (tokens move into the reduction slots)
//   V codes -> fp16 -> V^T through one-hot MFMAs -> acc += P V_latent (rows: heads, columns:
//   latent coordinates).  The value basis is applied once per (b, head) in the merge, since
//   sum_t p_t B c_t = B sum_t p_t c_t.
// RoPE is split as R(t0 + pb + u) = R(t0 + pb) R(u) for the slot pb + u of the wave whose first slot is pb:
// R(u), u < 64, from an LDS table on the key side; R(q_pos - t0 - pb) q on the query side, rotated once per page
// and wave.
// Softmax keeps a reference maximum m per head and only raises it (rescaling acc and l) when a score
// exceeds it by more than 2^8 in the exp2 domain; the probabilities then stay below 256, within the
// fp16 operand range at full relative precision.  The merge uses the same m.
#include <math.h>

#include "kvc_common.hpp"

namespace kvc {

struct Int4Args {
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
  int hb_max;
  double theta;
  HeadSections S_uniform;
};

typedef float f16v __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

namespace i4 {
constexpr int D = 128, GQ = 4, NP = 64;
constexpr int MAX_SPLIT_PAGES = 128;
constexpr float TAU = 8.0f;   // lazy-max slack, log2 units
constexpr int QROW = NP + 4;  // dwords per row of the rotated-query and RoPE tables (padded against bank conflicts)
// the kernel's own LDS arrays (bytes): per wave the rotated query of 4 heads, the RoPE factors of the offsets
// 0..63 from a wave's first slot, per wave the probabilities of a super-tile, per wave the decode order of its 64
// slots
constexpr int STATIC_LDS = 4 * GQ * QROW * 4 + 64 * QROW * 4 + 4 * 32 * GQ * 2 + 4 * 64;

struct Lds {
  int meta_addr, meta_hb, meta_page, theta, qsrc, stage, stage_bytes, off_bytes, total;
};
__host__ __device__ inline Lds lds_layout(int P, int hb_max) {
  Lds L;
  int o = 0;
  L.meta_addr = o; o += MAX_SPLIT_PAGES * 8;
  L.meta_hb = o; o += MAX_SPLIT_PAGES * 4;
  L.meta_page = o; o += MAX_SPLIT_PAGES * 4;
  L.theta = o; o += NP * 8;                     // RoPE frequencies, turns per position
  L.qsrc = o; o += NP * 2 * GQ * 4;             // scaled query, pair j: x_j of heads 0-3, then x_{j+64}
  // stage buffer: the page's offset row (whole 64-dword rows, the tail zero-filled), then the head block
  L.off_bytes = 256 * ceil_div(P + 1, 64);
  L.stage_bytes = L.off_bytes + (int)pad16(hb_max);
  L.stage = o; o += 2 * L.stage_bytes;
  L.total = o;
  return L;
}
}  // namespace i4

__device__ inline uint32_t lds_u32(const uint8_t* base, int byte_off) { return *(const uint32_t*)(base + byte_off); }

// Scale/zero pair, or zero when the lane's eight coordinates lie beyond the token's rank.
__device__ inline uint32_t pair_if(bool ok, uint32_t sz) { return ok ? sz : 0u; }

__device__ inline f16v mfma32(h8 a, h8 b, f16v c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }

// eight consecutive accumulator entries (from entry e0) as an fp16 operand
__device__ inline h8 cvt_h8(const f16v& v, int e0) {
  h8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (_Float16)v[e0 + j];
  return r;
}

// s_waitcnt vmcnt(k) for a run-time k (this wave's vector-memory operations still allowed in flight)
__device__ inline void vmcnt_wait(int k) {
  switch (k) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F77); break;
  }
}

// The lane index computed afresh (volatile, so that it is not merged with another computation of it and kept
// in a register across a loop).
__device__ inline int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

template <int N>
struct Steps {
  static constexpr int value = N;
};

// KS, VS: 16-coordinate steps of the key / value rank caps (2..4); VT: 32-coordinate value tiles; KB, VB: bits
// of the key / value codes (4, or the lower-bit codecs 3 and 2, spread to the INT4 nibble layout as they are read)
//
// Wave w decodes the 64 slots 64w..64w+63 of every page (two 32-token super-tiles; a page of fewer slots
// leaves later waves idle).  Variable rank: the wave takes its 64 slots in order of their number of
// 16-coordinate steps (the "class", ceil(rank / 16)), equal classes in slot order -- a ballot per class, no
// exchange with the other waves -- so that a super-tile runs only the steps of its largest rank instead of the
// cap's.  Its token at page slot pb + u then sits at an arbitrary lane and reads its own R(u) from the table; the
// query side is the same for all 64 slots, so every row of the score product holds a head of one rotated query.
template <int KS, int VS, bool VAR, int STG, int KB, int VB>
__global__ __launch_bounds__(256, 2) void decode_int4_kernel(Int4Args a) {
  using namespace i4;
  constexpr int VT = (VS + 1) / 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int P = a.P;
  const Lds LY = lds_layout(P, a.hb_max);
  int64_t* meta_addr = (int64_t*)(smem + LY.meta_addr);
  int32_t* meta_hb = (int32_t*)(smem + LY.meta_hb);
  int32_t* meta_page = (int32_t*)(smem + LY.meta_page);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int t = lane & 31, hf = lane >> 5;
  const int split = blockIdx.x % a.n_splits;
  const int h = (blockIdx.x / a.n_splits) % a.Hkv;
  const int b = blockIdx.x / (a.n_splits * a.Hkv);
  const int T = a.seq_len[b];
  const int qpos = a.q_pos ? a.q_pos[b] : T;
  const int lb0 = split * a.pages_per_split;
  const int n_pages = max(0, min((T + P - 1) / P, lb0 + a.pages_per_split) - lb0);
  // Buffers that the page copies never touch live in arrays of their own, so that the compiler can tell
  // their reads apart from the LDS the copies write and does not wait for copies in flight before them.
  // qbuf: per wave the rotated query of 4 heads (row = head), fp16 pairs (x_j, x_{j+64}); rtab:
  // (cos, sin)(u theta_j) for u < 64; pbuf: per wave the probabilities of 32 tokens x 4 heads, fp16; sorder:
  // per wave the decode order of its 64 slots.
  __shared__ __attribute__((aligned(16))) uint32_t qbuf_all[4 * GQ * QROW];
  __shared__ __attribute__((aligned(16))) uint32_t rtab[64 * QROW];
  __shared__ __attribute__((aligned(16))) _Float16 pbuf_all[4 * 32 * GQ];
  __shared__ uint8_t sorder_all[4 * 64];
  static_assert(sizeof(qbuf_all) + sizeof(rtab) + sizeof(pbuf_all) + sizeof(sorder_all) == STATIC_LDS,
                "static LDS accounting");
  uint32_t* qbuf = qbuf_all + wv * GQ * QROW;
  uint8_t* sorder = sorder_all + wv * 64;

  // ---- page addresses of the split
  for (int i = tid; i < n_pages; i += 256) {
    const int page = a.block_table[(size_t)b * a.max_blocks + lb0 + i];
    int64_t hb = a.S_uniform.hb;
    if constexpr (VAR) {
      const uint32_t tot = a.tok_off[(size_t)page * (P + 1) + P];
      const int64_t cb = (int64_t)(tot & 0xFFFFu) * KB / 8, mb = 4 * (int64_t)(tot >> 16);  // variable rank: KB == VB
      hb = head_sections(cb, cb, mb, mb, P, D, 0).hb;
    }
    meta_addr[i] = a.page_off[page] + (int64_t)h * hb;
    meta_hb[i] = (int32_t)hb;
    meta_page[i] = page;
  }

  // ---- key basis as A fragments (registers): row = head dim 32m + t, k-slot 8hf + j <-> coordinate
  // 16s + 8hf + perm8(j) (the order in which a code dword dequantizes)
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
          const u4 raw = *(const u4*)(Bk + (size_t)(32 * m + t) * a.rk + col0);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int e = perm8(j);
            const uint32_t w = raw[e >> 1];
            f[j] = bf16_to_h((uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu)));
          }
        }
        bf[s][m] = f;
      }
    }
  }
  // ---- RoPE frequencies, once per workgroup: theta_j (fp64 pow) in turns per position
  double* tturn = (double*)(smem + LY.theta);
  if (tid < NP) tturn[tid] = (a.theta > 0.0 ? pow(a.theta, -2.0 * tid / D) : 0.0) * 0.15915494309189535;
  // one-hot B operands of the value transpose: k-slot 8hf + j of step s holds coordinate 16s + 8hf + perm8(j);
  // it goes to column (16 (s % 2) + 8hf + perm8(j)) of value tile s / 2
  h8 ohv[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int j = 0; j < 8; ++j) ohv[e][j] = (t == 16 * e + 8 * hf + perm8(j)) ? (_Float16)1.0f : (_Float16)0.0f;
  // probabilities of this wave's super-tile, [token][head] fp16: the transposing LDS read turns them into
  // the A operand of the value product (row = head, k-slot 8hf + j <-> token 16w + 8(j / 4) + 4hf + j % 4)
  _Float16* pbuf = pbuf_all + wv * 32 * GQ;

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
  __syncthreads();  // frequencies and the scaled query visible
  // (cos, sin)(u theta_j) for the offsets u < 64 of a wave's slots from its base and every pair j (the angle reduced
  // to half a turn in fp64; v_sin / v_cos take turns)
  for (int e = tid; e < 64 * NP; e += 256) {
    const int u = e / NP, j = e % NP;
    double rev = u * tturn[j];
    rev -= rint(rev);
    rtab[u * QROW + j] = pack_h2(__builtin_amdgcn_cosf((float)rev), __builtin_amdgcn_sinf((float)rev));
  }
  const double fj = tturn[lane];  // turns per position of pair `lane` (query rotation)

  // ---- page staging.  Wave w copies the 16-byte chunks 256k + 64w + l of the head block (and a share of
  // the page's offset row) into buffer i % 2.
  auto issue = [&](int i) {
    uint8_t* dst = smem + LY.stage + (i % 2) * LY.stage_bytes;
    const int bytes = __builtin_amdgcn_readfirstlane(meta_hb[i]);
    // buffer resources: scalar base and size (reads past the size return zeros)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.pool + uniform64(meta_addr[i])), (short)0, bytes, 0x00020000);
    // The lane index is recomputed here, and the lane test compares it with a scalar count of 16-byte chunks:
    // a register kept across the page loop for it, or a per-copy lane offset, could be spilled, and the wait
    // for its reload would also wait for the copies issued before it.
    const int ln = fresh_lane_id();
#pragma unroll
    for (int k = 0; k < STG; ++k) {
      const int base = 16 * (256 * k + 64 * wv);
      if (base >= bytes) break;  // wave-uniform: every issued copy has lane 0 active
      if (ln < ((bytes - base) >> 4))
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + LY.off_bytes + base),
                                                 16, 16 * ln, base, 0, 0);
    }
    if constexpr (VAR) {
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.tok_off + (size_t)__builtin_amdgcn_readfirstlane(meta_page[i]) * (P + 1)), (short)0, 4 * (P + 1),
          0x00020000);
      for (int base = 64 * wv; base <= P; base += 256)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (__attribute__((address_space(3))) void*)(dst + 4 * base), 4,
                                                 4 * ln, 4 * base, 0, 0);
    }
  };
  // every copy this wave issued has landed, and after the barrier everyone's have.  The copies write LDS
  // directly, and LDS is coherent within the workgroup, so the barrier needs no memory fence of its own.  The
  // wavefront-scope LDS fences only keep the compiler from moving LDS accesses across it.
  auto settle = [&]() {
    vmcnt_wait(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };

  // running state: value accumulator (4 heads x the lane's latent coordinates), sums, reference maxima
  float acc[VT][4], psum[4], m_ref[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    psum[i] = 0.0f;
    m_ref[i] = 0.0f;
#pragma unroll
    for (int w = 0; w < VT; ++w) acc[w][i] = 0.0f;
  }
  bool fresh = true;  // no token seen yet

  const int kcb = a.rk * KB / 8, vcb = a.rv * VB / 8;                        // uniform: code bytes per slot
  const int kmb = 4 * ceil_div(a.rk, a.G), vmb = 4 * ceil_div(a.rv, a.G);  // uniform: pair bytes per slot

  struct Words {  // a lane's LDS words for one super-tile: code dword and (scale, zero) word per step
    uint32_t k[KS], pk[KS];
    int co_v, po_v, r, rv, slot, ns;  // r, rv: key and value rank (0 past the sequence end); slot in the page
    bool ok;
  };

  __syncthreads();  // page addresses, the RoPE table visible
  if (n_pages > 0) issue(0);
  settle();
  for (int ip = 0; ip < n_pages; ++ip) {
    if (ip + 1 < n_pages) issue(ip + 1);  // into the buffer everyone finished with before the last barrier
    const uint32_t* so = (const uint32_t*)(smem + LY.stage + (ip % 2) * LY.stage_bytes);
    const uint8_t* sb = (const uint8_t*)so + LY.off_bytes;
    HeadSections S;
    if constexpr (VAR) {
      const uint32_t tot = so[P];
      const int64_t cb = (int64_t)(tot & 0xFFFFu) * KB / 8, mb = 4 * (int64_t)(tot >> 16);
      S = head_sections(cb, cb, mb, mb, P, D, 0);
    } else {
      S = a.S_uniform;
    }
    const uint8_t* kcs = sb + S.kc;
    const uint8_t* vcs = sb + S.vc;
    const uint8_t* kms = sb + S.km;
    const uint8_t* vms = sb + S.vm;
    const int page_t0 = (lb0 + ip) * P;
    const int pb = 64 * wv;                                   // this wave's first slot of the page
    const int nvb = max(0, min(64, min(P, T - page_t0) - pb));  // its slots holding tokens
    // the query rotated to the wave's base slot, q~ = R(q_pos - t0 - pb) q; lane j: pair j
    {
      const f4 qa = *(const f4*)&qsrc[lane * 8], qb = *(const f4*)&qsrc[lane * 8 + 4];
      double rev = (double)(qpos - page_t0 - pb) * fj;
      rev -= rint(rev);  // |rev| <= 1/2 turn; v_sin / v_cos take turns
      const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
#pragma unroll
      for (int hq = 0; hq < GQ; ++hq)
        qbuf[hq * QROW + lane] = pack_h2(qa[hq] * cs - qb[hq] * sn, qb[hq] * cs + qa[hq] * sn);
    }
    // decode order of the wave's slots (variable rank): lane l holds slot pb + l, of class c (0 past the end)
    if constexpr (VAR) {
      int c = 0;
      if (lane < nvb) {
        const int r = (int)((so[pb + lane + 1] - so[pb + lane]) & 0xFFFFu);
        c = min(KS, max(1, (r + 15) >> 4));
      }
      int base = 0, pos = 0;
#pragma unroll
      for (int cl = 1; cl <= KS; ++cl) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(c == cl);
        if (c == cl) pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        base += (int)__builtin_popcountll(m);
      }
      if (c > 0) sorder[pos] = (uint8_t)lane;
    }
    wave_sync();  // the rotated query and the order visible to the whole wave
    const uint32_t* qrow = qbuf + (t & 3) * QROW + 4 * hf;  // score A operand row t: head t % 4
    const int nst_w = (nvb + 31) / 32;

    // the LDS words of super-tile k of this wave (decode position 32 k + t of its block), one super-tile ahead
    auto fetch = [&](int k) -> Words {
      const int idx = 32 * k + t;
      Words w;
      w.ok = idx < nvb;
      int co_k, po_k;
      if constexpr (VAR) {
        w.slot = pb + (w.ok ? (int)sorder[idx] : 0);
        const uint32_t o0 = so[w.slot], o1 = so[w.slot + 1];
        w.r = w.rv = w.ok ? (int)((o1 - o0) & 0xFFFFu) : 0;
        co_k = w.co_v = (int)((o0 & 0xFFFFu) * KB / 8);
        po_k = w.po_v = (int)(o0 >> 16) * 4;
        // steps of the super-tile: the class of its last token (the order puts classes in increasing order)
        const int cls = min(KS, max(1, (w.r + 15) >> 4));
        w.ns = __builtin_amdgcn_readlane(cls, min(31, nvb - 1 - 32 * k));
      } else {
        w.slot = pb + idx;
        w.r = w.ok ? a.rk : 0;
        w.rv = w.ok ? a.rv : 0;
        co_k = w.slot * kcb;
        w.co_v = w.slot * vcb;
        po_k = w.slot * kmb;
        w.po_v = w.slot * vmb;
        w.ns = KS;
      }
      // every step's words are read (a step past the token's rank reads bytes of the same head block, and its
      // scale and zero are zeroed); the super-tile uses the first ns of them
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        w.k[s] = codes8_as_nibbles<KB>(kcs, co_k + KB * hf + 2 * KB * s);
        w.pk[s] = pair_if(16 * s + 8 * hf < w.r, lds_u32(kms, po_k + 4 * ((16 * s + 8 * hf) / a.G)));
      }
      return w;
    };

    // One super-tile with NS key steps (NSV value steps, NT value tiles), straight-line code for each NS.
    auto tile = [&](auto nsc, const Words& cur, int k) {
      constexpr int NS = decltype(nsc)::value;
      constexpr int NSV = VAR ? NS : VS;  // variable rank: one rank for K and V
      constexpr int NT = (NSV + 1) / 2;
      uint32_t vw[NSV], vp[NSV];
#pragma unroll
      for (int s = 0; s < NSV; ++s) {
        vw[s] = codes8_as_nibbles<VB>(vcs, cur.co_v + VB * hf + 2 * VB * s);
        vp[s] = pair_if(16 * s + 8 * hf < cur.rv, lds_u32(vms, cur.po_v + 4 * ((16 * s + 8 * hf) / a.G)));
      }

      // ---- keys: dequantize the steps, then per half m the tiles m and m + 2 (head dims d and d + 64), RoPE R(u)
      // of the token's in-block position u, and the score steps u = 4m + q (pairs 32m + 8q + 4hf + p in k-slots
      // 8hf + 2p, 8hf + 2p + 1)
      h8 kb[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) kb[s] = dequant_int4x8(cur.k[s], cur.pk[s]);
      const uint32_t* rrow = rtab + (cur.slot & 63) * QROW + 4 * hf;  // R(u), u = the slot's offset from pb
      f16v sc = {};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f16v ka = {}, kz = {};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          ka = mfma32(bf[s][m], kb[s], ka);
          kz = mfma32(bf[s][m + 2], kb[s], kz);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u4 rf = *(const u4*)(rrow + 32 * m + 8 * q);
          h8 kq;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const h2 rr = as_h2(rope_pair(pack_h2(ka[4 * q + p], kz[4 * q + p]), rf[p]));
            kq[2 * p] = rr.x;
            kq[2 * p + 1] = rr.y;
          }
          const h8 qf = *(const h8*)(qrow + 32 * m + 8 * q);
          sc = mfma32(qf, kq, sc);
        }
      }

      // ---- values: dequantize, transpose into (coordinate, token) tiles through one-hot MFMAs
      h8 vop[NT][2];
      {
        f16v vt[NT];
#pragma unroll
        for (int w = 0; w < NT; ++w) vt[w] = f16v{};
#pragma unroll
        for (int s = 0; s < NSV; ++s) vt[s / 2] = mfma32(dequant_int4x8(vw[s], vp[s]), ohv[s & 1], vt[s / 2]);
#pragma unroll
        for (int w = 0; w < NT; ++w) {
          vop[w][0] = cvt_h8(vt[w], 0);
          vop[w][1] = cvt_h8(vt[w], 8);
        }
      }

      // ---- the token's four scores: entries 0-3 (rows 4hf + head)
      float s4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[i] = sc[i] - m_ref[i];
      if (32 * (k + 1) > nvb && !cur.ok)
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = -INFINITY;
      const float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
      if (fresh || __builtin_amdgcn_ballot_w64(mx > TAU) != 0) {
        // exact per-head maximum over the super-tile, then raise the reference (or set it, first time)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float c = s4[i];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) c = fmaxf(c, __shfl_xor(c, o));
          const float d = fresh ? c : fmaxf(c, 0.0f);
          const float alpha = fresh ? 1.0f : __builtin_amdgcn_exp2f(-d);
#pragma unroll
          for (int w = 0; w < VT; ++w) acc[w][i] *= alpha;
          psum[i] *= alpha;
          s4[i] -= d;
          m_ref[i] += d;
        }
        fresh = false;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s4[i]);  // 2^-inf = 0
        psum[i] += p[i];
      }
      // P^T through LDS: token t's four probabilities, then the transposing read.  Lane group G (lanes
      // 16G..16G+15, half G / 2) reads the rows of tokens 16w + 8u + 4(G / 2) + (l % 16) / 4; lane i of the group
      // receives head i % 4 of those 4 tokens (k-slots 8hf + 4u + 0..3)
      if (hf == 0) {
        const h4 pv4 = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
        *(h4*)(pbuf + 4 * t) = pv4;
      }
      wave_sync();
      h8 pop[2];
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int tok = 16 * w + 8 * u + 4 * hf + (lane & 15) / 4;
          const h4 x = __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                  (__attribute__((address_space(3))) i16x4*)(pbuf + 4 * tok)));
          pop[w][4 * u + 0] = x[0];
          pop[w][4 * u + 1] = x[1];
          pop[w][4 * u + 2] = x[2];
          pop[w][4 * u + 3] = x[3];
        }
      // acc[head, coordinate] += sum_t p[head, t] v[t, coordinate]; rows replicate the 4 heads.  Tiles past the
      // super-tile's steps would add only zeros and are skipped.
#pragma unroll
      for (int w = 0; w < NT; ++w) {
        const f16v o = mfma32(pop[1], vop[w][1], mfma32(pop[0], vop[w][0], f16v{}));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[w][i] += o[i];
      }
    };

    auto run = [&](const Words& cur, int k) {
      if constexpr (VAR) {
        switch (cur.ns) {  // wave-uniform
          case 1: tile(Steps<1>{}, cur, k); break;
          case 2: tile(Steps<2 <= KS ? 2 : KS>{}, cur, k); break;
          case 3: tile(Steps<3 <= KS ? 3 : KS>{}, cur, k); break;
          default: tile(Steps<KS>{}, cur, k); break;
        }
      } else {
        tile(Steps<KS>{}, cur, k);
      }
    };
    // the wave's (at most) two super-tiles, the second's words read before the first is decoded
    if (nst_w > 0) {
      const Words w0 = fetch(0);
      Words w1 = {};
      if (nst_w > 1) w1 = fetch(1);
      run(w0, 0);
      if (nst_w > 1) run(w1, 1);
    }
    settle();  // the next page landed (and everyone is done with this buffer)
  }

  // ---- partial of the workgroup: the four waves' (m, l, acc) combined in LDS (the staging buffers are
  // idle now), then m[GQ], l[GQ], acc[GQ][2 VT * 16] (latent coordinates) for the merge; m = -inf when
  // the split holds no token
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float l = hf == 0 ? psum[i] : 0.0f;  // the two halves of the wave hold the same tokens
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
    psum[i] = l;
  }
  constexpr int NC = 2 * VT * 16;  // latent coordinates per head in the partial
  float* red = (float*)(smem + LY.stage);  // [wave][2 GQ + GQ NC]
  float* mine = red + wv * (2 * GQ + GQ * NC);
  if (lane < GQ) {
    mine[lane] = fresh ? -INFINITY : m_ref[lane];
    mine[GQ + lane] = psum[lane];
  }
  if (hf == 0)
#pragma unroll
    for (int w = 0; w < VT; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[2 * GQ + i * NC + 32 * w + t] = acc[w][i];
  __syncthreads();
  float* part = a.ws + (size_t)((b * a.Hkv + h) * a.n_splits + split) * a.part_stride;
  for (int e = tid; e < GQ * NC; e += 256) {
    const int hq = e / NC, c = e % NC;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, red[w * (2 * GQ + GQ * NC) + hq]);
    float av = 0.0f, lv = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* pw = red + w * (2 * GQ + GQ * NC);
      const float wt = pw[hq] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(pw[hq] - mx);
      av += wt * pw[2 * GQ + hq * NC + c];
      lv += wt * pw[GQ + hq];
    }
    part[2 * GQ + hq * NC + c] = av;
    if (c == 0) {
      part[hq] = mx;
      part[GQ + hq] = lv;
    }
  }
}

// Final combine over the context splits and the value basis: one workgroup of 256 threads per (sequence, KV head).
// Thread (hq, c) = (t / NC, t % NC) combines c*[hq][c] = sum_s 2^(m_s - m*) acc_s and l*[hq] = sum_s 2^(m_s - m*) l_s
// over the splits; thread t then computes out[d] = (B_v c*)[d] / l* for d = t % 128 and the query heads 2 (t / 128)
// and 2 (t / 128) + 1, with the basis row d loaded once for both.  The kernel is a chain of memory round trips, so
// its loads are issued together: the value basis row at the start, then every split's (m, l, acc) in groups of up to
// 16, combined with a running maximum (the same value as a maximum taken first, up to rounding).  The four query
// heads of a KV head share one workgroup, so the basis rows are read once per KV head.
template <int NC>
__global__ __launch_bounds__(256) void merge_int4_kernel(const float* ws, const uint16_t* wv, float* out, int Hkv,
                                                          int Hq, int rv, int n_splits, int part_stride) {
  constexpr int NB = NC / 8;  // 16-byte groups of the value basis row
  constexpr int SG = 16;      // splits loaded together
  static_assert(i4::GQ * NC <= 256 && i4::D * 2 == 256, "thread mapping");
  __shared__ float cst[i4::GQ][NC];
  __shared__ float lst[i4::GQ];
  const int bh = blockIdx.x, h = bh % Hkv, b = bh / Hkv;
  const int tid = threadIdx.x;
  const int d = tid % i4::D, hp = tid / i4::D;  // output dim, pair of query heads
  const uint16_t* row = wv + ((size_t)h * i4::D + d) * rv;  // B_v row d, rv bf16 values
  u4 braw[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) braw[i] = 8 * i < rv ? *(const u4*)(row + 8 * i) : u4{0, 0, 0, 0};
  const float* parts = ws + (size_t)(b * Hkv + h) * n_splits * part_stride;
  if (tid < i4::GQ * NC) {
    const int hq = tid / NC, c = tid % NC;
    float mx = -INFINITY, cc = 0.0f, l = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += SG) {
      float ms[SG], ls[SG], as[SG];
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        const bool ok = s0 + u < n_splits;
        const float* ps = parts + (size_t)(ok ? s0 + u : 0) * part_stride;
        ms[u] = ok ? ps[hq] : -INFINITY;
        ls[u] = ok ? ps[i4::GQ + hq] : 0.0f;
        as[u] = ok ? ps[2 * i4::GQ + hq * NC + c] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        if (ms[u] == -INFINITY) continue;  // a split with no token
        const float mn = fmaxf(mx, ms[u]);
        const float a0 = mx == -INFINITY ? 0.0f : exp2f(mx - mn), a1 = exp2f(ms[u] - mn);
        cc = cc * a0 + a1 * as[u];
        l = l * a0 + a1 * ls[u];
        mx = mn;
      }
    }
    cst[hq][c] = cc;
    if (c == 0) lst[hq] = l;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int hq = 2 * hp + k;
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (8 * i >= rv) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = braw[i][e >> 1];
        o += __builtin_bit_cast(float, (e & 1) ? (w & 0xFFFF0000u) : (w << 16)) * cst[hq][8 * i + e];
      }
    }
    out[((size_t)b * Hq + h * i4::GQ + hq) * i4::D + d] = o / lst[hq];
  }
}

template <int KS, int VS, bool VAR, int STG, int KB, int VB>
static hipError_t launch_int4(const Int4Args& a, int grid, const uint16_t* wv, float* out, hipStream_t st) {
  const int lds = i4::lds_layout(a.P, a.hb_max).total;
  auto kern = decode_int4_kernel<KS, VS, VAR, STG, KB, VB>;
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
  constexpr int NC = 32 * ((VS + 1) / 2);
  hipLaunchKernelGGL((merge_int4_kernel<NC>), dim3(a.B * a.Hkv), dim3(256), 0, st, a.ws, wv, out, a.Hkv, a.Hq, a.rv,
                     a.n_splits, a.part_stride);
  return hipGetLastError();
}

int int4_max_pages_per_split() { return i4::MAX_SPLIT_PAGES; }

// The compiled variants (key steps, value steps, variable rank, staging chunks, key bits, value bits), used both to
// decide support and to launch, so that a layout this kernel accepts always has a variant.
#define KVC_INT4_VARIANTS(X)  \
  X(4, 4, true, 5, 4, 4)      \
  X(4, 4, false, 5, 4, 4)     \
  X(3, 4, false, 5, 4, 4)     \
  X(2, 2, true, 3, 4, 4)      \
  X(2, 2, false, 3, 4, 4)     \
  X(4, 4, true, 5, 3, 3)      \
  X(4, 4, true, 5, 2, 2)      \
  X(4, 4, false, 5, 3, 3)     \
  X(4, 4, false, 5, 3, 2)     \
  X(3, 4, false, 5, 3, 3)     \
  X(3, 4, false, 5, 3, 2)     \
  X(3, 4, false, 5, 2, 2)

static bool int4_has_variant(int KS, int VS, bool var, int stg, int kb, int vb) {
#define KVC_HAS(KS_, VS_, VAR_, STG_, KB_, VB_) \
  if (KS == KS_ && VS == VS_ && var == VAR_ && stg <= STG_ && kb == KB_ && vb == VB_) return true;
  KVC_INT4_VARIANTS(KVC_HAS)
#undef KVC_HAS
  return false;
}

bool int4_supported(const kvc_layout& L, int64_t hb_max) {
  if (L.shared || L.residual_bits || L.head_dim != 128 || L.latent_bits == 32) return false;
  if (!int4_has_variant(ceil_div(L.r_k_cap, 16), ceil_div(L.r_v_cap, 16), L.variable_rank != 0,
                        ceil_div((int)hb_max, 16 * 256), lat_bits_k(L), lat_bits_v(L)))
    return false;
  if (L.n_q_heads != i4::GQ * L.n_kv_heads) return false;
  if (L.r_k_cap > 64 || L.r_v_cap > 64 || L.r_k_cap < 17 || L.r_v_cap < 17 || L.group % 16) return false;
  if (L.variable_rank && L.r_k_cap != L.r_v_cap) return false;
  if (hb_max > 16 * 256 * 5) return false;
  // two workgroups per compute unit: dynamic and static LDS within half of the 160 KiB
  return i4::lds_layout(L.page_size, (int)hb_max).total + i4::STATIC_LDS <= 80 * 1024;
}

hipError_t launch_decode_int4(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out, void* ws,
                              int n_splits, int pages_per_split, int part_stride, const HeadSections& S_uniform,
                              int hb_max, hipStream_t st) {
  Int4Args a;
  a.pool = C.pool; a.page_off = C.page_off; a.tok_off = C.tok_off;
  a.block_table = in.block_table; a.seq_len = in.seq_len; a.q_pos = in.q_pos; a.q = in.q; a.wk = in.wk;
  a.ws = (float*)ws; a.q_bf16 = in.q_dtype == KVC_BF16;
  a.B = in.B; a.Hkv = L.n_kv_heads; a.Hq = L.n_q_heads; a.max_blocks = in.max_blocks; a.P = L.page_size;
  a.rk = L.r_k_cap; a.rv = L.r_v_cap; a.G = L.group; a.n_splits = n_splits; a.pages_per_split = pages_per_split;
  a.part_stride = part_stride; a.hb_max = hb_max; a.theta = L.rope_theta; a.S_uniform = S_uniform;
  const int grid = in.B * L.n_kv_heads * n_splits;
  const int KS = ceil_div(L.r_k_cap, 16), VS = ceil_div(L.r_v_cap, 16);
  const bool var = L.variable_rank != 0;
  const int stg = ceil_div(hb_max, 16 * 256);
  const int kb = lat_bits_k(L), vb = lat_bits_v(L);
#define KVC_TRY4(KS_, VS_, VAR_, STG_, KB_, VB_)                                              \
  if (KS == KS_ && VS == VS_ && var == VAR_ && stg <= STG_ && kb == KB_ && vb == VB_)         \
    return launch_int4<KS_, VS_, VAR_, STG_, KB_, VB_>(a, grid, in.wv, out, st);
  KVC_INT4_VARIANTS(KVC_TRY4)
#undef KVC_TRY4
  return hipErrorInvalidValue;
}

}  // namespace kvc
