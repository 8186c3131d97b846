// evict.hip -- block-level eviction decision: one token keep mask per sequence for a block of layers (prefill
// side).  Layers of a block rank token importance alike, so one decision made from all the block's layers'
// scores is applied once to the shared latent (BellowsKV page, "Three Measurements, Three Operators" and "Key
// Findings").
//
// A token's block score is the fp32 sum of its per-layer scores in layer order (plain additions, no fused
// arithmetic, so the host's fp32 sums are bit-identical).  Sequence b of T tokens keeps
// n = min(T, max(1, floor(keep_ratio T))) of them: the n largest block scores, equal scores taken in increasing
// position.  One workgroup per sequence: bisection over the 32-bit order key of the block score finds the
// n-th largest key K (32 counting passes); tokens above K are kept, and tokens equal to K in position order
// until n are kept (a workgroup prefix count over 1024-token chunks).  Each wave writes the two mask words of
// its 64 tokens from one ballot.  Up to 32768 tokens per sequence the keys are computed once into LDS and the
// passes read them there; longer sequences recompute them from the scores in every pass.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kvc_common.hpp"

namespace kvc {

namespace {

constexpr int ET = 1024;             // threads per workgroup
constexpr int EVICT_LDS_TOKENS = 32768;  // keys staged in LDS up to this many tokens per sequence

struct EvictArgs {
  const float* scores;  // [n_layers][B][max_T]
  const int32_t* seq_len;
  uint32_t* mask;       // [B][words]
  int B, max_T, n_layers, words;
  double keep_ratio;
};

// increasing in f over all non-NaN floats, with -0 and +0 the same key
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint32_t key_at(const EvictArgs& e, const float* s, int t) {
  const size_t ls = (size_t)e.B * e.max_T;
  float a = s[t];
  for (int l = 1; l < e.n_layers; ++l) a = a + s[(size_t)l * ls + t];
  return order_key(a);
}

template <bool STAGE>
__global__ __launch_bounds__(ET) void evict_select_kernel(EvictArgs e) {
  __shared__ int red[ET / 64];
  extern __shared__ uint32_t keys[];  // STAGE: the sequence's keys
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = max(0, min(e.seq_len[b], e.max_T));  // (a length outside 0..max_T is the caller's error)
  const float* s = e.scores + (size_t)b * e.max_T;
  uint32_t* out = e.mask + (size_t)b * e.words;
  const int n_keep = T <= 0 ? 0 : min(T, max(1, (int)floor(e.keep_ratio * (double)T)));
  if (STAGE) {
    for (int t = tid; t < T; t += ET) keys[t] = key_at(e, s, t);
    __syncthreads();
  }
  auto key = [&](int t) { return STAGE ? keys[t] : key_at(e, s, t); };

  // workgroup sum of one int per thread (every thread gets it)
  auto wg_sum = [&](int c) {
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    if (lane == 0) red[wv] = c;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int i = 0; i < ET / 64; ++i) tot += red[i];
    __syncthreads();
    return tot;
  };
  auto count_ge = [&](uint32_t K) {
    int c = 0;
    for (int t = tid; t < T; t += ET) c += key(t) >= K;
    return wg_sum(c);
  };

  uint32_t K = 0xFFFFFFFFu;
  int need = 0;
  if (n_keep > 0) {
    // largest K with at least n_keep keys >= K (K = 0 always qualifies: every key counts)
    uint32_t lo = 0, hi = 0xFFFFFFFFu;
    while (lo < hi) {
      const uint32_t mid = (uint32_t)(((uint64_t)lo + hi + 1) >> 1);
      if (count_ge(mid) >= n_keep)
        lo = mid;
      else
        hi = mid - 1;
    }
    K = lo;
    need = n_keep - (K == 0xFFFFFFFFu ? 0 : count_ge(K + 1));  // ties at K to keep, in position order
  }

  int before = 0;  // tokens equal to K in earlier chunks
  for (int base = 0; base < e.words * 32; base += ET) {
    const int t = base + tid;
    bool gt = false, eq = false;
    if (n_keep > 0 && t < T) {
      const uint32_t k = key(t);
      gt = k > K;
      eq = k == K;
    }
    const uint64_t eb = __builtin_amdgcn_ballot_w64(eq);
    const int in_wave = __builtin_popcountll(eb & ((1ull << lane) - 1ull));
    if (lane == 0) red[wv] = __builtin_popcountll(eb);
    __syncthreads();
    int wave_off = 0, chunk = 0;
#pragma unroll
    for (int i = 0; i < ET / 64; ++i) {
      wave_off += i < wv ? red[i] : 0;
      chunk += red[i];
    }
    __syncthreads();
    const bool keep = gt || (eq && before + wave_off + in_wave < need);
    const uint64_t kb = __builtin_amdgcn_ballot_w64(keep);
    const int w = (base + 64 * wv + (lane & 32)) >> 5;
    if ((lane & 31) == 0 && w < e.words) out[w] = (uint32_t)(kb >> (lane & 32));
    before += chunk;
  }
}

// ---- compaction of the evicted tokens (block-shared cache): kept tokens in position order into tiles of CT = 32
// slots, a tile spanning at most CSPAN blocks of 32 positions from its first token's block; each slot records its
// source position.
constexpr int CT = 32, CSPAN = 4;
constexpr int CMAX_BLOCKS = 8192;  // 32-position blocks per sequence: two LDS words each

struct CompactArgs {
  const uint8_t* src;
  const int64_t* src_off;
  const int32_t* bt;
  const int32_t* seq_len;
  const uint32_t* keep;
  uint8_t* dst;
  const int64_t* dst_off;
  const int32_t* obt;
  int32_t* out_len;
  int32_t* tok_pos;
  int keep_words, max_blocks, P, cb, moff, mb;
};

// One workgroup per sequence.  The tile rule is a left-to-right recurrence, but it only changes state at a
// block's first kept token, so wave 0 walks the blocks with wave-uniform (scalar) state: 64 mask words at a time
// are loaded into its lanes and read back one by one, a popcount each, giving each block the slot of its first
// kept token; within a block the kept tokens take consecutive slots (a tile that fills mid-block continues in the
// next slot, which opens the next tile with the same block as its base).  Then every thread writes the positions
// of its blocks' tokens, after the row is set to -1.
__global__ __launch_bounds__(256) void compact_scan_kernel(CompactArgs a) {
  extern __shared__ uint32_t cl[];  // [n_blk] keep words, then [n_blk] first slots
  const int b = blockIdx.x, tid = threadIdx.x;
  const int row = a.max_blocks * a.P;
  const int T = max(0, min(min(a.seq_len[b], row), 32 * a.keep_words));
  const int n_blk = (T + 31) / 32;
  uint32_t* words = cl;
  int* first = (int*)(cl + n_blk);
  for (int i = tid; i < n_blk; i += 256) {
    uint32_t w = a.keep[(size_t)b * a.keep_words + i];
    const int left = T - 32 * i;  // positions of this block below T
    if (left < 32) w &= (1u << left) - 1u;
    words[i] = w;
  }
  int32_t* pos = a.tok_pos + (size_t)b * row;
  for (int i = tid; i < row; i += 256) pos[i] = -1;
  __syncthreads();
  if (tid < 64) {  // wave 0; slot, count and base are the same in every lane
    const int lane = tid;
    int slot = 0, count = 0, base = 0;
    for (int c0 = 0; c0 < n_blk; c0 += 64) {
      const uint32_t wl = c0 + lane < n_blk ? words[c0 + lane] : 0u;
      int fr = 0;
      const int m = min(64, n_blk - c0);
      for (int j = 0; j < m; ++j) {
        const int c = __builtin_popcount((uint32_t)__builtin_amdgcn_readlane((int)wl, j));
        if (c == 0) continue;
        const int i = c0 + j;
        if (count > 0 && i - base >= CSPAN) {  // out of the tile's span: close it, its spare slots stay empty
          slot = (slot + CT - 1) / CT * CT;
          count = 0;
        }
        if (count == 0) base = i;
        fr = lane == j ? slot : fr;
        slot += c;
        count += c;
        if (count >= CT) {  // the tile filled at one of this block's tokens; the rest open the next tile here
          count -= CT;
          base = i;
        }
      }
      if (c0 + lane < n_blk) first[c0 + lane] = fr;
    }
    if (lane == 0) a.out_len[b] = slot;
  }
  __syncthreads();
  for (int i = tid; i < n_blk; i += 256) {
    uint32_t w = words[i];
    int s = first[i];
    while (w) {
      pos[s++] = 32 * i + __builtin_ctz(w);
      w &= w - 1u;
    }
  }
}

// One workgroup per (sequence, destination page): every slot of a page below the compacted length gets its
// token's code and pair bytes, or zeros (no token); pages past it are left alone.  Dword copies (code and pair
// sections of a slot are whole dwords).
__global__ __launch_bounds__(256) void compact_copy_kernel(CompactArgs a) {
  const int b = blockIdx.x / a.max_blocks, i = blockIdx.x % a.max_blocks;
  const int len = a.out_len[b];
  if (i * a.P >= len) return;
  const int row = a.max_blocks * a.P;
  const int32_t* pos = a.tok_pos + (size_t)b * row + (size_t)i * a.P;
  uint32_t* dst = (uint32_t*)(a.dst + a.dst_off[a.obt[(size_t)b * a.max_blocks + i]]);
  const int cw = a.cb / 4, mw = a.mb / 4;
  for (int e = threadIdx.x; e < a.P * (cw + mw); e += 256) {
    const bool code = e < a.P * cw;
    const int s = code ? e / cw : (e - a.P * cw) / mw;
    const int k = code ? e % cw : (e - a.P * cw) % mw;
    const int p = i * a.P + s < len ? pos[s] : -1;
    uint32_t v = 0u;
    if (p >= 0) {
      const uint32_t* src = (const uint32_t*)(a.src + a.src_off[a.bt[(size_t)b * a.max_blocks + p / a.P]]);
      v = code ? src[(p % a.P) * cw + k] : src[a.moff / 4 + (p % a.P) * mw + k];
    }
    if (code)
      dst[s * cw + k] = v;
    else
      dst[a.moff / 4 + s * mw + k] = v;
  }
}

}  // namespace

bool shared_supported(const kvc_layout& L);

kvc_status compact_impl(const kvc_layout& L, const kvc_cache& src, const kvc_cache& dst, const kvc_compact_in& in,
                        int32_t* out_len, int32_t* tok_pos, hipStream_t st) {
  if (!L.shared) return KVC_ERR_INVALID_ARG;
  if (in.B < 1 || in.max_blocks < 1 || in.keep_words < 1 || !in.block_table || !in.seq_len || !in.keep_mask ||
      !in.out_block_table || !out_len || !tok_pos || !src.pool || !src.page_off || !dst.pool || !dst.page_off)
    return KVC_ERR_INVALID_ARG;
  if ((int64_t)in.max_blocks * L.page_size > (int64_t)32 * CMAX_BLOCKS || in.B > (1 << 20)) return KVC_ERR_INVALID_ARG;
  if (!shared_supported(L) || L.residual_bits) return KVC_ERR_UNSUPPORTED;  // (records with residuals: not moved)
  const void* ptrs[] = {in.block_table, in.seq_len, in.out_block_table, out_len, tok_pos, src.pool, src.page_off,
                        dst.pool, dst.page_off};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return KVC_ERR_MISALIGNED;
  if ((uintptr_t)in.keep_mask & 3) return KVC_ERR_MISALIGNED;
  CompactArgs a;
  a.src = src.pool; a.src_off = src.page_off; a.bt = in.block_table; a.seq_len = in.seq_len; a.keep = in.keep_mask;
  a.dst = dst.pool; a.dst_off = dst.page_off; a.obt = in.out_block_table; a.out_len = out_len; a.tok_pos = tok_pos;
  a.keep_words = in.keep_words; a.max_blocks = in.max_blocks; a.P = L.page_size;
  a.cb = L.r_k_cap * L.latent_bits / 8;
  a.moff = (int)pad16((int64_t)L.page_size * a.cb);
  a.mb = 4 * (L.r_k_cap / L.group);
  const int n_blk = (in.max_blocks * L.page_size + 31) / 32;
  const int lds = 8 * n_blk;
  hipError_t err = hipFuncSetAttribute((const void*)compact_scan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return hip_fail(err);
  hipLaunchKernelGGL(compact_scan_kernel, dim3(in.B), dim3(256), lds, st, a);
  if ((err = hipGetLastError()) != hipSuccess) return hip_fail(err);
  hipLaunchKernelGGL(compact_copy_kernel, dim3(in.B * in.max_blocks), dim3(256), 0, st, a);
  err = hipGetLastError();
  return err == hipSuccess ? KVC_OK : hip_fail(err);
}

kvc_status evict_impl(const kvc_evict_in& in, uint32_t* mask, hipStream_t st) {
  if (in.B < 1 || in.max_T < 1 || in.n_layers < 1 || !in.seq_len || !in.scores || !mask) return KVC_ERR_INVALID_ARG;
  if (!(in.keep_ratio > 0.0) || in.keep_ratio > 1.0) return KVC_ERR_INVALID_ARG;
  if ((int64_t)in.n_layers * in.B * in.max_T > ((int64_t)1 << 40) || in.B > (1 << 24)) return KVC_ERR_INVALID_ARG;
  const void* ptrs[] = {in.seq_len, in.scores, mask};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 3) return KVC_ERR_MISALIGNED;
  EvictArgs e{in.scores, in.seq_len, mask, in.B, in.max_T, in.n_layers, (in.max_T + 31) / 32, in.keep_ratio};
  hipError_t err;
  if (in.max_T <= EVICT_LDS_TOKENS) {
    const int lds = in.max_T * 4;
    err = hipFuncSetAttribute((const void*)evict_select_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return hip_fail(err);
    hipLaunchKernelGGL(evict_select_kernel<true>, dim3(in.B), dim3(ET), lds, st, e);
  } else {
    hipLaunchKernelGGL(evict_select_kernel<false>, dim3(in.B), dim3(ET), 0, st, e);
  }
  err = hipGetLastError();
  return err == hipSuccess ? KVC_OK : hip_fail(err);
}

}  // namespace kvc
