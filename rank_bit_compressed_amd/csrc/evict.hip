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

}  // namespace

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
