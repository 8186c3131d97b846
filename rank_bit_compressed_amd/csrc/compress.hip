// compress.hip -- the prefill side: quantize and pack latents into the paged pool (gfx950).
//
// Steps (all on the caller's stream; no host synchronization):
//   1. clear the pool and tables (fill kernels, so the sequence can be graph-captured);
//   2. variable rank: scatter each token's rank to its (page, slot);
//   3. per page: exclusive prefix of ranks and group counts over slots (tok_off), record size;
//   4. exclusive prefix of record sizes over pages (page_off) and the total (used_bytes);
//   5. one thread per (token, head, K|V, group): INT4 min/max quantizer, nibble packing, pair store;
//      one thread per (token, head, K|V): 2-bit quantizer of the rotated residual.
// From dense K/V, a projection kernel first writes the fp32 latents c = B_r^T x (truncated to the
// token's rank) and the rotated truncation residual H (x - B_r c), which step 5 then quantizes.
//
// The quantizers reproduce IEEE fp32 round-to-nearest-even arithmetic step by step (no
// contraction into FMA, correctly rounded division) so that codes are bit-exact.
#include <math.h>

#include <algorithm>

#include "kvc_common.hpp"

namespace kvc {

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void scatter_ranks_kernel(const int32_t* block_table, const int32_t* seq_len, const uint8_t* ranks,
                                     uint8_t* tok_rank, int max_T, int max_blocks, int P, int cap) {
  const int b = blockIdx.y;
  const int T = seq_len[b];
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
    int r = ranks[(size_t)b * max_T + t];
    r = min(max(r & ~7, 8), cap);  // out-of-contract ranks are clamped (documented as undefined)
    const int page = block_table[(size_t)b * max_blocks + t / P];
    tok_rank[(size_t)page * P + t % P] = (uint8_t)r;
  }
}

// One workgroup per page: tok_off prefix over slots and the page record size (into page_off).
__global__ __launch_bounds__(256) void page_prefix_kernel(const uint8_t* tok_rank, uint32_t* tok_off,
                                                          int64_t* page_off, int P, int G, int Hkv, int residual,
                                                          int d, int bits) {
  __shared__ uint32_t sr[256], sg[256];
  const int page = blockIdx.x, s = threadIdx.x;
  const uint32_t r = s < P ? tok_rank[(size_t)page * P + s] : 0u;
  const uint32_t gcount = (r + G - 1) / G;
  sr[s] = r;
  sg[s] = gcount;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
    const uint32_t a = s >= off ? sr[s - off] : 0u, c = s >= off ? sg[s - off] : 0u;
    __syncthreads();
    sr[s] += a;
    sg[s] += c;
    __syncthreads();
  }
  if (s < P) tok_off[(size_t)page * (P + 1) + s] = (sr[s] - r) | ((sg[s] - gcount) << 16);
  if (s == P - 1) {
    tok_off[(size_t)page * (P + 1) + P] = sr[s] | (sg[s] << 16);
    const int64_t cb = (int64_t)sr[s] * bits / 8, mb = 4 * (int64_t)sg[s];
    page_off[page] = head_sections(cb, cb, mb, mb, P, d, residual).hb * Hkv;
  }
}

// Exclusive prefix of page record sizes, in place; writes the total.  One workgroup.
__global__ __launch_bounds__(1024) void page_scan_kernel(int64_t* page_off, int n_pages, int64_t uniform_size,
                                                         int64_t* used_bytes) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  const int per = (n_pages + 1023) / 1024;
  const int lo = min(n_pages, tid * per), hi = min(n_pages, lo + per);
  int64_t sum = 0;
  for (int p = lo; p < hi; ++p) sum += uniform_size >= 0 ? uniform_size : page_off[p];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int64_t x = part[i];
      part[i] = run;
      run += x;
    }
    if (used_bytes) *used_bytes = run;
  }
  __syncthreads();
  int64_t run = part[tid];
  for (int p = lo; p < hi; ++p) {
    const int64_t sz = uniform_size >= 0 ? uniform_size : page_off[p];
    page_off[p] = run;
    run += sz;
  }
}

#pragma clang fp contract(off)

__device__ inline uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ inline float f16_val(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

struct PackArgs {
  const int32_t* block_table;
  const int32_t* seq_len;
  const float* lat_k;
  const float* lat_v;
  const float* res_k;
  const float* res_v;
  uint8_t* pool;
  const int64_t* page_off;
  const uint8_t* tok_rank;
  const uint32_t* tok_off;
  int B, max_T, max_blocks, P, Hkv, d, rk, rv, G, latent_bits, latent_bits_v, residual, variable_rank, shared;
  int n_layers;  // shared mode: layers with their own residuals
  int64_t lat_bytes;  // shared mode: bytes of the latent's sections of a record
  HeadSections S_uniform;
};

// Thread = (b, t, head, which, group).  Groups of G coordinates from coordinate 0; the last may be short.
__global__ __launch_bounds__(256) void pack_latent_kernel(PackArgs a, int groups_per_item) {
  const int items_per_tok = a.shared ? 1 : 2 * a.Hkv;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)items_per_tok * groups_per_item;
  const int64_t tok = idx / per_tok;
  if (tok >= (int64_t)a.B * a.max_T) return;
  const int b = (int)(tok / a.max_T), t = (int)(tok % a.max_T);
  if (t >= a.seq_len[b]) return;
  const int item = (int)((idx % per_tok) / groups_per_item), gi = (int)(idx % groups_per_item);
  const int P = a.P, page = a.block_table[(size_t)b * a.max_blocks + t / P], slot = t % P;
  uint8_t* rec = a.pool + a.page_off[page];
  const float* src;
  uint8_t* codes;
  uint8_t* meta;
  int r, bits = a.latent_bits;
  if (a.shared) {
    r = a.rk;
    src = a.lat_k + ((size_t)b * a.max_T + t) * r;
    codes = rec + (int64_t)slot * (r * bits / 8);
    meta = rec + pad16((int64_t)P * r * bits / 8) + (int64_t)slot * 4 * ceil_div(r, a.G);
  } else {
    const int h = item >> 1, which = item & 1;
    const int rcap = which ? a.rv : a.rk;
    bits = which ? a.latent_bits_v : a.latent_bits;
    HeadSections S;
    int64_t co, mo;
    if (a.variable_rank) {
      const uint32_t tot = a.tok_off[(size_t)page * (P + 1) + P], o = a.tok_off[(size_t)page * (P + 1) + slot];
      const int64_t cb = (int64_t)(tot & 0xFFFFu) * bits / 8, mb = 4 * (int64_t)(tot >> 16);  // K, V share bits
      S = head_sections(cb, cb, mb, mb, P, a.d, a.residual);
      r = a.tok_rank[(size_t)page * P + slot];
      co = (int64_t)(o & 0xFFFFu) * bits / 8;
      mo = 4 * (int64_t)(o >> 16);
    } else {
      S = a.S_uniform;
      r = rcap;
      co = (int64_t)slot * slot_code_bytes(bits, r);
      mo = (int64_t)slot * slot_meta_bytes(bits, r, a.G);
    }
    uint8_t* hb = rec + (int64_t)h * S.hb;
    src = (which ? a.lat_v : a.lat_k) + (((size_t)b * a.max_T + t) * a.Hkv + h) * rcap;
    codes = hb + (which ? S.vc : S.kc) + co;
    meta = hb + (which ? S.vm : S.km) + mo;
  }
  if (bits == 32) {  // fp32 latents: one thread copies the token's r values
    if (gi == 0)
      for (int i = 0; i < r; ++i) ((float*)codes)[i] = src[i];
    return;
  }
  const int g0 = gi * a.G;
  if (g0 >= r) return;
  const int n = min(a.G, r - g0);
  float lo = src[g0], hi = src[g0];
  for (int i = 1; i < n; ++i) {  // strict comparisons: the first of equal values (e.g. -0 and +0) is kept
    const float x = src[g0 + i];
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
  }
  const float levels = (float)((1 << bits) - 1);
  const float s32 = __fdiv_rn(hi - lo, levels);
  const uint16_t s16 = f16_bits(s32), z16 = f16_bits(lo);
  const float s = f16_val(s16), z = f16_val(z16);
  for (int i0 = 0; i0 < n; i0 += 8) {  // n is a multiple of 8: 8 codes fill `bits` whole bytes
    uint32_t word = 0;
    for (int j = 0; j < 8; ++j) {
      uint32_t q = 0;
      if (s != 0.0f) {
        const float ratio = __fdiv_rn(__fsub_rn(src[g0 + i0 + j], z), s);
        q = (uint32_t)fminf(fmaxf(rintf(ratio), 0.0f), levels);
      }
      word |= q << (bits * j);
    }
    uint8_t* dst = codes + (g0 + i0) * bits / 8;
    for (int k = 0; k < bits; ++k) dst[k] = (uint8_t)(word >> (8 * k));
  }
  *(uint32_t*)(meta + 4 * gi) = (uint32_t)s16 | ((uint32_t)z16 << 16);
}

// Thread = (b, t, [layer,] head, which): 2-bit quantizer of the 128-value rotated residual.  Block-shared mode:
// one residual per (layer, head), res_k / res_v [B][max_T][n_layers][Hkv][d].
__global__ __launch_bounds__(256) void pack_residual_kernel(PackArgs a) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int nl = a.shared ? a.n_layers : 1;
  const int64_t tok = idx / (2 * a.Hkv * nl);
  if (tok >= (int64_t)a.B * a.max_T) return;
  const int b = (int)(tok / a.max_T), t = (int)(tok % a.max_T);
  if (t >= a.seq_len[b]) return;
  const int lh = (int)(idx % (2 * a.Hkv * nl)) >> 1, which = (int)(idx & 1);  // lh = layer * Hkv + head
  const int h = lh % a.Hkv;
  const int P = a.P, page = a.block_table[(size_t)b * a.max_blocks + t / P], slot = t % P;
  const float* y = (which ? a.res_v : a.res_k) + (((size_t)b * a.max_T + t) * a.Hkv * nl + lh) * a.d;
  uint8_t* codes;
  uint16_t* scale;
  if (a.shared) {
    uint8_t* rec = a.pool + a.page_off[page];
    const int n = a.n_layers * a.Hkv;
    codes = rec + shared_res_part(a.lat_bytes, P, a.d, n, which, lh) + (int64_t)slot * (a.d / 4);
    scale = (uint16_t*)(rec + shared_res_part(a.lat_bytes, P, a.d, n, 2 + which, lh)) + slot;
  } else {
    HeadSections S;
    if (a.variable_rank) {
      const uint32_t tot = a.tok_off[(size_t)page * (P + 1) + P];
      const int64_t cb = (int64_t)(tot & 0xFFFFu) * a.latent_bits / 8, mb = 4 * (int64_t)(tot >> 16);
      S = head_sections(cb, cb, mb, mb, P, a.d, 1);
    } else {
      S = a.S_uniform;
    }
    uint8_t* hb = a.pool + a.page_off[page] + (int64_t)h * S.hb;
    codes = hb + (which ? S.vr : S.kr) + (int64_t)slot * (a.d / 4);
    scale = (uint16_t*)(hb + (which ? S.vs : S.ks)) + slot;
  }
  float amax = 0.0f;
  for (int i = 0; i < a.d; ++i) {
    const float m = fabsf(y[i]);
    amax = m > amax ? m : amax;
  }
  const uint16_t s16 = f16_bits(__fdiv_rn(amax, 1.5f));
  const float s = f16_val(s16);
  for (int i0 = 0; i0 < a.d; i0 += 16) {
    uint32_t word = 0;
    for (int j = 0; j < 16; ++j) {
      uint32_t c = 2;
      if (s != 0.0f) {
        const float v = __fadd_rn(__fdiv_rn(y[i0 + j], s), 1.5f);
        c = (uint32_t)fminf(fmaxf(rintf(v), 0.0f), 3.0f);
      }
      word |= c << (2 * j);
    }
    *(uint32_t*)(codes + i0 / 4) = word;
  }
  *scale = s16;
}

#pragma clang fp contract(on)

// From dense: one wave per (b, t, head, which).  c_i = sum_j B[j][i] x_j over i < r (fp32, j ascending),
// e_j = x_j - sum_{i<r} B[j][i] c_i, y = H e with the normalized Sylvester Hadamard (fast transform
// in LDS, log2(d) butterfly stages, then the 1/sqrt(d) scale).
__global__ __launch_bounds__(256) void project_kernel(const float* k, const float* v, const uint16_t* basis_k,
                                                      const uint16_t* basis_v, const uint8_t* ranks,
                                                      const int32_t* seq_len, float* lat_k, float* lat_v,
                                                      float* res_k, float* res_v, int B, int max_T, int Hkv, int d,
                                                      int rk, int rv, int variable_rank, int residual) {
  __shared__ float xs[4][128], cs[4][64], es[4][128];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = blockIdx.x * 4LL + wv;
  if (item >= (int64_t)B * max_T * Hkv * 2) return;
  const int which = (int)(item & 1);
  const int64_t th = item >> 1;
  const int h = (int)(th % Hkv);
  const int64_t tok = th / Hkv;
  const int b = (int)(tok / max_T), t = (int)(tok % max_T);
  if (t >= seq_len[b]) return;
  const int rcap = which ? rv : rk;
  const int r = variable_rank ? min((int)ranks[(size_t)b * max_T + t], rcap) : rcap;
  const float* x = (which ? v : k) + (((size_t)b * max_T + t) * Hkv + h) * d;
  const uint16_t* Bm = (which ? basis_v : basis_k) + (size_t)h * d * rcap;
  for (int j = lane; j < d; j += 64) xs[wv][j] = x[j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  float* c_out = (which ? lat_v : lat_k) + (((size_t)b * max_T + t) * Hkv + h) * rcap;
  for (int i = lane; i < rcap; i += 64) {
    float acc = 0.0f;
    if (i < r)
      for (int j = 0; j < d; ++j) acc = fmaf(__builtin_bit_cast(float, (uint32_t)Bm[(size_t)j * rcap + i] << 16), xs[wv][j], acc);
    c_out[i] = acc;
    if (i < 64) cs[wv][i] = acc;
  }
  if (!residual) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  for (int j = lane; j < d; j += 64) {
    float acc = 0.0f;
    for (int i = 0; i < r; ++i) acc = fmaf(__builtin_bit_cast(float, (uint32_t)Bm[(size_t)j * rcap + i] << 16), cs[wv][i], acc);
    es[wv][j] = xs[wv][j] - acc;
  }
  for (int hstep = 1; hstep < d; hstep <<= 1) {  // Sylvester order: pairs (i, i + hstep) in blocks of 2*hstep
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    float lo_v = 0.0f, hi_v = 0.0f;
    int i0 = 0;
    if (lane < d / 2) {
      const int blk = lane / hstep, off = lane % hstep;
      i0 = blk * 2 * hstep + off;
      const float a0 = es[wv][i0], a1 = es[wv][i0 + hstep];
      lo_v = a0 + a1;
      hi_v = a0 - a1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    if (lane < d / 2) {
      es[wv][i0] = lo_v;
      es[wv][i0 + hstep] = hi_v;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  float* y_out = (which ? res_v : res_k) + (((size_t)b * max_T + t) * Hkv + h) * d;
  const float sc = 1.0f / sqrtf((float)d);
  for (int j = lane; j < d; j += 64) y_out[j] = es[wv][j] * sc;
}

static bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

kvc_status compress_impl(const kvc_layout& L, const kvc_compress_in& in, const kvc_cache& C, hipStream_t st) {
  if (in.mode != KVC_FROM_LATENT && in.mode != KVC_FROM_DENSE) return KVC_ERR_INVALID_ARG;
  if (in.B <= 0 || in.max_T <= 0 || in.max_blocks <= 0) return KVC_ERR_INVALID_ARG;
  if ((int64_t)in.max_blocks * L.page_size < in.max_T) return KVC_ERR_INVALID_ARG;
  if (!in.block_table || !in.seq_len || !C.pool || !C.page_off || C.n_pages <= 0) return KVC_ERR_INVALID_ARG;
  if (L.variable_rank && (!in.ranks || !C.tok_rank || !C.tok_off)) return KVC_ERR_INVALID_ARG;
  if (!in.lat_k || (!L.shared && !in.lat_v)) return KVC_ERR_INVALID_ARG;
  if (L.residual_bits && (!in.res_k || !in.res_v)) return KVC_ERR_INVALID_ARG;
  if (in.mode == KVC_FROM_DENSE) {
    if (L.shared || lat_bits_k(L) == 32 || lat_bits_v(L) == 32 || !in.k || !in.v || !in.basis_k || !in.basis_v)
      return KVC_ERR_INVALID_ARG;
    if (L.r_k_cap > 64 || L.r_v_cap > 64 || L.head_dim > 128) return KVC_ERR_UNSUPPORTED;
  }
  const void* ptrs[] = {in.block_table, in.seq_len, in.ranks, in.lat_k, in.lat_v, in.res_k, in.res_v, in.k, in.v,
                        in.basis_k, in.basis_v, C.pool, C.page_off, C.tok_rank, C.tok_off, C.used_bytes};
  for (const void* p : ptrs)
    if (p && !al16(p)) return KVC_ERR_MISALIGNED;
  const int64_t need = uniform_page_bytes(L) * (int64_t)C.n_pages;
  if (C.pool_bytes < need) return KVC_ERR_WORKSPACE;
  const int P = L.page_size, Hkv = L.n_kv_heads, d = L.head_dim;
  hipError_t e;
#define KVC_CHECK()                          \
  do {                                       \
    e = hipGetLastError();                   \
    if (e != hipSuccess) return hip_fail(e); \
  } while (0)

  if (in.mode == KVC_FROM_DENSE) {
    const int64_t items = (int64_t)in.B * in.max_T * Hkv * 2;
    hipLaunchKernelGGL(project_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, in.k, in.v, in.basis_k,
                       in.basis_v, in.ranks, in.seq_len, in.lat_k, in.lat_v, in.res_k, in.res_v, in.B, in.max_T, Hkv,
                       d, L.r_k_cap, L.r_v_cap, L.variable_rank, L.residual_bits);
    KVC_CHECK();
  }
  hipLaunchKernelGGL(fill_u32_kernel, dim3(2048), dim3(256), 0, st, (uint32_t*)C.pool, C.pool_bytes / 4, 0u);
  KVC_CHECK();
  if (L.variable_rank) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(256), dim3(256), 0, st, (uint32_t*)C.tok_rank,
                       (int64_t)C.n_pages * P / 4, 0u);
    KVC_CHECK();
    hipLaunchKernelGGL(scatter_ranks_kernel, dim3((in.max_T + 255) / 256, in.B), dim3(256), 0, st, in.block_table,
                       in.seq_len, in.ranks, C.tok_rank, in.max_T, in.max_blocks, P, L.r_k_cap);
    KVC_CHECK();
    hipLaunchKernelGGL(page_prefix_kernel, dim3(C.n_pages), dim3(256), 0, st, C.tok_rank, C.tok_off, C.page_off, P,
                       L.group, Hkv, L.residual_bits, d, L.latent_bits);
    KVC_CHECK();
    hipLaunchKernelGGL(page_scan_kernel, dim3(1), dim3(1024), 0, st, C.page_off, C.n_pages, (int64_t)-1,
                       C.used_bytes);
  } else {
    hipLaunchKernelGGL(page_scan_kernel, dim3(1), dim3(1024), 0, st, C.page_off, C.n_pages, uniform_page_bytes(L),
                       C.used_bytes);
  }
  KVC_CHECK();
  PackArgs a;
  a.block_table = in.block_table; a.seq_len = in.seq_len; a.lat_k = in.lat_k; a.lat_v = in.lat_v;
  a.res_k = in.res_k; a.res_v = in.res_v; a.pool = C.pool; a.page_off = C.page_off; a.tok_rank = C.tok_rank;
  a.tok_off = C.tok_off; a.B = in.B; a.max_T = in.max_T; a.max_blocks = in.max_blocks; a.P = P; a.Hkv = Hkv;
  a.d = d; a.rk = L.r_k_cap; a.rv = L.r_v_cap; a.G = L.group; a.latent_bits = lat_bits_k(L);
  a.latent_bits_v = lat_bits_v(L);
  a.residual = L.residual_bits; a.variable_rank = L.variable_rank; a.shared = L.shared;
  a.n_layers = L.n_layers; a.lat_bytes = shared_latent_bytes(L);
  a.S_uniform = head_sections((int64_t)P * slot_code_bytes(lat_bits_k(L), L.r_k_cap),
                              (int64_t)P * slot_code_bytes(lat_bits_v(L), L.r_v_cap),
                              (int64_t)P * slot_meta_bytes(lat_bits_k(L), L.r_k_cap, L.group),
                              (int64_t)P * slot_meta_bytes(lat_bits_v(L), L.r_v_cap, L.group), P, d, L.residual_bits);
  const int gpi = L.latent_bits == 32 ? 1 : ceil_div(std::max(L.r_k_cap, L.r_v_cap), L.group);
  const int64_t threads = (int64_t)in.B * in.max_T * (L.shared ? 1 : 2 * Hkv) * gpi;
  hipLaunchKernelGGL(pack_latent_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a, gpi);
  KVC_CHECK();
  if (L.residual_bits) {
    const int64_t rt = (int64_t)in.B * in.max_T * 2 * Hkv * (L.shared ? L.n_layers : 1);
    hipLaunchKernelGGL(pack_residual_kernel, dim3((unsigned)((rt + 255) / 256)), dim3(256), 0, st, a);
    KVC_CHECK();
  }
#undef KVC_CHECK
  return KVC_OK;
}

}  // namespace kvc
