// kvc_common.hpp -- shared definitions of the gfx950 kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc.h"

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

#define KVC_WAVE 64

namespace kvc {

// Record the HIP error of this thread and map it to a status.
kvc_status hip_fail(hipError_t e);

// Optional pair of caller-owned HIP events that the launchers record on their stream right before and
// right after the measured kernel: the attention kernel of a decode (not the split merge), the Gram
// kernel of a basis fit.  Set only for the duration of one kvc_decode_attn_timed / kvc_fit_basis_timed
// call on the calling thread; null otherwise.
struct LaunchMarks {
  hipEvent_t begin = nullptr, end = nullptr;
};
extern thread_local LaunchMarks g_marks;
inline hipError_t mark(hipEvent_t e, hipStream_t st) { return e ? hipEventRecord(e, st) : hipSuccess; }

__host__ __device__ inline int64_t pad16(int64_t x) { return (x + 15) & ~int64_t(15); }
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Byte offsets of the sections of one head block (per-head mode) relative to the head block start,
// and the head block size.  ck/cv: code bytes of the page, mk/mv: pair bytes of the page.
struct HeadSections {
  int64_t kc, vc, km, vm, kr, vr, ks, vs, hb;
};

__host__ __device__ inline HeadSections head_sections(int64_t ck, int64_t cv, int64_t mk, int64_t mv, int P,
                                                      int d, int residual) {
  HeadSections S;
  int64_t off = 0;
  S.kc = off; off += pad16(ck);
  S.vc = off; off += pad16(cv);
  S.km = off; off += pad16(mk);
  S.vm = off; off += pad16(mv);
  S.kr = S.vr = S.ks = S.vs = off;
  if (residual) {
    S.kr = off; off += pad16((int64_t)P * d / 4);
    S.vr = off; off += pad16((int64_t)P * d / 4);
    S.ks = off; off += pad16((int64_t)P * 2);
    S.vs = off; off += pad16((int64_t)P * 2);
  }
  S.hb = off;
  return S;
}

// Latent bits of keys and values (latent_bits_v = 0: the same as the keys).
__host__ __device__ inline int lat_bits_k(const kvc_layout& L) { return L.latent_bits; }
__host__ __device__ inline int lat_bits_v(const kvc_layout& L) { return L.latent_bits_v ? L.latent_bits_v : L.latent_bits; }

// Code and pair bytes of a slot of rank r with b-bit codes (b = 32: fp32 latents, no pairs).
__host__ __device__ inline int slot_code_bytes(int latent_bits, int r) { return latent_bits == 32 ? 4 * r : r * latent_bits / 8; }
__host__ __device__ inline int slot_meta_bytes(int latent_bits, int r, int G) {
  return latent_bits == 32 ? 0 : 4 * ceil_div(r, G);
}

// Block-shared record: the latent's code and pair sections (each padded to 16), then with the rotated residual
// Kr, Vr (one part of P x d/4 code bytes per (layer, kv head), layer-major) and Ks, Vs (one part of P fp16 scales,
// padded to 16, per (layer, kv head)).  Bytes of the latent's part:
__host__ __device__ inline int64_t shared_latent_bytes(const kvc_layout& L) {
  const int P = L.page_size;
  return pad16((int64_t)P * L.r_k_cap * lat_bits_k(L) / 8) + pad16((int64_t)P * 4 * ceil_div(L.r_k_cap, L.group));
}
// Byte offset in a block-shared record of residual part `part` (0 Kr, 1 Vr, 2 Ks, 3 Vs) of (layer, kv head) idx.
__host__ __device__ inline int64_t shared_res_part(int64_t lat_bytes, int P, int d, int n_parts, int part, int idx) {
  const int64_t cb = (int64_t)P * (d / 4), sb = pad16((int64_t)P * 2);
  if (part < 2) return lat_bytes + ((int64_t)part * n_parts + idx) * cb;
  return lat_bytes + 2 * n_parts * cb + ((int64_t)(part - 2) * n_parts + idx) * sb;
}

// Uniform-rank page record size (per-head or shared mode).
__host__ __device__ inline int64_t uniform_page_bytes(const kvc_layout& L) {
  const int P = L.page_size;
  if (L.shared)
    return shared_latent_bytes(L) + (L.residual_bits ? 2 * (int64_t)L.n_layers * L.n_kv_heads *
                                                           ((int64_t)P * (L.head_dim / 4) + pad16((int64_t)P * 2))
                                                     : 0);
  HeadSections S = head_sections((int64_t)P * slot_code_bytes(lat_bits_k(L), L.r_k_cap),
                                 (int64_t)P * slot_code_bytes(lat_bits_v(L), L.r_v_cap),
                                 (int64_t)P * slot_meta_bytes(lat_bits_k(L), L.r_k_cap, L.group),
                                 (int64_t)P * slot_meta_bytes(lat_bits_v(L), L.r_v_cap, L.group), P, L.head_dim,
                                 L.residual_bits);
  return S.hb * L.n_kv_heads;
}

// Eight b-bit codes (b = 2, 3, 4) starting at byte off of a 4-byte-aligned buffer in LDS or global memory, as the
// INT4 dword layout (code k in the low b bits of nibble k) that dequant_int4x8 takes.  The codes of a slot form a
// little-endian bit string, code i at bits b*i.., so the 8 codes of group w start at byte b*w.  Reads up to 7
// bytes past the group, which the 16-byte padding of every section keeps inside the block.  The address is kept
// as base + offset (never rebuilt from an integer): that keeps the read an LDS read the compiler can tell apart
// from the copies in flight into other LDS buffers.
template <int B>
__device__ inline uint32_t codes8_as_nibbles(const uint8_t* base, int off) {
  if constexpr (B == 4) {
    return *(const uint32_t*)(base + off);
  } else if constexpr (B == 2) {
    uint32_t y = *(const uint16_t*)(base + off);  // 2-byte aligned: slot offsets are multiples of r / 4 bytes, r % 8 == 0
    y = (y | (y << 8)) & 0x00FF00FFu;
    y = (y | (y << 4)) & 0x0F0F0F0Fu;
    y = (y | (y << 2)) & 0x33333333u;
    return y;
  } else {
    // the two aligned words around the group, and v_alignbyte for the 3 bytes from byte off (a 64-bit shift
    // costs more instructions; and as read here, the compiler does not make the reads wait for copies in flight)
    const uint32_t* w = (const uint32_t*)(base + (off & ~3));
    const uint32_t x = __builtin_amdgcn_alignbyte(w[1], w[0], (uint32_t)(off & 3)) & 0xFFFFFFu;  // codes 0..7 at bits 3k
    uint32_t y = (x & 0xFFFu) | ((x & 0xFFF000u) << 4);      // codes 0-3 at bits 0.., codes 4-7 at bits 16..
    y = (y & 0x003F003Fu) | ((y & 0x0FC00FC0u) << 2);        // code pairs at bytes 0..3
    y = (y & 0x07070707u) | ((y & 0x38383838u) << 1);        // code k at bits 4k
    return y;
  }
}

// ---- device helpers ----

__device__ inline h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ inline uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// fp32 pair -> packed fp16 pair, round to nearest even.
__device__ inline uint32_t pack_h2(float a, float b) {
  h2 v = {(_Float16)a, (_Float16)b};
  return as_u32(v);
}

// fp32 -> bf16 bits, rounded to nearest even.
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// bf16 bits -> fp16 (exact for the normal range of fp16).
__device__ inline _Float16 bf16_to_h(uint16_t b) {
  return (_Float16)__builtin_bit_cast(float, (uint32_t)b << 16);
}

// Eight INT4 codes (one dword, coordinate 2j in the low nibble of byte j) dequantized as
// code * scale + zero in fp16; sz holds (scale, zero) as two fp16.  A code q placed in a byte is the
// fp8 e4m3 bit pattern of q * 2^-9 (0x00-0x07 subnormal, 0x08-0x0F the first binade), so the gfx950
// fp8 -> fp16 conversion with the power-of-two scale 2^9 yields q exactly; one fused multiply-add in
// fp16 then applies scale and zero (a single rounding).  Result order: element j is coordinate
// perm8(j) = 2j for j < 4 and 2(j - 4) + 1 otherwise.
__device__ inline h8 dequant_int4x8(uint32_t x, uint32_t sz) {
  const uint32_t lo = x & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
  const h2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
  const h2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
  const h2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
  const h2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
  const h2 s = as_h2(sz);
  const h2 ss = s.xx, zz = s.yy;
  const h2 a0 = c0 * ss + zz, a1 = c1 * ss + zz, a2 = c2 * ss + zz, a3 = c3 * ss + zz;
  h8 r = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
  return r;
}

// RoPE on one fp16 pair v = (x, y) with f = (cos, sin): (x cos - y sin, y cos + x sin).  Written so
// that it compiles to two packed instructions (the swap and the sign become operand selects).
__device__ inline uint32_t rope_pair(uint32_t v, uint32_t f) {
  const h2 x = as_h2(v), c = as_h2(f);
  const h2 t = x * c.yy;  // (x sin, y sin)
  const h2 m = {-t.y, t.x};
  return as_u32(x * c.xx + m);
}

__host__ __device__ inline int perm8(int j) { return j < 4 ? 2 * j : 2 * (j - 4) + 1; }

// Eight 2-bit residual codes (16 bits, code j at bits 2j) as (2 code - 3) * s2 in fp16, order
// permr(j) = j/2 + 4 (j%2).
// Each code is placed doubled in the low mantissa bits of fp16 1024, so (1024 + 2c) - 1027 = 2c - 3 is
// exact (1027 is an fp16 integer; 1025.5 would not be); with s2 = scale / 2 this is (c - 1.5) * scale.
__device__ inline h8 dequant_res2x8(uint32_t u16, h2 s2) {
  const uint32_t magic = 0x64006400u;
  const uint32_t w = ((u16 & 0xFFu) | ((u16 & 0xFF00u) << 8)) << 1;  // codes 0-3 at bits 1-8, 4-7 at 17-24
  const uint32_t y0 = (w & 0x00060006u) | magic;
  const uint32_t y1 = ((w >> 2) & 0x00060006u) | magic;
  const uint32_t y2 = ((w >> 4) & 0x00060006u) | magic;
  const uint32_t y3 = ((w >> 6) & 0x00060006u) | magic;
  const h2 off = {(_Float16)1027.0f, (_Float16)1027.0f};
  const h2 a0 = (as_h2(y0) - off) * s2;
  const h2 a1 = (as_h2(y1) - off) * s2;
  const h2 a2 = (as_h2(y2) - off) * s2;
  const h2 a3 = (as_h2(y3) - off) * s2;
  h8 r = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
  return r;
}

__host__ __device__ inline int permr(int j) { return (j >> 1) + 4 * (j & 1); }

__device__ inline f4 mfma16x16x32(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

template <typename T>
__device__ inline T uniform(T v) {
  return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ inline int64_t uniform64(int64_t v) {
  int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uint64_t)v);
  int hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

}  // namespace kvc
