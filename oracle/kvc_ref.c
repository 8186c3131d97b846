/*
 * kvc_ref.c -- plain, slow CPU reference for compressed-KV decode attention.
 * TEST INFRASTRUCTURE ONLY (see kvc_ref.h).  Shares no code, header, table or
 * constant generator with the GPU library.
 *
 * Byte layout of the compressed cache (this project's format; the pages fix
 * no layout).  All multi-byte fields are little-endian.
 *
 *   The pool is a sequence of page records, one per physical page id p, at
 *   byte offset page_off[p]; page_off is the exclusive prefix sum of record
 *   sizes in increasing p.  Token (b, t) lives in physical page
 *   block_table[b][t / P] at slot t % P.
 *
 *   Per-head mode: a record is Hkv head blocks, head h first-to-last, all of
 *   equal size (ranks are per token, shared by every head).  A head block is
 *     Kc  key codes, slot order, slot s taking code_bytes(r_k(s))
 *     Vc  value codes, same for r_v(s)
 *     Km  key (scale, zero) pairs, slot order, ceil(r_k(s)/G) pairs per slot
 *     Vm  value pairs
 *     Kr  key residual codes, P x 32 bytes           (residual_bits = 2)
 *     Vr  value residual codes, P x 32 bytes         (residual_bits = 2)
 *     Ks  key residual scale, P x fp16               (residual_bits = 2)
 *     Vs  value residual scale, P x fp16             (residual_bits = 2)
 *   each section padded to a multiple of 16 bytes.  code_bytes(r) = r*b/8 for
 *   b-bit codes (b = 2, 3, 4; code i at bits b*i .. b*i + b - 1 of the slot's
 *   little-endian bit string, so for INT4 coordinate 2j is the low nibble of
 *   byte j) and 4r for fp32 latents (no Km/Vm then).  Keys use latent_bits,
 *   values latent_bits_v (0 = the same).  A (scale, zero) pair
 *   is two fp16 values, scale first.  Residual element i of a slot is bits
 *   2(i%4)..2(i%4)+1 of byte i/4.
 *
 *   Shared mode: a record is Lc (P x latent*latent_bits/8 code bytes) then Lm
 *   (P x latent/G pairs), each padded to 16 bytes.  With the rotated residual
 *   (JoLT: a Tucker form plus a rotated low-bit residual; each layer and head
 *   has its own) then Kr, Vr (one part per (layer, kv head), layer-major, of
 *   P x 32 code bytes) and Ks, Vs (one part per (layer, kv head) of P x fp16,
 *   each part padded to 16 bytes).
 *
 *   Uniform rank: every slot of every page holds r_k_cap / r_v_cap, so all
 *   records have the same size.  Variable rank: slot s of page p holds rank
 *   tok_rank[p][s] (0 for a slot no sequence uses) for K and V alike, and
 *   tok_off[p][s] packs the exclusive prefix over slots < s of the ranks
 *   (low 16 bits) and of ceil(rank/G) (high 16 bits); tok_off[p][P] holds
 *   the page totals.
 */
#include "kvc_ref.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#define KVC_REF_EINVAL (-1)

/* ------------------------------------------------------------------------ */
/* number formats                                                           */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* IEEE binary32 -> binary16, round to nearest, ties to even. */
uint16_t kvc_ref_f32_to_f16(float x) {
  uint32_t u = f32_bits(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t absu = u & 0x7fffffffu;
  if (absu >= 0x7f800000u) {                       /* inf or nan */
    if (absu > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);
    return (uint16_t)(sign | 0x7c00u);
  }
  int e = (int)(absu >> 23) - 127;                 /* unbiased exponent */
  uint32_t mant = absu & 0x7fffffu;
  if (e > 15) return (uint16_t)(sign | 0x7c00u);  /* overflow -> inf */
  if (e >= -14) {                                  /* normal half */
    uint32_t m = mant >> 13, rest = mant & 0x1fffu;
    uint32_t h = ((uint32_t)(e + 15) << 10) | m;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1;  /* may carry into exponent: still right */
    return (uint16_t)(sign | h);
  }
  if (e < -25) return sign;                        /* below half of the smallest subnormal */
  /* subnormal half: value = m * 2^-24.  With the 24-bit significand
   * full = 1.mant * 2^23 the value is full * 2^(e-23), so m = full * 2^(e+1),
   * a right shift by -(e+1) >= 14 whose dropped bits decide the rounding. */
  uint32_t full = mant | 0x800000u;
  int shift = -e - 1;
  uint32_t m = full >> shift;
  uint32_t rest = full & ((1u << shift) - 1u), half = 1u << (shift - 1);
  if (rest > half || (rest == half && (m & 1u))) m += 1;
  return (uint16_t)(sign | m);
}

double kvc_ref_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x400), e - 25);
  return sign ? -v : v;
}

double kvc_ref_bf16_to_f64(uint16_t b) { return (double)bits_f32((uint32_t)b << 16); }

/* ------------------------------------------------------------------------ */
/* quantizers (fp32, every operation rounded to nearest even, no FMA)       */
/* ------------------------------------------------------------------------ */

/* b-bit asymmetric min/max quantizer of one group, the form of the BellowsKV
 * page's "Worked Example" (scale = (max - min) / (2^bits - 1), offset = min,
 * Python's round = half to even), with the scale and offset stored as fp16
 * and the codes taken against the stored fp16 values.  INT4 is the main
 * form; the same page's INT3 and 2-bit variants ("Reading the Retention
 * Table") use bits 3 and 2. */
void kvc_ref_quant_intb(const float* x, int n, int bits, uint16_t* s16, uint16_t* z16, uint8_t* codes) {
  float lo = x[0], hi = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  float levels = (float)((1 << bits) - 1);
  float range = hi - lo;
  float s32 = range / levels;
  *s16 = kvc_ref_f32_to_f16(s32);
  *z16 = kvc_ref_f32_to_f16(lo);
  float s = (float)kvc_ref_f16_to_f64(*s16);
  float z = (float)kvc_ref_f16_to_f64(*z16);
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) { codes[i] = 0; continue; }
    float diff = x[i] - z;
    float ratio = diff / s;
    float r = rintf(ratio);
    if (r < 0.0f) r = 0.0f;
    if (r > levels) r = levels;
    codes[i] = (uint8_t)r;
  }
}

void kvc_ref_quant_int4(const float* x, int n, uint16_t* s16, uint16_t* z16, uint8_t* codes) {
  kvc_ref_quant_intb(x, n, 4, s16, z16, codes);
}

/* 2-bit symmetric quantizer of a rotated residual vector (JoLT's rotated
 * low-bit residual; the pages fix only "2 bits, one fp16 scale per token"):
 * levels (c - 1.5) * s for c in 0..3, s = max|y| / 1.5. */
void kvc_ref_quant_res2(const float* y, int n, uint16_t* s16, uint8_t* codes) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i) {
    float m = fabsf(y[i]);
    if (m > a) a = m;
  }
  float s32 = a / 1.5f;
  *s16 = kvc_ref_f32_to_f16(s32);
  float s = (float)kvc_ref_f16_to_f64(*s16);
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) { codes[i] = 2; continue; }
    float ratio = y[i] / s;
    float shifted = ratio + 1.5f;
    float r = rintf(shifted);
    if (r < 0.0f) r = 0.0f;
    if (r > 3.0f) r = 3.0f;
    codes[i] = (uint8_t)r;
  }
}

/* Sylvester construction (as in the BellowsKV "Worked Example": start from
 * [[1]], each step stacks [[H, H], [H, -H]]), scaled by 1/sqrt(n) so that
 * H is orthonormal and its own inverse. */
void kvc_ref_hadamard(int n, double* H) {
  H[0] = 1.0;
  for (int m = 1; m < n; m *= 2)
    for (int i = 0; i < m; ++i)
      for (int j = 0; j < m; ++j) {
        double h = H[i * n + j];
        H[i * n + (j + m)] = h;
        H[(i + m) * n + j] = h;
        H[(i + m) * n + (j + m)] = -h;
      }
  double sc = 1.0 / sqrt((double)n);
  for (int i = 0; i < n * n; ++i) H[i] *= sc;
}

/* Rotary position embedding, rotate-half pairing (x_j, x_{j+d/2}) with
 * frequency theta^(-2j/d), applied to keys after reconstruction because the
 * cache stores them before RoPE (JoLT thesis page, "Key findings"). */
void kvc_ref_rope(double* x, int d, double pos, double theta) {
  if (theta == 0.0) return;
  int h = d / 2;
  for (int j = 0; j < h; ++j) {
    double freq = pow(theta, -2.0 * j / d);
    double ang = pos * freq, c = cos(ang), s = sin(ang);
    double a = x[j], b = x[j + h];
    x[j] = a * c - b * s;
    x[j + h] = b * c + a * s;
  }
}

void kvc_ref_f32_to_f16_n(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvc_ref_f32_to_f16(x[i]);
}

void kvc_ref_quant_int4_n(const float* x, int64_t n_groups, int n, uint16_t* s16, uint16_t* z16, uint8_t* codes) {
  for (int64_t g = 0; g < n_groups; ++g) kvc_ref_quant_int4(x + g * n, n, s16 + g, z16 + g, codes + g * n);
}

void kvc_ref_quant_intb_n(const float* x, int64_t n_groups, int n, int bits, uint16_t* s16, uint16_t* z16,
                          uint8_t* codes) {
  for (int64_t g = 0; g < n_groups; ++g) kvc_ref_quant_intb(x + g * n, n, bits, s16 + g, z16 + g, codes + g * n);
}

void kvc_ref_quant_res2_n(const float* y, int64_t n_rows, int n, uint16_t* s16, uint8_t* codes) {
  for (int64_t r = 0; r < n_rows; ++r) kvc_ref_quant_res2(y + r * n, n, s16 + r, codes + r * n);
}

/* ------------------------------------------------------------------------ */
/* layout                                                                   */
/* ------------------------------------------------------------------------ */

static int64_t pad16(int64_t x) { return (x + 15) & ~(int64_t)15; }
static int ceil_div(int a, int b) { return (a + b - 1) / b; }
/* bits of the key (which = 0) or value (which = 1) latent */
static int lat_bits(const kvc_ref_layout* L, int which) {
  return which && L->latent_bits_v ? L->latent_bits_v : L->latent_bits;
}
static int code_bytes(const kvc_ref_layout* L, int which, int r) {
  int b = lat_bits(L, which);
  return b == 32 ? 4 * r : r * b / 8;
}
static int meta_bytes(const kvc_ref_layout* L, int which, int r) {
  return lat_bits(L, which) == 32 ? 0 : 4 * ceil_div(r, L->group);
}
static int quant_bits_ok(int b) { return b == 2 || b == 3 || b == 4; }

int kvc_ref_layout_check(const kvc_ref_layout* L) {
  if (!L) return KVC_REF_EINVAL;
  if (L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->n_q_heads % L->n_kv_heads) return KVC_REF_EINVAL;
  if (L->head_dim <= 0 || L->head_dim % 2) return KVC_REF_EINVAL;
  if (L->page_size <= 0 || L->page_size > 256) return KVC_REF_EINVAL;
  {
    int bk = L->latent_bits, bv = lat_bits(L, 1);
    if (L->latent_bits_v != 0 && !quant_bits_ok(L->latent_bits_v) && L->latent_bits_v != 32) return KVC_REF_EINVAL;
    if (!(quant_bits_ok(bk) && quant_bits_ok(bv)) && !(bk == 32 && bv == 32)) return KVC_REF_EINVAL;
  }
  if (L->r_k_cap <= 0 || L->r_v_cap <= 0 || L->r_k_cap % 8 || L->r_v_cap % 8) return KVC_REF_EINVAL;
  if (L->latent_bits != 32 && (L->group <= 0 || L->group % 8)) return KVC_REF_EINVAL;
  if (L->residual_bits != 0 && L->residual_bits != 2) return KVC_REF_EINVAL;
  if (L->residual_bits && L->head_dim != 128) return KVC_REF_EINVAL;
  if (L->shared) {
    /* one latent for keys and values: one width (BellowsKV's retention table lists INT4 and INT3 for it) */
    if (L->n_layers <= 0 || !quant_bits_ok(L->latent_bits) || lat_bits(L, 1) != L->latent_bits || L->variable_rank ||
        L->r_k_cap != L->r_v_cap)
      return KVC_REF_EINVAL;
  } else if (L->n_layers != 1) {
    return KVC_REF_EINVAL;
  }
  if (L->variable_rank && (L->latent_bits == 32 || lat_bits(L, 1) != L->latent_bits || L->r_k_cap != L->r_v_cap))
    return KVC_REF_EINVAL;
  if (L->r_k_cap > 1024 || L->r_v_cap > 1024) return KVC_REF_EINVAL;
  if (L->variable_rank && L->page_size * L->r_k_cap > 65535) return KVC_REF_EINVAL;
  if (L->rope_theta < 0.0) return KVC_REF_EINVAL;
  return 0;
}

/* sizes of the sections of one head block, from the page's rank totals */
typedef struct {
  int64_t kc, vc, km, vm, kr, vr, ks, vs, total;
} sections;

static sections head_sections(const kvc_ref_layout* L, int sum_code_k, int sum_code_v, int sum_meta_k, int sum_meta_v) {
  sections S;
  int64_t off = 0, P = L->page_size;
  S.kc = off; off += pad16(sum_code_k);
  S.vc = off; off += pad16(sum_code_v);
  S.km = off; off += pad16(sum_meta_k);
  S.vm = off; off += pad16(sum_meta_v);
  S.kr = S.vr = S.ks = S.vs = off;
  if (L->residual_bits) {
    S.kr = off; off += pad16(P * L->head_dim / 4);
    S.vr = off; off += pad16(P * L->head_dim / 4);
    S.ks = off; off += pad16(P * 2);
    S.vs = off; off += pad16(P * 2);
  }
  S.total = off;
  return S;
}

/* Block-shared record: [Lc codes][Lm pairs], each padded to 16 bytes; with the residual (residual_bits = 2) then
 * [Kr][Vr][Ks][Vs], each holding one part per (layer, kv head) in layer-major order: P x d/4 code bytes per part,
 * P x fp16 scales per part padded to 16 bytes.  Returns the latent part's bytes. */
static int64_t shared_latent_bytes(const kvc_ref_layout* L) {
  int64_t P = L->page_size;
  return pad16(P * L->r_k_cap * L->latent_bits / 8) + pad16(P * 4 * ceil_div(L->r_k_cap, L->group));
}

/* the residual codes and scales of slot s for (layer, head) in a block-shared record */
static void shared_residual_at(const kvc_ref_layout* L, const uint8_t* rec, int layer, int head, int s,
                               const uint8_t** kr, const uint8_t** vr, const uint8_t** ks, const uint8_t** vs) {
  int64_t P = L->page_size, n = (int64_t)L->n_layers * L->n_kv_heads, idx = (int64_t)layer * L->n_kv_heads + head;
  int64_t cb = L->head_dim / 4, sb = pad16(P * 2);
  const uint8_t* base = rec + shared_latent_bytes(L);
  *kr = base + (idx * P + s) * cb;
  *vr = base + (n + idx) * P * cb + s * cb;
  *ks = base + 2 * n * P * cb + idx * sb + 2 * s;
  *vs = base + 2 * n * P * cb + (n + idx) * sb + 2 * s;
}

int64_t kvc_ref_page_bytes_uniform(const kvc_ref_layout* L) {
  if (kvc_ref_layout_check(L)) return KVC_REF_EINVAL;
  int64_t P = L->page_size;
  if (L->shared)
    return shared_latent_bytes(L) +
           (L->residual_bits ? 2 * (int64_t)L->n_layers * L->n_kv_heads * (P * L->head_dim / 4 + pad16(P * 2)) : 0);
  sections S = head_sections(L, (int)(P * code_bytes(L, 0, L->r_k_cap)), (int)(P * code_bytes(L, 1, L->r_v_cap)),
                             (int)(P * meta_bytes(L, 0, L->r_k_cap)), (int)(P * meta_bytes(L, 1, L->r_v_cap)));
  return S.total * L->n_kv_heads;
}

/* Everything needed to find one slot's bytes: filled by locate(). */
typedef struct {
  const uint8_t* kc; const uint8_t* vc;  /* start of the slot's codes           */
  const uint8_t* km; const uint8_t* vm;  /* start of the slot's (scale, zero)s  */
  const uint8_t* kr; const uint8_t* vr;  /* slot's residual codes               */
  const uint8_t* ks; const uint8_t* vs;  /* slot's residual scales              */
  int rk, rv;                            /* the slot's ranks                    */
} slot_view;

/* Page sums of code/meta bytes (same for every head of the page). */
static void page_sums(const kvc_ref_layout* L, const uint8_t* ranks_of_page, int* ck, int* cv, int* mk, int* mv) {
  *ck = *cv = *mk = *mv = 0;
  for (int s = 0; s < L->page_size; ++s) {
    int rk = L->variable_rank ? ranks_of_page[s] : L->r_k_cap;
    int rv = L->variable_rank ? ranks_of_page[s] : L->r_v_cap;
    *ck += code_bytes(L, 0, rk); *cv += code_bytes(L, 1, rv);
    *mk += meta_bytes(L, 0, rk); *mv += meta_bytes(L, 1, rv);
  }
}

static slot_view locate(const kvc_ref_layout* L, const uint8_t* pool, const int64_t* page_off,
                        const uint8_t* tok_rank, const uint32_t* tok_off, int page, int slot, int head) {
  slot_view v;
  int P = L->page_size;
  const uint8_t* rec = pool + page_off[page];
  int ck, cv, mk, mv, pre_code_k, pre_code_v, pre_meta_k, pre_meta_v;
  if (L->variable_rank) {
    const uint32_t* off = tok_off + (size_t)page * (P + 1);
    int tot_r = (int)(off[P] & 0xffffu), tot_g = (int)(off[P] >> 16);
    int pre_r = (int)(off[slot] & 0xffffu), pre_g = (int)(off[slot] >> 16);
    v.rk = v.rv = tok_rank[(size_t)page * P + slot];
    ck = cv = tot_r * L->latent_bits / 8; mk = mv = 4 * tot_g;  /* K and V share the bits (variable rank) */
    pre_code_k = pre_code_v = pre_r * L->latent_bits / 8;
    pre_meta_k = pre_meta_v = 4 * pre_g;
  } else {
    v.rk = L->r_k_cap; v.rv = L->r_v_cap;
    ck = P * code_bytes(L, 0, v.rk); cv = P * code_bytes(L, 1, v.rv);
    mk = P * meta_bytes(L, 0, v.rk); mv = P * meta_bytes(L, 1, v.rv);
    pre_code_k = slot * code_bytes(L, 0, v.rk); pre_code_v = slot * code_bytes(L, 1, v.rv);
    pre_meta_k = slot * meta_bytes(L, 0, v.rk); pre_meta_v = slot * meta_bytes(L, 1, v.rv);
  }
  sections S = head_sections(L, ck, cv, mk, mv);
  const uint8_t* hb = rec + (int64_t)head * S.total;
  v.kc = hb + S.kc + pre_code_k; v.vc = hb + S.vc + pre_code_v;
  v.km = hb + S.km + pre_meta_k; v.vm = hb + S.vm + pre_meta_v;
  v.kr = hb + S.kr + (int64_t)slot * (L->head_dim / 4);
  v.vr = hb + S.vr + (int64_t)slot * (L->head_dim / 4);
  v.ks = hb + S.ks + 2 * slot; v.vs = hb + S.vs + 2 * slot;
  return v;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }

/* ------------------------------------------------------------------------ */
/* compression                                                              */
/* ------------------------------------------------------------------------ */

/* quantize the first r coordinates of x in groups of G with `bits`-bit codes, write codes + pairs; code i
 * occupies bits bits*i .. bits*i + bits - 1 of the slot's little-endian bit string (for INT4: coordinate 2j
 * in the low nibble of byte j) */
static void pack_latent(const kvc_ref_layout* L, int bits, const float* x, int r, uint8_t* codes, uint8_t* meta) {
  if (bits == 32) {
    memcpy(codes, x, (size_t)4 * r);
    return;
  }
  int G = L->group;
  uint8_t q[4096];
  for (int g0 = 0, gi = 0; g0 < r; g0 += G, ++gi) {
    int n = r - g0 < G ? r - g0 : G;
    uint16_t s16, z16;
    kvc_ref_quant_intb(x + g0, n, bits, &s16, &z16, q + g0);
    wr16(meta + 4 * gi, s16);
    wr16(meta + 4 * gi + 2, z16);
  }
  memset(codes, 0, (size_t)r * bits / 8);
  for (int i = 0; i < r; ++i)
    for (int k = 0; k < bits; ++k)
      if ((q[i] >> k) & 1) codes[(bits * i + k) / 8] |= (uint8_t)(1u << ((bits * i + k) % 8));
}

static void pack_residual(const float* y, int n, uint8_t* codes, uint8_t* scale) {
  uint16_t s16;
  uint8_t c[256];
  kvc_ref_quant_res2(y, n, &s16, c);
  for (int i = 0; i < n / 4; ++i) codes[i] = (uint8_t)(c[4 * i] | (c[4 * i + 1] << 2) | (c[4 * i + 2] << 4) | (c[4 * i + 3] << 6));
  wr16(scale, s16);
}

int64_t kvc_ref_compress(const kvc_ref_layout* L, int B, int max_T, int max_blocks,
                         const int32_t* block_table, const int32_t* seq_len, const uint8_t* ranks,
                         const float* lat_k, const float* lat_v, const float* res_k, const float* res_v,
                         int n_pages, uint8_t* pool, int64_t pool_bytes, int64_t* page_off,
                         uint8_t* tok_rank, uint32_t* tok_off) {
  if (kvc_ref_layout_check(L)) return KVC_REF_EINVAL;
  int P = L->page_size, Hkv = L->n_kv_heads, rk = L->r_k_cap, rv = L->r_v_cap;
  /* every (b, logical block) in use must name a distinct page */
  int* owner = (int*)malloc(sizeof(int) * (size_t)n_pages);
  for (int p = 0; p < n_pages; ++p) owner[p] = -1;
  for (int b = 0; b < B; ++b) {
    if (seq_len[b] < 0 || seq_len[b] > max_T || seq_len[b] > max_blocks * P) { free(owner); return KVC_REF_EINVAL; }
    for (int lb = 0; lb * P < seq_len[b]; ++lb) {
      int p = block_table[(size_t)b * max_blocks + lb];
      if (p < 0 || p >= n_pages || owner[p] >= 0) { free(owner); return KVC_REF_EINVAL; }
      owner[p] = b * max_blocks + lb;
    }
  }
  /* per-slot ranks of every page (0 for slots no sequence uses) */
  uint8_t* pr = (uint8_t*)calloc((size_t)n_pages * P, 1);
  if (L->variable_rank) {
    for (int p = 0; p < n_pages; ++p) {
      if (owner[p] < 0) continue;
      int b = owner[p] / max_blocks, lb = owner[p] % max_blocks;
      for (int s = 0; s < P && lb * P + s < seq_len[b]; ++s) {
        int r = ranks[(size_t)b * max_T + lb * P + s];
        if (r < 8 || r > rk || r % 8) { free(owner); free(pr); return KVC_REF_EINVAL; }
        pr[(size_t)p * P + s] = (uint8_t)r;
      }
    }
    for (int p = 0; p < n_pages; ++p) {
      uint32_t er = 0, eg = 0;
      for (int s = 0; s <= P; ++s) {
        tok_off[(size_t)p * (P + 1) + s] = er | (eg << 16);
        if (s < P) {
          int r = pr[(size_t)p * P + s];
          tok_rank[(size_t)p * P + s] = (uint8_t)r;
          er += (uint32_t)r;
          eg += (uint32_t)ceil_div(r, L->group);
        }
      }
    }
  }
  /* record sizes and their exclusive prefix */
  int64_t total = 0;
  for (int p = 0; p < n_pages; ++p) {
    int64_t size;
    if (L->shared) {
      size = kvc_ref_page_bytes_uniform(L);
    } else if (L->variable_rank) {
      int ck, cv, mk, mv;
      page_sums(L, pr + (size_t)p * P, &ck, &cv, &mk, &mv);
      size = head_sections(L, ck, cv, mk, mv).total * Hkv;
    } else {
      size = kvc_ref_page_bytes_uniform(L);
    }
    page_off[p] = total;
    total += size;
  }
  if (total > pool_bytes) { free(owner); free(pr); return KVC_REF_EINVAL; }
  memset(pool, 0, (size_t)total);
  /* quantize and place every valid token */
  for (int b = 0; b < B; ++b) {
    for (int t = 0; t < seq_len[b]; ++t) {
      int p = block_table[(size_t)b * max_blocks + t / P], s = t % P;
      if (L->shared) {
        int lat = L->r_k_cap, G = L->group;
        uint8_t* rec = pool + page_off[p];
        const int lb = L->latent_bits;
        uint8_t* codes = rec + (int64_t)s * (lat * lb / 8);
        uint8_t* meta = rec + pad16((int64_t)P * lat * lb / 8) + (int64_t)s * 4 * ceil_div(lat, G);
        pack_latent(L, lb, lat_k + ((size_t)b * max_T + t) * lat, lat, codes, meta);
        if (L->residual_bits) {  /* res_k, res_v [B][max_T][n_layers][Hkv][d] */
          int d = L->head_dim;
          for (int l = 0; l < L->n_layers; ++l)
            for (int h = 0; h < Hkv; ++h) {
              const uint8_t *kr, *vr, *ks, *vs;
              shared_residual_at(L, rec, l, h, s, &kr, &vr, &ks, &vs);
              size_t tk = (((size_t)b * max_T + t) * L->n_layers + l) * Hkv + h;
              pack_residual(res_k + tk * d, d, (uint8_t*)kr, (uint8_t*)ks);
              pack_residual(res_v + tk * d, d, (uint8_t*)vr, (uint8_t*)vs);
            }
        }
        continue;
      }
      for (int h = 0; h < Hkv; ++h) {
        slot_view v = locate(L, pool, page_off, tok_rank, tok_off, p, s, h);
        size_t tk = (((size_t)b * max_T + t) * Hkv + h);
        pack_latent(L, lat_bits(L, 0), lat_k + tk * rk, v.rk, (uint8_t*)v.kc, (uint8_t*)v.km);
        pack_latent(L, lat_bits(L, 1), lat_v + tk * rv, v.rv, (uint8_t*)v.vc, (uint8_t*)v.vm);
        if (L->residual_bits) {
          int d = L->head_dim;
          pack_residual(res_k + tk * d, d, (uint8_t*)v.kr, (uint8_t*)v.ks);
          pack_residual(res_v + tk * d, d, (uint8_t*)v.vr, (uint8_t*)v.vs);
        }
      }
    }
  }
  free(owner);
  free(pr);
  return total;
}

int kvc_ref_project(const kvc_ref_layout* L, int B, int max_T, const int32_t* seq_len, const uint8_t* ranks,
                    const float* k, const float* v, const uint16_t* basis_k, const uint16_t* basis_v,
                    float* lat_k, float* lat_v, float* res_k, float* res_v) {
  if (kvc_ref_layout_check(L) || L->shared) return KVC_REF_EINVAL;
  int Hkv = L->n_kv_heads, d = L->head_dim, rk = L->r_k_cap, rv = L->r_v_cap;
  double* H = NULL;
  if (L->residual_bits) { H = (double*)malloc(sizeof(double) * d * d); kvc_ref_hadamard(d, H); }
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < seq_len[b]; ++t)
      for (int h = 0; h < Hkv; ++h)
        for (int which = 0; which < 2; ++which) {
          int rcap = which ? rv : rk;
          int r = L->variable_rank ? ranks[(size_t)b * max_T + t] : rcap;
          const uint16_t* Bm = (which ? basis_v : basis_k) + (size_t)h * d * rcap;
          size_t tk = ((size_t)b * max_T + t) * Hkv + h;
          const float* x = (which ? v : k) + tk * d;
          float* c_out = (which ? lat_v : lat_k) + tk * rcap;
          double c[1024], e[1024];
          for (int i = 0; i < rcap; ++i) {        /* c = B_r^T x (truncated to the token's rank) */
            double acc = 0.0;
            if (i < r) for (int j = 0; j < d; ++j) acc += kvc_ref_bf16_to_f64(Bm[(size_t)j * rcap + i]) * (double)x[j];
            c[i] = acc;
            c_out[i] = (float)acc;
          }
          if (!L->residual_bits) continue;
          for (int j = 0; j < d; ++j) {           /* truncation residual e = x - B_r c */
            double acc = (double)x[j];
            for (int i = 0; i < r; ++i) acc -= kvc_ref_bf16_to_f64(Bm[(size_t)j * rcap + i]) * c[i];
            e[j] = acc;
          }
          float* y_out = (which ? res_v : res_k) + tk * d;
          for (int i = 0; i < d; ++i) {           /* rotate: y = H e */
            double acc = 0.0;
            for (int j = 0; j < d; ++j) acc += H[i * d + j] * e[j];
            y_out[i] = (float)acc;
          }
        }
  free(H);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* decode attention                                                         */
/* ------------------------------------------------------------------------ */

/* dequantized latent of one slot: c_i = q_i * scale_g + zero_g, g = i / G;
 * coordinates at or beyond the slot's rank are zero */
static void unpack_latent(const kvc_ref_layout* L, int bits, const uint8_t* codes, const uint8_t* meta, int r, int rcap,
                          double* c) {
  for (int i = 0; i < rcap; ++i) c[i] = 0.0;
  if (bits == 32) {
    for (int i = 0; i < r; ++i) { float f; memcpy(&f, codes + 4 * i, 4); c[i] = f; }
    return;
  }
  for (int i = 0; i < r; ++i) {
    int q = 0;
    for (int k = 0; k < bits; ++k) q |= ((codes[(bits * i + k) / 8] >> ((bits * i + k) % 8)) & 1) << k;
    int g = i / L->group;
    double s = kvc_ref_f16_to_f64(rd16(meta + 4 * g)), z = kvc_ref_f16_to_f64(rd16(meta + 4 * g + 2));
    c[i] = q * s + z;
  }
}

/* dequantized rotated residual: e_i = (code_i - 1.5) * scale */
static void unpack_residual(const uint8_t* codes, const uint8_t* scale, int n, double* e) {
  double s = kvc_ref_f16_to_f64(rd16(scale));
  for (int i = 0; i < n; ++i) e[i] = (((codes[i / 4] >> (2 * (i % 4))) & 3) - 1.5) * s;
}

/* per-head mode: x = B c over the slot's rank, B stored [d][rcap] */
static void rebuild_per_head(const uint16_t* Bm, int d, int rcap, const double* c, int r, double* x) {
  for (int j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int i = 0; i < r; ++i) acc += kvc_ref_bf16_to_f64(Bm[(size_t)j * rcap + i]) * c[i];
    x[j] = acc;
  }
}

/* shared mode: x = W[:, h*d:(h+1)*d]^T c, W stored [latent][Hkv*d] */
static void rebuild_shared(const uint16_t* W, int lat, int width, int col0, int d, const double* c, double* x) {
  for (int j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int i = 0; i < lat; ++i) acc += kvc_ref_bf16_to_f64(W[(size_t)i * width + col0 + j]) * c[i];
    x[j] = acc;
  }
}

/* x += H e (the residual is stored in the rotated domain; H is its own inverse) */
static void add_residual(const double* H, int d, const double* e, double* x) {
  for (int j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += H[j * d + i] * e[i];
    x[j] += acc;
  }
}

/* the key (which = 0) or value (which = 1) of token t, pre-RoPE */
static void rebuild_token(const kvc_ref_layout* L, int which, int layer, int b, int h, int t, int max_blocks,
                          const int32_t* block_table, const uint8_t* pool, const int64_t* page_off,
                          const uint8_t* tok_rank, const uint32_t* tok_off, const uint16_t* w,
                          const double* H, double* c, double* e, double* x) {
  int d = L->head_dim, P = L->page_size, Hkv = L->n_kv_heads;
  int p = block_table[(size_t)b * max_blocks + t / P], s = t % P;
  if (L->shared) {
    int lat = L->r_k_cap;
    const uint8_t* rec = pool + page_off[p];
    const int lb = L->latent_bits;
    const uint8_t* codes = rec + (int64_t)s * (lat * lb / 8);
    const uint8_t* meta = rec + pad16((int64_t)P * lat * lb / 8) + (int64_t)s * 4 * ceil_div(lat, L->group);
    unpack_latent(L, lb, codes, meta, lat, lat, c);
    rebuild_shared(w + (size_t)layer * lat * Hkv * d, lat, Hkv * d, h * d, d, c, x);
    if (L->residual_bits) {  /* the (layer, head)'s own rotated residual */
      const uint8_t *kr, *vr, *ks, *vs;
      shared_residual_at(L, rec, layer, h, s, &kr, &vr, &ks, &vs);
      unpack_residual(which ? vr : kr, which ? vs : ks, d, e);
      add_residual(H, d, e, x);
    }
    return;
  }
  slot_view v = locate(L, pool, page_off, tok_rank, tok_off, p, s, h);
  int rcap = which ? L->r_v_cap : L->r_k_cap, r = which ? v.rv : v.rk;
  unpack_latent(L, lat_bits(L, which), which ? v.vc : v.kc, which ? v.vm : v.km, r, rcap, c);
  rebuild_per_head(w + (size_t)h * d * rcap, d, rcap, c, r, x);
  if (L->residual_bits) {
    unpack_residual(which ? v.vr : v.kr, which ? v.vs : v.ks, d, e);
    add_residual(H, d, e, x);
  }
}

/* Softmax attention of one (sequence, kv head[, layer]) group of query heads.
 * Pass 1 rebuilds each key, applies RoPE at its position and scores it;
 * pass 2 rebuilds each value and sums it with the softmax weights. */
static void attend_group(const kvc_ref_layout* L, int layer, int b, int h, int T, int qpos, int max_blocks,
                         const int32_t* block_table, const uint8_t* pool, const int64_t* page_off,
                         const uint8_t* tok_rank, const uint32_t* tok_off, const float* q,
                         const uint16_t* wk, const uint16_t* wv, const double* H, const uint32_t* keep,
                         double* out) {
  int d = L->head_dim, gsz = L->n_q_heads / L->n_kv_heads;
  double* qr = (double*)malloc(sizeof(double) * gsz * d);
  double* w = (double*)malloc(sizeof(double) * (size_t)gsz * T);
  double* c = (double*)malloc(sizeof(double) * 1024);
  double* e = (double*)malloc(sizeof(double) * 256);
  double* x = (double*)malloc(sizeof(double) * d);
  for (int g = 0; g < gsz; ++g) {               /* query heads of this kv head, rotated at q_pos */
    for (int j = 0; j < d; ++j) qr[g * d + j] = q[(size_t)(h * gsz + g) * d + j];
    kvc_ref_rope(qr + g * d, d, (double)qpos, L->rope_theta);
  }
  for (int t = 0; t < T; ++t) {                 /* scores q~ . k~_t / sqrt(d); an evicted token takes no part */
    if (keep && !((keep[t >> 5] >> (t & 31)) & 1u)) {
      for (int g = 0; g < gsz; ++g) w[(size_t)g * T + t] = -INFINITY;
      continue;
    }
    rebuild_token(L, 0, layer, b, h, t, max_blocks, block_table, pool, page_off, tok_rank, tok_off, wk, H, c, e, x);
    kvc_ref_rope(x, d, (double)t, L->rope_theta);
    for (int g = 0; g < gsz; ++g) {
      double dot = 0.0;
      for (int j = 0; j < d; ++j) dot += qr[g * d + j] * x[j];
      w[(size_t)g * T + t] = dot / sqrt((double)d);
    }
  }
  for (int g = 0; g < gsz; ++g) {               /* softmax over t, max-subtracted */
    double* wg = w + (size_t)g * T;
    double m = -INFINITY, l = 0.0;
    for (int t = 0; t < T; ++t) if (wg[t] > m) m = wg[t];
    if (m == -INFINITY) {                       /* every token evicted: no weight anywhere, output zero */
      for (int t = 0; t < T; ++t) wg[t] = 0.0;
      continue;
    }
    for (int t = 0; t < T; ++t) { wg[t] = exp(wg[t] - m); l += wg[t]; }
    for (int t = 0; t < T; ++t) wg[t] /= l;
  }
  for (int i = 0; i < gsz * d; ++i) out[i] = 0.0;
  for (int t = 0; t < T; ++t) {                 /* out = sum_t p_t v_t */
    if (keep && !((keep[t >> 5] >> (t & 31)) & 1u)) continue;
    rebuild_token(L, 1, layer, b, h, t, max_blocks, block_table, pool, page_off, tok_rank, tok_off, wv, H, c, e, x);
    for (int g = 0; g < gsz; ++g)
      for (int j = 0; j < d; ++j) out[(size_t)g * d + j] += w[(size_t)g * T + t] * x[j];
  }
  free(qr); free(w); free(c); free(e); free(x);
}

int kvc_ref_decode_attn(const kvc_ref_layout* L, int B, int max_blocks, const int32_t* block_table,
                        const int32_t* seq_len, const int32_t* q_pos, const uint8_t* pool,
                        const int64_t* page_off, const uint8_t* tok_rank, const uint32_t* tok_off,
                        const float* q, const uint16_t* wk, const uint16_t* wv,
                        const uint8_t* sel_b, const uint8_t* sel_h, double* out) {
  return kvc_ref_decode_attn_masked(L, B, max_blocks, block_table, seq_len, q_pos, pool, page_off, tok_rank, tok_off,
                                    q, wk, wv, NULL, 0, sel_b, sel_h, out);
}

int kvc_ref_decode_attn_masked(const kvc_ref_layout* L, int B, int max_blocks, const int32_t* block_table,
                               const int32_t* seq_len, const int32_t* q_pos, const uint8_t* pool,
                               const int64_t* page_off, const uint8_t* tok_rank, const uint32_t* tok_off,
                               const float* q, const uint16_t* wk, const uint16_t* wv, const uint32_t* keep,
                               int keep_words, const uint8_t* sel_b, const uint8_t* sel_h, double* out) {
  if (kvc_ref_layout_check(L)) return KVC_REF_EINVAL;
  int d = L->head_dim, Hq = L->n_q_heads, Hkv = L->n_kv_heads, NL = L->n_layers;
  int gsz = Hq / Hkv;
  double* H = NULL;
  if (L->residual_bits) { H = (double*)malloc(sizeof(double) * d * d); kvc_ref_hadamard(d, H); }
  for (int b = 0; b < B; ++b)
    if (seq_len[b] < 1 || seq_len[b] > max_blocks * L->page_size || (keep && seq_len[b] > 32 * keep_words)) {
      free(H);
      return KVC_REF_EINVAL;
    }
  int n_items = NL * B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int it = 0; it < n_items; ++it) {
    int layer = it / (B * Hkv), b = (it / Hkv) % B, h = it % Hkv;
    if (sel_b && !sel_b[b]) continue;
    if (sel_h && !sel_h[h]) continue;
    int qpos = q_pos ? q_pos[b] : seq_len[b];
    const float* ql = q + (((size_t)layer * B + b) * Hq) * d;
    double* o = out + ((((size_t)layer * B + b) * Hq) + (size_t)h * gsz) * d;
    attend_group(L, layer, b, h, seq_len[b], qpos, max_blocks, block_table, pool, page_off, tok_rank,
                 tok_off, ql, wk, wv, H, keep ? keep + (size_t)b * keep_words : NULL, o);
  }
  free(H);
  return 0;
}

/* OpenMP threads a parallel region of this library uses (1 without OpenMP). */
int kvc_ref_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

int kvc_ref_dense_attn(int Hq, int Hkv, int d, int P, int B, int max_blocks, const int32_t* block_table,
                       const int32_t* seq_len, const uint16_t* k_pages, const uint16_t* v_pages,
                       const float* q, const uint8_t* sel_b, double* out) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || P <= 0) return KVC_REF_EINVAL;
  int gsz = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int it = 0; it < B * Hq; ++it) {
    int b = it / Hq, hq = it % Hq, h = hq / gsz, T = seq_len[b];
    if (sel_b && !sel_b[b]) continue;
    double* sc = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double m = -INFINITY, l = 0.0;
    for (int t = 0; t < T; ++t) {
      int p = block_table[(size_t)b * max_blocks + t / P], s = t % P;
      const uint16_t* kr = k_pages + (((size_t)p * Hkv + h) * P + s) * d;
      double dot = 0.0;
      for (int j = 0; j < d; ++j) dot += (double)q[((size_t)b * Hq + hq) * d + j] * kvc_ref_bf16_to_f64(kr[j]);
      sc[t] = dot / sqrt((double)d);
      if (sc[t] > m) m = sc[t];
    }
    for (int t = 0; t < T; ++t) { sc[t] = exp(sc[t] - m); l += sc[t]; }
    double* o = out + ((size_t)b * Hq + hq) * d;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    for (int t = 0; t < T; ++t) {
      int p = block_table[(size_t)b * max_blocks + t / P], s = t % P;
      const uint16_t* vr = v_pages + (((size_t)p * Hkv + h) * P + s) * d;
      for (int j = 0; j < d; ++j) o[j] += sc[t] / l * kvc_ref_bf16_to_f64(vr[j]);
    }
    free(sc);
  }
  return 0;
}
