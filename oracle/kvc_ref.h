/*
 * kvc_ref.h -- CPU reference ("oracle") for decode attention over a
 * rank/bit-compressed KV cache.  TEST INFRASTRUCTURE ONLY: nothing in the
 * product library includes this header, links this code or calls it.  Only
 * the tests, the smoke check and the bench's CPU-baseline leg load it.
 *
 * Sources of the arithmetic (page titles, sections):
 *  - "BELT Connects KV-Cache Compression to Faster Long-Context Decoding",
 *    s.2-3: keys/values kept as low-rank coefficients, combined with a
 *    low-bit quantizer.
 *  - "BellowsKV Architecture ...", "Three Measurements, Three Operators":
 *    uniform integer quantization of a latent; "Share the Input, Not the
 *    Cache": each layer rebuilds its K and V from a shared latent through
 *    its own up-projection; "Worked Example": min/max asymmetric uniform
 *    quantizer (scale = range / (2^bits - 1), offset = group minimum,
 *    round-half-to-even) and the Sylvester Hadamard construction.
 *  - "A JoLT for the KV cache" abstract and the JoLT thesis page, "How JoLT
 *    works" / "Key findings": per-head feature-mode basis, keys decomposed
 *    before RoPE, a rotated low-bit quantizer on the truncation residual,
 *    attention evaluated directly over the stored factors.
 *  - "VarRate" summary, "Method": per-token variable rank, every token kept
 *    at nonzero rank.
 * The byte layout the oracle reads and writes is this project's own format
 * (the pages give none); it is written out in full in kvc_ref.c.
 *
 * All floating-point arithmetic of the attention is fp64.  The quantizers
 * work in fp32 with IEEE round-to-nearest-even and no contraction, because
 * their integer outputs must be bit-exact.
 */
#ifndef KVC_REF_H
#define KVC_REF_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int n_q_heads;     /* query heads per layer                                  */
  int n_kv_heads;    /* key/value heads per layer (GQA: q head h uses kv h/(Hq/Hkv)) */
  int head_dim;      /* d                                                      */
  int shared;        /* 0: per-KV-head bases; 1: one latent shared by n_layers */
  int n_layers;      /* layers served by one shared latent (1 when shared=0)  */
  int r_k_cap;       /* key rank (cap when variable_rank); shared: latent dim  */
  int r_v_cap;       /* value rank (cap); shared: equal to r_k_cap             */
  int group;         /* quantization group size along the latent axis          */
  int latent_bits;   /* key latent: 2, 3, 4 (codes + fp16 scale/zero) or 32 (fp32) */
  int residual_bits; /* 0 or 2 (Hadamard-rotated 2-bit residual, head_dim 128; per layer and head in shared mode) */
  int page_size;     /* tokens per page                                        */
  int variable_rank; /* 1: one rank per token, shared by K, V and all heads    */
  double rope_theta; /* RoPE base; 0 switches RoPE off                         */
  int latent_bits_v; /* value latent bits; 0 = latent_bits                     */
} kvc_ref_layout;

/* status codes: 0 ok, negative = invalid input */
int kvc_ref_layout_check(const kvc_ref_layout* L);
/* bytes of one page record when every slot holds rank r (uniform) */
int64_t kvc_ref_page_bytes_uniform(const kvc_ref_layout* L);

/* --- scalar helpers (exposed so tests can pin them) --- */
uint16_t kvc_ref_f32_to_f16(float x);     /* IEEE binary16, round to nearest even */
double   kvc_ref_f16_to_f64(uint16_t h);
double   kvc_ref_bf16_to_f64(uint16_t b);
void kvc_ref_quant_int4(const float* x, int n, uint16_t* s16, uint16_t* z16, uint8_t* codes);
/* the same quantizer with 2^bits - 1 levels, bits 2..4 */
void kvc_ref_quant_intb(const float* x, int n, int bits, uint16_t* s16, uint16_t* z16, uint8_t* codes);
void kvc_ref_quant_res2(const float* y, int n, uint16_t* s16, uint8_t* codes);
void kvc_ref_hadamard(int n, double* H);  /* normalized Sylvester matrix, row-major */
void kvc_ref_rope(double* x, int d, double pos, double theta);
/* array forms of the above, for tests */
void kvc_ref_f32_to_f16_n(const float* x, int64_t n, uint16_t* out);
void kvc_ref_quant_int4_n(const float* x, int64_t n_groups, int n, uint16_t* s16, uint16_t* z16, uint8_t* codes);
void kvc_ref_quant_intb_n(const float* x, int64_t n_groups, int n, int bits, uint16_t* s16, uint16_t* z16,
                          uint8_t* codes);
void kvc_ref_quant_res2_n(const float* y, int64_t n_rows, int n, uint16_t* s16, uint8_t* codes);

/* --- compression (from fp32 latents / rotated residuals) ---
 * block_table [B][max_blocks]; seq_len [B]; ranks [B][max_T] (variable_rank only)
 * lat_k, lat_v: [B][max_T][Hkv][r_cap] fp32 (shared mode: lat_k [B][max_T][latent])
 * res_k, res_v: [B][max_T][Hkv][128] fp32 (shared mode: [B][max_T][n_layers][Hkv][128]), already in the
 *   rotated domain (residual only)
 * outputs: pool (pool_bytes), page_off [n_pages], tok_rank [n_pages][P], tok_off [n_pages][P+1]
 * returns total bytes used (>= 0) or a negative status. */
int64_t kvc_ref_compress(const kvc_ref_layout* L, int B, int max_T, int max_blocks,
                         const int32_t* block_table, const int32_t* seq_len, const uint8_t* ranks,
                         const float* lat_k, const float* lat_v, const float* res_k, const float* res_v,
                         int n_pages, uint8_t* pool, int64_t pool_bytes, int64_t* page_off,
                         uint8_t* tok_rank, uint32_t* tok_off);

/* --- projection of dense pre-RoPE K/V onto the bases (the prefill side) ---
 * k, v: [B][max_T][Hkv][d] fp32; basis_k/v: bf16 bits [Hkv][d][r_cap]
 * writes lat_k/lat_v [B][max_T][Hkv][r_cap] (c = B_r^T k, rounded to fp32; zero beyond the
 * token's rank) and, when residual_bits, res_k/res_v = H (k - B_r B_r^T k) rounded to fp32. */
int kvc_ref_project(const kvc_ref_layout* L, int B, int max_T, const int32_t* seq_len, const uint8_t* ranks,
                    const float* k, const float* v, const uint16_t* basis_k, const uint16_t* basis_v,
                    float* lat_k, float* lat_v, float* res_k, float* res_v);

/* --- decode attention over the compressed cache, fp64 ---
 * q: fp32 [(L)][B][Hq][d] pre-RoPE; q_pos [B] (NULL: seq_len)
 * per-head mode: wk = basis_k, wv = basis_v (bf16 bits [Hkv][d][r_cap])
 * shared mode:   wk = W_k, wv = W_v (bf16 bits [n_layers][latent][Hkv*d])
 * sel_b [B] / sel_h [Hkv]: nonzero = compute (NULL = all); out [(L)][B][Hq][d] */
int kvc_ref_decode_attn(const kvc_ref_layout* L, int B, int max_blocks, const int32_t* block_table,
                        const int32_t* seq_len, const int32_t* q_pos, const uint8_t* pool,
                        const int64_t* page_off, const uint8_t* tok_rank, const uint32_t* tok_off,
                        const float* q, const uint16_t* wk, const uint16_t* wv,
                        const uint8_t* sel_b, const uint8_t* sel_h, double* out);

/* The same with a token keep mask (BellowsKV-Evict: one eviction decision per block of layers, applied to
 * the shared latent, so to every layer and head): keep [B][keep_words], bit t % 32 of word t / 32 set for a
 * kept token; an evicted token takes no part in the softmax or the value sum; a sequence that keeps no token
 * gets zero output.  keep NULL = every token kept.  seq_len[b] <= 32 keep_words. */
int kvc_ref_decode_attn_masked(const kvc_ref_layout* L, int B, int max_blocks, const int32_t* block_table,
                               const int32_t* seq_len, const int32_t* q_pos, const uint8_t* pool,
                               const int64_t* page_off, const uint8_t* tok_rank, const uint32_t* tok_off,
                               const float* q, const uint16_t* wk, const uint16_t* wv, const uint32_t* keep,
                               int keep_words, const uint8_t* sel_b, const uint8_t* sel_h, double* out);

/* OpenMP threads the parallel loops above use */
int kvc_ref_threads(void);

/* --- plain softmax attention over a paged bf16 cache (the dense comparison) ---
 * k_pages, v_pages: bf16 bits [n_pages][Hkv][P][d] (K already rotated); q fp32 [B][Hq][d] */
int kvc_ref_dense_attn(int Hq, int Hkv, int d, int P, int B, int max_blocks, const int32_t* block_table,
                       const int32_t* seq_len, const uint16_t* k_pages, const uint16_t* v_pages,
                       const float* q, const uint8_t* sel_b, double* out);

#ifdef __cplusplus
}
#endif
#endif
