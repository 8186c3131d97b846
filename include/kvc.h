/*
 * kvc.h -- C ABI of librbc_kvc.so: decode-step attention read directly from
 * a rank/bit-compressed KV cache, on AMD Instinct MI355X (gfx950).
 *
 * What is computed (page titles and sections of the method's descriptions):
 *  - Keys and values of each cached token are kept as rank-r latent
 *    coefficients against a per-KV-head basis ("BELT Connects KV-Cache
 *    Compression ...", s.2-3; JoLT thesis page, "Key findings": per-head
 *    SVD), or as one latent per token shared by a block of layers, from
 *    which each layer rebuilds its own K and V through its own
 *    up-projection ("BellowsKV Architecture ...", "Share the Input, Not
 *    the Cache").
 *  - The latents are stored as INT4 codes with one fp16 scale and one fp16
 *    zero per group of coordinates (BellowsKV, "Three Measurements, Three
 *    Operators"; "Worked Example" gives the min/max quantizer form).
 *  - Optional: a per-token rank, every token kept at nonzero rank
 *    ("VarRate", "Method"); a 2-bit residual in a Hadamard-rotated domain
 *    ("A JoLT for the KV cache", abstract: rotated low-bit residual).
 *  - Keys are stored before RoPE and rotated after reconstruction (JoLT
 *    thesis page, "Key findings"); attention is evaluated over the stored
 *    factors without writing a dense K/V to memory (JoLT abstract,
 *    FlashJoLT decode kernel).
 *
 * Conventions for every call:
 *  - Device pointers are HIP device memory on the current device; the
 *    caller owns and allocates all of it (inputs, outputs, workspace).
 *    Structs and their host fields are read during the call only.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *    Nothing synchronizes; errors raised by kernels surface on the stream.
 *  - A non-zero return means nothing was launched.  All argument checks
 *    happen before the first launch.  No C++ exception crosses the ABI.
 *  - Device data is trusted: out-of-range page ids in a block table or
 *    ranks that disagree with the offset tables are undefined behaviour.
 *  - Pointers must be 16-byte aligned (KVC_ERR_MISALIGNED otherwise).
 *  - Same inputs and the same num_splits give bit-identical output; the
 *    summation order depends on logical positions only, so a permuted page
 *    table changes nothing.
 *
 * Byte layout of the compressed cache ("KVC-1"):
 *  The pool is a sequence of page records, one per physical page p, at byte
 *  offset page_off[p] (the exclusive prefix sum of record sizes over p).
 *  Token t of sequence b sits in page block_table[b][t / P], slot t % P.
 *  Per-head mode: a record is n_kv_heads head blocks of equal size, head 0
 *  first; a head block is the sections
 *     Kc key codes   | Vc value codes | Km key (scale, zero) | Vm value pairs
 *     [Kr key residual codes P x 32 B | Vr | Ks key residual scale P x fp16 | Vs]
 *  each padded to a multiple of 16 bytes.  Codes of a slot are its rank r
 *  b-bit values (b = latent_bits for keys, latent_bits_v for values; 2, 3 or
 *  4), code i at bits b*i .. b*i + b - 1 of the slot's little-endian bit
 *  string, r*b/8 bytes (INT4: coordinate 2j in the low nibble of byte j;
 *  fp32 latents: 4r bytes and no pairs); pairs are (fp16 scale, fp16 zero), one
 *  per group of `group` coordinates, ceil(r/group) per slot; residual
 *  element i is bits 2(i%4).. of byte i/4, value (code - 1.5) * scale.
 *  Slots follow one another in slot order inside each section.  Uniform
 *  rank: every slot of every page holds r_k_cap / r_v_cap.  Variable rank:
 *  tok_rank[p][s] (0 for unused slots) is the rank of K and V for all heads,
 *  and tok_off[p][s] holds the exclusive prefix over slots of the ranks
 *  (bits 0-15) and of ceil(rank/group) (bits 16-31); tok_off[p][P] = totals.
 *  Block-shared mode: a record is Lc (P x latent*b/8 code bytes) and Lm
 *  (P x latent/group pairs), each padded to 16 bytes; with the residual
 *  (each layer and kv head its own: JoLT thesis page, "How JoLT works", a
 *  Tucker form plus a rotated low-bit residual) then Kr and Vr (one part of
 *  P x 32 code bytes per (layer, kv head), layer-major) and Ks and Vs (one
 *  part of P fp16 scales per (layer, kv head), each padded to 16 bytes).
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 8

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = -1,     /* a size, pointer or layout field is out of range        */
  KVC_ERR_UNSUPPORTED = -2,     /* valid, but no kernel for this geometry                 */
  KVC_ERR_WORKSPACE = -3,       /* workspace or pool smaller than required                */
  KVC_ERR_MISALIGNED = -4,      /* a pointer is not 16-byte aligned                       */
  KVC_ERR_HIP = -5,             /* a HIP runtime call failed (see kvc_last_hip_error)     */
  KVC_ERR_SCRATCH = -6          /* kvc_decode_attn_noalloc: the step needs more scratch than
                                   KVC_NOALLOC_SCRATCH_BYTES (ABI version 6)              */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* Geometry and format of a compressed cache. */
typedef struct {
  int32_t n_q_heads;      /* query heads per layer                                         */
  int32_t n_kv_heads;     /* KV heads per layer; q head h reads kv head h / (Hq / Hkv)     */
  int32_t head_dim;       /* d: 64 or 128                                                  */
  int32_t shared;         /* 0: per-KV-head bases; 1: one latent per token for n_layers    */
  int32_t n_layers;       /* layers served by a shared latent (1 when shared = 0)          */
  int32_t r_k_cap;        /* key rank (cap with variable_rank); shared: latent dimension   */
  int32_t r_v_cap;        /* value rank (cap); shared: equal to r_k_cap                    */
  int32_t group;          /* quantization group along the latent axis (multiple of 16)     */
  int32_t latent_bits;    /* key latent: 2, 3, 4 (codes + fp16 scale/zero) or 32 (fp32)   */
  int32_t residual_bits;  /* 0 or 2 (Hadamard-rotated residual; head_dim 128; shared mode:  */
                          /*   one per layer and kv head, INT4 latent)                     */
  int32_t page_size;      /* tokens per page, a multiple of 32, at most 256                */
  int32_t variable_rank;  /* 1: per-token rank in tok_rank / tok_off                       */
  double rope_theta;      /* RoPE base (rotate-half pairs (j, j + d/2)); 0 = no RoPE       */
  int32_t latent_bits_v;  /* value latent bits, 2..4 or 32; 0 = latent_bits (ABI version 2)  */
} kvc_layout;

/* A compressed cache in device memory (caller-allocated). */
typedef struct {
  uint8_t* pool;          /* page records                                                  */
  int64_t pool_bytes;     /* capacity of pool                                              */
  int64_t* page_off;      /* [n_pages] byte offset of each record                          */
  uint8_t* tok_rank;      /* [n_pages][page_size], variable rank only (else NULL)          */
  uint32_t* tok_off;      /* [n_pages][page_size + 1], variable rank only (else NULL)      */
  int64_t* used_bytes;    /* [1] written by kvc_compress: bytes of pool in use (may be NULL) */
  int32_t n_pages;
} kvc_cache;

typedef enum { KVC_FROM_LATENT = 0, KVC_FROM_DENSE = 1 } kvc_compress_mode;

/* Inputs of kvc_compress.  All arrays are device memory. */
typedef struct {
  int32_t mode;                  /* kvc_compress_mode                                          */
  int32_t B, max_T, max_blocks;  /* sequences, row length of the token arrays, table width     */
  const int32_t* block_table;    /* [B][max_blocks]; distinct pages for blocks in use           */
  const int32_t* seq_len;        /* [B], 1..max_T tokens to compress per sequence               */
  const uint8_t* ranks;          /* [B][max_T] variable rank: multiple of 8 in [8, cap]        */
  /* FROM_LATENT: fp32 latents [B][max_T][Hkv][r_cap] (shared mode: lat_k [B][max_T][latent]),
   * rotated-domain residuals [B][max_T][Hkv][head_dim] (residual_bits = 2; shared mode
   * [B][max_T][n_layers][Hkv][head_dim]).
   * FROM_DENSE: these four are outputs (required): the fp32 projection c = B_r^T k truncated to
   * the token's rank, and the rotated truncation residual H (k - B_r c), which are then quantized. */
  float* lat_k;
  float* lat_v;
  float* res_k;
  float* res_v;
  /* FROM_DENSE only: pre-RoPE keys/values [B][max_T][Hkv][head_dim] fp32, bases bf16 [Hkv][d][r_cap] */
  const float* k;
  const float* v;
  const uint16_t* basis_k;
  const uint16_t* basis_v;
} kvc_compress_in;

/* Inputs of kvc_decode_attn.  All arrays are device memory. */
typedef struct {
  int32_t B, max_blocks;         /* sequences, block-table width                               */
  int32_t max_T;                 /* host-side upper bound of seq_len (sizes the grid)          */
  const int32_t* block_table;    /* [B][max_blocks]                                             */
  const int32_t* seq_len;        /* [B], cached tokens, 1..max_T                                */
  const int32_t* q_pos;          /* [B] RoPE position of the query, NULL = seq_len              */
  const void* q;                 /* [(n_layers)][B][Hq][d] pre-RoPE, q_dtype                     */
  int32_t q_dtype;               /* kvc_dtype                                                   */
  const uint16_t* wk;            /* bf16 basis [Hkv][d][r_k_cap]; shared: W_k [L][latent][Hkv*d] */
  const uint16_t* wv;            /* bf16 basis [Hkv][d][r_v_cap]; shared: W_v [L][latent][Hkv*d] */
                                 /*   The matrix instructions take wk and wv as fp16, converted   */
                                 /*   exactly only for entries of magnitude 2^-14 .. 65504 (fp16's */
                                 /*   normal range; the orthonormal bases and the 1/sqrt(512)-scale */
                                 /*   W of the workloads here lie well inside it): larger entries */
                                 /*   overflow to infinity, smaller ones lose bits (subnormals down */
                                 /*   to 2^-24, then zero).  Outside that range the result is not */
                                 /*   the attention the header defines.                            */
  int32_t num_splits;            /* context splits per (sequence, head); 0 = automatic          */
  int64_t w_seq_stride;          /* shared mode: elements from one sequence's W_k (and W_v) to  */
                                 /*   the next, a multiple of 8; 0 = one pair for all sequences  */
                                 /*   (per-sequence up-projections, e.g. expanded from a Tucker */
                                 /*   core fitted per prefill cache).  Per-head mode: 0          */
  const uint32_t* keep_mask;     /* shared mode, optional: token keep mask [B][keep_words], bit  */
                                 /*   t % 32 of word t / 32 set for a kept token (BellowsKV-Evict */
                                 /*   page: one eviction decision for the block's layers, applied */
                                 /*   to the shared latent).  Evicted tokens take no part in the  */
                                 /*   softmax; a sequence keeping none gets zero output.  NULL =  */
                                 /*   all kept; per-head mode: NULL.  4-byte aligned              */
  int32_t keep_words;            /* words per sequence of keep_mask (tokens past 32 keep_words   */
                                 /*   count as evicted)                                           */
  int32_t kv_split;              /* shared mode: 0, or latent / 2 when the latent's lower half    */
                                 /*   feeds only the keys and the upper half only the values (W_k */
                                 /*   zero on rows >= latent / 2, W_v zero below: keys and values */
                                 /*   with their own token factors, kvc_tucker_expand).  The      */
                                 /*   kernel then skips those zero products; the output is that   */
                                 /*   of the full product.  Per-head mode: 0                      */
  const int32_t* tok_pos;        /* shared mode, optional (ABI version 8): [B][max_blocks *       */
                                 /*   page_size] source position of the token in each slot of a   */
                                 /*   compacted cache (kvc_evict_compact), -1 for a slot with no  */
                                 /*   token.  Keys are rotated at these positions and slots of -1 */
                                 /*   take no part.  Within each 32-slot tile the tokens must lie */
                                 /*   within 4 blocks of 32 positions of the tile's first slot's   */
                                 /*   block (the layout kvc_evict_compact writes; other tokens are */
                                 /*   ignored).  Requires q_pos and no keep_mask.  NULL: slot t   */
                                 /*   holds position t.  4-byte aligned                           */
} kvc_decode_in;

/* Inputs of kvc_dense_decode_attn: plain attention over a paged bf16 cache. */
typedef struct {
  int32_t n_q_heads, n_kv_heads, head_dim, page_size;
  int32_t B, max_blocks, max_T;
  const int32_t* block_table;    /* [B][max_blocks]                                             */
  const int32_t* seq_len;        /* [B]                                                          */
  const uint16_t* k_pages;       /* bf16 [n_pages][Hkv][page_size][d], keys already rotated     */
  const uint16_t* v_pages;       /* bf16 [n_pages][Hkv][page_size][d]                           */
  const void* q;                 /* [B][Hq][d], already rotated, q_dtype                        */
  int32_t q_dtype;
  int32_t num_splits;            /* 0 = automatic                                               */
} kvc_dense_in;

/* ABI version of the loaded library (KVC_ABI_VERSION). */
int32_t kvc_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* kvc_status_string(int32_t status);

/* hipError_t of the last failed HIP call made by this thread (0 if none). */
int32_t kvc_last_hip_error(void);

/* Checks a layout against what the library supports. KVC_OK, INVALID_ARG or UNSUPPORTED. */
kvc_status kvc_layout_check(const kvc_layout* layout);

/* Upper bound of the pool bytes for n_pages pages (every slot at the rank cap). */
kvc_status kvc_pool_bytes_max(const kvc_layout* layout, int32_t n_pages, int64_t* bytes);

/* Compression (the prefill side; "BELT ...", s.3 low rank + quantization; BellowsKV
 * "Three Measurements, Three Operators"; JoLT abstract for the rotated residual).
 * FROM_LATENT quantizes given fp32 latents (and rotated residuals) and packs them into
 * the pool; FROM_DENSE first projects dense pre-RoPE K/V onto the bases (truncated to each
 * token's rank), forms the truncation residual and rotates it with the normalized
 * 128-point Sylvester Hadamard, then quantizes as FROM_LATENT.  Quantizer, per group of
 * `group` coordinates of one token (the last group of a token may be shorter):
 * lo/hi = min/max, scale = fp16((hi - lo) / 15), zero = fp16(lo),
 * code = clamp(rint((x - zero) / scale), 0, 15) in fp32 (0 when scale = 0).  Residual
 * (128 values): scale = fp16(max|y| / 1.5), code = clamp(rint(y / scale + 1.5), 0, 3)
 * (2 when scale = 0).  Writes pool, page_off, tok_rank, tok_off and used_bytes;
 * fills every byte of the pool in use (padding zero).  Slots of pages that no sequence
 * uses hold rank 0 (variable rank).  Returns KVC_ERR_WORKSPACE if pool_bytes is below
 * kvc_pool_bytes_max. */
kvc_status kvc_compress(const kvc_layout* layout, const kvc_compress_in* in, const kvc_cache* cache,
                        void* stream);

/* Bytes of workspace kvc_decode_attn needs for B sequences of up to max_T tokens and the
 * given num_splits (0 = automatic: the same choice kvc_decode_attn makes). */
kvc_status kvc_decode_workspace_bytes(const kvc_layout* layout, int32_t B, int32_t max_T, int32_t num_splits,
                                      size_t* bytes);

/* One decode step of softmax attention over the compressed cache (hot path).
 * For every sequence b, layer l (shared mode) and query head h with kv head g = h / (Hq/Hkv):
 *   k_t = B_k[g] c_k(t) [+ H e_k(t)]   (shared: W_k[l][:, g*d:(g+1)*d]^T c(t) [+ H e_k(l, g, t)])
 *   v_t = B_v[g] c_v(t) [+ H e_v(t)]
 *   out[l][b][h] = sum_t softmax_t( RoPE(q, q_pos) . RoPE(k_t, t) / sqrt(d) ) v_t,  t < seq_len[b]
 * with c the dequantized latent (code * scale + zero, zero beyond the token's rank), e the
 * dequantized rotated residual and H the normalized 128-point Sylvester Hadamard.
 * out: fp32 [(n_layers)][B][Hq][d].  ws: workspace of kvc_decode_workspace_bytes.  A block-shared layout with
 * the residual takes no keep_mask or tok_pos (UNSUPPORTED). */
kvc_status kvc_decode_attn(const kvc_layout* layout, const kvc_cache* cache, const kvc_decode_in* in,
                           float* out, void* ws, size_t ws_bytes, void* stream);

/* kvc_decode_attn with a measurement hook: ev_begin and ev_end are caller-created hipEvent_t
 * handles (passed as void*), recorded on `stream` immediately before and after the launch of the
 * attention kernel; the split merge that follows lies outside the pair.  hipEventElapsedTime of
 * the pair is then the attention kernel's own duration.  Same results and errors as
 * kvc_decode_attn; both events are required (INVALID_ARG otherwise), and on an error returned
 * before the launch neither event is recorded.  The events stay owned by the caller. */
kvc_status kvc_decode_attn_timed(const kvc_layout* layout, const kvc_cache* cache, const kvc_decode_in* in,
                                 float* out, void* ws, size_t ws_bytes, void* stream, void* ev_begin,
                                 void* ev_end);

/* Bytes of the device array that holds kvc_decode_attn_noalloc's split partials (8 MiB; the largest
 * workload here, 8 sequences of 131072 tokens with the rotated residual, needs 3 MiB). */
#define KVC_NOALLOC_SCRATCH_BYTES (8u << 20)

/* kvc_decode_attn for callers that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid device allocation.  The same kernels and results as kvc_decode_attn with the same
 * num_splits, but the split partials go to a file-scope device array of KVC_NOALLOC_SCRATCH_BYTES per GPU,
 * which the library holds until the process ends; nothing is allocated or freed (the array's device address is
 * looked up once per GPU, on that GPU's first call, with hipGetSymbolAddress).  The caller still passes the
 * inputs and out.  Returns KVC_ERR_SCRATCH, before any device call, when kvc_decode_workspace_bytes for these
 * sizes exceeds KVC_NOALLOC_SCRATCH_BYTES; otherwise the statuses of kvc_decode_attn.  All calls on one GPU
 * share its array: calls that overlap on one GPU (other streams, other threads) race and give wrong results.
 * Each call writes every partial it reads, so the array needs no clearing between calls. */
kvc_status kvc_decode_attn_noalloc(const kvc_layout* layout, const kvc_cache* cache, const kvc_decode_in* in,
                                   float* out, void* stream);

/* Which decode kernel kvc_decode_attn runs for a layout: KVC_PATH_INT4 (per-head INT4 latents,
 * head_dim 128, no residual: the fast kernel), KVC_PATH_RES (per-head INT4 latents with the 2-bit
 * rotated residual, head_dim 128, four query heads per KV head, uniform ranks that are multiples of
 * 16 up to 64), KVC_PATH_HEAD (the general per-head kernel: fp32 latents, head_dim 64, the other
 * residual layouts) or KVC_PATH_SHARED (block-shared latents).  Host-only; returns the layout
 * check's status when the layout is not runnable. */
enum { KVC_PATH_HEAD = 0, KVC_PATH_INT4 = 1, KVC_PATH_SHARED = 2, KVC_PATH_RES = 3 };
kvc_status kvc_decode_path(const kvc_layout* layout, int32_t* path);

/* Inputs of kvc_fit_basis.  All arrays are device memory. */
typedef struct {
  int32_t B, max_T;              /* sequences, row length of x                                  */
  int32_t n_kv_heads;            /* Hkv                                                          */
  int32_t head_dim;              /* d: 128                                                       */
  int32_t rank;                  /* r: 1..head_dim columns of the basis                          */
  int32_t r_cap;                 /* columns of the bf16 basis, rank..head_dim (zero beyond rank) */
  const int32_t* seq_len;        /* [B] rows used per sequence, 0..max_T                         */
  const float* x;                /* [B][max_T][Hkv][head_dim] pre-RoPE keys (or values), fp32     */
} kvc_fit_in;

/* Workspace bytes of kvc_fit_basis for these sizes (pointers are not read). */
kvc_status kvc_fit_workspace_bytes(const kvc_fit_in* in, size_t* bytes);

/* Basis fitting for the prefill side: per KV head h, the rank leading right singular vectors of X_h, the
 * matrix whose rows are x[b][t][h][:] for every t < seq_len[b] of every sequence ("JoLT: Near-Lossless KV
 * Cache Compression", "Key findings": per-head SVD, keys taken before RoPE; "A JoLT for the KV cache",
 * abstract: the feature mode is the truncated one).  No mean is removed.  Columns are ordered by
 * decreasing singular value and signed so that each column's entry of largest magnitude is positive.
 * Computed as the eigenvectors of X_h^T X_h (fp32 accumulation on the matrix cores, then Jacobi rotations
 * in fp32).  Outputs (any may be NULL, not all):
 *   basis_bf16 [Hkv][d][r_cap] bf16, round to nearest even, columns rank..r_cap-1 zero: the layout
 *     kvc_compress (basis_k / basis_v) and kvc_decode_attn (wk / wv) take;
 *   basis_f32 [Hkv][d][rank];
 *   sigma2 [Hkv][d] the eigenvalues of X_h^T X_h (squared singular values), decreasing, clamped at 0.
 * A head with no rows gets the first rank coordinate axes.  Where singular values coincide the
 * columns are any orthonormal basis of their common space.  Non-finite inputs give unspecified (but
 * finite-time) results.  ws: workspace of kvc_fit_workspace_bytes.  Deterministic. */
kvc_status kvc_fit_basis(const kvc_fit_in* in, uint16_t* basis_bf16, float* basis_f32, float* sigma2, void* ws,
                         size_t ws_bytes, void* stream);

/* kvc_fit_basis with a measurement hook: ev_begin and ev_end are caller-created hipEvent_t handles
 * (passed as void*), recorded on `stream` immediately before and after the launch of the Gram-matrix
 * kernel (the data-parallel pass over the rows); the reduction and the eigensolver that follow lie
 * outside the pair.  Same results and errors as kvc_fit_basis; both events are required (INVALID_ARG
 * otherwise), and on an error returned before the launch neither event is recorded.  The events stay
 * owned by the caller. */
kvc_status kvc_fit_basis_timed(const kvc_fit_in* in, uint16_t* basis_bf16, float* basis_f32, float* sigma2, void* ws,
                               size_t ws_bytes, void* stream, void* ev_begin, void* ev_end);

/* Inputs of kvc_salience.  All arrays are device memory. */
typedef struct {
  int32_t B, max_T;              /* sequences, row length of k                                  */
  int32_t W;                     /* window queries per sequence, 1..32                           */
  int32_t n_q_heads, n_kv_heads; /* Hq = 4 Hkv                                                   */
  int32_t head_dim;              /* d: 128                                                       */
  double rope_theta;             /* RoPE base (rotate-half pairs (j, j + d/2)); 0 = no RoPE      */
  const int32_t* seq_len;        /* [B] tokens per sequence, 0..max_T                            */
  const float* q;                /* [B][W][Hq][d] pre-RoPE; query i at position seq_len - W + i  */
  const float* k;                /* [B][max_T][Hkv][d] pre-RoPE keys                             */
} kvc_salience_in;

/* Workspace bytes of kvc_salience for these sizes (pointers are not read). */
kvc_status kvc_salience_workspace_bytes(const kvc_salience_in* in, size_t* bytes);

/* Query salience of every cached token, the input of the per-token rank choice ("VarRate: Training-Free
 * Variable-Rate KV Cache Compression for Long-Context LLMs", "Method": a token's rank follows its query
 * salience).  The page defines no formula; the one computed: sal[b][t] is the attention probability that
 * the window queries put on token t, summed over the queries present (positions >= 0) and all query heads;
 * each query attends causally (keys t <= its position), RoPE rotates queries and keys at their positions,
 * scores are q.k / sqrt(d), and query head h reads KV head h / (Hq / Hkv).  A sequence's values sum to
 * (queries present) x Hq.  Scores in fp32 on the matrix cores, exp2 in fp32.  out: fp32 [B][max_T], zero
 * at t >= seq_len.  ws: workspace of kvc_salience_workspace_bytes.  Deterministic. */
kvc_status kvc_salience(const kvc_salience_in* in, float* out, void* ws, size_t ws_bytes, void* stream);

/* Inputs of kvc_rank_alloc.  sal and seq_len are device memory; the rest is read on the host. */
typedef struct {
  int32_t B, max_T;
  int32_t n_ladder;              /* m, 2..8 rungs                                               */
  int32_t ladder[8];             /* ranks r_0 < ... < r_{m-1}, each 1..255                       */
  float step_w[7];               /* w_j >= 0, non-increasing: value per rank unit of step j       */
  double mean_rank;              /* budget per token, in [r_0, r_{m-1}]                          */
  const int32_t* seq_len;        /* [B] tokens per sequence, 0..max_T                            */
  const float* sal;              /* [B][max_T] salience, >= 0 (for instance kvc_salience's)      */
} kvc_alloc_in;

/* Per-token ranks under a budget ("VarRate ...", "Method" and "Principles": ranks follow query salience
 * and no token drops to rank zero).  Every token starts at r_0; the step r_j -> r_{j+1} of token t costs
 * r_{j+1} - r_j and gains the fp32 product sal[b][t] * w_j.  Steps are taken in decreasing order of
 * gain, equal gains together, while the sequence's total rank stays within floor(mean_rank * seq_len[b])
 * (evaluated in double); the first group that does not fit ends it.  With w non-increasing a token's
 * steps are taken in order, and a more salient token never gets a lower rank.  ranks: uint8 [B][max_T],
 * 0 at t >= seq_len (the per-token ranks kvc_compress takes, with a ladder of multiples of 8).  One
 * workgroup per sequence.  Deterministic. */
kvc_status kvc_rank_alloc(const kvc_alloc_in* in, uint8_t* ranks, void* stream);

/* Inputs of kvc_plan_budget (host memory). */
typedef struct {
  int32_t n_cells;               /* cells, e.g. the keys and the values of each layer (group)   */
  int32_t n_options;             /* options per cell, 1..1024 (pad a shorter list with a copy); */
                                 /*   n_cells * n_options <= 2^22                                */
  const double* distortion;      /* [n_cells][n_options] reconstruction error of each option   */
  const double* bytes;           /* [n_cells][n_options] storage cost, >= 0 (whole numbers keep */
                                 /*   the sums exact)                                           */
  double budget;                 /* total bytes                                                 */
} kvc_plan_in;

/* Lagrangian allocation of a byte budget ("JoLT: Near-Lossless KV Cache Compression" thesis page, "How
 * JoLT works": one multiplier picks every cell's ranks and residual bit width under a shared budget).  For
 * a multiplier lam >= 0 each cell takes the option minimizing distortion + lam * bytes (ties: fewer bytes);
 * as lam falls the choice walks up the cell's lower convex hull of (bytes, distortion) points, switching at
 * breakpoints, and the choice at lam is decided by comparing lam with those breakpoints.  lam is the
 * smallest of 0 and the breakpoints whose choices fit the budget; then cells on a breakpoint equal to lam
 * move on along their hull, in cell order, while the bytes still fit.  No allocation of at most the same
 * bytes has less total distortion.  Host code, no device work.  choice: [n_cells] option per cell;
 * lambda (optional): the multiplier.  INVALID_ARG for non-finite or negative inputs, sizes out of range,
 * or a budget below the cheapest options. */
kvc_status kvc_plan_budget(const kvc_plan_in* in, int32_t* choice, double* lambda);

/* Inputs of kvc_tucker_expand (device memory). */
typedef struct {
  int32_t n_seq;                 /* sequences, each with its own factors and up-projections      */
  int32_t n_layers;              /* L, layers of the group                                       */
  int32_t n_kv_heads;            /* Hkv                                                          */
  int32_t head_dim;              /* d (128)                                                      */
  int32_t r_t;                   /* token rank: latent rows written                              */
  int32_t r_f;                   /* feature rank, 1..d                                           */
  int32_t latent;                /* rows of each W[l] (the shared latent dimension), <= 4096     */
  int32_t row0;                  /* first row written; row0 + r_t <= latent                      */
  const float* u_f;              /* [n_seq][d][r_f] feature factor                               */
  const float* core;             /* [n_seq][L][Hkv][r_t][r_f] core, one (layer, head) slice after */
                                 /*   another                                                    */
} kvc_tucker_in;

/* Up-projections of a partial Tucker cache ("JoLT: Near-Lossless KV Cache Compression" thesis page, "How
 * JoLT works": a layer group's keys or values as a token x feature x head x layer tensor, only the token
 * and feature modes truncated, X ~ G x_1 U_t x_2 U_f).  Token t's factor row U_t[t] is the block-shared
 * latent of every head and layer of the group; head h of layer l rebuilds its pre-RoPE key (value) as
 * W_hl^T U_t[t] with W_hl = U_f G[:, :, h, l]^T.  Writes, for c < r_t,
 *   w[s][l][row0 + c][h*d + i] = sum_j u_f[s][i][j] core[s][l][h][c][j]
 * (fp32 fused multiply-adds in increasing j, stored as bf16 rounded to nearest even; w_f32, optional, the
 * fp32 sums) in the layout kvc_decode_attn takes for per-sequence up-projections ([n_seq][L][latent][Hkv*d],
 * w_seq_stride = L * latent * Hkv * d).  Rows outside row0..row0+r_t-1 are not written: keys and values
 * with their own token factors share one latent as [U_t(keys) | U_t(values)], W_k holding the key rows
 * (values' rows zero) and W_v the reverse.  Asynchronous on stream.  INVALID_ARG for bad sizes or null
 * pointers, UNSUPPORTED for d != 128, MISALIGNED for pointers not 4-byte aligned. */
kvc_status kvc_tucker_expand(const kvc_tucker_in* in, uint16_t* w, float* w_f32, void* stream);

/* Inputs of kvc_tucker_fit (device memory). */
typedef struct {
  int32_t B, max_T;              /* sequences, token rows of x per sequence                        */
  int32_t n_layers;              /* L, layers of the group                                         */
  int32_t n_kv_heads;            /* Hkv                                                            */
  int32_t head_dim;              /* d (128)                                                        */
  int32_t r_t;                   /* token rank: a multiple of 4, 4..256, at most seq_len[b]        */
  int32_t r_f;                   /* feature rank: a multiple of 4, 4..d                            */
  int32_t power_iters;           /* q, 0..8                                                        */
  int32_t ut_ld;                 /* row stride of u_t in floats, a multiple of 4 >= r_t (0: r_t)   */
  const int32_t* seq_len;        /* [B] token rows used per sequence (clamped to 0..max_T)         */
  const float* x;                /* [B][max_T][L][Hkv][d] the group's keys (or values), fp32       */
  const float* omega;            /* [L*Hkv*d][r_t] Gaussian test matrix, rows in (l, h, i) order    */
} kvc_tucker_fit_in;

/* Workspace bytes of kvc_tucker_fit for these sizes (pointers are not read). */
kvc_status kvc_tucker_fit_workspace_bytes(const kvc_tucker_fit_in* in, size_t* bytes);

/* Partial Tucker factors of each sequence's layer group ("JoLT: Near-Lossless KV Cache Compression" thesis
 * page, "How JoLT works": token and feature modes truncated, heads and layers kept; "A JoLT for the KV cache",
 * abstract: FlashJoLT's randomized token-mode factor).  With A the sequence's token-mode unfolding (row t:
 * x[b][t][...] flattened in (l, h, i) order, rows t < seq_len[b]):
 *   u_t [B][max_T][ut_ld]: columns 0..r_t-1 the randomized subspace iteration Q = orth(A omega), then
 *     power_iters times Z = orth(A^T Q), Q = orth(A Z), where orth(Y) is the Q factor of Y's QR decomposition
 *     with a positive diagonal R (CholeskyQR2, Gram matrices and Cholesky factors in fp64, products in fp32);
 *     rows t >= seq_len[b] are zero; other columns are not written;
 *   u_f [B][d][r_f]: the r_f leading left singular vectors of the feature-mode unfolding (every (t, l, h)
 *     row of the sequence), ordered and signed as by kvc_fit_basis;
 *   core [B][L][Hkv][r_t][r_f]: core[b][l][h][c][j] = sum_t sum_i u_t[b][t][c] x[b][t][l][h][i] u_f[b][i][j],
 *     the layout kvc_tucker_expand takes.
 * info [B] (optional): 0, or 1 where an orthonormalisation met a numerically dependent column (a Cholesky
 * pivot at or below 2^-40 of its diagonal entry: seq_len[b] < r_t, a token rank above the numerical rank of
 * the rows at fp32 precision) or a non-finite one; that sequence's factors are then unspecified (finite
 * where its rows are).  Products are summed in a fixed order: deterministic.  x, omega, u_t, u_f, core and
 * ws 16-byte aligned (MISALIGNED otherwise).  INVALID_ARG for bad sizes or null pointers, UNSUPPORTED for
 * d != 128 or ranks outside the ranges above, WORKSPACE for ws_bytes below kvc_tucker_fit_workspace_bytes.
 * Asynchronous on stream. */
kvc_status kvc_tucker_fit(const kvc_tucker_fit_in* in, float* u_t, float* u_f, float* core, int32_t* info, void* ws,
                          size_t ws_bytes, void* stream);

/* Inputs of kvc_evict_select (device memory). */
typedef struct {
  int32_t B, max_T;              /* sequences, scores per sequence and layer                     */
  int32_t n_layers;              /* layers of the block whose scores decide together             */
  double keep_ratio;             /* in (0, 1]: a sequence of T tokens keeps                      */
                                 /*   min(T, max(1, floor(keep_ratio * T))) of them (none if T=0)*/
  const int32_t* seq_len;        /* [B] tokens per sequence, 0..max_T                            */
  const float* scores;           /* [n_layers][B][max_T] per-layer token importance, not NaN      */
                                 /*   (for instance kvc_salience of each layer)                   */
} kvc_evict_in;

/* Block-level eviction decision ("BellowsKV" page, "Three Measurements, Three Operators": layers of a block
 * rank token importance alike, so one decision made from all the block's layers' scores is applied once to
 * the shared latent).  A token's block score is the fp32 sum of its layers' scores in layer order; each
 * sequence keeps the tokens of largest block score, equal scores in increasing position, as many as
 * keep_ratio gives (at least one).  keep_mask: [B][ceil(max_T / 32)] words, bit t % 32 of word t / 32 set
 * for a kept token, zero past seq_len: the mask kvc_decode_attn takes (keep_words = ceil(max_T / 32)).
 * One workgroup per sequence; deterministic; asynchronous on stream.  INVALID_ARG for bad sizes, a ratio
 * outside (0, 1] or null pointers, MISALIGNED for pointers not 4-byte aligned. */
kvc_status kvc_evict_select(const kvc_evict_in* in, uint32_t* keep_mask, void* stream);

/* Inputs of kvc_evict_compact (device memory unless noted). */
typedef struct {
  int32_t B, max_blocks;         /* sequences; width of both block tables (host values)          */
  const int32_t* block_table;    /* [B][max_blocks] pages of the source cache                    */
  const int32_t* seq_len;        /* [B] tokens per source sequence, 0..max_blocks * page_size    */
  const uint32_t* keep_mask;     /* [B][keep_words], as kvc_evict_select writes it               */
  int32_t keep_words;            /* words per sequence of keep_mask (host value, >= 1)           */
  const int32_t* out_block_table;/* [B][max_blocks] pages of the destination cache, distinct      */
} kvc_compact_in;

/* Compaction of the evicted tokens out of a block-shared cache ("BellowsKV" page, "Three Measurements, Three
 * Operators": the one decision is applied to the shared latent, so evicted tokens leave the cache and a decode
 * reads and computes only the kept ones).  Sequence b's kept tokens (bit set, position below seq_len[b]) move, in
 * increasing position, into consecutive slots of the pages out_block_table[b][0..], each with its slot bytes
 * (codes and scale/zero pairs) unchanged.  Slots come in tiles of 32; a tile holds only tokens within 4 blocks of
 * 32 positions of its first token's block: a token starts a new tile when the current one is full or its block
 * is 4 or more past the first token's, and the slots a closed tile leaves over hold no token (zero bytes).
 * Writes out_seq_len[b] (slots up to the last token, at most seq_len[b]), tok_pos[b][0 .. max_blocks *
 * page_size) (source position of each slot, -1 where there is no token: the table kvc_decode_attn takes) and
 * every slot of the destination pages below out_seq_len[b] (other pages are left as they were).  dst->page_off
 * holds the destination record offsets (multiples of 16; the same record layout and size as the source).
 * Decoding the result with tok_pos and the sequence's own q_pos gives the attention over the kept tokens that
 * the keep mask gives on the source cache.  Two launches (a scan per sequence, then a copy per destination
 * page); deterministic; asynchronous on stream.  INVALID_ARG for a per-head layout, null pointers or sizes out
 * of range (max_blocks * page_size above 262144), UNSUPPORTED for a layout the block-shared decode does not
 * serve or one with the residual, MISALIGNED for pointers not 16-byte aligned (keep_mask: 4-byte). */
kvc_status kvc_evict_compact(const kvc_layout* layout, const kvc_cache* src, const kvc_cache* dst,
                             const kvc_compact_in* in, int32_t* out_seq_len, int32_t* tok_pos, void* stream);

/* Flags of kvc_decode_check (or-ed). */
#define KVC_BAD_SEQ_LEN 1  /* a seq_len outside 1..min(max_T, max_blocks * page_size)              */
#define KVC_BAD_PAGE 2     /* a block-table entry of a used block outside 0..n_pages-1              */
#define KVC_BAD_OFFSET 4   /* a used page whose page_off lies outside 0..pool_bytes-1               */
#define KVC_BAD_Q_POS 8    /* a negative q_pos                                                      */
#define KVC_BAD_RANK 16    /* variable rank: a used slot whose rank is not a multiple of 8 in 8..cap */
#define KVC_BAD_TOK_OFF 32 /* variable rank: a used page whose tok_off row is not the exclusive prefix of its
                              tok_rank row (ranks in bits 0-15, ceil(rank / group) in bits 16-31, entry
                              page_size the totals), or one of whose slots holds a rank above the cap     */
#define KVC_BAD_RECORD 64  /* a used page whose record (n_kv_heads head blocks, sized from the page's
                              totals or the uniform rank) starts inside the pool but ends past pool_bytes */
#define KVC_BAD_TOK_POS 128 /* with tok_pos: a 32-slot tile below seq_len whose first slot holds no token
                              while a later one does, or holding a token 4 or more blocks of 32 positions past
                              the first slot's block, or positions not increasing over a sequence's tokens
                              (the decode would skip such a token).  A compacted length of 0 is valid. */

/* Opt-in check of the tables kvc_decode_attn reads and trusts (a bad page id there is undefined behaviour):
 * compares the sequence lengths, the used block-table entries, their page offsets and record ends, q_pos,
 * (variable rank) the used slots' ranks and every offset row of a used page, and (tok_pos) the slot positions
 * with their bounds and with each other, reading nothing through them.  Writes the or of the
 * KVC_BAD_* flags found, 0 if none, to flags (one int32 in device memory).  One workgroup; asynchronous on
 * stream: read flags after synchronizing.  INVALID_ARG for null tables or sizes out of range. */
kvc_status kvc_decode_check(const kvc_layout* layout, const kvc_cache* cache, const kvc_decode_in* in,
                            int32_t* flags, void* stream);

/* Workspace bytes of kvc_dense_decode_attn for these inputs. */
kvc_status kvc_dense_workspace_bytes(const kvc_dense_in* in, size_t* bytes);

/* Plain softmax decode attention over a paged bf16 cache whose keys are already rotated: the
 * dense comparison the JoLT thesis page measures against (FlashJoLT vs a dense bf16 cache).
 * out: fp32 [B][Hq][d]. */
kvc_status kvc_dense_decode_attn(const kvc_dense_in* in, float* out, void* ws, size_t ws_bytes, void* stream);

/* ---- Measurement probes (not on the decode path): measured peaks to set beside the published ones. ---- */

/* Reads `bytes` (a multiple of 16) of device memory at src once, 16 bytes per lane with nontemporal loads, eight in
 * flight per lane, over `grid` workgroups of 256 lanes; sink: [grid] uint32 (the xor of what each workgroup read).
 * Time it with events on `stream`: bytes / time is the HBM read rate a plain stream reaches (use a buffer well
 * beyond the 256 MB last-level cache).  Asynchronous; INVALID_ARG for bad sizes or a pointer not 16-byte aligned. */
kvc_status kvc_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t grid, void* stream);

/* `grid` workgroups of 4 waves, each wave running `iters` rounds of 8 independent v_mfma_f32_32x32x16_f16 on
 * register operands (2 * 32 * 32 * 16 flops each); sink: [grid] floats, normally left unwritten.  Time it with
 * events: the flops over the time is the rate the fp16 matrix instruction of the decode kernels reaches. */
kvc_status kvc_probe_mfma_f16(int32_t iters, int32_t grid, float* sink, void* stream);

/* One wave spins `spins` iterations and writes out[0] = shader clock cycles (s_memtime) and out[1] = ticks of the
 * 100 MHz reference (s_memrealtime) over the spin: out[0] / out[1] * 100 is the shader clock in MHz at that time. */
kvc_status kvc_probe_clock(int32_t spins, uint64_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
