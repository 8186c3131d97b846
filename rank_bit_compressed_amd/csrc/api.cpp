// api.cpp -- the C ABI of librbc_kvc.so: argument checks, launch geometry, dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "kvc_common.hpp"

namespace kvc {

static thread_local int32_t g_last_hip_error = 0;
thread_local LaunchMarks g_marks;

kvc_status hip_fail(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return KVC_ERR_HIP;
}

// launchers (defined with their kernels)
bool head_supported(const kvc_layout& L);
int head_part_stride(int rv_cap, int residual);
hipError_t launch_decode_head(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out, void* ws,
                              int n_splits, int pages_per_split, hipStream_t st, bool* unsupported);
int head_max_pages_per_split();
int head_decode_path(const kvc_layout& L);
bool shared_supported(const kvc_layout& L);
int shared_max_tiles_per_split();
size_t shared_ws_bytes(const kvc_layout& L, int B, int n_splits);
hipError_t launch_decode_shared(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, float* out,
                                void* ws, int n_splits, int st_per_split, hipStream_t st);
kvc_status compress_impl(const kvc_layout& L, const kvc_compress_in& in, const kvc_cache& C, hipStream_t st);
kvc_status fit_impl(const kvc_fit_in& in, uint16_t* basis_bf16, float* basis_f32, float* sigma2, void* ws,
                    size_t ws_bytes, hipStream_t st, size_t* bytes_out);
kvc_status salience_impl(const kvc_salience_in& in, float* out, void* ws, size_t ws_bytes, hipStream_t st,
                         size_t* bytes_out);
kvc_status rank_alloc_impl(const kvc_alloc_in& in, uint8_t* ranks, hipStream_t st);
kvc_status plan_impl(const kvc_plan_in& in, int32_t* choice, double* lambda);
kvc_status tucker_impl(const kvc_tucker_in& in, uint16_t* w, float* w32, hipStream_t st);
kvc_status tfit_impl(const kvc_tucker_fit_in& in, float* u_t, float* u_f, float* core, int32_t* info, void* ws,
                     size_t ws_bytes, hipStream_t st, size_t* bytes_out);
kvc_status evict_impl(const kvc_evict_in& in, uint32_t* mask, hipStream_t st);
kvc_status compact_impl(const kvc_layout& L, const kvc_cache& src, const kvc_cache& dst, const kvc_compact_in& in,
                        int32_t* out_len, int32_t* tok_pos, hipStream_t st);
kvc_status check_impl(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, int32_t* flags,
                      hipStream_t st);
kvc_status dense_impl(const kvc_dense_in& in, float* out, void* ws, size_t ws_bytes, hipStream_t st,
                      size_t* need);

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static kvc_status check_layout(const kvc_layout* L) {
  if (!L) return KVC_ERR_INVALID_ARG;
  if (L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->n_q_heads % L->n_kv_heads) return KVC_ERR_INVALID_ARG;
  if (L->head_dim <= 0 || L->head_dim % 2) return KVC_ERR_INVALID_ARG;
  if (L->page_size <= 0 || L->page_size > 256) return KVC_ERR_INVALID_ARG;
  {
    auto qb = [](int b) { return b == 2 || b == 3 || b == 4; };
    const int bk = L->latent_bits, bv = L->latent_bits_v ? L->latent_bits_v : L->latent_bits;
    if (L->latent_bits_v != 0 && !qb(L->latent_bits_v) && L->latent_bits_v != 32) return KVC_ERR_INVALID_ARG;
    if (!(qb(bk) && qb(bv)) && !(bk == 32 && bv == 32)) return KVC_ERR_INVALID_ARG;
  }
  if (L->r_k_cap <= 0 || L->r_v_cap <= 0 || L->r_k_cap % 8 || L->r_v_cap % 8) return KVC_ERR_INVALID_ARG;
  if (L->r_k_cap > 1024 || L->r_v_cap > 1024) return KVC_ERR_INVALID_ARG;
  if (L->latent_bits != 32 && (L->group <= 0 || L->group % 8)) return KVC_ERR_INVALID_ARG;
  if (L->residual_bits != 0 && L->residual_bits != 2) return KVC_ERR_INVALID_ARG;
  if (L->residual_bits && L->head_dim != 128) return KVC_ERR_INVALID_ARG;
  if (L->shared) {
    // one latent for keys and values: one width (4, or the lower-bit codecs 3 and 2)
    if (L->n_layers <= 0 || lat_bits_k(*L) == 32 || lat_bits_v(*L) != lat_bits_k(*L) || L->variable_rank ||
        L->r_k_cap != L->r_v_cap)
      return KVC_ERR_INVALID_ARG;
  } else if (L->n_layers != 1) {
    return KVC_ERR_INVALID_ARG;
  }
  if (L->variable_rank && (L->latent_bits == 32 || lat_bits_v(*L) != L->latent_bits || L->r_k_cap != L->r_v_cap))
    return KVC_ERR_INVALID_ARG;
  if (L->variable_rank && L->page_size * L->r_k_cap > 65535) return KVC_ERR_INVALID_ARG;
  if (!(L->rope_theta >= 0.0) || std::isinf(L->rope_theta)) return KVC_ERR_INVALID_ARG;
  // what the gfx950 kernels implement
  if (L->page_size % 32) return KVC_ERR_UNSUPPORTED;
  if (L->latent_bits != 32 && L->group % 16) return KVC_ERR_UNSUPPORTED;
  if (L->shared ? !shared_supported(*L) : !head_supported(*L)) return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}

// Context splits per (sequence, kv head[, layer]) and the work of one split: pages (per-head mode)
// or 32-token super-tiles (block-shared mode).
static void choose_splits(const kvc_layout& L, int B, int max_T, int requested, int* n_splits, int* per_split) {
  const int unit = L.shared ? 32 : L.page_size;
  const int n_units = (max_T + unit - 1) / unit;
  const int items = B * L.n_kv_heads * (L.shared ? L.n_layers : 1);
  int s = requested;
  if (s <= 0) {
    // workgroups: one per compute unit for the kernels that hold one (block-shared, INT4 residual), else two
    const bool one_per_cu = L.shared || head_decode_path(L) == KVC_PATH_RES;
    const int target = one_per_cu ? 256 : 512;
    s = std::max(1, (target + items - 1) / items);
  }
  s = std::max(1, std::min(s, n_units));
  int per = (n_units + s - 1) / s;
  per = std::min(per, L.shared ? shared_max_tiles_per_split() : head_max_pages_per_split());
  *per_split = per;
  *n_splits = (n_units + per - 1) / per;
}

static size_t decode_ws_bytes(const kvc_layout& L, int B, int n_splits) {
  if (L.shared) return shared_ws_bytes(L, B, n_splits);
  return (size_t)B * L.n_kv_heads * n_splits * 4 * head_part_stride(L.r_v_cap, L.residual_bits) * sizeof(float);
}

}  // namespace kvc

using namespace kvc;

extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_string(int32_t s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARG: return "invalid argument";
    case KVC_ERR_UNSUPPORTED: return "unsupported geometry";
    case KVC_ERR_WORKSPACE: return "workspace or pool too small";
    case KVC_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case KVC_ERR_HIP: return "HIP runtime error";
    case KVC_ERR_SCRATCH: return "decode needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int32_t kvc_last_hip_error(void) { return g_last_hip_error; }

kvc_status kvc_layout_check(const kvc_layout* layout) { return check_layout(layout); }

kvc_status kvc_pool_bytes_max(const kvc_layout* layout, int32_t n_pages, int64_t* bytes) {
  kvc_status s = check_layout(layout);
  if (s == KVC_ERR_INVALID_ARG) return s;
  if (!bytes || n_pages < 0) return KVC_ERR_INVALID_ARG;
  *bytes = uniform_page_bytes(*layout) * (int64_t)n_pages;
  return KVC_OK;
}

kvc_status kvc_decode_workspace_bytes(const kvc_layout* layout, int32_t B, int32_t max_T, int32_t num_splits,
                                      size_t* bytes) {
  kvc_status s = check_layout(layout);
  if (s) return s;
  if (!bytes || B <= 0 || max_T <= 0 || num_splits < 0) return KVC_ERR_INVALID_ARG;
  int ns, sps;
  choose_splits(*layout, B, max_T, num_splits, &ns, &sps);
  *bytes = decode_ws_bytes(*layout, B, ns);
  return KVC_OK;
}

kvc_status kvc_decode_attn(const kvc_layout* layout, const kvc_cache* cache, const kvc_decode_in* in, float* out,
                           void* ws, size_t ws_bytes, void* stream) {
  kvc_status s = check_layout(layout);
  if (s) return s;
  if (!cache || !in || !out || !ws) return KVC_ERR_INVALID_ARG;
  const kvc_layout& L = *layout;
  if (in->B <= 0 || in->max_blocks <= 0 || in->max_T <= 0 || in->num_splits < 0) return KVC_ERR_INVALID_ARG;
  if (in->w_seq_stride < 0 || in->w_seq_stride % 8 || (!L.shared && in->w_seq_stride)) return KVC_ERR_INVALID_ARG;
  if (in->keep_mask && (!L.shared || in->keep_words < 1)) return KVC_ERR_INVALID_ARG;
  if (in->kv_split && (!L.shared || 2 * in->kv_split != L.r_k_cap)) return KVC_ERR_INVALID_ARG;
  if (in->keep_mask && ((uintptr_t)in->keep_mask & 3)) return KVC_ERR_MISALIGNED;
  if (in->tok_pos && (!L.shared || in->keep_mask || !in->q_pos)) return KVC_ERR_INVALID_ARG;
  if (L.shared && L.residual_bits && (in->keep_mask || in->tok_pos)) return KVC_ERR_UNSUPPORTED;
  if (in->tok_pos && ((uintptr_t)in->tok_pos & 3)) return KVC_ERR_MISALIGNED;
  if ((int64_t)in->max_blocks * L.page_size < in->max_T) return KVC_ERR_INVALID_ARG;
  if (in->q_dtype != KVC_F32 && in->q_dtype != KVC_BF16) return KVC_ERR_INVALID_ARG;
  if (!cache->pool || !cache->page_off || cache->n_pages <= 0) return KVC_ERR_INVALID_ARG;
  if (L.variable_rank && (!cache->tok_rank || !cache->tok_off)) return KVC_ERR_INVALID_ARG;
  if (!in->block_table || !in->seq_len || !in->q || !in->wk || !in->wv) return KVC_ERR_INVALID_ARG;
  const void* ptrs[] = {cache->pool, cache->page_off, cache->tok_rank, cache->tok_off, in->block_table, in->seq_len,
                        in->q_pos, in->q, in->wk, in->wv, out, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVC_ERR_MISALIGNED;
  int ns, sps;
  choose_splits(L, in->B, in->max_T, in->num_splits, &ns, &sps);
  if (ws_bytes < decode_ws_bytes(L, in->B, ns)) return KVC_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (L.shared) {
    e = launch_decode_shared(L, *cache, *in, out, ws, ns, sps, st);
  } else {
    bool unsupported = false;
    e = launch_decode_head(L, *cache, *in, out, ws, ns, sps, st, &unsupported);
    if (unsupported) return KVC_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) return hip_fail(e);
  return KVC_OK;
}

kvc_status kvc_decode_attn_timed(const kvc_layout* layout, const kvc_cache* cache, const kvc_decode_in* in,
                                 float* out, void* ws, size_t ws_bytes, void* stream, void* ev_begin, void* ev_end) {
  if (!ev_begin || !ev_end) return KVC_ERR_INVALID_ARG;
  struct Reset {
    ~Reset() { g_marks = LaunchMarks{}; }
  } reset;
  g_marks.begin = (hipEvent_t)ev_begin;
  g_marks.end = (hipEvent_t)ev_end;
  return kvc_decode_attn(layout, cache, in, out, ws, ws_bytes, stream);
}

kvc_status kvc_compress(const kvc_layout* layout, const kvc_compress_in* in, const kvc_cache* cache, void* stream) {
  kvc_status s = check_layout(layout);
  if (s) return s;
  if (!in || !cache) return KVC_ERR_INVALID_ARG;
  return compress_impl(*layout, *in, *cache, (hipStream_t)stream);
}

kvc_status kvc_decode_path(const kvc_layout* layout, int32_t* path) {
  kvc_status s = check_layout(layout);
  if (s) return s;
  if (!path) return KVC_ERR_INVALID_ARG;
  *path = layout->shared ? KVC_PATH_SHARED : head_decode_path(*layout);
  return KVC_OK;
}

kvc_status kvc_fit_workspace_bytes(const kvc_fit_in* in, size_t* bytes) {
  if (!in || !bytes) return KVC_ERR_INVALID_ARG;
  return fit_impl(*in, nullptr, nullptr, nullptr, nullptr, 0, nullptr, bytes);
}

kvc_status kvc_fit_basis(const kvc_fit_in* in, uint16_t* basis_bf16, float* basis_f32, float* sigma2, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!in) return KVC_ERR_INVALID_ARG;
  return fit_impl(*in, basis_bf16, basis_f32, sigma2, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

kvc_status kvc_fit_basis_timed(const kvc_fit_in* in, uint16_t* basis_bf16, float* basis_f32, float* sigma2, void* ws,
                               size_t ws_bytes, void* stream, void* ev_begin, void* ev_end) {
  if (!ev_begin || !ev_end) return KVC_ERR_INVALID_ARG;
  struct Reset {
    ~Reset() { g_marks = LaunchMarks{}; }
  } reset;
  g_marks.begin = (hipEvent_t)ev_begin;
  g_marks.end = (hipEvent_t)ev_end;
  return kvc_fit_basis(in, basis_bf16, basis_f32, sigma2, ws, ws_bytes, stream);
}

kvc_status kvc_salience_workspace_bytes(const kvc_salience_in* in, size_t* bytes) {
  if (!in || !bytes) return KVC_ERR_INVALID_ARG;
  return salience_impl(*in, nullptr, nullptr, 0, nullptr, bytes);
}

kvc_status kvc_salience(const kvc_salience_in* in, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!in) return KVC_ERR_INVALID_ARG;
  return salience_impl(*in, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

kvc_status kvc_rank_alloc(const kvc_alloc_in* in, uint8_t* ranks, void* stream) {
  if (!in) return KVC_ERR_INVALID_ARG;
  return rank_alloc_impl(*in, ranks, (hipStream_t)stream);
}

kvc_status kvc_plan_budget(const kvc_plan_in* in, int32_t* choice, double* lambda) {
  if (!in) return KVC_ERR_INVALID_ARG;
  return plan_impl(*in, choice, lambda);
}

kvc_status kvc_tucker_expand(const kvc_tucker_in* in, uint16_t* w, float* w_f32, void* stream) {
  if (!in) return KVC_ERR_INVALID_ARG;
  return tucker_impl(*in, w, w_f32, (hipStream_t)stream);
}

kvc_status kvc_tucker_fit_workspace_bytes(const kvc_tucker_fit_in* in, size_t* bytes) {
  if (!in || !bytes) return KVC_ERR_INVALID_ARG;
  return tfit_impl(*in, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, bytes);
}

kvc_status kvc_tucker_fit(const kvc_tucker_fit_in* in, float* u_t, float* u_f, float* core, int32_t* info, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!in) return KVC_ERR_INVALID_ARG;
  return tfit_impl(*in, u_t, u_f, core, info, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

kvc_status kvc_evict_select(const kvc_evict_in* in, uint32_t* keep_mask, void* stream) {
  if (!in) return KVC_ERR_INVALID_ARG;
  return evict_impl(*in, keep_mask, (hipStream_t)stream);
}

kvc_status kvc_evict_compact(const kvc_layout* layout, const kvc_cache* src, const kvc_cache* dst,
                             const kvc_compact_in* in, int32_t* out_seq_len, int32_t* tok_pos, void* stream) {
  kvc_status s = check_layout(layout);
  if (s) return s;
  if (!src || !dst || !in) return KVC_ERR_INVALID_ARG;
  return compact_impl(*layout, *src, *dst, *in, out_seq_len, tok_pos, (hipStream_t)stream);
}

kvc_status kvc_decode_check(const kvc_layout* layout, const kvc_cache* cache, const kvc_decode_in* in,
                            int32_t* flags, void* stream) {
  const kvc_status s = check_layout(layout);
  if (s == KVC_ERR_INVALID_ARG) return s;
  if (!cache || !in) return KVC_ERR_INVALID_ARG;
  return check_impl(*layout, *cache, *in, flags, (hipStream_t)stream);
}

kvc_status kvc_dense_workspace_bytes(const kvc_dense_in* in, size_t* bytes) {
  if (!in || !bytes) return KVC_ERR_INVALID_ARG;
  return dense_impl(*in, nullptr, nullptr, 0, nullptr, bytes);
}

kvc_status kvc_dense_decode_attn(const kvc_dense_in* in, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!in || !out) return KVC_ERR_INVALID_ARG;
  return dense_impl(*in, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

}  // extern "C"
