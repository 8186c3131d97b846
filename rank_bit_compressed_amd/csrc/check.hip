// check.hip -- opt-in check of the tables a decode reads.  The decode kernels trust the block table, the
// sequence lengths, the page offsets, the stored ranks and the offset rows (reading through a bad page id is
// undefined); this kernel compares them with their bounds and with each other without reading the pool.  One workgroup: the tables are
// small (sequences x blocks).
#include <hip/hip_runtime.h>

#include "kvc_common.hpp"

namespace kvc {

namespace {

struct CheckArgs {
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* q_pos;
  const int64_t* page_off;
  const uint8_t* tok_rank;
  const uint32_t* tok_off;
  const int32_t* tok_pos;  // compacted cache: source position of each slot [B][max_blocks * P], -1 for none
  int64_t pool_bytes;
  int64_t record_uniform;  // bytes of a page record when ranks are uniform
  int B, max_blocks, max_T, P, n_pages, r_cap, G, Hkv, d, bits_k, bits_v, residual;
};

// Bytes of a variable-rank page record from its rank and group totals (every head block alike).
__device__ inline int64_t var_record_bytes(const CheckArgs& a, int64_t tot_r, int64_t tot_g) {
  return a.Hkv * head_sections(tot_r * a.bits_k / 8, tot_r * a.bits_v / 8, 4 * tot_g, 4 * tot_g, a.P, a.d, a.residual).hb;
}

__global__ __launch_bounds__(256) void decode_check_kernel(CheckArgs a, int32_t* flags) {
  __shared__ int f;
  if (threadIdx.x == 0) f = 0;
  __syncthreads();
  int my = 0;
  const int limit = min(a.max_T, a.max_blocks * a.P);
  for (int b = 0; b < a.B; ++b) {
    const int T = a.seq_len[b];
    if (threadIdx.x == 0) {
      if (T < (a.tok_pos ? 0 : 1) || T > limit) my |= KVC_BAD_SEQ_LEN;
      if (a.q_pos && a.q_pos[b] < 0) my |= KVC_BAD_Q_POS;
    }
    const int Tc = max(0, min(T, limit));
    for (int j = threadIdx.x; j * a.P < Tc; j += 256) {  // the blocks this sequence uses
      const int page = a.block_table[(size_t)b * a.max_blocks + j];
      if (page < 0 || page >= a.n_pages) {
        my |= KVC_BAD_PAGE;
        continue;
      }
      const int64_t off = a.page_off[page];
      if (off < 0 || off >= a.pool_bytes) my |= KVC_BAD_OFFSET;
      int64_t rec = a.record_uniform;
      if (a.tok_rank) {
        const int used = min(a.P, Tc - j * a.P);
        for (int s = 0; s < used; ++s) {
          const int r = a.tok_rank[(size_t)page * a.P + s];
          if (r < 8 || r > a.r_cap || (r & 7)) my |= KVC_BAD_RANK;
        }
        // the offset row must be the exclusive prefix over every slot of the page (ranks in bits 0-15, groups
        // in bits 16-31), entry P the totals; the decode derives each slot's rank and offsets from it
        const uint8_t* rk = a.tok_rank + (size_t)page * a.P;
        const uint32_t* ro = a.tok_off + (size_t)page * (a.P + 1);
        uint32_t pr = 0, pg = 0;
        bool ok = true;
        for (int s = 0; s < a.P; ++s) {
          const uint32_t r = rk[s];
          ok = ok && r <= (uint32_t)a.r_cap && ro[s] == (pr | (pg << 16));
          pr += r;
          pg += (r + a.G - 1) / a.G;
        }
        ok = ok && ro[a.P] == (pr | (pg << 16));
        if (!ok) my |= KVC_BAD_TOK_OFF;
        rec = var_record_bytes(a, pr, pg);
      }
      if (off >= 0 && off < a.pool_bytes && rec > a.pool_bytes - off) my |= KVC_BAD_RECORD;
    }
    if (a.tok_pos) {  // tiles of 32 slots: the first slot holds a token if any does, every token within 4 blocks
      // of 32 positions of the first's block, tokens increasing (also across the tile before)
      const int32_t* pos = a.tok_pos + (size_t)b * a.max_blocks * a.P;
      for (int i = threadIdx.x; 32 * i < Tc; i += 256) {
        const int end = min(32 * i + 32, Tc);
        int prev = -1;
        for (int s = 32 * i - 1; s >= 0 && s >= 32 * i - 32; --s)  // the last token of the tile before
          if (pos[s] >= 0) {
            prev = pos[s];
            break;
          }
        const int p0 = pos[32 * i];
        for (int s = 32 * i; s < end; ++s) {
          const int p = pos[s];
          if (p < 0) continue;
          if (p0 < 0 || (p >> 5) - (p0 >> 5) >= 4 || p <= prev) my |= KVC_BAD_TOK_POS;
          prev = p;
        }
      }
    }
  }
  atomicOr(&f, my);
  __syncthreads();
  if (threadIdx.x == 0) *flags = f;
}

}  // namespace

kvc_status check_impl(const kvc_layout& L, const kvc_cache& C, const kvc_decode_in& in, int32_t* flags,
                      hipStream_t st) {
  if (!flags || !in.block_table || !in.seq_len || !C.page_off || C.n_pages <= 0 || in.B <= 0 ||
      in.max_blocks <= 0 || in.max_T <= 0 || (L.variable_rank && (!C.tok_rank || !C.tok_off)))
    return KVC_ERR_INVALID_ARG;
  CheckArgs a{in.block_table, in.seq_len, in.q_pos, C.page_off, L.variable_rank ? C.tok_rank : nullptr,
              L.variable_rank ? C.tok_off : nullptr, L.shared ? in.tok_pos : nullptr, C.pool_bytes, uniform_page_bytes(L), in.B, in.max_blocks,
              in.max_T, L.page_size, C.n_pages, L.r_k_cap, L.group, L.n_kv_heads, L.head_dim, lat_bits_k(L),
              lat_bits_v(L), L.residual_bits};
  hipLaunchKernelGGL(decode_check_kernel, dim3(1), dim3(256), 0, st, a, flags);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVC_OK : hip_fail(e);
}

}  // namespace kvc
