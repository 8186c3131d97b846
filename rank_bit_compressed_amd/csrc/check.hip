// check.hip -- opt-in check of the tables a decode reads.  The decode kernels trust the block table, the
// sequence lengths, the page offsets and the stored ranks (reading through a bad page id is undefined); this
// kernel compares them with their bounds without reading anything through them.  One workgroup: the tables are
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
  int64_t pool_bytes;
  int B, max_blocks, max_T, P, n_pages, r_cap;
};

__global__ __launch_bounds__(256) void decode_check_kernel(CheckArgs a, int32_t* flags) {
  __shared__ int f;
  if (threadIdx.x == 0) f = 0;
  __syncthreads();
  int my = 0;
  const int limit = min(a.max_T, a.max_blocks * a.P);
  for (int b = 0; b < a.B; ++b) {
    const int T = a.seq_len[b];
    if (threadIdx.x == 0) {
      if (T < 1 || T > limit) my |= KVC_BAD_SEQ_LEN;
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
      if (a.tok_rank) {
        const int used = min(a.P, Tc - j * a.P);
        for (int s = 0; s < used; ++s) {
          const int r = a.tok_rank[(size_t)page * a.P + s];
          if (r < 8 || r > a.r_cap || (r & 7)) my |= KVC_BAD_RANK;
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
      in.max_blocks <= 0 || in.max_T <= 0 || (L.variable_rank && !C.tok_rank))
    return KVC_ERR_INVALID_ARG;
  CheckArgs a{in.block_table, in.seq_len, in.q_pos, C.page_off, L.variable_rank ? C.tok_rank : nullptr,
              C.pool_bytes, in.B, in.max_blocks, in.max_T, L.page_size, C.n_pages, L.r_k_cap};
  hipLaunchKernelGGL(decode_check_kernel, dim3(1), dim3(256), 0, st, a, flags);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVC_OK : hip_fail(e);
}

}  // namespace kvc
