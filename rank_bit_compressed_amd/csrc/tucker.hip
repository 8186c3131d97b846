// tucker.hip -- expansion of a partial Tucker core into the up-projections the block-shared decode reads
// (prefill side, once per sequence and layer group).
//
// A layer group's keys (or values) of one sequence, a tensor X[t, i, h, l] over token, feature, head and layer,
// are stored in partial Tucker form: X ~ G x_1 U_t x_2 U_f, the token and feature modes truncated and the head
// and layer modes kept ("JoLT: Near-Lossless KV Cache Compression" thesis page, "How JoLT works"; "A JoLT for
// the KV cache", abstract).  Token t's factor row U_t[t] is then one latent for every head and layer of the
// group, and head h of layer l rebuilds its key from it through W_hl = U_f G[:, :, h, l]^T: the block-shared
// decode with per-sequence up-projections.  This kernel forms them: one workgroup per (sequence, layer, head,
// 64 latent rows) computes a 64 x 128 tile of W[s][l][row0 + c][h d + i] = sum_j U_f[s][i][j] G[s][l][h][c][j]
// in fp32 (fused multiply-adds in increasing j), staged through LDS in chunks of 32 feature coordinates, and
// stores it rounded to bf16 (nearest even), optionally also in fp32.  About 2 d r_f flops per output: never the
// bottleneck (a 4-layer, 8-head group at latent 512 and r_f 64 is 0.27 GFLOP).
#include <hip/hip_runtime.h>

#include "kvc_common.hpp"

namespace kvc {

namespace {

constexpr int TD = 128;  // head dimension
constexpr int TC = 64;   // latent rows per workgroup
constexpr int TJ = 32;   // feature coordinates per LDS chunk

__global__ __launch_bounds__(256) void tucker_expand_kernel(const float* __restrict__ u_f, const float* __restrict__ core,
                                                            uint16_t* __restrict__ w, float* __restrict__ w32, int L,
                                                            int Hkv, int r_t, int r_f, int latent, int row0) {
  __shared__ float us[TD][TJ + 1];  // odd stride: lanes reading a column hit distinct banks
  __shared__ float gs[TC][TJ + 1];
  const int tid = threadIdx.x;
  int id = blockIdx.x;
  const int h = id % Hkv;
  id /= Hkv;
  const int l = id % L;
  const int s = id / L;
  const int c0 = blockIdx.y * TC;
  const float* U = u_f + (size_t)s * TD * r_f;
  const float* G = core + (((size_t)s * L + l) * Hkv + h) * (size_t)r_t * r_f;
  const int i = tid & (TD - 1), cq = tid >> 7;  // this thread: column i, rows cq, cq + 2, ... (one row per wave)
  float acc[TC / 2];
#pragma unroll
  for (int m = 0; m < TC / 2; ++m) acc[m] = 0.0f;
  for (int j0 = 0; j0 < r_f; j0 += TJ) {
    for (int e = tid; e < TD * TJ; e += 256) {
      const int ii = e / TJ, jj = e % TJ;
      us[ii][jj] = j0 + jj < r_f ? U[(size_t)ii * r_f + j0 + jj] : 0.0f;
    }
    for (int e = tid; e < TC * TJ; e += 256) {
      const int cc = e / TJ, jj = e % TJ;
      gs[cc][jj] = (c0 + cc < r_t && j0 + jj < r_f) ? G[(size_t)(c0 + cc) * r_f + j0 + jj] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int jj = 0; jj < TJ; ++jj) {
      const float u = us[i][jj];
#pragma unroll
      for (int m = 0; m < TC / 2; ++m) acc[m] = __builtin_fmaf(u, gs[cq + 2 * m][jj], acc[m]);
    }
    __syncthreads();
  }
  const size_t width = (size_t)Hkv * TD;
#pragma unroll
  for (int m = 0; m < TC / 2; ++m) {
    const int c = c0 + cq + 2 * m;
    if (c >= r_t) continue;
    const size_t o = (((size_t)s * L + l) * latent + row0 + c) * width + (size_t)h * TD + i;
    w[o] = f32_to_bf16_rne(acc[m]);
    if (w32) w32[o] = acc[m];
  }
}

}  // namespace

kvc_status tucker_impl(const kvc_tucker_in& in, uint16_t* w, float* w32, hipStream_t st) {
  if (in.n_seq < 1 || in.n_layers < 1 || in.n_kv_heads < 1 || in.r_t < 1 || in.r_f < 1 || in.row0 < 0 ||
      in.latent < 1 || in.latent > 4096 || (int64_t)in.row0 + in.r_t > in.latent || !in.u_f || !in.core || !w)
    return KVC_ERR_INVALID_ARG;
  if (in.r_f > in.head_dim || in.head_dim < 1) return KVC_ERR_INVALID_ARG;
  if (in.head_dim != TD) return KVC_ERR_UNSUPPORTED;
  const int64_t groups = (int64_t)in.n_seq * in.n_layers * in.n_kv_heads;
  if (groups > (1 << 30)) return KVC_ERR_INVALID_ARG;
  const void* ptrs[] = {in.u_f, in.core, w, w32};
  for (const void* p : ptrs)
    if (p && ((uintptr_t)p & 3)) return KVC_ERR_MISALIGNED;
  const dim3 grid((unsigned)groups, (unsigned)((in.r_t + TC - 1) / TC));
  hipLaunchKernelGGL(tucker_expand_kernel, grid, dim3(256), 0, st, in.u_f, in.core, w, w32, in.n_layers, in.n_kv_heads,
                     in.r_t, in.r_f, in.latent, in.row0);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVC_OK : hip_fail(e);
}

}  // namespace kvc
