// Block compression of the indexer keys (kernel a).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works, (A): the indexer
// keys of each block of r tokens are average-pooled and RMS-normalised, and
// RoPE is applied to 64 of the 128 dims after compression.  "Qwen Sparse
// Attention" gallery page, How block selection works: only complete blocks
// are pooled, and the rotation uses the first position of each block.
//
// Launcher: one wavefront per block (the per-wave arithmetic, fp64, is
// compress_wave in compress_block.h); 4 waves per workgroup, a grid-stride
// loop past 65535 workgroups.
#include "compress_block.h"

namespace qsa {
namespace {

constexpr int kWaves = 4;

template <bool BF16>
__global__ __launch_bounds__(256) void compress_kernel(
    const void* __restrict__ k_idx_v, int64_t cap, const int32_t* __restrict__ len_before,
    const int32_t* __restrict__ len_after, const float* __restrict__ gain, double base,
    double eps, int rope_dims, void* __restrict__ k_cmp_v, int lr) {
  const int s = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int64_t cap_blocks = cap >> lr;
  const int64_t lb = max(len_before[s], 0);
  const int64_t la = min((int64_t)max(len_after[s], 0), cap);
  const int64_t b_begin = lb >> lr;
  const int64_t b_end = min(la >> lr, cap_blocks);
  if (b_begin + (int64_t)blockIdx.x * kWaves >= b_end) return;  // nothing to build here
  compress_wave<BF16>(k_idx_v, cap, s, b_begin + (int64_t)blockIdx.x * kWaves + wave, b_end,
                      (int64_t)gridDim.x * kWaves, gain, base, eps, rope_dims, k_cmp_v, lr);
}

}  // namespace

hipError_t launch_compress(const Dims& d, int batch, const void* k_idx, int64_t cap,
                           const int32_t* len_before, const int32_t* len_after,
                           int max_new_blocks, const float* gain, void* k_cmp,
                           hipStream_t st) {
  if (max_new_blocks <= 0) return hipSuccess;
  int64_t gx = (max_new_blocks + kWaves - 1) / kWaves;
  if (gx > 65535) gx = 65535;  // grid-stride loop covers the rest
  dim3 grid((unsigned)gx, (unsigned)batch);
  if (d.bf16)
    hipLaunchKernelGGL(compress_kernel<true>, grid, dim3(256), 0, st, k_idx, cap, len_before,
                       len_after, gain, d.base, (double)d.eps, d.rope_dims, k_cmp, d.lr);
  else
    hipLaunchKernelGGL(compress_kernel<false>, grid, dim3(256), 0, st, k_idx, cap, len_before,
                       len_after, gain, d.base, (double)d.eps, d.rope_dims, k_cmp, d.lr);
  return hipGetLastError();
}

}  // namespace qsa
