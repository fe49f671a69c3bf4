// One wavefront's share of the block compression of the indexer keys.
//
// "QSA (Qwen Sparse Attention)", Key math / How it works, (A): the indexer
// keys of each block of r tokens are average-pooled and RMS-normalised, and
// RoPE is applied to 64 of the 128 dims after compression.  "Qwen Sparse
// Attention" gallery page, How block selection works: only complete blocks
// are pooled, and the rotation uses the first position of each block.
//
// Lane l owns dims 2l and 2l+1 of the 128-dim key, reads its 4 B (bf16) or
// 8 B (fp32) of each of the block's r = 2^lr rows (a row is one coalesced
// 256 B / 512 B wave access), and the sum of squares is a wave reduction.  All
// arithmetic is fp64 -- a few hundred flops per 1 KiB block, HBM-bound -- so
// the stored row is the exact result rounded once.  Rotate-half pairs
// (j, j + rope_dims/2) live in lanes l and l + rope_dims/4 and meet through
// one lane shuffle.
#pragma once

#include "qsa_common.h"

namespace qsa {

// Builds blocks b_first, b_first + stride, ... below b_end of sequence s,
// blocks of r = 2^lr tokens.  Called by all 64 lanes of a wave (the shuffles
// need the whole wave).
template <bool BF16>
__device__ __forceinline__ void compress_wave(const void* __restrict__ k_idx_v, int64_t cap,
                                              int s, int64_t b_first, int64_t b_end,
                                              int64_t stride, const float* __restrict__ gain,
                                              double base, double eps, int rope_dims,
                                              void* __restrict__ k_cmp_v, int lr) {
  const int lane = threadIdx.x & 63;
  const int r = 1 << lr;
  const int64_t cap_blocks = cap >> lr;
  const int d0 = 2 * lane;  // this lane's dims: d0, d0 + 1
  const int half = rope_dims / 2;
  // role: 0 = not rotated, 1 = first member of a pair, 2 = second member
  int role = 0, partner = lane;
  double theta0 = 0.0, theta1 = 0.0;
  if (d0 < half) {
    role = 1;
    partner = lane + rope_dims / 4;
    theta0 = pow(base, -2.0 * (double)d0 / (double)rope_dims);
    theta1 = pow(base, -2.0 * (double)(d0 + 1) / (double)rope_dims);
  } else if (d0 < rope_dims) {
    role = 2;
    partner = lane - rope_dims / 4;
    theta0 = pow(base, -2.0 * (double)(d0 - half) / (double)rope_dims);
    theta1 = pow(base, -2.0 * (double)(d0 + 1 - half) / (double)rope_dims);
  }
  const double g0 = gain ? (double)gain[d0] : 1.0;
  const double g1 = gain ? (double)gain[d0 + 1] : 1.0;

  for (int64_t b = b_first; b < b_end; b += stride) {
    double p0 = 0.0, p1 = 0.0;
    const int64_t row0 = ((int64_t)s * cap + ((int64_t)b << lr)) * 128 + d0;
#pragma unroll 4
    for (int t = 0; t < r; ++t) {
      if constexpr (BF16) {
        const uint32_t w =
            *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(k_idx_v) + row0 + t * 128);
        p0 += (double)bf16_to_f32(w & 0xFFFFu);
        p1 += (double)bf16_to_f32(w >> 16);
      } else {
        const float2 w = *reinterpret_cast<const float2*>(static_cast<const float*>(k_idx_v) + row0 + t * 128);
        p0 += (double)w.x;
        p1 += (double)w.y;
      }
    }
    const double inv_r = 1.0 / (double)r;  // exact: r is a power of two
    p0 *= inv_r;
    p1 *= inv_r;
    double ss = p0 * p0 + p1 * p1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const double rms = sqrt(ss / 128.0 + eps);
    const double n0 = p0 / rms * g0;
    const double n1 = p1 / rms * g1;
    const double o0 = __shfl(n0, partner);
    const double o1 = __shfl(n1, partner);
    double y0 = n0, y1 = n1;
    if (role != 0) {
      const double pos = (double)((int64_t)b << lr);
      double s0, c0, s1, c1;
      sincos(pos * theta0, &s0, &c0);
      sincos(pos * theta1, &s1, &c1);
      if (role == 1) {
        y0 = n0 * c0 - o0 * s0;
        y1 = n1 * c1 - o1 * s1;
      } else {
        y0 = n0 * c0 + o0 * s0;
        y1 = n1 * c1 + o1 * s1;
      }
    }
    const int64_t orow = ((int64_t)s * cap_blocks + b) * 128 + d0;
    if constexpr (BF16) {
      const uint32_t w = f64_to_bf16(y0) | (f64_to_bf16(y1) << 16);
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(k_cmp_v) + orow) = w;
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(k_cmp_v) + orow) = make_float2((float)y0, (float)y1);
    }
  }
}

}  // namespace qsa
