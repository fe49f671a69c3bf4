// Sparse core attention (kernel d): prefill (one workgroup per query) and
// decode (a query's token set split over several workgroups, then merged).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works: (B) full
// scaled-dot-product attention restricted to the selected blocks' tokens;
// (A) the selected blocks are expanded back to tokens and the tail of the
// current block is always included.  "Qwen Sparse Attention" gallery page:
// the attention input is every token of the selected blocks plus the visible
// tokens of the current incomplete block.
//
// Token set of the query at p (c = floor(p/4)): pseudo-blocks 0..count-1 are
// the selected blocks, pseudo-block `count` is the tail block c, whose
// tokens 4c+t count only while 4c+t <= p.
//
// MFMA path (16 query heads, Hkv in {1,2}, head_dim in {64,128}, bf16): the
// work item in attn_tile.h, one workgroup per query (prefill) or per split
// of a query's token set (decode); a small second kernel merges the decode
// splits (log-sum-exp).  Other layouts take the generic fp32-arithmetic
// kernel below.
#include <math.h>

#include "attn_tile.h"

namespace qsa {
namespace {

constexpr int kMaxTokens = 2048 + 128;  // r * k_B <= 2048 selected, tail <= r <= 128

// ------------------------------------------------------------- generic ----
template <bool BF16>
__device__ __forceinline__ float ldv(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

__device__ float block_reduce(float v, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float t = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, t) : v + t;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

// One workgroup per query row, heads in sequence; fp32 arithmetic.
template <bool BF16>
__global__ __launch_bounds__(256) void attn_generic_kernel(
    const void* __restrict__ q, const void* __restrict__ kc, const void* __restrict__ vc,
    int64_t cap, int n_q, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, int kB, int Hq, int Hkv, int D, float scale,
    void* __restrict__ out, float* __restrict__ lse, int lr) {
  __shared__ int32_t tok[kMaxTokens];
  __shared__ float wts[kMaxTokens];
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p >> lr;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  for (int i = threadIdx.x; i < (count << lr); i += blockDim.x) {
    int64_t b = sel[row * kB + (i >> lr)];
    b = min(max(b, (int64_t)0), c - 1);
    tok[i] = (int32_t)((b << lr) + (i & ((1 << lr) - 1)));
  }
  const int ntail = (int)(p - (c << lr) + 1);
  for (int i = threadIdx.x; i < ntail; i += blockDim.x)
    tok[(count << lr) + i] = (int32_t)((c << lr) + i);
  const int n = (count << lr) + ntail;
  __syncthreads();
  for (int h = 0; h < Hq; ++h) {
    const int g = (h * Hkv) / Hq;
    const int64_t qo = (row * Hq + h) * D;
    for (int t = threadIdx.x; t < n; t += blockDim.x) {
      const int64_t ko = (((int64_t)s * cap + tok[t]) * Hkv + g) * D;
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(ldv<BF16>(q, qo + d), ldv<BF16>(kc, ko + d), dot);
      wts[t] = dot * scale;
    }
    __syncthreads();
    float m = -INFINITY;
    for (int t = threadIdx.x; t < n; t += blockDim.x) m = fmaxf(m, wts[t]);
    m = block_reduce(m, true, red);
    float z = 0.0f;
    for (int t = threadIdx.x; t < n; t += blockDim.x) {
      const float w = expf(wts[t] - m);
      wts[t] = w;
      z += w;
    }
    z = block_reduce(z, false, red);  // its barriers also publish wts
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float acc = 0.0f;
      for (int t = 0; t < n; ++t)
        acc = fmaf(wts[t], ldv<BF16>(vc, (((int64_t)s * cap + tok[t]) * Hkv + g) * D + d), acc);
      const float o = acc / z;
      if constexpr (BF16) static_cast<uint16_t*>(out)[qo + d] = (uint16_t)f32_to_bf16(o);
      else static_cast<float*>(out)[qo + d] = o;
    }
    if (lse && threadIdx.x == 0) lse[row * Hq + h] = m + logf(z);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- MFMA ----
template <int HKV, int D>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t cap, int n_q, const int32_t* __restrict__ q_pos0,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int kB, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part,
    int n_split, int pb_per_split, int lr) {
  using S = MfmaShape<HKV, D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[S::LDS_BYTES];
  __shared__ int32_t sbid[kMaxPB];
  // Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b % 8):
  // give each XCD one contiguous run of items, so that neighbouring queries,
  // whose selections overlap, share an L2.  A bijection for any grid size.
  int64_t item;
  {
    const uint32_t n = gridDim.x, b = blockIdx.x;
    const uint32_t q = n / 8u, r = n % 8u, x = b % 8u;
    item = (int64_t)(x * q + min(x, r) + b / 8u);
  }
  const int64_t row = item / n_split;
  const int split = (int)(item % n_split);
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p >> lr;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  // 4-token pseudo-blocks: selected block b is m = r/4 of them (b*m .. b*m+m-1),
  // then the tail block c up to the one holding p
  const int lm = lr - 2;
  const int nsel = count << lm;
  const int npb = nsel + (int)((p - (c << lr)) >> 2) + 1;
  const int pb_lo = split * pb_per_split;
  const int pb_hi = min(pb_lo + pb_per_split, npb);
  const int32_t* srow = sel + row * kB;
  for (int i = pb_lo + (int)threadIdx.x; i < pb_hi; i += 256)
    sbid[i - pb_lo] =
        i < nsel ? (int32_t)((min(max((int64_t)srow[i >> lm], (int64_t)0), c - 1) << lm) +
                             (i & ((1 << lm) - 1)))
                 : (int32_t)((c << lm) + (i - nsel));
  u32x4 qb[S::NK];
  load_qbd<HKV, D>(q, row, qb);
  __syncthreads();
  attn_mfma_tiles<HKV, D, false>(qb, kc, vc, cap, s, p, row, item, pb_lo, pb_hi, sbid,
                                 scale_log2, out, lse, part, n_split, lds);
}

// Decode: log-sum-exp merge of a row's split states.  One workgroup per
// (row, head); thread d owns output dim d.  The splits' states were written
// by the previous kernel, so plain loads see them.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ part,
                                                       int n_split, uint16_t* __restrict__ out,
                                                       float* __restrict__ lse) {
  constexpr int PF = part_floats(D);
  const int64_t row = blockIdx.x / 16;
  const int n = (int)(blockIdx.x % 16);
  const int dd = threadIdx.x;
  const float* base = part + row * n_split * PF;
  float m[kMaxSplits], z[kMaxSplits], o[kMaxSplits];
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k) {  // every split's loads in flight at once
    if (k < n_split) {
      const float* pk = base + k * PF;
      m[k] = pk[n];
      z[k] = pk[16 + n];
      o[k] = pk[32 + n * D + dd];
    }
  }
  float mx, zs, acc;
  lse_merge(m, z, o, n_split, mx, zs, acc);
  out[(row * 16 + n) * D + dd] = (uint16_t)f32_to_bf16(acc / zs);
  if (lse && dd == 0) lse[row * 16 + n] = (mx + log2f(zs)) * kLn2;
}


bool use_mfma(const Dims& d) {
  return d.bf16 && d.q_heads == 16 &&
         ((d.kv_heads == 2 && (d.head_dim == 64 || d.head_dim == 128)) ||
          (d.kv_heads == 1 && d.head_dim == 128));
}

// 4-token pseudo-blocks of a largest token set: k_B + 1 blocks of r / 4
int max_pseudo_blocks(const Dims& d) { return (d.kB + 1) << (d.lr - 2); }

int decode_splits(const Dims& d) {
  return (max_pseudo_blocks(d) + kDecodeSplitPB - 1) / kDecodeSplitPB;
}

template <int HKV, int D>
hipError_t launch_mfma(const Dims& d, int rows, int n_q, const void* q, const void* kc,
                       const void* vc, int64_t cap, const int32_t* q_pos0, const int32_t* sel,
                       const int32_t* cnt, void* out, float* lse, void* ws, bool decode,
                       hipStream_t st) {
  const float sl2 = d.scale * kLog2e;
  const int ns = decode ? decode_splits(d) : 1;
  float* part = decode ? static_cast<float*>(ws) : nullptr;
  hipLaunchKernelGGL((attn_mfma_kernel<HKV, D>), dim3((unsigned)(rows * ns)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), cap, n_q, q_pos0, sel, cnt, d.kB, sl2,
                     static_cast<uint16_t*>(out), lse, part, ns,
                     decode ? kDecodeSplitPB : max_pseudo_blocks(d), d.lr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !decode || ns == 1) return e;  // one split wrote the output itself
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)(rows * 16)), dim3(D), 0, st, part,
                     ns, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(const Dims& d, int rows, bool decode) {
  if (!decode || !use_mfma(d)) return 0;
  return sizeof(float) * (size_t)rows * decode_splits(d) * part_floats(d.head_dim);
}

hipError_t launch_attn(const Dims& d, int batch, int n_q, const void* q, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* q_pos0,
                       const int32_t* sel, const int32_t* cnt, void* out, float* lse,
                       void* workspace, bool decode, hipStream_t st) {
  const int rows = batch * n_q;
  if (use_mfma(d)) {
#define QSA_MFMA(HKV, DD)                                                                     \
  if (d.kv_heads == HKV && d.head_dim == DD)                                                 \
    return launch_mfma<HKV, DD>(d, rows, n_q, q, k_cache, v_cache, cap, q_pos0, sel, cnt, out, \
                                lse, workspace, decode, st);
    QSA_MFMA(2, 128)
    QSA_MFMA(1, 128)
    QSA_MFMA(2, 64)
#undef QSA_MFMA
  }
  if (d.bf16)
    hipLaunchKernelGGL(attn_generic_kernel<true>, dim3(rows), dim3(256), 0, st, q, k_cache,
                       v_cache, cap, n_q, q_pos0, sel, cnt, d.kB, d.q_heads, d.kv_heads,
                       d.head_dim, d.scale, out, lse, d.lr);
  else
    hipLaunchKernelGGL(attn_generic_kernel<false>, dim3(rows), dim3(256), 0, st, q, k_cache,
                       v_cache, cap, n_q, q_pos0, sel, cnt, d.kB, d.q_heads, d.kv_heads,
                       d.head_dim, d.scale, out, lse, d.lr);
  return hipGetLastError();
}

}  // namespace qsa
