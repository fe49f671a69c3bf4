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
// MFMA path (16 query heads, Hkv in {1,2}, head_dim in {64,128}, bf16):
//   * Work unit: one wave, one tile of 8 pseudo-blocks = 32 tokens.  The 16
//     heads are the 16 MFMA columns; the contraction dim is the KV rows of
//     all Hkv heads concatenated (Hkv*D values, contiguous in the cache), and
//     the query operand is block-diagonal (head h is non-zero only on its
//     own KV head's dims), so one pass serves every GQA group.
//   * S^T = K_tile * Qbd: K rows are gathered from HBM straight into A-operand
//     registers (16 tokens x 64 contiguous bytes per load).  Lane l's result
//     holds 4 consecutive tokens of one pseudo-block for head l%16.
//   * Online softmax per head in the log2 domain.  Masked tokens read a safe
//     row (position p) and get weight 0.
//   * O^T += V_tile^T * P^T: P^T is already in the B-operand layout (each
//     lane's 8 probabilities fill its 8 k-slots, the k<->token map chosen to
//     match).  V rows go from HBM straight into a per-wave LDS tile
//     (global_load_lds_dwordx4, 16-byte chunks XOR-swizzled so four token
//     rows read together fall in distinct banks) and are read transposed,
//     two dims per 4-byte read feeding two MFMAs.  No V staging registers.
//   * Each query's selected-block list is loaded into LDS once, so the K/V
//     addresses of a tile never wait on a dependent global load.
//   * The 4 waves of a workgroup interleave tiles and merge their (m, l, O)
//     states in LDS at the end.
//   * Decode splits a query's token set over workgroups; each writes its
//     merged (m, l, O) state and a small second kernel merges the splits
//     (log-sum-exp) -- a kernel boundary is a far cheaper hand-off here than
//     coherent cross-workgroup stores of 8 KiB states.
#include <math.h>

#include "qsa_common.h"

namespace qsa {
namespace {

constexpr int kMaxTokens = 4 * 512 + 4;

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
    void* __restrict__ out, float* __restrict__ lse) {
  __shared__ int32_t tok[kMaxTokens];
  __shared__ float wts[kMaxTokens];
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p / 4;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  for (int i = threadIdx.x; i < 4 * count; i += blockDim.x) {
    int64_t b = sel[row * kB + i / 4];
    b = min(max(b, (int64_t)0), c - 1);
    tok[i] = (int32_t)(4 * b + (i & 3));
  }
  const int ntail = (int)(p - 4 * c + 1);
  for (int i = threadIdx.x; i < ntail; i += blockDim.x) tok[4 * count + i] = (int32_t)(4 * c + i);
  const int n = 4 * count + ntail;
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
struct MfmaShape {
  static constexpr int HQ = 16;
  static constexpr int G = HQ / HKV;        // query heads per KV head
  static constexpr int KD = HKV * D;        // concatenated KV row (elements)
  static constexpr int NK = KD / 32;        // k-steps of S, dim pairs-of-16 of PV
  static constexpr int ROWB = KD * 2;       // bytes per staged V row
  static constexpr int CH = KD / 8;         // 16-byte chunks per V row
  static constexpr int RPI = 64 / CH;       // V rows per wave-wide load
  static constexpr int TILE_LDS = 32 * ROWB;
  static constexpr int MERGE_FLOATS = 2 * HQ + HQ * D;  // per wave
  static constexpr int LDS_BYTES = (4 * TILE_LDS > 4 * MERGE_FLOATS * 4) ? 4 * TILE_LDS
                                                                          : 4 * MERGE_FLOATS * 4;
  static_assert(CH == 16 || CH == 32, "the V swizzle needs 16 or 32 chunks per row");
};

constexpr int kMaxPB = 4 * 512 / 4 + 1;   // pseudo-blocks of one query (k_B + tail)
constexpr int kMaxSplits = 17;            // decode splits: ceil((k_B + 1) / 32)

// XOR swizzle of a V row's 16-byte chunks: rows 4 apart start their chunks
// at different 64-byte offsets, so the transposed 4-byte reads of one wave
// (four token rows at a time) hit distinct banks.
__device__ __forceinline__ int vswz(int tk) { return 4 * ((tk >> 2) & 3); }

template <int HKV, int D>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t cap, int n_q, const int32_t* __restrict__ q_pos0,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int kB, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part,
    int n_split, int pb_per_split) {
  using S = MfmaShape<HKV, D>;
  constexpr int KD = S::KD, NK = S::NK, ROWB = S::ROWB, G = S::G, CH = S::CH, RPI = S::RPI;
  static_assert(2 * kMaxSplits * 16 * 4 <= S::LDS_BYTES, "decode merge area must fit");
  __shared__ __attribute__((aligned(16))) unsigned char lds[S::LDS_BYTES];
  __shared__ int32_t sbid[kMaxPB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const int64_t item = blockIdx.x;
  const int64_t row = item / n_split;
  const int split = (int)(item % n_split);
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p / 4;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  const int n_pb = count + 1;
  const int pb_lo = split * pb_per_split;
  const int pb_hi = min(pb_lo + pb_per_split, n_pb);
  const uint16_t* kbase = kc + (int64_t)s * cap * KD;
  const uint16_t* vbase = vc + (int64_t)s * cap * KD;

  // block ids of this work item's pseudo-blocks, relative to pb_lo
  {
    const int32_t* srow = sel + row * kB;
    for (int i = pb_lo + (int)threadIdx.x; i < pb_hi; i += 256) {
      int32_t b = (int32_t)c;
      if (i < count) b = (int32_t)min(max((int64_t)srow[i], (int64_t)0), c - 1);
      sbid[i - pb_lo] = b;
    }
  }
  // block id of pseudo-block pb, -1 outside this work item
  auto bid = [&](int pb) -> int64_t { return (pb < pb_hi) ? (int64_t)sbid[pb - pb_lo] : -1; };

  // block-diagonal query operand: head l16 is non-zero on its KV head's dims
  u32x4 qb[NK];
  {
    const int gn = l16 / G;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int dim0 = 32 * kk + 8 * gq;
      const int grp = dim0 / D;
      qb[kk] = (grp == gn) ? ld16(q + (row * 16 + l16) * D + (dim0 - grp * D))
                           : u32x4{0, 0, 0, 0};
    }
  }
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 oacc[NK][2];
#pragma unroll
  for (int pp = 0; pp < NK; ++pp) oacc[pp][0] = oacc[pp][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned char* vt = lds + wave * S::TILE_LDS;

  for (int pb0 = pb_lo + 8 * wave; pb0 < pb_hi; pb0 += 32) {
    // ---- V rows of the tile's 32 tokens: straight from HBM into this wave's
    // LDS tile (lane-ordered 1 KiB per instruction, chunk-swizzled)
#pragma unroll
    for (int u = 0; u < 32 / RPI; ++u) {
      const int tk = RPI * u + lane / CH;
      const int chunk = (lane % CH) ^ vswz(tk);
      const int64_t b = bid(pb0 + (tk >> 2));
      const int64_t tp = 4 * b + (tk & 3);
      const int64_t rp = (b >= 0 && tp <= p) ? tp : p;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(vbase + rp * KD + chunk * 8),
          (__attribute__((address_space(3))) void*)(vt + u * 1024), 16, 0, 0);
    }
    // ---- K rows straight into A-operand registers
    u32x4 kreg[2][NK];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int tk = 16 * st + l16;
      const int64_t b = bid(pb0 + (tk >> 2));
      const int64_t tp = 4 * b + (tk & 3);
      const int64_t rp = (b >= 0 && tp <= p) ? tp : p;
      const uint16_t* kp = kbase + rp * KD + 8 * gq;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) kreg[st][kk] = ld16(kp + 32 * kk);
    }
    // ---- S^T = K * Qbd: lane holds tokens 16st + 4gq + i for head l16
    f32x4 sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kreg[st][kk]),
                                                           as_bf16x8(qb[kk]), sacc[st], 0, 0, 0);
    }
    float x[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int64_t b = bid(pb0 + 4 * st + gq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = b >= 0 && 4 * b + i <= p;
        x[st][i] = ok ? sacc[st][i] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[st][i]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const bool any = m_new != -INFINITY;
    const float alpha = any ? exp2f(m_run - m_new) : 1.0f;
    float pr[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[st][i] = any ? exp2f(x[st][i] - m_new) : 0.0f;
        psum += pr[st][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int pp = 0; pp < NK; ++pp) {
      oacc[pp][0] *= alpha;
      oacc[pp][1] *= alpha;
    }
    u32x4 pv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int st = e >> 1, i0 = 2 * (e & 1);
      pv[e] = f32_to_bf16(pr[st][i0]) | (f32_to_bf16(pr[st][i0 + 1]) << 16);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's V tile has landed in LDS
    wave_sync();
    // ---- O^T += V^T * P^T; k-slot (gq, e) <-> token (e<4 ? 4gq+e : 16+4gq+e-4)
#pragma unroll
    for (int pp = 0; pp < NK; ++pp) {
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tr = (e < 4) ? (4 * gq + e) : (16 + 4 * gq + e - 4);
        const int chunk = (4 * pp + (l16 >> 2)) ^ vswz(tr);
        w[e] = *reinterpret_cast<const uint32_t*>(vt + tr * ROWB + chunk * 16 + 4 * (l16 & 3));
      }
      u32x4 a0, a1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0[e] = (w[2 * e] & 0xFFFFu) | (w[2 * e + 1] << 16);
        a1[e] = (w[2 * e] >> 16) | (w[2 * e + 1] & 0xFFFF0000u);
      }
      oacc[pp][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(pv),
                                                            oacc[pp][0], 0, 0, 0);
      oacc[pp][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(pv),
                                                            oacc[pp][1], 0, 0, 0);
    }
    wave_sync();  // all reads of this tile issued before the next tile's loads
  }

  // ---- merge the four waves' states
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();
  float* mg = reinterpret_cast<float*>(lds);
  float* my = mg + wave * S::MERGE_FLOATS;  // [m 16][l 16][o 16 x D]
  if (gq == 0) {
    my[l16] = m_run;
    my[16 + l16] = l_run;
  }
  {
    const int gn = l16 / G;
#pragma unroll
    for (int pp = 0; pp < NK; ++pp) {
      if (pp / (D / 32) != gn) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rel = 32 * pp + 8 * gq + 2 * i + h - gn * D;
          my[32 + l16 * D + rel] = oacc[pp][h][i];
        }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
    const int n = idx / D, dd = idx % D;
    float mw[4], mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = mg[w * S::MERGE_FLOATS + n];
      mx = fmaxf(mx, mw[w]);
    }
    float z = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (mw[w] == -INFINITY) continue;
      const float f = exp2f(mw[w] - mx);
      z += f * mg[w * S::MERGE_FLOATS + 16 + n];
      o += f * mg[w * S::MERGE_FLOATS + 32 + n * D + dd];
    }
    if (n_split == 1) {
      out[(row * 16 + n) * D + dd] = (uint16_t)f32_to_bf16(o / z);
      if (lse && dd == 0) lse[row * 16 + n] = (mx + log2f(z)) * kLn2;
    } else {
      float* po = part + item * (16 * D + 32);
      po[32 + n * D + dd] = o;
      if (dd == 0) {
        po[n] = mx;
        po[16 + n] = z;
      }
    }
  }
}

// Decode: log-sum-exp merge of a row's split states.  One workgroup per
// (row, head); thread d owns output dim d.  The splits' states were written
// by the previous kernel, so plain loads see them.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ part,
                                                       int n_split, uint16_t* __restrict__ out,
                                                       float* __restrict__ lse) {
  const int64_t row = blockIdx.x / 16;
  const int n = (int)(blockIdx.x % 16);
  const int dd = threadIdx.x;
  const float* base = part + row * n_split * (16 * D + 32);
  float m[kMaxSplits], z[kMaxSplits], o[kMaxSplits];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k) {  // every split's loads in flight at once
    if (k < n_split) {
      const float* pk = base + k * (16 * D + 32);
      m[k] = pk[n];
      z[k] = pk[16 + n];
      o[k] = pk[32 + n * D + dd];
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k)
    if (k < n_split) mx = fmaxf(mx, m[k]);
  float zs = 0.0f, acc = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k) {
    if (k < n_split && m[k] != -INFINITY) {
      const float f = exp2f(m[k] - mx);
      zs += f * z[k];
      acc += f * o[k];
    }
  }
  out[(row * 16 + n) * D + dd] = (uint16_t)f32_to_bf16(acc / zs);
  if (lse && dd == 0) lse[row * 16 + n] = (mx + log2f(zs)) * kLn2;
}

constexpr int kDecodeSplitPB = 32;  // pseudo-blocks per decode work item

bool use_mfma(const Dims& d) {
  return d.bf16 && d.q_heads == 16 &&
         ((d.kv_heads == 2 && (d.head_dim == 64 || d.head_dim == 128)) ||
          (d.kv_heads == 1 && d.head_dim == 128));
}

int decode_splits(const Dims& d) { return (d.kB + 1 + kDecodeSplitPB - 1) / kDecodeSplitPB; }

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
                     decode ? kDecodeSplitPB : d.kB + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !decode) return e;
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)(rows * 16)), dim3(D), 0, st, part,
                     ns, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(const Dims& d, int rows, bool decode) {
  if (!decode || !use_mfma(d)) return 0;
  return sizeof(float) * (size_t)rows * decode_splits(d) * (16 * d.head_dim + 32);
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
                       d.head_dim, d.scale, out, lse);
  else
    hipLaunchKernelGGL(attn_generic_kernel<false>, dim3(rows), dim3(256), 0, st, q, k_cache,
                       v_cache, cap, n_q, q_pos0, sel, cnt, d.kB, d.q_heads, d.kv_heads,
                       d.head_dim, d.scale, out, lse);
  return hipGetLastError();
}

}  // namespace qsa
