// Gradients of the sparse core attention (qsa_sparse_attn_backward).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works: (B) full
// scaled-dot-product attention restricted to each query's selected tokens,
// (A) the selected blocks expanded to tokens plus the tail.  The pages give
// the forward only; these kernels compute its exact derivative with every
// token set held fixed (no gradient reaches the indexer through the top-k_B
// choice).  Per query i, head h, KV head g = floor(h * Hkv / Hq), token j in
// S_i, with P the forward's softmax (recomputed from its log-sum-exp):
//     dP_j = <dO_h, V_j>,  D_h = sum_j P_j dP_j (= <dO_h, O_h>),
//     dS_j = P_j (dP_j - D_h),
//     dq_h = scale sum_j dS_j K_j,  dK_j += scale dS_j q_h,  dV_j += P_j dO_h.
//
// Two sides, no atomics on the gradients:
//   * query side (one workgroup per query row): D_h, then dq, heads in turn;
//   * key side (one workgroup per 4-token unit of the cache): the unit's K/V
//     rows stay in LDS while the workgroup walks the queries whose token set
//     holds the unit's block -- a transposed index built by counting (per
//     block), scanning and filling -- and adds the unit's dK/dV once.
// The transposed lists are filled with atomics, so the order in which a
// unit sums its queries, and with it the last bits of dK/dV, can change from
// run to run; dq is deterministic.
#include <math.h>

#include "qsa_common.h"
#include "select_common.h"

namespace qsa {
namespace {

constexpr int kBwdMaxTokens = 2048 + 128;   // r * k_B <= 2048 selected, tail <= r
constexpr int kNT = 256;

template <bool BF16>
__device__ __forceinline__ float ldx(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// Token set of query row `row` (positions) into tok[]; returns its size.
__device__ __forceinline__ int token_set(const int32_t* __restrict__ sel,
                                         const int32_t* __restrict__ cnt, int64_t row, int kB,
                                         int64_t p, int lr, int32_t* tok) {
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
  return (count << lr) + ntail;
}

__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = row16_sum_to_last(v);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15)) +
      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31)) +
      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47)) +
      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += red[w];
  __syncthreads();
  return r;
}

// ------------------------------------------------------------- query side --
// One workgroup per query row; heads in turn.  P and dP over the token set
// (in LDS) give D_h exactly, then dS, then dq_h with one thread per dim.
template <bool BF16>
__global__ __launch_bounds__(kNT) void bwd_query_kernel(
    const void* __restrict__ q, const void* __restrict__ kc, const void* __restrict__ vc,
    int64_t cap, int n_q, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, int kB, int Hq, int Hkv, int D, float scale,
    const void* __restrict__ out, const float* __restrict__ lse, const void* __restrict__ dout,
    void* __restrict__ dq, float* __restrict__ dsum, int lr) {
  __shared__ int32_t tok[kBwdMaxTokens];
  __shared__ float ps[kBwdMaxTokens], ds[kBwdMaxTokens];
  __shared__ float qh[128], doh[128];
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int n = token_set(sel, cnt, row, kB, p, lr, tok);
  for (int h = 0; h < Hq; ++h) {
    const int g = (h * Hkv) / Hq;
    const int64_t qo = (row * Hq + h) * D;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      qh[d] = ldx<BF16>(q, qo + d);
      doh[d] = ldx<BF16>(dout, qo + d);
    }
    __syncthreads();
    // P_t from the forward's log-sum-exp, dP_t, and D_h = sum_t P_t dP_t
    // (exact over the token set, not <dO, O> of the rounded output)
    const float lse_h = lse[row * Hq + h];
    float part = 0.0f;
    for (int t = threadIdx.x; t < n; t += blockDim.x) {
      const int64_t ko = (((int64_t)s * cap + tok[t]) * Hkv + g) * D;
      float sd = 0.0f, pd = 0.0f;
      for (int d = 0; d < D; ++d) {
        sd = fmaf(qh[d], ldx<BF16>(kc, ko + d), sd);
        pd = fmaf(doh[d], ldx<BF16>(vc, ko + d), pd);
      }
      const float P = expf(sd * scale - lse_h);
      ps[t] = P;
      ds[t] = pd;
      part = fmaf(P, pd, part);
    }
    const float Dh = block_sum(part, red);  // its barriers also publish ps, ds
    for (int t = threadIdx.x; t < n; t += blockDim.x) ds[t] = ps[t] * (ds[t] - Dh);
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float acc = 0.0f;
      for (int t = 0; t < n; ++t)
        acc = fmaf(ds[t], ldx<BF16>(kc, (((int64_t)s * cap + tok[t]) * Hkv + g) * D + d), acc);
      acc *= scale;
      if constexpr (BF16) static_cast<uint16_t*>(dq)[qo + d] = (uint16_t)f32_to_bf16(acc);
      else static_cast<float*>(dq)[qo + d] = acc;
    }
    if (threadIdx.x == 0) dsum[row * Hq + h] = Dh;
    __syncthreads();
  }
}

// -------------------------------------------------------- transposed index --
struct BwdIndex {
  uint32_t* cnt;   // [batch * nb] queries per block
  uint32_t* cur;   // [batch * nb] fill cursors
  uint32_t* off;   // [batch * nb + 1] exclusive scan of cnt
  uint32_t* list;  // query rows, grouped by block
  int64_t nb;      // blocks per sequence covered (ceil(max_pos_end / r))
};

__global__ __launch_bounds__(kNT) void bwd_clear_kernel(BwdIndex ix, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kNT) {
    ix.cnt[i] = 0u;
    ix.cur[i] = 0u;
  }
}

// Blocks of row `row`'s token set, slot k < count + 1 (the last is the tail
// block); returns -1 past them.
__device__ __forceinline__ int64_t row_block(const int32_t* __restrict__ sel,
                                             const int32_t* __restrict__ cnt, int64_t row,
                                             int kB, int64_t p, int lr, int k) {
  const int64_t c = p >> lr;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  if (k > count) return -1;
  if (k == count) return c;
  return min(max((int64_t)sel[row * kB + k], (int64_t)0), c - 1);
}

template <bool FILL>
__global__ __launch_bounds__(kNT) void bwd_list_kernel(
    BwdIndex ix, int64_t cap, int n_q, const int32_t* __restrict__ q_pos0,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int kB, int lr) {
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  for (int k = threadIdx.x; k <= kB; k += kNT) {
    const int64_t b = row_block(sel, cnt, row, kB, p, lr, k);
    if (b < 0 || b >= ix.nb) continue;
    const int64_t e = (int64_t)s * ix.nb + b;
    if constexpr (FILL) {
      const uint32_t at = atomicAdd(&ix.cur[e], 1u);
      ix.list[ix.off[e] + at] = (uint32_t)row;
    } else {
      atomicAdd(&ix.cnt[e], 1u);
    }
  }
}

// Exclusive scan of the per-block counts (one workgroup; batch * nb entries).
__global__ __launch_bounds__(kNT) void bwd_scan_kernel(BwdIndex ix, int64_t n) {
  __shared__ uint32_t scratch[64];
  uint32_t run = 0;
  constexpr int E = 8;
  for (int64_t base = 0; base < n; base += (int64_t)E * kNT) {
    uint32_t v[E], sum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i = base + (int64_t)threadIdx.x * E + e;
      v[e] = i < n ? ix.cnt[i] : 0u;
      sum += v[e];
    }
    uint32_t tot;
    uint32_t pos = run + block_excl_scan<kNT>(sum, scratch, &tot);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i = base + (int64_t)threadIdx.x * E + e;
      if (i < n) ix.off[i] = pos;
      pos += v[e];
    }
    run += tot;
  }
  if (threadIdx.x == 0) ix.off[n] = run;
}

// --------------------------------------------------------------- key side --
// One workgroup per (sequence, 4-token unit u); its block is u >> (lr - 2).
// The unit's K/V rows (4 tokens x Hkv x D) sit in LDS; each wave takes the
// block's queries in turn.  Per query, lane l computes the score and dP of
// one (head, token) pair (l = 4 h + t, in chunks of 16 heads); P and dS then
// meet the query's q/dO rows with one lane per pair of dims.  The four waves'
// sums meet in LDS and are added to dK/dV once.
template <bool BF16>
__global__ __launch_bounds__(kNT) void bwd_key_kernel(
    BwdIndex ix, const void* __restrict__ q, const void* __restrict__ kc,
    const void* __restrict__ vc, int64_t cap, int n_q, const int32_t* __restrict__ q_pos0,
    int Hq, int Hkv, int D, float scale, const float* __restrict__ lse,
    const void* __restrict__ dout, const float* __restrict__ dsum, float* __restrict__ dk,
    float* __restrict__ dv, int64_t units, int lr) {
  __shared__ float ks[4 * 2 * 128], vs[4 * 2 * 128];   // [t][g][d], Hkv <= 2 staged at once
  __shared__ float acc_k[4][4 * 2 * 128];              // per wave [t][g][d]
  __shared__ float acc_v[4][4 * 2 * 128];
  __shared__ float pw[4][64], dw[4][64];               // per wave: P, dS of the 64 pairs
  const int s = (int)(blockIdx.x / units);
  const int64_t u = blockIdx.x % units;
  const int64_t b = u >> (lr - 2);
  const int64_t e = (int64_t)s * ix.nb + b;
  const uint32_t nq = b < ix.nb ? ix.cnt[e] : 0u;
  if (nq == 0u) return;
  const uint32_t* lst = ix.list + ix.off[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = u * 4;                             // first token of the unit
  const int HD = Hkv * D;
  // stage K/V of the unit's tokens (rows past cap read as 0, never written)
  for (int i = threadIdx.x; i < 4 * HD; i += kNT) {
    const int t = i / HD;
    const int64_t pos = t0 + t;
    ks[i] = pos < cap ? ldx<BF16>(kc, ((int64_t)s * cap + pos) * HD + (i % HD)) : 0.0f;
    vs[i] = pos < cap ? ldx<BF16>(vc, ((int64_t)s * cap + pos) * HD + (i % HD)) : 0.0f;
  }
  for (int i = lane; i < 4 * HD; i += 64) {
    acc_k[wave][i] = 0.0f;
    acc_v[wave][i] = 0.0f;
  }
  __syncthreads();
  const int G = Hq / Hkv;
  for (uint32_t qi = wave; qi < nq; qi += 4) {
    const int64_t row = lst[qi];
    const int rs = (int)(row / n_q);
    const int64_t p = min(max((int64_t)q_pos0[rs] + (int)(row % n_q), (int64_t)0), cap - 1);
    for (int h0 = 0; h0 < Hq; h0 += 16) {
      // ---- pair phase: lane = 4 * (h - h0) + t
      {
        const int h = h0 + (lane >> 2), t = lane & 3;
        float P = 0.0f, dS = 0.0f;
        if (h < Hq) {
          const int g = (h * Hkv) / Hq;
          const int64_t qo = (row * Hq + h) * D;
          float sd = 0.0f, pd = 0.0f;
          for (int d = 0; d < D; ++d) {
            sd = fmaf(ldx<BF16>(q, qo + d), ks[(t * Hkv + g) * D + d], sd);
            pd = fmaf(ldx<BF16>(dout, qo + d), vs[(t * Hkv + g) * D + d], pd);
          }
          if (t0 + t <= p) {   // tokens past the query's position are masked
            P = expf(sd * scale - lse[row * Hq + h]);
            dS = P * (pd - dsum[row * Hq + h]);
          }
        }
        pw[wave][lane] = P;
        dw[wave][lane] = dS;
      }
      wave_sync();
      // ---- accumulate: lane owns dims lane, lane + 64 (D <= 128)
      const int hn = min(16, Hq - h0);
      for (int hh = 0; hh < hn; ++hh) {
        const int h = h0 + hh, g = (h * Hkv) / Hq;
        const int64_t qo = (row * Hq + h) * D;
        for (int d = lane; d < D; d += 64) {
          const float qv = ldx<BF16>(q, qo + d) * scale, ov = ldx<BF16>(dout, qo + d);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc_k[wave][(t * Hkv + g) * D + d] += dw[wave][4 * hh + t] * qv;
            acc_v[wave][(t * Hkv + g) * D + d] += pw[wave][4 * hh + t] * ov;
          }
        }
      }
      wave_sync();
    }
    (void)G;
  }
  __syncthreads();
  // ---- the four waves' sums, added once into dK/dV
  for (int i = threadIdx.x; i < 4 * HD; i += kNT) {
    const int t = i / HD;
    const int64_t pos = t0 + t;
    if (pos >= cap) continue;
    const float sk = acc_k[0][i] + acc_k[1][i] + acc_k[2][i] + acc_k[3][i];
    const float sv = acc_v[0][i] + acc_v[1][i] + acc_v[2][i] + acc_v[3][i];
    const int64_t o = ((int64_t)s * cap + pos) * HD + (i % HD);
    dk[o] += sk;
    dv[o] += sv;
  }
}

struct BwdPlan {
  int64_t nb;
  size_t off_cnt, off_cur, off_off, off_list, off_dsum, bytes;
};

BwdPlan bwd_plan(const Dims& d, int batch, int n_q, int32_t max_pos_end) {
  BwdPlan p{};
  p.nb = ((int64_t)max_pos_end + d.r - 1) >> d.lr;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t rows = (size_t)batch * n_q;
  size_t o = 0;
  p.off_cnt = o;  o = al(o + 4 * (size_t)batch * p.nb);
  p.off_cur = o;  o = al(o + 4 * (size_t)batch * p.nb);
  p.off_off = o;  o = al(o + 4 * ((size_t)batch * p.nb + 1));
  p.off_list = o; o = al(o + 4 * rows * (size_t)(d.kB + 1));
  p.off_dsum = o; o = al(o + 4 * rows * (size_t)d.q_heads);
  p.bytes = o;
  return p;
}

}  // namespace

size_t bwd_workspace_bytes(const Dims& d, int batch, int n_q, int32_t max_pos_end) {
  return bwd_plan(d, batch, n_q, max_pos_end).bytes;
}

hipError_t launch_attn_backward(const Dims& d, int batch, int n_q, const void* q,
                                const void* k_cache, const void* v_cache, int64_t cap,
                                const int32_t* q_pos0, int32_t max_pos_end, const int32_t* sel,
                                const int32_t* cnt, const void* out, const float* lse,
                                const void* dout, void* dq, float* dk, float* dv,
                                void* workspace, hipStream_t st) {
  const BwdPlan pl = bwd_plan(d, batch, n_q, max_pos_end);
  char* ws = static_cast<char*>(workspace);
  BwdIndex ix{reinterpret_cast<uint32_t*>(ws + pl.off_cnt), reinterpret_cast<uint32_t*>(ws + pl.off_cur),
              reinterpret_cast<uint32_t*>(ws + pl.off_off), reinterpret_cast<uint32_t*>(ws + pl.off_list),
              pl.nb};
  float* dsum = reinterpret_cast<float*>(ws + pl.off_dsum);
  const int64_t rows = (int64_t)batch * n_q;
  const int64_t nblk = (int64_t)batch * pl.nb;
  hipLaunchKernelGGL(bwd_clear_kernel, dim3((unsigned)min((nblk + kNT - 1) / kNT, (int64_t)65535)),
                     dim3(kNT), 0, st, ix, nblk);
  hipLaunchKernelGGL((bwd_list_kernel<false>), dim3((unsigned)rows), dim3(kNT), 0, st, ix, cap,
                     n_q, q_pos0, sel, cnt, d.kB, d.lr);
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(kNT), 0, st, ix, nblk);
  hipLaunchKernelGGL((bwd_list_kernel<true>), dim3((unsigned)rows), dim3(kNT), 0, st, ix, cap,
                     n_q, q_pos0, sel, cnt, d.kB, d.lr);
  const int64_t units = (pl.nb << d.lr) / 4;   // 4-token units of the covered blocks
#define QSA_BWD(BF)                                                                            \
  hipLaunchKernelGGL((bwd_query_kernel<BF>), dim3((unsigned)rows), dim3(kNT), 0, st, q, k_cache, \
                     v_cache, cap, n_q, q_pos0, sel, cnt, d.kB, d.q_heads, d.kv_heads,         \
                     d.head_dim, d.scale, out, lse, dout, dq, dsum, d.lr);                     \
  hipLaunchKernelGGL((bwd_key_kernel<BF>), dim3((unsigned)(batch * units)), dim3(kNT), 0, st, ix, \
                     q, k_cache, v_cache, cap, n_q, q_pos0, d.q_heads, d.kv_heads, d.head_dim, \
                     d.scale, lse, dout, dsum, dk, dv, units, d.lr);
  if (d.bf16) {
    QSA_BWD(true)
  } else {
    QSA_BWD(false)
  }
#undef QSA_BWD
  return hipGetLastError();
}

}  // namespace qsa
