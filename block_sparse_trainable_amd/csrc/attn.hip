// Sparse core attention (kernel d): prefill (one workgroup per query) and
// decode (a query's token set split over several workgroups, then merged).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works: (B) each query
// runs ordinary softmax attention (logits scaled by 1/sqrt(d)), but only over
// the tokens of its chosen blocks; (A) a chosen block contributes all of its
// tokens, and the already visible part of the query's own block is added.
// "Qwen Sparse Attention" gallery page, How block selection works: the same
// token set, as the pseudocode's attention input.
//
// Token set of the query at p (c = floor(p/r)): a selected block b is the
// r/4 pseudo-blocks (4-token units) of its tokens, then come the tail's
// pseudo-blocks up to the one holding p, whose tokens count only while they
// are <= p.  Blocks of r < 4 tokens (down to single tokens, r = 1) take the
// token mode: the set is written out as a list of positions -- the selected
// blocks' tokens, then the tail r*c .. p -- and the tiles read it 32 slots
// at a time.
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
constexpr int kSweep = 64;   // prefill walk: rows per sweep (about the workgroups resident per XCD)
// T16: the 16-token tile walk, three workgroups per CU (prefill of the two-
// 128-dim-KV-head shape, not the token mode); otherwise 32-token tiles, two
// per CU.  Decode splits keep the 32-token walk: the fused decode step
// attends with it and must give the same bits.
template <int HKV, int D, bool TOK, bool T16>
__global__ __launch_bounds__(256, (T16 ? 3 : 2)) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t cap, int n_q, const int32_t* __restrict__ q_pos0,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int kB, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part,
    int n_split, int pb_per_split, int lr, const int32_t* __restrict__ order,
    const int32_t* __restrict__ first) {
  using S = MfmaShape<HKV, D>;
  static_assert(!T16 || (!TOK && HKV == 2 && D == 128), "16-token walk: two 128-dim KV heads");
  __shared__ __attribute__((aligned(16))) unsigned char lds[T16 ? S::LDS16_BYTES : S::LDS_BYTES];
  __shared__ int32_t sbid[TOK ? kMaxTok : kMaxPB];
  // the 16-token walk reads its query operand from LDS
  __shared__ u32x4 qlds[T16 ? S::NK * 64 : 1];
  // Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b % 8):
  // give each XCD one contiguous run of items, so that the queries it holds
  // at once, whose selections overlap, share an L2.  A bijection for any
  // grid size.
  int64_t item;
  {
    const uint32_t n = gridDim.x, b = blockIdx.x;
    const uint32_t q = n / 8u, r = n % 8u, x = b % 8u;
    item = (int64_t)(x * q + min(x, r) + b / 8u);
  }
  int64_t row = item / n_split;
  const int split = (int)(item % n_split);
  // prefill with a row order (one split per row): item i attends row
  // order[i], so rows that read the same region of the cache run together
  if (order) row = min(max((int64_t)order[item], (int64_t)0), (int64_t)gridDim.x - 1);
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p >> lr;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  const int32_t* srow = sel + row * kB;
  u32x4 qb[S::NK];
  if constexpr (TOK) {
    // the token list: count*r selected tokens, then the tail r*c .. p
    const int nsel = count << lr;
    const int ntok = nsel + (int)(p - (c << lr)) + 1;
    const int pb_lo = split * pb_per_split;
    const int pb_hi = min(pb_lo + pb_per_split, (ntok + 3) >> 2);
    const int t_lo = 4 * pb_lo, t_hi = min(4 * pb_hi, ntok);
    // One split per row (prefill): a row whose selection clusters in one
    // region lists its tokens from the first one of that region on, and
    // wraps (see the pseudo-block walk below); the others from the start.
    int rot = 0;
    if (n_split == 1 && first) {
      const int f = first[row];
      if (f >= 0) rot = min(f << lr, ntok - 1);
    }
    for (int k = t_lo + (int)threadIdx.x; k < t_hi; k += 256) {
      int i = k + rot;
      i -= i >= ntok ? ntok : 0;
      sbid[k - t_lo] =
          i < nsel ? (int32_t)((min(max((int64_t)srow[i >> lr], (int64_t)0), c - 1) << lr) +
                               (i & ((1 << lr) - 1)))
                   : (int32_t)((c << lr) + (i - nsel));
    }
    load_qbd<HKV, D>(q, row, qb);
    __syncthreads();
    attn_mfma_tiles<HKV, D, false, true>(qb, kc, vc, cap, s, p, row, item, pb_lo, pb_hi, sbid,
                                         scale_log2, out, lse, part, n_split, lds, t_hi);
  } else {
    // 4-token pseudo-blocks: selected block b is m = r/4 of them
    // (b*m .. b*m+m-1), then the tail block c up to the one holding p
    const int lm = lr - 2;
    const int nsel = count << lm;
    const int npb = nsel + (int)((p - (c << lr)) >> 2) + 1;
    const int pb_lo = split * pb_per_split;
    const int pb_hi = min(pb_lo + pb_per_split, npb);
    for (int i = pb_lo + (int)threadIdx.x; i < pb_hi; i += 256)
      sbid[i - pb_lo] =
          i < nsel ? (int32_t)((min(max((int64_t)srow[i >> lm], (int64_t)0), c - 1) << lm) +
                               (i & ((1 << lm) - 1)))
                   : (int32_t)((c << lm) + (i - nsel));
    load_qbd<HKV, D>(q, row, qb);
    if (T16 && threadIdx.x < 64) {
#pragma unroll
      for (int kk = 0; kk < S::NK; ++kk) qlds[kk * 64 + threadIdx.x] = qb[kk];
    }
    __syncthreads();
    // One split per row (prefill): the walk starts rot entries into the
    // list and wraps.  A row whose selection clusters in one region starts
    // at that region's first block: it runs among rows of the same region
    // (see the row order below), which read the region while it is in
    // their XCD's L2.  Any other row runs among its neighbours in position,
    // which start at staggered times, so it starts a fraction
    // (p mod kSweep) / kSweep into its list: rows in flight together are
    // then at the same fraction of their lists, where neighbouring rows'
    // shared blocks sit.  The row's own selection and position fix the
    // start, so a query gives the same bits in any call.
    constexpr int SW = T16 ? 3 * kSweep / 2 : kSweep;   // resident rows per XCD
    int rot = n_split == 1 ? (int)((p % SW) * npb / SW) : 0;
    if (first) {
      const int f = first[row];
      if (f >= 0) rot = min(f << lm, npb - 1);
    }
    if constexpr (T16)
      attn_mfma_tiles16<HKV, D>(qlds, kc, vc, cap, s, p, row, item, pb_lo, pb_hi, sbid,
                                scale_log2, out, lse, part, n_split, lds, rot);
    else
      attn_mfma_tiles<HKV, D, false>(qb, kc, vc, cap, s, p, row, item, pb_lo, pb_hi, sbid,
                                     scale_log2, out, lse, part, n_split, lds, 0, rot);
  }
}

// Decode: log-sum-exp merge of a row's split states.  One workgroup per
// (row, head); thread d owns output dim d.  The splits' states were written
// by the previous kernel, so plain loads see them.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ part,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ lse) {
  constexpr int PF = part_floats(D);
  __shared__ float ml[2 * kDecodeSplits];
  const int64_t row = blockIdx.x / 16;
  const int n = (int)(blockIdx.x % 16);
  const int dd = threadIdx.x;
  const float* base = part + row * kDecodeSplits * PF;
  for (int i = dd; i < 2 * kDecodeSplits; i += D) ml[i] = base[(i >> 1) * PF + 16 * (i & 1) + n];
  float o[kDecodeSplits];
#pragma unroll
  for (int k = 0; k < kDecodeSplits; ++k) o[k] = base[k * PF + 32 + n * D + dd];  // all in flight
  __syncthreads();
  float mx, zs, acc;
  lse_merge_splits(ml, o, mx, zs, acc);
  out[(row * 16 + n) * D + dd] = (uint16_t)f32_to_bf16(acc / zs);
  if (lse && dd == 0) lse[row * 16 + n] = (mx + log2f(zs)) * kLn2;
}


// ---------------------------------------------------------- row order ----
// Prefill rows are independent, so the order in which the attention runs
// them is free; what the L2 of an XCD can catch depends on it.  Where a
// query's selected blocks cluster in one region of the cache, rows are
// grouped by that region: the rows of a group then run together on one XCD
// and read the region's K/V rows while they are in its L2.  A region is
// 1,024 tokens (1 MB of K and V at 2 x 128 bf16 dims, a quarter of an XCD's
// L2); a row's regions are binned modulo kOrderBins (256 regions span 256K
// tokens).  A row counts as clustered when its most frequent region holds at
// least 1/8 of its selected blocks and at least 4 times the share an even
// spread over its candidates would give it; the other rows keep their
// natural order, after the clustered ones, where neighbouring positions
// share their candidate ranges.  The order changes no result: every row
// computes the same bits wherever it runs.
constexpr int kOrderRegionShift = 10;  // log2 tokens per region
constexpr int kOrderBins = 256;        // region bins of one row's histogram
constexpr int kOrderKeys = 8192;       // sort keys: batch x bins per sequence
constexpr int kOrderMinRows = 1024;    // smaller calls keep the natural order

int order_bins_per_seq(int batch) {
  const int nb = kOrderKeys / batch < kOrderBins ? kOrderKeys / batch : kOrderBins;
  return nb > 0 ? nb : 1;
}

// One wave per row: key[row] = s * nb + (the row's most frequent region bin
// mod nb, the lower bin on ties) and first[row] = the index of its first
// selected block in that bin for a clustered row; -1 and -1 otherwise.
__global__ __launch_bounds__(256) void attn_order_key_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ q_pos0, int n_q, int rows, int64_t cap, int kB, int lr, int nb,
    int32_t* __restrict__ key, int32_t* __restrict__ first) {
  __shared__ uint32_t h[4][kOrderBins];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  const bool live = row < rows;
  for (int i = lane; i < kOrderBins; i += 64) h[wave][i] = 0u;
  __syncthreads();
  int s = 0, count = 0;
  int64_t c = 0;
  const int32_t* srow = sel + (int64_t)(live ? row : 0) * kB;
  if (live) {
    s = row / n_q;
    const int64_t p = min(max((int64_t)q_pos0[s] + row % n_q, (int64_t)0), cap - 1);
    c = p >> lr;
    count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
    // lane l counts entries [l*E, l*E + E) in runs of equal bins: an
    // ascending list has few runs, so few (contended) LDS atomics
    const int E = (count + 63) >> 6;
    const int i1 = min(count, (lane + 1) * E);
    int cur = 0;
    uint32_t run = 0u;
    for (int i = lane * E; i < i1; ++i) {
      const int64_t b = min(max((int64_t)srow[i], (int64_t)0), c - 1);
      const int bin = (int)(((b << lr) >> kOrderRegionShift) & (kOrderBins - 1));
      if (bin != cur) {
        if (run) atomicAdd(&h[wave][cur], run);
        cur = bin;
        run = 0u;
      }
      ++run;
    }
    if (run) atomicAdd(&h[wave][cur], run);
  }
  __syncthreads();
  // (count << 16) | (0xFFFF - bin): the largest is the most frequent bin,
  // the lower one on ties (counts stay below 2^16)
  uint32_t best = 0u;
  for (int i = lane; i < kOrderBins; i += 64)
    best = max(best, (h[wave][i] << 16) | (uint32_t)(0xFFFF - i));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) best = max(best, (uint32_t)__shfl_xor((int)best, off));
  const int64_t top = best >> 16;
  const int bin = (int)(0xFFFF - (best & 0xFFFFu));
  // top / count >= 1/8 and >= 4 * (region blocks) / c
  const int64_t region_blocks = (int64_t)1 << (kOrderRegionShift - lr);
  const bool clustered = count > 0 && 8 * top >= count && top * c >= 4 * region_blocks * count;
  // the first list entry in the top bin (a clustered row only; the test is
  // uniform over the wave)
  int f = 0x7FFFFFFF;
  if (clustered) {
    for (int i = lane; i < count; i += 64) {
      const int64_t b = min(max((int64_t)srow[i], (int64_t)0), c - 1);
      if ((int)(((b << lr) >> kOrderRegionShift) & (kOrderBins - 1)) == bin) f = min(f, i);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) f = min(f, __shfl_xor(f, off));
  }
  if (live && lane == 0) {
    key[row] = clustered ? s * nb + bin % nb : -1;
    first[row] = clustered && f < count ? f : -1;
  }
}

// One workgroup: order[] becomes a permutation of 0 .. rows-1 -- the
// clustered rows by key (keys < nkeys <= kOrderKeys; rows of one key in any
// order among themselves), then the others in their natural order.
__global__ __launch_bounds__(1024) void attn_order_sort_kernel(const int32_t* __restrict__ key,
                                                               int rows, int nkeys,
                                                               int32_t* __restrict__ order) {
  __shared__ uint32_t h[kOrderKeys];
  __shared__ uint32_t part[1024 / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < kOrderKeys; i += 1024) h[i] = 0u;
  __syncthreads();
  for (int r = t; r < rows; r += 1024) {
    const int k = key[r];
    if (k >= 0) atomicAdd(&h[min(k, nkeys - 1)], 1u);
  }
  __syncthreads();
  // exclusive scan: thread t owns keys 8t .. 8t+7
  constexpr int PER = kOrderKeys / 1024;
  uint32_t v[PER], sum = 0u;
#pragma unroll
  for (int k = 0; k < PER; ++k) { v[k] = h[PER * t + k]; sum += v[k]; }
  uint32_t inc = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) part[wave] = inc;
  __syncthreads();
  uint32_t base = 0u, clustered = 0u;
  for (int w = 0; w < 1024 / 64; ++w) {
    base += w < wave ? part[w] : 0u;
    clustered += part[w];
  }
  uint32_t run = base + inc - sum;
#pragma unroll
  for (int k = 0; k < PER; ++k) { h[PER * t + k] = run; run += v[k]; }
  __syncthreads();
  for (int r = t; r < rows; r += 1024) {
    const int k = key[r];
    if (k >= 0) {
      const uint32_t pos = atomicAdd(&h[min(k, nkeys - 1)], 1u);
      if (pos < (uint32_t)rows) order[pos] = r;
    }
  }
  // the other rows, in order: with no clustered row that is the identity;
  // otherwise 1,024 rows per round, ranked by ballots
  if (clustered == 0u) {
    for (int r = t; r < rows; r += 1024) order[r] = r;
    return;
  }
  uint32_t done = clustered;
  for (int r0 = 0; r0 < rows; r0 += 1024) {
    const int r = r0 + t;
    const bool other = r < rows && key[r] < 0;
    const uint64_t m = __ballot(other);
    __syncthreads();  // the previous round's part[] reads are over
    if (lane == 0) part[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0u, total = 0u;
    for (int w = 0; w < 1024 / 64; ++w) {
      before += w < wave ? part[w] : 0u;
      total += part[w];
    }
    const uint32_t pos = done + before + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (other && pos < (uint32_t)rows) order[pos] = r;
    done += total;
  }
}

bool use_mfma(const Dims& d) {
  return d.bf16 && d.q_heads == 16 &&
         ((d.kv_heads == 2 && (d.head_dim == 64 || d.head_dim == 128)) ||
          (d.kv_heads == 1 && d.head_dim == 128));
}

// 4-token pseudo-blocks (token-list slots of 4 in token mode) of a largest
// token set: k_B + 1 blocks of r tokens
int max_pseudo_blocks(const Dims& d) {
  return d.lr >= 2 ? (d.kB + 1) << (d.lr - 2) : (((d.kB + 1) << d.lr) + 3) / 4;
}

int decode_splits(const Dims&) { return kDecodeSplits; }

// Prefill calls on the MFMA path take a walk start per row from the key
// pass, and with enough rows a row order (batch <= 1024 leaves at least 8
// region bins per sequence).  Single-token blocks (r = 1) take neither: on
// the 2 x 8K chunk over 128K their attention measured 4.10 ms in natural
// order from each list's start and 4.70 ms grouped by region.
bool use_keys(const Dims& d, bool decode) { return !decode && d.lr >= 1 && use_mfma(d); }

bool use_order(const Dims& d, int batch, int rows, bool decode) {
  return use_keys(d, decode) && rows >= kOrderMinRows && batch <= kOrderKeys / 8;
}

// Workspace of a prefill call on the MFMA path: key [rows], first [rows],
// and order [rows] when it orders its rows.
size_t order_bytes(int rows, bool sorted) {
  return (sorted ? 3 : 2) * sizeof(int32_t) * (size_t)rows;
}

template <int HKV, int D>
hipError_t launch_mfma(const Dims& d, int batch, int n_q, const void* q, const void* kc,
                       const void* vc, int64_t cap, const int32_t* q_pos0, const int32_t* sel,
                       const int32_t* cnt, void* out, float* lse, void* ws, bool decode,
                       hipStream_t st) {
  const int rows = batch * n_q;
  const float sl2 = d.scale * kLog2e;
  const int ns = decode ? decode_splits(d) : 1;
  float* part = decode ? static_cast<float*>(ws) : nullptr;
  const int32_t* order = nullptr;
  const int32_t* first = nullptr;
  if (use_keys(d, decode)) {
    int32_t* key = static_cast<int32_t*>(ws);
    int32_t* fst = key + rows;
    int32_t* ord = use_order(d, batch, rows, decode) ? fst + rows : nullptr;
    const hipError_t e = launch_row_order(d, batch, n_q, q_pos0, cap, sel, cnt, key, fst, ord, st);
    if (e != hipSuccess) return e;
    first = fst;
    order = ord;
  }
  const dim3 grid((unsigned)(rows * ns));
  constexpr bool kT16 = HKV == 2 && D == 128;
  if (d.lr >= 2 && !decode && kT16)
    hipLaunchKernelGGL((attn_mfma_kernel<HKV, D, false, kT16>), grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                       static_cast<const uint16_t*>(vc), cap, n_q, q_pos0, sel, cnt, d.kB, sl2,
                       static_cast<uint16_t*>(out), lse, part, ns, max_pseudo_blocks(d), d.lr,
                       order, first);
  else if (d.lr < 2)
    hipLaunchKernelGGL((attn_mfma_kernel<HKV, D, true, false>), grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                       static_cast<const uint16_t*>(vc), cap, n_q, q_pos0, sel, cnt, d.kB, sl2,
                       static_cast<uint16_t*>(out), lse, part, ns,
                       decode ? decode_pb_per_split(max_pseudo_blocks(d)) : max_pseudo_blocks(d), d.lr,
                       order, first);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<HKV, D, false, false>), grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                       static_cast<const uint16_t*>(vc), cap, n_q, q_pos0, sel, cnt, d.kB, sl2,
                       static_cast<uint16_t*>(out), lse, part, ns,
                       decode ? decode_pb_per_split(max_pseudo_blocks(d)) : max_pseudo_blocks(d), d.lr,
                       order, first);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !decode) return e;
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)(rows * 16)), dim3(D), 0, st, part,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace

bool row_order_sorts(const Dims& d, int batch, int n_q) {
  return use_order(d, batch, batch * n_q, false);
}

hipError_t launch_row_order(const Dims& d, int batch, int n_q, const int32_t* q_pos0,
                            int64_t cap, const int32_t* sel, const int32_t* cnt, int32_t* key,
                            int32_t* first, int32_t* order, hipStream_t st) {
  const int rows = batch * n_q;
  const int nb = order_bins_per_seq(batch);
  hipLaunchKernelGGL(attn_order_key_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                     sel, cnt, q_pos0, n_q, rows, cap, d.kB, d.lr, nb, key, first);
  if (order)
    hipLaunchKernelGGL(attn_order_sort_kernel, dim3(1), dim3(1024), 0, st, key, rows,
                       batch * nb, order);
  return hipGetLastError();
}

size_t attn_workspace_bytes(const Dims& d, int batch, int n_q, bool decode) {
  const int rows = batch * n_q;
  if (!use_mfma(d)) return 0;
  if (!decode) return use_keys(d, decode) ? order_bytes(rows, use_order(d, batch, rows, decode)) : 0;
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
    return launch_mfma<HKV, DD>(d, batch, n_q, q, k_cache, v_cache, cap, q_pos0, sel, cnt, out, \
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
