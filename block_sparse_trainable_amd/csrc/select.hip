// Top-k_B block selection (kernel c).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works, (A): keep the
// k_B = ceil(K/r) highest-scoring blocks (at most 512 with K = 2048, r = 4,
// per the "Config" line and the gallery page's budget table).  Equal scores
// go to the lower block index, and the kept ids are written in ascending
// order, so the result is unique.
//
// One workgroup per query row.  Scores are ReLU sums, hence >= +0.0, so
// their IEEE bit patterns order like unsigned integers.  An MSB-first radix
// select (digits of 11, 11 and 9 bits over bits 30..0, LDS histograms) finds
// the k_B-th largest key exactly, stopping early once the keys sharing the
// current prefix are exactly the ones still needed.  A second sweep then
// walks the row in index order and keeps every key above the threshold plus
// the first `need` keys equal to it; a workgroup prefix scan gives each kept
// block its output slot, so the output is ascending with no sort.  Rows that
// fit (<= 36,864 scores) are read from HBM once into LDS; longer rows are
// swept from global memory (L2-resident) on every pass.
#include "qsa_common.h"

namespace qsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kScratch = 64;
constexpr int64_t kCacheMax = 36864;

__device__ __forceinline__ uint32_t key_of(uint32_t bits) {
  return (bits & 0x80000000u) ? 0u : bits;  // scores are >= 0; guard anyway
}

// Exclusive prefix sum over the workgroup in thread order; returns the
// exclusive value, total in *total.  Contains two barriers.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = scratch[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

template <bool CACHE>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ scores, int64_t W, int n_q, const int32_t* __restrict__ q_pos0,
    int64_t cap_blocks, int kB, int32_t* __restrict__ sel, int32_t* __restrict__ cnt,
    float* __restrict__ sel_scores) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;
  uint32_t* scratch = smem + kBins;
  uint32_t* rowc = smem + kBins + kScratch;

  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = max((int64_t)q_pos0[s] + j, (int64_t)0);
  const int64_t c = min(p / 4, min(cap_blocks, W));
  const float* src = scores + row * W;
  const uint32_t* src_bits = reinterpret_cast<const uint32_t*>(src);
  int32_t* out = sel + row * kB;
  float* outs = sel_scores ? sel_scores + row * kB : nullptr;
  const int tid = threadIdx.x;

  if (c <= kB) {  // every candidate is kept
    for (int i = tid; i < kB; i += kThreads) {
      out[i] = i < c ? i : -1;
      if (outs) outs[i] = i < c ? src[i] : 0.0f;
    }
    if (tid == 0) cnt[row] = (int32_t)c;
    return;
  }

  if constexpr (CACHE) {
    for (int64_t i = 4 * tid; i < c; i += 4 * kThreads) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src_bits + i);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < c) rowc[i + e] = key_of(v[e]);
    }
    __syncthreads();
  }
  auto key4 = [&](int64_t i) -> u32x4 {  // keys i..i+3 (i % 4 == 0, i < c)
    if constexpr (CACHE) {
      return *reinterpret_cast<const u32x4*>(rowc + i);
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src_bits + i);
      return u32x4{key_of(v[0]), key_of(v[1]), key_of(v[2]), key_of(v[3])};
    }
  };

  // ---- radix select of the kB-th largest key --------------------------
  uint32_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)kB;
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const int nb = 1 << widths[pass];
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < nb; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t i = 4 * tid; i < c; i += 4 * kThreads) {
      const u32x4 k = key4(i);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < c && (k[e] & mask) == prefix) atomicAdd(&hist[(k[e] >> sh) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns the bins [nb - (t+1)*per, nb - t*per): top bins first
    const int per = nb / kThreads;
    const int hi = nb - tid * per;
    uint32_t local = 0;
    for (int e = hi - 1; e >= hi - per; --e) local += hist[e];
    uint32_t tot;
    const uint32_t above = block_excl_scan(local, scratch, &tot);
    if (above < need && need <= above + local) {
      uint32_t acc = above;
      for (int e = hi - 1; e >= hi - per; --e) {
        if (acc + hist[e] >= need) {
          scratch[kWaves] = (uint32_t)e;
          scratch[kWaves + 1] = acc;
          scratch[kWaves + 2] = hist[e];
          break;
        }
        acc += hist[e];
      }
    }
    __syncthreads();
    const uint32_t d = scratch[kWaves];
    const uint32_t above_d = scratch[kWaves + 1];
    const uint32_t in_d = scratch[kWaves + 2];
    __syncthreads();
    need -= above_d;
    prefix |= d << sh;
    mask |= dmask << sh;
    if (in_d == need) break;  // every key with this prefix is kept
  }

  // ---- ordered compaction: keys above the prefix, then the first `need`
  // keys equal to it, in index order --------------------------------------
  uint32_t gt_seen = 0, eq_seen = 0;
  for (int64_t base = 0; base < c; base += 4 * kThreads) {
    const int64_t i0 = base + 4 * tid;
    uint32_t k[4] = {0, 0, 0, 0};
    bool valid[4] = {false, false, false, false};
    if (i0 < c) {
      const u32x4 kv = key4(i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k[e] = kv[e];
        valid[e] = i0 + e < c;
      }
    }
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t m = k[e] & mask;
      ngt += (valid[e] && m > prefix) ? 1u : 0u;
      neq += (valid[e] && m == prefix) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((ngt << 16) | neq, scratch, &tot);
    uint32_t gt_before = gt_seen + (ex >> 16);
    uint32_t eq_before = eq_seen + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!valid[e]) continue;
      const uint32_t m = k[e] & mask;
      if (m > prefix) {
        const uint32_t pos = gt_before + min(eq_before, need);
        out[pos] = (int32_t)(i0 + e);
        if (outs) outs[pos] = __uint_as_float(k[e]);
        ++gt_before;
      } else if (m == prefix) {
        if (eq_before < need) {
          const uint32_t pos = gt_before + eq_before;
          out[pos] = (int32_t)(i0 + e);
          if (outs) outs[pos] = __uint_as_float(k[e]);
        }
        ++eq_before;
      }
    }
    gt_seen += tot >> 16;
    eq_seen += tot & 0xFFFFu;
  }
  if (tid == 0) cnt[row] = kB;
}

}  // namespace

hipError_t launch_select(const Dims& d, int batch, int n_q, const int32_t* q_pos0,
                         int64_t cap, const float* scores, int64_t W, int32_t* sel,
                         int32_t* cnt, float* sel_scores, hipStream_t st) {
  const int64_t cap_blocks = cap / d.r;
  const unsigned rows = (unsigned)((int64_t)batch * n_q);
  const size_t base_shm = sizeof(uint32_t) * (kBins + kScratch);
  if (W <= kCacheMax) {
    const size_t shm = base_shm + sizeof(uint32_t) * (size_t)W;
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_kernel<true>, dim3(rows), dim3(kThreads), shm, st, scores, W, n_q,
                       q_pos0, cap_blocks, d.kB, sel, cnt, sel_scores);
  } else {
    hipLaunchKernelGGL(select_kernel<false>, dim3(rows), dim3(kThreads), base_shm, st, scores, W,
                       n_q, q_pos0, cap_blocks, d.kB, sel, cnt, sel_scores);
  }
  return hipGetLastError();
}

}  // namespace qsa
