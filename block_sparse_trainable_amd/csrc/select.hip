// Top-k_B block selection (kernel c).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works, (A): keep the
// k_B = ceil(K/r) highest-scoring blocks (at most 512 with K = 2048, r = 4,
// per the "Config" line and the gallery page's budget table).  Equal scores
// go to the lower block index, and the kept ids are written in ascending
// order, so the result is unique.
//
// Scores are ReLU sums, hence >= +0.0, so their IEEE bit patterns ("keys")
// order like unsigned integers.  The scoring kernels leave, beside each score
// row, per-segment histograms over 256 monotone bins (score_bin).  Selection:
//   1. sum the row's segment histograms; the threshold bin d* is the highest
//      bin whose suffix count reaches k_B.  Every key in a bin above d* is
//      kept (A of them, A < k_B); need = k_B - A keys of bin d* are kept.
//   2. one sweep over the row in index order keeps the candidates (bin >= d*,
//      typically k_B plus a few hundred) in LDS, still in index order (a
//      workgroup scan gives each its slot).
//   3. an MSB-first radix select (11/11/9-bit digits) over the bin-d*
//      candidates only finds the need-th largest key; a final ordered pass
//      writes the kept ids, ascending, ties to the lower index.
// Long rows (decode) are split into filter segments handled by separate
// workgroups; each hands its candidates over in a global slot and the last
// one to finish (device-scope counter, zeroed by the scoring kernel of the
// same call) gathers the slots in segment order and finishes the row.  If the
// candidates ever exceed the LDS capacity, the row falls back to an exact
// radix select over the whole row in global memory.
#include "qsa_common.h"

namespace qsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRadixBins = 2048;
constexpr int kCandCap = 4096;       // candidates finished in LDS
constexpr int64_t kFilterSeg = 8192; // scores per filter segment of a long row
constexpr uint32_t kOverflow = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t key_of(uint32_t bits) {
  return (bits & 0x80000000u) ? 0u : bits;  // scores are >= 0; guard anyway
}

// Exclusive prefix sum over the workgroup in thread order; total in *total.
// Contains two barriers.
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

struct Radix {
  uint32_t prefix, mask, need;
};

// MSB-first radix select over n keys (key(i)), counting only keys with
// elig(i).  Returns (prefix, mask, need): among eligible keys, those with
// (k & mask) > prefix number need_in - need, and the `need` lowest-index
// eligible keys with (k & mask) == prefix complete the top need_in.
template <class KeyFn, class EligFn>
__device__ Radix radix_select(KeyFn key, EligFn elig, int64_t n, uint32_t need_in,
                              uint32_t* hist, uint32_t* scratch) {
  const int tid = threadIdx.x;
  Radix r{0u, 0u, need_in};
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const int nb = 1 << widths[pass];
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < nb; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kThreads) {
      if (!elig(i)) continue;
      const uint32_t k = key(i);
      if ((k & r.mask) == r.prefix) atomicAdd(&hist[(k >> sh) & dmask], 1u);
    }
    __syncthreads();
    const int per = nb / kThreads;  // thread t owns the bins just below nb - t*per
    const int hi = nb - tid * per;
    uint32_t local = 0;
    for (int e = hi - 1; e >= hi - per; --e) local += hist[e];
    uint32_t tot;
    const uint32_t above = block_excl_scan(local, scratch, &tot);
    if (above < r.need && r.need <= above + local) {
      uint32_t acc = above;
      for (int e = hi - 1; e >= hi - per; --e) {
        if (acc + hist[e] >= r.need) {
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
    r.need -= above_d;
    r.prefix |= d << sh;
    r.mask |= dmask << sh;
    if (in_d == r.need) break;  // every eligible key with this prefix is kept
  }
  return r;
}

// Exact selection over a whole row of c keys in global memory (fallback).
__device__ void select_row_global(const uint32_t* bits, int64_t c, int kB, int32_t* out,
                                  float* outs, uint32_t* hist, uint32_t* scratch) {
  auto key = [&](int64_t i) { return key_of(bits[i]); };
  auto all = [&](int64_t) { return true; };
  const Radix r = radix_select(key, all, c, (uint32_t)kB, hist, scratch);
  uint32_t gt_seen = 0, eq_seen = 0;
  const int tid = threadIdx.x;
  for (int64_t base = 0; base < c; base += 4 * kThreads) {
    const int64_t i0 = base + 4 * tid;
    uint32_t k[4];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k[e] = i0 + e < c ? key(i0 + e) : 0u;
      const uint32_t m = k[e] & r.mask;
      ngt += (i0 + e < c && m > r.prefix) ? 1u : 0u;
      neq += (i0 + e < c && m == r.prefix) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((ngt << 16) | neq, scratch, &tot);
    uint32_t gt_before = gt_seen + (ex >> 16);
    uint32_t eq_before = eq_seen + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e >= c) continue;
      const uint32_t m = k[e] & r.mask;
      if (m > r.prefix) {
        const uint32_t pos = gt_before + min(eq_before, r.need);
        out[pos] = (int32_t)(i0 + e);
        if (outs) outs[pos] = __uint_as_float(k[e]);
        ++gt_before;
      } else if (m == r.prefix) {
        if (eq_before < r.need) {
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
}

struct FilterArgs {
  const float* scores;
  int64_t W;
  const uint32_t* hist;     // per-score-segment histograms
  int64_t sseg, n_sseg;
  uint2* slots;             // [rows][n_fseg][kSlotCap]  (n_fseg > 1 only)
  uint32_t* slotcnt;        // [rows][n_fseg]
  uint32_t* done;           // [rows]
  int64_t fseg, n_fseg;
  int n_q;
  const int32_t* q_pos0;
  int64_t cap_blocks;
  int kB;
  int32_t* sel;
  int32_t* cnt;
  float* sel_scores;
};

__global__ __launch_bounds__(kThreads) void filter_select_kernel(FilterArgs a) {
  __shared__ uint32_t ckey[kCandCap];
  __shared__ uint32_t cidx[kCandCap];
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t scratch[64];

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t fs = blockIdx.y;
  const int s = (int)(row / a.n_q);
  const int j = (int)(row % a.n_q);
  const int64_t p = max((int64_t)a.q_pos0[s] + j, (int64_t)0);
  const int64_t c = min(p / 4, min(a.cap_blocks, a.W));
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(a.scores + row * a.W);
  int32_t* out = a.sel + row * a.kB;
  float* outs = a.sel_scores ? a.sel_scores + row * a.kB : nullptr;
  const int kB = a.kB;

  if (c <= kB) {  // every candidate is kept
    if (fs != 0) return;
    for (int i = tid; i < kB; i += kThreads) {
      out[i] = i < c ? i : -1;
      if (outs) outs[i] = i < c ? __uint_as_float(bits[i]) : 0.0f;
    }
    if (tid == 0) a.cnt[row] = (int32_t)c;
    return;
  }

  // ---- 1. row histogram and threshold bin --------------------------------
  {
    const int64_t nseg = (c + a.sseg - 1) / a.sseg;
    uint32_t lo = 0, hi = 0;
    if (tid < kHistWords) {
      const int w = kHistWords - 1 - tid;  // thread 0 owns the top bins
      for (int64_t g = 0; g < nseg; ++g) {
        const uint32_t v = a.hist[hist_offset(row, g, a.n_sseg) + w];
        lo += v & 0xFFFFu;
        hi += v >> 16;
      }
    }
    uint32_t tot;
    const uint32_t above = block_excl_scan(lo + hi, scratch, &tot);
    if (tid < kHistWords && above < (uint32_t)kB && (uint32_t)kB <= above + lo + hi) {
      const int w = kHistWords - 1 - tid;
      if (above + hi >= (uint32_t)kB) {      // bin 2w+1 holds the k_B-th key
        scratch[kWaves] = 2 * w + 1;
        scratch[kWaves + 1] = above;
        scratch[kWaves + 2] = hi;
      } else {
        scratch[kWaves] = 2 * w;
        scratch[kWaves + 1] = above + hi;
        scratch[kWaves + 2] = lo;
      }
    }
    __syncthreads();
  }
  const uint32_t dstar = scratch[kWaves];
  const uint32_t n_sure = scratch[kWaves + 1];
  const uint32_t n_maybe = scratch[kWaves + 2];
  const uint32_t need = (uint32_t)kB - n_sure;
  __syncthreads();

  // ---- 2. ordered sweep of this filter segment --------------------------
  const int64_t lo_i = fs * a.fseg;
  const int64_t hi_i = min(lo_i + a.fseg, c);
  const uint32_t cap = a.n_fseg == 1 ? (uint32_t)kCandCap : (uint32_t)kSlotCap;
  uint32_t ncand = 0;
  bool overflow = false;
  for (int64_t base = lo_i; base < hi_i; base += 4 * kThreads) {
    const int64_t i0 = base + 4 * tid;   // lo_i, base multiples of 4: aligned loads
    uint32_t k[4] = {0, 0, 0, 0};
    uint32_t m = 0;
    if (i0 < hi_i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(bits + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k[e] = key_of(v[e]);
        if (i0 + e < hi_i && score_bin(k[e]) >= dstar) m |= 1u << e;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((uint32_t)__popc(m), scratch, &tot);
    if (ncand + tot > cap) overflow = true;
    if (!overflow) {
      uint32_t pos = ncand + ex;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (m & (1u << e)) {
          ckey[pos] = k[e];
          cidx[pos] = (uint32_t)(i0 + e);
          ++pos;
        }
    }
    ncand += tot;
  }
  __syncthreads();

  uint32_t total = ncand;
  if (a.n_fseg > 1) {
    // hand the candidates over, then the last segment to finish gathers all
    uint2* slot = a.slots + (row * a.n_fseg + fs) * kSlotCap;
    if (!overflow)
      for (uint32_t i = tid; i < ncand; i += kThreads) slot[i] = make_uint2(ckey[i], cidx[i]);
    if (tid == 0) a.slotcnt[row * a.n_fseg + fs] = overflow ? kOverflow : ncand;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = atomicAdd(&a.done[row], 1u);
      scratch[kWaves + 3] = (old == (uint32_t)a.n_fseg - 1u) ? 1u : 0u;
    }
    __syncthreads();
    if (scratch[kWaves + 3] == 0u) return;
    __threadfence();
    if (tid == 0) a.done[row] = 0u;  // leave the counter zeroed
    // gather slots in segment order
    total = 0;
    overflow = false;
    for (int64_t g = 0; g < a.n_fseg; ++g) {
      const uint32_t n = a.slotcnt[row * a.n_fseg + g];
      if (n == kOverflow || total + n > (uint32_t)kCandCap) {
        overflow = true;
        break;
      }
      const uint2* src = a.slots + (row * a.n_fseg + g) * kSlotCap;
      for (uint32_t i = tid; i < n; i += kThreads) {
        const uint2 v = src[i];
        ckey[total + i] = v.x;
        cidx[total + i] = v.y;
      }
      total += n;
    }
    __syncthreads();
  }

  if (overflow || total != n_sure + n_maybe) {
    select_row_global(bits, c, kB, out, outs, hist, scratch);
    if (tid == 0) a.cnt[row] = kB;
    return;
  }

  // ---- 3. exact choice among the threshold-bin candidates ---------------
  Radix r{0u, 0u, need};
  if (need < n_maybe) {
    auto key = [&](int64_t i) { return ckey[i]; };
    auto elig = [&](int64_t i) { return score_bin(ckey[i]) == dstar; };
    r = radix_select(key, elig, (int64_t)total, need, hist, scratch);
  }
  // ordered output: bin > d* always; bin == d* by (k & mask) vs prefix
  uint32_t written = 0, eq_seen = 0;
  for (uint32_t base = 0; base < total; base += 8 * kThreads) {
    const uint32_t i0 = base + 8 * tid;
    uint32_t take = 0, eqm = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t i = i0 + e;
      if (i >= total) break;
      const uint32_t k = ckey[i];
      if (score_bin(k) != dstar) {
        take |= 1u << e;
      } else if (need >= n_maybe || (k & r.mask) > r.prefix) {
        take |= 1u << e;
      } else if ((k & r.mask) == r.prefix) {
        eqm |= 1u << e;
      }
    }
    // ties: the first r.need equal keys (index order) are kept
    uint32_t tot_eq;
    const uint32_t ex_eq = block_excl_scan((uint32_t)__popc(eqm), scratch, &tot_eq);
    uint32_t eq_rank = eq_seen + ex_eq;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (eqm & (1u << e)) {
        if (eq_rank < r.need) take |= 1u << e;
        ++eq_rank;
      }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((uint32_t)__popc(take), scratch, &tot);
    uint32_t pos = written + ex;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (take & (1u << e)) {
        out[pos] = (int32_t)cidx[i0 + e];
        if (outs) outs[pos] = __uint_as_float(ckey[i0 + e]);
        ++pos;
      }
    written += tot;
    eq_seen += tot_eq;
  }
  if (tid == 0) a.cnt[row] = kB;
}

}  // namespace

SelectPlan select_plan(const Dims& d, int batch, int n_q, int32_t max_pos_end) {
  SelectPlan p{};
  const bool mfma = d.bf16 && d.idx_heads == 4 && d.idx_dim == 128;
  p.kernel = !mfma ? 0 : (n_q >= 16 ? 1 : 2);
  p.W = score_row_width(d.r, max_pos_end);
  const int64_t c_max = max((int64_t)1, (int64_t)(max_pos_end - 1) / d.r);
  p.sseg = p.kernel == 0 ? 256 : 2048;
  p.n_sseg = (c_max + p.sseg - 1) / p.sseg;
  const int64_t rows = (int64_t)batch * n_q;
  if (rows >= 256 || c_max <= kFilterSeg) {
    p.fseg = (c_max + 3) / 4 * 4;
    p.n_fseg = 1;
  } else {
    p.fseg = kFilterSeg;
    p.n_fseg = (c_max + kFilterSeg - 1) / kFilterSeg;
  }
  auto align = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t off = align(sizeof(float) * (size_t)rows * (size_t)p.W);
  p.off_hist = off;
  off = align(off + sizeof(uint32_t) * (size_t)rows * p.n_sseg * kHistWords);
  p.off_slots = off;
  if (p.n_fseg > 1) off = align(off + sizeof(uint2) * (size_t)rows * p.n_fseg * kSlotCap);
  p.off_slotcnt = off;
  off = align(off + sizeof(uint32_t) * (size_t)rows * p.n_fseg);
  p.off_done = off;
  off = align(off + sizeof(uint32_t) * (size_t)rows);
  p.bytes = off;
  return p;
}

hipError_t launch_select(const Dims& d, const SelectPlan& pl, int batch, int n_q,
                         const int32_t* q_pos0, int64_t cap, void* workspace, int32_t* sel,
                         int32_t* cnt, float* sel_scores, hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  FilterArgs a;
  a.scores = reinterpret_cast<const float*>(ws);
  a.W = pl.W;
  a.hist = reinterpret_cast<const uint32_t*>(ws + pl.off_hist);
  a.sseg = pl.sseg;
  a.n_sseg = pl.n_sseg;
  a.slots = reinterpret_cast<uint2*>(ws + pl.off_slots);
  a.slotcnt = reinterpret_cast<uint32_t*>(ws + pl.off_slotcnt);
  a.done = reinterpret_cast<uint32_t*>(ws + pl.off_done);
  a.fseg = pl.fseg;
  a.n_fseg = pl.n_fseg;
  a.n_q = n_q;
  a.q_pos0 = q_pos0;
  a.cap_blocks = cap / d.r;
  a.kB = d.kB;
  a.sel = sel;
  a.cnt = cnt;
  a.sel_scores = sel_scores;
  dim3 grid((unsigned)((int64_t)batch * n_q), (unsigned)pl.n_fseg);
  hipLaunchKernelGGL(filter_select_kernel, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qsa
