// Top-k_B block selection (kernel c).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works, (A): keep the
// k_B = ceil(K/r) highest-scoring blocks (512 with K = 2048, r = 4, per the
// "Config" line and the gallery page's budget table; up to 2,048 single
// tokens at r = 1, the token-level end of the QSA-vs-DSA table).  Equal scores
// go to the lower block index, and the kept ids are written in ascending
// order, so the result is unique.
//
// Scores are ReLU sums, hence >= +0.0, so their IEEE bit patterns ("keys")
// order like unsigned integers.  The scoring kernels leave, beside each score
// row, per-segment histograms over 256 monotone bins (score_bin).  Selection:
//   1. sum the row's segment histograms; the threshold bin d* is the highest
//      bin whose suffix count reaches k_B.  Every key in a bin above d* is
//      kept (A of them, A < k_B); need = k_B - A keys of bin d* are kept.
//   2. the same histograms give every segment's exact number of candidates
//      (keys with bin >= d*, typically k_B plus a few hundred per row), hence
//      its exact output offset; each wave then sweeps whole segments with all
//      loads in flight and a ballot compaction, so the candidates land in
//      index order without any workgroup-wide barrier.
//   3. an MSB-first radix select (11/11/9-bit digits) over the bin-d*
//      candidates only finds the need-th largest key; a final ordered pass
//      writes the kept ids, ascending, ties to the lower index.
// Long rows (decode) are split over several filter workgroups, which write
// their candidates at their exact offsets into a row-wide array; the last one
// to finish (device-scope counter, zeroed by the scoring kernel of the same
// call) loads them and finishes the row.  If a row ever has more candidates
// than the LDS capacity, it falls back to an exact radix select over the
// whole row in global memory.
#include "qsa_common.h"
#include "select_common.h"

namespace qsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int64_t kFilterSeg = 8192; // scores per filter segment of a long row
constexpr uint32_t kOverflow = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t key_of(uint32_t bits) {
  return (bits & 0x80000000u) ? 0u : bits;  // scores are >= 0; guard anyway
}

// Exact selection over a whole row of c keys in global memory (fallback),
// by a workgroup of NT threads.
template <int NT>
__device__ __forceinline__ void select_row_global_nt(const uint32_t* bits, int64_t c, int kB,
                                                     int32_t* out, float* outs, uint32_t* hist,
                                                     uint32_t* scratch) {
  auto key = [&](int64_t i) { return key_of(bits[i]); };
  auto all = [&](int64_t) { return true; };
  const Radix r = radix_select<NT>(key, all, c, (uint32_t)kB, hist, scratch);
  uint32_t gt_seen = 0, eq_seen = 0;
  const int tid = threadIdx.x;
  for (int64_t base = 0; base < c; base += 4 * NT) {
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
    const uint32_t ex = block_excl_scan<NT>((ngt << 16) | neq, scratch, &tot);
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
  const float* scores;      // f32 rows (16-bit keys on the streamed prefill path)
  const uint16_t* q_idx;    // indexer queries and compressed keys (bf16): exact
  const uint16_t* k_cmp;    //   scores of keys tied at a 16-bit threshold
  int64_t W;
  const uint32_t* hist;     // per-score-segment histograms
  int64_t sseg, n_sseg;     // blocks per score segment, segments per row (max)
  uint2* cand;              // [rows][kCandCap] candidates of split rows
  uint32_t* done;           // [rows] completion counters of split rows
  int64_t spw;              // score segments per filter workgroup
  int64_t n_fseg;           // filter workgroups per row
  int n_q;
  int64_t nq_pad;           // score rows per sequence
  const int32_t* q_pos0;
  int64_t cap_blocks;
  int lr;             // log2 of the block size r
  int kB;
  int32_t* sel;
  int32_t* cnt;
  float* sel_scores;
};

constexpr int kMaxSeg = 2048;  // score segments per row the offsets table holds

// PRE: split rows whose workgroup sweeps one segment per wave load those
// scores up front (only the decode shape; it costs registers).
template <bool PRE>
__global__ __launch_bounds__(kThreads) void filter_select_kernel(FilterArgs a) {
  __shared__ uint32_t ckey[kCandCap];
  __shared__ uint32_t cidx[kCandCap];
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t segoff[kMaxSeg];
  __shared__ uint32_t scratch[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t fs = blockIdx.y;
  const int s = (int)(row / a.n_q);
  const int j = (int)(row % a.n_q);
  const int64_t p = max((int64_t)a.q_pos0[s] + j, (int64_t)0);
  const int64_t c = min(p >> a.lr, min(a.cap_blocks, a.W));
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(a.scores + (s * a.nq_pad + j) * a.W);
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
  const int64_t nseg = (c + a.sseg - 1) / a.sseg;
  const uint32_t* hrow = a.hist + hist_offset(row, 0, a.n_sseg);

  // ---- 1. row histogram and threshold bin ---------------------------------
  // A split workgroup (long decode rows) also issues its own segment's score
  // loads here, so they overlap the histogram work (one segment of <= 1024
  // scores per wave).
  const bool split = a.n_fseg > 1;
  const bool pre_sweep = PRE && split && a.sseg <= 1024 && a.spw <= kWaves;
  u32x4 pv[4];
  if constexpr (PRE) {
    const int64_t g = fs * a.spw + wave;
    const int64_t i_lo = g * a.sseg;
    const int64_t i_hi = min(i_lo + a.sseg, c);
    const bool mine = g < min(fs * a.spw + a.spw, nseg);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i0 = i_lo + 256 * u + 4 * lane;
      pv[u] = (mine && i0 < i_hi) ? *reinterpret_cast<const u32x4*>(bits + i0) : u32x4{0, 0, 0, 0};
    }
  }
  {
    // 512 threads: word w = 127 - (tid & 127) of every 4th segment
    uint32_t* part = hist;  // [4][128][2] partial sums (lo, hi)
    {
      const int w = kHistWords - 1 - (tid & 127);
      uint32_t lo = 0, hi = 0;
#pragma unroll 8
      for (int64_t g = tid >> 7; g < nseg; g += 4) {
        const uint32_t v = hrow[g * kHistWords + w];
        lo += v & 0xFFFFu;
        hi += v >> 16;
      }
      part[(tid >> 7) * 256 + 2 * (tid & 127)] = lo;
      part[(tid >> 7) * 256 + 2 * (tid & 127) + 1] = hi;
    }
    __syncthreads();
    uint32_t lo = 0, hi = 0;
    if (tid < kHistWords) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        lo += part[q4 * 256 + 2 * tid];
        hi += part[q4 * 256 + 2 * tid + 1];
      }
    }
    uint32_t tot;
    const uint32_t above = block_excl_scan<kThreads>(lo + hi, scratch, &tot);
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
  const uint32_t total = n_sure + n_maybe;
  __syncthreads();

  // ---- 2. exact candidate offset of every score segment -------------------
  // candidates of segment g = its keys with bin >= d*, read off its histogram
  const bool fits = total <= (uint32_t)kCandCap && nseg <= kMaxSeg;
  if (fits) {
    const int w0 = (int)(dstar >> 1);
    const int nw = kHistWords - w0;  // words holding bins >= d*
    for (int64_t g = tid; g < nseg; g += kThreads) segoff[g] = 0u;
    __syncthreads();
    const int64_t pairs = nseg * nw;
#pragma unroll 4
    for (int64_t i = tid; i < pairs; i += kThreads) {
      const int64_t g = i / nw;
      const int w = w0 + (int)(i % nw);
      const uint32_t v = hrow[g * kHistWords + w];
      const uint32_t n = (v >> 16) + ((w == w0 && (dstar & 1u)) ? 0u : (v & 0xFFFFu));
      if (n) atomicAdd(&segoff[g], n);
    }
    __syncthreads();
    // exclusive scan of segoff[0..nseg): thread t owns entries 4t..4t+3
    uint32_t v[4], sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t g = 4 * tid + e;
      v[e] = g < nseg ? segoff[g] : 0u;
      sum += v[e];
    }
    uint32_t tot;
    uint32_t run = block_excl_scan<kThreads>(sum, scratch, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t g = 4 * tid + e;
      if (g < nseg) segoff[g] = run;
      run += v[e];
    }
    __syncthreads();
  }

  // ---- 3. sweep this workgroup's segments; waves take whole segments ------
  uint2* gcand = split ? a.cand + row * kCandCap : nullptr;
  if (fits) {
    const int64_t g_lo = fs * a.spw;
    const int64_t g_hi = min(g_lo + a.spw, nseg);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // keys i0..i0+3 (lane-ordered stretch of 256): keep those with bin >= d*
    auto take4 = [&](int64_t i0, int64_t i_hi, const u32x4& v, uint32_t& pos) {
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e < i_hi && score_bin(key_of(v[e])) >= dstar) m |= 1u << e;
      // order within the stretch: lane-major, then element
      uint32_t before = 0, all = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t b = __ballot((m >> e) & 1u);
        before += (uint32_t)__popcll(b & lt);
        all += (uint32_t)__popcll(b);
      }
      uint32_t at = pos + before;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((m >> e) & 1u) {
          const uint32_t k = key_of(v[e]);
          const uint32_t idx = (uint32_t)(i0 + e);
          if (at < (uint32_t)kCandCap) {
            if (split) {
              coherent_store(reinterpret_cast<unsigned long long*>(gcand + at),
                             (unsigned long long)k | ((unsigned long long)idx << 32));
            } else {
              ckey[at] = k;
              cidx[at] = idx;
            }
          }
          ++at;
        }
      pos += all;
    };
    if (PRE && pre_sweep) {
      const int64_t g = g_lo + wave;   // this wave's one segment, already loaded
      if (g < g_hi) {
        const int64_t i_lo = g * a.sseg;
        const int64_t i_hi = min(i_lo + a.sseg, c);
        uint32_t pos = segoff[g];
#pragma unroll
        for (int u = 0; u < 4; ++u) take4(i_lo + 256 * u + 4 * lane, i_hi, pv[u], pos);
      }
    } else {
      for (int64_t g = g_lo + wave; g < g_hi; g += kWaves) {
        const int64_t i_lo = g * a.sseg;
        const int64_t i_hi = min(i_lo + a.sseg, c);
        uint32_t pos = segoff[g];
        for (int64_t base = i_lo; base < i_hi; base += 256 * 8) {
          u32x4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {   // all of this stretch's loads in flight
            const int64_t i0 = base + 256 * u + 4 * lane;
            v[u] = i0 < i_hi ? *reinterpret_cast<const u32x4*>(bits + i0) : u32x4{0, 0, 0, 0};
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) take4(base + 256 * u + 4 * lane, i_hi, v[u], pos);
        }
      }
    }
  }

  if (split) {
    // the last filter workgroup of the row finishes it
    stores_complete();
    __syncthreads();
    if (tid == 0) scratch[kWaves + 3] = arrive_last(&a.done[row], (uint32_t)a.n_fseg) ? 1u : 0u;
    __syncthreads();
    if (scratch[kWaves + 3] == 0u) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (tid == 0) coherent_store(&a.done[row], 0u);  // leave the counter zeroed
    if (fits)
      for (uint32_t i = tid; i < total; i += kThreads) {
        const unsigned long long v =
            coherent_load(reinterpret_cast<const unsigned long long*>(gcand + i));
        ckey[i] = (uint32_t)v;
        cidx[i] = (uint32_t)(v >> 32);
      }
  }
  __syncthreads();

  if (!fits) {
    select_row_global_nt<kThreads>(bits, c, kB, out, outs, hist, scratch);
    if (tid == 0) a.cnt[row] = kB;
    return;
  }

  // ---- 4. exact choice among the threshold-bin candidates ---------------
  Radix r{0u, 0u, need};
  if (need < n_maybe) {
    auto key = [&](int64_t i) { return ckey[i]; };
    auto elig = [&](int64_t i) { return score_bin(ckey[i]) == dstar; };
    if (dstar > 0u && dstar < (uint32_t)kHistBins - 1u) {
      // an unclamped bin fixes bits 30..20 of its keys: start at the second digit
      r = radix_select<kThreads, true>(key, elig, (int64_t)total, need, hist, scratch, 1, (dstar + 888u) << 20,
                       0x7FFu << 20);
    } else {
      r = radix_select<kThreads, true>(key, elig, (int64_t)total, need, hist, scratch);
    }
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
    const uint32_t ex_eq = block_excl_scan<kThreads>((uint32_t)__popc(eqm), scratch, &tot_eq);
    uint32_t eq_rank = eq_seen + ex_eq;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (eqm & (1u << e)) {
        if (eq_rank < r.need) take |= 1u << e;
        ++eq_rank;
      }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kThreads>((uint32_t)__popc(take), scratch, &tot);
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

// ---------------------------------------------------------------------------
// Rows selected without histograms (the prefill shape: many rows of at most
// kStreamMax candidates).  The scoring kernel leaves 16-bit keys for these
// rows: the top half of each score's bits, which orders like the score.  One
// workgroup per row:
//   1. a strided sample of the row gives its mean and spread, hence a floor F
//      with, for a normal row, about 1.4 k_B keys at or above it (normal
//      upper-tail quantile; score rows have heavier upper tails, so the pool
//      holds more);
//   2. the row is streamed once; the keys >= F are compacted, in index order,
//      into an LDS pool.  Long rows let F rise when the pool fills: it moves
//      to the (k_B + kPrune)-th largest key kept so far, still a valid floor
//      since at least k_B keys of the row are at or above it.  Unless
//      k_B <= pool size, F moves down and the row is streamed again (a few
//      tries, then the exact whole-row fallback);
//   3. a radix select over the pool finds the 16-bit threshold key T.  Keys
//      above T are kept.  If the keys equal to T are more than the places
//      left, their exact scores are recomputed in fp32 from the indexer
//      query and the compressed keys, and the largest are kept, equal exact
//      scores going to the lower index;
//   4. the ordered pass writes the kept ids ascending.  The reported score is
//      the exact one for keys equal to T, else the key's value (its top 16
//      bits: at most 2^-8 below the score).
// In the pool a key is stored as key << 15 (bits 30..15), so the generic
// radix select resolves it in two digits.
constexpr int64_t kStreamMax = int64_t{1} << 20;   // candidates per row this path takes
constexpr int kRowCap = 3072;                      // pool capacity (candidates), k_B <= 512
constexpr int kRowCapBig = 6144;                   // ... for k_B up to 2048
// pool slot i lives at i + i / 16: the ordered pass reads 16 consecutive
// slots per thread, which would otherwise all fall in two banks
__device__ __forceinline__ uint32_t pslot(uint32_t i) { return i + (i >> 4); }
constexpr int64_t kRowShortMax = 40960;            // candidates of a "short" row
constexpr int kPrune = 256;                        // keys kept above k_B when the pool is pruned
constexpr uint32_t kBand = 0x80000000u;            // cidx flag: key equal to the threshold
constexpr uint32_t kBandKept = 0x40000000u;        // cidx flag: ... and kept
constexpr uint32_t kIdxMask = 0x3FFFFFFFu;
constexpr int kBandMax = 256;                      // band keys resolved in the pool

// z with P(Z > z) = p for a standard normal Z and 0 < p < 0.5: Abramowitz &
// Stegun 26.2.23 (absolute error below 4.5e-4).
__device__ __forceinline__ float normal_upper_quantile(float p) {
  const float t = sqrtf(-2.0f * __logf(p));
  return t - (2.515517f + t * (0.802853f + t * 0.010328f)) /
                 (1.0f + t * (1.432788f + t * (0.189269f + t * 0.001308f)));
}

// Block importance of one block in fp32 ("QSA (Qwen Sparse Attention)", Key
// math / How it works, (A)): qs holds the row's 4 x 128 indexer query in fp32
// (LDS, read as a broadcast), kb the block's 128 bf16 compressed-key values.
// Returns the bits of the non-negative result.
__device__ __forceinline__ uint32_t exact_score_bits(const float* qs, const uint16_t* kb) {
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int c16 = 0; c16 < 16; ++c16) {
    const u32x4 w = ld16(kb + 8 * c16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kv = bf16_to_f32((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
#pragma unroll
      for (int h = 0; h < 4; ++h) acc[h] = fmaf(qs[h * 128 + 8 * c16 + e], kv, acc[h]);
    }
  }
  return __float_as_uint(relu(acc[0]) + relu(acc[1]) + relu(acc[2]) + relu(acc[3]));
}

__device__ __forceinline__ float key16_value(uint32_t pool_key) {
  return __uint_as_float((pool_key >> 15) << 16);
}

// Exact selection over a whole row of 16-bit keys in global memory (the
// fallback), with keys tied at the threshold resolved from exact scores.
template <int NT, class ExactFn>
__device__ __forceinline__ void select_row_global16(const uint16_t* keys, int64_t c, int kB, int32_t* out,
                                    float* outs, uint32_t* hist, uint32_t* scratch, ExactFn exact) {
  auto key = [&](int64_t i) { return (uint32_t)keys[i] << 15; };
  auto all = [&](int64_t) { return true; };
  const Radix r = radix_select<NT, false, 8>(key, all, c, (uint32_t)kB, hist, scratch, 0, 0u, 0u, 1);
  const bool band = r.need < r.avail;
  Radix r2{0u, 0u, 0u, 0u}, r3{0u, 0u, 0u, 0u};
  bool ties = false;
  auto in_band = [&](int64_t i) { return (key(i) & r.mask) == r.prefix; };
  if (band) {
    auto ex = [&](int64_t i) { return exact((uint32_t)i); };
    r2 = radix_select<NT, false, 8>(ex, in_band, c, r.need, hist, scratch);
    ties = r2.need < r2.avail;
    if (ties) {
      auto ik = [&](int64_t i) { return 0x7FFFFFFFu - (uint32_t)i; };
      auto eq = [&](int64_t i) { return in_band(i) && (exact((uint32_t)i) & r2.mask) == r2.prefix; };
      r3 = radix_select<NT, false, 8>(ik, eq, c, r2.need, hist, scratch);
    }
  }
  uint32_t written = 0;
  const int tid = threadIdx.x;
  for (int64_t base = 0; base < c; base += 4 * NT) {
    const int64_t i0 = base + 4 * tid;
    uint32_t take = 0;
    float val[4];
    // branch-free per element: the exact score is computed once (band keys
    // only), then the kept value is chosen among the key's, the exact one
    // and 0 (a nested conditional assignment of the exact value here was
    // compiled to store 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      const bool in = i < c;
      const uint32_t kf = in ? key(i) : 0u;
      const uint32_t k = kf & r.mask;
      const bool at_t = in && band && k == r.prefix;
      const uint32_t x = at_t ? exact((uint32_t)i) : 0u;
      const uint32_t m = x & r2.mask;
      const bool hi = in && (k > r.prefix || (!band && k == r.prefix));
      const bool kb = at_t && (m > r2.prefix ||
                               (m == r2.prefix &&
                                (!ties || ((0x7FFFFFFFu - (uint32_t)i) & r3.mask) >= r3.prefix)));
      take |= (hi || kb) ? 1u << e : 0u;
      val[e] = hi ? key16_value(kf) : (kb ? __uint_as_float(x) : 0.0f);
    }
    uint32_t tot;
    uint32_t pos = written + block_excl_scan<NT>((uint32_t)__popc(take), scratch, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (take & (1u << e)) {
        out[pos] = (int32_t)(i0 + e);
        if (outs) outs[pos] = val[e];
        ++pos;
      }
    written += tot;
  }
}

// One workgroup of NT threads per row: sample, stream in batches of BATCH
// 16-byte pieces (8 keys each) per thread, DEPTH batches in flight,
// compacting into the LDS pool of CAP candidates in index order, then the
// threshold and the ordered output.  PRUNE (long rows) lets the floor rise
// during the pass instead of streaming the row again.
template <int NT, int BATCH, bool PRUNE, int DEPTH, int CAP>
__global__ __launch_bounds__(NT) void select_row_kernel(FilterArgs a) {
  constexpr int NW = NT / 64;
  constexpr int kRowCap = CAP;
  constexpr int kSlots = kRowCap + kRowCap / 16;
  static_assert(NW % 4 == 0, "batch offsets read 4-wave groups of counts");
  __shared__ uint32_t ckey[kSlots];
  __shared__ uint32_t cidx[kSlots];
  // 8-bit radix digits (256 words), or the band: indices, exact scores, ranks
  __shared__ uint32_t hist[3 * kBandMax];
  __shared__ __attribute__((aligned(16))) uint32_t wt[BATCH * NW];
  __shared__ float fred[3 * NW];
  __shared__ float qs[512];
  __shared__ uint32_t scratch[64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int s = (int)(row / a.n_q);
  const int j = (int)(row % a.n_q);
  const int64_t p = max((int64_t)a.q_pos0[s] + j, (int64_t)0);
  const int64_t c = min(p >> a.lr, min(a.cap_blocks, a.W));
  const uint16_t* keys = reinterpret_cast<const uint16_t*>(a.scores) + (s * a.nq_pad + j) * a.W;
  int32_t* out = a.sel + row * a.kB;
  float* outs = a.sel_scores ? a.sel_scores + row * a.kB : nullptr;
  const int kB = a.kB;

  if (c <= kB) {  // every candidate is kept
    for (int i = tid; i < kB; i += NT) {
      out[i] = i < c ? i : -1;
      if (outs) outs[i] = i < c ? key16_value((uint32_t)keys[i] << 15) : 0.0f;
    }
    if (tid == 0) a.cnt[row] = (int32_t)c;
    return;
  }
  const int ci = (int)c;
  // the row's indexer query in fp32, for exact scores of tied keys
  {
    const uint16_t* qrow = a.q_idx + ((int64_t)s * a.n_q + j) * 512;
    for (int i = tid; i < 512; i += NT) qs[i] = bf16_to_f32(qrow[i]);
  }
  const uint16_t* kseq = a.k_cmp + (int64_t)s * a.cap_blocks * 128;
  auto exact = [&](uint32_t b) { return exact_score_bits(qs, kseq + (int64_t)b * 128); };

  // ---- 1. sampled mean and spread (the barrier also publishes qs) --------
  float sm = 0.0f, sq = 0.0f, sn = 0.0f;
  {
    const int n8 = (ci + 7) / 8;
    const int k = (int)((int64_t)tid * n8 / NT);
    const u32x4 w = *reinterpret_cast<const u32x4*>(keys + 8 * k);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (8 * k + e < ci) {
        const float x = __uint_as_float(((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu)) << 16);
        sm += x;
        sq = fmaf(x, x, sq);
        sn += 1.0f;
      }
  }
  {  // wave sums: per row of 16 lanes, then the four rows' last lanes
    auto wsum = [](float v) {
      v = row16_sum_to_last(v);
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15)) +
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31)) +
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47)) +
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    };
    sm = wsum(sm);
    sq = wsum(sq);
    sn = wsum(sn);
  }
  if (lane == 0) {
    fred[wave] = sm;
    fred[NW + wave] = sq;
    fred[2 * NW + wave] = sn;
  }
  __syncthreads();
  sm = sq = sn = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    sm += fred[w];
    sq += fred[NW + w];
    sn += fred[2 * NW + w];
  }
  const float mu = sm / sn;
  const float sd = sqrtf(fmaxf(sq / sn - mu * mu, 0.0f));
  const float pfrac = 1.4f * (float)kB / (float)ci;
  float z = pfrac < 0.5f ? normal_upper_quantile(pfrac) : -INFINITY;

  // ---- 2. stream the row into the pool; accept or move the floor ---------
  constexpr int kStep = 8 * NT * BATCH;
  const int last8 = (ci - 1) & ~7;
  uint32_t n_f = 0u;
  bool ok = false;
  for (int attempt = 0; attempt < 4 && !ok; ++attempt) {
    // F as a pool key, at least the smallest positive one: zero keys never
    // count (a row that needs them takes the fallback)
    const float f = z == -INFINITY ? 0.0f : fmaxf(mu + z * sd, 0.0f);
    uint32_t fkey = max(__float_as_uint(f) >> 16, 1u) << 15;
    uint32_t total = 0u;   // uniform: candidates before this batch
    bool overflow = false;
    // batches prefetched DEPTH deep in registers; loads are unconditional
    // (addresses clamped to the row's last piece, keys past c masked by
    // index) so the compiler waits for the current batch only
    u32x4 nx[DEPTH][BATCH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        nx[d][b] = *reinterpret_cast<const u32x4*>(keys + min(d * kStep + 8 * (tid + NT * b), last8));
    for (int base = 0; base < ci; base += kStep) {
      u32x4 v[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) v[b] = nx[0][b];
#pragma unroll
      for (int d = 0; d + 1 < DEPTH; ++d)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) nx[d][b] = nx[d + 1][b];
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        nx[DEPTH - 1][b] =
            *reinterpret_cast<const u32x4*>(keys + min(base + DEPTH * kStep + 8 * (tid + NT * b), last8));
      // the row's last batch: keys at or past c read as 0 (never taken)
      if (base + kStep > ci) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          const int lim = min(max(ci - (base + 8 * (tid + NT * b)), 0), 8);
#pragma unroll
          for (int w = 0; w < 4; ++w)
            v[b][w] &= (2 * w < lim ? 0xFFFFu : 0u) | (2 * w + 1 < lim ? 0xFFFF0000u : 0u);
        }
      }
      // key e of piece b for a lane-varying e (selects instead of indexing)
      auto k16v = [&](int b, uint32_t e) {
        const uint32_t w = (e & 4u) ? ((e & 2u) ? v[b][3] : v[b][2]) : ((e & 2u) ? v[b][1] : v[b][0]);
        return ((e & 1u) ? (w >> 16) : (w & 0xFFFFu)) << 15;
      };
      // candidates of piece b: bit e set for key e >= F (the high key of a
      // word compares whole; the low one after a shift)
      // Index order within the batch is (b, wave, lane, e).  Each lane's
      // count per piece (0..8) is scanned across the wave three pieces at a
      // time in 10-bit fields; the wave totals per piece go through LDS.
      uint32_t excl[BATCH];
      uint32_t msk[BATCH];
      for (int pass = 0;; ++pass) {
        uint32_t cnt[BATCH];
        const uint32_t f_hi = (fkey >> 15) << 16;
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          uint32_t m = 0;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            m |= (v[b][w] << 16) >= f_hi ? 1u << (2 * w) : 0u;
            m |= v[b][w] >= f_hi ? 1u << (2 * w + 1) : 0u;
          }
          msk[b] = m;
          cnt[b] = (uint32_t)__popc(m);
        }
#pragma unroll
        for (int g = 0; g < BATCH; g += 3) {
          uint32_t x = 0;
#pragma unroll
          for (int q = 0; q < 3; ++q)
            if (g + q < BATCH) x |= cnt[g + q] << (10 * q);
          const uint32_t incl = wave_incl_add(x);
          const uint32_t ex = incl - x;
          const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
#pragma unroll
          for (int q = 0; q < 3; ++q)
            if (g + q < BATCH) {
              excl[g + q] = (ex >> (10 * q)) & 1023u;
              if (lane == 0) wt[(g + q) * NW + wave] = (tot >> (10 * q)) & 1023u;
            }
        }
        __syncthreads();
        uint32_t btot = 0u;
#pragma unroll
        for (int q = 0; q < BATCH * NW; q += 4) {
          const u32x4 r4 = *reinterpret_cast<const u32x4*>(&wt[q]);
          btot += r4[0] + r4[1] + r4[2] + r4[3];
        }
        if (total + btot <= (uint32_t)kRowCap) break;
        if (!PRUNE || pass > 0 || total < (uint32_t)(kB + kPrune)) {   // no room for the batch
          overflow = true;
          break;
        }
        if constexpr (PRUNE) {
          // raise the floor to the (k_B + kPrune)-th largest pool key and keep
          // only the keys at or above it, compacted in place: every thread
          // holds its E consecutive entries in registers, and the scan's
          // barriers separate all reads from the writes (an entry only moves
          // down)
          auto pkey = [&](int64_t i) { return ckey[pslot((uint32_t)i)]; };
          auto pall = [&](int64_t) { return true; };
          const Radix rp = radix_select<NT, true, 8>(pkey, pall, (int64_t)total, (uint32_t)(kB + kPrune), hist,
                                            scratch, 0, 0u, 0u, 1);
          fkey = max(fkey, rp.prefix);
          constexpr int E = kRowCap / NT;
          uint32_t pk[E], px[E];
          uint32_t keep = 0, kmask = 0;
#pragma unroll
          for (int q = 0; q < E; ++q) {
            const uint32_t i = (uint32_t)(E * tid + q);
            const uint32_t ic = i < total ? i : 0u;
            pk[q] = ckey[pslot(ic)];
            px[q] = cidx[pslot(ic)];
            const bool kp = i < total && pk[q] >= fkey;
            kmask |= kp ? 1u << q : 0u;
            keep += kp ? 1u : 0u;
          }
          uint32_t kept;
          uint32_t at = block_excl_scan<NT>(keep, scratch, &kept);
#pragma unroll
          for (int q = 0; q < E; ++q)
            if ((kmask >> q) & 1u) {
              ckey[pslot(at)] = pk[q];
              cidx[pslot(at)] = px[q];
              ++at;
            }
          total = kept;
          __syncthreads();
        }
      }
      if (overflow) break;
      // wave-uniform offsets in (b, wave) order; each lane writes only its
      // candidates, in key order (every candidate fits: total + btot <=
      // kRowCap)
      uint32_t run = total;
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        uint32_t off = run;
#pragma unroll
        for (int w4 = 0; w4 < NW; w4 += 4) {
          const u32x4 r4 = *reinterpret_cast<const u32x4*>(&wt[b * NW + w4]);
#pragma unroll
          for (int w = 0; w < 4; ++w) off += w4 + w < wave ? r4[w] : 0u;
          run += r4[0] + r4[1] + r4[2] + r4[3];
        }
        uint32_t at = off + excl[b];
        const int i0 = base + 8 * (tid + NT * b);
        for (uint32_t m = msk[b]; m != 0u; m &= m - 1u) {
          const uint32_t e = (uint32_t)__builtin_ctz(m);
          ckey[pslot(at)] = k16v(b, e);
          cidx[pslot(at)] = (uint32_t)i0 + e;
          ++at;
        }
      }
      total = run;
      __syncthreads();
    }
    n_f = total;
    if (overflow) {
      z = z == -INFINITY ? 0.0f : z + 0.5f;
    } else if (total < (uint32_t)kB) {
      if (fkey == (1u << 15)) break;        // too few positive scores
      z = z - 1.0f < -3.0f ? -INFINITY : z - 1.0f;
    } else {
      ok = true;
    }
  }
  if (__builtin_expect(!ok, 0)) {
    select_row_global16<NT>(keys, c, kB, out, outs, hist, scratch, exact);
    if (tid == 0) a.cnt[row] = kB;
    return;
  }

  // ---- 3. the 16-bit threshold, then exact scores for the keys equal to it
  auto key = [&](int64_t i) { return ckey[pslot((uint32_t)i)]; };
  auto all = [&](int64_t) { return true; };
  const Radix r = radix_select<NT, true, 8>(key, all, (int64_t)n_f, (uint32_t)kB, hist, scratch, 0, 0u, 0u, 1);
  const bool band = r.need < r.avail;
  if (band) {
    // the band (keys equal to T) listed in hist: [0, nb) pool indices, then
    // [kBandMax, +nb) exact score bits, then [2 kBandMax, +nb) block ids
    uint32_t* blist = hist;
    uint32_t* bval = hist + kBandMax;
    uint32_t* bid = hist + 2 * kBandMax;
    uint32_t* bcount = &scratch[48];
    if (tid == 0) *bcount = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n_f; i += NT)
      if ((ckey[pslot(i)] & r.mask) == r.prefix) {
        const uint32_t at = atomicAdd(bcount, 1u);
        if (at < (uint32_t)kBandMax) blist[at] = i;
      }
    __syncthreads();
    const uint32_t nb = *bcount;
    if (__builtin_expect(nb > (uint32_t)kBandMax, 0)) {
      select_row_global16<NT>(keys, c, kB, out, outs, hist, scratch, exact);
      if (tid == 0) a.cnt[row] = kB;
      return;
    }
    // exact scores, one 16-lane group per band key: lane g16 takes dims
    // 8 g16 .. 8 g16 + 7 of the four heads; partial sums meet in lane 15
    {
      const int grp = tid >> 4, g16 = tid & 15;
      constexpr int NG = NT / 16;
      for (uint32_t e0 = 0; e0 < nb; e0 += 4 * NG) {
        u32x4 kw[4];
        uint32_t ent[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t e = e0 + (uint32_t)(grp + NG * q);
          ent[q] = e;
          const uint32_t b = e < nb ? cidx[pslot(blist[e])] : 0u;
          kw[q] = ld16(kseq + (int64_t)b * 128 + 8 * g16);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kv = bf16_to_f32((e & 1) ? (kw[q][e >> 1] >> 16) : (kw[q][e >> 1] & 0xFFFFu));
#pragma unroll
            for (int h = 0; h < 4; ++h) acc[h] = fmaf(qs[h * 128 + 8 * g16 + e], kv, acc[h]);
          }
#pragma unroll
          for (int h = 0; h < 4; ++h) acc[h] = row16_sum_to_last(acc[h]);  // the group's lane 15
          if (g16 == 15 && ent[q] < nb) {
            bval[ent[q]] = __float_as_uint(relu(acc[0]) + relu(acc[1]) + relu(acc[2]) + relu(acc[3]));
            bid[ent[q]] = cidx[pslot(blist[ent[q]])];
          }
        }
      }
    }
    __syncthreads();
    // rank inside the band: larger exact score first, then the lower index;
    // the r.need best are kept.  The ranks read only the band's own arrays,
    // so each member's pool slot is updated by its thread right away.
    for (uint32_t e = tid; e < nb; e += NT) {
      const uint32_t ve = bval[e];
      const uint32_t ie = bid[e];
      uint32_t rank = 0;
#pragma unroll 4
      for (uint32_t f = 0; f < nb; ++f) {
        const uint32_t vf = bval[f];
        const uint32_t iff = bid[f];
        rank += (vf > ve || (vf == ve && iff < ie)) ? 1u : 0u;
      }
      const uint32_t sl = pslot(blist[e]);
      ckey[sl] = ve;
      cidx[sl] = ie | kBand | (rank < r.need ? kBandKept : 0u);
    }
    __syncthreads();
  }

  // ---- 4. the ordered output ---------------------------------------------
  // With k_B <= 512 the kept ids and scores are staged by position in LDS
  // (hist and qs are free now) and written out in coalesced runs.
  constexpr bool kStage = CAP <= 3072;
  static_assert(!kStage || 3 * kBandMax >= 512, "staging room");
  uint32_t* ostage = hist;
  float* vstage = qs;
  uint32_t written = 0;
  for (uint32_t base = 0; base < n_f; base += 16 * NT) {
    const uint32_t i0 = base + 16 * tid;
    uint32_t take = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t i = i0 + e;
      if (i < n_f) {
        const uint32_t sl = pslot(i);
        const uint32_t k = ckey[sl], x = cidx[sl];
        const uint32_t m = k & r.mask;
        const bool keep = (x & kBand) ? (x & kBandKept) != 0u : (m > r.prefix || (!band && m == r.prefix));
        if (keep) take |= 1u << e;
      }
    }
    uint32_t tot;
    uint32_t pos = written + block_excl_scan<NT>((uint32_t)__popc(take), scratch, &tot);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (take & (1u << e)) {
        const uint32_t sl = pslot(i0 + e);
        const uint32_t x = cidx[sl];
        const float v = (x & kBand) ? __uint_as_float(ckey[sl]) : key16_value(ckey[sl]);
        if constexpr (kStage) {
          if (pos < (uint32_t)kB) {
            ostage[pos] = x & kIdxMask;
            vstage[pos] = v;
          }
        } else {
          out[pos] = (int32_t)(x & kIdxMask);
          if (outs) outs[pos] = v;
        }
        ++pos;
      }
    written += tot;
  }
  if constexpr (kStage) {
    __syncthreads();
    for (int i = tid; i < kB; i += NT) {
      out[i] = (int32_t)ostage[i];
      if (outs) outs[i] = vstage[i];
    }
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
  p.sseg = p.kernel == 0 ? 256 : (p.kernel == 1 ? 2048 : kDecodeScoreSeg);
  p.n_sseg = (c_max + p.sseg - 1) / p.sseg;
  const int64_t rows = (int64_t)batch * n_q;
  // The prefill tiles write whole 64-query x 64-block chunks: pad each
  // sequence's rows to 64 queries and each row to 64 blocks.
  p.nq_pad = p.kernel == 1 ? ((int64_t)n_q + 63) / 64 * 64 : n_q;
  if (p.kernel == 1) p.W = (p.W + 63) / 64 * 64;
  // Prefill rows are selected by streaming them once: no histograms.
  p.resident = p.kernel == 1 && c_max <= kStreamMax;
  if (rows >= 256 || c_max <= kFilterSeg) {
    p.fseg = p.n_sseg;          // score segments per filter workgroup
    p.n_fseg = 1;
  } else {
    p.fseg = max((int64_t)1, kFilterSeg / p.sseg);
    p.n_fseg = (p.n_sseg + p.fseg - 1) / p.fseg;
  }
  auto align = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t key_bytes = p.resident ? sizeof(uint16_t) : sizeof(float);
  size_t off = align(key_bytes * (size_t)batch * (size_t)p.nq_pad * (size_t)p.W);
  p.off_hist = off;
  if (!p.resident) off = align(off + sizeof(uint32_t) * (size_t)rows * p.n_sseg * kHistWords);
  p.off_slots = off;
  if (p.n_fseg > 1) off = align(off + sizeof(uint2) * (size_t)rows * kCandCap);
  p.off_slotcnt = off;
  p.off_done = off;
  off = align(off + sizeof(uint32_t) * (size_t)rows);
  p.bytes = off;
  return p;
}

hipError_t launch_select(const Dims& d, const SelectPlan& pl, int batch, int n_q,
                         const int32_t* q_pos0, int64_t cap, void* workspace, int32_t* sel,
                         int32_t* cnt, float* sel_scores, const void* q_idx, const void* k_cmp,
                         hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  FilterArgs a;
  a.scores = reinterpret_cast<const float*>(ws);
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.k_cmp = static_cast<const uint16_t*>(k_cmp);
  a.W = pl.W;
  a.hist = reinterpret_cast<const uint32_t*>(ws + pl.off_hist);
  a.sseg = pl.sseg;
  a.n_sseg = pl.n_sseg;
  a.cand = reinterpret_cast<uint2*>(ws + pl.off_slots);
  a.done = reinterpret_cast<uint32_t*>(ws + pl.off_done);
  a.spw = pl.fseg;
  a.n_fseg = pl.n_fseg;
  a.n_q = n_q;
  a.nq_pad = pl.nq_pad;
  a.q_pos0 = q_pos0;
  a.cap_blocks = cap / d.r;
  a.lr = d.lr;
  a.kB = d.kB;
  a.sel = sel;
  a.cnt = cnt;
  a.sel_scores = sel_scores;
  dim3 grid((unsigned)((int64_t)batch * n_q), (unsigned)pl.n_fseg);
  if (pl.resident) {
    const dim3 g((unsigned)((int64_t)batch * n_q));
    const bool big = d.kB > 512;   // the token-level budgets (r < 4)
    if (pl.W <= kRowShortMax && !big)
      hipLaunchKernelGGL((select_row_kernel<256, 4, false, 1, kRowCap>), g, dim3(256), 0, st, a);
    else if (!big)
      hipLaunchKernelGGL((select_row_kernel<256, 4, true, 1, kRowCap>), g, dim3(256), 0, st, a);
    else if (pl.W <= kRowShortMax)
      hipLaunchKernelGGL((select_row_kernel<256, 2, false, 1, kRowCapBig>), g, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((select_row_kernel<256, 2, true, 1, kRowCapBig>), g, dim3(256), 0, st, a);
  } else if (pl.n_fseg > 1 && pl.sseg <= 1024 && pl.fseg <= kWaves)
    hipLaunchKernelGGL(filter_select_kernel<true>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(filter_select_kernel<false>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qsa
