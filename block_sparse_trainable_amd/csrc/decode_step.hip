// One decode step of a QSA layer in a single launch: block compression of
// the block the new token completes, block scoring, top-k_B selection and
// sparse attention with its split merge.
//
// "QSA (Qwen Sparse Attention)", Key math / How it works: (A) compressed
// lightweight indexer (block compression, I_ib = sum_h ReLU(<q^h, k_b>) over
// complete earlier blocks, top-k_B blocks expanded to tokens plus the tail)
// and (B) sparse core attention over those tokens; the concept page's "Why
// it matters" reports the decode phase at long context.  "Qwen Sparse
// Attention" gallery page, How block selection works.
//
// The arithmetic is that of qsa_index_build + qsa_select_topk (n_q = 1) +
// qsa_sparse_attn_decode -- the same device code (compress_block.h, the
// decode scoring MFMA layout, select_common.h, attn_tile.h) -- so the results
// are bit-identical to those three calls.  What differs is the hand-off
// between the stages: instead of kernel boundaries (each of which costs a
// few microseconds and drains the GPU), workgroups hand data to each other
// through the workspace with coherent (agent-scope) accesses, each hand-off
// a single coalesced round trip:
//
//   score workgroups (row, segment of 1024 blocks; a row's last segment also
//   takes a remainder of up to 512, so 65,5xx-block rows need 64 of them)
//     - MFMA scores of the segment (the decode scoring kernel's layout), then
//       a counting sort of the segment's (score, id) pairs by histogram bin,
//       highest bin first, staged in LDS and stored whole, with the
//       segment's suffix counts cum[b] = #scores with bin >= b, which are
//       also added (atomically) into the row's suffix counts;
//     - the last workgroup of a row to finish (completion counter) selects:
//       the row's suffix counts give the threshold bin d*, each segment's
//       candidates (bin >= d*) are a prefix of its sorted list (all fetched
//       at once), an MSB radix select finds the exact threshold among bin d*,
//       equal scores go to the lower id (a second radix select over the
//       ids), and an id bitmap with prefix popcounts ranks the kept ids in
//       ascending order.  It writes the outputs and the row's selection
//       record: entry i = id_i + 1 for i < count, NONE for count <= i <= k_B;
//   attention workgroups (row, split of 32 pseudo-blocks), last in the grid
//     - split 0 first compresses the block the new token completes (not a
//       candidate of this step: the candidates are blocks < floor(p/4));
//     - load the query, then poll the record entries of the split (and the
//       one before it) until all are written -- the entries themselves are
//       the ready signal; the first NONE marks the tail pseudo-block;
//     - attend over the split, store the split state; the last split to
//       finish clears the record and merges the states (log-sum-exp).
//
// Forward progress: a score workgroup never waits, and a launch holds at most
// as many attention workgroups (which wait) as the device keeps resident
// minus 64 (measured occupancy x CUs; larger batches are split over several
// launches), so they cannot crowd out the score workgroups: every score
// workgroup is eventually resident and every record is eventually written.
// The spin is bounded all the same; on expiry the workgroup records an error
// word in the workspace and proceeds (wrong values, no hang).
//
// The control area at the start of the workspace must be zero-filled before
// its first use; every completed call leaves it zero.
#include <atomic>

#include "attn_tile.h"
#include "compress_block.h"
#include "select_common.h"

namespace qsa {
namespace {

constexpr int kNT = 256;
constexpr int kNW = kNT / 64;
constexpr int kCpw = 2;                          // 64-block chunks per wave per round
constexpr int kRoundBlocks = kNW * kCpw * 64;    // 512
constexpr int kMaxRounds = kStepSegMax / kRoundBlocks;  // 3
constexpr int kPerThread = kStepSegMax / kNT;    // 6 scores per thread in the sort
constexpr int kFCap = 4096;                      // candidates held in LDS
constexpr int kGatherPT = kFCap / kNT;           // 16 candidate loads per thread
constexpr int kDirect = kNT;                     // bin-d* sets ranked directly (<= kNT)
constexpr int kSegArr = 2 * kNT;                 // per-segment arrays (>= kStepMaxSegs)
constexpr uint32_t kNone = 0xFFFFFFFFu;          // record entry past the count
constexpr uint32_t kSpinLimit = 1u << 22;
static_assert(kStepMaxSegs <= kSegArr, "segment arrays");
static_assert(kMaxRounds * kRoundBlocks == kStepSegMax, "segments are whole rounds");
static_assert(kStepRecStride >= 512 + 1, "record holds k_B + 1 entries");

// LDS carve-up of the selection role (bytes)
constexpr int kOffKey = 0;
constexpr int kOffIdx = kOffKey + 4 * kFCap;
constexpr int kOffBm = kOffIdx + 4 * kFCap;
constexpr int kOffRh = kOffBm + 4 * kStepBmWords;
constexpr int kOffSegLen = kOffRh + 4 * kRadixBins;
constexpr int kOffSegOff = kOffSegLen + 4 * kSegArr;
constexpr int kOffTbase = kOffSegOff + 4 * kSegArr;
constexpr int kOffScr = kOffTbase + 4 * kNT;
constexpr int kSelLds = kOffScr + 4 * 64;
// score role (aliases the start of the selection area)
constexpr int kOffSc = 0;                           // float [kStepSegMax]
constexpr int kOffBins = kOffSc + 4 * kStepSegMax;  // u32 [256]
constexpr int kOffCurs = kOffBins + 4 * 256;        // u32 [256]
constexpr int kOffSorted = kOffCurs + 4 * 256;      // u64 [kStepSegMax]
static_assert(kOffSorted + 8 * kStepSegMax <= kOffRh, "score role fits below the radix area");

struct StepArgs {
  const uint16_t* q_idx;  // [B][4][128]
  const uint16_t* q;      // [B][16][D]
  const uint16_t* k_idx;  // [B][cap][128]
  uint16_t* k_cmp;        // [B][cap/4][128]
  const float* gain;
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t cap, cap_blocks, c_cap;
  const int32_t* q_pos;
  int kB;
  double base, eps;
  int rope_dims;
  float scale_log2;
  int32_t* sel;
  int32_t* cnt;
  float* sel_scores;
  uint16_t* out;
  float* lse;
  uint32_t* rowcnt;   // [B] score arrivals
  uint32_t* attncnt;  // [B] split arrivals
  uint32_t* err;
  uint32_t* rec;      // [B][kStepRecStride] selection records
  uint2* pairs;       // [B][n_seg][kStepSegMax]
  uint32_t* cum;      // [B][n_seg][128]  (u16 pairs: bins 2w, 2w+1)
  uint32_t* acc;      // [B][256] row suffix counts, summed by the segments (control area)
  float* part;        // [B][n_split][part_floats(D)]
  int n_seg, n_split, n_score_wg;
};

__device__ __forceinline__ int64_t row_c(const StepArgs& a, int s) {
  const int64_t p = max((int64_t)a.q_pos[s], (int64_t)0);
  return min(p / 4, a.c_cap);
}

__device__ __forceinline__ unsigned long long pack_pair(uint32_t key, uint32_t id) {
  return (unsigned long long)key | ((unsigned long long)id << 32);
}

__device__ __forceinline__ uint32_t cum_field(unsigned long long v, int e) {
  return (uint32_t)(v >> (16 * e)) & 0xFFFFu;
}

// ------------------------------------------------------------- selection ----
// Ranks through the id bitmap bm (a set bit per kept id).  After
// bitmap_prefix, pre[G] (u16) is the number of kept ids below word 4G, so the
// rank of a kept id -- the number of kept ids below it -- takes the group
// prefix, at most three whole words and one masked word, all independent
// reads.  Each thread sums its contiguous run of wpt words (a multiple of 4,
// read 16 bytes at a time; nwords is a multiple of 4, the bitmap cleared up
// to it).
__device__ __forceinline__ void bitmap_prefix(const uint32_t* bm, uint16_t* pre, uint32_t* scr,
                                              int nwords, int wpt) {
  const int w0 = (int)threadIdx.x * wpt, w1 = min(w0 + wpt, nwords);
  uint32_t pc = 0;
  for (int w = w0; w < w1; w += 4) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(bm + w);
    pc += __popc(q[0]) + __popc(q[1]) + __popc(q[2]) + __popc(q[3]);
  }
  uint32_t tot;
  uint32_t run = block_excl_scan<kNT>(pc, scr, &tot);
  for (int w = w0; w < w1; w += 4) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(bm + w);
    pre[w >> 2] = (uint16_t)run;
    run += __popc(q[0]) + __popc(q[1]) + __popc(q[2]) + __popc(q[3]);
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t bitmap_rank(const uint32_t* bm, const uint16_t* pre,
                                                uint32_t id) {
  const int w = (int)(id >> 5);
  const int g0 = w & ~3;
  uint32_t rank = pre[w >> 2] + __popc(bm[w] & ((1u << (id & 31u)) - 1u));
  rank += (g0 + 0 < w) ? __popc(bm[g0 + 0]) : 0u;
  rank += (g0 + 1 < w) ? __popc(bm[g0 + 1]) : 0u;
  rank += (g0 + 2 < w) ? __popc(bm[g0 + 2]) : 0u;
  return rank;
}

// Selects row s (run by the row's last score workgroup); writes sel, cnt,
// sel_scores and the row's record.
__device__ __forceinline__ void select_row(const StepArgs& a, int s, int64_t c, int nseg_row,
                           unsigned char* smem) {
  const int tid = threadIdx.x;
  uint32_t* ckey = reinterpret_cast<uint32_t*>(smem + kOffKey);
  uint32_t* cidx = reinterpret_cast<uint32_t*>(smem + kOffIdx);
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem + kOffBm);
  uint32_t* rh = reinterpret_cast<uint32_t*>(smem + kOffRh);
  uint32_t* seglen = reinterpret_cast<uint32_t*>(smem + kOffSegLen);
  uint32_t* segoff = reinterpret_cast<uint32_t*>(smem + kOffSegOff);
  uint32_t* scr = reinterpret_cast<uint32_t*>(smem + kOffScr);
  uint16_t* pre = reinterpret_cast<uint16_t*>(rh);  // bitmap group prefixes (after the radix)
  uint32_t* o_id = seglen;     // staged output (after the gather)
  uint32_t* o_key = segoff;
  const int kB = a.kB;
  int32_t* out = a.sel + (int64_t)s * kB;
  float* outs = a.sel_scores ? a.sel_scores + (int64_t)s * kB : nullptr;
  uint32_t* rec = a.rec + (int64_t)s * kStepRecStride;
  const unsigned long long* prow =
      reinterpret_cast<const unsigned long long*>(a.pairs) + (int64_t)s * a.n_seg * kStepSegMax;

  uint32_t* racc = a.acc + (int64_t)s * 256;
  if (c <= kB) {  // every candidate is kept; they all sit in segment 0
    coherent_store(&racc[tid], 0u);  // leave the row's counts zeroed
    for (int i = tid; i < c; i += kNT) {
      const unsigned long long v = coherent_load(&prow[i]);
      o_key[(uint32_t)(v >> 32)] = (uint32_t)v;
    }
    __syncthreads();
    for (int i = tid; i <= kB; i += kNT) {
      if (i < kB) {
        out[i] = i < c ? i : -1;
        if (outs) outs[i] = i < c ? __uint_as_float(o_key[i]) : 0.0f;
      }
      coherent_store(&rec[i], i < c ? (uint32_t)i + 1u : kNone);
    }
    if (tid == 0) a.cnt[s] = (int32_t)c;
    return;
  }

  // ---- 1. row suffix counts S(b), summed by the segments as they finished,
  // and in the same round trip the first P entries of every segment's list
  // (P = 64, 32 or 16 as the segments number up to 64, 128 or 256): a
  // segment's candidates lead its list, and there are rarely more than P.
  const int lp = nseg_row <= 64 ? 6 : (nseg_row <= 128 ? 5 : 4);
  const bool pre_ok = nseg_row <= kFCap / 16;
  const uint32_t nslot = pre_ok ? (uint32_t)nseg_row << lp : 0u;
  const uint32_t S_t = coherent_load(&racc[tid]);  // thread t: bin t
  unsigned long long pv[kGatherPT];
#pragma unroll
  for (int u = 0; u < kGatherPT; ++u) {  // unconditional: past the slots, slot 0 again
    const uint32_t i = (uint32_t)tid + (uint32_t)kNT * u;
    const uint32_t ic = i < nslot ? i : 0u;
    pv[u] = coherent_load(&prow[(int64_t)(ic >> lp) * kStepSegMax + (ic & ((1u << lp) - 1u))]);
  }
  {
    coherent_store(&racc[tid], 0u);                   // leave the row's counts zeroed
    rh[1024 + tid] = S_t;
    __syncthreads();
    const uint32_t S_next = tid < 255 ? rh[1024 + tid + 1] : 0u;
    if (S_t >= (uint32_t)kB && S_next < (uint32_t)kB) {  // S(0) = c > k_B: one such bin
      scr[8] = (uint32_t)tid;
      scr[9] = S_next;
      scr[10] = S_t;
    }
    __syncthreads();
  }
  const uint32_t dstar = scr[8];
  const uint32_t n_sure = scr[9];
  const uint32_t total = scr[10];
  const uint32_t n_maybe = total - n_sure;
  const uint32_t need = (uint32_t)kB - n_sure;
  // ---- 2. the candidates (bin >= d*) in LDS, slots [0, N) of ckey/cidx --
  // fast: the loaded prefixes, when they hold all S(d*) candidates (each
  // segment's candidates lead its prefix; the other slots hold entries below
  // d*); else gathered: the first cum[g][d*] entries of every segment's list,
  // packed.
  bool fast = false, gathered = false;
  uint32_t N = 0;
  if (pre_ok) {
    uint32_t ncand = 0;
#pragma unroll
    for (int u = 0; u < kGatherPT; ++u) {
      const uint32_t i = (uint32_t)tid + (uint32_t)kNT * u;
      ckey[i] = (uint32_t)pv[u];
      cidx[i] = (uint32_t)(pv[u] >> 32);
      ncand += (i < nslot && score_bin((uint32_t)pv[u]) >= dstar) ? 1u : 0u;
    }
    uint32_t nloaded;
    (void)block_excl_scan<kNT>(ncand, scr, &nloaded);
    fast = nloaded == total;
    N = nslot;
  }
  const int nwords = (int)((c + 127) / 128) * 4;          // whole groups of 4 words
  const int wpt = (nwords + 4 * kNT - 1) / (4 * kNT) * 4;  // contiguous words per thread
  if (!fast) {
    {
      const uint32_t* crow32 = a.cum + (int64_t)s * a.n_seg * 128;
      for (int g = tid; g < nseg_row; g += kNT) {
        const uint32_t w = coherent_load(&crow32[(int64_t)g * 128 + (dstar >> 1)]);
        seglen[g] = (dstar & 1u) ? (w >> 16) : (w & 0xFFFFu);
      }
    }
    __syncthreads();
    {
      const uint32_t v0 = 2 * tid < nseg_row ? seglen[2 * tid] : 0u;
      const uint32_t v1 = 2 * tid + 1 < nseg_row ? seglen[2 * tid + 1] : 0u;
      uint32_t tot;
      const uint32_t ex = block_excl_scan<kNT>(v0 + v1, scr, &tot);
      segoff[2 * tid] = ex;
      segoff[2 * tid + 1] = ex + v0;
      __syncthreads();
    }
    if (total <= (uint32_t)kFCap) {
      // Slot i (< total <= 4096) belongs to the last segment starting at or
      // before it: mark each non-empty segment at its first slot, take a
      // running max over the slots (16 consecutive per thread, then across
      // threads), then issue every slot's load at once.
      uint32_t* tab = cidx;  // slot -> segment, overwritten by the ids below
      for (int i = 4 * tid; i < kFCap; i += 4 * kNT)  // every slot: segments stay in range
        *reinterpret_cast<u32x4*>(tab + i) = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
      for (int g = tid; g < nseg_row; g += kNT)
        if (seglen[g] != 0u) tab[segoff[g]] = (uint32_t)g;
      __syncthreads();
      uint32_t run[kGatherPT];
      uint32_t mx = 0u;
#pragma unroll
      for (int u = 0; u < kGatherPT; u += 4) {
        const u32x4 t4 = *reinterpret_cast<const u32x4*>(tab + kGatherPT * tid + u);
        run[u] = t4[0];
        run[u + 1] = t4[1];
        run[u + 2] = t4[2];
        run[u + 3] = t4[3];
      }
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u) run[u] = mx = max(mx, run[u]);
      // exclusive max over the threads before this one (segments only grow)
      {
        const int lane = tid & 63, wave = tid >> 6;
        const uint32_t incl = wave_incl_max(mx);
        if (lane == 63) scr[20 + wave] = incl;
        __syncthreads();
        uint32_t before = __shfl_up(incl, 1);
        if (lane == 0) before = 0u;
#pragma unroll
        for (int w = 0; w < kNW; ++w)
          if (w < wave) before = max(before, scr[20 + w]);
#pragma unroll
        for (int u = 0; u < kGatherPT; ++u) run[u] = max(run[u], before);
      }
      unsigned long long v[kGatherPT];
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u) {
        const uint32_t i = (uint32_t)(kGatherPT * tid + u);
        const uint32_t g = run[u];
        v[u] = i < total ? coherent_load(&prow[(int64_t)g * kStepSegMax + (i - segoff[g])]) : 0ull;
      }
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u) {
        const uint32_t i = (uint32_t)(kGatherPT * tid + u);
        if (i < total) {
          ckey[i] = (uint32_t)v[u];
          cidx[i] = (uint32_t)(v[u] >> 32);
        }
      }
      gathered = true;
      N = total;
    }
  }

  if (fast || gathered) {
    for (int w = 4 * tid; w < nwords; w += 4 * kNT)  // nwords: a multiple of 4
      *reinterpret_cast<u32x4*>(bm + w) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    // ---- 3. exact choice among the bin-d* candidates -------------------------
    // need of the n_maybe candidates in bin d* are kept: the largest scores,
    // equal scores to the lower id.  Packed as (key << 32 | ~id), that order
    // is the integer order of distinct 64-bit values.  Up to kDirect of them
    // are ranked directly (rank = number of larger packed values); larger
    // sets go through an MSB radix select, then one over the ids for ties.
    // Slots below d* (fast path only) are never eligible.
    const bool some = need < n_maybe;  // else every bin-d* candidate is kept
    const bool direct = some && n_maybe <= (uint32_t)kDirect;
    Radix r{0u, 0u, need, need}, r2{0u, 0u, 0u, 0u};
    if (direct) {
      unsigned long long* mk = reinterpret_cast<unsigned long long*>(rh);  // [kDirect + 16]
      uint32_t* mslot = rh + 2 * (kDirect + 16);                           // [kDirect]
      uint32_t cm = 0;
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)kNT * u;
        cm += (i < N && score_bin(ckey[i]) == dstar) ? 1u : 0u;
      }
      uint32_t tot;
      uint32_t pos = block_excl_scan<kNT>(cm, scr, &tot);
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)kNT * u;
        if (i < N && score_bin(ckey[i]) == dstar) {
          mk[pos] = ((unsigned long long)ckey[i] << 32) | (0x7FFFFFFFu - cidx[i]);
          mslot[pos] = i;
          ++pos;
        }
      }
      // pad to a multiple of 16 with values below every member
      if (tid < 16) mk[n_maybe + tid] = 0ull;
      __syncthreads();
      if (tid < (int)n_maybe) {
        const unsigned long long me = mk[tid];
        uint32_t rank = 0;
        for (uint32_t j = 0; j < n_maybe; j += 16) {  // 16 broadcast reads in flight
          unsigned long long w[16];
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(mk + j + e);
            w[e] = (unsigned long long)q[0] | ((unsigned long long)q[1] << 32);
            w[e + 1] = (unsigned long long)q[2] | ((unsigned long long)q[3] << 32);
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) rank += w[e] > me ? 1u : 0u;
        }
        if (rank < need) cidx[mslot[tid]] |= 0x80000000u;  // kept
      }
      __syncthreads();
    } else if (some) {
      auto key = [&](int64_t i) { return ckey[i]; };
      auto elig = [&](int64_t i) { return score_bin(ckey[i]) == dstar; };
      if (dstar > 0u && dstar < (uint32_t)kHistBins - 1u)
        r = radix_select<kNT, true>(key, elig, (int64_t)N, need, rh, scr, 1, (dstar + 888u) << 20,
                              0x7FFu << 20);
      else
        r = radix_select<kNT, true>(key, elig, (int64_t)N, need, rh, scr);
    }
    const bool tie = some && !direct && r.avail > r.need;
    if (tie) {  // equal scores at the threshold: the lowest ids win
      auto key2 = [&](int64_t i) { return 0x7FFFFFFFu - cidx[i]; };
      auto elig2 = [&](int64_t i) {
        return score_bin(ckey[i]) == dstar && (ckey[i] & r.mask) == r.prefix;
      };
      r2 = radix_select<kNT, true>(key2, elig2, (int64_t)N, r.need, rh, scr);
    }
    __syncthreads();
    // ---- 4. the kept entries, packed into slots [0, k_B) (all reads first,
    // then the branch-free choice), then in ascending order via an id bitmap
    {
      uint32_t kk[kGatherPT], kx[kGatherPT];
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)kNT * u;
        kk[u] = ckey[i];
        kx[u] = cidx[i];
      }
      uint32_t kmask = 0, nk = 0;
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)kNT * u;
        const uint32_t b = score_bin(kk[u]);
        const uint32_t m = kk[u] & r.mask;
        const bool won = direct ? (kx[u] >> 31) != 0u
                                : (m > r.prefix ||
                                   (m == r.prefix &&
                                    (!tie || ((0x7FFFFFFFu - kx[u]) & r2.mask) >= r2.prefix)));
        const bool kp = i < N && (b > dstar || (b == dstar && (!some || won)));
        kmask |= kp ? 1u << u : 0u;
        nk += kp ? 1u : 0u;
      }
      uint32_t nkept;
      uint32_t pos = block_excl_scan<kNT>(nk, scr, &nkept);  // reads above precede its barriers
#pragma unroll
      for (int u = 0; u < kGatherPT; ++u)
        if ((kmask >> u) & 1u) {
          ckey[pos] = kk[u];
          cidx[pos] = kx[u] & 0x7FFFFFFFu;
          ++pos;
        }
    }
    __syncthreads();
    constexpr int kPerT = 512 / kNT;  // kept entries per thread (k_B <= 512)
#pragma unroll
    for (int e = 0; e < kPerT; ++e) {
      const int i = tid + kNT * e;
      if (i < kB) {
        const uint32_t id = cidx[i];
        atomicOr(&bm[id >> 5], 1u << (id & 31u));
      }
    }
    __syncthreads();
    bitmap_prefix(bm, pre, scr, nwords, wpt);
#pragma unroll
    for (int e = 0; e < kPerT; ++e) {
      const int i = tid + kNT * e;
      if (i < kB) {
        const uint32_t id = cidx[i];
        const uint32_t rank = bitmap_rank(bm, pre, id);
        if (rank < (uint32_t)kB) {
          o_id[rank] = id;
          o_key[rank] = ckey[i];
        }
      }
    }
  } else {
    // ---- fallback: exact selection over the whole row ---------------------
    // Entry i of the row's c entries: segment min(i / 1024, last), whose
    // list holds that segment's entries at stride kStepSegMax.
    for (int w = 4 * tid; w < nwords; w += 4 * kNT)  // (published by the barriers below)
      *reinterpret_cast<u32x4*>(bm + w) = u32x4{0u, 0u, 0u, 0u};
    auto at = [&](int64_t i) {
      const int64_t g = min(i / kStepSeg, (int64_t)nseg_row - 1);
      return coherent_load(&prow[g * kStepSegMax + (i - g * kStepSeg)]);
    };
    auto key = [&](int64_t i) { return (uint32_t)at(i); };
    auto all = [&](int64_t) { return true; };
    const Radix r = radix_select<kNT>(key, all, c, (uint32_t)kB, rh, scr);
    const bool tie = r.avail > r.need;
    Radix r2{0u, 0u, 0u, 0u};
    if (tie) {
      auto key2 = [&](int64_t i) { return 0x7FFFFFFFu - (uint32_t)(at(i) >> 32); };
      auto elig2 = [&](int64_t i) { return (key(i) & r.mask) == r.prefix; };
      r2 = radix_select<kNT>(key2, elig2, c, r.need, rh, scr);
    }
    auto keep = [&](unsigned long long v) {
      const uint32_t m = (uint32_t)v & r.mask;
      if (m != r.prefix) return m > r.prefix;
      return !tie || ((0x7FFFFFFFu - (uint32_t)(v >> 32)) & r2.mask) >= r2.prefix;
    };
    __syncthreads();
    for (int64_t i = tid; i < c; i += kNT) {
      const unsigned long long v = at(i);
      const uint32_t id = (uint32_t)(v >> 32);
      if (keep(v)) atomicOr(&bm[id >> 5], 1u << (id & 31u));
    }
    __syncthreads();
    bitmap_prefix(bm, pre, scr, nwords, wpt);
    for (int64_t i = tid; i < c; i += kNT) {
      const unsigned long long v = at(i);
      if (!keep(v)) continue;
      const uint32_t rank = bitmap_rank(bm, pre, (uint32_t)(v >> 32));
      if (rank < (uint32_t)kB) {
        o_id[rank] = (uint32_t)(v >> 32);
        o_key[rank] = (uint32_t)v;
      }
    }
  }
  __syncthreads();
  // ---- 5. outputs and the record (coalesced) -------------------------------
  for (int i = tid; i <= kB; i += kNT) {
    if (i < kB) {
      out[i] = (int32_t)o_id[i];
      if (outs) outs[i] = __uint_as_float(o_key[i]);
    }
    coherent_store(&rec[i], i < kB ? o_id[i] + 1u : kNone);
  }
  if (tid == 0) a.cnt[s] = (int32_t)kB;
}

// ---------------------------------------------------------------- scoring ----
// Workgroup (row s, segment g): the scores of the segment's blocks, as the
// decode scoring kernel computes them (rows of the A tile = 4 x query +
// head; only query 0 is live), sorted by bin and stored.
__device__ __forceinline__ void score_segment(const StepArgs& a, int64_t wg, unsigned char* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const int s = (int)(wg / a.n_seg);
  const int g = (int)(wg % a.n_seg);
  const int64_t c = row_c(a, s);
  const int nseg_row = step_nseg(c);
  if (g >= nseg_row) return;  // not part of this row
  const int64_t seg_lo = (int64_t)g * kStepSeg;
  const int64_t seg_hi = (g == nseg_row - 1) ? c : seg_lo + kStepSeg;
  const int n_here = (int)max(seg_hi - seg_lo, (int64_t)0);
  float* sc = reinterpret_cast<float*>(smem + kOffSc);
  uint32_t* bins = reinterpret_cast<uint32_t*>(smem + kOffBins);
  uint32_t* curs = reinterpret_cast<uint32_t*>(smem + kOffCurs);
  unsigned long long* sorted = reinterpret_cast<unsigned long long*>(smem + kOffSorted);
  uint32_t* scr = reinterpret_cast<uint32_t*>(smem + kOffScr);
  bins[tid] = 0u;

  u32x4 qa[4];
  {
    const bool ok = l16 < 4;  // A row l16 = head l16 of the one query
    const uint16_t* src = a.q_idx + ((int64_t)s * 4 + (ok ? l16 : 0)) * 128 + 8 * gq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qa[kk] = ok ? ld16(src + 32 * kk) : u32x4{0, 0, 0, 0};
  }
  const uint16_t* kbase = a.k_cmp + (int64_t)s * a.cap_blocks * 128 + 8 * gq;
#pragma unroll
  for (int rd = 0; rd < kMaxRounds; ++rd) {
    if (rd * kRoundBlocks >= n_here) break;
    const int64_t rb = seg_lo + (int64_t)rd * kRoundBlocks;
    u32x4 kb[kCpw][4][4];
#pragma unroll
    for (int cc = 0; cc < kCpw; ++cc)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int64_t b = rb + 64 * (cc * kNW + wave) + 16 * ct + l16;
        const bool ok = b < seg_hi;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          kb[cc][ct][kk] = ok ? ld16(kbase + b * 128 + 32 * kk) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
    for (int cc = 0; cc < kCpw; ++cc)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[kk]),
                                                        as_bf16x8(kb[cc][ct][kk]), acc, 0, 0, 0);
        const int64_t b = rb + 64 * (cc * kNW + wave) + 16 * ct + l16;
        const float v = relu(acc[0]) + relu(acc[1]) + relu(acc[2]) + relu(acc[3]);
        if (gq == 0 && b < seg_hi) sc[b - seg_lo] = v;
      }
  }
  __syncthreads();

  // counting sort of the segment by bin, highest bin first, staged in LDS
  uint32_t key[kPerThread], bin[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = tid + kNT * e;
    key[e] = i < n_here ? __float_as_uint(sc[i]) : 0u;
    bin[e] = score_bin(key[e]);
    if (i < n_here) atomicAdd(&bins[bin[e]], 1u);
  }
  __syncthreads();
  {
    const uint32_t nb = bins[255 - tid];  // thread t owns bin 255 - t
    uint32_t tot;
    const uint32_t start = block_excl_scan<kNT>(nb, scr, &tot);
    curs[255 - tid] = start;
    bins[255 - tid] = start + nb;  // suffix count: scores with bin >= 255 - t
    // the row's suffix counts accumulate as the segments finish
    if (start + nb)
      __hip_atomic_fetch_add(&a.acc[(int64_t)s * 256 + 255 - tid], start + nb, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = tid + kNT * e;
    if (i < n_here)
      sorted[atomicAdd(&curs[bin[e]], 1u)] = pack_pair(key[e], (uint32_t)(seg_lo + i));
  }
  __syncthreads();
  unsigned long long* dst =
      reinterpret_cast<unsigned long long*>(a.pairs) + ((int64_t)s * a.n_seg + g) * kStepSegMax;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = tid + kNT * e;
    if (i < n_here) coherent_store(&dst[i], sorted[i]);
  }
  if (tid < 128)
    coherent_store(&a.cum[((int64_t)s * a.n_seg + g) * 128 + tid],
                   bins[2 * tid] | (bins[2 * tid + 1] << 16));
  stores_complete();
  __syncthreads();
  if (tid == 0) scr[12] = arrive_last(&a.rowcnt[s], (uint32_t)nseg_row) ? 1u : 0u;
  __syncthreads();
  if (scr[12] == 0u) return;
  if (tid == 0) coherent_store(&a.rowcnt[s], 0u);  // leave the counter zeroed
  select_row(a, s, c, nseg_row, smem);
}

// -------------------------------------------------------------- attention ----
template <int HKV, int D>
__device__ __forceinline__ void attend_split(const StepArgs& a, int64_t item, unsigned char* smem) {
  using S = MfmaShape<HKV, D>;
  constexpr int PF = part_floats(D);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = item / a.n_split;
  const int split = (int)(item % a.n_split);
  const int kB = a.kB;
  const int64_t p = min(max((int64_t)a.q_pos[row], (int64_t)0), a.cap - 1);
  const int64_t c = p / 4;
  uint32_t* scr = reinterpret_cast<uint32_t*>(smem + kOffScr);
  int32_t* sbid = reinterpret_cast<int32_t*>(smem + S::LDS_BYTES);
  uint32_t* rec = a.rec + row * kStepRecStride;
  const int pb_lo = split * kDecodeSplitPB;

  if (split == 0 && tid < 64) {  // the block the new token completes, if any
    const int64_t pr = a.q_pos[row];
    const int64_t lb = max(pr, (int64_t)0);
    const int64_t la = min(max(pr + 1, (int64_t)0), a.cap);
    const int64_t b_begin = lb / 4;
    const int64_t b_end = min(la / 4, a.cap_blocks);
    if (b_begin < b_end)
      compress_wave<true>(a.k_idx, a.cap, (int)row, b_begin, b_end, 1, a.gain, a.base, a.eps,
                          a.rope_dims, a.k_cmp, 2);  // blocks of 4 tokens
  }
  u32x4 qb[S::NK];
  load_qbd<HKV, D>(a.q, row, qb);  // in flight while the selection is made

  // wait for record entries pb_lo - 1 .. pb_lo + 31 (lane L <-> pb_lo - 1 + L);
  // the split's pseudo-blocks are [pb_lo, pb_hi), the first NONE the tail
  if (tid < 64) {
    const int e = pb_lo - 1 + lane;
    const bool mine = lane <= kDecodeSplitPB && e >= 0 && e <= kB;
    uint32_t v = (e < 0) ? 1u : kNone;  // before the record: "an id"; past it: NONE
    uint32_t n = 0;
    while (true) {
      if (mine) v = coherent_load(&rec[e]);
      if (__ballot(mine && v == 0u) == 0ull) break;
      if (++n >= kSpinLimit) {
        if (lane == 0) coherent_store(a.err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const unsigned long long none =
        __ballot(lane >= 1 && lane <= kDecodeSplitPB && v == kNone);
    int hi = pb_lo + kDecodeSplitPB;
    if (__shfl(v, 0) == kNone) hi = pb_lo;         // the count ends before this split
    else if (none) hi = pb_lo + (__ffsll(none) - 1);  // lane L holds the tail: pb_hi = pb_lo + L
    if (lane >= 1 && lane <= hi - pb_lo)
      sbid[lane - 1] = (v == kNone) ? (int32_t)c
                                    : (int32_t)min(max((int64_t)v - 1, (int64_t)0), c - 1);
    if (lane == 0) scr[13] = (uint32_t)hi;
  }
  __syncthreads();
  const int pb_hi = (int)scr[13];
  attn_mfma_tiles<HKV, D, true>(qb, a.kc, a.vc, a.cap, (int)row, p, row, item, pb_lo, pb_hi,
                                sbid, a.scale_log2, a.out, a.lse, a.part, a.n_split, smem);
  if (a.n_split == 1) {  // the split wrote the output itself; clear the record
    for (int i = tid; i <= kB; i += kNT) coherent_store(&rec[i], 0u);
    return;
  }
  stores_complete();
  __syncthreads();
  if (tid == 0) scr[12] = arrive_last(&a.attncnt[row], (uint32_t)a.n_split) ? 1u : 0u;
  __syncthreads();
  if (scr[12] == 0u) return;
  if (tid == 0) coherent_store(&a.attncnt[row], 0u);
  for (int i = tid; i <= kB; i += kNT) coherent_store(&rec[i], 0u);

  // ---- log-sum-exp merge of the splits (all loads coalesced): per head
  // M = max_k m_k, f_k = 2^(m_k - M), Z = sum_k f_k l_k once, then
  // O = sum_k f_k O_k per output -- lse_merge's expressions, in split order
  const float* base = a.part + row * a.n_split * PF;
  float* msz = reinterpret_cast<float*>(smem);  // [split][m 16, l 16]
  float* fac = msz + kMaxSplits * 32;           // [head][split]: f_k, or -1 when skipped
  float* hz = fac + 16 * kMaxSplits;            // [head] Z
  float* hm = hz + 16;                          // [head] M
  // (m, l) pairs of every split first, then the O values: the loads return
  // in order, so storing the pairs waits for them alone
  const int nmz = a.n_split * 16;
  unsigned long long mz[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + kNT * r;
    mz[r] = i < nmz ? coherent_load(reinterpret_cast<const unsigned long long*>(base + (i >> 4) * PF) + (i & 15))
                    : 0ull;
  }
  constexpr int NJ = 16 * D / 2 / kNT;  // float pairs per thread
  unsigned long long ov[NJ][kMaxSplits];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k)
      ov[jj][k] = k < a.n_split ? coherent_load(reinterpret_cast<const unsigned long long*>(
                                      base + k * PF + 32) + tid + kNT * jj)
                                : 0ull;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + kNT * r;  // splits past n_split read as zero (unused)
    if (i < kMaxSplits * 16) {
      const int k = i >> 4, w = i & 15;
      msz[k * 32 + 2 * w] = __uint_as_float((uint32_t)mz[r]);
      msz[k * 32 + 2 * w + 1] = __uint_as_float((uint32_t)(mz[r] >> 32));
    }
  }
  __syncthreads();
  if (tid < 16) {
    const int n = tid;
    float mk[kMaxSplits], lk[kMaxSplits];
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k) {  // (reads outside any condition)
      mk[k] = msz[k * 32 + n];
      lk[k] = msz[k * 32 + 16 + n];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k)
      if (k < a.n_split) mx = fmaxf(mx, mk[k]);
    float zs = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k) {
      float f = -1.0f;
      if (k < a.n_split && mk[k] != -INFINITY) {
        f = exp2f(mk[k] - mx);
        zs += f * lk[k];
      }
      fac[n * kMaxSplits + k] = f;
    }
    hz[n] = zs;
    hm[n] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int e2 = 2 * (tid + kNT * jj);  // first of the two floats
    const int n = e2 / D, d = e2 % D;
    float fk[kMaxSplits];
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k) fk[k] = fac[n * kMaxSplits + k];  // -1 past n_split
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k) {
      const float f = fk[k];
      if (f >= 0.0f) {
        acc0 += f * __uint_as_float((uint32_t)ov[jj][k]);
        acc1 += f * __uint_as_float((uint32_t)(ov[jj][k] >> 32));
      }
    }
    const float zs = hz[n];
    *reinterpret_cast<uint32_t*>(a.out + (row * 16 + n) * D + d) =
        f32_to_bf16(acc0 / zs) | (f32_to_bf16(acc1 / zs) << 16);
    if (a.lse && d == 0) a.lse[row * 16 + n] = (hm[n] + log2f(zs)) * kLn2;
  }
}

template <int HKV, int D>
constexpr int step_lds_bytes() {
  return (MfmaShape<HKV, D>::LDS_BYTES + 4 * kMaxPB > kSelLds)
             ? MfmaShape<HKV, D>::LDS_BYTES + 4 * kMaxPB
             : kSelLds;
}

template <int HKV, int D>
__global__ __launch_bounds__(kNT, 2) void decode_step_kernel(StepArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[step_lds_bytes<HKV, D>()];
  static_assert(MfmaShape<HKV, D>::LDS_BYTES + 4 * kMaxPB <= kOffScr,
                "attention LDS stays below the scratch words");
  const int64_t wg = blockIdx.x;
  if (wg < a.n_score_wg)
    score_segment(a, wg, smem);
  else
    attend_split<HKV, D>(a, wg - a.n_score_wg, smem);
}

}  // namespace

StepPlan step_plan(const Dims& d, int batch, int32_t max_pos_end) {
  StepPlan p{};
  p.c_max = max((int64_t)1, (int64_t)(max_pos_end - 1) / d.r);
  p.n_seg = step_nseg(p.c_max);
  p.n_split = (d.kB + 1 + kDecodeSplitPB - 1) / kDecodeSplitPB;
  auto align = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t off = align(kStepCtlBytes);
  p.off_pairs = off;
  off = align(off + sizeof(uint2) * (size_t)batch * p.n_seg * kStepSegMax);
  p.off_cum = off;
  off = align(off + sizeof(uint32_t) * (size_t)batch * p.n_seg * 128);
  p.off_part = off;
  off = align(off + sizeof(float) * (size_t)batch * p.n_split * part_floats(d.head_dim));
  p.bytes = off;
  return p;
}

bool decode_step_layout_ok(const Dims& d) {
  return d.bf16 && d.r == 4 && d.idx_heads == 4 && d.idx_dim == 128 && d.q_heads == 16 &&
         ((d.kv_heads == 2 && (d.head_dim == 64 || d.head_dim == 128)) ||
          (d.kv_heads == 1 && d.head_dim == 128));
}

// Workgroups of the fused kernel the current device keeps resident
// (occupancy x CUs), cached per device.
template <int HKV, int D>
int step_capacity() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cap = cache[dev].load(std::memory_order_relaxed);
  if (cap > 0) return cap;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_step_kernel<HKV, D>, kNT, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cap = per_cu * cus;
  cache[dev].store(cap, std::memory_order_relaxed);
  return cap;
}

hipError_t launch_decode_step(const Dims& d, const StepPlan& pl, int batch, const void* q_idx,
                              const void* q, const void* k_idx, void* k_cmp, const float* gain,
                              const void* k_cache, const void* v_cache, int64_t cap,
                              const int32_t* q_pos, int32_t* sel, int32_t* cnt,
                              float* sel_scores, void* out, float* lse, void* workspace,
                              hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  const int D = d.head_dim;
  const int64_t KD = (int64_t)d.kv_heads * D;
  const int64_t cap_blocks = cap / d.r;
  int capacity = 0;
  if (d.kv_heads == 2 && D == 128) capacity = step_capacity<2, 128>();
  else if (d.kv_heads == 1 && D == 128) capacity = step_capacity<1, 128>();
  else if (d.kv_heads == 2 && D == 64) capacity = step_capacity<2, 64>();
  if (capacity - 64 < pl.n_split) return hipErrorInvalidConfiguration;
  const int per_launch = max(1, (capacity - 64) / pl.n_split);
  for (int r0 = 0; r0 < batch; r0 += per_launch) {
    const int nb = min(per_launch, batch - r0);
    StepArgs a;
    a.q_idx = static_cast<const uint16_t*>(q_idx) + (int64_t)r0 * 4 * 128;
    a.q = static_cast<const uint16_t*>(q) + (int64_t)r0 * 16 * D;
    a.k_idx = static_cast<const uint16_t*>(k_idx) + (int64_t)r0 * cap * 128;
    a.k_cmp = static_cast<uint16_t*>(k_cmp) + (int64_t)r0 * cap_blocks * 128;
    a.gain = gain;
    a.kc = static_cast<const uint16_t*>(k_cache) + (int64_t)r0 * cap * KD;
    a.vc = static_cast<const uint16_t*>(v_cache) + (int64_t)r0 * cap * KD;
    a.cap = cap;
    a.cap_blocks = cap_blocks;
    a.c_cap = min(pl.c_max, cap_blocks);
    a.q_pos = q_pos + r0;
    a.kB = d.kB;
    a.base = d.base;
    a.eps = (double)d.eps;
    a.rope_dims = d.rope_dims;
    a.scale_log2 = d.scale * kLog2e;
    a.sel = sel + (int64_t)r0 * d.kB;
    a.cnt = cnt + r0;
    a.sel_scores = sel_scores ? sel_scores + (int64_t)r0 * d.kB : nullptr;
    a.out = static_cast<uint16_t*>(out) + (int64_t)r0 * 16 * D;
    a.lse = lse ? lse + (int64_t)r0 * 16 : nullptr;
    uint32_t* ctl = reinterpret_cast<uint32_t*>(ws);
    a.rowcnt = ctl + r0;
    a.attncnt = ctl + kStepOffAttn + r0;
    a.err = ctl + kStepOffErr;
    a.rec = ctl + kStepOffRec + (int64_t)r0 * kStepRecStride;
    a.pairs = reinterpret_cast<uint2*>(ws + pl.off_pairs) + (int64_t)r0 * pl.n_seg * kStepSegMax;
    a.cum = reinterpret_cast<uint32_t*>(ws + pl.off_cum) + (int64_t)r0 * pl.n_seg * 128;
    a.acc = ctl + kStepOffAcc + (int64_t)r0 * 256;
    a.part = reinterpret_cast<float*>(ws + pl.off_part) + (int64_t)r0 * pl.n_split * part_floats(D);
    a.n_seg = pl.n_seg;
    a.n_split = pl.n_split;
    a.n_score_wg = nb * pl.n_seg;
    const dim3 grid((unsigned)(nb * (pl.n_seg + pl.n_split)));
    bool launched = false;
#define QSA_STEP(HKV, DD)                                                              \
    if (!launched && d.kv_heads == HKV && d.head_dim == DD) {                          \
      hipLaunchKernelGGL((decode_step_kernel<HKV, DD>), grid, dim3(kNT), 0, st, a);    \
      launched = true;                                                                 \
    }
    QSA_STEP(2, 128)
    QSA_STEP(1, 128)
    QSA_STEP(2, 64)
#undef QSA_STEP
    if (!launched) return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qsa
