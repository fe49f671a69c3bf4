// One decode step of a QSA layer in a single launch: block compression of
// the block the new token completes, block scoring, top-k_B selection and
// sparse attention with its split merge.
//
// "QSA (Qwen Sparse Attention)", Key math / How it works: (A) the compressed
// indexer (block compression, I_ib = sum_h ReLU(<q^h, k_b>) over complete
// earlier blocks, top-k_B blocks expanded to tokens plus the tail) and (B)
// softmax attention over those tokens only; the concept page's "Why it
// matters" reports the decode phase at long context.  "Qwen Sparse
// Attention" gallery page, How block selection works.
//
// The arithmetic is that of qsa_index_build + qsa_select_topk (n_q = 1) +
// qsa_sparse_attn_decode -- the same device code (compress_block.h, the
// decode scoring MFMA layout, select_common.h, attn_tile.h) and the same
// split partition and merge order -- so the results are bit-identical to
// those three calls.  What differs is the hand-off between the stages.
//
// A row (one sequence's new token) is served by the workgroups of its score
// segments (1024 blocks each; the last one also takes a remainder of up to
// 512):
//   P1 every workgroup scores its segment with MFMA, sorts the (score, id)
//      pairs by score bin (256 monotone bins, highest first), stores them
//      with the segment's suffix counts cum[b] = #scores with bin >= b, adds
//      those counts into the row's, and raises its flag.  Workgroups past
//      the first kDecodeSplits leave here.
//   P2 the first min(n_seg, kDecodeSplits) workgroups wait for every flag of
//      the row; then each derives the selection by itself: the threshold bin
//      d* from the row's counts, every segment's number of entries above and
//      at d* (its entries with bin >= d* head its sorted list), all of those
//      entries at once, which bin-d* ones are kept -- the largest scores,
//      equal scores to the lower id -- and each kept id's position (its rank
//      among the kept ids).  It writes the positions its attention splits
//      cover and the splits' block lists;
//   P3 it attends that split (the token set cut into kDecodeSplits runs of
//      pseudo-blocks), stores the split's (m, l, O) state and raises the
//      split's flag;
//   P4 up to 16 of them wait for every split flag and merge one head each
//      (log-sum-exp, in split order) into the output.
// So a row crosses two waits: one after scoring, one before the merge.  A
// wait is a poll of the row's flags (one load per flag, all in flight), not
// a shared counter: arrivals are plain stores and never queue on one address.
//
// A flag holds the epoch of the call that raised it: the row's generation
// word plus one.  Every workgroup of the row reads the generation word when
// it starts; workgroup 0 advances it once all scoring flags are up (so every
// reader has read it), and flags never need clearing.  The row's score-bin
// counts alternate between two buffers by epoch parity; workgroup 0 clears
// the one the row's next call will use.
//
// Forward progress: a row's workgroups are consecutive in the grid and the
// dispatcher starts workgroups in grid order.  Only the row's first
// kDecodeSplits workgroups wait, and only for workgroups of their own row,
// which either run (scoring never waits) or are next to start once a slot
// frees.  Every wait is bounded all the same; on expiry the workgroup sets
// the error word in the workspace and proceeds (wrong values, no hang).
//
// The control area at the start of the workspace must be zero-filled before
// the first call.  Between calls it holds the generation words, flags and
// counts; zero-filling it again between calls is always allowed (and needed
// after a call that set the error word).
#include <atomic>

#include "attn_tile.h"
#include "compress_block.h"
#include "select_common.h"

namespace qsa {
namespace {

constexpr int kNT = 256;
constexpr int kNW = kNT / 64;
constexpr int kCpw = 1;                          // 64-block chunks per wave per round
constexpr int kRoundBlocks = kNW * kCpw * 64;    // 256
constexpr int kMaxRounds = kStepSegMax / kRoundBlocks;  // 6
constexpr int kPerThread = kStepSegMax / kNT;    // 6 scores per thread in the sort
constexpr int kMaxKB = 512;                      // k_B of the fused step
constexpr int kFlatCap = 2560;                   // entries with bin >= d* held by a workgroup
constexpr int kFPT = kFlatCap / kNT;             // 10 per thread
constexpr int kMkCap = kFlatCap;                 // boundary-group entries ranked in LDS
constexpr int kGroupPT = kMkCap / kNT;           // 10 per thread
constexpr int kSegArr = 2 * kNT;                 // per-segment arrays (>= kStepMaxSegs)
constexpr int kMaxRunPB = 32;                    // pseudo-blocks of one split (>= P)
constexpr int kFlagPerLane = (kStepFaStride + 63) / 64;
constexpr uint32_t kSpinLimit = 1u << 22;
static_assert(kStepMaxSegs <= kSegArr && kStepMaxSegs <= kStepFaStride, "segment arrays");
static_assert(kDecodeSplits <= kStepFcStride, "split flags");
static_assert(kMaxRounds * kRoundBlocks == kStepSegMax, "segments are whole rounds");
static_assert(decode_pb_per_split(kMaxKB + 1) <= kMaxRunPB, "split size");
static_assert(kFlatCap % kNT == 0 && kMkCap % kNT == 0, "per-thread shares");

// LDS carve-up (bytes).  Scoring: scores, bin counts, sorted pairs.  The
// selection reuses that room once scoring is over (a row with c <= k_B
// keeps its scores for the outputs and never selects).
constexpr int kOffSc = 0;                                // float [kStepSegMax] scores
constexpr int kOffBins = kOffSc + 4 * kStepSegMax;       // u32 [256]: this segment's suffix counts
constexpr int kOffCurs = kOffBins + 4 * 256;             // u32 [256]
constexpr int kOffSorted = kOffCurs + 4 * 256;           // u64 [kStepSegMax] (key, id) by bin
constexpr int kOffFseg = 0;                              // u32 [kFlatCap] list slot -> segment
constexpr int kOffMk = kOffFseg + 4 * kFlatCap;          // u64 [kMkCap + 16] boundary group
constexpr int kOffRh = kOffMk + 8 * (kMkCap + 16);       // u32 [kRadixBins] radix / sub-bins
constexpr int kOffHi = kOffRh + 4 * kRadixBins;          // u32 [kSegArr] per segment: bin > d*
constexpr int kOffEq = kOffHi + 4 * kSegArr;             // u32 [kSegArr] ... bin == d*
constexpr int kOffFo = kOffEq + 4 * kSegArr;             // u32 [kSegArr] ... list offsets
constexpr int kOffSFirst = kOffFo + 4 * kSegArr;         // u32 [kSegArr] ... first kept index
constexpr int kOffSLast = kOffSFirst + 4 * kSegArr;      // u32 [kSegArr] ... last kept index
constexpr int kOffKId = kOffSLast + 4 * kSegArr;         // u32 [kMaxKB] kept ids
constexpr int kOffKKey = kOffKId + 4 * kMaxKB;           // u32 [kMaxKB] ... their keys
constexpr int kOffKSeg = kOffKKey + 4 * kMaxKB;          // u32 [kMaxKB] ... their segments
constexpr int kOffScr = kOffKSeg + 4 * kMaxKB;           // u32 [64] scratch
constexpr int kSelLds = kOffScr + 4 * 64;

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
  uint32_t* gen;      // [kStepMaxBatch] per-row generation             (control area)
  uint32_t* fa;       // [kStepMaxBatch][kStepFaStride] scoring flags   (control)
  uint32_t* fc;       // [kStepMaxBatch][kStepFcStride] split flags     (control)
  uint32_t* err;      //                                                (control)
  uint32_t* acc;      // [kStepMaxBatch][2][256] row suffix counts      (control)
  uint2* pairs;       // [B][n_seg][kStepSegMax]
  uint32_t* cum;      // [B][n_seg][128]  (u16 pairs: bins 2w, 2w+1)
  float* part;        // [B][kDecodeSplits][part_floats(D)]
  int n_seg, pb_per_split;
};

__device__ __forceinline__ int64_t row_c(const StepArgs& a, int s) {
  const int64_t p = max((int64_t)a.q_pos[s], (int64_t)0);
  return min(p / 4, a.c_cap);
}

__device__ __forceinline__ unsigned long long pack_pair(uint32_t key, uint32_t id) {
  return (unsigned long long)key | ((unsigned long long)id << 32);
}

// Wave 0 polls flags[0 .. n) (n <= kStepFaStride) until each holds epoch,
// bounded (on expiry the error word is set); the barrier after it releases
// the workgroup.
__device__ __forceinline__ void wait_flags(const StepArgs& a, const uint32_t* flags, int n,
                                           uint32_t epoch) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint32_t spins = 0;
    while (true) {
      uint32_t v[kFlagPerLane];
#pragma unroll
      for (int u = 0; u < kFlagPerLane; ++u) {
        const int i = lane + 64 * u;
        v[u] = i < n ? coherent_load(&flags[i]) : epoch;
      }
      bool up = true;
#pragma unroll
      for (int u = 0; u < kFlagPerLane; ++u) up = up && v[u] == epoch;
      if (__ballot(!up) == 0ull) break;
      if (++spins >= kSpinLimit) {
        if (lane == 0) coherent_store(a.err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Suffix count of bin b (0..256) from a segment's packed cum words.
__device__ __forceinline__ uint32_t cum_at(const uint32_t* words, uint32_t b) {
  if (b >= 256u) return 0u;
  const uint32_t w = coherent_load(&words[b >> 1]);
  return (b & 1u) ? (w >> 16) : (w & 0xFFFFu);
}

// ---------------------------------------------------------------- P1 -------
// Scores of the segment's blocks, as the decode scoring kernel computes them
// (rows of the A tile = 4 x query + head; only query 0 is live), sorted by
// bin, stored, their suffix counts added into the row's (acc_row), and the
// segment's flag raised.  Leaves the scores in sc.
__device__ __forceinline__ void score_segment(const StepArgs& a, int s, int g, int64_t c,
                                              int nseg_row, uint32_t* acc_row, uint32_t epoch,
                                              unsigned char* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
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
  // rounds are software-pipelined: the next round's B-tile loads are in
  // flight while this round's MFMAs run
  auto load_round = [&](int rd, u32x4 (&kb)[kCpw][4][4]) {
    const int64_t rb = seg_lo + (int64_t)rd * kRoundBlocks;
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
  };
  u32x4 kn[kCpw][4][4];
  if (n_here > 0) load_round(0, kn);
#pragma unroll
  for (int rd = 0; rd < kMaxRounds; ++rd) {
    if (rd * kRoundBlocks >= n_here) break;
    const int64_t rb = seg_lo + (int64_t)rd * kRoundBlocks;
    u32x4 kb[kCpw][4][4];
#pragma unroll
    for (int cc = 0; cc < kCpw; ++cc)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kb[cc][ct][kk] = kn[cc][ct][kk];
    if (rd + 1 < kMaxRounds && (rd + 1) * kRoundBlocks < n_here) load_round(rd + 1, kn);
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
      __hip_atomic_fetch_add(&acc_row[255 - tid], start + nb, __ATOMIC_RELAXED,
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
  if (tid == 0) coherent_store(&a.fa[(int64_t)s * kStepFaStride + g], epoch);
}

// ---------------------------------------------------------------- P2 -------
// The selection of a row with c > k_B candidates, derived by each waiting
// workgroup from every segment's published counts and pairs:
//   * d* from the row's suffix counts S(b): S(d*) >= k_B > S(d*+1);
//   * per segment, hi (entries above d*) and eq (at d*) from its cum words;
//     its entries with bin >= d* are the first hi + eq of its sorted list,
//     and all of them (fewer than k_B + kGCap) are loaded at once, thread t
//     holding kFPT consecutive ones of the row's list in segment order;
//   * the need = k_B - S(d*+1) largest bin-d* entries are kept (equal
//     scores to the lower id): a 256-bin histogram of the next 8 key bits
//     finds the sub-bin t* that holds the boundary, and only t*'s entries
//     are ranked one against another;
//   * the kept entries, compacted in list order, are grouped by segment in
//     ascending segment order, so a kept id's position in the selection is
//     its segment's first index there plus its rank by id within the segment.
// If the entries with bin >= d* do not fit (bin d* holds thousands of
// equal scores), an exact radix select over the whole row decides instead.
// Writes the selection outputs for the positions of this workgroup's splits
// and their block lists (sball: split kl's list at kl * P).
__device__ __forceinline__ void select_runs(const StepArgs& a, int s, int g, int64_t c,
                                            int nseg_row, int nsw, const uint32_t* acc_row,
                                            int32_t* sball, unsigned char* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kB = a.kB;
  const int P = a.pb_per_split;
  const int count = kB;  // c > k_B
  uint32_t* fseg = reinterpret_cast<uint32_t*>(smem + kOffFseg);
  unsigned long long* mk = reinterpret_cast<unsigned long long*>(smem + kOffMk);
  uint32_t* rh = reinterpret_cast<uint32_t*>(smem + kOffRh);
  uint32_t* hi = reinterpret_cast<uint32_t*>(smem + kOffHi);
  uint32_t* eq = reinterpret_cast<uint32_t*>(smem + kOffEq);
  uint32_t* fo = reinterpret_cast<uint32_t*>(smem + kOffFo);
  uint32_t* kid = reinterpret_cast<uint32_t*>(smem + kOffKId);
  uint32_t* kkey = reinterpret_cast<uint32_t*>(smem + kOffKKey);
  uint32_t* kseg = reinterpret_cast<uint32_t*>(smem + kOffKSeg);
  uint32_t* sfirst = reinterpret_cast<uint32_t*>(smem + kOffSFirst);
  uint32_t* slast = reinterpret_cast<uint32_t*>(smem + kOffSLast);
  uint32_t* scr = reinterpret_cast<uint32_t*>(smem + kOffScr);
  const unsigned long long* prow =
      reinterpret_cast<const unsigned long long*>(a.pairs) + (int64_t)s * a.n_seg * kStepSegMax;

  // ---- the threshold bin from the row's suffix counts S(b) -------------------
  if (tid == 0) {  // defaults, kept only if the counts are inconsistent
    scr[8] = 0u;
    scr[9] = 0u;
    scr[10] = (uint32_t)c;
    scr[12] = 0u;  // kept entries (fallback)
    scr[13] = 0u;  // boundary entries
    scr[16] = 0u;  // t*
    scr[17] = 0u;  // entries above t*
    scr[18] = 0u;  // entries in t*
  }
  {
    const uint32_t S_t = coherent_load(&acc_row[tid]);  // thread t: bin t
    rh[tid] = S_t;
    __syncthreads();
    const uint32_t S_next = tid < 255 ? rh[tid + 1] : 0u;
    if (S_t >= (uint32_t)kB && S_next < (uint32_t)kB) {  // S(0) = c > k_B: one such bin
      scr[8] = (uint32_t)tid;
      scr[9] = S_next;
      scr[10] = S_t;
    }
    __syncthreads();
  }
  const uint32_t dstar = scr[8];
  const uint32_t n_sure = scr[9];
  const uint32_t n_maybe = scr[10] - min(n_sure, scr[10]);
  const uint32_t need = (uint32_t)kB - min(n_sure, (uint32_t)kB);
  const bool all_eq = need >= n_maybe;

  // ---- every segment's entries above and at d*, and their list offsets ------
  const uint32_t* crow = a.cum + (int64_t)s * a.n_seg * 128;
  for (int i = tid; i < nseg_row; i += kNT) {
    const uint32_t* cw = crow + (int64_t)i * 128;
    const uint32_t above = min(cum_at(cw, dstar + 1u), (uint32_t)kStepSegMax);
    const uint32_t at = cum_at(cw, dstar);
    hi[i] = above;
    eq[i] = min(at - min(at, above), (uint32_t)kStepSegMax - above);
  }
  __syncthreads();
  uint32_t total;
  {  // two segments per thread
    const uint32_t v0 = 2 * tid < nseg_row ? hi[2 * tid] + eq[2 * tid] : 0u;
    const uint32_t v1 = 2 * tid + 1 < nseg_row ? hi[2 * tid + 1] + eq[2 * tid + 1] : 0u;
    const uint32_t ex = block_excl_scan<kNT>(v0 + v1, scr, &total);
    fo[2 * tid] = ex;
    fo[2 * tid + 1] = ex + v0;
    __syncthreads();
  }
  const bool fallback = total > (uint32_t)kFlatCap;

  // this workgroup's block lists start valid, whatever happens below
  for (int k = g, kl = 0; k < kDecodeSplits; k += nsw, ++kl)
    for (int i = tid; i < P; i += kNT) sball[kl * P + i] = 0;
  uint32_t nk;

  if (!fallback) {
    // ---- load the list: slot f belongs to the last segment starting at or
    // before it (marks, then a running max over the slots, consecutive per
    // thread), then every slot's load at once
    for (int i = tid; i < kFlatCap; i += kNT) fseg[i] = 0u;
    __syncthreads();
    for (int i = tid; i < nseg_row; i += kNT)
      if (hi[i] + eq[i] != 0u && fo[i] < (uint32_t)kFlatCap) fseg[fo[i]] = (uint32_t)i;
    __syncthreads();
    uint32_t run[kFPT];
    uint32_t mx = 0u;
#pragma unroll
    for (int u = 0; u < kFPT; ++u) run[u] = mx = max(mx, fseg[kFPT * tid + u]);
    {  // exclusive max over the threads before this one (segments only grow)
      const uint32_t incl = wave_incl_max(mx);
      if (lane == 63) scr[20 + wave] = incl;
      __syncthreads();
      uint32_t before = __shfl_up(incl, 1);
      if (lane == 0) before = 0u;
#pragma unroll
      for (int w = 0; w < kNW; ++w)
        if (w < wave) before = max(before, scr[20 + w]);
#pragma unroll
      for (int u = 0; u < kFPT; ++u) run[u] = max(run[u], before);
    }
    unsigned long long v[kFPT];
#pragma unroll
    for (int u = 0; u < kFPT; ++u) {
      const uint32_t f = (uint32_t)(kFPT * tid + u);
      const uint32_t sg = run[u];
      const uint32_t at = min(f - min(f, fo[sg]), (uint32_t)kStepSegMax - 1u);
      v[u] = f < total ? coherent_load(&prow[(int64_t)sg * kStepSegMax + at]) : 0ull;
    }
    // class of slot u: 2 kept for sure (bin > d*), 1 at d*, 0 empty
    uint32_t cls[kFPT];
#pragma unroll
    for (int u = 0; u < kFPT; ++u) {
      const uint32_t f = (uint32_t)(kFPT * tid + u);
      const uint32_t b = score_bin((uint32_t)v[u]);
      cls[u] = f >= total ? 0u : (b > dstar ? 2u : (b == dstar ? 1u : 0u));
    }
    if (!all_eq) {
      // ---- the boundary sub-bin t* of bin d*: bits 19..12 of the key order
      // the bin's entries (bits 30..20 are the bin); the end bins, which
      // clamp, go whole to the ranking instead
      const bool split_bin = dstar > 0u && dstar < (uint32_t)kHistBins - 1u;
      uint32_t tstar = 0u, above = 0u, m = n_maybe;
      if (split_bin) {
        rh[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kFPT; ++u)
          if (cls[u] == 1u) atomicAdd(&rh[((uint32_t)v[u] >> 12) & 255u], 1u);
        __syncthreads();
        const uint32_t nb = rh[255 - tid];  // thread t: sub-bin 255 - t
        uint32_t tot;
        const uint32_t ex = block_excl_scan<kNT>(nb, scr, &tot);  // entries above it
        if (ex + nb >= need && ex < need) {
          scr[16] = 255u - (uint32_t)tid;
          scr[17] = ex;
          scr[18] = nb;
        }
        __syncthreads();
        tstar = scr[16];
        above = scr[17];
        m = scr[18];
      }
      const uint32_t need2 = need - min(above, need);
      // slot u is in the boundary group: at d*, and in t* when the bin splits
      auto in_group = [&](int u) {
        return cls[u] == 1u && (!split_bin || (((uint32_t)v[u] >> 12) & 255u) == tstar);
      };
      uint32_t qidx[kFPT];
      const bool rank_group = m > need2;  // else every group entry is kept
      if (rank_group) {
        // gather the group, packed (key << 32 | ~id) so that the integer
        // order of distinct entries is the selection order; slots in thread
        // order (one scan, no chain of atomics)
        uint32_t ng = 0;
#pragma unroll
        for (int u = 0; u < kFPT; ++u) ng += in_group(u) ? 1u : 0u;
        uint32_t n_all;
        uint32_t q = block_excl_scan<kNT>(ng, scr, &n_all);
#pragma unroll
        for (int u = 0; u < kFPT; ++u) {
          const bool want = in_group(u);
          qidx[u] = q;
          q += want ? 1u : 0u;
          if (want && qidx[u] < (uint32_t)kMkCap)
            mk[qidx[u]] = (v[u] << 32) | (0x7FFFFFFFu - (uint32_t)(v[u] >> 32));
        }
        __syncthreads();
        const uint32_t n = min(n_all, (uint32_t)kMkCap);
        if (n <= (uint32_t)kNT) {  // pairwise ranks
          if (tid < 16) mk[n + tid] = 0ull;  // pad with values below every member
          __syncthreads();
          const unsigned long long me = tid < (int)n ? mk[tid] : ~0ull;
          uint32_t rank = 0;
          for (uint32_t j = 0; j < n; j += 16) {  // 16 broadcast reads in flight
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
          __syncthreads();
          if (tid < (int)n && rank < need2) mk[tid] |= 0x80000000ull;  // kept mark
        } else {
          auto key = [&](int64_t i) { return (uint32_t)(mk[i] >> 32); };
          auto all = [&](int64_t) { return true; };
          Radix r;
          if (split_bin)
            r = radix_select<kNT, true>(key, all, (int64_t)n, need2, rh, scr, 1,
                                        (dstar + 888u) << 20, 0x7FFu << 20);
          else
            r = radix_select<kNT, true>(key, all, (int64_t)n, need2, rh, scr);
          const bool tie = r.avail > r.need;
          Radix r2{0u, 0u, 0u, 0u};
          if (tie) {  // equal scores at the threshold: the lowest ids win
            auto key2 = [&](int64_t i) { return (uint32_t)mk[i] & 0x7FFFFFFFu; };
            auto elig2 = [&](int64_t i) { return (key(i) & r.mask) == r.prefix; };
            r2 = radix_select<kNT, true>(key2, elig2, (int64_t)n, r.need, rh, scr);
          }
          __syncthreads();
          bool won[kGroupPT];
#pragma unroll
          for (int e = 0; e < kGroupPT; ++e) {
            const uint32_t i = (uint32_t)(tid + kNT * e);
            won[e] = false;
            if (i < n) {
              const uint32_t mm = key(i) & r.mask;
              won[e] = mm > r.prefix ||
                       (mm == r.prefix &&
                        (!tie || (((uint32_t)mk[i] & 0x7FFFFFFFu) & r2.mask) >= r2.prefix));
            }
          }
          __syncthreads();
#pragma unroll
          for (int e = 0; e < kGroupPT; ++e)
            if (won[e]) mk[tid + kNT * e] |= 0x80000000ull;
        }
        __syncthreads();
      }
#pragma unroll
      for (int u = 0; u < kFPT; ++u) {
        if (cls[u] != 1u) continue;
        const uint32_t sb = ((uint32_t)v[u] >> 12) & 255u;
        bool keep;
        if (split_bin && sb != tstar) keep = sb > tstar;
        else keep = !rank_group || (qidx[u] < (uint32_t)kMkCap && (mk[qidx[u]] & 0x80000000ull));
        cls[u] = keep ? 2u : 0u;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kFPT; ++u)
        if (cls[u] == 1u) cls[u] = 2u;
    }
    // ---- the kept entries in list order (grouped by segment, ascending)
    uint32_t mine = 0;
#pragma unroll
    for (int u = 0; u < kFPT; ++u) mine += cls[u] == 2u ? 1u : 0u;
    uint32_t tot;
    uint32_t o = block_excl_scan<kNT>(mine, scr, &tot);
#pragma unroll
    for (int u = 0; u < kFPT; ++u)
      if (cls[u] == 2u) {
        if (o < (uint32_t)kMaxKB) {
          kid[o] = (uint32_t)(v[u] >> 32);
          kkey[o] = (uint32_t)v[u];
          kseg[o] = run[u];
        }
        ++o;
      }
    nk = min(tot, (uint32_t)kMaxKB);
  } else {
    // ---- fallback: exact selection over the whole row ---------------------
    // Entry i of the row's c entries: segment min(i / 1024, last), whose
    // list holds that segment's entries at stride kStepSegMax.
    auto seg_of = [&](int64_t i) { return min(i / kStepSeg, (int64_t)nseg_row - 1); };
    auto at = [&](int64_t i) {
      const int64_t sg = seg_of(i);
      return coherent_load(&prow[sg * kStepSegMax + (i - sg * kStepSeg)]);
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
    __syncthreads();
    // the kept entries all have bin >= d*: stream those (segment j's list
    // range [fo[j], fo[j] + hi[j] + eq[j])), appended in any order
    for (uint32_t f = tid; f < total; f += kNT) {
      int lo = 0, up = nseg_row - 1;  // the last segment with fo <= f
      while (lo < up) {
        const int mid = (lo + up + 1) >> 1;
        if (fo[mid] <= f) lo = mid;
        else up = mid - 1;
      }
      const uint32_t at_ = min(f - fo[lo], (uint32_t)kStepSegMax - 1u);
      const unsigned long long e = coherent_load(&prow[(int64_t)lo * kStepSegMax + at_]);
      const uint32_t mm = (uint32_t)e & r.mask;
      const bool k = mm != r.prefix
                         ? mm > r.prefix
                         : (!tie || ((0x7FFFFFFFu - (uint32_t)(e >> 32)) & r2.mask) >= r2.prefix);
      if (k) {
        const uint32_t q = atomicAdd(&scr[12], 1u);
        if (q < (uint32_t)kMaxKB) {
          kid[q] = (uint32_t)(e >> 32);
          kkey[q] = (uint32_t)e;
          kseg[q] = 0u;  // one group: ranked over all kept ids
        }
      }
    }
    __syncthreads();
    nk = min(scr[12], (uint32_t)kMaxKB);
  }
  __syncthreads();

  // ---- positions: first index of the id's segment group + rank within it ----
  for (uint32_t i = tid; i < nk; i += kNT) {
    const uint32_t sg = kseg[i];
    if (i == 0u || kseg[i - 1] != sg) sfirst[sg] = i;
    if (i + 1u == nk || kseg[i + 1] != sg) slast[sg] = i;
  }
  __syncthreads();
  int32_t* outsel = a.sel + (int64_t)s * kB;
  float* outsc = a.sel_scores ? a.sel_scores + (int64_t)s * kB : nullptr;
  // quotients by P and nsw as products with their reciprocals: exact for
  // these small operands (pos < 2^10), with half a step of margin
  const float inv_p = 1.0f / (float)P;
  const float inv_nsw = 1.0f / (float)nsw;
  for (uint32_t i = tid; i < nk; i += kNT) {
    const uint32_t id = kid[i];
    const uint32_t sg = kseg[i];
    const uint32_t lo = sfirst[sg], up = slast[sg];
    uint32_t pos = lo;
    uint32_t j = lo;
    for (; j + 3u <= up; j += 4u)  // four reads in flight
      pos += (kid[j] < id ? 1u : 0u) + (kid[j + 1] < id ? 1u : 0u) + (kid[j + 2] < id ? 1u : 0u) +
             (kid[j + 3] < id ? 1u : 0u);
    for (; j <= up; ++j) pos += kid[j] < id ? 1u : 0u;
    if (pos >= (uint32_t)count) continue;
    const int k = (int)(((float)pos + 0.5f) * inv_p);
    const int kl = (int)(((float)k + 0.5f) * inv_nsw);
    if (k - kl * nsw != g) continue;  // another workgroup's split
    sball[kl * P + ((int)pos - k * P)] = (int32_t)min((int64_t)id, c - 1);
    outsel[pos] = (int32_t)id;
    if (outsc) outsc[pos] = __uint_as_float(kkey[i]);
  }
  if (tid == 0)  // the tail block c ends the token set
    for (int k = g, kl = 0; k < kDecodeSplits; k += nsw, ++kl)
      if (k * P <= count && count < k * P + P) sball[kl * P + (count - k * P)] = (int32_t)c;
  __syncthreads();
}

// ------------------------------------------------------------ P2 + P3 ------
// LDS past the selection's (and the attention tiles') room: the block lists
// of a workgroup's splits, then the row's main query (loaded at the start).
template <int HKV, int D>
constexpr int sbid_offset() {
  return MfmaShape<HKV, D>::LDS_BYTES > kSelLds ? MfmaShape<HKV, D>::LDS_BYTES : kSelLds;
}
template <int HKV, int D>
constexpr int q_offset() {
  return sbid_offset<HKV, D>() + 4 * kDecodeSplits * kMaxRunPB;
}

// load_qbd from the query staged in LDS (16 heads x D).
template <int HKV, int D>
__device__ __forceinline__ void load_qbd_lds(const uint16_t* qs,
                                             u32x4 (&qb)[MfmaShape<HKV, D>::NK]) {
  using S = MfmaShape<HKV, D>;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const int gn = l16 / S::G;
#pragma unroll
  for (int kk = 0; kk < S::NK; ++kk) {
    const int dim0 = 32 * kk + 8 * gq;
    const int grp = dim0 / D;
    qb[kk] = (grp == gn) ? *reinterpret_cast<const u32x4*>(qs + l16 * D + (dim0 - grp * D))
                         : u32x4{0, 0, 0, 0};
  }
}

// Split k of the row's token set: pseudo-blocks [k P, min((k+1) P, npb)),
// the selected blocks then the tail block c.  Workgroup g takes splits
// g, g + nsw, ...; their block lists are all built before any attention
// (the attention reuses the selection's LDS).
template <int HKV, int D>
__device__ __forceinline__ void select_and_attend(const StepArgs& a, int s, int g, int64_t c,
                                                  int nseg_row, int nsw, const uint32_t* acc_row,
                                                  uint32_t epoch, unsigned char* smem) {
  using S = MfmaShape<HKV, D>;
  const int tid = threadIdx.x;
  const int kB = a.kB;
  const int64_t p = min(max((int64_t)a.q_pos[s], (int64_t)0), a.cap - 1);
  const int count = (int)min((int64_t)kB, c);
  const int npb = count + 1;  // r = 4: the tail is one pseudo-block
  const int P = a.pb_per_split;
  int32_t* sball = reinterpret_cast<int32_t*>(smem + sbid_offset<HKV, D>());
  const uint16_t* qs = reinterpret_cast<const uint16_t*>(smem + q_offset<HKV, D>());

  wait_flags(a, a.fa + (int64_t)s * kStepFaStride, nseg_row, epoch);
  if (g == 0 && tid == 0) {  // every workgroup of the row has read the generation
    coherent_store(&a.gen[s], epoch);
    a.cnt[s] = count;
  }

  if (c <= kB) {  // every candidate is kept: the row has one segment, its scores in sc
    const float* sc = reinterpret_cast<const float*>(smem + kOffSc);
    int32_t* outsel = a.sel + (int64_t)s * kB;
    float* outsc = a.sel_scores ? a.sel_scores + (int64_t)s * kB : nullptr;
    for (int i = tid; i < kB; i += kNT) {
      outsel[i] = i < c ? i : -1;
      if (outsc) outsc[i] = i < c ? sc[i] : 0.0f;
    }
    int kl = 0;
    for (int k = g; k < kDecodeSplits; k += nsw, ++kl)
      for (int pb = k * P + tid; pb < min(k * P + P, npb); pb += kNT)
        sball[kl * P + (pb - k * P)] = pb < count ? pb : (int32_t)c;
    __syncthreads();
  } else {
    select_runs(a, s, g, c, nseg_row, nsw, acc_row, sball, smem);
  }

  u32x4 qb[S::NK];
  load_qbd_lds<HKV, D>(qs, qb);
  int kl = 0;
  for (int k = g; k < kDecodeSplits; k += nsw, ++kl) {
    const int pb_lo = k * P;
    const int pb_hi = min(pb_lo + P, npb);
    if (pb_lo >= pb_hi) {  // an empty split: the state attn_mfma_tiles leaves for no token
      float* po = a.part + ((int64_t)s * kDecodeSplits + k) * part_floats(D);
      for (int i = tid; i < part_floats(D); i += kNT)
        coherent_store(&po[i], i < 16 ? -INFINITY : 0.0f);
      continue;
    }
    attn_mfma_tiles<HKV, D, true>(qb, a.kc, a.vc, a.cap, s, p, s,
                                  (int64_t)s * kDecodeSplits + k, pb_lo, pb_hi, sball + kl * P,
                                  a.scale_log2, a.out, a.lse, a.part, kDecodeSplits, smem);
    __syncthreads();  // the tiles' LDS is reused by the next split
  }
  stores_complete();
  __syncthreads();
  if (tid == 0)
    for (int k = g; k < kDecodeSplits; k += nsw)
      coherent_store(&a.fc[(int64_t)s * kStepFcStride + k], epoch);
}

// ---------------------------------------------------------------- P4 -------
// Head h of the output: the log-sum-exp merge of the row's splits, in split
// order (lse_merge_splits, as the stand-alone merge kernel).
template <int D>
__device__ __forceinline__ void merge_heads(const StepArgs& a, int s, int g, int nsw,
                                            uint32_t epoch, unsigned char* smem) {
  constexpr int PF = part_floats(D);
  const int nm = min(nsw, 16);
  if (g >= nm) return;
  const int tid = threadIdx.x;
  wait_flags(a, a.fc + (int64_t)s * kStepFcStride, kDecodeSplits, epoch);
  float* ml = reinterpret_cast<float*>(smem);  // [2 * kDecodeSplits] per pass
  const float* base = a.part + (int64_t)s * kDecodeSplits * PF;
  for (int h = g; h < 16; h += nm) {
    for (int i = tid; i < 2 * kDecodeSplits; i += kNT)
      ml[i] = coherent_load(&base[(i >> 1) * PF + 16 * (i & 1) + h]);
    float o[kDecodeSplits];
    const int dd = tid < D ? tid : 0;
#pragma unroll
    for (int k = 0; k < kDecodeSplits; ++k) o[k] = coherent_load(&base[k * PF + 32 + h * D + dd]);
    __syncthreads();
    if (tid < D) {
      float mx, zs, acc;
      lse_merge_splits(ml, o, mx, zs, acc);
      a.out[((int64_t)s * 16 + h) * D + tid] = (uint16_t)f32_to_bf16(acc / zs);
      if (a.lse && tid == 0) a.lse[(int64_t)s * 16 + h] = (mx + log2f(zs)) * kLn2;
    }
    __syncthreads();
  }
}

template <int HKV, int D>
constexpr int step_lds_bytes() {
  return q_offset<HKV, D>() + 2 * 16 * D;
}

// The block the new token completes, if any: not a candidate of this step
// (candidates are the blocks before the query's own), so it is built off the
// critical path by the row's last workgroup.
__device__ __forceinline__ void compress_new_block(const StepArgs& a, int s) {
  if (threadIdx.x >= 64) return;
  const int64_t pr = a.q_pos[s];
  const int64_t lb = max(pr, (int64_t)0);
  const int64_t la = min(max(pr + 1, (int64_t)0), a.cap);
  const int64_t b_begin = lb / 4;
  const int64_t b_end = min(la / 4, a.cap_blocks);
  if (b_begin < b_end)
    compress_wave<true>(a.k_idx, a.cap, s, b_begin, b_end, 1, a.gain, a.base, a.eps, a.rope_dims,
                        a.k_cmp, 2);  // blocks of 4 tokens
}

template <int HKV, int D>
__global__ __launch_bounds__(kNT, 2) void decode_step_kernel(StepArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[step_lds_bytes<HKV, D>()];
  const int s = (int)(blockIdx.x / (unsigned)a.n_seg);
  const int g = (int)(blockIdx.x % (unsigned)a.n_seg);
  const int64_t c = row_c(a, s);
  const int nseg_row = step_nseg(c);
  if (g >= nseg_row) return;  // not part of this row
  const int tid = threadIdx.x;
  const int nsw = min(nseg_row, kDecodeSplits);  // the row's waiting workgroups
  const uint32_t epoch = coherent_load(&a.gen[s]) + 1u;
  uint32_t* acc_row = a.acc + ((int64_t)s * 2 + (epoch & 1u)) * 256;
  if (g == 0)  // the counts the row's next call adds into
    coherent_store(&a.acc[((int64_t)s * 2 + ((epoch & 1u) ^ 1u)) * 256 + tid], 0u);
  if (g < nsw && tid < 2 * D) {  // the main query, for the attention at the end
    uint16_t* qs = reinterpret_cast<uint16_t*>(smem + q_offset<HKV, D>());
    *reinterpret_cast<u32x4*>(qs + 8 * tid) = ld16(a.q + (int64_t)s * 16 * D + 8 * tid);
  }
  score_segment(a, s, g, c, nseg_row, acc_row, epoch, smem);
  if (g >= nsw) {
    if (g == nseg_row - 1) compress_new_block(a, s);
    return;
  }
  __syncthreads();
  select_and_attend<HKV, D>(a, s, g, c, nseg_row, nsw, acc_row, epoch, smem);
  merge_heads<D>(a, s, g, nsw, epoch, smem);
  if (g == nseg_row - 1) compress_new_block(a, s);
}

}  // namespace

StepPlan step_plan(const Dims& d, int batch, int32_t max_pos_end) {
  StepPlan p{};
  p.c_max = max((int64_t)1, (int64_t)(max_pos_end - 1) / d.r);
  p.n_seg = step_nseg(p.c_max);
  p.n_split = kDecodeSplits;
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
  int capacity = 0;
  if (d.kv_heads == 2 && D == 128) capacity = step_capacity<2, 128>();
  else if (d.kv_heads == 1 && D == 128) capacity = step_capacity<1, 128>();
  else if (d.kv_heads == 2 && D == 64) capacity = step_capacity<2, 64>();
  // a row's waiting workgroups (at most kDecodeSplits, on the 8 XCDs in
  // turn) plus one more slot on every XCD must fit
  if (capacity / 8 < (kDecodeSplits + 7) / 8 + 1) return hipErrorInvalidConfiguration;
  StepArgs a;
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.q = static_cast<const uint16_t*>(q);
  a.k_idx = static_cast<const uint16_t*>(k_idx);
  a.k_cmp = static_cast<uint16_t*>(k_cmp);
  a.gain = gain;
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.cap = cap;
  a.cap_blocks = cap / d.r;
  a.c_cap = min(pl.c_max, a.cap_blocks);
  a.q_pos = q_pos;
  a.kB = d.kB;
  a.base = d.base;
  a.eps = (double)d.eps;
  a.rope_dims = d.rope_dims;
  a.scale_log2 = d.scale * kLog2e;
  a.sel = sel;
  a.cnt = cnt;
  a.sel_scores = sel_scores;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  uint32_t* ctl = reinterpret_cast<uint32_t*>(ws);
  a.gen = ctl + kStepOffGen;
  a.err = ctl + kStepOffErr;
  a.fc = ctl + kStepOffFc;
  a.fa = ctl + kStepOffFa;
  a.acc = ctl + kStepOffAcc;
  a.pairs = reinterpret_cast<uint2*>(ws + pl.off_pairs);
  a.cum = reinterpret_cast<uint32_t*>(ws + pl.off_cum);
  a.part = reinterpret_cast<float*>(ws + pl.off_part);
  a.n_seg = pl.n_seg;
  a.pb_per_split = decode_pb_per_split(d.kB + 1);
  const dim3 grid((unsigned)(batch * pl.n_seg));
#define QSA_STEP(HKV, DD)                                                              \
  if (d.kv_heads == HKV && d.head_dim == DD) {                                         \
    hipLaunchKernelGGL((decode_step_kernel<HKV, DD>), grid, dim3(kNT), 0, st, a);      \
    return hipGetLastError();                                                          \
  }
  QSA_STEP(2, 128)
  QSA_STEP(1, 128)
  QSA_STEP(2, 64)
#undef QSA_STEP
  return hipErrorInvalidValue;
}

}  // namespace qsa
