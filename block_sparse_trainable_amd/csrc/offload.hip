// Selection-driven host-offloaded KV for decode (qsa_offload_stage).
//
// "QSA" knowledge-card page (kongchang.com), Timeline and All Facts: a
// serving port keeps each request's full KV history in host memory and only
// hot data in GPU memory, fetches what each step selects, and each of the
// QSA layers keeps its own selection (so no index is shared across layers).
// That page reports another party's port, not an algorithm; the reading
// taken here: the K/V rows of every token live in pinned host memory
// ([batch][cap][Hkv][d], read by the kernel over the host link); the
// compressed index stays in HBM, so scoring and top-k run as usual; per
// decode step this call copies the query's token set -- the selected blocks
// in ascending order, then the tail -- into a contiguous staging buffer in
// HBM, taking each 4-token unit from a direct-mapped HBM hot cache when the
// unit is there and from host memory otherwise, then promotes the missed
// units into the hot cache.  It also writes the selection in staged
// coordinates (blocks 0 .. count-1, the tail after them), so
// qsa_sparse_attn_decode on the staging buffer attends over exactly the
// query's token set.
//
// Only units that are complete at the step (every row at or before the
// query's position p) are cached or read from the cache: the unit holding p
// also covers rows p+1 .. that the caller has not written yet, so it always
// comes from host memory, where the next steps will find their new rows.
#include "qsa_common.h"

namespace qsa {
namespace {

constexpr int kOT = 256;
constexpr int kClaim = 2048;   // promotion claims per step (a hash of the slot)
constexpr int kGatherSplit = 32;   // gathering workgroups per sequence
constexpr int kPT = 1024;          // threads of the promoting workgroup

// The query's token set in 4-token units: the selected blocks' units in
// ascending order, then the tail's.
struct UnitList {
  const int32_t* srow;
  int64_t p, c;
  int count, lm, nsel, npb;
  __device__ UnitList(const int32_t* sel, const int32_t* cnt, const int32_t* q_pos, int s, int kB,
                      int lr, int64_t cap) {
    p = min(max((int64_t)q_pos[s], (int64_t)0), cap - 1);
    c = p >> lr;
    count = (int)min((int64_t)max(cnt[s], 0), min((int64_t)kB, c));
    lm = lr - 2;
    nsel = count << lm;
    npb = nsel + (int)((p - (c << lr)) >> 2) + 1;
    srow = sel + (int64_t)s * kB;
  }
  __device__ int64_t operator()(int i) const {
    return i < nsel ? (min(max((int64_t)srow[i >> lm], (int64_t)0), c - 1) << lm) +
                          (i & ((1 << lm) - 1))
                    : (c << lm) + (i - nsel);
  }
};

// Gathering: kGatherSplit workgroups per sequence, each a contiguous share of
// the units; a wave moves one unit at a time (4 x KD bf16 of K and of V, in
// 16-byte chunks), from the hot cache when the unit's slot holds it, else
// from host memory.  The hot cache is only read here.
__global__ __launch_bounds__(kOT) void offload_gather_kernel(
    int kB, int lr, int KD, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, const uint16_t* __restrict__ kh,
    const uint16_t* __restrict__ vh, int64_t cap, const uint16_t* __restrict__ hk,
    const uint16_t* __restrict__ hv, const int32_t* __restrict__ htag, int hot_units,
    uint16_t* __restrict__ sk, uint16_t* __restrict__ sv, int64_t stage_tokens) {
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const UnitList unit(sel, cnt, q_pos, s, kB, lr, cap);
  const int per = (unit.npb + kGatherSplit - 1) / kGatherSplit;
  const int i0 = blockIdx.x * per, i1 = min(i0 + per, unit.npb);
  const int CH = 4 * KD / 8;   // 16-byte chunks of one unit's K (or V) rows
  const int32_t* tags = htag + (int64_t)s * hot_units;
  for (int i = i0 + wave; i < i1; i += kOT / 64) {
    const int64_t u = unit(i);
    const int slot = (int)(u % hot_units);
    const bool hit = 4 * u + 3 <= unit.p && tags[slot] == (int32_t)u;
    uint16_t* dk = sk + ((int64_t)s * stage_tokens + 4 * (int64_t)i) * KD;
    uint16_t* dv = sv + ((int64_t)s * stage_tokens + 4 * (int64_t)i) * KD;
    for (int ch = lane; ch < CH; ch += 64) {
      // token t of the unit; rows past the cache end (a last, partial unit:
      // tokens after p, never attended) repeat the last row
      const int t = ch / (KD / 8), e = ch % (KD / 8);
      const int64_t src = hit ? (((int64_t)s * hot_units + slot) * 4 + t) * KD + 8 * e
                              : ((int64_t)s * cap + min(4 * u + t, cap - 1)) * KD + 8 * e;
      const u32x4 a = *reinterpret_cast<const u32x4*>((hit ? hk : kh) + src);
      const u32x4 b = *reinterpret_cast<const u32x4*>((hit ? hv : vh) + src);
      *reinterpret_cast<u32x4*>(dk + 8 * ch) = a;
      *reinterpret_cast<u32x4*>(dv + 8 * ch) = b;
    }
  }
}

// Promotion, one workgroup per sequence, after the gathering: counts the hits
// and misses against the tags the gathering saw, then writes each missed
// complete unit from the staging buffer into its slot -- one unit per hash
// bucket of the slot, so a slot gets data and tag from a single unit -- and
// writes the selection in staging coordinates.
__global__ __launch_bounds__(kPT) void offload_promote_kernel(
    int kB, int lr, int KD, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, int64_t cap, uint16_t* __restrict__ hk,
    uint16_t* __restrict__ hv, int32_t* __restrict__ htag, int hot_units,
    const uint16_t* __restrict__ sk, const uint16_t* __restrict__ sv, int64_t stage_tokens,
    int32_t* __restrict__ ssel, int32_t* __restrict__ scnt, int32_t* __restrict__ spos,
    int32_t* __restrict__ stats) {
  __shared__ int claim[kClaim];
  __shared__ int n_hit, n_miss;
  const int s = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const UnitList unit(sel, cnt, q_pos, s, kB, lr, cap);
  for (int i = threadIdx.x; i < kClaim; i += kPT) claim[i] = -1;
  if (threadIdx.x == 0) n_hit = n_miss = 0;
  __syncthreads();
  int32_t* tags = htag + (int64_t)s * hot_units;
  int h = 0, m = 0;
  for (int i = threadIdx.x; i < unit.npb; i += kPT) {
    const int64_t u = unit(i);
    if (4 * u + 3 <= unit.p && tags[u % hot_units] == (int32_t)u) ++h; else ++m;
  }
  atomicAdd(&n_hit, h);
  atomicAdd(&n_miss, m);
  __syncthreads();   // every tag read before any is rewritten
  const int CH = 4 * KD / 8;
  for (int i = wave; i < unit.npb; i += kPT / 64) {
    const int64_t u = unit(i);
    const int slot = (int)(u % hot_units);
    if (4 * u + 3 > unit.p) continue;                // rows past p: not final yet
    if (tags[slot] == (int32_t)u) continue;          // a hit (or already promoted)
    int owner = 0;
    if (lane == 0) owner = atomicCAS(&claim[slot & (kClaim - 1)], -1, slot) == -1;
    owner = __shfl(owner, 0);
    if (!owner) continue;                            // the bucket went to another unit
    const uint16_t* srck = sk + ((int64_t)s * stage_tokens + 4 * (int64_t)i) * KD;
    const uint16_t* srcv = sv + ((int64_t)s * stage_tokens + 4 * (int64_t)i) * KD;
    uint16_t* dk = hk + ((int64_t)s * hot_units + slot) * 4 * KD;
    uint16_t* dv = hv + ((int64_t)s * hot_units + slot) * 4 * KD;
    for (int ch = lane; ch < CH; ch += 64) {
      *reinterpret_cast<u32x4*>(dk + 8 * ch) = *reinterpret_cast<const u32x4*>(srck + 8 * ch);
      *reinterpret_cast<u32x4*>(dv + 8 * ch) = *reinterpret_cast<const u32x4*>(srcv + 8 * ch);
    }
    if (lane == 0) tags[slot] = (int32_t)u;           // read by later calls only
  }
  for (int k = threadIdx.x; k < kB; k += kPT) ssel[(int64_t)s * kB + k] = k < unit.count ? k : -1;
  if (threadIdx.x == 0) {
    scnt[s] = unit.count;
    spos[s] = (int32_t)(((int64_t)unit.count << lr) + (unit.p - (unit.c << lr)));
    stats[2 * s] = n_hit;
    stats[2 * s + 1] = n_miss;
  }
}

}  // namespace

hipError_t launch_offload_stage(const Dims& d, int batch, const int32_t* q_pos,
                                const int32_t* sel, const int32_t* cnt, const void* k_host_dev,
                                const void* v_host_dev, int64_t cap, void* hot_k, void* hot_v,
                                int32_t* hot_tag, int hot_units, void* stage_k, void* stage_v,
                                int64_t stage_tokens, int32_t* stage_sel, int32_t* stage_cnt,
                                int32_t* stage_pos, int32_t* stats, hipStream_t st) {
  const int KD = d.kv_heads * d.head_dim;
  hipLaunchKernelGGL(offload_gather_kernel, dim3(kGatherSplit, (unsigned)batch), dim3(kOT), 0, st,
                     d.kB, d.lr, KD, q_pos, sel, cnt, static_cast<const uint16_t*>(k_host_dev),
                     static_cast<const uint16_t*>(v_host_dev), cap,
                     static_cast<const uint16_t*>(hot_k), static_cast<const uint16_t*>(hot_v),
                     hot_tag, hot_units, static_cast<uint16_t*>(stage_k),
                     static_cast<uint16_t*>(stage_v), stage_tokens);
  hipLaunchKernelGGL(offload_promote_kernel, dim3((unsigned)batch), dim3(kPT), 0, st, d.kB, d.lr,
                     KD, q_pos, sel, cnt, cap, static_cast<uint16_t*>(hot_k),
                     static_cast<uint16_t*>(hot_v), hot_tag, hot_units,
                     static_cast<const uint16_t*>(stage_k), static_cast<const uint16_t*>(stage_v),
                     stage_tokens, stage_sel, stage_cnt, stage_pos, stats);
  return hipGetLastError();
}

}  // namespace qsa
