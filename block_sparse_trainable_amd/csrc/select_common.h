// Workgroup-wide scan and MSB-first radix select used by the selection
// kernels ("QSA (Qwen Sparse Attention)", Key math / How it works, (A): the
// top-k_B blocks by importance).  Templated on the workgroup size NT (a
// multiple of 64, at most 512).
#pragma once

#include "qsa_common.h"

namespace qsa {

constexpr int kRadixBins = 2048;

// Exclusive prefix sum over the workgroup in thread order; total in *total.
// scratch holds NT/64 words.  Contains two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_add(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = scratch[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Result of a radix select: among eligible keys, those with
// (k & mask) > prefix number need_in - need; `avail` keys have
// (k & mask) == prefix, and `need` of them (need <= avail) complete the top
// need_in.  avail == need means every key with the prefix is kept.
struct Radix {
  uint32_t prefix, mask, need, avail;
};

// MSB-first radix select over key bits 30..0 in digits of DB bits from the
// top (DB = 11: bits 30..20, 19..9, 8..0; DB = 8: 30..23, 22..15, 14..7,
// 6..0) over n keys key(i), counting only keys with elig(i).  first_pass > 0
// starts at a later digit with the bits above it already fixed to
// prefix0/mask0; a last_pass below the last digit stops early for keys whose
// low bits are all zero.  hist holds 2^DB words, scratch NT/64 + 3.  CHEAP:
// key(i) and elig(i) are cheap reads of any index below n (LDS): they are
// evaluated four elements at a time, unconditionally, so their latencies
// overlap; otherwise key(i) is only evaluated for eligible elements.
template <int NT, bool CHEAP = false, int DB = 11, class KeyFn, class EligFn>
__device__ __forceinline__ Radix radix_select(KeyFn key, EligFn elig, int64_t n, uint32_t need_in,
                              uint32_t* hist, uint32_t* scratch, int first_pass = 0,
                              uint32_t prefix0 = 0u, uint32_t mask0 = 0u,
                              int last_pass = (31 + DB - 1) / DB - 1) {
  static_assert(DB == 8 || DB == 11, "digit widths");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  Radix r{prefix0, mask0, need_in, 0xFFFFFFFFu};
  for (int pass = first_pass; pass <= last_pass; ++pass) {
    const int top = 30 - DB * pass;            // the digit's highest bit
    const int sh = top - DB + 1 > 0 ? top - DB + 1 : 0;
    const int nb = 1 << (top - sh + 1);
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < nb; i += NT) hist[i] = 0;
    __syncthreads();
    if constexpr (CHEAP) {
      constexpr int U = 4;
      for (int64_t i0 = tid; i0 < n; i0 += (int64_t)U * NT) {
        uint32_t kv[U];
        bool ok[U];
#pragma unroll
        for (int e = 0; e < U; ++e) {
          const int64_t i = i0 + (int64_t)e * NT;
          const int64_t ic = i < n ? i : 0;
          const bool el = elig(ic);
          kv[e] = key(ic);
          ok[e] = (i < n) & el;
        }
#pragma unroll
        for (int e = 0; e < U; ++e)
          if (ok[e] && (kv[e] & r.mask) == r.prefix) atomicAdd(&hist[(kv[e] >> sh) & dmask], 1u);
      }
    } else {
      for (int64_t i = tid; i < n; i += NT) {
        if (!elig(i)) continue;
        const uint32_t k = key(i);
        if ((k & r.mask) == r.prefix) atomicAdd(&hist[(k >> sh) & dmask], 1u);
      }
    }
    __syncthreads();
    // thread t owns the per = max(nb / NT, 1) bins just below nb - t*per
    // (none once that is 0), read at once, highest first
    constexpr int kMaxPer = (1 << DB) / NT > 1 ? (1 << DB) / NT : 1;
    const int per = nb / NT > 1 ? nb / NT : 1;
    const int hi = nb - tid * per;
    uint32_t hv[kMaxPer];
    uint32_t local = 0;
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) {
      hv[e] = (e < per && hi - 1 - e >= 0) ? hist[hi - 1 - e] : 0u;
      local += hv[e];
    }
    uint32_t tot;
    const uint32_t above = block_excl_scan<NT>(local, scratch, &tot);
    if (above < r.need && r.need <= above + local) {
      uint32_t acc = above;
      bool found = false;
#pragma unroll
      for (int e = 0; e < kMaxPer; ++e) {
        if (!found && e < per && acc + hv[e] >= r.need) {
          scratch[NW] = (uint32_t)(hi - 1 - e);
          scratch[NW + 1] = acc;
          scratch[NW + 2] = hv[e];
          found = true;
        }
        acc += hv[e];
      }
    }
    __syncthreads();
    const uint32_t d = scratch[NW];
    const uint32_t above_d = scratch[NW + 1];
    const uint32_t in_d = scratch[NW + 2];
    __syncthreads();
    r.need -= above_d;
    r.prefix |= d << sh;
    r.mask |= dmask << sh;
    r.avail = in_d;
    if (in_d == r.need) break;  // every eligible key with this prefix is kept
  }
  return r;
}

}  // namespace qsa
