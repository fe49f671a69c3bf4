// One work item of the MFMA sparse-attention path: a query's token set, or
// one split of it, attended by a 256-thread workgroup.  Shared by the
// stand-alone attention kernels and the fused decode step.
//
// "QSA (Qwen Sparse Attention)", Key math / How it works: (B) each query
// runs ordinary softmax attention (logits scaled by 1/sqrt(d)), but only over
// the tokens of its chosen blocks; (A) a chosen block contributes all of its
// tokens, and the already visible part of the query's own block is added.
//
// Token set of the query at p (c = floor(p/4)): pseudo-blocks 0..count-1 are
// the selected blocks, pseudo-block `count` is the tail block c, whose
// tokens 4c+t count only while 4c+t <= p.
//
// Layout (16 query heads, Hkv in {1,2}, head_dim in {64,128}, bf16):
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
//   * The item's selected-block list is loaded into LDS once, so the K/V
//     addresses of a tile never wait on a dependent global load.
//   * The 4 waves interleave tiles and merge their (m, l, O) states in LDS.
//     A single-split item writes the bf16 output and the log-sum-exp; a split
//     writes its (m, l, O) state for a log-sum-exp merge of the splits.
#pragma once

#include <math.h>

#include "fast_exp.h"
#include "qsa_common.h"

namespace qsa {

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
  static constexpr int DP = D + 4;                       // padded head row of the merge area
  static constexpr int MERGE_FLOATS = 2 * HQ + HQ * DP;  // per wave
  // the four V tiles, or the wave merge: 4 states + per-head factors, Z, M
  static constexpr int MERGE_BYTES = 4 * MERGE_FLOATS * 4 + (4 * HQ + 2 * HQ) * 4;
  static constexpr int LDS_BYTES = (4 * TILE_LDS > MERGE_BYTES) ? 4 * TILE_LDS : MERGE_BYTES;
  // 16-token tiles (attn_mfma_tiles16): half the V tile per wave
  static constexpr int TILE16_LDS = 16 * ROWB;
  static constexpr int LDS16_BYTES = (4 * TILE16_LDS > MERGE_BYTES) ? 4 * TILE16_LDS : MERGE_BYTES;
  static_assert(CH == 16 || CH == 32, "the V swizzle needs 16 or 32 chunks per row");
};

// Pseudo-blocks are 4-token units: a block of r = 4m tokens is m of them.
// A token set holds at most 2048 selected tokens (r * k_B <= 2048) plus a
// tail of at most r <= 128 tokens.  Blocks of r < 4 tokens are attended from
// an explicit token list instead (token mode): list slots 4i .. 4i+3 play
// the part of pseudo-block i.
constexpr int kMaxPB = (2048 + 128) / 4;  // pseudo-blocks of one query
constexpr int kMaxTok = 2048 + 4;         // token-mode list: r*k_B <= 2048 plus a tail of r < 4
constexpr int kDecodeSplits = 17;         // decode: splits of a query's token set

// Pseudo-blocks per decode split: the largest token set (max_pb pseudo-
// blocks) cut into kDecodeSplits equal runs (32 at k_B = 512, r = 4: one
// 32-token tile for each of a workgroup's four waves).
__host__ __device__ constexpr int decode_pb_per_split(int max_pb) {
  return (max_pb + kDecodeSplits - 1) / kDecodeSplits;
}

// Floats of one split's state [m 16][l 16][O 16 x D].
constexpr int part_floats(int D) { return 32 + 16 * D; }

// XOR swizzle of a V row's 16-byte chunks: rows 4 apart start their chunks
// at different 64-byte offsets, so the transposed 4-byte reads of one wave
// (four token rows at a time) hit distinct banks.
__device__ __forceinline__ int vswz(int tk) { return 4 * ((tk >> 2) & 3); }

// Block-diagonal query operand of query row `row` (16 heads): head l16 is
// non-zero only on its KV head's dims of the concatenated KV row.
template <int HKV, int D>
__device__ __forceinline__ void load_qbd(const uint16_t* __restrict__ q, int64_t row,
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
    qb[kk] = (grp == gn) ? ld16(q + (row * 16 + l16) * D + (dim0 - grp * D))
                         : u32x4{0, 0, 0, 0};
  }
}

// s_waitcnt immediate (gfx9 encoding) for vmcnt <= 2 NK with no expcnt or
// lgkmcnt wait: vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt
// [11:8] = 15.
template <int NK>
constexpr int kWaitVm2NK = ((2 * NK) & 15) | (((2 * NK) >> 4) << 14) | (7 << 4) | (15 << 8);
static_assert(2 * 8 < 64, "vmcnt has 6 bits");

// Merges the four waves' (m, l, O) states of one work item and writes the
// bf16 output and log-sum-exp (n_split == 1) or the split's state to part
// (with coherent stores when COHERENT).  Called by all 256 threads; lds:
// MfmaShape::MERGE_BYTES bytes no wave reads any more.
template <int HKV, int D, bool COHERENT>
__device__ __forceinline__ void attn_merge_waves(
    float m_run, float l_run, const f32x4 (&oacc)[MfmaShape<HKV, D>::NK][2], int64_t row,
    int64_t item, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part, int n_split, unsigned char* lds) {
  using S = MfmaShape<HKV, D>;
  constexpr int NK = S::NK, G = S::G, MF = S::MERGE_FLOATS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  // ---- merge the four waves' states: per head, M = max_w m_w,
  // f_w = 2^(m_w - M) (waves without tokens skipped), Z = sum_w f_w l_w,
  // O = sum_w f_w O_w, in wave order
  l_run = wave_add_xor32(wave_add_xor16(l_run));
  __syncthreads();
  float* mg = reinterpret_cast<float*>(lds);
  float* my = mg + wave * MF;  // [m 16][l 16][o 16 x DP] (rows padded: no bank conflicts)
  float* fac = mg + 4 * MF;    // [4 waves][16 heads]: f_w, or -1 when skipped
  float* hz = fac + 4 * 16;    // [16] Z
  float* hm = hz + 16;         // [16] M
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
          my[32 + l16 * S::DP + rel] = oacc[pp][h][i];
        }
    }
  }
  __syncthreads();
  // (all LDS reads hoisted out of the conditionals: they issue together)
  if (threadIdx.x < 16) {
    const int n = threadIdx.x;
    float mw[4], lw[4], mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = mg[w * MF + n];
      lw[w] = mg[w * MF + 16 + n];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, mw[w]);
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float f = -1.0f;
      if (mw[w] != -INFINITY) {
        f = exp2_fast(mw[w] - mx);
        z += f * lw[w];
      }
      fac[w * 16 + n] = f;
    }
    hz[n] = z;
    hm[n] = mx;
  }
  __syncthreads();
  // four consecutive outputs (one head) per thread and pass
  for (int q4 = threadIdx.x; q4 < 4 * D; q4 += 256) {
    const int n = q4 / (D / 4);
    const int dd = 4 * (q4 % (D / 4));
    float fw[4];
    f32x4 vw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      fw[w] = fac[w * 16 + n];
      vw[w] = *reinterpret_cast<const f32x4*>(mg + w * MF + 32 + n * S::DP + dd);
    }
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (fw[w] < 0.0f) continue;
      o[0] += fw[w] * vw[w][0];
      o[1] += fw[w] * vw[w][1];
      o[2] += fw[w] * vw[w][2];
      o[3] += fw[w] * vw[w][3];
    }
    const float z = hz[n];
    if (n_split == 1) {
      const uint32_t lo = f32_to_bf16(o[0] / z) | (f32_to_bf16(o[1] / z) << 16);
      const uint32_t hi = f32_to_bf16(o[2] / z) | (f32_to_bf16(o[3] / z) << 16);
      *reinterpret_cast<uint2*>(out + (row * 16 + n) * D + dd) = make_uint2(lo, hi);
      if (lse && dd == 0) lse[row * 16 + n] = (hm[n] + log2f(z)) * kLn2;
    } else {
      float* po = part + item * part_floats(D);
      if constexpr (COHERENT) {
        coherent_store(reinterpret_cast<unsigned long long*>(po + 32 + n * D + dd),
                       (unsigned long long)__float_as_uint(o[0]) |
                           ((unsigned long long)__float_as_uint(o[1]) << 32));
        coherent_store(reinterpret_cast<unsigned long long*>(po + 32 + n * D + dd + 2),
                       (unsigned long long)__float_as_uint(o[2]) |
                           ((unsigned long long)__float_as_uint(o[3]) << 32));
        if (dd == 0) {
          coherent_store(&po[n], hm[n]);
          coherent_store(&po[16 + n], z);
        }
      } else {
        *reinterpret_cast<f32x4*>(po + 32 + n * D + dd) = o;
        if (dd == 0) {
          po[n] = hm[n];
          po[16 + n] = z;
        }
      }
    }
  }
}

// The walk of attn_mfma_tiles in 16-token tiles (prefill of the two-128-dim-
// KV-head shape, not the token mode; decode splits keep the 32-token walk
// the fused step shares): wave w takes tiles of 4 pseudo-blocks at
// pb_lo + 4 w, pb_lo + 4 w + 16, ...  Half the V tile per
// wave, half the K registers and P.V products of 16 x 16 x 16 (the k-slots
// are the tile's 16 tokens), so the kernel fits three workgroups per CU
// instead of two: more gathers in flight per CU, which is what bounds this
// walk once the L2 catches the shared blocks.  Software-pipelined per wave:
// the next tile's K loads are issued as soon as this tile's scores have
// consumed kreg (they fly during the softmax), its V loads after a full
// wait that follows this tile's P.V products (they fly during the next
// tile's scores and softmax).  The compiler counts loads into registers and
// loads into LDS as events that may complete out of order, so any wait it
// placed for kreg while V loads fly would be a wait for all of them; the
// explicit full wait before each V issue leaves kreg complete, and it
// places none.  qlds: the query operand qb of every lane, [NK][64] in lane
// order (kept out of registers), published with sbid.
template <int HKV, int D>
__device__ __forceinline__ void attn_mfma_tiles16(
    const u32x4* qlds, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    int64_t cap, int s, int64_t p, int64_t row, int64_t item, int pb_lo, int pb_hi,
    const int32_t* sbid, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part, int n_split, unsigned char* lds, int rot) {
  using S = MfmaShape<HKV, D>;
  constexpr int KD = S::KD, NK = S::NK, ROWB = S::ROWB, CH = S::CH, RPI = S::RPI;
  static_assert(S::MERGE_BYTES <= S::LDS16_BYTES, "merge area must fit");
  typedef short s16x4 __attribute__((ext_vector_type(4)));

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const uint16_t* kbase = kc + (int64_t)s * cap * KD;
  const uint16_t* vbase = vc + (int64_t)s * cap * KD;
  const int nlist = pb_hi - pb_lo;
  // (branch-free: the LDS read is clamped into the list, its value
  // discarded past the list)
  auto bid = [&](int pb) -> int64_t {
    int i = pb - pb_lo + rot;
    i -= i >= nlist ? nlist : 0;
    const int32_t v = sbid[max(min(i, nlist - 1), 0)];
    return pb < pb_hi ? (int64_t)v : (int64_t)-1;
  };
  // row of token tk (0..15) of the tile at pb0; a masked token reads row p
  auto trow = [&](int pb0, int tk) -> int64_t {
    const int64_t b = bid(pb0 + (tk >> 2));
    const int64_t tp = 4 * b + (tk & 3);
    return (b >= 0 && tp <= p) ? tp : p;
  };
  unsigned char* vt = lds + wave * S::TILE16_LDS;
  auto load_k = [&](int pb0, u32x4 (&kreg)[NK]) {
    const uint16_t* kp = kbase + trow(pb0, l16) * KD + 8 * gq;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kreg[kk] = ld16(kp + 32 * kk);
  };
  auto load_v = [&](int pb0) {
#pragma unroll
    for (int u = 0; u < 16 / RPI; ++u) {
      const int tk = RPI * u + lane / CH;
      const int chunk = (lane % CH) ^ vswz(tk);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(vbase + trow(pb0, tk) * KD + chunk * 8),
          (__attribute__((address_space(3))) void*)(vt + u * 1024), 16, 0, 0);
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 oacc[NK][2];
#pragma unroll
  for (int pp = 0; pp < NK; ++pp) oacc[pp][0] = oacc[pp][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 kreg[NK];
  load_k(pb_lo + 4 * wave, kreg);   // (a wave without tiles reads row p)
  __builtin_amdgcn_s_waitcnt(0);
  load_v(pb_lo + 4 * wave);
  for (int pb0 = pb_lo + 4 * wave; pb0 < pb_hi; pb0 += 16) {
    const bool more = pb0 + 16 < pb_hi;
    // ---- S^T = K * Qbd: lane holds tokens 4gq + i for head l16
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kreg[kk]),
                                                     as_bf16x8(qlds[kk * 64 + lane]), sacc, 0,
                                                     0, 0);
    if (more) load_k(pb0 + 16, kreg);
    float x[4];
    float mt = -INFINITY;
    {
      const int64_t b = bid(pb0 + gq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = b >= 0 && 4 * b + i <= p;
        x[i] = ok ? sacc[i] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[i]);
      }
    }
    mt = wave_max_xor32(wave_max_xor16(mt));
    const float m_new = fmaxf(m_run, mt);
    const bool any = m_new != -INFINITY;
    const float alpha = any ? exp2_fast(m_run - m_new) : 1.0f;
    float pr[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = any ? exp2_fast(x[i] - m_new) : 0.0f;
      psum += pr[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // once the running maxima settle most tiles leave every alpha at 1:
    // skipping the 4 NK multiplies by 1.0 changes no bit
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int pp = 0; pp < NK; ++pp) {
        oacc[pp][0] *= alpha;
        oacc[pp][1] *= alpha;
      }
    }
    // P^T operand: k-slot (gq, e) <-> token 4gq + e, column = head l16
    s16x4 pv;
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = (short)f32_to_bf16(pr[e]);
    // this wave's V tile has landed in LDS (the compiler also waits for
    // every load before the LDS reads below: see attn_mfma_tiles)
    if (more)
      __builtin_amdgcn_s_waitcnt(kWaitVm2NK<NK / 2>);
    else
      __builtin_amdgcn_s_waitcnt(0);
    wave_sync();
    // ---- O^T += V^T * P^T: A row l16 <-> dims 32 pp + 2 l16 (+1 for a1)
#pragma unroll
    for (int pp = 0; pp < NK; ++pp) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tr = 4 * gq + e;
        const int chunk = (4 * pp + (l16 >> 2)) ^ vswz(tr);
        w[e] = *reinterpret_cast<const uint32_t*>(vt + tr * ROWB + chunk * 16 + 4 * (l16 & 3));
      }
      s16x4 a0, a1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0[e] = (short)(w[e] & 0xFFFFu);
        a1[e] = (short)(w[e] >> 16);
      }
      oacc[pp][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, pv, oacc[pp][0], 0, 0, 0);
      oacc[pp][1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, pv, oacc[pp][1], 0, 0, 0);
    }
    wave_sync();  // all reads of this tile issued before the next tile's loads
    if (more) {
      __builtin_amdgcn_s_waitcnt(0);  // the next K has landed in kreg
      load_v(pb0 + 16);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // (a wave without tiles: its loads)

  attn_merge_waves<HKV, D, false>(m_run, l_run, oacc, row, item, out, lse, part, n_split, lds);
}

// Attends query row `row` (sequence s, position p) over pseudo-blocks
// [pb_lo, pb_hi) whose block ids the caller has put in sbid[0 ..) (the tail
// block c = floor(p/4) included as an ordinary id), for work item `item` =
// row * n_split + split.  TOK (token mode): sbid[i] is instead the position
// of token slot 4*pb_lo + i, and slots at or past t_hi are empty.
// n_split == 1 writes the bf16 output and the
// log-sum-exp; otherwise the split's (m, l, O) state goes to part (with
// coherent stores when COHERENT: another workgroup of the same kernel reads
// it).  lds: MfmaShape::LDS_BYTES bytes.  Called by all 256 threads after a
// barrier that publishes sbid.
template <int HKV, int D, bool COHERENT, bool TOK = false>
__device__ __forceinline__ void attn_mfma_tiles(
    const u32x4 (&qb)[MfmaShape<HKV, D>::NK], const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t cap, int s, int64_t p, int64_t row, int64_t item,
    int pb_lo, int pb_hi, const int32_t* sbid, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part, int n_split, unsigned char* lds,
    int t_hi = 0, int rot = 0) {
  using S = MfmaShape<HKV, D>;
  constexpr int KD = S::KD, NK = S::NK, ROWB = S::ROWB, G = S::G, CH = S::CH, RPI = S::RPI;
  constexpr int MF = S::MERGE_FLOATS;
  static_assert(S::MERGE_BYTES <= S::LDS_BYTES, "merge area must fit");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const uint16_t* kbase = kc + (int64_t)s * cap * KD;
  const uint16_t* vbase = vc + (int64_t)s * cap * KD;
  // block id of pseudo-block pb, -1 outside this work item; the walk may
  // start rot entries into the list and wrap (the softmax sums do not
  // depend on the order)
  const int nlist = pb_hi - pb_lo;
  auto bid = [&](int pb) -> int64_t {
    if (pb >= pb_hi) return -1;
    int i = pb - pb_lo + rot;
    i -= i >= nlist ? nlist : 0;
    return (int64_t)sbid[i];
  };
  // token mode: position of list slot sl, -1 past the list
  auto tok = [&](int sl) -> int64_t { return (sl < t_hi) ? (int64_t)sbid[sl - 4 * pb_lo] : -1; };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 oacc[NK][2];
#pragma unroll
  for (int pp = 0; pp < NK; ++pp) oacc[pp][0] = oacc[pp][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned char* vt = lds + wave * S::TILE_LDS;

  // K rows of the tile at pb0 straight into A-operand registers
  auto load_k = [&](int pb0, u32x4 (&kreg)[2][NK]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int tk = 16 * st + l16;
      int64_t rp;
      if constexpr (TOK) {
        const int64_t tp = tok(4 * pb0 + tk);
        rp = tp >= 0 ? tp : p;
      } else {
        const int64_t b = bid(pb0 + (tk >> 2));
        const int64_t tp = 4 * b + (tk & 3);
        rp = (b >= 0 && tp <= p) ? tp : p;
      }
      const uint16_t* kp = kbase + rp * KD + 8 * gq;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) kreg[st][kk] = ld16(kp + 32 * kk);
    }
  };
  // V rows of the tile's 32 tokens: straight from HBM into this wave's LDS
  // tile (lane-ordered 1 KiB per instruction, chunk-swizzled)
  auto load_v = [&](int pb0) {
#pragma unroll
    for (int u = 0; u < 32 / RPI; ++u) {
      const int tk = RPI * u + lane / CH;
      const int chunk = (lane % CH) ^ vswz(tk);
      int64_t rp;
      if constexpr (TOK) {
        const int64_t tp = tok(4 * pb0 + tk);
        rp = tp >= 0 ? tp : p;
      } else {
        const int64_t b = bid(pb0 + (tk >> 2));
        const int64_t tp = 4 * b + (tk & 3);
        rp = (b >= 0 && tp <= p) ? tp : p;
      }
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(vbase + rp * KD + chunk * 8),
          (__attribute__((address_space(3))) void*)(vt + u * 1024), 16, 0, 0);
    }
  };

  // each tile issues its K and V loads at its start
  u32x4 kreg[2][NK];
  for (int pb0 = pb_lo + 8 * wave; pb0 < pb_hi; pb0 += 32) {
    load_k(pb0, kreg);
    load_v(pb0);
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
      const int64_t b = TOK ? 0 : bid(pb0 + 4 * st + gq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = TOK ? 4 * (pb0 + 4 * st + gq) + i < t_hi : (b >= 0 && 4 * b + i <= p);
        x[st][i] = ok ? sacc[st][i] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[st][i]);
      }
    }
    mt = wave_max_xor32(wave_max_xor16(mt));
    const float m_new = fmaxf(m_run, mt);
    const bool any = m_new != -INFINITY;
    const float alpha = any ? exp2_fast(m_run - m_new) : 1.0f;
    float pr[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[st][i] = any ? exp2_fast(x[st][i] - m_new) : 0.0f;
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

  attn_merge_waves<HKV, D, COHERENT>(m_run, l_run, oacc, row, item, out, lse, part, n_split, lds);
}

// Log-sum-exp merge of one (row, head, dim) over a row's kDecodeSplits split
// states, in split order: M = max_k m_k, Z = sum_k 2^(m_k - M) l_k,
// A = sum_k 2^(m_k - M) O_k (splits with m_k = -inf hold no token).
// out = A / Z, lse = (M + log2 Z) ln 2.  ml[2k], ml[2k+1] hold m_k, l_k (the
// caller loads them, and the O values o[k]).
__device__ __forceinline__ void lse_merge_splits(const float* ml, const float (&o)[kDecodeSplits],
                                                 float& mx, float& zs, float& acc) {
  mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kDecodeSplits; ++k) mx = fmaxf(mx, ml[2 * k]);
  zs = 0.0f;
  acc = 0.0f;
#pragma unroll
  for (int k = 0; k < kDecodeSplits; ++k) {
    const float mk = ml[2 * k];
    if (mk != -INFINITY) {
      const float f = exp2_fast(mk - mx);
      zs += f * ml[2 * k + 1];
      acc += f * o[k];
    }
  }
}

}  // namespace qsa
