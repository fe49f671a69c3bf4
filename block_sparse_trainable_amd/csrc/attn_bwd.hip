// Gradients of the sparse core attention (qsa_sparse_attn_backward).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works: (B) softmax
// attention over each query's token set only, (A) that set being the chosen
// blocks' tokens plus the visible part of the query's block.  The pages give
// the forward only; these kernels compute its exact derivative with every
// token set held fixed (no gradient reaches the indexer through the top-k_B
// choice).  Per query i, head h, KV head g = floor(h * Hkv / Hq), token j in
// S_i, with P the forward's softmax (recomputed from its log-sum-exp):
//     dP_j = <dO_h, V_j>,  D_h = sum_j P_j dP_j (= <dO_h, O_h>),
//     dS_j = P_j (dP_j - D_h),
//     dq_h = scale sum_j dS_j K_j,  dK_j += scale dS_j q_h,  dV_j += P_j dO_h.
//
// Two sides, no atomics on the gradients:
//   * query side (one workgroup per query row): dq.  MFMA path (bf16, 16
//     query heads): one pass over the forward's 32-token tiles with a
//     reference D~ from the forward output and an exact correction; it also
//     exports what the key side needs.  VALU path: D_h, then dq, heads in
//     turn;
//   * key side, from a transposed index (the queries whose token set holds
//     each piece of the cache, built by counting, scanning and filling).
//     MFMA path: one workgroup per 16-token group, four waves in two pairs
//     each owning half of the KV dims, 16x16x16 MFMAs contracting over the
//     16 heads, dK/dV added once per group.  VALU path: one workgroup per
//     4-token unit, the unit's K/V rows in LDS while it walks its queries.
// The transposed lists are filled with atomics, so the order in which a
// group or unit sums its queries, and with it the last bits of dK/dV, can
// change from run to run; dq is deterministic.
#include <math.h>

#include "attn_tile.h"
#include "fast_exp.h"
#include "qsa_common.h"
#include "select_common.h"

namespace qsa {
namespace {

constexpr int kBwdMaxTokens = 2048 + 128;   // r * k_B <= 2048 selected, tail <= r
constexpr int kNT = 256;
constexpr int kKeySplit = 2;   // key side: dim groups of waves (1, 2 or 4)
constexpr int kBwdSweep = 64;  // query side: rows per sweep of the walk's start

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

// ------------------------------------------------------ query side, MFMA --
// bf16 layers of 16 query heads, Hkv in {1, 2}, head_dim in {64, 128} (the
// forward's MFMA shapes).  One workgroup per query row; its 4 waves take
// 32-token tiles in turn, as the forward does.  Per tile:
//   * V rows go from HBM into A-operand registers: dP^T = V_tile * dObd
//     (dO block-diagonal over the KV heads, like the forward's query operand);
//   * K rows go from HBM into the wave's LDS tile, read twice: as the A
//     operand of S^T = K_tile * Qbd, and transposed for the dq contraction;
//   * P = 2^(S scale log2e - lse log2e) from the forward's log-sum-exp.
// D_h = sum_j P_j dP_j is only known after the last tile, so the weights fed
// to the dq MFMAs use a reference D~_h = <dO_h, O_h> from the forward's
// (rounded) output and the kernel also sums B_h = sum_j P_j K_j:
//     dq_h = scale (sum_j P_j (dP_j - D~_h) K_j - (D_h - D~_h) B_h),
// which is the exact derivative for any D~; D~ only keeps the weights
// P_j (dP_j - D~_h) close to the true dS_j (they enter as bf16 hi + lo).  With two KV heads each
// group's dims need only its own 8 heads, so the 16 MFMA columns carry the 8
// heads' weights and their P (no extra MFMAs for B); with one KV head B has
// accumulators of its own.  The waves' sums meet in LDS once per row.

// Element (row, KV head grp, dim d of that head, query head hl of its group)
// of the transposed q / dO.  Lane (l16, gq) of the key side reads 16 bytes
// at index(row, grp, 32 bp + l16, 4 gql): heads 4 gql .. 4 gql + 3 of dims
// 32 bp + l16 and 32 bp + 16 + l16, i.e. the B operands of two 16-dim
// blocks; the 64 lanes of one read cover 512 (or, with 8 heads per group and
// half the lanes repeating, 256 x 2) contiguous bytes.
template <int HKV, int D>
__device__ __forceinline__ int64_t qt_index(int64_t row, int grp, int d, int hl) {
  constexpr int GQ = 16 / HKV / 4;  // 4-head lane groups per KV head
  const int bp = d >> 5, blk = (d >> 4) & 1, l16 = d & 15, gql = hl >> 2, i = hl & 3;
  return (((((row * HKV + grp) * (D / 32) + bp) * GQ + gql) * 16 + l16) * 2 + blk) * 4 + i;
}

// 16-byte chunk c of token row tk sits at slot c ^ (tk & 15) of the K tile:
// the S operand reads (16 rows, one chunk each) and the transposed reads
// (4 rows x 64 contiguous bytes) both fall in distinct banks.
__device__ __forceinline__ int kswz(int tk) { return tk & 15; }

// Value of lane l ^ 8 (the other half of each 16-lane row).
__device__ __forceinline__ uint32_t swap8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
}
__device__ __forceinline__ float swap8f(float v) { return __uint_as_float(swap8(__float_as_uint(v))); }

// TT: tokens of a wave's tile, 32 or 16.  The two-KV-head, 128-dim shape
// takes 16-token tiles: its V rows held in registers for a 32-token tile
// need about 300 registers, one wave per SIMD; with 16 the kernel fits two
// (the k-slots of the dq MFMAs past the tile are zero).
template <int HKV, int D, int TT>
__global__ __launch_bounds__(256, 2) void bwd_query_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t cap, int n_q, const int32_t* __restrict__ q_pos0,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int kB, float scale,
    const uint16_t* __restrict__ out, const float* __restrict__ lse,
    const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq, float* __restrict__ dlt,
    float2* __restrict__ pw, int max_pb, uint16_t* __restrict__ qt, uint16_t* __restrict__ dot,
    int lr, const int32_t* __restrict__ order, const int32_t* __restrict__ first) {
  using S = MfmaShape<HKV, D>;
  constexpr int KD = S::KD, NK = S::NK, ROWB = S::ROWB, CH = S::CH, RPI = S::RPI;
  constexpr int MF = S::MERGE_FLOATS, DP = S::DP;
  constexpr int NACC = HKV == 2 ? 1 : 2;   // accumulator sets (A and B share one with 2 KV heads)
  static_assert(16 * DP <= MF, "a wave's dq part must fit its merge slot");
  static_assert(TT == 16 || TT == 32, "tile tokens");
  constexpr int NST = TT / 16;                 // 16-token halves of a tile
  constexpr int TILE = TT * ROWB;              // LDS bytes of a wave's K tile
  constexpr int LB = 4 * TILE > S::MERGE_BYTES ? 4 * TILE : S::MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LB];
  __shared__ int32_t sbid[kMaxPB];
  __shared__ float dref[16], dpart[4][16];
  __shared__ u32x4 dbs[NK * 64];   // dObd in lane order (kept out of registers)
  int64_t row;
  {  // contiguous runs of items per XCD (workgroup b goes to XCD b % 8)
    const uint32_t n = gridDim.x, b = blockIdx.x;
    const uint32_t qn = n / 8u, rn = n % 8u, x = b % 8u;
    row = (int64_t)(x * qn + min(x, rn) + b / 8u);
  }
  // as in the forward: item i takes row order[i], rows whose selections
  // cluster in one region of the cache running together
  if (order) row = min(max((int64_t)order[row], (int64_t)0), (int64_t)gridDim.x - 1);
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p >> lr;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  const int lm = lr - 2;
  const int nsel = count << lm;
  const int npb = nsel + (int)((p - (c << lr)) >> 2) + 1;
  const int32_t* srow = sel + row * kB;
  for (int i = (int)threadIdx.x; i < npb; i += 256)
    sbid[i] = i < nsel ? (int32_t)((min(max((int64_t)srow[i >> lm], (int64_t)0), c - 1) << lm) +
                                   (i & ((1 << lm) - 1)))
                       : (int32_t)((c << lm) + (i - nsel));
  {  // D~_h = <dO_h, O_h>: 16 threads per head, D/16 dims each
    constexpr int E = D / 16;
    const int h = (int)threadIdx.x >> 4;
    const int64_t o = (row * 16 + h) * D + (threadIdx.x & 15) * E;
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) a = fmaf(bf16_to_f32(out[o + e]), bf16_to_f32(dout[o + e]), a);
    a = row16_sum_to_last(a);
    if ((threadIdx.x & 15) == 15) dref[h] = a;
  }
  u32x4 qb[NK];
  load_qbd<HKV, D>(q, row, qb);
  if (threadIdx.x < 64) {
    u32x4 db[NK];
    load_qbd<HKV, D>(dout, row, db);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) dbs[kk * 64 + threadIdx.x] = db[kk];
    // q and dO transposed for the key side's contraction over heads, in the
    // order its MFMA operands are read (see qt_index): lane (head l, dims
    // dim0 .. dim0 + 7 of the concatenated KV row)
    const int l = threadIdx.x & 15, g4 = threadIdx.x >> 4, gn = l / S::G;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int dim0 = 32 * kk + 8 * g4;
      const int grp = dim0 / D;
      if (grp != gn) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const int64_t o = qt_index<HKV, D>(row, grp, dim0 - grp * D + e, l - grp * S::G);
        qt[o] = (uint16_t)(qb[kk][e >> 1] >> sh);
        dot[o] = (uint16_t)(db[kk][e >> 1] >> sh);
      }
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const float sl2 = scale * kLog2e;
  const float lse2 = lse[row * 16 + l16] * kLog2e;
  const float dt = dref[l16];
  const uint16_t* kbase = kc + (int64_t)s * cap * KD;
  const uint16_t* vbase = vc + (int64_t)s * cap * KD;
  auto bid = [&](int pb) -> int64_t { return (pb < npb) ? (int64_t)sbid[pb] : -1; };
  // token tk of the tile at pb0 reads row rp (a masked token reads row p)
  auto trow = [&](int pb0, int tk) -> int64_t {
    const int64_t b = bid(pb0 + (tk >> 2));
    const int64_t tp = 4 * b + (tk & 3);
    return (b >= 0 && tp <= p) ? tp : p;
  };

  f32x4 acc[NACC][NK][2];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int pp = 0; pp < NK; ++pp) acc[a][pp][0] = acc[a][pp][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dacc = 0.0f;
  unsigned char* kt = lds + wave * TILE;

  // Tiles of TT / 4 list entries, wave w taking tiles w, w + 4, ...  As in
  // the forward, the walk starts at the tile holding the first block of the
  // row's top region when its selection clusters there, else
  // (p mod kBwdSweep) / kBwdSweep of the way into the list, and wraps, so
  // the rows resident on an XCD read shared blocks together; a tile keeps
  // its list index (pb0), which places its {P, weight} export, and the sums
  // do not depend on the order.
  const int ntile = (npb + TT / 4 - 1) / (TT / 4);
  int trot = (int)((p % kBwdSweep) * ntile / kBwdSweep);
  if (first) {
    const int f = first[row];
    if (f >= 0) trot = min((f << lm) / (TT / 4), ntile - 1);
  }
  for (int t = wave; t < ntile; t += 4) {
    const int pb0 = (TT / 4) * (t + trot < ntile ? t + trot : t + trot - ntile);
    // ---- V rows into A-operand registers
    u32x4 vreg[NST][NK];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const uint16_t* vp = vbase + trow(pb0, 16 * st + l16) * KD + 8 * gq;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) vreg[st][kk] = ld16(vp + 32 * kk);
    }
    // ---- K rows into this wave's LDS tile (lane-ordered 1 KiB per load)
#pragma unroll
    for (int u = 0; u < TT / RPI; ++u) {
      const int tk = RPI * u + lane / CH;
      const int chunk = (lane % CH) ^ kswz(tk);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kbase + trow(pb0, tk) * KD + chunk * 8),
          (__attribute__((address_space(3))) void*)(kt + u * 1024), 16, 0, 0);
    }
    // ---- dP^T = V * dObd: lane holds tokens 16st + 4gq + i for head l16
    f32x4 dpa[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      dpa[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        dpa[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(vreg[st][kk]), as_bf16x8(dbs[kk * 64 + lane]), dpa[st], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's K tile has landed in LDS
    wave_sync();
    // ---- S^T = K * Qbd from the tile
    f32x4 sa[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int tk = 16 * st + l16;
      sa[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt + tk * ROWB +
                                                        (((4 * kk + gq) ^ kswz(tk)) * 16));
        sa[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qb[kk]),
                                                         sa[st], 0, 0, 0);
      }
    }
    // ---- P, D partial, weights P (dP - D~) and P
    float w1[2][4], w2[2][4];   // half st = 1 stays zero with 16-token tiles
#pragma unroll
    for (int i = 0; i < 4; ++i) w1[1][i] = w2[1][i] = 0.0f;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int64_t b = bid(pb0 + 4 * st + gq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = b >= 0 && 4 * b + i <= p;
        const float P = ok ? exp2_fast(fmaf(sa[st][i], sl2, -lse2)) : 0.0f;
        dacc = fmaf(P, dpa[st][i], dacc);
        w1[st][i] = P * (dpa[st][i] - dt);
        w2[st][i] = P;
      }
    }
    // the key side's inputs: {P, P (dP - D~)} per token of the row's set
    // ([row][token][head]; tokens past p hold zeros)
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (pb0 + 4 * st + gq < npb) {
        float2* dst = pw + ((row * max_pb + pb0 + 4 * st + gq) * 4) * 16 + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[16 * i] = make_float2(w2[st][i], w1[st][i]);
      }
    }
    // B-operand layout of the forward's P^T: k-slot (gq, e) <-> token
    // (e < 4 ? 4gq + e : 16 + 4gq + e - 4)
    // The weights go in as bf16 hi + lo pairs (about 16 significant bits):
    // a single bf16 rounding of P (dP - D~) costs up to 2^-9 of each term,
    // which rows of few, sharply weighted tokens turn into percent-level
    // errors in dq.  P (for B, scaled by the small D - D~) needs only hi.
    u32x4 p1, p1l, p2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int st = e >> 1, i0 = 2 * (e & 1);
      const uint32_t h0 = f32_to_bf16(w1[st][i0]), h1 = f32_to_bf16(w1[st][i0 + 1]);
      p1[e] = h0 | (h1 << 16);
      p1l[e] = f32_to_bf16(w1[st][i0] - bf16_to_f32(h0)) |
               (f32_to_bf16(w1[st][i0 + 1] - bf16_to_f32(h1)) << 16);
      p2[e] = f32_to_bf16(w2[st][i0]) | (f32_to_bf16(w2[st][i0 + 1]) << 16);
    }
    u32x4 bop[2], bol[2];
    if constexpr (HKV == 2) {
      // group g's columns: 0..7 the weights of heads 8g .. 8g+7, 8..15 their
      // P (the lo operand carries 0 there)
      u32x4 x1, x1l, x2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x1[e] = swap8(p1[e]);
        x1l[e] = swap8(p1l[e]);
        x2[e] = swap8(p2[e]);
      }
      const u32x4 zero = {0u, 0u, 0u, 0u};
      bop[0] = l16 < 8 ? p1 : x2;
      bop[1] = l16 < 8 ? x1 : p2;
      bol[0] = l16 < 8 ? p1l : zero;
      bol[1] = l16 < 8 ? x1l : zero;
    } else {
      bop[0] = p1;
      bop[1] = p2;
      bol[0] = p1l;
    }
    // ---- dq^T (and B^T) += K^T * weights, K read transposed from the tile
#pragma unroll
    for (int pp = 0; pp < NK; ++pp) {
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tr = (e < 4) ? (4 * gq + e) : (16 + 4 * gq + e - 4);
        const int chunk = (4 * pp + (l16 >> 2)) ^ kswz(tr);
        // (with 16-token tiles the slots of tokens 16.. hold zero weights:
        // their K values are read as 0, not from the next wave's tile)
        w[e] = (TT == 32 || e < 4)
                   ? *reinterpret_cast<const uint32_t*>(kt + tr * ROWB + chunk * 16 + 4 * (l16 & 3))
                   : 0u;
      }
      u32x4 a0, a1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0[e] = (w[2 * e] & 0xFFFFu) | (w[2 * e + 1] << 16);
        a1[e] = (w[2 * e] >> 16) | (w[2 * e + 1] & 0xFFFF0000u);
      }
      const u32x4 bw = bop[HKV == 2 ? pp / (D / 32) : 0];
      const u32x4 bl = bol[HKV == 2 ? pp / (D / 32) : 0];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 ah = as_bf16x8(h ? a1 : a0);
        acc[0][pp][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(bw), acc[0][pp][h],
                                                                0, 0, 0);
        acc[0][pp][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(bl), acc[0][pp][h],
                                                                0, 0, 0);
        if constexpr (HKV == 1)
          acc[1][pp][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(bop[1]),
                                                                  acc[1][pp][h], 0, 0, 0);
      }
    }
    wave_sync();  // all reads of this tile issued before the next tile's loads
  }

  // ---- D_h over the four waves, then each wave's part of dq into LDS
  const float dw = wave_add_xor32(wave_add_xor16(dacc));
  if (gq == 0) dpart[wave][l16] = dw;
  __syncthreads();  // also: every wave is done with its tile
  const float dfull = dpart[0][l16] + dpart[1][l16] + dpart[2][l16] + dpart[3][l16];
  const float delta = dfull - dt;
  float* mg = reinterpret_cast<float*>(lds);
  float* my = mg + wave * MF;  // [16 heads][DP]
  if constexpr (HKV == 2) {
    const float dx = swap8f(delta);  // delta of head l16 ^ 8
#pragma unroll
    for (int pp = 0; pp < NK; ++pp) {
      const int gp = pp / (D / 32);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = acc[0][pp][h][i];
          const float bx = swap8f(a);  // column l16 + 8: P-weighted K of the same head
          if (l16 < 8) {
            const int head = 8 * gp + l16;
            my[head * DP + 32 * pp + 8 * gq + 2 * i + h - gp * D] = a - (gp ? dx : delta) * bx;
          }
        }
    }
  } else {
#pragma unroll
    for (int pp = 0; pp < NK; ++pp)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          my[l16 * DP + 32 * pp + 8 * gq + 2 * i + h] = acc[0][pp][h][i] - delta * acc[1][pp][h][i];
  }
  __syncthreads();
  for (int q4 = threadIdx.x; q4 < 4 * D; q4 += 256) {
    const int n = q4 / (D / 4);
    const int dd = 4 * (q4 % (D / 4));
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(mg + w * MF + n * DP + dd);
      o[0] += v[0];
      o[1] += v[1];
      o[2] += v[2];
      o[3] += v[3];
    }
    const uint32_t lo = f32_to_bf16(o[0] * scale) | (f32_to_bf16(o[1] * scale) << 16);
    const uint32_t hi = f32_to_bf16(o[2] * scale) | (f32_to_bf16(o[3] * scale) << 16);
    *reinterpret_cast<uint2*>(dq + (row * 16 + n) * D + dd) = make_uint2(lo, hi);
  }
  if (threadIdx.x < 16) {  // D_h - D~_h: the key side's dS = P (dP - D~) - (D - D~) P
    const int h = threadIdx.x;
    dlt[row * 16 + h] = dpart[0][h] + dpart[1][h] + dpart[2][h] + dpart[3][h] - dref[h];
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

// ------------------------------------------------- key side, MFMA shapes --
// Transposed index over 16-token groups (four 4-token units): an entry
// {row << 4 | unit mask, i0} says that row's token set holds the group's
// units in `mask`, the first of them at position i0 of the row's unit list
// (the units of one group are adjacent there: the list ascends).  Rows stay
// below 2^27 (the entry points bound batch * n_q), so row << 4 fits.
template <bool FILL>
__global__ __launch_bounds__(kNT) void bwd_group_list_kernel(
    BwdIndex ix, uint2* __restrict__ glist, int64_t cap, int n_q,
    const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, int kB, int lr) {
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p >> lr;
  const int count = (int)min((int64_t)max(cnt[row], 0), min((int64_t)kB, c));
  const int lm = lr - 2;
  const int nsel = count << lm;
  const int npb = nsel + (int)((p - (c << lr)) >> 2) + 1;
  const int32_t* srow = sel + row * kB;
  auto unit = [&](int i) -> int64_t {
    return i < nsel ? (min(max((int64_t)srow[i >> lm], (int64_t)0), c - 1) << lm) +
                          (i & ((1 << lm) - 1))
                    : (c << lm) + (i - nsel);
  };
  for (int i = threadIdx.x; i < npb; i += kNT) {
    const int64_t u = unit(i), g = u >> 2;
    if (g >= ix.nb || (i > 0 && (unit(i - 1) >> 2) == g)) continue;  // not its group's first
    uint32_t mask = 1u << (u & 3);
    for (int k = 1; k < 4 && i + k < npb; ++k) {
      const int64_t v = unit(i + k);
      if ((v >> 2) != g) break;
      mask |= 1u << (v & 3);
    }
    const int64_t e = (int64_t)s * ix.nb + g;
    if constexpr (FILL) {
      const uint32_t at = atomicAdd(&ix.cur[e], 1u);
      glist[ix.off[e] + at] = make_uint2(((uint32_t)row << 4) | mask, (uint32_t)i);
    } else {
      atomicAdd(&ix.cnt[e], 1u);
    }
  }
}

typedef short bf16x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4s pack4(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(bf16x4s, make_uint2(a, b));
}

// fourth word of a raw buffer resource on gfx9 parts (32-bit data format,
// no swizzle): offsets past num_records read as zero
constexpr int kBufWord3 = 0x00020000;

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// bf16 pair of (x, y), nearest-even (one packed conversion on gfx950); with
// sel = 1 the pair of the remainders x - hi, y - hi left by that rounding:
// hi + lo carries about 16 significant bits of each value.
__device__ __forceinline__ uint32_t bf16_pk2(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x, y}, bf16x2v));
}
__device__ __forceinline__ uint32_t bf16_hilo2(float x, float y, float sel) {
  const uint32_t h = bf16_pk2(x, y);
  return bf16_pk2(fmaf(-sel, __uint_as_float(h << 16), x),
                  fmaf(-sel, __uint_as_float(h & 0xFFFF0000u), y));
}

// One workgroup per (sequence, 16-token group); its waves, in kKeySplit
// groups that each own a share of the Hkv*d dims, take the group's entries in
// turn.  Per entry, lane (token l16, heads 4gq .. 4gq+3) forms
// dS = P (dP - D~) - (D - D~) P and P from the query side's export, as
// bf16 hi + lo A operands; the B operands are the row's transposed q / dO
// (a 16-dim block, 4 heads per lane, zero where the head's KV group is not
// the block's).  16x16x16 MFMAs contract over the 16 heads:
//     dK[token][dim] += sum_h dS[h][token] q[h][dim],
//     dV[token][dim] += sum_h  P[h][token] dO[h][dim].
// The waves' sums meet in LDS and are added to dK (times scale) and dV once.
template <int HKV, int D>
__global__ __launch_bounds__(256, 2) void bwd_key_mfma_kernel(
    BwdIndex gx, const uint2* __restrict__ glist, const float2* __restrict__ pw, int max_pb,
    const uint16_t* __restrict__ qt, const uint16_t* __restrict__ dot,
    const float* __restrict__ dlt, int64_t cap, float scale, float* __restrict__ dk,
    float* __restrict__ dv) {
  constexpr int KD = HKV * D, NB = KD / 16, G = 16 / HKV;
  // the dims are split over kKeySplit groups of waves: wave w takes the
  // 16-dim blocks of part w % kKeySplit and every (4 / kKeySplit)-th entry
  constexpr int NS = kKeySplit, NBW = NB / NS, STEP = 4 / NS;
  static_assert(NBW % 2 == 0 && 4 % NS == 0, "dim split must leave pairs of blocks");
  // the group's list is staged here during the loop; the waves' dK / dV sums
  // meet here after it
  __shared__ __attribute__((aligned(16))) float sbuf[2 * 16 * KD];
  constexpr uint32_t LCAP = 16 * KD;  // list entries (uint2) per staged chunk
  float* sk = sbuf;
  float* sv = sbuf + 16 * KD;
  uint2* sl = reinterpret_cast<uint2*>(sbuf);
  int64_t item;
  {  // Newest groups first, the sequences interleaved: the groups at each
     // sequence's end (its local windows and every query's tail) hold about
     // twice the entries of the rest, and blocks leave in index order, spread
     // round-robin over the XCDs, so the longest groups start first and every
     // XCD gets its share of them.  (The grid is batch * nb blocks.)
    const uint32_t b = blockIdx.x;
    const uint32_t batch = gridDim.x / (uint32_t)gx.nb;
    item = (int64_t)(b % batch) * gx.nb + (gx.nb - 1 - (int64_t)(b / batch));
  }
  const uint32_t nq = gx.cnt[item];
  if (nq == 0u) return;
  const int s = (int)(item / gx.nb);
  const int64_t t0 = (item % gx.nb) * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int u = l16 >> 2, t = l16 & 3;
  const int bbase = (wave % NS) * NBW;   // this wave's first 16-dim block
  f32x4 ak[NBW], av[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) ak[b] = av[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint2* lst = glist + gx.off[item];
  // Heads of the lane's A operand and of its B operand's q / dO rows.
  // Two KV heads: a wave's dims are one KV head's (g), whose 8 query heads
  // fill half of a 16-head contraction; lanes gq and gq ^ 2 take heads
  // 8g + 4 (gq & 1) .. + 3, the first pair carrying the bf16 hi part of the
  // weights and the second the lo part, so k-slots 0..7 and 8..15 of one
  // MFMA add hi and lo.  One KV head: lane gq takes heads 4gq .. 4gq + 3, and
  // hi and lo go through two MFMAs.
  constexpr bool FUSE = HKV == 2;
  const uint32_t wv = __builtin_amdgcn_readfirstlane((uint32_t)wave);
  const int g = (16 * bbase) / D;
  const uint32_t gs = (16u * ((wv % NS) * NBW)) / D;   // g, wave-uniform
  const int hb = FUSE ? 8 * g + 4 * (gq & 1) : 4 * gq;
  const float lo_sel = (FUSE && gq >= 2) ? 1.0f : 0.0f;
  // Per-lane byte offsets of an entry's loads within the row's {P, weight}
  // slots and transposed q / dO.  With two KV heads lanes gq and gq ^ 2 need
  // the same values, so each is loaded once: lanes gq < 2 load the {P,
  // weight} pairs of heads hb, hb + 1 and the q / dO of 16-dim blocks 4j,
  // 4j + 1, lanes gq >= 2 those of heads hb + 2, hb + 3 and blocks 4j + 2,
  // 4j + 3, and a swap of the wave's halves (v_permlane32_swap) hands every
  // lane both parts.  D - D~ of the wave's 8 heads is one scalar load.
  constexpr int NQ = FUSE ? NBW / 4 : NBW / 2;   // 16-byte q (and dO) loads per entry
  const uint32_t pw_lane = (uint32_t)(t * 16 + hb) * 8u + ((FUSE && gq >= 2) ? 16u : 0u);
  uint32_t q_lane[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int b = FUSE ? 4 * j + (gq >= 2 ? 2 : 0) : 2 * j;
    const int grp = (16 * (bbase + b)) / D;
    q_lane[j] = 2u * (uint32_t)qt_index<HKV, D>(0, grp, 16 * (bbase + b) - grp * D + l16,
                                                 4 * (gq % (G / 4)));
  }
  struct Stage {
    u32x4 p0, p1;       // {P, weight} pairs (two KV heads: p0 only, half per lane)
    f32x4 dl0, dl1;     // D - D~: the wave's heads (two KV heads), else the lane's in dl0
    u32x4 qx[NQ], dx[NQ];  // transposed q / dO, 4 heads per lane and 16-dim block pair
  };
  // An entry's loads go through buffer resources built per row in scalar
  // registers, with the lane offsets fixed above.  Lanes of units outside
  // the entry, and every lane of a stage past the list, give their {P,
  // weight} loads an offset past the resource: those return zero without a
  // memory access, so the A operands of tokens outside the entry are zero
  // with no branch.  Every fetch thus issues the same loads and the waits
  // before a stage's use cover that stage's loads only.  (One-KV-head
  // layout: lanes whose heads are not a block's KV head never occur.)
  auto fetch = [&](uint32_t k, uint32_t n, Stage& S) {
    const uint2 en = sl[min(k, n - 1u)];
    const uint32_t ex = __builtin_amdgcn_readfirstlane(en.x);
    const uint32_t ey = __builtin_amdgcn_readfirstlane(en.y);
    const int64_t row = ex >> 4;
    const uint32_t mask = k < n ? ex & 15u : 0u;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float2*>(pw + row * max_pb * 64), 0, max_pb * 512, kBufWord3);
    const uint32_t off = ((mask >> u) & 1u)
                             ? (ey + (uint32_t)__popc(mask & ((1u << u) - 1u))) * 512u + pw_lane
                             : 0x80000000u;
    S.p0 = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, 0);
    if constexpr (FUSE) {
      typedef const f32x4 __attribute__((address_space(4))) cf32x4;
      const cf32x4* dp = reinterpret_cast<const cf32x4*>(
          reinterpret_cast<uintptr_t>(dlt + row * 16 + 8 * gs));
      S.dl0 = dp[0];
      S.dl1 = dp[1];
    } else {
      S.p1 = __builtin_amdgcn_raw_buffer_load_b128(rp, off + 16u, 0, 0);
      S.dl0 = *reinterpret_cast<const f32x4*>(dlt + row * 16 + hb);
    }
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(qt + row * (16 * D)), 0, 32 * D, kBufWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(dot + row * (16 * D)), 0, 32 * D, kBufWord3);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      S.qx[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, q_lane[j], 0, 0);
      S.dx[j] = __builtin_amdgcn_raw_buffer_load_b128(rd, q_lane[j], 0, 0);
    }
  };
  // lanes 0..31 of the result are x's lanes 0..31 (first) or 32..63 (second),
  // repeated in lanes 32..63
  auto halves = [](const u32x4& x, u32x4& lo, u32x4& hi) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto r = __builtin_amdgcn_permlane32_swap(x[e], x[e], false, false);
      lo[e] = r[0];
      hi[e] = r[1];
    }
  };
  // dS = P (dP - D~) - (D - D~) P and P as bf16 A operands, then the MFMAs
  auto consume = [&](const Stage& S) {
    if constexpr (FUSE) {
      u32x4 pa, pb;
      halves(S.p0, pa, pb);
      const float4 a = __builtin_bit_cast(float4, pa), b = __builtin_bit_cast(float4, pb);
      const f32x4 dl = (gq & 1) ? S.dl1 : S.dl0;
      const float s0 = fmaf(-dl[0], a.x, a.y), s1 = fmaf(-dl[1], a.z, a.w);
      const float s2 = fmaf(-dl[2], b.x, b.y), s3 = fmaf(-dl[3], b.z, b.w);
      const bf16x4s aS = pack4(bf16_hilo2(s0, s1, lo_sel), bf16_hilo2(s2, s3, lo_sel));
      const bf16x4s aP = pack4(bf16_hilo2(a.x, a.z, lo_sel), bf16_hilo2(b.x, b.z, lo_sel));
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        u32x4 q01, q23, d01, d23;
        halves(S.qx[j], q01, q23);
        halves(S.dx[j], d01, d23);
        const u32x4 qv[2] = {q01, q23}, dv[2] = {d01, d23};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int bb = 4 * j + h;
          const uint2 qb = make_uint2(qv[h >> 1][2 * (h & 1)], qv[h >> 1][2 * (h & 1) + 1]);
          const uint2 db = make_uint2(dv[h >> 1][2 * (h & 1)], dv[h >> 1][2 * (h & 1) + 1]);
          ak[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              aS, __builtin_bit_cast(bf16x4s, qb), ak[bb], 0, 0, 0);
          av[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              aP, __builtin_bit_cast(bf16x4s, db), av[bb], 0, 0, 0);
        }
      }
    } else {
      const float4 a = __builtin_bit_cast(float4, S.p0), b = __builtin_bit_cast(float4, S.p1);
      const f32x4 dl = S.dl0;
      const float s0 = fmaf(-dl[0], a.x, a.y), s1 = fmaf(-dl[1], a.z, a.w);
      const float s2 = fmaf(-dl[2], b.x, b.y), s3 = fmaf(-dl[3], b.z, b.w);
      const bf16x4s aSh = pack4(bf16_pk2(s0, s1), bf16_pk2(s2, s3));
      const bf16x4s aSl = pack4(bf16_hilo2(s0, s1, 1.0f), bf16_hilo2(s2, s3, 1.0f));
      const bf16x4s aPh = pack4(bf16_pk2(a.x, a.z), bf16_pk2(b.x, b.z));
      const bf16x4s aPl = pack4(bf16_hilo2(a.x, a.z, 1.0f), bf16_hilo2(b.x, b.z, 1.0f));
#pragma unroll
      for (int bb = 0; bb < NBW; ++bb) {
        const bool mine = (4 * gq) / G == (16 * (bbase + bb)) / D;
        const u32x4& qx = S.qx[bb / 2];
        const u32x4& dx = S.dx[bb / 2];
        const uint2 z = make_uint2(0u, 0u);
        const uint2 qb = make_uint2(qx[2 * (bb & 1)], qx[2 * (bb & 1) + 1]);
        const uint2 db = make_uint2(dx[2 * (bb & 1)], dx[2 * (bb & 1) + 1]);
        const bf16x4s bq = __builtin_bit_cast(bf16x4s, mine ? qb : z);
        const bf16x4s bd = __builtin_bit_cast(bf16x4s, mine ? db : z);
        ak[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aSh, bq, ak[bb], 0, 0, 0);
        ak[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aSl, bq, ak[bb], 0, 0, 0);
        av[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aPh, bd, av[bb], 0, 0, 0);
        av[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aPl, bd, av[bb], 0, 0, 0);
      }
    }
  };

  for (uint32_t base = 0; base < nq; base += LCAP) {
    const uint32_t n = min(nq - base, LCAP);
    __syncthreads();  // the previous chunk's entries are read
    for (uint32_t i = threadIdx.x; i < n; i += 256) sl[i] = lst[base + i];
    __syncthreads();
    uint32_t k = wv / NS;
    if (k >= n) continue;
    // two stages in turn: an entry's loads are issued before the previous
    // entry is consumed.  The loop's only exit test is at its end (a stage
    // past the list is consumed with zero weights), so the compiler cannot
    // sink a fetch past an exit to its use; the scheduling barriers keep
    // the machine scheduler from doing the same.
    Stage A, B;
    fetch(k, n, A);
    do {
      fetch(k + STEP, n, B);
      __builtin_amdgcn_sched_barrier(0);
      consume(A);
      fetch(k + 2 * STEP, n, A);
      __builtin_amdgcn_sched_barrier(0);
      consume(B);
      k += 2 * STEP;
    } while (k < n);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * 16 * KD; i += 256) sbuf[i] = 0.0f;
  __syncthreads();
  // lane (dim 16 (bbase + b) + l16) holds tokens 4gq + i
#pragma unroll
  for (int b = 0; b < NBW; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      atomicAdd(&sk[(4 * gq + i) * KD + 16 * (bbase + b) + l16], ak[b][i]);
      atomicAdd(&sv[(4 * gq + i) * KD + 16 * (bbase + b) + l16], av[b][i]);
    }
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * KD; i += 256) {
    const int64_t pos = t0 + i / KD;
    if (pos >= cap) continue;
    const int64_t o = ((int64_t)s * cap + pos) * KD + (i % KD);
    dk[o] += scale * sk[i];
    dv[o] += sv[i];
  }
}

bool bwd_mfma(const Dims& d) {
  return d.bf16 && d.q_heads == 16 &&
         ((d.kv_heads == 2 && (d.head_dim == 64 || d.head_dim == 128)) ||
          (d.kv_heads == 1 && d.head_dim == 128));
}

// Workspace: the transposed index, then per path
//   generic: per-block lists (rows x (k_B + 1)), D per (row, head);
//   MFMA:    per-group lists of uint2 (rows x max units), D - D~ per (row,
//            head), q / dO transposed (rows x 16 x head_dim bf16 each), and
//            {P, P (dP - D~)} per (row, token of the set, head) as fp32.
struct BwdPlan {
  bool mfma;
  int64_t nb;   // blocks (generic) or 16-token groups (MFMA) per sequence
  int max_pb;   // 4-token units of a largest token set
  size_t off_cnt, off_cur, off_off, off_list, off_dsum, off_qt, off_dot, off_pw, off_ord, bytes;
};

BwdPlan bwd_plan(const Dims& d, int batch, int n_q, int32_t max_pos_end) {
  BwdPlan p{};
  p.mfma = bwd_mfma(d);
  p.max_pb = (d.kB + 1) << (d.lr - 2);
  p.nb = p.mfma ? ((int64_t)max_pos_end + 15) >> 4 : ((int64_t)max_pos_end + d.r - 1) >> d.lr;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t rows = (size_t)batch * n_q;
  const size_t hd = (size_t)d.q_heads;
  size_t o = 0;
  p.off_cnt = o;  o = al(o + 4 * (size_t)batch * p.nb);
  p.off_cur = o;  o = al(o + 4 * (size_t)batch * p.nb);
  p.off_off = o;  o = al(o + 4 * ((size_t)batch * p.nb + 1));
  p.off_list = o;
  o = al(o + (p.mfma ? 8 * rows * (size_t)p.max_pb : 4 * rows * (size_t)(d.kB + 1)));
  p.off_dsum = o; o = al(o + 4 * rows * hd);
  p.off_qt = p.off_dot = p.off_pw = o;
  if (p.mfma) {
    p.off_qt = o;  o = al(o + 2 * rows * hd * (size_t)d.head_dim);
    p.off_dot = o; o = al(o + 2 * rows * hd * (size_t)d.head_dim);
    p.off_pw = o;  o = al(o + 8 * rows * (size_t)p.max_pb * 4 * hd);
    p.off_ord = o; o = al(o + 3 * 4 * rows);   // row order: key, first, order
  }
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
  if (pl.mfma) {
    uint2* glist = reinterpret_cast<uint2*>(ws + pl.off_list);
    uint16_t* qt = reinterpret_cast<uint16_t*>(ws + pl.off_qt);
    uint16_t* dot = reinterpret_cast<uint16_t*>(ws + pl.off_dot);
    float2* pw = reinterpret_cast<float2*>(ws + pl.off_pw);
    hipLaunchKernelGGL((bwd_group_list_kernel<false>), dim3((unsigned)rows), dim3(kNT), 0, st, ix,
                       glist, cap, n_q, q_pos0, sel, cnt, d.kB, d.lr);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(kNT), 0, st, ix, nblk);
    hipLaunchKernelGGL((bwd_group_list_kernel<true>), dim3((unsigned)rows), dim3(kNT), 0, st, ix,
                       glist, cap, n_q, q_pos0, sel, cnt, d.kB, d.lr);
    int32_t* okey = reinterpret_cast<int32_t*>(ws + pl.off_ord);
    int32_t* ofirst = okey + rows;
    int32_t* oorder = row_order_sorts(d, batch, n_q) ? ofirst + rows : nullptr;
    const hipError_t e = launch_row_order(d, batch, n_q, q_pos0, cap, sel, cnt, okey, ofirst,
                                          oorder, st);
    if (e != hipSuccess) return e;
#define QSA_BWD_MFMA(HKV, DD)                                                                  \
  if (d.kv_heads == HKV && d.head_dim == DD) {                                                 \
    hipLaunchKernelGGL((bwd_query_mfma_kernel<HKV, DD, (HKV == 2 && DD == 128) ? 16 : 32>),    \
                       dim3((unsigned)rows), dim3(256), 0, st,                                \
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache), \
                       static_cast<const uint16_t*>(v_cache), cap, n_q, q_pos0, sel, cnt, d.kB, \
                       d.scale, static_cast<const uint16_t*>(out), lse,                       \
                       static_cast<const uint16_t*>(dout), static_cast<uint16_t*>(dq), dsum, pw, \
                       pl.max_pb, qt, dot, d.lr, oorder, ofirst);                              \
    hipLaunchKernelGGL((bwd_key_mfma_kernel<HKV, DD>), dim3((unsigned)nblk), dim3(256), 0, st, ix, \
                       glist, pw, pl.max_pb, qt, dot, dsum, cap, d.scale, dk, dv);             \
  }
    QSA_BWD_MFMA(2, 128)
    QSA_BWD_MFMA(1, 128)
    QSA_BWD_MFMA(2, 64)
#undef QSA_BWD_MFMA
    return hipGetLastError();
  }
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
